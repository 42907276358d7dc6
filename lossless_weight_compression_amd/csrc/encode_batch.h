// encode_batch.h -- device tables of the batched single-pass encoder.
//
// "ENEC: A Lossless AI Model Compression Method Enabling Fast Inference on
// Ascend NPUs", Abstract: the per-block coding and the decoupled prefix scan
// are those of one stream; a batch only puts many streams in one launch.
#pragma once
#include "enc_common.h"

namespace enc {

// Device table of k_enc_onepass_batch: EncBatchHeader, then `count`
// EncodeArgs (each with its own status words, size slot and error word,
// ntiles counted in kOnePassMaxSub-sub-tile workgroups), then `count + 1`
// u64 prefixes of the streams' workgroup counts (the last is the total).
struct EncBatchHeader {
  uint64_t total_wgs;
  uint32_t count;
  uint32_t magic;
  uint64_t reserved[6];
};
static_assert(sizeof(EncBatchHeader) == 64, "table header layout");
constexpr uint32_t kEncBatchMagic = 0x45424348u;   // "HCBE"

inline uint64_t onepass_batch_tiles(uint64_t n) {
  return (tiles_for(n) + kOnePassMaxSub - 1) / kOnePassMaxSub;
}

hipError_t launch_encode_onepass_batch(const void *table, uint64_t total_wgs, hipStream_t s);

// Header and section pads of many coded streams: one workgroup per item.
struct PadsItem {
  EncodeArgs a;
  HeaderImage h;
};
hipError_t launch_encode_pads_batch(const void *items, uint32_t count, hipStream_t s);

}  // namespace enc
