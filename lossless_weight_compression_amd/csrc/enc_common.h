// enc_common.h -- internal definitions shared by the gfx950 kernels and the
// host side of libenc.so. Not part of the C ABI.
//
// Work decomposition used by every codec kernel:
//  * group   = 8 consecutive elements, owned by one lane. 8 codes of w bits
//              fill exactly w bytes, so every group's codes start on a byte
//              boundary for any width and any block size that is a multiple
//              of 8.
//  * block   = B elements = B/8 groups (B a power of two, 128..4096).
//  * segment = 64 blocks, one per lane of a wave64 for the intra-segment
//              scan of block payload sizes ("ENEC: A Lossless AI Model
//              Compression Method Enabling Fast Inference on Ascend NPUs",
//              Abstract: dependency-decoupled intra-segment scan).
//  * tile    = kTileGroups consecutive groups handled by one 256-thread
//              workgroup; a tile never straddles a segment (segments hold
//              64*B/8 >= 1024 groups) and always holds whole blocks.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "enc.h"

namespace enc {

constexpr uint32_t kHeaderBytes = 256;
constexpr uint32_t kSegBlocks = 64;
constexpr uint32_t kSectionAlign = 256;
constexpr uint32_t kPayloadAlign = 16;
constexpr uint32_t kThreads = 256;                                // 4 x wave64
constexpr uint32_t kGroupsPerThread = 4;
constexpr uint32_t kTileGroups = kThreads * kGroupsPerThread;     // 1024
constexpr uint64_t kTileElems = uint64_t(kTileGroups) * 8;        // 8192
constexpr uint32_t kMinLog2B = 7, kMaxLog2B = 12;

__host__ __device__ inline uint64_t align_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

// 16-byte store with the non-temporal hint, for stream and output bytes a
// kernel writes once and does not read back: they need not stay in the
// caches (measured: the 8B-shaped set decodes 1.4% and encodes 2% faster,
// FP32 batches decode 6% faster than with plain stores).
typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_nt16(void *p, uint4 v) {
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4_nt, v), static_cast<u32x4_nt *>(p));
}

// Block width of a code range r: the bits of r, or, for streams with
// power-of-two widths, the next of 0, 1, 2, 4, 8 ("ENEC: A Lossless AI Model
// Compression Method Enabling Fast Inference on Ascend NPUs", Abstract:
// bit-width quantization).
__host__ __device__ inline uint32_t block_width(uint32_t r, uint32_t pow2) {
  uint32_t w = 0;
  while (r >> w) ++w;
  return pow2 ? (w <= 2 ? w : (w <= 4 ? 4u : 8u)) : w;
}

// One stream to decode (by value for a single call, in the batch table for
// batched calls). 80 bytes.
struct DecodeDesc {
  const uint8_t *stream;   // device stream base
  void *out;               // device output (element type from dtype)
  uint64_t n;              // elements
  uint64_t nb;             // blocks (0 for RAW)
  uint64_t meta_off;       // section offsets inside the stream
  uint64_t segoff_off;
  uint64_t payload_off;
  uint64_t total;          // stream bytes (reads never go past it)
  uint32_t log2b;          // log2 of the block size
  uint32_t raw;            // 1 = RAW stream (verbatim values at offset 256)
  uint32_t dtype;          // header element type: 0 or 1 BF16, 2 FP16, 3 FP32
  uint32_t reserved;
};
static_assert(sizeof(DecodeDesc) == 80, "table entry layout");

// Batch table in device memory: header, then `count` DecodeDesc, then two
// lists of `count + 1` u64 tile prefixes (first tile of each item, then the
// total): over the BF16 items' tiles, then over the FP16 / FP32 items' tiles
// (an item's tiles count in its own list only); then, at map_off and
// wide_map_off (256-byte aligned), the item index (u32) of every tile of
// each list, so a workgroup finds its item with one load.
struct BatchHeader {
  uint64_t total_tiles;   // tiles of BF16 items
  uint32_t count;
  uint32_t magic;
  uint64_t wide_tiles;    // tiles of FP16 and FP32 items
  uint64_t map_off;       // byte offset of the BF16 tiles' item indices
  uint64_t wide_map_off;  // byte offset of the FP16 / FP32 tiles' item indices
  uint64_t reserved[3];
};
static_assert(sizeof(BatchHeader) == 64, "table header layout");
constexpr uint32_t kBatchMagic = 0x42434E45u;  // "ENCB"

inline uint64_t tiles_for(uint64_t n) { return (n + kTileElems - 1) / kTileElems; }
// The decoder's work unit: one workgroup decodes a tile of consecutive
// groups, decode_groups_per_thread(dtype) per lane: 2 for BF16 and FP32
// (4096 values), 4 for FP16 (8192). Each tile is a power of two of at most
// 1024 groups, so it never crosses a segment (64 blocks of at least 16
// groups).
__host__ __device__ constexpr uint32_t decode_groups_per_thread(uint32_t dtype) {
  return dtype == 2 ? 4u : 2u;
}
__host__ __device__ constexpr uint32_t decode_tile_groups(uint32_t dtype) {
  return kThreads * decode_groups_per_thread(dtype);
}
static_assert(decode_tile_groups(1) <= 1024 && decode_tile_groups(2) <= 1024 &&
                  decode_tile_groups(3) <= 1024,
              "decode tiles must not cross a segment");
// Decode tiles of an n-value stream of the given dtype.
inline uint64_t decode_tiles_for(uint64_t n, uint32_t dtype) {
  const uint64_t t = 8ull * decode_tile_groups(dtype);
  return (n + t - 1) / t;
}

// The single-pass encoder handles onepass_sub(n) consecutive tiles per
// workgroup and runs one look-back per workgroup: 4 for large inputs (fewer
// look-backs), fewer for small ones (more workgroups to fill the device;
// measured on 4M / 16.8M / 58.7M / 525M-value tensors).
constexpr uint32_t kOnePassMaxSub = 4;
inline uint32_t onepass_sub(uint64_t n) { return n <= (8ull << 20) ? 1 : n <= (32ull << 20) ? 2 : 4; }
inline uint64_t onepass_tiles(uint64_t n) { return (tiles_for(n) + onepass_sub(n) - 1) / onepass_sub(n); }

// ---- launchers (defined in the .hip files) --------------------------------
hipError_t launch_decode(const DecodeDesc &d, hipStream_t s);
// One workgroup per tile of each list (tiles: BF16 list, wide_tiles: FP16
// and FP32 list), as recorded in the table when it was prepared.
hipError_t launch_decode_batch(const void *table, uint64_t tiles, uint64_t wide_tiles, hipStream_t s);

struct EncodeArgs {
  const uint16_t *in;
  uint8_t *out;          // stream base
  uint8_t *ws_meta;      // 2 bytes per block
  uint64_t *ws_segsum;   // per-segment payload bytes, scanned in place to offsets
  uint64_t *ws_total;    // payload bytes (one u64)
  uint64_t n, nb, nseg;
  uint64_t meta_off, segoff_off, payload_off;
  uint32_t log2b;
  uint32_t pow2;         // 1: widths rounded up to 0, 1, 2, 4 or 8
  uint32_t dtype;        // 1 (or 0) BF16, 2 FP16, 3 FP32: the single pass and its pads
  // single pass only
  uint64_t *status;      // one word per tile: flag (bits 63..62) | payload bytes
  uint32_t *error;       // nonzero: a look-back wait gave up
  uint32_t spin_limit;   // polls of a not-yet-published tile before giving up
  uint32_t short_sleep;  // 1: poll the look-back window after a short sleep (small launches)
  uint64_t cap;          // output capacity: payload stores beyond it are dropped
  uint64_t ntiles;
};
hipError_t launch_encode_params(const EncodeArgs &a, hipStream_t s);
hipError_t launch_encode_onepass(const EncodeArgs &a, hipStream_t s);
// FP16 / FP32 single pass (a.dtype 2 or 3), one stream or a batch of one dtype
hipError_t launch_encode_wide_onepass(const EncodeArgs &a, hipStream_t s);
hipError_t launch_encode_wide_onepass_batch(const void *table, uint64_t total_wgs, uint32_t dtype,
                                            hipStream_t s);
hipError_t launch_encode_scan(const EncodeArgs &a, hipStream_t s);
hipError_t launch_encode_pack(const EncodeArgs &a, hipStream_t s);

struct HeaderImage {
  uint8_t bytes[256];
};
hipError_t launch_encode_finish(const EncodeArgs &a, const HeaderImage &h, hipStream_t s);
hipError_t launch_encode_pads(const EncodeArgs &a, const HeaderImage &h, hipStream_t s);
hipError_t launch_encode_raw(const uint16_t *in, uint8_t *out, uint64_t n, const HeaderImage &h,
                             hipStream_t s);
// FP16 (dtype 2) and FP32 (dtype 3) input; the scan is launch_encode_scan.
hipError_t launch_encode_wide_params(const EncodeArgs &a, uint32_t dtype, hipStream_t s);
hipError_t launch_encode_wide_pack(const EncodeArgs &a, uint32_t dtype, hipStream_t s);
hipError_t launch_encode_wide_finish(const EncodeArgs &a, uint32_t dtype, const HeaderImage &h,
                                     hipStream_t s);

// Sets the library's thread-local last-error text (enc_api.cpp) and returns st.
enc_status set_error(enc_status st, const char *fmt, ...);

// ---- measurement: streaming kernel with the decoder's access shape --------
hipError_t launch_stream_probe(const void *src, uint64_t src_bytes, void *dst, uint64_t dst_bytes,
                               uint32_t items, uint32_t threads, hipStream_t s);

// ---- deep stream check ------------------------------------------------------
struct ValidateArgs {
  const uint8_t *stream;
  unsigned long long *result;   // [3]: first failing block / offset per kind, ~0 = none
  uint64_t n, nb, nseg;
  uint64_t meta_off, segoff_off, payload_off, payload_bytes;
  uint32_t log2b;
  uint32_t pow2;         // 1: the stream declares power-of-two widths
  uint32_t emax;         // largest exponent field value: 255 (BF16, FP32), 31 (FP16)
};
hipError_t launch_validate(const ValidateArgs &a, hipStream_t s);

// ---- fused decompress-GEMM ------------------------------------------------
struct GemmArgs {
  const uint16_t *x;       // X [M, K] bf16
  const uint8_t *wstream;  // compressed W stream (nullptr for dense)
  const uint16_t *wdense;  // dense W [K, N] bf16 (RAW stream data or dense GEMM)
  float *y;                // Y [M, N] fp32
  float *partial;          // [ksplit, M, N] split-K partial sums (workspace)
  uint32_t M, K, N;
  uint32_t log2b;
  uint64_t nb;
  uint64_t meta_off, segoff_off, payload_off;
  uint64_t total;          // stream bytes (reads never go past it)
  uint32_t ksplit;         // number of K ranges
  uint32_t krows;          // rows per K range
  uint32_t *counters;      // per-strip arrival counts (zero between calls), or nullptr
};
// [K, N] GEMM workspace: gemm_counter_bytes(N) of strip arrival counters
// (zero between calls), then the split-K partial slices.
uint64_t gemm_counter_bytes(uint32_t N);
uint64_t gemm_workspace_bytes(uint32_t M, uint32_t K, uint32_t N);
hipError_t launch_gemm(const GemmArgs &a, hipStream_t s);
// W stored [N, K] (linear-layer layout), Y = X . W^T; needs N % 64 == 0 and
// K a multiple of the block size (dense: of 32).
uint64_t gemm_nt_workspace_bytes(uint32_t M, uint32_t K, uint32_t N, uint32_t log2b);
hipError_t launch_gemm_nt(const GemmArgs &a, hipStream_t s);
void gemm_plan(uint32_t M, uint32_t K, uint32_t N, uint32_t *ksplit, uint32_t *krows);

}  // namespace enc
