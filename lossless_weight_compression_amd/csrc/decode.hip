// decode.hip -- gfx950 decoder for the block-based fixed-length BF16 stream.
//
// "ENEC: A Lossless AI Model Compression Method Enabling Fast Inference on
// Ascend NPUs", Abstract: block-based fixed-length code with per-block bit
// width and an intra-segment prefix scan of block sizes. "ZipServ: Fast and
// Memory-Efficient LLM Inference with Hardware-Aware Lossless Compression",
// Abstract: a fixed-length format decodes in constant time and in parallel.
//
// Mapping onto CDNA4 (wave64, 256 CUs in 8 XCDs):
//  * a workgroup (4 waves) decodes one tile of 512 groups = 4096 BF16
//    values (512 for FP32, 1024 for FP16); lane t owns groups t and t+256 of
//    the tile, so every wave instruction touches 64 consecutive groups: 512
//    contiguous bytes of the sign+mantissa plane, one contiguous run of
//    packed codes, and 1 KiB of contiguous output (one 16-byte store per
//    lane);
//  * each wave re-derives the payload offsets of the tile's 64-block segment
//    itself: lane j reads block j's {base, width}, computes the padded payload
//    size and a wave64 inclusive scan gives every block's start -- no
//    workgroup barrier and no LDS;
//  * a group's 8 codes of w bits are exactly w bytes starting on a byte
//    boundary; the lane loads the three dwords that cover them with one
//    buffer_load_dwordx3 (dwords past the stream's end read as zero),
//    funnel-shifts them into place (v_alignbit) and cuts the fields with
//    v_bfe; exponent bytes get the block base with one packed add (a valid
//    stream never carries out of a byte), and v_bfi/v_perm interleave them
//    with the sign+mantissa bytes into four BF16 pairs;
//  * every load of a tile's groups is issued before any of them is decoded,
//    so each lane keeps its groups' reads in flight together;
//  * one workgroup per tile, in tile order (workgroup b decodes tile
//    tile0 + b): the resident workgroups then cover one contiguous window of
//    the stream and of the output that sweeps through memory as a single
//    front; the same kernel body serves the batched decode of a whole
//    weight set in one launch.
#include <cstdlib>

#include "enc_common.h"
#include "group_math.h"

namespace enc {
namespace {

constexpr uint32_t GPT = decode_groups_per_thread(1);   // BF16 tiles
constexpr uint32_t kDecodeTileGroups = decode_tile_groups(1);
constexpr uint64_t kDecodeTileElems = 8ull * kDecodeTileGroups;

// Every access of the stream and the output goes through these byte
// pointers in the global address space. The batch kernels read their
// descriptors from the table, and generic pointers loaded from memory made
// the compiler address the stream with flat instructions; flat loads count
// against the LDS wait counter as well, so each lane shuffle of the next
// group waited for all of this group's loads (one group of loads in flight
// per lane instead of four). With global loads issued on every path the
// 8B-shaped set decodes in 4.82-4.84 ms instead of 4.89-4.94.
#define ENC_GLOBAL __attribute__((address_space(1)))
typedef const ENC_GLOBAL uint8_t *gsrc;
typedef ENC_GLOBAL uint8_t *gdst;

__device__ __forceinline__ gsrc stream_of(const DecodeDesc &d) { return (gsrc)d.stream; }
__device__ __forceinline__ gdst output_of(const DecodeDesc &d) { return (gdst)d.out; }

typedef uint32_t u32x2_g __attribute__((ext_vector_type(2)));
template <class T>   // scalar types
__device__ __forceinline__ T ldg(gsrc p) {
  return *(const ENC_GLOBAL T *)p;
}
__device__ __forceinline__ uint4 ldg4(gsrc p) {
  const u32x4_nt v = *(const ENC_GLOBAL u32x4_nt *)p;
  return make_uint4(v.x, v.y, v.z, v.w);
}
// Raw buffer descriptors over the stream. Range checking as the CDNA3 ISA
// reference guide defines it for buffer instructions (section on buffer
// addressing, range checking; CDNA4 keeps the rule): with stride 0 an access
// is out of range when its byte offset is at or past num_records, the check
// is made for each dword of a multi-dword access, and out-of-range dwords
// load as zero without a memory access.
typedef uint32_t u32x3_g __attribute__((ext_vector_type(3)));
constexpr uint32_t kPastRange = 0xFFFFFFF0u;   // an offset no descriptor here reaches
// Descriptor over the stream bytes [from, total), at most kPastRange of them.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t stream_rsrc_from(const DecodeDesc &d, uint64_t from) {
  const uint64_t room = d.total > from ? d.total - from : 0;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(d.stream + from), 0,
                                           (int)(room < kPastRange ? room : kPastRange), 0x00020000);
}
// A value the caller knows to be equal in every lane, in scalar registers.
// (The builtin returns int: each half goes through uint32_t, so the low half
// is not sign-extended into the high one.)
__device__ __forceinline__ uint64_t wave_uniform(uint64_t v) {
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
  return ((uint64_t)hi << 32) | lo;
}
template <class T>
__device__ __forceinline__ void stg(gdst p, T v) {
  *(ENC_GLOBAL T *)p = v;
}

// Decoded output is written once: 16-byte stores with the non-temporal hint.
__device__ __forceinline__ void store_out16(gdst p, uint4 v) {
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4_nt, v), (ENC_GLOBAL u32x4_nt *)p);
}

// Tail group: store only the elements below n (no dynamically indexed array,
// so nothing is placed in scratch or LDS). ob: the output's bytes.
__device__ __forceinline__ void store_partial(gdst ob, uint64_t e0, uint64_t n, uint4 o) {
#pragma unroll
  for (uint32_t k = 0; k < 8; ++k) {
    const uint32_t word = k < 2 ? o.x : k < 4 ? o.y : k < 6 ? o.z : o.w;
    if (e0 + k < n) stg<uint16_t>(ob + 2 * (e0 + k), (uint16_t)(word >> (16 * (k & 1))));
  }
}

// src, ob: the RAW values' bytes and the output's bytes.
__device__ __forceinline__ void copy_group_raw(gsrc src, gdst ob, uint64_t e0, uint64_t n, uint4 v) {
  if (e0 + 8 <= n) {
    store_out16(ob + 2 * e0, v);
  } else {
    for (uint64_t e = e0; e < n; ++e) stg<uint16_t>(ob + 2 * e, ldg<uint16_t>(src + 2 * e));
  }
}

// RAW stream: the values sit verbatim after the header; copy the tile with
// all of a lane's 16-byte loads issued before the stores.
__device__ __forceinline__ void copy_tile_raw(const DecodeDesc &d, uint64_t tile, uint32_t tid) {
  const gsrc src = stream_of(d) + kHeaderBytes;
  const gdst ob = output_of(d);
  const uint64_t e_first = tile * kDecodeTileElems + (uint64_t)tid * 8;
  const uint4 z = make_uint4(0, 0, 0, 0);
  uint4 v[GPT];
#pragma unroll
  for (uint32_t it = 0; it < GPT; ++it) {
    const uint64_t e = e_first + (uint64_t)it * 8 * kThreads;
    v[it] = e + 8 <= d.n ? ldg4(src + 2 * e) : z;
  }
#pragma unroll
  for (uint32_t it = 0; it < GPT; ++it) {
    const uint64_t e = e_first + (uint64_t)it * 8 * kThreads;
    if (e < d.n) copy_group_raw(src, ob, e, d.n, v[it]);
  }
}

// Per-wave scan of the tile's segment: pk (lane j) = block j's base << 24 |
// width << 20 | payload offset inside the segment, seg_payload = the
// segment's payload start in the stream.
__device__ __forceinline__ void segment_scan(const DecodeDesc &d, uint64_t seg, uint32_t lane,
                                             uint32_t &pk, uint64_t &seg_payload) {
  const gsrc s = stream_of(d);
  const uint64_t n = d.n;
  const uint64_t blk = (seg << 6) + lane;
  uint32_t m = 0;
  if (blk < d.nb) m = ldg<uint16_t>(s + d.meta_off + 2 * blk);
  const uint32_t w = m >> 8;
  const bool wide = __any(w > 8);   // wave-uniform
  const uint32_t L = (blk + 1 == d.nb) ? (uint32_t)(n - ((d.nb - 1) << d.log2b)) : (1u << d.log2b);
  const uint32_t P = (((w * L + 7) >> 3) + 15) & ~15u & (blk < d.nb ? ~0u : 0u);
  pk = ((m & 0xFFu) << 24) | ((w & 15u) << 20);
  const uint32_t incl = wave_incl_scan(P);
  pk |= incl - P;   // exclusive offset < 2^18 whenever every width is at most 8
  const uint64_t seg_rel = ldg<uint64_t>(s + d.segoff_off + 8 * seg);
  seg_payload = d.payload_off + seg_rel;
  // Guard against corrupted streams (checked once per wave, not per group):
  // a width above 8 or a segment whose payload runs past the stream end
  // decodes as width 0, so no lane ever reads outside [0, total). The test
  // is written without sums that could wrap (payload_off <= total holds for
  // every header the host accepts).
  // a lane shuffle, not v_readlane: with the total in a scalar register the
  // guard below became a branch that waited early for the offset load
  // (measured: the 8B-shaped set decodes 1% slower)
  const uint32_t seg_bytes = __shfl(incl, 63, 64);
  const uint64_t room = d.total - d.payload_off;
  if (wide || seg_rel > room || seg_bytes > room - seg_rel) {
    pk = 0;
    seg_payload = d.payload_off;
  }
}

__device__ __forceinline__ void decode_tile(const DecodeDesc &d, uint64_t tile, uint32_t tid) {
  if (d.raw) {
    copy_tile_raw(d, tile, tid);
    return;
  }
  const gdst ob = output_of(d);
  const uint64_t n = d.n;
  const uint32_t lane = tid & 63;
  const uint32_t log2gpb = d.log2b - 3;       // groups per block
  const uint32_t log2gps = log2gpb + 6;       // groups per segment
  const uint64_t g0 = tile * kDecodeTileGroups;
  const uint64_t seg = g0 >> log2gps;
  const uint32_t gs0 = (uint32_t)(g0 & ((1ull << log2gps) - 1));

  uint32_t pk;
  uint64_t seg_payload;
  segment_scan(d, seg, lane, pk, seg_payload);

  // Phase 1: issue every load of this lane's groups: the 8 sign+mantissa
  // bytes (one dwordx2) and the 12 bytes from the code dword holding the
  // group's first code bit (one dwordx3), both off raw buffer descriptors.
  // A lane with nothing to read points its load past the range (zeros, no
  // memory access), and a dwordx3 that runs past the stream's end loads
  // zeros for the dwords outside it, so no load needs a guard or a
  // substitute address.
  const uint64_t segp = wave_uniform(seg_payload);
  const __amdgpu_buffer_rsrc_t code_rs = stream_rsrc_from(d, segp);
  const __amdgpu_buffer_rsrc_t sm_rs = stream_rsrc_from(d, kHeaderBytes + g0 * 8);
  uint32_t sml[GPT], smh[GPT], q0[GPT], q1[GPT], q2[GPT], info[GPT];
#pragma unroll
  for (uint32_t it = 0; it < GPT; ++it) {
    const uint32_t q = it * kThreads + tid;
    const uint64_t e0 = (g0 + q) * 8;
    const uint32_t gs = gs0 + q;
    const uint32_t p = __shfl(pk, (int)(gs >> log2gpb), 64);
    const uint32_t u = gs & ((1u << log2gpb) - 1);
    const uint32_t w = (p >> 20) & 15u;
    const uint64_t rem = e0 < n ? n - e0 : 0;
    const uint32_t valid = rem < 8 ? (uint32_t)rem : 8u;
    const uint32_t nbytes = (valid * w + 7) >> 3;
    const uint32_t off = (p & 0xFFFFFu) + u * w;   // from the segment's payload start (16-byte aligned)
    const u32x2_g smv = __builtin_amdgcn_raw_buffer_load_b64(sm_rs, valid ? 8 * q : kPastRange, 0, 0);
    const u32x3_g qv = __builtin_amdgcn_raw_buffer_load_b96(code_rs, nbytes ? (off & ~3u) : kPastRange, 0, 0);
    sml[it] = smv.x;
    smh[it] = smv.y;
    q0[it] = qv.x;
    q1[it] = qv.y;
    q2[it] = qv.z;
    info[it] = (p & 0xFFF00000u) | ((off & 3u) << 3) | (valid << 8);
  }

  // Phase 2: decode and store. Every group is decoded, also one past the
  // end whose loads read zeros, and only the store depends on `valid`: with
  // `if (!valid) continue` here the compiler moved the second group's loads
  // under that test, behind the first group's wait (8B-shaped set: 4.65-4.70
  // ms per decode with global loads and the skip, 4.60-4.64 without the
  // skip, 4.48-4.57 with the buffer loads as well).
#pragma unroll
  for (uint32_t it = 0; it < GPT; ++it) {
    const uint32_t valid = (info[it] >> 8) & 15u;
    const uint32_t q = it * kThreads + tid;
    const uint64_t e0 = (g0 + q) * 8;
    const uint32_t w = (info[it] >> 20) & 15u;
    const uint32_t sh = info[it] & 31u;
    const uint32_t base4 = (info[it] >> 24) * 0x01010101u;
    const uint32_t lo = __builtin_amdgcn_alignbit(q1[it], q0[it], sh);
    const uint32_t hi = __builtin_amdgcn_alignbit(q2[it], q1[it], sh);
    const uint4 o = join_group(lo, hi, w, base4, sml[it], smh[it]);
    if (valid == 8)
      store_out16(ob + 2 * e0, o);
    else if (valid)
      store_partial(ob, e0, n, o);
  }
}

// ---------------------------------------------------------------------------
// FP16 (DT 2) and FP32 (DT 3) streams: the same exponent codes; the
// sign+mantissa field is 11 / 24 bits per value, packed LSB first, so a
// group's fields are 11 / 24 bytes at 11 g / 24 g of the section. Output
// values are rebuilt field by field (sign << top | exponent << shift |
// mantissa).
// ---------------------------------------------------------------------------
template <uint32_t DT>
__device__ __forceinline__ void decode_tile_wide(const DecodeDesc &d, uint64_t tile, uint32_t tid) {
  constexpr uint32_t ES = DT == 3 ? 4 : 2;        // element bytes
  const gsrc s = stream_of(d);
  const gdst outb = output_of(d);
  const uint64_t n = d.n;
  constexpr uint32_t WGPT = decode_groups_per_thread(DT);
  const uint64_t g0 = tile * decode_tile_groups(DT);
  if (d.raw) {
    // the tile's bytes as 16-byte chunks, consecutive lanes on consecutive
    // chunks (every store instruction writes whole lines)
    constexpr uint32_t CPT = WGPT * ES / 2;   // chunks per thread
    const uint64_t b0 = tile * 8ull * decode_tile_groups(DT) * ES, bn = n * ES;
    for (uint32_t it = 0; it < CPT; ++it) {
      const uint64_t b = b0 + 16 * (uint64_t)(it * kThreads + tid);
      if (b + 16 <= bn)
        store_out16(outb + b, ldg4(s + kHeaderBytes + b));
      else
        for (uint64_t k = b; k < bn; ++k) stg<uint8_t>(outb + k, ldg<uint8_t>(s + kHeaderBytes + k));
    }
    return;
  }
  const uint32_t lane = tid & 63;
  const uint32_t log2gpb = d.log2b - 3, log2gps = log2gpb + 6;
  const uint64_t seg = g0 >> log2gps;
  const uint32_t gs0 = (uint32_t)(g0 & ((1ull << log2gps) - 1));
  uint32_t pk;
  uint64_t seg_payload;
  segment_scan(d, seg, lane, pk, seg_payload);

  if (DT == 3) {
    // FP32: a lane decodes half a group (4 values: 12 bytes of 24-bit fields
    // at 24 g + 12 h, codes 4h .. 4h+3), so consecutive lanes write
    // consecutive 16-byte pieces: with whole groups per lane (32 bytes each)
    // every store instruction wrote half of each line it touched (a batch
    // of 28 FP32 tensors: 1.72 ms that way, 1.48 ms this way).
    // Every load of the lane's half groups first (addresses clamped in
    // bounds, no branch), then decode and store.
    constexpr uint32_t NH = 2 * WGPT;
    const __amdgpu_buffer_rsrc_t code_rs = stream_rsrc_from(d, wave_uniform(seg_payload));
    const __amdgpu_buffer_rsrc_t fld_rs = stream_rsrc_from(d, kHeaderBytes + 24 * g0);
    uint32_t q0[NH], q1[NH], q2[NH], fd[NH][3], info[NH];
#pragma unroll
    for (uint32_t it = 0; it < NH; ++it) {
      const uint32_t hq = it * kThreads + tid;
      const uint32_t q = hq >> 1, h = hq & 1;
      const uint64_t g = g0 + q;
      const uint64_t e0 = g * 8 + 4 * h;
      const uint32_t gs = gs0 + q;
      const uint32_t p = __shfl(pk, (int)(gs >> log2gpb), 64);   // with every lane active
      const uint32_t u = gs & ((1u << log2gpb) - 1);
      const uint32_t w = (p >> 20) & 15u;
      const bool live = e0 < n;
      const uint64_t remg = live ? n - g * 8 : 0;
      const uint32_t validg = remg < 8 ? (uint32_t)remg : 8u;   // values of the group
      const uint32_t nbytes = (validg * w + 7) >> 3;
      const uint32_t off = (p & 0xFFFFFu) + u * w;
      // codes as in the BF16 tile; the half group's 12 bytes of fields at
      // 24 g + 12 h (4-aligned; a tail group's read stays in the stream,
      // whose metadata sections follow)
      const u32x3_g qv = __builtin_amdgcn_raw_buffer_load_b96(code_rs, nbytes ? (off & ~3u) : kPastRange, 0, 0);
      const u32x3_g fv = __builtin_amdgcn_raw_buffer_load_b96(fld_rs, live ? 24 * q + 12 * h : kPastRange, 0, 0);
      q0[it] = qv.x;
      q1[it] = qv.y;
      q2[it] = qv.z;
      fd[it][0] = fv.x;
      fd[it][1] = fv.y;
      fd[it][2] = fv.z;
      info[it] = (p & 0xFFF00000u) | ((uint32_t)live << 8) | ((off & 3u) << 3);
    }
    // every half group is decoded (those past n from zeros) and only the
    // store depends on it being live, so no load moves under a branch
#pragma unroll
    for (uint32_t it = 0; it < NH; ++it) {
      const uint32_t hq = it * kThreads + tid;
      const uint32_t h = hq & 1;
      const uint64_t e0 = (g0 + (hq >> 1)) * 8 + 4 * h;
      const uint32_t w = (info[it] >> 20) & 15u;
      const uint32_t lsh = info[it] & 31u;
      uint32_t el, eh;
      codes_to_bytes(__builtin_amdgcn_alignbit(q1[it], q0[it], lsh),
                     __builtin_amdgcn_alignbit(q2[it], q1[it], lsh), w, el, eh);
      const uint32_t eb = (h ? eh : el) + (info[it] >> 24) * 0x01010101u;
      const uint32_t d0 = fd[it][0], d1 = fd[it][1], d2 = fd[it][2];
      const uint32_t f[4] = {d0 & 0xFFFFFFu, __builtin_amdgcn_alignbit(d1, d0, 24) & 0xFFFFFFu,
                             __builtin_amdgcn_alignbit(d2, d1, 16) & 0xFFFFFFu, d2 >> 8};
      uint32_t o[4];
#pragma unroll
      for (uint32_t k = 0; k < 4; ++k)
        o[k] = ((f[k] >> 23) << 31) | (((eb >> (8 * k)) & 0xFFu) << 23) | (f[k] & 0x7FFFFFu);
      const gdst dst = outb + 4 * e0;
      const uint64_t rem = e0 < n ? n - e0 : 0;
      if (rem >= 4) {
        store_out16(dst, make_uint4(o[0], o[1], o[2], o[3]));
      } else if (rem) {
#pragma unroll
        for (uint32_t k = 0; k < 4; ++k)
          if (k < rem) stg<uint32_t>(dst + 4 * k, o[k]);
      }
    }
    return;
  }

  // FP16: every load of the lane's groups first, then decode and store, as
  // in the BF16 tile (buffer loads, lanes with nothing to read past the
  // range; every group decoded, only the store depends on its valid count).
  const __amdgpu_buffer_rsrc_t code_rs = stream_rsrc_from(d, wave_uniform(seg_payload));
  const uint64_t fbase = (kHeaderBytes + 11 * g0) & ~15ull;
  const __amdgpu_buffer_rsrc_t fld_rs = stream_rsrc_from(d, fbase);
  uint32_t q0[WGPT], q1[WGPT], q2[WGPT], fw[WGPT][4], info[WGPT];
#pragma unroll
  for (uint32_t it = 0; it < WGPT; ++it) {
    const uint32_t q = it * kThreads + tid;
    const uint64_t g = g0 + q;
    const uint64_t e0 = g * 8;
    const uint32_t gs = gs0 + q;
    const uint32_t p = __shfl(pk, (int)(gs >> log2gpb), 64);   // with every lane active
    const uint32_t u = gs & ((1u << log2gpb) - 1);
    const uint32_t w = (p >> 20) & 15u;
    const uint64_t rem = e0 < n ? n - e0 : 0;
    const uint32_t valid = rem < 8 ? (uint32_t)rem : 8u;
    const uint32_t nbytes = (valid * w + 7) >> 3;
    const uint32_t off = (p & 0xFFFFFu) + u * w;
    // 11-bit fields of 8 values: 11 bytes at 11 g (any alignment), read as
    // the 16-byte aligned-dword window that covers them (a tail group's
    // window stays in the stream: the metadata sections follow)
    const uint32_t fo = (uint32_t)(kHeaderBytes + 11 * g - fbase);
    const u32x3_g qv = __builtin_amdgcn_raw_buffer_load_b96(code_rs, nbytes ? (off & ~3u) : kPastRange, 0, 0);
    const u32x4_nt fv = __builtin_amdgcn_raw_buffer_load_b128(fld_rs, valid ? (fo & ~3u) : kPastRange, 0, 0);
    q0[it] = qv.x;
    q1[it] = qv.y;
    q2[it] = qv.z;
    fw[it][0] = fv.x;
    fw[it][1] = fv.y;
    fw[it][2] = fv.z;
    fw[it][3] = fv.w;
    info[it] = (p & 0xFFF00000u) | ((fo & 3u) << 15) | (valid << 8) | ((off & 3u) << 3);
  }
#pragma unroll
  for (uint32_t it = 0; it < WGPT; ++it) {
    const uint32_t valid = (info[it] >> 8) & 15u;
    const uint64_t e0 = (g0 + it * kThreads + tid) * 8;
    const uint32_t w = (info[it] >> 20) & 15u;
    const uint32_t lsh = info[it] & 31u;
    const uint32_t fsh = (info[it] >> 12) & 31u;
    const uint32_t base4 = (info[it] >> 24) * 0x01010101u;
    uint32_t el, eh;
    codes_to_bytes(__builtin_amdgcn_alignbit(q1[it], q0[it], lsh),
                   __builtin_amdgcn_alignbit(q2[it], q1[it], lsh), w, el, eh);
    el += base4;
    eh += base4;
    const uint32_t f0 = __builtin_amdgcn_alignbit(fw[it][1], fw[it][0], fsh);
    const uint32_t f1 = __builtin_amdgcn_alignbit(fw[it][2], fw[it][1], fsh);
    const uint32_t f2 = __builtin_amdgcn_alignbit(fw[it][3], fw[it][2], fsh);
    // field k = bits [11 k, 11 k + 11) of f2:f1:f0
    uint32_t sm[8];
    sm[0] = f0 & 0x7FFu;
    sm[1] = (f0 >> 11) & 0x7FFu;
    sm[2] = __builtin_amdgcn_alignbit(f1, f0, 22) & 0x7FFu;
    sm[3] = (f1 >> 1) & 0x7FFu;
    sm[4] = (f1 >> 12) & 0x7FFu;
    sm[5] = __builtin_amdgcn_alignbit(f2, f1, 23) & 0x7FFu;
    sm[6] = (f2 >> 2) & 0x7FFu;
    sm[7] = (f2 >> 13) & 0x7FFu;
    uint32_t o[8];
#pragma unroll
    for (uint32_t k = 0; k < 8; ++k) {
      const uint32_t e = ((k < 4 ? el : eh) >> (8 * (k & 3))) & 0x1Fu;
      o[k] = ((sm[k] >> 10) << 15) | (e << 10) | (sm[k] & 0x3FFu);
    }
    const gdst dst = outb + 2 * e0;
    if (valid == 8) {
      store_out16(dst, make_uint4(o[0] | o[1] << 16, o[2] | o[3] << 16, o[4] | o[5] << 16,
                                  o[6] | o[7] << 16));
    } else if (valid) {
#pragma unroll
      for (uint32_t k = 0; k < 8; ++k)
        if (k < valid) stg<uint16_t>(dst + 2 * k, (uint16_t)o[k]);
    }
  }
}

// Schedule: workgroup b of a launch decodes tile tile0 + b, and a launch has
// at most kMaxGrid workgroups (larger inputs take several launches). The
// hardware dispatches workgroups in index order, round-robin over the XCDs,
// so the resident ones decode consecutive tiles and the whole device
// streams one contiguous region at a time. Measured on the 8B-shaped set
// with 8192-value tiles: 4.88 ms per decode, against 5.47 ms with a
// persistent grid of 65536
// workgroups that gave each XCD a contiguous eighth of the tiles (each XCD
// then streamed its own region, eight fronts at once), 5.26 ms for that
// split with one tile per workgroup, and 5.9-6.5 ms with a persistent grid
// of 2048-8192 workgroups stepping through the tiles in order. With the
// current 4096-value tiles, other orders of the same grid (the tile of
// workgroup b taken from b mod 8, the XCD, and b / 8) measured: each XCD a
// contiguous eighth of the tiles 4.83-5.01 ms, each of 2 or 4 XCD groups a
// contiguous half or quarter 4.75-4.88 ms, a tile's four quarters on four
// XCDs 6.4-6.7 ms, against 4.65-4.71 ms in order.
constexpr uint32_t kMaxGrid = 1u << 23;

// Workgroups per launch: kMaxGrid, or fewer when ENC_DECODE_MAX_GRID says
// so (lets tests run the several-launch path on small inputs).
uint32_t max_grid() {
  const char *v = getenv("ENC_DECODE_MAX_GRID");
  if (v && v[0]) {
    const unsigned long g = strtoul(v, nullptr, 10);
    if (g >= 1 && g < kMaxGrid) return (uint32_t)g;
  }
  return kMaxGrid;
}

__global__ __launch_bounds__(kThreads) void k_decode(DecodeDesc d, uint64_t tile0, uint64_t ntiles) {
  const uint64_t t = tile0 + blockIdx.x;
  if (t < ntiles) decode_tile(d, t, threadIdx.x);
}

template <uint32_t DT>
__global__ __launch_bounds__(kThreads) void k_decode_wide(DecodeDesc d, uint64_t tile0, uint64_t ntiles) {
  const uint64_t t = tile0 + blockIdx.x;
  if (t < ntiles) decode_tile_wide<DT>(d, t, threadIdx.x);
}

// The table holds two tile-prefix lists: BF16 items' tiles, then FP16 and
// FP32 items' tiles (an item has tiles in one list only). k_decode_batch
// covers the first, k_decode_batch_wide the second, each with one
// workgroup per tile; the host launches each only if its list has tiles.
// A workgroup reads its item's index from the table's per-tile map (one
// load; a binary search over the prefixes took eight dependent loads before
// any stream byte was requested: 4.77-4.90 ms per set decode against
// 4.67-4.68 with the map). Tiles beyond the table's own count (a launch
// sized from a stale plan) exit at once.
__global__ __launch_bounds__(kThreads) void k_decode_batch(const uint8_t *__restrict__ table,
                                                           uint64_t tile0) {
  const BatchHeader *h = reinterpret_cast<const BatchHeader *>(table);
  const uint64_t t = tile0 + blockIdx.x;
  if (t >= h->total_tiles) return;
  const DecodeDesc *items = reinterpret_cast<const DecodeDesc *>(table + sizeof(BatchHeader));
  const uint32_t count = h->count;
  const uint64_t *tile_begin =
      reinterpret_cast<const uint64_t *>(table + sizeof(BatchHeader) + count * sizeof(DecodeDesc));
  const uint32_t k = reinterpret_cast<const uint32_t *>(table + h->map_off)[t];
  const DecodeDesc d = items[k];
  decode_tile(d, t - tile_begin[k], threadIdx.x);
}

__global__ __launch_bounds__(kThreads) void k_decode_batch_wide(const uint8_t *__restrict__ table,
                                                                uint64_t tile0) {
  const BatchHeader *h = reinterpret_cast<const BatchHeader *>(table);
  const uint64_t t = tile0 + blockIdx.x;
  if (t >= h->wide_tiles) return;
  const DecodeDesc *items = reinterpret_cast<const DecodeDesc *>(table + sizeof(BatchHeader));
  const uint32_t count = h->count;
  const uint64_t *wide_begin = reinterpret_cast<const uint64_t *>(
                                   table + sizeof(BatchHeader) + count * sizeof(DecodeDesc)) + count + 1;
  const uint32_t k = reinterpret_cast<const uint32_t *>(table + h->wide_map_off)[t];
  const DecodeDesc d = items[k];
  if (d.dtype == 2)
    decode_tile_wide<2>(d, t - wide_begin[k], threadIdx.x);
  else
    decode_tile_wide<3>(d, t - wide_begin[k], threadIdx.x);
}

}  // namespace

hipError_t launch_decode(const DecodeDesc &d, hipStream_t s) {
  const uint64_t ntiles = decode_tiles_for(d.n, d.dtype);
  const uint32_t gmax = max_grid();
  for (uint64_t t0 = 0; t0 < ntiles; t0 += gmax) {
    const dim3 grid((uint32_t)(ntiles - t0 < gmax ? ntiles - t0 : gmax));
    if (d.dtype == 2)
      hipLaunchKernelGGL(k_decode_wide<2>, grid, dim3(kThreads), 0, s, d, t0, ntiles);
    else if (d.dtype == 3)
      hipLaunchKernelGGL(k_decode_wide<3>, grid, dim3(kThreads), 0, s, d, t0, ntiles);
    else
      hipLaunchKernelGGL(k_decode, grid, dim3(kThreads), 0, s, d, t0, ntiles);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_decode_batch(const void *table, uint64_t tiles, uint64_t wide_tiles, hipStream_t s) {
  const uint8_t *tb = reinterpret_cast<const uint8_t *>(table);
  const uint32_t gmax = max_grid();
  for (uint64_t t0 = 0; t0 < tiles; t0 += gmax) {
    const dim3 grid((uint32_t)(tiles - t0 < gmax ? tiles - t0 : gmax));
    hipLaunchKernelGGL(k_decode_batch, grid, dim3(kThreads), 0, s, tb, t0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  for (uint64_t t0 = 0; t0 < wide_tiles; t0 += gmax) {
    const dim3 grid((uint32_t)(wide_tiles - t0 < gmax ? wide_tiles - t0 : gmax));
    hipLaunchKernelGGL(k_decode_batch_wide, grid, dim3(kThreads), 0, s, tb, t0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace enc
