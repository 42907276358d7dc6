// group_math.h -- per-lane decode arithmetic of one 8-element group, shared
// by the decoder and the fused decompress-GEMM, and the wave scan the
// decoder, the encoders and the deep check use (device code only).
//
// A group's 8 codes of w bits occupy exactly w bytes of its block payload,
// starting on a byte boundary (8 codes x w bits = w bytes). Packing is LSB
// first, so code k is bits [k*w, k*w + w) of that little-endian byte string
// ("ENEC: A Lossless AI Model Compression Method Enabling Fast Inference on
// Ascend NPUs", Abstract: fixed-length bit-packing at a per-block width).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace enc {

constexpr uint32_t kH8 = 0x80808080u;

// Inclusive prefix sum over the 64 lanes of a wave (all lanes active). The
// lane exchanges are DPP operand modifiers of the adds: shifts by 1, 2, 4
// and 8 inside each 16-lane row (a lane with no source adds 0), then row
// 0's total into row 1 and row 2's into row 3 (row broadcast of lane 15),
// then rows 0-1's total into rows 2 and 3 (row broadcast of lane 31). Six
// dependent VALU adds; the lane-shuffle form was six dependent LDS permutes.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);   // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);   // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);   // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);   // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);   // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);   // row_bcast:31
  return v;
}

// Lane-wise max of two pairs of 16-bit integers.
__device__ __forceinline__ uint32_t pmax16(uint32_t a, uint32_t b) {
  typedef unsigned short h2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(h2, a),
                                                                __builtin_bit_cast(h2, b)));
}

// Packed 16-bit max of `key` over each aligned run of `span` lanes (16, 32
// or 64; all lanes active), complete in the run's last lane. The lane
// exchanges are DPP operand modifiers: quad permutes (pairs, then quads),
// the half-row and row mirrors (8, then 16 lanes), then the row broadcasts
// of lane 15 into rows 1 and 3 (32 lanes) and of lane 31 into rows 2 and 3
// (64). With lane shuffles (LDS permutes) this reduction took 12% of the
// single-pass encoder's time.
__device__ __forceinline__ uint32_t span_max16(uint32_t key, uint32_t span) {
  key = pmax16(key, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)key, 0xB1, 0xF, 0xF, false));
  key = pmax16(key, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)key, 0x4E, 0xF, 0xF, false));
  key = pmax16(key, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)key, 0x141, 0xF, 0xF, false));
  key = pmax16(key, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)key, 0x140, 0xF, 0xF, false));
  if (span >= 32)
    key = pmax16(key, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)key, 0x142, 0xA, 0xF, false));
  if (span >= 64)
    key = pmax16(key, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)key, 0x143, 0xC, 0xF, false));
  return key;
}

__device__ __forceinline__ uint32_t ld32(const uint8_t *p) {
  return *reinterpret_cast<const uint32_t *>(p);
}

// Eight w-bit codes (LSB first, starting at bit 0 of lo:hi) -> eight code
// bytes: byte k of el (k < 4) / eh (k >= 4) is code k.
__device__ __forceinline__ void codes_to_bytes(uint32_t lo, uint32_t hi, uint32_t w, uint32_t &el,
                                               uint32_t &eh) {
  const uint32_t mid = (uint32_t)((((uint64_t)hi << 32) | lo) >> (4 * w));
  const uint32_t w2 = w + w, w3 = w2 + w;
  el = __builtin_amdgcn_ubfe(lo, 0, w);
  el |= __builtin_amdgcn_ubfe(lo, w, w) << 8;
  el |= __builtin_amdgcn_ubfe(lo, w2, w) << 16;
  el |= __builtin_amdgcn_ubfe(lo, w3, w) << 24;
  eh = __builtin_amdgcn_ubfe(mid, 0, w);
  eh |= __builtin_amdgcn_ubfe(mid, w, w) << 8;
  eh |= __builtin_amdgcn_ubfe(mid, w2, w) << 16;
  eh |= __builtin_amdgcn_ubfe(mid, w3, w) << 24;
}

// The same for w == 4 (the width of most blocks of Gaussian-like weights at
// B >= 512): the eight nibbles of one dword are split into even and odd
// nibbles and interleaved with two v_perm -- 5 operations instead of 14.
__device__ __forceinline__ void codes_to_bytes_w4(uint32_t lo, uint32_t &el, uint32_t &eh) {
  const uint32_t ev = lo & 0x0F0F0F0Fu;          // bytes: codes 0, 2, 4, 6
  const uint32_t od = (lo >> 4) & 0x0F0F0F0Fu;   // bytes: codes 1, 3, 5, 7
  el = __builtin_amdgcn_perm(od, ev, 0x05010400u);
  eh = __builtin_amdgcn_perm(od, ev, 0x07030602u);
}

// Exponent bytes (code + block base; a valid stream never carries out of a
// byte) joined with eight sign+mantissa bytes into eight BF16 values
// (4 dwords, element 0 in the low half of .x). BF16 = sign | exponent << 7 |
// mantissa: high byte = sign | e >> 1, low byte = (e & 1) << 7 | mantissa.
__device__ __forceinline__ uint4 bytes_to_bf16(uint32_t el, uint32_t eh, uint32_t base4,
                                               uint32_t sml, uint32_t smh) {
  el += base4;
  eh += base4;
  const uint32_t hl = (sml & kH8) | ((el >> 1) & ~kH8);
  const uint32_t ll = ((el << 7) & kH8) | (sml & ~kH8);
  const uint32_t hh = (smh & kH8) | ((eh >> 1) & ~kH8);
  const uint32_t lh = ((eh << 7) & kH8) | (smh & ~kH8);
  uint4 o;
  o.x = __builtin_amdgcn_perm(hl, ll, 0x05010400u);
  o.y = __builtin_amdgcn_perm(hl, ll, 0x07030602u);
  o.z = __builtin_amdgcn_perm(hh, lh, 0x05010400u);
  o.w = __builtin_amdgcn_perm(hh, lh, 0x07030602u);
  return o;
}

// Eight w-bit codes at bit 0 of lo:hi -> eight BF16 values.
__device__ __forceinline__ uint4 join_group(uint32_t lo, uint32_t hi, uint32_t w, uint32_t base4,
                                            uint32_t sml, uint32_t smh) {
  uint32_t el, eh;
  codes_to_bytes(lo, hi, w, el, eh);
  return bytes_to_bf16(el, eh, base4, sml, smh);
}

// Payload dwords of a group whose code bytes start at byte pb of the stream
// and span nbytes (0..8) bytes: only dwords holding a needed byte are read;
// otherwise the lane re-reads `fallback` (an address it reads anyway), so no
// access leaves [0, stream size) -- branch-free. Returns the 64 code bits
// aligned to bit 0 in lo:hi.
__device__ __forceinline__ void load_codes(const uint8_t *__restrict__ s, uint64_t pb,
                                           uint32_t nbytes, uint64_t fallback, uint32_t &q0,
                                           uint32_t &q1, uint32_t &q2, uint32_t &lead) {
  const uint64_t a = pb & ~3ull;
  lead = (uint32_t)(pb & 3);
  const uint64_t a0 = nbytes ? a : fallback;
  const uint64_t a1 = (lead + nbytes > 4) ? a + 4 : a0;
  const uint64_t a2 = (lead + nbytes > 8) ? a + 8 : a0;
  q0 = ld32(s + a0);
  q1 = ld32(s + a1);
  q2 = ld32(s + a2);
}

__device__ __forceinline__ void align_codes(uint32_t q0, uint32_t q1, uint32_t q2, uint32_t lead,
                                            uint32_t &lo, uint32_t &hi) {
  lo = __builtin_amdgcn_alignbit(q1, q0, lead * 8);
  hi = __builtin_amdgcn_alignbit(q2, q1, lead * 8);
}

}  // namespace enc
