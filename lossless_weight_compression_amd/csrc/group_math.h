// group_math.h -- per-lane decode arithmetic of one 8-element group, shared
// by the decoder and the fused decompress-GEMM (device code only).
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

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, uint32_t lane) {
#pragma unroll
  for (uint32_t d = 1; d < 64; d <<= 1) {
    uint32_t t = __shfl_up(v, d, 64);
    if (lane >= d) v += t;
  }
  return v;
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
