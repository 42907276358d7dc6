// validate.hip -- deep check of a coded stream on the device.
//
// A coded stream is usable only if (1) every block width is at most 8 (and
// a power of two in a stream that declares power-of-two widths),
// (2) the stored segment offsets are the exclusive prefix sums of the padded
// block payload sizes (and payload_bytes is their total), and (3) every
// decoded exponent base + code fits the element type's exponent field (255
// for BF16 and FP32, 31 for FP16). Condition (2) is what lets a
// decoder locate any block from its segment offset and an intra-segment scan
// ("ENEC: A Lossless AI Model Compression Method Enabling Fast Inference on
// Ascend NPUs", Abstract: intra-segment prefix scan of block sizes); (3) is
// implied by the branch-free transform d = exponent - base with base the
// block minimum (same Abstract). The header itself is checked on the host.
//
// One wave per segment, lane j = block 64s + j:
//  * width:   w_j > 8, or not a power of two in a flag-2 stream;
//  * offsets: stored[s+1] - stored[s] must equal the wave's sum of padded
//             sizes (stored[nseg] means payload_bytes) and stored[0] must be
//             0. If stored[0..k) are right and stored[k] is not, the first
//             failing difference is at s = k - 1, so reporting s + 1 yields
//             the first wrong offset, k, as the minimum over all waves;
//  * exponent: only lanes whose base + 2^w - 1 can exceed the maximum read
//             their codes (never, for streams the encoders write), and only
//             when the segment's payload range lies inside the payload
//             section, so every read stays in bounds; a width-0 block fails
//             on its base alone, without a read.
// Failures are reported with one 64-bit atomic minimum per failing lane into
// result[kind] (initialised to all ones by the host).
#include "enc_common.h"
#include "group_math.h"

namespace enc {

__global__ __launch_bounds__(kThreads) void k_validate(ValidateArgs a) {
  const uint32_t lane = threadIdx.x & 63;
  const uint64_t waves = (uint64_t)gridDim.x * (kThreads / 64);
  const uint8_t *__restrict__ s = a.stream;
  for (uint64_t seg = (uint64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6); seg < a.nseg;
       seg += waves) {
    const uint64_t blk = (seg << 6) + lane;
    const bool valid = blk < a.nb;
    uint32_t base = 0, w = 0, L = 0, P = 0;
    if (valid) {
      base = s[a.meta_off + 2 * blk];
      w = s[a.meta_off + 2 * blk + 1];
      L = (blk + 1 == a.nb) ? (uint32_t)(a.n - ((a.nb - 1) << a.log2b)) : (1u << a.log2b);
      P = (((w * L + 7) >> 3) + 15) & ~15u;   // w <= 255: fits easily in 32 bits
    }
    if (valid && (w > 8 || (a.pow2 && (w & (w - 1)))))
      atomicMin(&a.result[0], (unsigned long long)blk);

    const uint32_t incl = wave_incl_scan(P);
    const uint32_t seg_sum = __builtin_amdgcn_readlane(incl, 63);
    const uint64_t so = *reinterpret_cast<const uint64_t *>(s + a.segoff_off + 8 * seg);
    const uint64_t next = seg + 1 < a.nseg
                              ? *reinterpret_cast<const uint64_t *>(s + a.segoff_off + 8 * (seg + 1))
                              : a.payload_bytes;
    if (lane == 0) {
      if (seg == 0 && so != 0) atomicMin(&a.result[1], 0ull);
      if (next - so != seg_sum) atomicMin(&a.result[1], (unsigned long long)(seg + 1));
    }

    const bool inside = so <= a.payload_bytes && seg_sum <= a.payload_bytes - so;
    if (valid && w == 0 && base > a.emax) atomicMin(&a.result[2], (unsigned long long)blk);
    if (valid && inside && w >= 1 && w <= 8 && base + (1u << w) - 1 > a.emax) {
      const uint8_t *q = s + a.payload_off + so + (incl - P);
      for (uint32_t t = 0; t < L; ++t) {
        const uint32_t bit = t * w, byte = bit >> 3, sh = bit & 7;
        uint32_t v = q[byte];
        if (sh + w > 8) v |= (uint32_t)q[byte + 1] << 8;   // the field's bits end in that byte
        const uint32_t d = (v >> sh) & ((1u << w) - 1);
        if (base + d > a.emax) {
          atomicMin(&a.result[2], (unsigned long long)blk);
          break;
        }
      }
    }
  }
}

hipError_t launch_validate(const ValidateArgs &a, hipStream_t s) {
  if (a.nseg == 0) return hipSuccess;
  const uint64_t wgs = (a.nseg + 3) / 4;
  hipLaunchKernelGGL(k_validate, dim3((uint32_t)(wgs < 8192 ? wgs : 8192)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace enc
