// probe.hip -- a streaming kernel with the decoder's access shape, used to
// measure the HBM rate a kernel of that shape reaches on the device at hand
// (the ceiling the decoder's bandwidth is compared with).
//
// Decoding moves the stream (about 1.51 bytes per value) into the output
// (2 bytes per value). This kernel does the same with no decoding: workgroup
// b (of `threads` threads) writes the b-th run of the output, `items` 16-byte
// items per thread (non-temporal stores, as the decoder's), and reads the
// b-th proportional run of the source (16-byte loads). Lanes with no source item of their own
// re-read one of the run (a cache hit, no extra HBM bytes), so every store
// depends on a load and nothing is optimised away. Workgroups are launched in
// index order, one per run, as the decoder's tiles are.
#include "enc_common.h"

namespace enc {
namespace {

template <uint32_t ITEMS>
__global__ __launch_bounds__(256) void k_stream_probe(const uint4 *__restrict__ src, uint64_t src_items,
                                                      uint4 *__restrict__ dst, uint64_t dst_items,
                                                      uint64_t wg0, uint64_t ratio_q32) {
  const uint64_t b = wg0 + blockIdx.x;
  const uint32_t T = blockDim.x;
  const uint64_t d0 = b * T * ITEMS;
  // source run of this workgroup: [s0, s1), s = floor(b * src_items / workgroups)
  // through the host's 32.32 fixed-point ratio (no division per workgroup)
  const uint64_t s0 = (b * ratio_q32) >> 32;
  const uint64_t s1 = ((b + 1) * ratio_q32) >> 32;
  const uint32_t ns = s1 > s0 ? (uint32_t)(s1 - s0) : 1u;
  uint4 v[ITEMS];
#pragma unroll
  for (uint32_t i = 0; i < ITEMS; ++i) {
    const uint32_t j = threadIdx.x + T * i;
    const uint32_t jj = j < ns ? j : (j - ns < ns ? j - ns : j % ns);
    const uint64_t s = s0 + jj;
    v[i] = s < src_items ? src[s] : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (uint32_t i = 0; i < ITEMS; ++i) {
    const uint64_t d = d0 + threadIdx.x + (uint64_t)T * i;
    if (d < dst_items) store_nt16(dst + d, v[i]);
  }
}

}  // namespace

hipError_t launch_stream_probe(const void *src, uint64_t src_bytes, void *dst, uint64_t dst_bytes,
                               uint32_t items, uint32_t threads, hipStream_t s) {
  const uint64_t si = src_bytes / 16, di = dst_bytes / 16;
  const uint64_t per = (uint64_t)threads * items;
  const uint64_t nwg = (di + per - 1) / per;
  const uint64_t ratio_q32 = (uint64_t)(((unsigned __int128)si << 32) / nwg);
  const uint64_t kMaxGrid = (1ull << 30) / threads;   // workgroups per launch (work items < 2^31)
  for (uint64_t w0 = 0; w0 < nwg; w0 += kMaxGrid) {
    const uint32_t g = (uint32_t)(nwg - w0 < kMaxGrid ? nwg - w0 : kMaxGrid);
    const uint4 *sp = static_cast<const uint4 *>(src);
    uint4 *dp = static_cast<uint4 *>(dst);
    switch (items) {
      case 1: hipLaunchKernelGGL(k_stream_probe<1>, dim3(g), dim3(threads), 0, s, sp, si, dp, di, w0, ratio_q32); break;
      case 2: hipLaunchKernelGGL(k_stream_probe<2>, dim3(g), dim3(threads), 0, s, sp, si, dp, di, w0, ratio_q32); break;
      case 4: hipLaunchKernelGGL(k_stream_probe<4>, dim3(g), dim3(threads), 0, s, sp, si, dp, di, w0, ratio_q32); break;
      default: return hipErrorInvalidValue;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace enc
