// encode_wide.hip -- gfx950 encoder for FP16 and FP32 streams (header dtype
// 2 and 3).
//
// "ENEC: A Lossless AI Model Compression Method Enabling Fast Inference on
// Ascend NPUs", Abstract: the same block code as for BF16 -- per-block base
// and minimal width for the exponent field, bit-packed codes, an
// intra-segment prefix scan of block sizes -- applied to the other float
// layouts: FP16 (5 exponent bits; sign and 10 mantissa bits kept as an
// 11-bit field) and FP32 (8 exponent bits; sign and 23 mantissa bits kept as
// a 24-bit field). The kept fields are packed LSB first, so a group of 8
// values owns exactly 11 or 24 bytes of that section.
//
// Passes, as in the two-pass BF16 encoder: k_encw_params (block widths and
// segment totals), the shared segment scan, k_encw_pack (one 1024-group
// tile per workgroup iteration: the tile's codes and kept fields are
// assembled in zeroed LDS images and written out with 16-byte stores) and
// k_encw_finish (header, metas, offsets, section padding). The single-pass
// kernels of encode_onepass.hip write the same streams and serve FP16 and
// FP32 too; these passes run when the output buffer is smaller than the RAW
// size (the single pass writes in place up to it) or a look-back wait gave
// up.
#include "enc_common.h"
#include "group_math.h"

namespace enc {
namespace {

template <uint32_t DT>
struct Wide;
template <>
struct Wide<2> {   // FP16: s eeeee mmmmmmmmmm
  static constexpr uint32_t kBytes = 2, kSmBits = 11, kShift = 10, kExpMask = 0x1Fu;
};
template <>
struct Wide<3> {   // FP32: s eeeeeeee m x 23
  static constexpr uint32_t kBytes = 4, kSmBits = 24, kShift = 23, kExpMask = 0xFFu;
};

// The `valid` values of the group starting at element e0 (the rest read as 0
// and are never used).
template <uint32_t DT>
__device__ __forceinline__ void load_values(const uint8_t *__restrict__ in, uint64_t e0,
                                            uint32_t valid, uint32_t (&x)[8]) {
  if (DT == 3) {
    const uint32_t *p = reinterpret_cast<const uint32_t *>(in) + e0;
    if (valid == 8) {
      const uint4 a = reinterpret_cast<const uint4 *>(p)[0], b = reinterpret_cast<const uint4 *>(p)[1];
      x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
      x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    } else {
#pragma unroll
      for (uint32_t k = 0; k < 8; ++k) x[k] = k < valid ? p[k] : 0u;
    }
  } else {
    const uint16_t *p = reinterpret_cast<const uint16_t *>(in) + e0;
    if (valid == 8) {
      const uint4 a = *reinterpret_cast<const uint4 *>(p);
      const uint32_t wd[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
      for (uint32_t k = 0; k < 8; ++k) x[k] = (wd[k >> 1] >> (16 * (k & 1))) & 0xFFFFu;
    } else {
#pragma unroll
      for (uint32_t k = 0; k < 8; ++k) x[k] = k < valid ? (uint32_t)p[k] : 0u;
    }
  }
}

template <uint32_t DT>
__device__ __forceinline__ uint32_t exponent_of(uint32_t x) {
  return (x >> Wide<DT>::kShift) & Wide<DT>::kExpMask;
}

// Sign on top of the mantissa: the kept field of a value.
template <uint32_t DT>
__device__ __forceinline__ uint32_t kept_field(uint32_t x) {
  constexpr uint32_t top = Wide<DT>::kBytes * 8 - 1;
  return ((x >> top) << Wide<DT>::kShift) | (x & ((1u << Wide<DT>::kShift) - 1));
}

template <uint32_t DT>
__global__ __launch_bounds__(kThreads) void k_encw_params(EncodeArgs a) {
  __shared__ uint32_t smin[kSegBlocks], smax[kSegBlocks];
  const uint32_t tid = threadIdx.x;
  const uint64_t seg = blockIdx.x;
  const uint8_t *in = reinterpret_cast<const uint8_t *>(a.in);
  if (tid < kSegBlocks) {
    smin[tid] = 255;
    smax[tid] = 0;
  }
  __syncthreads();
  const uint32_t log2gpb = a.log2b - 3;
  const uint32_t gps = 1u << (log2gpb + 6);
  const uint64_t gseg = seg * gps;
  // As in the BF16 parameter pass: whole waves run every round, the lanes of
  // a block reduce with span_max16, one lane per block and wave updates LDS.
  const uint32_t span = log2gpb < 6 ? (1u << log2gpb) : 64u;
  for (uint32_t q0 = 0; q0 < gps && (gseg + q0) * 8 < a.n; q0 += kThreads) {
    const uint32_t q = q0 + tid;
    const uint64_t e0 = (gseg + q) * 8;
    const uint32_t valid = e0 < a.n ? (a.n - e0 < 8 ? (uint32_t)(a.n - e0) : 8u) : 0u;
    uint32_t x[8];
    load_values<DT>(in, e0, valid, x);
    uint32_t mn = 255, mx = 0;
#pragma unroll
    for (uint32_t k = 0; k < 8; ++k) {
      const uint32_t e = exponent_of<DT>(x[k]);
      mn = k < valid && e < mn ? e : mn;
      mx = k < valid && e > mx ? e : mx;
    }
    const uint32_t key = span_max16(((255u - mn) << 16) | mx, span);
    if ((tid & (span - 1)) == span - 1 && key != 0) {
      atomicMin(&smin[q >> log2gpb], 255u - (key >> 16));
      atomicMax(&smax[q >> log2gpb], key & 0xFFFFu);
    }
  }
  __syncthreads();
  if (tid < kSegBlocks) {
    const uint64_t blk = seg * kSegBlocks + tid;
    uint32_t P = 0;
    if (blk < a.nb) {
      const uint32_t base = smin[tid];
      const uint32_t w = block_width(smax[tid] - base, a.pow2);
      const uint32_t L = (blk + 1 == a.nb) ? (uint32_t)(a.n - ((a.nb - 1) << a.log2b)) : (1u << a.log2b);
      P = (((w * L + 7) >> 3) + 15) & ~15u;
      *reinterpret_cast<uint16_t *>(a.ws_meta + 2 * blk) = (uint16_t)(base | (w << 8));
    }
    const uint32_t tot = wave_incl_scan(P);
    if (tid == kSegBlocks - 1) a.ws_segsum[seg] = tot;
  }
}

template <uint32_t DT>
__global__ __launch_bounds__(kThreads) void k_encw_pack(EncodeArgs a, uint64_t ntiles) {
  constexpr uint32_t S = Wide<DT>::kSmBits;
  constexpr uint32_t kTileSm = kTileGroups * S;               // bytes of kept fields per tile
  __shared__ uint32_t pay[kTileGroups * 2];                    // codes: at most 8 bytes per group
  __shared__ uint32_t smi[kTileSm / 4 + 1];                   // + the dword a last group may touch
  uint8_t *payb = reinterpret_cast<uint8_t *>(pay);
  const uint8_t *in = reinterpret_cast<const uint8_t *>(a.in);
  const uint32_t tid = threadIdx.x, lane = tid & 63;
  const uint32_t log2gpb = a.log2b - 3, log2gps = log2gpb + 6;
  const uint64_t ngroups = (a.n + 7) / 8;
  const uint64_t sm_total = (S * a.n + 7) / 8;
  for (uint64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const uint64_t g0 = tile * kTileGroups;
    const uint64_t seg = g0 >> log2gps;
    const uint32_t gs0 = (uint32_t)(g0 & ((1ull << log2gps) - 1));
    const uint64_t blk = (seg << 6) + lane;
    uint32_t P = 0, pk = 0;
    if (blk < a.nb) {
      const uint32_t m = *reinterpret_cast<const uint16_t *>(a.ws_meta + 2 * blk);
      const uint32_t w = m >> 8;
      const uint32_t L = (blk + 1 == a.nb) ? (uint32_t)(a.n - ((a.nb - 1) << a.log2b)) : (1u << a.log2b);
      P = (((w * L + 7) >> 3) + 15) & ~15u;
      pk = ((m & 0xFFu) << 24) | (w << 20);
    }
    const uint32_t incl = wave_incl_scan(P);
    pk |= incl - P;
    const uint64_t glast = (g0 + kTileGroups < ngroups ? g0 + kTileGroups : ngroups) - 1;
    const uint32_t jb0 = gs0 >> log2gpb;
    const uint32_t jb1 = (uint32_t)(glast - (g0 - gs0)) >> log2gpb;
    const uint32_t tstart = __shfl(pk, (int)jb0, 64) & 0xFFFFFu;
    const uint32_t tbytes = __shfl(incl, (int)jb1, 64) - tstart;   // multiple of 16, <= 8192
    for (uint32_t i = tid; i < tbytes / 4; i += kThreads) pay[i] = 0;
    for (uint32_t i = tid; i < kTileSm / 4; i += kThreads) smi[i] = 0;
    __syncthreads();
    for (uint32_t it = 0; it < kGroupsPerThread; ++it) {
      const uint32_t q = it * kThreads + tid;
      const uint32_t gs = gs0 + q;
      const uint32_t p = __shfl(pk, (int)(gs >> log2gpb), 64);   // with every lane active
      const uint64_t e0 = (g0 + q) * 8;
      if (e0 >= a.n) continue;
      const uint64_t rem = a.n - e0;
      const uint32_t valid = rem < 8 ? (uint32_t)rem : 8u;
      uint32_t x[8];
      load_values<DT>(in, e0, valid, x);
      const uint32_t base = p >> 24, w = (p >> 20) & 15u;
      uint32_t f[8];
      unsigned long long codes = 0;
#pragma unroll
      for (uint32_t k = 0; k < 8; ++k) {
        f[k] = k < valid ? kept_field<DT>(x[k]) : 0u;
        if (k < valid) codes |= (unsigned long long)(exponent_of<DT>(x[k]) - base) << (k * w);
      }
      if (DT == 3) {
        // 24 bytes at byte 24 q: six whole dwords, this lane's alone
        uint32_t *d = smi + 6 * q;
        d[0] = f[0] | f[1] << 24;
        d[1] = f[1] >> 8 | f[2] << 16;
        d[2] = f[2] >> 16 | f[3] << 8;
        d[3] = f[4] | f[5] << 24;
        d[4] = f[5] >> 8 | f[6] << 16;
        d[5] = f[6] >> 16 | f[7] << 8;
      } else {
        // 88 bits at bit 88 q: OR-ed into the four dwords they can touch
        // (the first and last are shared with the neighbouring groups)
        const unsigned long long lo = (unsigned long long)f[0] | (unsigned long long)f[1] << 11 |
                                      (unsigned long long)f[2] << 22 | (unsigned long long)f[3] << 33 |
                                      (unsigned long long)f[4] << 44 | (unsigned long long)f[5] << 55;
        const uint32_t hi = f[5] >> 9 | f[6] << 2 | f[7] << 13;   // bits 64..87
        const uint32_t v0 = (uint32_t)lo, v1 = (uint32_t)(lo >> 32), v2 = hi;
        const uint32_t bit = 88 * q, d0 = bit >> 5, sh = bit & 31;   // sh is 0, 8, 16 or 24
        const uint32_t w0 = v0 << sh;
        const uint32_t w1 = sh ? (v0 >> (32 - sh)) | (v1 << sh) : v1;
        const uint32_t w2 = sh ? (v1 >> (32 - sh)) | (v2 << sh) : v2;
        const uint32_t w3 = sh ? v2 >> (32 - sh) : 0u;
        if (w0) atomicOr(&smi[d0], w0);
        if (w1) atomicOr(&smi[d0 + 1], w1);
        if (w2) atomicOr(&smi[d0 + 2], w2);
        if (w3) atomicOr(&smi[d0 + 3], w3);
      }
      const uint32_t u = gs & ((1u << log2gpb) - 1);
      const uint32_t pos = (p & 0xFFFFFu) - tstart + u * w;
      const uint32_t nbytes = (valid * w + 7) >> 3;
      for (uint32_t b = 0; b < nbytes; ++b) payb[pos + b] = (uint8_t)(codes >> (8 * b));
    }
    __syncthreads();
    uint8_t *dst = a.out + a.payload_off + a.ws_segsum[seg] + tstart;
    for (uint32_t i = tid; i < tbytes / 16; i += kThreads)
      store_nt16(dst + 16 * i, reinterpret_cast<const uint4 *>(pay)[i]);
    // kept fields: the tile's bytes start 16-byte aligned (1024 S is a
    // multiple of 16); bytes past the section's last field are not written
    const uint64_t sm0 = (uint64_t)kTileSm * tile;
    const uint32_t len = (uint32_t)(sm_total - sm0 < kTileSm ? sm_total - sm0 : kTileSm);
    uint8_t *sdst = a.out + kHeaderBytes + sm0;
    for (uint32_t i = tid; i < len / 16; i += kThreads)
      store_nt16(sdst + 16 * i, reinterpret_cast<const uint4 *>(smi)[i]);
    if (tid < (len & 15)) {
      const uint32_t b = (len & ~15u) + tid;
      sdst[b] = reinterpret_cast<const uint8_t *>(smi)[b];
    }
    __syncthreads();
  }
}

template <uint32_t DT>
__global__ __launch_bounds__(kThreads) void k_encw_finish(EncodeArgs a, HeaderImage h) {
  const uint64_t tid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  if (tid < 64) reinterpret_cast<uint32_t *>(a.out)[tid] = reinterpret_cast<const uint32_t *>(h.bytes)[tid];
  const uint64_t meta_bytes = align_up(2 * a.nb, kSectionAlign);
  for (uint64_t i = tid; i < meta_bytes; i += stride)
    a.out[a.meta_off + i] = i < 2 * a.nb ? a.ws_meta[i] : 0;
  const uint64_t seg_words = align_up(8 * a.nseg, kSectionAlign) / 8;
  for (uint64_t i = tid; i < seg_words; i += stride)
    reinterpret_cast<uint64_t *>(a.out + a.segoff_off)[i] = i < a.nseg ? a.ws_segsum[i] : 0;
  const uint64_t sm_end = kHeaderBytes + (Wide<DT>::kSmBits * a.n + 7) / 8;
  for (uint64_t i = sm_end + tid; i < a.meta_off; i += stride) a.out[i] = 0;
}

uint32_t grid_for(uint64_t items, uint64_t per_block, uint32_t cap) {
  const uint64_t g = (items + per_block - 1) / per_block;
  return (uint32_t)(g < 1 ? 1 : (g > cap ? cap : g));
}

}  // namespace

hipError_t launch_encode_wide_params(const EncodeArgs &a, uint32_t dtype, hipStream_t s) {
  if (dtype == 2)
    hipLaunchKernelGGL(k_encw_params<2>, dim3((uint32_t)a.nseg), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(k_encw_params<3>, dim3((uint32_t)a.nseg), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_encode_wide_pack(const EncodeArgs &a, uint32_t dtype, hipStream_t s) {
  const uint64_t ntiles = tiles_for(a.n);
  const dim3 grid(grid_for(ntiles, 1, 2048));
  if (dtype == 2)
    hipLaunchKernelGGL(k_encw_pack<2>, grid, dim3(kThreads), 0, s, a, ntiles);
  else
    hipLaunchKernelGGL(k_encw_pack<3>, grid, dim3(kThreads), 0, s, a, ntiles);
  return hipGetLastError();
}

hipError_t launch_encode_wide_finish(const EncodeArgs &a, uint32_t dtype, const HeaderImage &h,
                                     hipStream_t s) {
  const uint64_t work = align_up(2 * a.nb, kSectionAlign) + a.nseg + kSectionAlign;
  const dim3 grid(grid_for(work, kThreads, 1024));
  if (dtype == 2)
    hipLaunchKernelGGL(k_encw_finish<2>, grid, dim3(kThreads), 0, s, a, h);
  else
    hipLaunchKernelGGL(k_encw_finish<3>, grid, dim3(kThreads), 0, s, a, h);
  return hipGetLastError();
}

}  // namespace enc
