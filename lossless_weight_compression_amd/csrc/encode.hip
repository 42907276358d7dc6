// encode.hip -- gfx950 encoder for the block-based fixed-length BF16 stream.
//
// "ENEC: A Lossless AI Model Compression Method Enabling Fast Inference on
// Ascend NPUs", Abstract: per-block bit width ("bit-width quantization"),
// bit-packing, a branch-free integer transform and an intra-segment prefix
// scan of block sizes. Three passes:
//  1. k_enc_params  one workgroup per 64-block segment: exponent min/max per
//                   block (LDS atomics), base and width, padded payload size,
//                   and the segment's payload total;
//  2. k_enc_scan    one workgroup: exclusive scan of the segment totals
//                   (64-bit, deterministic) -> segment offsets and the stream's
//                   payload size, which the host reads back to decide RAW;
//  3. k_enc_pack    per 1024-group tile, like the decoder: a wave scan of the
//                   segment's block sizes places every group's w code bytes;
//                   the tile's payload is assembled in LDS (zeroed, so pad
//                   bits are zero) and written out with 16-byte stores; the
//                   sign+mantissa plane is written directly;
//  4. k_enc_finish  header, meta and segment-offset sections, section padding.
// The bytes are exactly those the format definition prescribes (the stream
// is unique for a given input and block size).
#include "enc_common.h"
#include "group_math.h"

namespace enc {
namespace {

__device__ __forceinline__ unsigned long long wave_incl_scan64(unsigned long long v, uint32_t lane) {
#pragma unroll
  for (uint32_t d = 1; d < 64; d <<= 1) {
    unsigned long long t = __shfl_up(v, d, 64);
    if (lane >= d) v += t;
  }
  return v;
}

__device__ __forceinline__ uint32_t exp_of(uint32_t word, uint32_t half) {
  return (word >> (7 + 16 * half)) & 0xFFu;
}

// Loads group e0 (valid elements; the rest read as 0) as 4 dwords.
__device__ __forceinline__ uint4 load_group(const uint16_t *__restrict__ in, uint64_t e0,
                                            uint32_t valid) {
  if (valid == 8) return *reinterpret_cast<const uint4 *>(in + e0);
  uint32_t v[4] = {0, 0, 0, 0};
  for (uint32_t k = 0; k < valid; ++k) v[k >> 1] |= (uint32_t)in[e0 + k] << (16 * (k & 1));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__global__ __launch_bounds__(kThreads) void k_enc_params(EncodeArgs a) {
  __shared__ uint32_t smin[kSegBlocks], smax[kSegBlocks];
  const uint32_t tid = threadIdx.x;
  const uint64_t seg = blockIdx.x;
  if (tid < kSegBlocks) {
    smin[tid] = 255;
    smax[tid] = 0;
  }
  __syncthreads();
  const uint32_t log2gpb = a.log2b - 3;
  const uint32_t gps = 1u << (log2gpb + 6);
  const uint64_t gseg = seg * gps;
  // Every lane of a wave runs every round (the lane exchanges of span_max16
  // need them all); lanes past the end hold no value (key 0). The lanes of
  // one block reduce ((255 - min) << 16 | max) first, so one lane per block
  // and wave updates LDS (a per-lane atomic on one address serialises).
  const uint32_t span = log2gpb < 6 ? (1u << log2gpb) : 64u;
  for (uint32_t q0 = 0; q0 < gps && (gseg + q0) * 8 < a.n; q0 += kThreads) {
    const uint32_t q = q0 + tid;
    const uint64_t e0 = (gseg + q) * 8;
    const uint32_t valid = e0 < a.n ? (a.n - e0 < 8 ? (uint32_t)(a.n - e0) : 8u) : 0u;
    const uint4 g = load_group(a.in, e0, valid);
    const uint32_t words[4] = {g.x, g.y, g.z, g.w};
    uint32_t mn = 255, mx = 0;
    for (uint32_t k = 0; k < valid; ++k) {
      const uint32_t e = exp_of(words[k >> 1], k & 1);
      mn = e < mn ? e : mn;
      mx = e > mx ? e : mx;
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
      const uint32_t r = smax[tid] - base;
      const uint32_t w = block_width(r, a.pow2);
      const uint32_t L = (blk + 1 == a.nb) ? (uint32_t)(a.n - ((a.nb - 1) << a.log2b)) : (1u << a.log2b);
      P = (((w * L + 7) >> 3) + 15) & ~15u;
      *reinterpret_cast<uint16_t *>(a.ws_meta + 2 * blk) = (uint16_t)(base | (w << 8));
    }
    const uint32_t tot = wave_incl_scan(P);
    if (tid == kSegBlocks - 1) a.ws_segsum[seg] = tot;
  }
}

__global__ __launch_bounds__(1024) void k_enc_scan(EncodeArgs a) {
  __shared__ unsigned long long wsum[16];
  const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  unsigned long long carry = 0;
  for (uint64_t base = 0; base < a.nseg; base += 1024) {
    const uint64_t i = base + tid;
    const unsigned long long v = i < a.nseg ? a.ws_segsum[i] : 0ull;
    const unsigned long long incl = wave_incl_scan64(v, lane);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    unsigned long long before = 0, chunk = 0;
    for (uint32_t w = 0; w < 16; ++w) {
      before += w < wave ? wsum[w] : 0ull;
      chunk += wsum[w];
    }
    if (i < a.nseg) a.ws_segsum[i] = carry + before + incl - v;
    carry += chunk;
    __syncthreads();
  }
  if (tid == 0) *a.ws_total = carry;
}

__global__ __launch_bounds__(kThreads) void k_enc_pack(EncodeArgs a, uint64_t ntiles) {
  __shared__ uint32_t lds[kTileGroups * 2];   // tile payload, at most 8 bytes per group
  uint8_t *ldsb = reinterpret_cast<uint8_t *>(lds);
  const uint32_t tid = threadIdx.x, lane = tid & 63;
  const uint32_t log2gpb = a.log2b - 3, log2gps = log2gpb + 6;
  const uint64_t ngroups = (a.n + 7) / 8;
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
    const uint32_t tend = __shfl(incl, (int)jb1, 64);
    const uint32_t tbytes = tend - tstart;    // multiple of 16, <= 8192
    for (uint32_t i = tid; i < tbytes / 4; i += kThreads) lds[i] = 0;
    __syncthreads();
    for (uint32_t it = 0; it < kGroupsPerThread; ++it) {
      const uint32_t q = it * kThreads + tid;
      const uint32_t gs = gs0 + q;
      const uint32_t p = __shfl(pk, (int)(gs >> log2gpb), 64);
      const uint64_t e0 = (g0 + q) * 8;
      if (e0 >= a.n) continue;
      const uint64_t rem = a.n - e0;
      const uint32_t valid = rem < 8 ? (uint32_t)rem : 8u;
      const uint4 g = load_group(a.in, e0, valid);
      const uint32_t words[4] = {g.x, g.y, g.z, g.w};
      const uint32_t base = p >> 24, w = (p >> 20) & 15u;
      uint32_t sm[2] = {0, 0};
      unsigned long long codes = 0;
      for (uint32_t k = 0; k < valid; ++k) {
        const uint32_t x = (words[k >> 1] >> (16 * (k & 1))) & 0xFFFFu;
        const uint32_t smb = ((x >> 8) & 0x80u) | (x & 0x7Fu);
        sm[k >> 2] |= smb << (8 * (k & 3));
        codes |= (unsigned long long)(((x >> 7) & 0xFFu) - base) << (k * w);
      }
      *reinterpret_cast<uint2 *>(a.out + kHeaderBytes + e0) = make_uint2(sm[0], sm[1]);
      const uint32_t u = gs & ((1u << log2gpb) - 1);
      const uint32_t pos = (p & 0xFFFFFu) - tstart + u * w;
      const uint32_t nbytes = (valid * w + 7) >> 3;
      for (uint32_t b = 0; b < nbytes; ++b) ldsb[pos + b] = (uint8_t)(codes >> (8 * b));
    }
    __syncthreads();
    uint8_t *dst = a.out + a.payload_off + a.ws_segsum[seg] + tstart;
    for (uint32_t i = tid; i < tbytes / 16; i += kThreads)
      store_nt16(dst + 16 * i, reinterpret_cast<const uint4 *>(lds)[i]);
    __syncthreads();
  }
}

__global__ __launch_bounds__(kThreads) void k_enc_finish(EncodeArgs a, HeaderImage h) {
  const uint64_t tid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  if (tid < 64) reinterpret_cast<uint32_t *>(a.out)[tid] = reinterpret_cast<const uint32_t *>(h.bytes)[tid];
  const uint64_t meta_bytes = align_up(2 * a.nb, kSectionAlign);
  for (uint64_t i = tid; i < meta_bytes; i += stride)
    a.out[a.meta_off + i] = i < 2 * a.nb ? a.ws_meta[i] : 0;
  const uint64_t seg_words = align_up(8 * a.nseg, kSectionAlign) / 8;
  for (uint64_t i = tid; i < seg_words; i += stride)
    reinterpret_cast<uint64_t *>(a.out + a.segoff_off)[i] = i < a.nseg ? a.ws_segsum[i] : 0;
  const uint64_t sm_end = kHeaderBytes + align_up(a.n, kSectionAlign);
  for (uint64_t i = kHeaderBytes + align_up(a.n, 8) + tid; i < sm_end; i += stride) a.out[i] = 0;
}

__global__ __launch_bounds__(kThreads) void k_enc_raw(const uint16_t *__restrict__ in,
                                                      uint8_t *__restrict__ out, uint64_t n,
                                                      HeaderImage h) {
  const uint64_t tid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  if (tid < 64) reinterpret_cast<uint32_t *>(out)[tid] = reinterpret_cast<const uint32_t *>(h.bytes)[tid];
  uint16_t *dst = reinterpret_cast<uint16_t *>(out + kHeaderBytes);
  const uint64_t nvec = n / 8;
  for (uint64_t i = tid; i < nvec; i += stride)
    store_nt16(dst + 8 * i, reinterpret_cast<const uint4 *>(in)[i]);
  for (uint64_t i = nvec * 8 + tid; i < n; i += stride) dst[i] = in[i];
}

uint32_t grid_for(uint64_t items, uint64_t per_block, uint32_t cap) {
  const uint64_t g = (items + per_block - 1) / per_block;
  return (uint32_t)(g < 1 ? 1 : (g > cap ? cap : g));
}

}  // namespace

hipError_t launch_encode_params(const EncodeArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(k_enc_params, dim3((uint32_t)a.nseg), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_encode_scan(const EncodeArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(k_enc_scan, dim3(1), dim3(1024), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_encode_pack(const EncodeArgs &a, hipStream_t s) {
  const uint64_t ntiles = tiles_for(a.n);
  hipLaunchKernelGGL(k_enc_pack, dim3(grid_for(ntiles, 1, 2048)), dim3(kThreads), 0, s, a, ntiles);
  return hipGetLastError();
}

hipError_t launch_encode_finish(const EncodeArgs &a, const HeaderImage &h, hipStream_t s) {
  const uint64_t work = align_up(2 * a.nb, kSectionAlign) + a.nseg + kSectionAlign;
  hipLaunchKernelGGL(k_enc_finish, dim3(grid_for(work, kThreads, 1024)), dim3(kThreads), 0, s, a, h);
  return hipGetLastError();
}

hipError_t launch_encode_raw(const uint16_t *in, uint8_t *out, uint64_t n, const HeaderImage &h,
                             hipStream_t s) {
  hipLaunchKernelGGL(k_enc_raw, dim3(grid_for(n / 8 + 1, kThreads, 4096)), dim3(kThreads), 0, s, in,
                     out, n, h);
  return hipGetLastError();
}

}  // namespace enc
