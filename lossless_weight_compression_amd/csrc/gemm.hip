// gemm.hip -- fused decompress-GEMM on gfx950:  Y[M,N] (fp32) = X[M,K] (bf16) x W[K,N]
// with W row-major and held only in compressed form.
//
// "ZipServ: Fast and Memory-Efficient LLM Inference with Hardware-Aware
// Lossless Compression", Abstract: the weights are decompressed on the fly
// inside the GEMM kernel: compressed bytes are what is loaded, decoded values
// are what the matrix units consume, so the decoded W never goes back to HBM
// and the kernel reads only the compressed bytes.
//
// Both paths locate the block of a row the way the decoder does: the stored
// offset of the block's 64-block segment plus the payload sizes of the earlier
// blocks of that segment. Every block of W is full (N % B == 0), so a block's
// payload is w * B / 8 bytes.
//
// Small M runs on VALU FMAs, larger M on MFMA: from M = 2 on for the
// uniform-row kernels (kMfmaMinMUniform), from M = 3 for the generic ones
// (kMfmaMinM). Above the crossover the MFMA kernels' cost hardly depends on
// M (4096 x 14336 W, GPU time per call: M = 2 29.5 us with k_gemm_rowu<2>,
// 27.2 with k_gemm_mfmau; M = 3 29.2 on VALU vs 27.7 on MFMA, M = 4 31.3 vs
// 28.0 for the generic pair).
//  * k_gemm_rowu (small M, B >= 512): a wave owns a 512-column strip and 64
//    rows; every row's width, base and block offset are wave-uniform, so
//    codes come in with one buffer load per lane and row and the byte planes
//    turn into fp32 with v_perm; M x 8 fp32 FMAs per row.
//  * k_gemm_mfmau (larger M, B >= 512, or dense W): wave-uniform rows are
//    decoded into k-pair dwords in an LDS tile, B fragments of
//    v_mfma_f32_16x16x32_bf16 are read from it, A fragments from the step's
//    X slice, staged in LDS once per workgroup.
//  * k_gemm_valu / k_gemm_mfma: the same two schemes for B < 512, where a
//    512-column run spans several blocks and each lane finds its own block.
//  * W stored [N, K] (a linear layer's layout, Y = X W^T): k_gemm_ntu
//    decodes 128-k runs of TN rows into an LDS tile read as MFMA fragments
//    (B >= 512, or dense W); k_gemm_nt decodes groups straight into
//    fragments (any other block size); k_gemv_nt serves M = 1 (whole rows
//    of W per workgroup, no split over K).
//  * split K: workgroups over K ranges write fp32 partial slices, added in
//    K order (deterministic) by k_splitk_reduce, launched next on the same
//    stream -- or, in k_gemm_rowu, by the last workgroup of each strip.
#include "enc_common.h"
#include "group_math.h"

// 1: split-K arrivals ordered by agent-scope release / acquire fences;
// 0: by waiting for the slice's agent-scope stores to complete.
#ifndef ENC_FIXUP_FENCE
#define ENC_FIXUP_FENCE 0
#endif
// Load pipelining: rows per batch and batches in the ring of the small-M
// kernel; K steps in the ring of the MFMA kernel.
#ifndef ENC_ROWU_RB
#define ENC_ROWU_RB 4
#endif
#ifndef ENC_ROWU_NB
#define ENC_ROWU_NB 2
#endif
#ifndef ENC_MFMAU_NB
#define ENC_MFMAU_NB 2
#endif
#ifndef ENC_MFMAU_NB_BIG
#define ENC_MFMAU_NB_BIG 2
#endif
#ifndef ENC_MFMAU_KS
#define ENC_MFMAU_KS 32
#endif


namespace enc {
namespace {

constexpr uint32_t kMfmaMinM = 3;              // smallest M on the generic MFMA kernel
constexpr uint32_t kMfmaMinMUniform = 2;       // smallest M on the uniform-row MFMA kernel
static_assert(kMfmaMinM == 3 && kMfmaMinMUniform == 2,
              "the VALU launchers instantiate M = 1..2 (generic) and M = 1 (uniform rows)");
constexpr uint32_t kStrip = 512;               // VALU path: columns per workgroup
constexpr uint32_t kValuRowsPerWave = 64;
constexpr uint32_t kValuRows = 4 * kValuRowsPerWave;
constexpr uint32_t kTileN = 128;               // MFMA path: columns per workgroup
constexpr uint32_t kKStep = 32;                // MFMA path: rows per K step
constexpr uint32_t kWPitch = kTileN + 2;       // bf16 per LDS row of the W tile
constexpr uint32_t kXPitch = kKStep + 8;       // bf16 per LDS row of the X tile

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// Payload offset of block i0 (a full block of W) and its meta word: segment
// offset plus (B/8) x the widths of the earlier blocks of the segment. With
// `run512` (i0 starts a 512-column run, so i0 is a multiple of 512/B) the
// word holds the 512/B {base, width} pairs of the run for B < 512 (naturally
// aligned); otherwise only block i0's pair. All loads are issued at once (the
// segment's 64 metas are 128 bytes inside the meta section).
template <bool run512>
__device__ __forceinline__ void row_block(const GemmArgs &a, uint64_t i0, uint64_t &off,
                                          uint64_t &mw) {
  const uint64_t seg = i0 >> 6;
  const uint32_t t = (uint32_t)(i0 & 63);
  const uint4 *m4 = reinterpret_cast<const uint4 *>(a.wstream + a.meta_off + 128 * seg);
  const uint8_t *mp = a.wstream + a.meta_off + 2 * i0;
  const uint64_t so = *reinterpret_cast<const uint64_t *>(a.wstream + a.segoff_off + 8 * seg);
  if (!run512 || a.log2b >= 9)
    mw = *reinterpret_cast<const uint16_t *>(mp);
  else if (a.log2b == 8)
    mw = ld32(mp);
  else
    mw = *reinterpret_cast<const uint64_t *>(mp);
  uint4 v[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) v[q] = m4[q];
  uint32_t wsum = 0;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const uint32_t d[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const uint32_t b = 8 * q + 2 * h;   // blocks b, b+1 of the segment
      wsum += (b < t ? (d[h] >> 8) & 0xFFu : 0u) + (b + 1 < t ? d[h] >> 24 : 0u);
    }
  }
  off = a.payload_off + so + ((uint64_t)wsum << (a.log2b - 3));
}

// Raw material of one group of a compressed row: sign+mantissa dwords, code
// dwords, and the packed {base, width, lead} needed to decode it.
struct GroupRaw {
  uint32_t sml, smh, q0, q1, q2, info;
};

// Loads group g of the run of columns that starts at element e (e is the
// first element of a 512- or 128-column run; the run lies in one segment).
// blk_off / mw are row_block()'s results for block e >> log2b. For B < 512 a
// 512-column run spans 512/B blocks; the lane adds the sizes of the earlier
// ones, read from the meta word.
__device__ __forceinline__ GroupRaw load_group(const GemmArgs &a, uint64_t e, uint32_t g,
                                               uint64_t blk_off, uint64_t mw) {
  const uint8_t *__restrict__ s = a.wstream;
  const uint32_t log2b = a.log2b;
  uint32_t meta, extra = 0, u;
  if (log2b >= 9 || g < (1u << (log2b - 3))) {
    meta = (uint32_t)mw & 0xFFFFu;
    u = (uint32_t)((e & ((1u << log2b) - 1)) >> 3) + g;
  } else {
    const uint32_t bl = g >> (log2b - 3);       // block of the run (1..3)
    meta = (uint32_t)(mw >> (16 * bl)) & 0xFFFFu;
    for (uint32_t j = 0; j < bl; ++j) extra += (uint32_t)((mw >> (16 * j + 8)) & 0xFFu);
    extra <<= (log2b - 3);
    u = g & ((1u << (log2b - 3)) - 1);
  }
  uint32_t w = meta >> 8;
  // corrupted stream guard: a width above 8, or a block running past the
  // stream end, decodes as width 0 (wrong values, but no stray reads); no
  // sum here can wrap, whatever the stored segment offset
  if (w > 8 || blk_off > a.total || extra + ((uint64_t)w << (log2b - 3)) > a.total - blk_off) w = 0;
  const uint64_t pb = blk_off + extra + (uint64_t)u * w;
  const uint64_t sm_addr = kHeaderBytes + e + 8 * (uint64_t)g;
  const uint2 sm = *reinterpret_cast<const uint2 *>(s + sm_addr);
  GroupRaw r;
  r.sml = sm.x;
  r.smh = sm.y;
  uint32_t lead;
  load_codes(s, pb, w, sm_addr, r.q0, r.q1, r.q2, lead);
  r.info = ((meta & 0xFFu) << 16) | (w << 24) | (lead << 3);
  return r;
}

__device__ __forceinline__ uint4 decode_raw(const GroupRaw &r) {
  const uint32_t w = (r.info >> 24) & 15u;
  const uint32_t base4 = ((r.info >> 16) & 0xFFu) * 0x01010101u;
  uint32_t lo, hi;
  align_codes(r.q0, r.q1, r.q2, (r.info >> 3) & 3u, lo, hi);
  return join_group(lo, hi, w, base4, r.sml, r.smh);
}

// Split-K epilogue shared by all kernels. for_each(fn) calls fn(y_index,
// value) for every value this thread holds (y_index < 0: no output); it is
// unrolled by the caller, so accumulator registers are never indexed
// dynamically. With one K range the values go to Y; otherwise to this
// range's slice of the partial buffer, which k_splitk_reduce (the next
// launch on the stream) adds up in K order -- deterministic, and every CU
// takes part in the reduction. (Letting the last workgroup of a tile add
// the slices needs no second launch, but that one workgroup then streams
// all slices of its tile alone: up to 512 KB through one CU.)
template <class ForEach>
__device__ __forceinline__ void splitk_finish(const GemmArgs &a, uint32_t ks, ForEach for_each) {
  float *dst = a.ksplit == 1 ? a.y : a.partial + (uint64_t)ks * a.M * a.N;
  for_each([&](int64_t y, float v) {
    if (y >= 0) dst[y] = v;
  });
}

// Y[i] = sum over K ranges of partial[k][i], k ascending. One output per
// thread and CH (>= ksplit when ksplit <= 32) slices' loads in flight at
// once: the reduction is a few MB at most, so it is latency-bound and wants
// one round trip, not a chain.
template <uint32_t CH>
__global__ __launch_bounds__(256) void k_splitk_reduce(const float *__restrict__ partial,
                                                       float *__restrict__ y, uint64_t mn,
                                                       uint32_t ksplit) {
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < mn;
       i += (uint64_t)gridDim.x * blockDim.x) {
    float sum = 0.f;
    for (uint32_t k = 0; k < ksplit; k += CH) {
      float v[CH];
#pragma unroll
      for (uint32_t j = 0; j < CH; ++j)   // unconditional (clamped) loads, masked after
        v[j] = partial[(uint64_t)min(k + j, ksplit - 1) * mn + i];
#pragma unroll
      for (uint32_t j = 0; j < CH; ++j) sum += k + j < ksplit ? v[j] : 0.f;
    }
    y[i] = sum;
  }
}

// The VALU kernels' strip result sits in LDS (red[m * 512 + col]).
template <int MM>
__device__ __forceinline__ void strip_finish(const GemmArgs &a, uint32_t c, uint32_t ks,
                                             const float *red) {
  const uint64_t col0 = (uint64_t)c * kStrip;
  splitk_finish(a, ks, [&](auto fn) {
    for (uint32_t i = threadIdx.x; i < MM * kStrip; i += blockDim.x)
      fn((int64_t)(i / kStrip) * a.N + (int64_t)col0 + (i % kStrip), red[i]);
  });
}

// Strip and K range of workgroup b (1-D grid of nstrips x ksplit). The
// hardware hands workgroups to the eight XCDs round-robin, b mod 8; when
// ksplit is a multiple of 8, K range ks runs entirely on XCD ks mod 8, so
// the strips of one row -- whose code payloads share the cache lines at
// their ends, and whose rows share segment metadata -- meet in one L2.
__device__ __forceinline__ void xcd_strip_range(uint32_t b, uint32_t nstrips, uint32_t ksplit,
                                                uint32_t &c, uint32_t &ks) {
  if ((ksplit & 7) == 0) {
    const uint32_t j = b >> 3;
    ks = (b & 7) + 8 * (j / nstrips);
    c = j % nstrips;
  } else {
    c = b % nstrips;
    ks = b / nstrips;
  }
}

// In-kernel split-K reduction of a strip (no second launch): each K range
// publishes its slice with agent-scope stores, waits until they have
// completed (they are performed at the device's coherence point, past the
// XCD-private L2s), and counts its arrival on the strip's counter; the last
// workgroup to arrive adds the slices in K order (its own from LDS), writes
// Y and resets the counter to zero for the next call. The order of the sum
// is fixed, so the result does not depend on which workgroup is last (and
// equals k_splitk_reduce's).
// Publishes this K range's slice of a strip (for_each as in splitk_finish)
// with agent-scope stores, waits until they have completed, and counts the
// arrival on the strip's counter. Returns true in the last workgroup to
// arrive (all slices are then in place).
template <class ForEach>
__device__ __forceinline__ bool strip_arrive(const GemmArgs &a, uint32_t c, uint32_t ks,
                                             ForEach for_each) {
  __shared__ uint32_t last;
  float *mine = a.partial + (uint64_t)ks * a.M * a.N;
  for_each([&](int64_t y, float v) {
    if (y >= 0) __hip_atomic_store(mine + y, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  });
#if ENC_FIXUP_FENCE
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
#else
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#endif
  __syncthreads();
  if (threadIdx.x == 0)
    last = __hip_atomic_fetch_add(a.counters + c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
           a.ksplit - 1;
  __syncthreads();
#if ENC_FIXUP_FENCE
  if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
#endif
  return last;
}

// In the last workgroup of strip c: Y[m, strip] = sum of the slices in K
// order (the order is fixed, so the result does not depend on which
// workgroup is last, and equals k_splitk_reduce's); then the strip's counter
// goes back to zero for the next call.
__device__ __forceinline__ void strip_reduce(const GemmArgs &a, uint32_t c) {
  const uint64_t col0 = (uint64_t)c * kStrip, mn = (uint64_t)a.M * a.N;
  // kCh loads in flight per output before any is added
  constexpr uint32_t kCh = 16;
  for (uint32_t i = threadIdx.x; i < a.M * kStrip; i += blockDim.x) {
    const uint64_t yi = (i / kStrip) * a.N + col0 + (i % kStrip);
    float sum = 0.f;
    for (uint32_t k0 = 0; k0 < a.ksplit; k0 += kCh) {
      float v[kCh];
#pragma unroll
      for (uint32_t j = 0; j < kCh; ++j)
        v[j] = __hip_atomic_load(a.partial + (uint64_t)min(k0 + j, a.ksplit - 1) * mn + yi,
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (uint32_t j = 0; j < kCh; ++j) sum += k0 + j < a.ksplit ? v[j] : 0.f;
    }
    a.y[yi] = sum;
  }
  if (threadIdx.x == 0) __hip_atomic_store(a.counters + c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// In-kernel split-K reduction of a strip (no second launch): each K range
// publishes its slice and counts its arrival; the last workgroup to arrive
// adds the slices (its own included, read back) and writes Y.
template <int MM>
__device__ __forceinline__ void strip_fixup(const GemmArgs &a, uint32_t c, uint32_t ks,
                                            const float *red) {
  const uint64_t col0 = (uint64_t)c * kStrip;
  const bool last = strip_arrive(a, c, ks, [&](auto fn) {
    for (uint32_t i = threadIdx.x; i < MM * kStrip; i += blockDim.x)
      fn((int64_t)(i / kStrip) * a.N + (int64_t)col0 + (i % kStrip), red[i]);
  });
  if (last) strip_reduce(a, c);
}

// --------------------------------------------------------------------------
// M < kMfmaMinM: VALU FMA path.
// --------------------------------------------------------------------------
template <int MM, bool DENSE>
__global__ __launch_bounds__(256) void k_gemm_valu(GemmArgs a) {
  constexpr uint32_t RB = MM <= 4 ? 8 : 4;      // rows per batch; two batches in flight
  __shared__ float red[MM * kStrip];
  const uint32_t tid = threadIdx.x, lane = tid & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const uint32_t c = blockIdx.x, ks = blockIdx.y;
  const uint32_t N = a.N, K = a.K;
  const uint32_t rows_w = a.krows / 4;          // <= 64
  const uint32_t kw0 = ks * a.krows + wave * rows_w;
  const uint32_t kw1 = min(kw0 + rows_w, K);
  const uint32_t nrows = kw1 > kw0 ? kw1 - kw0 : 0;
  const uint64_t col0 = (uint64_t)c * kStrip;

  // Prologue: lane l describes row kw0 + l -- block offset and meta word of
  // the strip's first block, and X[m][row]. Rows are then broadcast with
  // v_readlane, so the row loop has no dependent loads.
  uint64_t r_off = 0, r_mw = 0;
  float xr[MM];
#pragma unroll
  for (int m = 0; m < MM; ++m) xr[m] = 0.f;
  if (lane < nrows) {
    const uint32_t kr = kw0 + lane;
    if (!DENSE) row_block<true>(a, ((uint64_t)kr * N + col0) >> a.log2b, r_off, r_mw);
#pragma unroll
    for (int m = 0; m < MM; ++m) xr[m] = bf_lo(a.x[(uint64_t)m * K + kr]);
  }

  float acc[MM][8];
#pragma unroll
  for (int m = 0; m < MM; ++m)
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[m][q] = 0.f;

  auto load_batch = [&](uint32_t r0, GroupRaw(&raw)[RB], uint4(&dv)[RB]) {
#pragma unroll
    for (uint32_t j = 0; j < RB; ++j) {
      const uint32_t r = r0 + j;
      if (r < nrows) {
        const uint64_t e = (uint64_t)(kw0 + r) * N + col0;
        if (DENSE) {
          dv[j] = *reinterpret_cast<const uint4 *>(a.wdense + e + 8 * lane);
        } else {
          const uint64_t off = ((uint64_t)__builtin_amdgcn_readlane((uint32_t)(r_off >> 32), r) << 32) |
                               __builtin_amdgcn_readlane((uint32_t)r_off, r);
          const uint64_t mw = ((uint64_t)__builtin_amdgcn_readlane((uint32_t)(r_mw >> 32), r) << 32) |
                              __builtin_amdgcn_readlane((uint32_t)r_mw, r);
          raw[j] = load_group(a, e, lane, off, mw);
        }
      }
    }
  };
  auto compute_batch = [&](uint32_t r0, const GroupRaw(&raw)[RB], const uint4(&dv)[RB]) {
#pragma unroll
    for (uint32_t j = 0; j < RB; ++j) {
      const uint32_t r = r0 + j;
      if (r < nrows) {
        const uint4 v = DENSE ? dv[j] : decode_raw(raw[j]);
        const float f[8] = {bf_lo(v.x), bf_hi(v.x), bf_lo(v.y), bf_hi(v.y),
                            bf_lo(v.z), bf_hi(v.z), bf_lo(v.w), bf_hi(v.w)};
#pragma unroll
        for (int m = 0; m < MM; ++m) {
          const float xm = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(xr[m]), r));
#pragma unroll
          for (int q = 0; q < 8; ++q) acc[m][q] = fmaf(xm, f[q], acc[m][q]);
        }
      }
    }
  };
  GroupRaw rawA[RB], rawB[RB];
  uint4 dvA[RB], dvB[RB];
  if (nrows) load_batch(0, rawA, dvA);
  for (uint32_t r0 = 0; r0 < nrows; r0 += 2 * RB) {
    if (r0 + RB < nrows) load_batch(r0 + RB, rawB, dvB);
    compute_batch(r0, rawA, dvA);
    if (r0 + 2 * RB < nrows) load_batch(r0 + 2 * RB, rawA, dvA);
    if (r0 + RB < nrows) compute_batch(r0 + RB, rawB, dvB);
  }
  // deterministic reduction of the four waves' rows: wave 0, then 1, 2, 3
  for (uint32_t w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int m = 0; m < MM; ++m)
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const uint32_t idx = m * kStrip + 8 * lane + q;
          red[idx] = (w == 0 ? 0.f : red[idx]) + acc[m][q];
        }
    }
    __syncthreads();
  }
  strip_finish<MM>(a, c, ks, red);
}

// --------------------------------------------------------------------------
// M < kMfmaMinM and B >= 512: wave-uniform rows.
//
// A 512-column strip of a row lies inside one block when B >= 512, so the
// width, base and block offset of every row a wave touches are uniform
// across the wave: they live in SGPRs (v_readlane of a per-lane prologue
// table), payload dwords are fetched with 32-bit offsets off the stream's
// SGPR base, and the exponent/sign+mantissa byte planes turn into fp32 with
// one v_perm per value (high byte = sign | e >> 1, next byte = (e & 1) << 7 |
// mantissa, low bytes zero).
// --------------------------------------------------------------------------
// Rows per wave of k_gemm_rowu (K range of a workgroup: 4 waves x 64 = 256
// rows; 16 K ranges for K = 4096). The prologue describes one row per lane,
// so at most 64. Measured on a 4096 x 14336 W, GPU time per call at M = 1 /
// M = 2: 32 rows 25.7 / 27.3 us, 64 rows 24.1 / 26.0 (half the split-K
// slices); 8 waves x 64 rows 23.9 / 26.1, 16 waves x 64 36.4 / 39.9.
constexpr uint32_t kRowuWaves = 4;
constexpr uint32_t kRowuRange = 256;            // rows per K range (workgroup)
constexpr uint32_t kRowsPerWaveU = kRowuRange / kRowuWaves;
static_assert(kRowsPerWaveU <= 64, "k_gemm_rowu keeps one row per lane");
static_assert(kRowuRange % kRowuWaves == 0, "whole rows per wave");

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));

// Raw buffer descriptor over a whole stream (< 4 GiB): loads take a 32-bit
// offset. Range checking as the CDNA3 ISA reference guide defines it for
// buffer instructions (section on buffer addressing, range checking; CDNA4
// keeps the rule): with stride 0 an access is out of range when its byte
// offset is at or past num_records (here the stream size), the check is made
// for each dword of a multi-dword access, out-of-range dwords load as zero
// and out-of-range stores are not performed. So a group's three code dwords
// are one buffer_load_dwordx3 even at the very end of the stream.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t stream_rsrc(const uint8_t *s, uint64_t total) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(s), 0, (int)(uint32_t)total,
                                           0x00020000);
}

template <int MM>
__global__ __launch_bounds__(kRowuWaves * 64) void k_gemm_rowu(GemmArgs a) {
  const uint32_t RW = a.krows / kRowuWaves;      // <= 64 (the plan's choice)
  constexpr uint32_t RB = ENC_ROWU_RB;            // rows per batch
  constexpr uint32_t NB = ENC_ROWU_NB;            // batches in the load ring
  __shared__ float red[MM * kStrip];
  const uint32_t tid = threadIdx.x, lane = tid & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  uint32_t c, ks;
  xcd_strip_range(blockIdx.x, a.N / kStrip, a.ksplit, c, ks);
  const uint32_t N = a.N, K = a.K, log2b = a.log2b;
  const uint32_t kw0 = ks * a.krows + wave * RW;
  const uint32_t nrows = kw0 < K ? min(RW, K - kw0) : 0u;
  const uint32_t col0 = c * kStrip;
  const __amdgpu_buffer_rsrc_t rs = stream_rsrc(a.wstream, a.total);

  // Prologue: lane l describes row kw0 + l (block offset, {base, width},
  // first group of the strip inside its block) and holds X[:, kw0 + l].
  uint32_t r_off = 0, r_meta = 0;
  float xr[MM];
#pragma unroll
  for (int m = 0; m < MM; ++m) xr[m] = 0.f;
  if (lane < nrows) {
    const uint32_t kr = kw0 + lane;
    const uint64_t e = (uint64_t)kr * N + col0;
    uint64_t off, mw;
    row_block<false>(a, e >> log2b, off, mw);
    uint32_t w = (uint32_t)(mw >> 8) & 0xFFu;
    if (w > 8) w = 0;   // corrupted stream: decode as width 0 (reads stay bounds-checked)
    const uint32_t u0 = (uint32_t)((e & ((1ull << log2b) - 1)) >> 3);
    r_off = (uint32_t)off;
    r_meta = ((uint32_t)mw & 0xFFu) | (w << 8) | (u0 << 16);
#pragma unroll
    for (int m = 0; m < MM; ++m) xr[m] = bf_lo(a.x[(uint64_t)m * K + kr]);
  }

  float acc[MM][8];
#pragma unroll
  for (int m = 0; m < MM; ++m)
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[m][q] = 0.f;

  struct Batch {
    u32x2 sm[RB];
    u32x3 q[RB];
  };
  // Loads are issued on every path (see k_gemm_mfmau): loads under branches
  // make the compiler wait for all outstanding loads, the next batch's
  // prefetch included. Rows past the last one load from past the
  // descriptor's range (zeros, no memory access).
  auto load_batch = [&](uint32_t r0, Batch &bt) {
#pragma unroll
    for (uint32_t j = 0; j < RB; ++j) {
      const uint32_t r = min(r0 + j, nrows - 1);
      const uint32_t dead = r0 + j < nrows ? 0u : 0x80000000u;
      const uint32_t off = __builtin_amdgcn_readlane(r_off, r);
      const uint32_t meta = __builtin_amdgcn_readlane(r_meta, r);
      const uint32_t w = (meta >> 8) & 15u;
      const uint32_t pb = off + ((meta >> 16) + lane) * w;
      const uint32_t row_sm = kHeaderBytes + (kw0 + r) * N + col0;   // uniform
      bt.sm[j] = __builtin_amdgcn_raw_buffer_load_b64(rs, (8 * lane) | dead, row_sm, 0);
      bt.q[j] = __builtin_amdgcn_raw_buffer_load_b96(rs, (pb & ~3u) | dead, 0, 0);
    }
  };
  auto compute_batch = [&](uint32_t r0, const Batch &bt) {
#pragma unroll
    for (uint32_t j = 0; j < RB; ++j) {
      const uint32_t r = r0 + j;
      if (r < nrows) {
        const uint32_t off = __builtin_amdgcn_readlane(r_off, r);
        const uint32_t meta = __builtin_amdgcn_readlane(r_meta, r);
        const uint32_t w = (meta >> 8) & 15u;           // wave-uniform
        const uint32_t base4 = (meta & 0xFFu) * 0x01010101u;
        uint32_t el, eh;
        if (w == 4) {
          // block payloads start on 16-byte boundaries, so a 4-byte group
          // is dword-aligned: its codes are exactly q.x
          codes_to_bytes_w4(bt.q[j].x, el, eh);
        } else {
          const uint32_t sh = ((off + ((meta >> 16) + lane) * w) & 3u) * 8;
          const uint32_t lo = __builtin_amdgcn_alignbit(bt.q[j].y, bt.q[j].x, sh);
          const uint32_t hi = __builtin_amdgcn_alignbit(bt.q[j].z, bt.q[j].y, sh);
          codes_to_bytes(lo, hi, w, el, eh);
        }
        el += base4;
        eh += base4;
        const uint32_t sml = bt.sm[j].x, smh = bt.sm[j].y;
        const uint32_t hl = (sml & kH8) | ((el >> 1) & ~kH8);
        const uint32_t ll = ((el << 7) & kH8) | (sml & ~kH8);
        const uint32_t hh = (smh & kH8) | ((eh >> 1) & ~kH8);
        const uint32_t lh = ((eh << 7) & kH8) | (smh & ~kH8);
        // fp32 of value k: bytes [0, 0, L_k, H_k]
        const float f[8] = {
            __uint_as_float(__builtin_amdgcn_perm(hl, ll, 0x04000C0Cu)),
            __uint_as_float(__builtin_amdgcn_perm(hl, ll, 0x05010C0Cu)),
            __uint_as_float(__builtin_amdgcn_perm(hl, ll, 0x06020C0Cu)),
            __uint_as_float(__builtin_amdgcn_perm(hl, ll, 0x07030C0Cu)),
            __uint_as_float(__builtin_amdgcn_perm(hh, lh, 0x04000C0Cu)),
            __uint_as_float(__builtin_amdgcn_perm(hh, lh, 0x05010C0Cu)),
            __uint_as_float(__builtin_amdgcn_perm(hh, lh, 0x06020C0Cu)),
            __uint_as_float(__builtin_amdgcn_perm(hh, lh, 0x07030C0Cu))};
#pragma unroll
        for (int m = 0; m < MM; ++m) {
          const float xm = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(xr[m]), r));
#pragma unroll
          for (int q = 0; q < 8; ++q) acc[m][q] = fmaf(xm, f[q], acc[m][q]);
        }
      }
    }
  };
  // NB batches in a ring: batch j + NB - 1 is loaded while batch j is
  // computed (rows past nrows are skipped inside compute_batch)
  Batch bt[NB];
#pragma unroll
  for (uint32_t p = 0; p + 1 < NB; ++p) load_batch(p * RB, bt[p]);
  for (uint32_t r0 = 0; r0 < nrows; r0 += NB * RB) {
#pragma unroll
    for (uint32_t j = 0; j < NB; ++j) {
      load_batch(r0 + (j + NB - 1) * RB, bt[(j + NB - 1) % NB]);
      compute_batch(r0 + j * RB, bt[j]);
    }
  }
  for (uint32_t w = 0; w < kRowuWaves; ++w) {
    if (wave == w) {
#pragma unroll
      for (int m = 0; m < MM; ++m)
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const uint32_t idx = m * kStrip + 8 * lane + q;
          red[idx] = (w == 0 ? 0.f : red[idx]) + acc[m][q];
        }
    }
    __syncthreads();
  }
  if (a.counters && a.ksplit > 1)
    strip_fixup<MM>(a, c, ks, red);
  else
    strip_finish<MM>(a, c, ks, red);
}

// --------------------------------------------------------------------------
// M >= kMfmaMinM: MFMA path.
// --------------------------------------------------------------------------
template <int MT, bool DENSE>
__global__ __launch_bounds__(256) void k_gemm_mfma(GemmArgs a) {
  constexpr int MSUB = MT / 16;
  __shared__ __attribute__((aligned(16))) uint16_t wt[kKStep * kWPitch];
  __shared__ __attribute__((aligned(16))) uint16_t xt[MT * kXPitch];
  __shared__ uint32_t row_off_lo[1024], row_off_hi[1024], row_meta[1024];
  const uint32_t tid = threadIdx.x, lane = tid & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const uint32_t nt = blockIdx.x, ks = blockIdx.y, mt = blockIdx.z;
  const uint32_t N = a.N, K = a.K, M = a.M;
  const uint32_t n0 = nt * kTileN, m0 = mt * MT;
  const uint32_t k0 = ks * a.krows;
  const uint32_t k1 = min(k0 + a.krows, K);
  const uint32_t nsteps = (k1 - k0 + kKStep - 1) / kKStep;

  if (!DENSE) {
    for (uint32_t r = tid; r < k1 - k0; r += 256) {
      uint64_t off, mw;
      row_block<false>(a, ((uint64_t)(k0 + r) * N + n0) >> a.log2b, off, mw);
      row_off_lo[r] = (uint32_t)off;
      row_off_hi[r] = (uint32_t)(off >> 32);
      row_meta[r] = (uint32_t)mw & 0xFFFFu;
    }
    __syncthreads();
  }

  // each thread: two W groups per step (rows tr and tr + 16, 8 columns at tg)
  const uint32_t tr = tid >> 4, tg = tid & 15;
  // X tile: MT x 32 bf16 = MT*4 16-byte pieces
  constexpr uint32_t XPIECES = MT * 4;

  GroupRaw raw[2];
  uint4 dv[2];
  uint4 xv[(XPIECES + 255) / 256];

  auto load_step = [&](uint32_t step) {
    const uint32_t kb = k0 + step * kKStep;
#pragma unroll
    for (uint32_t h = 0; h < 2; ++h) {
      const uint32_t kr = kb + tr + 16 * h;
      if (kr < k1) {
        const uint64_t e = (uint64_t)kr * N + n0;
        if (DENSE) {
          dv[h] = *reinterpret_cast<const uint4 *>(a.wdense + e + 8 * tg);
        } else {
          const uint32_t r = kr - k0;
          const uint64_t off = ((uint64_t)row_off_hi[r] << 32) | row_off_lo[r];
          raw[h] = load_group(a, e, tg, off, row_meta[r]);
        }
      }
    }
#pragma unroll
    for (uint32_t p = 0; p < (XPIECES + 255) / 256; ++p) {
      const uint32_t piece = tid + 256 * p;
      const uint32_t m = piece >> 2, q = piece & 3;
      const uint32_t kx = kb + 8 * q;
      xv[p] = make_uint4(0, 0, 0, 0);
      if (piece < XPIECES && m0 + m < M && kx < k1)
        xv[p] = *reinterpret_cast<const uint4 *>(a.x + (uint64_t)(m0 + m) * K + kx);
    }
  };

  f32x4 acc[MSUB][2];
#pragma unroll
  for (int t = 0; t < MSUB; ++t)
    for (int s = 0; s < 2; ++s) acc[t][s] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (nsteps) load_step(0);
  for (uint32_t step = 0; step < nsteps; ++step) {
    const uint32_t kb = k0 + step * kKStep;
    // decoded W groups -> LDS (row-major, rows past K are zero)
#pragma unroll
    for (uint32_t h = 0; h < 2; ++h) {
      const uint32_t r = tr + 16 * h;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (kb + r < k1) v = DENSE ? dv[h] : decode_raw(raw[h]);
      uint32_t *dst = reinterpret_cast<uint32_t *>(wt + r * kWPitch + 8 * tg);
      dst[0] = v.x;
      dst[1] = v.y;
      dst[2] = v.z;
      dst[3] = v.w;
    }
#pragma unroll
    for (uint32_t p = 0; p < (XPIECES + 255) / 256; ++p) {
      const uint32_t piece = tid + 256 * p;
      if (piece < XPIECES)
        *reinterpret_cast<uint4 *>(xt + (piece >> 2) * kXPitch + 8 * (piece & 3)) = xv[p];
    }
    __syncthreads();
    if (step + 1 < nsteps) load_step(step + 1);
    // MFMA: wave owns columns [32 wave, 32 wave + 32) of the tile
    const uint32_t kq = 8 * (lane >> 4);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const uint32_t n = 32 * wave + 16 * s + (lane & 15);
      bf16x8 b;
#pragma unroll
      for (int j = 0; j < 8; ++j) b[j] = __builtin_bit_cast(__bf16, wt[(kq + j) * kWPitch + n]);
#pragma unroll
      for (int t = 0; t < MSUB; ++t) {
        const bf16x8 av = *reinterpret_cast<const bf16x8 *>(xt + (16 * t + (lane & 15)) * kXPitch + kq);
        acc[t][s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, b, acc[t][s], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // lane holds D[4 (lane >> 4) + j][lane & 15] of each 16x16 subtile
  splitk_finish(a, ks, [&](auto fn) {
#pragma unroll
    for (int t = 0; t < MSUB; ++t)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t m = m0 + 16 * t + 4 * (lane >> 4) + j;
          const uint32_t n = n0 + 32 * wave + 16 * s2 + (lane & 15);
          fn(m < M ? (int64_t)m * N + n : (int64_t)-1, acc[t][s2][j]);
        }
  });
}

// --------------------------------------------------------------------------
// M >= kMfmaMinM and B >= 512 (or dense W): MFMA on wave-uniform rows.
//
// Output tile MT x 512 (one strip) per workgroup of WAVES waves, split over
// K ranges. Per K step of 32 rows, wave w decodes rows [w*RPW, w*RPW + RPW)
// of the step over the full 512 columns (lane: 8 columns; width, base and
// block offset wave-uniform as in k_gemm_rowu), two rows at a time, and
// writes k-pair dwords (W[k][n] | W[k+1][n] << 16) into an LDS tile of
// 16 k-pairs x 516 dwords. The 4-dword pad makes the MFMA B-fragment reads
// (4 x ds_read_b32: k-pairs 4*(lane/16)+p, column lane%16) hit distinct banks
// for 32- and 64-bank LDS alike. Two tiles alternate, so one barrier per step
// separates a step's decode from its MFMAs; the next step's compressed bytes
// and X fragments are loaded before the current step is decoded.
// v_mfma_f32_16x16x32_bf16: A fragment = 8 consecutive k of one X row (one
// 16-byte load), D = 4 rows x 1 column per lane.
// --------------------------------------------------------------------------
constexpr uint32_t kPitchU = 516;

// Workgroup barrier for LDS hand-off only. __syncthreads() also fences
// global memory, so the compiler waits for every outstanding global load
// (vmcnt 0) first -- including the next K step's prefetched loads, which
// would serialise each step on a full memory round trip. Here only this
// wave's LDS operations are waited for; the "memory" clobber keeps the
// compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// This lane's index, computed where it is used. The asm is volatile, so the
// compiler neither hoists it out of a loop nor keeps it in a register across
// one: at 128 registers per lane such loop-invariant values get spilled, and
// each reload from scratch waits for every outstanding global load (it counts
// in the same counter), which drains the prefetch ring.
__device__ __forceinline__ uint32_t lane_here() {
  uint32_t l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// M tile of k_gemm_mfmau; larger M runs several 128-row tiles.
uint32_t mfmau_tile_m(uint32_t M) { return M <= 16 ? 16 : M <= 32 ? 32 : M <= 64 ? 64 : 128; }

// The X slice in LDS: one row per X row, KS bf16 (KS / 8 16-byte chunks),
// rows padded by 16 bf16. ds_read_b128 serves 16 lanes per cycle, but not
// 16 consecutive ones: measured on gfx950 with the SQ_LDS_BANK_CONFLICT
// counter, the MFMA A-fragment read (lane l: row l % 16, chunk l / 16) costs
// twice the cycles of a conflict-free read from rows padded to 80, 144 or
// 272 bytes, and none from 288-byte rows; the lane groups that fit those
// measurements make 96-byte (KS = 32) and 160-byte (KS = 64) rows
// conflict-free as well, and the writes of whole rows by consecutive lanes
// stay so.
constexpr uint32_t xs_pitch(uint32_t ks) { return ks + 16; }   // bf16 per LDS row of the X slice

// Each K step, the workgroup's threads load the step's X slice (MT rows x 32
// k, one 16-byte piece per thread) and store it in LDS next to the decoded W
// rows; every wave then reads its A fragments there. Compared with each wave
// loading its own A fragments from X, this keeps the accumulators and the
// two-step ring within 128 registers at 16 waves for every M tile, so W is
// decoded once for M up to 128 (measured on a 4096 x 14336 W: M = 32 38.7 ->
// 34.1 us, M = 64 50.5 -> 39.7, M = 128 57.8 -> 52.7).
template <int MT, int WAVES, bool DENSE, int NB, int KS>
__global__ __launch_bounds__(WAVES * 64) void k_gemm_mfmau(GemmArgs a) {
  constexpr uint32_t RPW = KS / WAVES;          // rows decoded per wave per step
  constexpr uint32_t NSUB = 32 / WAVES;         // 16-column subtiles per wave
  constexpr uint32_t MSUB = MT / 16;
  constexpr uint32_t NTHR = WAVES * 64;
  constexpr uint32_t XP = MT * KS / 8;          // 16-byte pieces of a step's X slice
  constexpr uint32_t XPITCH = xs_pitch(KS);
  static_assert(WAVES == 16 && (KS == 32 || KS == 64), "16 waves, steps of 32 or 64 rows");
  static_assert(XP <= NTHR && XP % 64 == 0, "at most one X piece per thread, whole waves");
  __shared__ __attribute__((aligned(16))) uint32_t tile[2][KS / 2 * kPitchU];
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][MT * XPITCH];
  const uint32_t tid = threadIdx.x, lane = tid & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const uint32_t mt = blockIdx.y;
  uint32_t c, ks;
  xcd_strip_range(blockIdx.x, a.N / kStrip, a.ksplit, c, ks);
  const uint32_t N = a.N, K = a.K, M = a.M, log2b = a.log2b;
  const uint32_t k0 = ks * a.krows;
  const uint32_t k1 = min(k0 + a.krows, K);
  const uint32_t nsteps = (k1 - k0 + KS - 1) / KS;   // RPW * nsteps <= 64: at most 1024 rows
  const uint32_t col0 = c * kStrip, m0 = mt * MT;
  const __amdgpu_buffer_rsrc_t rs = stream_rsrc(a.wstream, a.total);
  // The thread index where the X slice is loaded and stored. The 128-row tile
  // uses all 128 registers of a lane, and a loop-invariant index there was
  // spilled and reloaded every step (with a wait for all loads in flight):
  // it recomputes the index each time (M = 128 56.7 -> 53.0 us per call on a
  // 4096 x 14336 W). The smaller tiles have room and keep it (recomputing
  // cost them 1-2%).
  auto xtid = [&]() -> uint32_t { return MT >= 128 ? wave * 64 + lane_here() : tid; };

  // Row table of this wave (coded W): lane l describes row KS (l / RPW) +
  // RPW wave + l % RPW of the K range -- a row the wave decodes in step
  // l / RPW -- by its block offset and a meta word (base, width, first group
  // of the strip inside its block). Steps read their rows with v_readlane
  // into SGPRs: no LDS table and no barrier before the first loads. Rows
  // past the K range keep offset and meta word 0 (width 0, base 0).
  uint32_t t_off = 0, t_meta = 0;
  auto build_table = [&]() {
    if (!DENSE && k0 + KS * (lane / RPW) + RPW * wave + (lane % RPW) < k1) {
      const uint32_t kr = k0 + KS * (lane / RPW) + RPW * wave + (lane % RPW);
      const uint64_t e = (uint64_t)kr * N + col0;
      uint64_t off, mw;
      row_block<false>(a, e >> log2b, off, mw);
      uint32_t w = (uint32_t)(mw >> 8) & 0xFFu;
      if (w > 8) w = 0;   // corrupted stream: decode as width 0
      t_off = (uint32_t)off;
      t_meta = ((uint32_t)mw & 0xFFu) | (w << 8) | ((uint32_t)((e & ((1ull << log2b) - 1)) >> 3) << 16);
    }
  };

  struct Step {
    u32x2 sm[RPW];
    u32x3 q[RPW];
    uint4 dv[RPW];
    uint32_t off[RPW], meta[RPW];   // rows' block offset and meta word (uniform)
    uint4 x;                    // this thread's piece of the X slice, as loaded
    uint32_t xm;                // all ones if that piece lies inside the K range
  };
  // Every load is issued unconditionally, from a clamped (always valid) row
  // or X element; out-of-range data is discarded after the load. Loads under
  // branches would make the compiler wait for all outstanding loads (vmcnt 0)
  // before the decode, i.e. also for the next step's prefetch.
  // Ring slots past the last step, and rows past the K range: the stream
  // loads get an offset past the descriptor's range (zeros, no memory
  // access) -- with width and base 0 such a row decodes to zeros -- the
  // others a clamped row.
  // The loads of a step in two parts: rows' sign+mantissa bytes (or dense
  // values) and the X piece, which need no row table, then the code bytes,
  // which do (so the first steps' byte planes are in flight while the table
  // is built).
  auto load_codes = [&](uint32_t st, Step &S) {
    if (DENSE) return;
    const uint32_t sc = min(st, nsteps - 1);
    const uint32_t kb = k0 + KS * sc;
#pragma unroll
    for (uint32_t j = 0; j < RPW; ++j) {
      const uint32_t dead = (st < nsteps && kb + wave * RPW + j < k1) ? 0u : 0x80000000u;
      const uint32_t off = __builtin_amdgcn_readlane(t_off, RPW * sc + j);
      const uint32_t meta = __builtin_amdgcn_readlane(t_meta, RPW * sc + j);
      const uint32_t w = (meta >> 8) & 15u;
      const uint32_t pb = off + ((meta >> 16) + lane) * w;
      S.off[j] = off;
      S.meta[j] = meta;
      S.q[j] = __builtin_amdgcn_raw_buffer_load_b96(rs, (pb & ~3u) | dead, 0, 0);
    }
  };
  auto load_planes = [&](uint32_t st, Step &S) {
    const uint32_t sc = min(st, nsteps - 1);
    const uint32_t kb = k0 + KS * sc;
#pragma unroll
    for (uint32_t j = 0; j < RPW; ++j) {
      const uint32_t dead = (st < nsteps && kb + wave * RPW + j < k1) ? 0u : 0x80000000u;
      const uint32_t kr = min(kb + wave * RPW + j, k1 - 1);
      if (DENSE)
        S.dv[j] = *reinterpret_cast<const uint4 *>(a.wdense + (uint64_t)kr * N + col0 + 8 * lane);
      else
        S.sm[j] = __builtin_amdgcn_raw_buffer_load_b64(rs, (8 * lane) | dead, kHeaderBytes + kr * N + col0, 0);
    }
    // piece p = tid mod XP: row p / (KS / 8), k = kb + 8 (p % (KS / 8)) .. + 7 (threads
    // past XP load a duplicate and do not store it). Rows past M are clamped
    // copies of row M - 1 and only reach output rows that are not stored;
    // pieces past the K range are zeroed when the last step stores them (a
    // select right after the load would make the compiler wait for it, i.e.
    // for every load just issued).
    const uint32_t p = xtid() % XP;
    const uint32_t m = m0 + p / (KS / 8), kx = kb + 8 * (p % (KS / 8));
    S.x = *reinterpret_cast<const uint4 *>(a.x + (uint64_t)min(m, M - 1) * K + min(kx, k1 - 8));
    S.xm = (st < nsteps && kx < k1) ? ~0u : 0u;
  };
  // Dense W: rows as loaded (zero past the K range).
  auto dense_row = [&](uint32_t st, const Step &S, uint32_t j) -> uint4 {
    const uint32_t kr = k0 + KS * st + wave * RPW + j;   // uniform
    return kr < k1 ? S.dv[j] : make_uint4(0, 0, 0, 0);
  };
  // Coded W: the w-bit codes of row j's eight values as bytes, E0 = values
  // 0, 2, 4, 6 and E1 = values 1, 3, 5, 7 (the order the 4-bit split gives).
  auto code_bytes = [&](const Step &S, uint32_t j, uint32_t &E0, uint32_t &E1) {
    const uint32_t w = (S.meta[j] >> 8) & 15u;   // wave-uniform
    if (w == 4) {
      // block payloads start on 16-byte boundaries, so a 4-byte group is
      // dword-aligned: its codes are exactly q.x
      E0 = S.q[j].x & 0x0F0F0F0Fu;
      E1 = (S.q[j].x >> 4) & 0x0F0F0F0Fu;
    } else {
      const uint32_t sh = ((S.off[j] + ((S.meta[j] >> 16) + lane) * w) & 3u) * 8;
      const uint32_t lo = __builtin_amdgcn_alignbit(S.q[j].y, S.q[j].x, sh);
      const uint32_t hi = __builtin_amdgcn_alignbit(S.q[j].z, S.q[j].y, sh);
      uint32_t el, eh;
      codes_to_bytes(lo, hi, w, el, eh);
      E0 = __builtin_amdgcn_perm(eh, el, 0x06040200u);
      E1 = __builtin_amdgcn_perm(eh, el, 0x07050301u);
    }
  };
  // Row pair (a = k even, b = k + 1) of this lane's eight columns as k-pair
  // dwords, BF16 of row a in the low half: per column, the two code bytes
  // side by side as 16-bit lanes (v_perm), shifted to the exponent field
  // with both bases added (v_lshl_add), and merged with the sign+mantissa
  // bytes placed at bits 0..6 and 15 of each half (v_perm, v_bfi) --
  // sign | exponent << 7 | mantissa, four operations per two values.
  auto decode_step = [&](uint32_t st, const Step &S, uint32_t buf) {
    const uint32_t kb = k0 + KS * st;
    const bool tail = kb + KS > k1;               // uniform: the last, partial step
#pragma unroll
    for (uint32_t pr = 0; pr < RPW / 2; ++pr) {   // row pairs 2 pr, 2 pr + 1 of this wave
      uint32_t *dst = &tile[buf][(wave * (RPW / 2) + pr) * kPitchU + 8 * lane];
      if (DENSE) {
        const uint4 ra = dense_row(st, S, 2 * pr), rb = dense_row(st, S, 2 * pr + 1);
        *reinterpret_cast<uint4 *>(dst) = make_uint4(
            __builtin_amdgcn_perm(rb.x, ra.x, 0x05040100u), __builtin_amdgcn_perm(rb.x, ra.x, 0x07060302u),
            __builtin_amdgcn_perm(rb.y, ra.y, 0x05040100u), __builtin_amdgcn_perm(rb.y, ra.y, 0x07060302u));
        *reinterpret_cast<uint4 *>(dst + 4) = make_uint4(
            __builtin_amdgcn_perm(rb.z, ra.z, 0x05040100u), __builtin_amdgcn_perm(rb.z, ra.z, 0x07060302u),
            __builtin_amdgcn_perm(rb.w, ra.w, 0x05040100u), __builtin_amdgcn_perm(rb.w, ra.w, 0x07060302u));
      } else {
        uint32_t E0a, E1a, E0b, E1b;
        code_bytes(S, 2 * pr, E0a, E1a);
        code_bytes(S, 2 * pr + 1, E0b, E1b);
        const uint32_t b7 = ((S.meta[2 * pr] & 0xFFu) << 7) | ((S.meta[2 * pr + 1] & 0xFFu) << 23);
#pragma unroll
        for (uint32_t h = 0; h < 2; ++h) {   // columns 4h .. 4h + 3
          const uint32_t sa = h ? S.sm[2 * pr].y : S.sm[2 * pr].x;
          const uint32_t sb = h ? S.sm[2 * pr + 1].y : S.sm[2 * pr + 1].x;
          uint32_t kp[4];
#pragma unroll
          for (uint32_t q = 0; q < 4; ++q) {
            const uint32_t col = 4 * h + q, i = col >> 1;
            const uint32_t ea = (col & 1) ? E1a : E0a, eb = (col & 1) ? E1b : E0b;
            const uint32_t e16 = __builtin_amdgcn_perm(eb, ea, 0x0C000C00u | ((4u + i) << 16) | i);
            const uint32_t x16 = (e16 << 7) + b7;
            const uint32_t s2 = __builtin_amdgcn_perm(sb, sa, q | (q << 8) | ((4u + q) << 16) | ((4u + q) << 24));
            kp[q] = (s2 & 0x807F807Fu) | (x16 & ~0x807F807Fu);
          }
          *reinterpret_cast<uint4 *>(dst + 4 * h) = make_uint4(kp[0], kp[1], kp[2], kp[3]);
        }
      }
    }
    if (wave * 64 < XP) {   // tid < XP; XP is a multiple of 64
      uint4 x = S.x;
      if (tail) x = make_uint4(x.x & S.xm, x.y & S.xm, x.z & S.xm, x.w & S.xm);
      const uint32_t t = xtid();
      *reinterpret_cast<uint4 *>(&xs[buf][(t / (KS / 8)) * XPITCH + 8 * (t % (KS / 8))]) = x;
    }
  };
  f32x4 acc[MSUB][NSUB];
#pragma unroll
  for (uint32_t mi = 0; mi < MSUB; ++mi)
#pragma unroll
    for (uint32_t ns = 0; ns < NSUB; ++ns) acc[mi][ns] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto mfma_step = [&](uint32_t buf) {
#pragma unroll
    for (uint32_t kc = 0; kc < KS / 32; ++kc) {   // 32-k chunks of the step
      const uint32_t kq = 16 * kc + 4 * (lane >> 4);
      bf16x8 b[NSUB];
#pragma unroll
      for (uint32_t ns = 0; ns < NSUB; ++ns) {
        const uint32_t n = wave * (kStrip / WAVES) + 16 * ns + (lane & 15);
        uint4 bw;
        bw.x = tile[buf][(kq + 0) * kPitchU + n];
        bw.y = tile[buf][(kq + 1) * kPitchU + n];
        bw.z = tile[buf][(kq + 2) * kPitchU + n];
        bw.w = tile[buf][(kq + 3) * kPitchU + n];
        b[ns] = __builtin_bit_cast(bf16x8, bw);
      }
#pragma unroll
      for (uint32_t mi = 0; mi < MSUB; ++mi) {
        const uint4 av = *reinterpret_cast<const uint4 *>(
            &xs[buf][(16 * mi + (lane & 15)) * XPITCH + 32 * kc + 8 * (lane >> 4)]);
        const bf16x8 af = __builtin_bit_cast(bf16x8, av);
#pragma unroll
        for (uint32_t ns = 0; ns < NSUB; ++ns)
          acc[mi][ns] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, b[ns], acc[mi][ns], 0, 0, 0);
      }
    }
  };

  // NB step buffers in a ring: step s + NB - 1 is loaded while step s is
  // decoded and multiplied. Loads are issued unconditionally (see
  // load_codes for slots past the last step), and the step count is rounded up to a
  // multiple of NB (steps past the K range decode to zeros), so every path
  // through the loop body is the same and the compiler waits for exactly the
  // step it needs.
  const uint32_t nst = (nsteps + NB - 1) / NB * NB;
  Step S[NB];
#pragma unroll
  for (uint32_t p = 0; p + 1 < NB; ++p) load_planes(p, S[p]);
  build_table();
#pragma unroll
  for (uint32_t p = 0; p + 1 < NB; ++p) load_codes(p, S[p]);
  for (uint32_t st = 0; st < nst; st += NB) {
#pragma unroll
    for (uint32_t j = 0; j < NB; ++j) {
      load_planes(st + j + NB - 1, S[(j + NB - 1) % NB]);
      load_codes(st + j + NB - 1, S[(j + NB - 1) % NB]);
      decode_step(st + j, S[j], (st + j) & 1);
      lds_barrier();
      mfma_step((st + j) & 1);
    }
  }

  auto outputs = [&](auto fn) {
#pragma unroll
    for (uint32_t mi = 0; mi < MSUB; ++mi)
#pragma unroll
      for (uint32_t ns = 0; ns < NSUB; ++ns)
#pragma unroll
        for (uint32_t j = 0; j < 4; ++j) {
          const uint32_t m = m0 + 16 * mi + 4 * (lane >> 4) + j;
          const uint32_t n = col0 + wave * (kStrip / WAVES) + 16 * ns + (lane & 15);
          fn(m < M ? (int64_t)m * N + n : (int64_t)-1, acc[mi][ns][j]);
        }
  };
  splitk_finish(a, ks, outputs);
}

template <bool DENSE>
hipError_t launch_valu(const GemmArgs &a, hipStream_t s) {
  const dim3 grid(a.N / kStrip, a.ksplit);
  switch (a.M) {
#define CASE(m) \
  case m: hipLaunchKernelGGL((k_gemm_valu<m, DENSE>), grid, dim3(256), 0, s, a); break;
    CASE(1) CASE(2)
#undef CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_rowu(const GemmArgs &a, hipStream_t s) {
  const dim3 grid(a.N / kStrip * a.ksplit);
  switch (a.M) {
#define CASE(m) \
  case m: hipLaunchKernelGGL((k_gemm_rowu<m>), grid, dim3(kRowuWaves * 64), 0, s, a); break;
    CASE(1)
#undef CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Step buffers per M tile size (ring depth of the prefetch). Measured at
// M = 16 / 32 / 128: two beat three (register pressure).
// K steps in the load ring (16- and 32-row tiles; 64 and 128)
constexpr int mfmau_nb(int MT) { return MT <= 32 ? ENC_MFMAU_NB : ENC_MFMAU_NB_BIG; }
// Rows per K step (16- and 32-row tiles; 64 and 128, whose X slice would not
// fit twice in LDS with 64-row steps)
constexpr int mfmau_ks(int MT) { return MT <= 32 ? ENC_MFMAU_KS : 32; }
// 16 waves per workgroup for every M tile: more waves share one decoded LDS
// tile and need fewer registers each (2 rows per wave per step), so the
// device holds more rows in flight with fewer split-K slices (measured on a
// 4096 x 14336 W, 16 waves over 4: M = 8 35.9 -> 29.8 us, M = 16 36.6 ->
// 31.6, M = 32 42.3 -> 38.9; with the X slice in LDS the 64- and 128-row
// tiles gained from 16 waves over 8 too). The split-K plan aims at one
// workgroup per CU for every M tile: two resident 16-row workgroups per CU
// (their registers and LDS allow it) were slower on a 4096 x 14336 W at
// M = 4 / 16 (29.3 / 31.8 us per call against 27.5 / 29.2): the CU's
// decode, LDS and barrier work per K step is the limit, not memory.
constexpr int kMfmauWaves = 16;
constexpr uint64_t kSlots16 = 256;
constexpr uint64_t kSlots32 = 256;
constexpr uint64_t kSlots64 = 256;
constexpr uint64_t kSlots128 = 256;

template <bool DENSE>
hipError_t launch_mfmau(const GemmArgs &a, hipStream_t s) {
  constexpr int W = kMfmauWaves;
  const uint32_t MT = mfmau_tile_m(a.M);
  const dim3 grid(a.N / kStrip * a.ksplit, (a.M + MT - 1) / MT), block(W * 64);
  switch (MT) {
    case 16: hipLaunchKernelGGL((k_gemm_mfmau<16, W, DENSE, mfmau_nb(16), mfmau_ks(16)>), grid, block, 0, s, a); break;
    case 32: hipLaunchKernelGGL((k_gemm_mfmau<32, W, DENSE, mfmau_nb(32), mfmau_ks(32)>), grid, block, 0, s, a); break;
    case 64: hipLaunchKernelGGL((k_gemm_mfmau<64, W, DENSE, mfmau_nb(64), mfmau_ks(64)>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((k_gemm_mfmau<128, W, DENSE, mfmau_nb(128), mfmau_ks(128)>), grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

uint32_t mfma_tile_m(uint32_t M) { return M <= 16 ? 16 : M <= 32 ? 32 : M <= 64 ? 64 : 128; }

template <bool DENSE>
hipError_t launch_mfma(const GemmArgs &a, hipStream_t s) {
  const uint32_t MT = mfma_tile_m(a.M);
  const dim3 grid(a.N / kTileN, a.ksplit, (a.M + MT - 1) / MT);
  switch (MT) {
    case 16: hipLaunchKernelGGL((k_gemm_mfma<16, DENSE>), grid, dim3(256), 0, s, a); break;
    case 32: hipLaunchKernelGGL((k_gemm_mfma<32, DENSE>), grid, dim3(256), 0, s, a); break;
    case 64: hipLaunchKernelGGL((k_gemm_mfma<64, DENSE>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((k_gemm_mfma<128, DENSE>), grid, dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// W stored [N, K] row-major -- the weight layout of a linear layer (output
// features x input features) -- and Y = X . W^T.
//
// A block of W is then B consecutive k of one output column n, so the group
// a lane decodes (8 consecutive k of one column) is exactly that lane's part
// of an MFMA B fragment: for v_mfma_f32_16x16x32_bf16, lane L holds k =
// 8 (L / 16) .. + 7 of column L % 16 ("ZipServ: Fast and Memory-Efficient LLM
// Inference with Hardware-Aware Lossless Compression", Abstract: decode
// straight into the matrix units' registers). No LDS transpose and no
// barrier: each wave owns 16 columns and a K range, streams its 16 rows of W
// (one group per lane per 32-k step, kNtDepth steps in flight) and keeps
// MSUB 16 x 16 accumulator tiles. The A fragment is 16 bytes of an X row.
// A lane's row stays fixed, so its block changes only at multiples of B in
// k: the prologue finds the offsets and metas of the (at most kNtBlocks)
// blocks of its K range, and the loop picks them with a wave-uniform index.
// Rows past M read a clamped row and multiply zeros; steps past the range
// load from past the buffer's range (zeros, no memory access).
// Cost: every wave load instruction touches 16 rows of W (and 16 rows of X),
// 32 bytes each, so this kernel is bound by cache-line accesses rather than
// by HBM bytes or load latency (prefetch depth 2, 4 or 8 all measured the
// same). It serves the block sizes below 512; k_gemm_ntu below, which reads
// 256 contiguous bytes per row, serves the rest (M = 16: 55 -> 28 us on a
// 14336 x 4096 W).
// --------------------------------------------------------------------------
constexpr uint32_t kNtCols = 16;     // columns per wave
constexpr uint32_t kNtWaves = 4;     // waves per workgroup
constexpr uint32_t kNtDepth = 4;     // 32-k steps in flight per wave
constexpr uint32_t kNtBlocks = 4;    // blocks per row and K range, at most

template <int MSUB, bool DENSE>
__global__ __launch_bounds__(kNtWaves * 64) void k_gemm_nt(GemmArgs a) {
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t K = a.K, N = a.N, M = a.M;
  const uint32_t n = (blockIdx.x * kNtWaves + wave) * kNtCols + (lane & 15);   // row of W
  const uint32_t kq = lane >> 4;                                                // group of the step
  const uint32_t k0 = blockIdx.y * a.krows;
  const uint32_t k1 = min(k0 + a.krows, K);
  const uint32_t nsteps = (k1 - k0) / 32;
  const uint32_t m0 = blockIdx.z * 16 * MSUB;
  const uint32_t log2b = a.log2b;
  const __amdgpu_buffer_rsrc_t rs = stream_rsrc(a.wstream, a.total);

  uint32_t b_off[kNtBlocks], b_meta[kNtBlocks];
#pragma unroll
  for (uint32_t j = 0; j < kNtBlocks; ++j) {
    b_off[j] = 0;
    b_meta[j] = 0;
  }
  if (!DENSE) {
    const uint32_t nblk = (k1 - k0) >> log2b;
#pragma unroll
    for (uint32_t j = 0; j < kNtBlocks; ++j) {
      if (j < nblk) {
        uint64_t off, mw;
        row_block<false>(a, ((uint64_t)n * K + k0 + (j << log2b)) >> log2b, off, mw);
        uint32_t w = (uint32_t)(mw >> 8) & 0xFFu;
        if (w > 8) w = 0;   // corrupted stream: decode as width 0 (reads stay range-checked)
        b_off[j] = (uint32_t)off;
        b_meta[j] = ((uint32_t)mw & 0xFFu) | (w << 8);
      }
    }
  }

  struct Slot {
    u32x2 sm;
    u32x3 q;
    uint4 dv;
    uint4 x[MSUB];
    uint32_t info;   // base | w << 8 | lead byte << 16
  };
  auto load = [&](uint32_t st, Slot &S) {
    const uint32_t dead = st < nsteps ? 0u : 0x80000000u;
    const uint32_t stc = min(st, nsteps - 1);
    const uint32_t k = k0 + 32 * stc + 8 * kq;
    if (DENSE) {
      S.dv = *reinterpret_cast<const uint4 *>(a.wdense + (uint64_t)n * K + k);
    } else {
      const uint32_t j = (32 * stc) >> log2b;                      // wave-uniform
      uint32_t off = b_off[0], meta = b_meta[0];
#pragma unroll
      for (uint32_t t = 1; t < kNtBlocks; ++t) {
        off = j == t ? b_off[t] : off;
        meta = j == t ? b_meta[t] : meta;
      }
      const uint32_t w = meta >> 8;
      const uint32_t pb = off + ((k & ((1u << log2b) - 1)) >> 3) * w;
      S.sm = __builtin_amdgcn_raw_buffer_load_b64(rs, (kHeaderBytes + n * K + k) | dead, 0, 0);
      S.q = __builtin_amdgcn_raw_buffer_load_b96(rs, (pb & ~3u) | dead, 0, 0);
      S.info = meta | ((pb & 3u) << 16);
    }
#pragma unroll
    for (uint32_t mi = 0; mi < MSUB; ++mi) {
      const uint32_t m = m0 + 16 * mi + (lane & 15);
      const uint4 v = *reinterpret_cast<const uint4 *>(a.x + (uint64_t)min(m, M - 1) * K + k);
      const bool in = m < M;
      S.x[mi] = make_uint4(in ? v.x : 0u, in ? v.y : 0u, in ? v.z : 0u, in ? v.w : 0u);
    }
  };

  f32x4 acc[MSUB];
#pragma unroll
  for (uint32_t mi = 0; mi < MSUB; ++mi) acc[mi] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const Slot &S) {
    uint4 bw;
    if (DENSE) {
      bw = S.dv;
    } else {
      const uint32_t w = (S.info >> 8) & 0xFFu, sh = (S.info >> 16) * 8;
      const uint32_t lo = __builtin_amdgcn_alignbit(S.q.y, S.q.x, sh);
      const uint32_t hi = __builtin_amdgcn_alignbit(S.q.z, S.q.y, sh);
      bw = join_group(lo, hi, w, (S.info & 0xFFu) * 0x01010101u, S.sm.x, S.sm.y);
    }
    const bf16x8 b = __builtin_bit_cast(bf16x8, bw);
#pragma unroll
    for (uint32_t mi = 0; mi < MSUB; ++mi)
      acc[mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, S.x[mi]), b, acc[mi],
                                                         0, 0, 0);
  };

  Slot R[kNtDepth];
#pragma unroll
  for (uint32_t p = 0; p + 1 < kNtDepth; ++p) load(p, R[p]);
  for (uint32_t st = 0; st < nsteps; st += kNtDepth) {
#pragma unroll
    for (uint32_t j = 0; j < kNtDepth; ++j) {
      load(st + j + kNtDepth - 1, R[(j + kNtDepth - 1) % kNtDepth]);
      if (st + j < nsteps) compute(R[j]);
    }
  }

  splitk_finish(a, blockIdx.y, [&](auto fn) {
#pragma unroll
    for (uint32_t mi = 0; mi < MSUB; ++mi)
#pragma unroll
      for (uint32_t j = 0; j < 4; ++j) {
        const uint32_t m = m0 + 16 * mi + 4 * (lane >> 4) + j;
        fn(m < M ? (int64_t)m * N + n : (int64_t)-1, acc[mi][j]);
      }
  });
}

// --------------------------------------------------------------------------
// [N, K] layout, B >= 512 (or dense W with K % 128 == 0): staged rows.
//
// k_gemm_nt's loads touch 16 rows of W per instruction, 32 bytes each. Here a
// workgroup (16 waves) owns TN rows of W (output columns) and walks its K
// range in steps of 128 k: 16 lanes decode 16 consecutive groups of one row
// (256 contiguous sign+mantissa bytes, one contiguous code run: with B >= 512
// a 128-k run lies in one block, so its width, base and offset are shared),
// and store them row-major in an LDS tile, where an MFMA B fragment (8
// consecutive k of one column) is one 16-byte read. The step's X slice (MT
// rows x 128 k) is staged next to it. Wave w multiplies n-subtile w mod
// (TN/16) over its share of the step's four 32-k slices; the waves that share
// an n-subtile add their accumulators at the end, in wave order
// (deterministic). Loads run two steps ahead and are issued on every path,
// as in k_gemm_mfmau.
// --------------------------------------------------------------------------
constexpr uint32_t kNtuWaves = 16;
constexpr uint32_t kNtuStepK = 128;
constexpr uint32_t kNtuPitch = kNtuStepK;          // bf16 per LDS row (256 bytes)
// Chunk c (8 bf16) of LDS row r sits at position c ^ (r % 16): an MFMA
// fragment read (lane l: row l % 16, chunk c0 + l / 16) is then free of bank
// conflicts, and so are the writes of whole rows. (Rows padded to 272 bytes
// cost the fragment reads twice the LDS cycles, measured on gfx950 with the
// SQ_LDS_BANK_CONFLICT counter: ds_read_b128 serves 16 lanes per cycle, not
// 16 consecutive ones.)
__device__ __forceinline__ uint32_t ntu_at(uint32_t row, uint32_t chunk) {
  return row * kNtuPitch + 8 * (chunk ^ (row & 15));
}
constexpr uint32_t kNtuMaxBlocks = 8;              // blocks per row and K range, at most

template <int MT, int TN, bool DENSE>
__global__ __launch_bounds__(kNtuWaves * 64) void k_gemm_ntu(GemmArgs a) {
  constexpr uint32_t NTHR = kNtuWaves * 64;
  constexpr uint32_t MSUB = MT / 16;
  constexpr uint32_t NSUBT = TN / 16;                      // n-subtiles of the tile
  constexpr uint32_t KG = kNtuWaves / NSUBT;               // waves sharing an n-subtile
  constexpr uint32_t KPW = 4 / KG;                         // 32-k slices per wave per step
  constexpr uint32_t GPT = TN * 16 / NTHR;                 // W groups per thread per step
  constexpr uint32_t XP = MT * 16;                         // 16-byte X pieces per step
  constexpr uint32_t XPT = (XP + NTHR - 1) / NTHR;         // X pieces per thread
  constexpr uint32_t NB = 2;
  static_assert(GPT >= 1 && KPW >= 1 && KG * KPW == 4, "tile shape");
  __shared__ __attribute__((aligned(16))) uint16_t wt[2][TN * kNtuPitch];
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][MT * kNtuPitch];
  __shared__ uint32_t tbl_off[DENSE ? 1 : TN * kNtuMaxBlocks], tbl_meta[DENSE ? 1 : TN * kNtuMaxBlocks];
  const uint32_t tid = threadIdx.x, lane = tid & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t K = a.K, N = a.N, M = a.M, log2b = a.log2b;
  const uint32_t n0 = blockIdx.x * TN, m0 = blockIdx.z * MT;
  const uint32_t k0 = blockIdx.y * a.krows;
  const uint32_t k1 = min(k0 + a.krows, K);
  const uint32_t nsteps = (k1 - k0) / kNtuStepK;
  const __amdgpu_buffer_rsrc_t rs = stream_rsrc(a.wstream, a.total);

  if (!DENSE) {
    const uint32_t jb = (k1 - k0) >> log2b;                // blocks per row in the range
    for (uint32_t i = tid; i < TN * jb; i += NTHR) {
      const uint32_t r = i / jb, j = i % jb;
      uint64_t off, mw;
      row_block<false>(a, ((uint64_t)(n0 + r) * K + k0 + (j << log2b)) >> log2b, off, mw);
      uint32_t w = (uint32_t)(mw >> 8) & 0xFFu;
      if (w > 8) w = 0;   // corrupted stream: decode as width 0 (reads stay range-checked)
      tbl_off[r * kNtuMaxBlocks + j] = (uint32_t)off;
      tbl_meta[r * kNtuMaxBlocks + j] = ((uint32_t)mw & 0xFFu) | (w << 8);
    }
    __syncthreads();
  }

  struct Step {
    u32x2 sm[GPT];
    u32x3 q[GPT];
    uint4 dv[GPT];
    uint4 x[XPT];
  };
  // group q of the step: row q / 16, k = kb + 8 (q % 16)
  auto load_step = [&](uint32_t st, Step &S) {
    const uint32_t dead = st < nsteps ? 0u : 0x80000000u;
    const uint32_t kb = k0 + kNtuStepK * min(st, nsteps - 1);
#pragma unroll
    for (uint32_t h = 0; h < GPT; ++h) {
      const uint32_t q = tid + NTHR * h;
      const uint32_t r = q >> 4, k = kb + 8 * (q & 15);
      if (DENSE) {
        S.dv[h] = *reinterpret_cast<const uint4 *>(a.wdense + (uint64_t)(n0 + r) * K + k);
      } else {
        const uint32_t j = (k - k0) >> log2b;
        const uint32_t off = tbl_off[r * kNtuMaxBlocks + j];
        const uint32_t meta = tbl_meta[r * kNtuMaxBlocks + j];
        const uint32_t w = meta >> 8;
        const uint32_t pb = off + ((k & ((1u << log2b) - 1)) >> 3) * w;
        S.sm[h] = __builtin_amdgcn_raw_buffer_load_b64(rs, (kHeaderBytes + (n0 + r) * K + k) | dead, 0, 0);
        S.q[h] = __builtin_amdgcn_raw_buffer_load_b96(rs, (pb & ~3u) | dead, 0, 0);
      }
    }
#pragma unroll
    for (uint32_t h = 0; h < XPT; ++h) {
      // X piece p: row p / 16, k = kb + 8 (p % 16); threads past XP load a
      // duplicate and do not store it
      const uint32_t p = (tid + NTHR * h) % XP;
      const uint32_t m = m0 + (p >> 4), kx = kb + 8 * (p & 15);
      const uint4 v = *reinterpret_cast<const uint4 *>(a.x + (uint64_t)min(m, M - 1) * K + kx);
      const bool in = m < M;
      S.x[h] = make_uint4(in ? v.x : 0u, in ? v.y : 0u, in ? v.z : 0u, in ? v.w : 0u);
    }
  };
  auto decode_step = [&](uint32_t st, const Step &S, uint32_t buf) {
    const uint32_t kb = k0 + kNtuStepK * st;
#pragma unroll
    for (uint32_t h = 0; h < GPT; ++h) {
      const uint32_t q = tid + NTHR * h;
      const uint32_t r = q >> 4, g = q & 15;
      uint4 v;
      if (DENSE) {
        v = S.dv[h];
      } else {
        const uint32_t k = kb + 8 * g;
        const uint32_t j = (k - k0) >> log2b;
        const uint32_t off = tbl_off[r * kNtuMaxBlocks + j];
        const uint32_t meta = tbl_meta[r * kNtuMaxBlocks + j];
        const uint32_t w = (meta >> 8) & 15u;
        uint32_t el, eh;
        if (__ballot(w != 4) == 0) {
          // every row of the wave has width 4 (most blocks of these
          // weights): a group's codes are one dword-aligned dword
          codes_to_bytes_w4(S.q[h].x, el, eh);
        } else {
          const uint32_t sh = ((off + ((k & ((1u << log2b) - 1)) >> 3) * w) & 3u) * 8;
          const uint32_t lo = __builtin_amdgcn_alignbit(S.q[h].y, S.q[h].x, sh);
          const uint32_t hi = __builtin_amdgcn_alignbit(S.q[h].z, S.q[h].y, sh);
          codes_to_bytes(lo, hi, w, el, eh);
        }
        v = bytes_to_bf16(el, eh, (meta & 0xFFu) * 0x01010101u, S.sm[h].x, S.sm[h].y);
      }
      *reinterpret_cast<uint4 *>(&wt[buf][ntu_at(r, g)]) = v;
    }
#pragma unroll
    for (uint32_t h = 0; h < XPT; ++h) {
      const uint32_t p = tid + NTHR * h;
      if (p < XP) *reinterpret_cast<uint4 *>(&xs[buf][ntu_at(p >> 4, p & 15)]) = S.x[h];
    }
  };

  const uint32_t ns = wave % NSUBT, kg = wave / NSUBT;
  f32x4 acc[MSUB];
#pragma unroll
  for (uint32_t mi = 0; mi < MSUB; ++mi) acc[mi] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto mfma_step = [&](uint32_t buf) {
#pragma unroll
    for (uint32_t t = 0; t < KPW; ++t) {
      const uint32_t kc = 4 * (kg * KPW + t) + (lane >> 4);   // 8-k chunk of the fragment
      const bf16x8 b = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const uint4 *>(&wt[buf][ntu_at(16 * ns + (lane & 15), kc)]));
#pragma unroll
      for (uint32_t mi = 0; mi < MSUB; ++mi) {
        const bf16x8 af = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4 *>(&xs[buf][ntu_at(16 * mi + (lane & 15), kc)]));
        acc[mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, b, acc[mi], 0, 0, 0);
      }
    }
  };

  Step S[NB];
  load_step(0, S[0]);
  for (uint32_t st = 0; st < nsteps; st += NB) {
#pragma unroll
    for (uint32_t j = 0; j < NB; ++j) {
      load_step(st + j + 1, S[(j + 1) % NB]);
      if (st + j < nsteps) {
        decode_step(st + j, S[j], (st + j) & 1);
        lds_barrier();
        mfma_step((st + j) & 1);
      }
    }
  }

  // waves kg = 1 .. KG-1 hand their sums to wave kg = 0 of the same
  // n-subtile, one at a time, through the (now free) W tile
  float *red = reinterpret_cast<float *>(&wt[0][0]);
  static_assert(NSUBT * 64 * MSUB * 4 * 4 <= sizeof(wt), "reduction buffer");
#pragma unroll 1
  for (uint32_t r = 1; r < KG; ++r) {
    __syncthreads();
    if (kg == r) {
#pragma unroll
      for (uint32_t mi = 0; mi < MSUB; ++mi)
        *reinterpret_cast<f32x4 *>(&red[((ns * MSUB + mi) * 64 + lane) * 4]) = acc[mi];
    }
    __syncthreads();
    if (kg == 0) {
#pragma unroll
      for (uint32_t mi = 0; mi < MSUB; ++mi)
        acc[mi] += *reinterpret_cast<const f32x4 *>(&red[((ns * MSUB + mi) * 64 + lane) * 4]);
    }
  }
  if (kg != 0) return;
  splitk_finish(a, blockIdx.y, [&](auto fn) {
#pragma unroll
    for (uint32_t mi = 0; mi < MSUB; ++mi)
#pragma unroll
      for (uint32_t j = 0; j < 4; ++j) {
        const uint32_t m = m0 + 16 * mi + 4 * (lane >> 4) + j;
        const uint32_t n = n0 + 16 * ns + (lane & 15);
        fn(m < M ? (int64_t)m * N + n : (int64_t)-1, acc[mi][j]);
      }
  });
}

template <bool DENSE>
hipError_t launch_nt(const GemmArgs &a, hipStream_t s, uint32_t msub) {
  const uint32_t mt = 16 * msub;
  const dim3 grid(a.N / (kNtCols * kNtWaves), a.ksplit, (a.M + mt - 1) / mt);
  const dim3 block(kNtWaves * 64);
  switch (msub) {
    case 1: hipLaunchKernelGGL((k_gemm_nt<1, DENSE>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_gemm_nt<2, DENSE>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((k_gemm_nt<4, DENSE>), grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

// M tile of k_gemm_nt in 16-row units (MSUB).
uint32_t nt_msub(uint32_t M) { return M <= 16 ? 1 : M <= 32 ? 2 : 4; }

// k_gemm_ntu serves a call when its 128-k steps and blocks line up: coded W
// with B >= 512 (K % B == 0 is checked by the caller), or dense W with
// K % 128 == 0. TN = 128 rows of W per workgroup when N allows, else 64.
constexpr uint32_t kNtuTN = 128;
bool ntu_ok(bool dense, uint32_t K, uint32_t log2b) { return dense ? K % kNtuStepK == 0 : log2b >= 9; }
uint32_t ntu_tn(uint32_t N) { return N % kNtuTN == 0 ? kNtuTN : 64; }

template <bool DENSE, int TN>
hipError_t launch_ntu_tn(const GemmArgs &a, hipStream_t s) {
  const uint32_t MT = mfmau_tile_m(a.M);
  const dim3 grid(a.N / TN, a.ksplit, (a.M + MT - 1) / MT), block(kNtuWaves * 64);
  switch (MT) {
    case 16: hipLaunchKernelGGL((k_gemm_ntu<16, TN, DENSE>), grid, block, 0, s, a); break;
    case 32: hipLaunchKernelGGL((k_gemm_ntu<32, TN, DENSE>), grid, block, 0, s, a); break;
    case 64: hipLaunchKernelGGL((k_gemm_ntu<64, TN, DENSE>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((k_gemm_ntu<128, TN, DENSE>), grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

template <bool DENSE>
hipError_t launch_ntu(const GemmArgs &a, hipStream_t s) {
  return ntu_tn(a.N) == 128 ? launch_ntu_tn<DENSE, 128>(a, s) : launch_ntu_tn<DENSE, 64>(a, s);
}

// k_gemm_ntu plan: one workgroup per CU (16 waves, up to 144 KB of LDS);
// K ranges of whole 128-k steps and whole blocks, at most kNtuMaxBlocks
// blocks per row, as many as it takes to fill the CUs.
void gemm_ntu_plan(bool dense, uint32_t M, uint32_t K, uint32_t N, uint32_t log2b, uint32_t *ksplit,
                   uint32_t *krows) {
  const uint32_t MT = mfmau_tile_m(M);
  const uint64_t tiles = (uint64_t)(N / ntu_tn(N)) * ((M + MT - 1) / MT);
  const uint64_t slots = 256;
  uint64_t ks = tiles >= slots ? 1 : slots / tiles;
  const uint32_t align = dense ? kNtuStepK : (1u << log2b);
  uint32_t rows = (uint32_t)((K + ks - 1) / ks);
  rows = (rows + align - 1) / align * align;
  if (!dense && rows > kNtuMaxBlocks * align) rows = kNtuMaxBlocks * align;
  *krows = rows;
  *ksplit = (K + rows - 1) / rows;
}

}  // namespace

// Which kernel serves a call: 0 = generic VALU (M < kMfmaMinM), 1 =
// uniform-row VALU (M < kMfmaMinMUniform, compressed, B >= 512, stream below
// 2 GiB: 32-bit buffer offsets), 2 = generic MFMA (M >= kMfmaMinM, B < 512),
// 3 = uniform-row MFMA (M >= kMfmaMinMUniform, dense W or B >= 512).

uint32_t gemm_kind(uint32_t M, bool dense, uint32_t log2b, uint64_t total) {
  const bool uniform = dense || (log2b >= 9 && total < (1ull << 31));
  if (uniform) return M >= kMfmaMinMUniform ? 3 : dense ? 0 : 1;
  return M >= kMfmaMinM ? 2 : 0;
}


void gemm_plan_kind(uint32_t kind, uint32_t M, uint32_t K, uint32_t N, uint32_t *ksplit,
                    uint32_t *krows) {
  if (kind == 0 || kind == 1) {
    const uint32_t rows = kind == 0 ? kValuRows : kRowuRange;
    *krows = rows;
    *ksplit = (K + rows - 1) / rows;
    return;
  }
  // enough workgroups to cover the CUs; at most 1024 rows per K range (the
  // per-row block offsets are kept in LDS), at least 64
  const uint32_t MT = kind == 3 ? mfmau_tile_m(M) : mfma_tile_m(M);
  const uint32_t ncol = kind == 3 ? kStrip : kTileN;
  const uint64_t tiles = (uint64_t)(N / ncol) * ((M + MT - 1) / MT);
  uint64_t ks;
  if (kind == 3) {
    // Resident k_gemm_mfmau workgroups (kSlots*: one per CU). Fill the
    // slots in one round: a partial second round doubles the time.
    const uint64_t slots = MT == 128 ? kSlots128 : MT == 64 ? kSlots64 : (MT == 16 ? kSlots16 : kSlots32);
    ks = tiles >= slots ? 1 : slots / tiles;
    if (ks >= 8) ks &= ~7ull;   // whole XCD groups (xcd_strip_range)
  } else {
    const uint64_t target = M <= 32 ? 512 : 256;
    ks = (target + tiles - 1) / tiles;
  }
  const uint64_t ks_min = (K + 1023) / 1024, ks_max = (K + 63) / 64;
  if (ks < ks_min) ks = ks_min;
  if (ks > ks_max) ks = ks_max;
  if (ks < 1) ks = 1;
  uint32_t rows = (uint32_t)((K + ks - 1) / ks);
  rows = (rows + kKStep - 1) / kKStep * kKStep;   // never increases the range count
  *krows = rows;
  *ksplit = (K + rows - 1) / rows;
}

void gemm_plan(uint32_t M, uint32_t K, uint32_t N, uint32_t *ksplit, uint32_t *krows) {
  gemm_plan_kind(M >= kMfmaMinM ? 2 : 0, M, K, N, ksplit, krows);
}

uint64_t gemm_counter_bytes(uint32_t N) { return align_up(4ull * (N / kStrip), kSectionAlign); }

uint64_t gemm_workspace_bytes(uint32_t M, uint32_t K, uint32_t N) {
  // the strips' arrival counters, then the split-K partial slices of
  // whichever kernel the call selects
  uint64_t most = 256;
  for (uint32_t kind = 0; kind < 4; ++kind) {
    const bool mfma_kind = kind >= 2;
    const bool used = kind == 3 || kind == 1 ? (M >= kMfmaMinMUniform) == mfma_kind
                                             : (M >= kMfmaMinM) == mfma_kind;
    if (!used) continue;
    uint32_t ks, kr;
    gemm_plan_kind(kind, M, K, N, &ks, &kr);
    const uint64_t partial = ks > 1 ? (uint64_t)ks * M * N * 4 : 0;
    if (partial > most) most = partial;
  }
  return gemm_counter_bytes(N) + most;
}

// [N, K]-layout GEMM plan: K ranges of whole blocks (at most kNtBlocks), as
// many as it takes to give the device about 3072 workgroups (measured on a
// 14336 x 4096 W: 3072 beat 1536 by ~11% at M = 1..128, 768 was slower).
void gemm_nt_plan(uint32_t M, uint32_t K, uint32_t N, uint32_t log2b, uint32_t *ksplit,
                  uint32_t *krows) {
  const uint32_t B = 1u << log2b;
  const uint32_t mt = 16 * nt_msub(M);
  const uint64_t tiles = (uint64_t)(N / (kNtCols * kNtWaves)) * ((M + mt - 1) / mt);
  uint64_t ks = tiles >= 3072 ? 1 : 3072 / tiles;
  if (ks < 1) ks = 1;
  uint32_t rows = (uint32_t)((K + ks - 1) / ks);
  rows = (rows + B - 1) / B * B;                     // whole blocks
  if (rows > kNtBlocks * B) rows = kNtBlocks * B;
  *krows = rows;
  *ksplit = (K + rows - 1) / rows;
}

uint64_t gemm_nt_workspace_bytes(uint32_t M, uint32_t K, uint32_t N, uint32_t log2b) {
  // the split-K slices of whichever kernel and plan a call with this block
  // size can select (coded, or a RAW stream / dense W multiplied directly)
  uint64_t most = 256;
  uint32_t ks, kr;
  for (int v = 0; v < 4; ++v) {
    const bool dense = v & 1;
    const uint32_t lb = dense ? 9u : log2b;
    if (v < 2)
      gemm_nt_plan(M, K, N, lb, &ks, &kr);
    else if (ntu_ok(dense, K, lb))
      gemm_ntu_plan(dense, M, K, N, lb, &ks, &kr);
    else
      continue;
    const uint64_t partial = ks > 1 ? (uint64_t)ks * M * N * 4 : 0;
    if (partial > most) most = partial;
  }
  return most;
}

hipError_t launch_splitk_reduce(const GemmArgs &a, hipStream_t s) {
  const uint64_t mn = (uint64_t)a.M * a.N;
  uint64_t blocks = (mn + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  const dim3 g((uint32_t)blocks), t(256);
  if (a.ksplit <= 4)
    hipLaunchKernelGGL(k_splitk_reduce<4>, g, t, 0, s, a.partial, a.y, mn, a.ksplit);
  else if (a.ksplit <= 8)
    hipLaunchKernelGGL(k_splitk_reduce<8>, g, t, 0, s, a.partial, a.y, mn, a.ksplit);
  else if (a.ksplit <= 16)
    hipLaunchKernelGGL(k_splitk_reduce<16>, g, t, 0, s, a.partial, a.y, mn, a.ksplit);
  else
    hipLaunchKernelGGL(k_splitk_reduce<32>, g, t, 0, s, a.partial, a.y, mn, a.ksplit);
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// M = 1 in the linear-layer layout (W [N, K], y = W . x): a workgroup owns
// R consecutive rows of W, whose K values give y[n] in full -- no split over
// K, no partial sums, no second launch. (Written for M up to 4, but from
// M = 2 on the staged-row MFMA kernel below was faster: on a 14336 x 4096 W,
// GPU time per call, this kernel 26.2-26.6 / 33.3 / 34.8 / 40.2 us at M = 1
// / 2 / 3 / 4 against 27.1-30.9 / 27.4 / 27.3 / 27.5 us; 2, 8 or 16 rows per
// workgroup were no faster than 4 at M = 1.)
//
// First the rows' block table: thread j describes block b_first + j (the
// absolute payload offset through row_block, {base, width}) in LDS; one
// barrier. Then the R rows' groups are taken as one run: lane t of the
// workgroup owns groups t, t + 256, ..., so every wave instruction reads 512
// contiguous sign+mantissa bytes and one contiguous run of codes, and (K
// being a multiple of 512) all of its 64 groups lie in one row. The loads of
// kGemvBatch groups per lane are issued before any of them is decoded (raw
// buffer loads over the stream: out-of-range dwords read 0). A lane
// multiplies its values with X (fp32 products of BF16 values, fp32 sums, in
// a fixed order); whenever a wave moves on to the next row, it adds up its
// lanes' sums (a fixed butterfly) into LDS, and the workgroup adds the four
// waves' sums in wave order: the result is deterministic.
// --------------------------------------------------------------------------
namespace {

constexpr uint32_t kGemvMaxM = 1;
constexpr uint32_t kGemvMaxK = 65536;
constexpr uint32_t kGemvRows = 4;                        // rows of W per workgroup
// groups per lane in flight: their W and X loads all go out before any of
// them is decoded
__host__ __device__ constexpr uint32_t gemv_batch(int mm) { return mm <= 2 ? 4 : 2; }
constexpr uint32_t kGemvMaxBlocks = kGemvRows * (kGemvMaxK / 128) + 1;

// XFIXED: the host has checked that 256 * gemv_batch(MM) groups are a whole
// number of rows (groups per row, then a power of two, divide it), so lane
// t's X chunks are the same in every iteration and are loaded once, before
// the loop; and, for a coded W, that B >= 512, so the 64 groups of a wave
// instruction (512 values from a multiple of 512) lie in one block, whose
// offset and {base, width} are then wave-uniform (scalar registers).
template <int MM, bool DENSE, bool XFIXED>
__global__ __launch_bounds__(256) void k_gemv_nt(GemmArgs a) {
  constexpr uint32_t R = kGemvRows;
  __shared__ uint32_t t_off[DENSE ? 1 : kGemvMaxBlocks], t_meta[DENSE ? 1 : kGemvMaxBlocks];
  __shared__ float red[R][4][MM];
  const uint32_t tid = threadIdx.x, lane = tid & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t K = a.K, N = a.N, log2b = a.log2b;
  const uint32_t n0 = blockIdx.x * R;
  const uint32_t nrows = N - n0 < R ? N - n0 : R;
  const uint32_t gpr = K >> 3;                        // groups per row
  const uint32_t ng = nrows * gpr;                    // groups of the workgroup
  const uint64_t e0 = (uint64_t)n0 * K;               // first value
  const uint64_t b_first = e0 >> log2b;
  const __amdgpu_buffer_rsrc_t rs = stream_rsrc(a.wstream, a.total);
  for (uint32_t i = tid; i < R * 4 * MM; i += 256) (&red[0][0][0])[i] = 0.f;
  if (!DENSE) {
    const uint32_t nblk = (uint32_t)(((e0 + (uint64_t)nrows * K - 1) >> log2b) - b_first + 1);
    for (uint32_t j = tid; j < nblk; j += 256) {
      uint64_t off, mw;
      row_block<false>(a, b_first + j, off, mw);
      uint32_t w = (uint32_t)(mw >> 8) & 0xFFu;
      if (w > 8) w = 0;   // corrupted stream: decode as width 0 (reads stay bounds-checked)
      t_off[j] = (uint32_t)off;
      t_meta[j] = ((uint32_t)mw & 0xFFu) | (w << 8);
    }
  }
  __syncthreads();
  float acc[MM];
#pragma unroll
  for (int m = 0; m < MM; ++m) acc[m] = 0.f;
  uint32_t cur = (64 * wave) / gpr;                   // this wave's row (uniform)
  auto flush = [&](uint32_t row) {
#pragma unroll
    for (int m = 0; m < MM; ++m) {
      float v = acc[m];
#pragma unroll
      for (uint32_t d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
      if (lane == 0 && row < R) red[row][wave][m] = v;
      acc[m] = 0.f;
    }
  };
  constexpr uint32_t NB = gemv_batch(MM);
  // With XFIXED, lane t holds X[m, 8 (i 256 + t) mod K ..] for every i.
  // (A 16-byte read of X per group instead, L2 hits: 26.4 us per call
  // against 24.4 at M = 1 on a 14336x4096 W.)
  uint4 xpre[XFIXED ? NB : 1][MM];
  if (XFIXED) {
#pragma unroll
    for (uint32_t i = 0; i < NB; ++i) {
      const uint32_t kc = 8 * ((i * 256 + tid) % gpr);
#pragma unroll
      for (int m = 0; m < MM; ++m) xpre[i][m] = *reinterpret_cast<const uint4 *>(a.x + (uint64_t)m * K + kc);
    }
  }
  // wave-uniform block parameters and 32-bit offsets inside the workgroup's
  // rows: 24.1 -> 23.2 us per call (M = 1, 14336x4096 W), fewer VALU
  // instructions per group
  constexpr bool UNIF = !DENSE && XFIXED;
  const uint32_t bmask = (1u << log2b) - 1;
  const uint32_t e0m = (uint32_t)(e0 & bmask);
  const uint32_t smbase = kHeaderBytes + (uint32_t)e0;
  const uint32_t log2gpr = 31 - __builtin_clz(gpr);
  for (uint32_t f0 = 0; f0 < ng; f0 += 256 * NB) {
    uint4 wv[NB], xs[NB][MM];
    u32x2 sm[NB];
    u32x3 qd[NB];
    uint32_t info[NB];
#pragma unroll
    for (uint32_t i = 0; i < NB; ++i) {
      const uint32_t f = f0 + i * 256 + tid;
      const uint32_t fc = f < ng ? f : ng - 1;         // loads stay on the rows
      const uint64_t e = e0 + 8ull * fc;
      const uint32_t kc = 8 * (fc % gpr);
#pragma unroll
      for (int m = 0; m < MM; ++m)
        xs[i][m] = XFIXED ? xpre[XFIXED ? i : 0][m] : *reinterpret_cast<const uint4 *>(a.x + (uint64_t)m * K + kc);
      if (DENSE) {
        wv[i] = *reinterpret_cast<const uint4 *>(a.wdense + e);
      } else if (UNIF) {
        const uint32_t fw = f0 + i * 256 + 64 * wave;
        const uint32_t fwc = fw < ng ? fw : ng - 64;
        const uint32_t le = e0m + 8 * fwc;
        const uint32_t j = le >> log2b;
        const uint32_t meta = __builtin_amdgcn_readfirstlane(t_meta[j]);
        const uint32_t boff = __builtin_amdgcn_readfirstlane(t_off[j]);
        const uint32_t w = meta >> 8;
        const uint32_t u = ((le & bmask) >> 3) + lane;
        const uint32_t pb = boff + u * w;
        sm[i] = __builtin_amdgcn_raw_buffer_load_b64(rs, smbase + 8 * (fwc + lane), 0, 0);
        qd[i] = __builtin_amdgcn_raw_buffer_load_b96(rs, pb & ~3u, 0, 0);
        info[i] = (meta & 0xFFu) | (w << 8) | ((pb & 3u) << 16);
      } else {
        const uint32_t j = (uint32_t)((e >> log2b) - b_first);
        const uint32_t meta = t_meta[j];
        const uint32_t w = meta >> 8;
        const uint32_t u = (uint32_t)((e & ((1ull << log2b) - 1)) >> 3);
        const uint32_t pb = t_off[j] + u * w;
        sm[i] = __builtin_amdgcn_raw_buffer_load_b64(rs, kHeaderBytes + (uint32_t)e, 0, 0);
        qd[i] = __builtin_amdgcn_raw_buffer_load_b96(rs, pb & ~3u, 0, 0);
        info[i] = (meta & 0xFFu) | (w << 8) | ((pb & 3u) << 16);
      }
    }
#pragma unroll
    for (uint32_t i = 0; i < NB; ++i) {
      const uint32_t fw = f0 + i * 256 + 64 * wave;   // the wave's first group (uniform)
      if (fw >= ng) break;
      const uint32_t row = XFIXED ? fw >> log2gpr : fw / gpr;
      if (row != cur) {
        flush(cur);
        cur = row;
      }
      if (!DENSE) {
        const uint32_t w = (info[i] >> 8) & 15u;
        uint32_t el, eh;
        if (UNIF ? __builtin_amdgcn_readfirstlane(w) == 4 : __ballot(w != 4) == 0) {
          // width 4 across the wave: a group's codes are one aligned dword
          codes_to_bytes_w4(qd[i].x, el, eh);
        } else {
          const uint32_t sh = ((info[i] >> 16) & 3u) * 8;
          const uint32_t lo = __builtin_amdgcn_alignbit(qd[i].y, qd[i].x, sh);
          const uint32_t hi = __builtin_amdgcn_alignbit(qd[i].z, qd[i].y, sh);
          codes_to_bytes(lo, hi, w, el, eh);
        }
        wv[i] = bytes_to_bf16(el, eh, (info[i] & 0xFFu) * 0x01010101u, sm[i].x, sm[i].y);
      }
      const uint32_t wd[4] = {wv[i].x, wv[i].y, wv[i].z, wv[i].w};
#pragma unroll
      for (int m = 0; m < MM; ++m) {
        const uint32_t xd[4] = {xs[i][m].x, xs[i][m].y, xs[i][m].z, xs[i][m].w};
        // v_dot2c_f32_bf16: both products of a bf16 pair added to the fp32
        // sum in one instruction, where unpacking the pairs and two FMAs
        // took six (GPU time per call on a 14336x4096 W at M = 1: 27.1-27.9
        // -> 25.6-25.7 us; dense twin 21.5 -> 21.1)
        float sum = acc[m];
#pragma unroll
        for (int h = 0; h < 4; ++h)
          sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wd[h]),
                                                __builtin_bit_cast(bf16x2, xd[h]), sum, false);
        acc[m] = sum;
      }
    }
  }
  flush(cur);
  __syncthreads();
  if (tid < nrows * MM) {
    const uint32_t r = tid / MM, m = tid % MM;
    a.y[(uint64_t)m * N + n0 + r] = ((red[r][0][m] + red[r][1][m]) + red[r][2][m]) + red[r][3][m];
  }
}

template <bool DENSE>
hipError_t launch_gemv_nt(const GemmArgs &a, hipStream_t s) {
  const dim3 grid((a.N + kGemvRows - 1) / kGemvRows), block(256);
  static_assert(kGemvMaxM == 1, "one instantiation per M");
  if ((256u * gemv_batch(1)) % (a.K >> 3) == 0 && (DENSE || a.log2b >= 9))
    hipLaunchKernelGGL((k_gemv_nt<1, DENSE, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((k_gemv_nt<1, DENSE, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace

// The GEMV serves M = 1 when K is a multiple of 512 (a wave's 64 groups
// then lie in one block for every block size), K <= kGemvMaxK, and the
// stream's offsets fit the 32-bit buffer offsets.
bool gemv_ok(bool dense, uint32_t M, uint32_t K, uint64_t total) {
  return M <= kGemvMaxM && K % 512 == 0 && K <= kGemvMaxK && (dense || total < (1ull << 31));
}

hipError_t launch_gemm_nt(const GemmArgs &a_in, hipStream_t s) {
  GemmArgs a = a_in;
  const bool dense = a.wstream == nullptr;
  hipError_t e;
  if (gemv_ok(dense, a.M, a.K, a.total))
    return dense ? launch_gemv_nt<true>(a, s) : launch_gemv_nt<false>(a, s);
  if (ntu_ok(dense, a.K, a.log2b)) {
    gemm_ntu_plan(dense, a.M, a.K, a.N, a.log2b, &a.ksplit, &a.krows);
    e = dense ? launch_ntu<true>(a, s) : launch_ntu<false>(a, s);
  } else {
    gemm_nt_plan(a.M, a.K, a.N, a.log2b, &a.ksplit, &a.krows);
    e = dense ? launch_nt<true>(a, s, nt_msub(a.M)) : launch_nt<false>(a, s, nt_msub(a.M));
  }
  if (e != hipSuccess || a.ksplit == 1) return e;
  return launch_splitk_reduce(a, s);
}

hipError_t launch_gemm(const GemmArgs &a_in, hipStream_t s) {
  GemmArgs a = a_in;
  const bool dense = a.wstream == nullptr;
  const uint32_t kind = gemm_kind(a.M, dense, a.log2b, a.total);
  gemm_plan_kind(kind, a.M, a.K, a.N, &a.ksplit, &a.krows);
  hipError_t e;
  // arrival counters (in-kernel split-K reduction): the small-M kernel only.
  // (The MFMA kernels' last workgroup of a strip would add up to 256 KB of
  // slices alone; measured slower than the reduction kernel at every M.)
  if (kind != 1 || a.ksplit == 1) a.counters = nullptr;
  if (kind == 1)
    e = launch_rowu(a, s);
  else if (kind == 0)
    e = dense ? launch_valu<true>(a, s) : launch_valu<false>(a, s);
  else if (kind == 3)
    e = dense ? launch_mfmau<true>(a, s) : launch_mfmau<false>(a, s);
  else
    e = dense ? launch_mfma<true>(a, s) : launch_mfma<false>(a, s);
  if (e != hipSuccess || a.ksplit == 1 || a.counters) return e;
  return launch_splitk_reduce(a, s);
}

}  // namespace enc
