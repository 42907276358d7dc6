// encode_onepass.hip -- single-pass gfx950 encoder: reads the input once.
//
// "ENEC: A Lossless AI Model Compression Method Enabling Fast Inference on
// Ascend NPUs", Abstract: block widths, bit-packing and a branch-free
// transform per block, with a dependency-decoupled scan for the prefix sums
// of block sizes. The scan across tiles here is a decoupled look-back: every
// tile publishes its payload total as soon as it knows it, and a tile finds
// its own offset by walking back over its predecessors' published totals
// until it meets one that already carries a full prefix.
//
// One workgroup per tile of SUB x 1024 groups (SUB x 8192 values: whole
// blocks; tile = workgroup index). A published prefix can only advance about
// one 64-tile window per memory round trip, so large inputs take SUB = 4 (one
// look-back per 32768 values); small ones take fewer, to fill the device.
// Workgroups are dispatched in index order, so a workgroup only ever waits
// for tiles whose workgroups are already resident or finished: the lowest
// unfinished one always proceeds. (A shared atomic ticket would not need that
// ordering, but every workgroup would then update one address, which was
// slower still.) Should a wait ever give up anyway, the host discards the
// result and runs the two-pass encoder.
// For each 8192-value sub-tile, in turn (the next one's loads in flight):
//  1. per-block exponent min/max: lanes of one block reduce with packed
//     16-bit max over DPP lane exchanges, then one LDS atomic per block and
//     wave;
//  2. wave 0: base, width, padded payload size and offset (inside the
//     workgroup's payload) of each block; writes the block metas;
//  3. all lanes: sign+mantissa bytes to the stream, codes into a zeroed LDS
//     image of the workgroup's payload (so pad bits are zero).
// Per group the work is byte-parallel, as in the decoder: v_perm splits the
// exponent and sign+mantissa bytes of 4 values at once, min/max use packed
// 16-bit integer ops, and 4 codes pack with one bit-field extract each.
// Once the last sub-tile's block sizes are known, wave 0 publishes the
// workgroup's payload total and reads the first look-back window, and that
// read is in flight while the last sub-tile is packed. Then wave 0 finishes
// the look-back for the workgroup's offset, publishes the prefix, stores the offsets of the segments that
// start in this tile (and, in the last tile, the stream's payload size), and
// the LDS image goes out with 16-byte stores.
// Status words hold flag and value together and are read and written with
// agent-scope relaxed atomics, so no fence is needed; every wait is bounded
// (on give-up the kernel flags an error and the host falls back).
#include "encode_batch.h"
#include "group_math.h"

namespace enc {
namespace {

constexpr uint64_t kFlagAgg = 1ull << 62;    // value = this tile's payload bytes
constexpr uint64_t kFlagPre = 2ull << 62;    // value = payload bytes of tiles 0..t
constexpr uint64_t kValMask = (1ull << 62) - 1;

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Cache-policy operand of the buffer stores of the sm plane and payloads:
// the non-temporal hint (the stream is written once and not read back by
// the encoder; the 8B-shaped set encodes 2% faster with it).
constexpr int kStoreNT = 2;


__device__ __forceinline__ uint64_t wave_sum64(uint64_t v) {
#pragma unroll
  for (uint32_t d = 1; d < 64; d <<= 1) v += __shfl_xor(v, d, 64);
  return v;
}

// Status words, the size slot, the error word and the segment offsets are
// addressed through global-address-space pointers. In the batched kernel
// the arguments come from a table in memory, and the compiler would
// otherwise reach them with flat instructions, which count against the LDS
// wait counter as well: the early read of the first look-back window would
// then hold up every LDS wait of the last sub-tile's pack instead of
// overlapping it.
#define ENC_GLOBAL __attribute__((address_space(1)))
typedef ENC_GLOBAL uint64_t gu64;
#ifndef ENC_SHORT_SLEEP
#define ENC_SHORT_SLEEP 8
#endif
typedef ENC_GLOBAL uint32_t gu32;

__device__ __forceinline__ void publish(gu64 *status, uint64_t tile, uint64_t word) {
  __hip_atomic_store(status + tile, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Lane l's status word of the window whose top is tile `top` (positions
// below tile 0 read as a full prefix of 0).
__device__ __forceinline__ uint64_t window_word(gu64 *status, int64_t top, uint32_t lane) {
  const int64_t idx = top - (int64_t)lane;
  return idx >= 0 ? __hip_atomic_load(status + idx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                  : kFlagPre;
}

// Sum of the payload totals of tiles [0, tile), by the whole wave. Lane l
// reads tile top - l; the window is usable once every tile from the top down
// to the nearest full prefix has published; otherwise the wave sleeps
// (about 3 microseconds) and reads it again. `first` is the caller's read of the first
// window (top = tile - 1), issued early so that its latency overlaps work.
__device__ uint64_t look_back(gu64 *status, uint64_t tile, uint32_t lane, gu32 *error,
                              uint32_t spin_limit, uint32_t short_sleep, uint64_t first) {
  uint64_t excl = 0;
  int64_t top = (int64_t)tile - 1;
  uint32_t spins = 0;
  uint64_t v = first;
  // spin limit 0 (a test setting): every tile with a predecessor gives up at
  // once, whatever its window holds, so the host's fallback always runs
  if (spin_limit == 0 && top >= 0) {
    if (lane == 0) __hip_atomic_fetch_or(error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return 0;
  }
  while (top >= 0) {
    const uint64_t flag = v >> 62;
    const uint64_t pre = __ballot(flag == 2);
    const uint64_t none = __ballot(flag == 0);
    const uint64_t need = pre ? ((pre & (~pre + 1)) << 1) - 1 : ~0ull;   // lanes up to the first prefix
    if (none & need) {
      if (++spins > spin_limit) {
        if (lane == 0) __hip_atomic_fetch_or(error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return 0;
      }
      // Large launches: the longest sleep (127 x 64 clocks), so that the
      // polls of many waiting workgroups do not crowd the memory system
      // (measured on the 8B-shaped set, batched: sleep 1 6.77 ms, 32 6.41,
      // 64 6.20, 127 5.95, two of 127 6.13). Small launches (one tensor of
      // a few thousand tiles) poll after a short one: their few waiting
      // workgroups cost the memory system little, and each long sleep sat on
      // the tensor's critical path (4.2M-value tensor, 512 tiles: kernel
      // 12.2 -> 9.0 us; sleeps of 2, 8 and 32 x 64 clocks measured alike).
      // (Walking back with the whole workgroup, 256 tiles per round trip,
      // was slower: 11.3 us.)
      if (short_sleep)
        __builtin_amdgcn_s_sleep(ENC_SHORT_SLEEP);
      else
        __builtin_amdgcn_s_sleep(127);
      v = window_word(status, top, lane);
      continue;
    }
    excl += wave_sum64(((need >> lane) & 1) ? (v & kValMask) : 0);
    if (pre) break;
    top -= 64;
    v = window_word(status, top, lane);
  }
  return excl;
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Barrier that waits for LDS traffic only: __syncthreads() would also wait
// for every outstanding global load and store (on this part one counter
// covers both), which would drain the next sub-tile's prefetch.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Raw buffer descriptor over [base, base + bytes). The CDNA3 ISA reference
// guide's range checking for buffer instructions (stride 0: out of range at
// or past num_records, checked per dword of a multi-dword access; CDNA4 keeps
// the rule) makes the hardware drop stores and zero-fill loads of dwords that
// do not lie wholly inside, so every lane issues its loads and stores
// unconditionally (a load or store under a branch would make the compiler
// wait for all outstanding memory operations).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t range_rsrc(const void *base, uint64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0,
                                           (int)(uint32_t)(bytes < 0xFFFFFFF0ull ? bytes : 0xFFFFFFF0ull),
                                           0x00020000);
}

// Loads the 4 groups of this lane in sub-tile `sub` of the workgroup's tile;
// offsets are relative to the tile start. A group cut short by the end of
// the input is completed with copies of its first value (x_last: the input's
// last value, needed when n is odd because its dword straddles the end), so
// exponent min / max need no masking; the bytes it would add to the stream
// are masked off when packing.
__device__ __forceinline__ void load_sub(__amdgpu_buffer_rsrc_t in_rs, uint64_t left, uint32_t sub,
                                         uint32_t tid, uint32_t x_last,
                                         uint4 (&g)[kGroupsPerThread],
                                         uint32_t (&valid)[kGroupsPerThread]) {
#pragma unroll
  for (uint32_t it = 0; it < kGroupsPerThread; ++it) {
    const uint32_t e0 = (sub * kTileGroups + it * kThreads + tid) * 8;   // from the tile start
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(in_rs, 2 * e0, 0, 0);
    g[it] = make_uint4(v.x, v.y, v.z, v.w);
    valid[it] = e0 < left ? (left - e0 < 8 ? (uint32_t)(left - e0) : 8u) : 0u;
  }
  (void)x_last;
}

// The end-of-input fix-up described above (no memory access).
__device__ __forceinline__ void complete_group(uint4 &g, uint32_t valid, uint32_t x_last) {
  uint32_t x[8] = {g.x & 0xFFFFu, g.x >> 16, g.y & 0xFFFFu, g.y >> 16,
                   g.z & 0xFFFFu, g.z >> 16, g.w & 0xFFFFu, g.w >> 16};
  if (valid & 1) x[valid - 1] = x_last;   // n odd: the last value's dword read as 0
#pragma unroll
  for (uint32_t k = 1; k < 8; ++k)
    if (k >= valid) x[k] = x[0];
  g = make_uint4(x[0] | x[1] << 16, x[2] | x[3] << 16, x[4] | x[5] << 16, x[6] | x[7] << 16);
}

// Exponent bytes of a group's 8 values (el: values 0..3, eh: 4..7). A BF16
// value shifted left by one carries its exponent in its high byte.
__device__ __forceinline__ void exp_bytes(const uint4 &g, uint32_t &el, uint32_t &eh) {
  el = __builtin_amdgcn_perm(g.y << 1, g.x << 1, 0x07050301u);
  eh = __builtin_amdgcn_perm(g.w << 1, g.z << 1, 0x07050301u);
}

// Sign+mantissa bytes (sign in bit 7, mantissa in bits 6..0) of 4 values.
__device__ __forceinline__ uint32_t sm_bytes(uint32_t x01, uint32_t x23) {
  const uint32_t lo = __builtin_amdgcn_perm(x23, x01, 0x06040200u);   // low byte of each value
  const uint32_t hi = __builtin_amdgcn_perm(x23, x01, 0x07050301u);   // high byte of each value
  return (hi & 0x80808080u) | (lo & 0x7F7F7F7Fu);
}

// ((255 - min) << 16) | max over the 8 exponent bytes, with packed 16-bit
// min / max (no packed-float instructions involved).
__device__ __forceinline__ uint32_t minmax_key(uint32_t el, uint32_t eh) {
  const u16x2 a = __builtin_bit_cast(u16x2, el & 0x00FF00FFu);
  const u16x2 b = __builtin_bit_cast(u16x2, (el >> 8) & 0x00FF00FFu);
  const u16x2 c = __builtin_bit_cast(u16x2, eh & 0x00FF00FFu);
  const u16x2 d = __builtin_bit_cast(u16x2, (eh >> 8) & 0x00FF00FFu);
  const u16x2 mn = __builtin_elementwise_min(__builtin_elementwise_min(a, b),
                                             __builtin_elementwise_min(c, d));
  const u16x2 mx = __builtin_elementwise_max(__builtin_elementwise_max(a, b),
                                             __builtin_elementwise_max(c, d));
  const uint32_t lo = mn.x < mn.y ? mn.x : mn.y, hi = mx.x > mx.y ? mx.x : mx.y;
  return ((255u - lo) << 16) | hi;
}

// Four code bytes (each < 2^w) packed LSB first at width w: 4w bits.
__device__ __forceinline__ uint32_t pack4(uint32_t d, uint32_t w) {
  return __builtin_amdgcn_ubfe(d, 0, 8) | (__builtin_amdgcn_ubfe(d, 8, 8) << w) |
         (__builtin_amdgcn_ubfe(d, 16, 8) << (2 * w)) | ((d >> 24) << (3 * w));
}

// One workgroup's tile of stream `a` (the kernel body, shared by the
// single-stream and the batched launch).
template <uint32_t SUB>
__device__ __forceinline__ void onepass_tile(const EncodeArgs &a, uint64_t tile) {
  constexpr uint32_t kPayBytes = SUB * kTileGroups * 8 + 16;   // a tile's payload, at most
  __shared__ __attribute__((aligned(16))) uint32_t pay[kPayBytes / 4];
  __shared__ uint32_t smin[64], smax[64], sblk[64], s_suboff[SUB];
  __shared__ uint64_t s_excl;
  __shared__ uint32_t s_run;
  const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t log2b = a.log2b, log2gpb = log2b - 3;
  const uint32_t bps = (uint32_t)(kTileElems >> log2b);            // blocks per sub-tile
  const uint64_t n = a.n;
  const uint64_t start = tile * SUB * kTileElems;         // first value of the tile
  const uint64_t left = n - start;                                 // values from the tile start on
  const uint32_t nsub = (uint32_t)((left < SUB * kTileElems ? left : SUB * kTileElems) +
                                   kTileElems - 1) / kTileElems;
  const uint64_t span_vals = left < SUB * kTileElems ? left : SUB * kTileElems;
  const uint32_t span = (1u << log2gpb) < 64 ? (1u << log2gpb) : 64u;   // lanes of one block
  const __amdgpu_buffer_rsrc_t in_rs = range_rsrc(a.in + start, 2 * span_vals);
  // sign+mantissa plane of the tile, up to the 8-value boundary (the plane's
  // padding is zero, and so are the masked bytes of a short last group)
  const __amdgpu_buffer_rsrc_t sm_rs = range_rsrc(a.out + kHeaderBytes + start, align_up(span_vals, 8));
  const uint32_t x_last = *(const ENC_GLOBAL uint16_t *)(a.in + n - 1);
  gu64 *const status = (gu64 *)a.status;

  if (tid < 64) {
    smin[tid] = 255;
    smax[tid] = 0;
  }
  if (tid == 0) s_run = 0;
  for (uint32_t i = tid; i < kPayBytes / 16; i += kThreads)
    reinterpret_cast<uint4 *>(pay)[i] = make_uint4(0u, 0u, 0u, 0u);

  uint64_t lb_first = kFlagPre;   // wave 0: first look-back window, read early
  uint4 g[kGroupsPerThread], gn[kGroupsPerThread];
  uint32_t valid[kGroupsPerThread], vn[kGroupsPerThread];
  load_sub(in_rs, left, 0, tid, x_last, g, valid);
#pragma unroll 1
  for (uint32_t sub = 0; sub < nsub; ++sub) {
    const uint64_t st = tile * SUB + sub;                  // global sub-tile index
    const uint64_t blk0 = st * bps;
    // next sub-tile, in flight (past the tile's last one every dword is out of
    // the descriptor's range: zeros, and no memory access)
    load_sub(in_rs, left, sub + 1, tid, x_last, gn, vn);
#pragma unroll
    for (uint32_t it = 0; it < kGroupsPerThread; ++it)
      if (valid[it] - 1 < 7) complete_group(g[it], valid[it], x_last);   // 1 <= valid < 8
    lds_barrier();   // previous sub-tile packed (sblk free), min/max reset

    // per-block min / max exponent
#pragma unroll
    for (uint32_t it = 0; it < kGroupsPerThread; ++it) {
      uint32_t el, eh;
      exp_bytes(g[it], el, eh);
      uint32_t key = valid[it] ? minmax_key(el, eh) : 0u;   // 0: no valid value here
      key = span_max16(key, span);
      const uint32_t q = it * kThreads + tid;
      if ((lane & (span - 1)) == span - 1 && key != 0) {
        atomicMin(&smin[q >> log2gpb], 255u - (key >> 16));
        atomicMax(&smax[q >> log2gpb], key & 0xFFFFu);
      }
    }
    lds_barrier();

    // block parameters, metas, offsets inside the workgroup's payload
    if (wave == 0) {
      const uint64_t blk = blk0 + lane;
      uint32_t P = 0, base = 0, w = 0;
      if (lane < bps && blk < a.nb) {
        base = smin[lane];
        const uint32_t r = smax[lane] - base;
        w = block_width(r, a.pow2);
        const uint32_t L = (blk + 1 == a.nb) ? (uint32_t)(n - ((a.nb - 1) << log2b)) : (1u << log2b);
        P = (((w * L + 7) >> 3) + 15) & ~15u;
      }
      // metas of this sub-tile, two per dword store. The range is rounded up
      // to whole dwords (a lone last meta's neighbour is a zero pad byte pair
      // of the meta section); pairs past it are dropped.
      const __amdgpu_buffer_rsrc_t meta_rs = range_rsrc(
          a.out + a.meta_off + 2 * blk0, align_up(2 * (a.nb - blk0 < bps ? a.nb - blk0 : bps), 4));
      const uint32_t mw = base | (w << 8);
      const uint32_t pair = mw | (__shfl_down(mw, 1, 64) << 16);
      if (!(lane & 1)) __builtin_amdgcn_raw_buffer_store_b32(pair, meta_rs, 2 * lane, 0, 0);
      smin[lane] = 255;
      smax[lane] = 0;
      const uint32_t run = s_run;
      const uint32_t incl = wave_incl_scan(P);
      const uint32_t sub_total = __builtin_amdgcn_readlane(incl, 63);
      sblk[lane] = base | (w << 8) | ((run + incl - P) << 16);
      if (lane == 0) {
        s_suboff[sub] = run;
        s_run = run + sub_total;
      }
      if (sub + 1 == nsub) {
        // the workgroup's payload total is known: publish it and read the
        // first look-back window now, so that the read is in flight while
        // the last sub-tile is packed
        if (lane == 0) publish(status, tile, (tile == 0 ? kFlagPre : kFlagAgg) | (run + sub_total));
        lb_first = window_word(status, (int64_t)tile - 1, lane);
      }
    }
    lds_barrier();

    // sign+mantissa plane and the payload image. A group's codes are w bytes
    // at byte `pos` of the image; they are OR-ed into the (at most three)
    // dwords they touch, with LDS atomics since neighbouring groups share
    // dwords.
#pragma unroll
    for (uint32_t it = 0; it < kGroupsPerThread; ++it) {
      const uint32_t q = it * kThreads + tid;
      const uint32_t info = sblk[q >> log2gpb];
      const uint32_t w = (info >> 8) & 0xFFu, base4 = (info & 0xFFu) * 0x01010101u;
      uint32_t el, eh;
      exp_bytes(g[it], el, eh);
      uint32_t s0 = sm_bytes(g[it].x, g[it].y), s1 = sm_bytes(g[it].z, g[it].w);
      const uint32_t c0 = pack4(el - base4, w), c1 = pack4(eh - base4, w);   // bytes: no borrows
      uint32_t lo = w == 8 ? c0 : c0 | (c1 << (4 * w));
      uint32_t hi = w == 8 ? c1 : (w > 4 ? c1 >> (32 - 4 * w) : 0u);
      const uint32_t v = valid[it];
      if (v < 8) {   // zero what lies past the end of the input (all of it if v == 0)
        const uint32_t bits = v * w;
        s0 &= v >= 4 ? ~0u : (1u << (8 * v)) - 1;
        s1 &= v <= 4 ? 0u : (1u << (8 * (v - 4))) - 1;
        lo &= bits >= 32 ? ~0u : (1u << bits) - 1;
        hi &= bits <= 32 ? 0u : (1u << (bits - 32)) - 1;
      }
      __builtin_amdgcn_raw_buffer_store_b64((u32x2){s0, s1}, sm_rs, 8 * (sub * kTileGroups + q), 0, kStoreNT);
      const uint32_t pos = (info >> 16) + (q & ((1u << log2gpb) - 1)) * w;
      const uint32_t sh = (pos & 3) * 8, d0 = pos >> 2;
      const uint32_t w0 = lo << sh;
      const uint32_t w1 = sh ? (lo >> (32 - sh)) | (hi << sh) : hi;
      const uint32_t w2 = sh ? hi >> (32 - sh) : 0u;
      if (w0) atomicOr(&pay[d0], w0);
      if (w1) atomicOr(&pay[d0 + 1], w1);
      if (w2) atomicOr(&pay[d0 + 2], w2);
    }
#pragma unroll
    for (uint32_t it = 0; it < kGroupsPerThread; ++it) {
      g[it] = gn[it];
      valid[it] = vn[it];
    }
  }
  lds_barrier();

  // the workgroup's payload offset
  if (wave == 0) {
    const uint32_t agg = s_run;
    const uint64_t excl = look_back(status, tile, lane, (gu32 *)a.error, a.spin_limit, a.short_sleep,
                                    lb_first);
    if (lane == 0) {
      if (tile > 0) publish(status, tile, kFlagPre | (excl + agg));
      if (tile + 1 == a.ntiles) *(gu64 *)a.ws_total = excl + agg;
      s_excl = excl;
    }
    if (lane < nsub && (((tile * SUB + lane) * bps) & 63) == 0)   // segment starts
      *(gu64 *)(a.out + a.segoff_off +
                                    8 * (((tile * SUB + lane) * bps) >> 6)) = excl + s_suboff[lane];
  }
  lds_barrier();

  // payload out
  const uint64_t dst = a.payload_off + s_excl;
  const __amdgpu_buffer_rsrc_t pay_rs = range_rsrc(a.out + dst, a.cap > dst ? a.cap - dst : 0);
  for (uint32_t i = tid; i < s_run / 16; i += kThreads) {
    const uint4 d = reinterpret_cast<const uint4 *>(pay)[i];
    __builtin_amdgcn_raw_buffer_store_b128((u32x4){d.x, d.y, d.z, d.w}, pay_rs, 16 * i, 0, kStoreNT);
  }
}

template <uint32_t SUB>
__global__ __launch_bounds__(kThreads) void k_enc_onepass(EncodeArgs a) {
  onepass_tile<SUB>(a, blockIdx.x);
}

// Many streams in one launch (table layout in encode_batch.h): workgroup b
// runs tile b - begin[k] of the stream k whose range holds b. Tiles of one
// stream keep their order, so the look-back still only waits for workgroups
// dispatched earlier. All streams take the largest tile (kOnePassMaxSub
// sub-tiles): with many streams in flight at once, small ones no longer
// need more workgroups to fill the device.
__global__ __launch_bounds__(kThreads) void k_enc_onepass_batch(const uint8_t *__restrict__ table) {
  const EncBatchHeader *h = reinterpret_cast<const EncBatchHeader *>(table);
  const uint32_t count = h->count;
  const EncodeArgs *items = reinterpret_cast<const EncodeArgs *>(table + sizeof(EncBatchHeader));
  const uint64_t *begin = reinterpret_cast<const uint64_t *>(table + sizeof(EncBatchHeader) +
                                                             count * sizeof(EncodeArgs));
  const uint64_t b = blockIdx.x;
  uint32_t lo = 0, hi = count;
  while (hi - lo > 1) {
    const uint32_t mid = (lo + hi) / 2;
    if (begin[mid] <= b) lo = mid; else hi = mid;
  }
  const EncodeArgs a = items[lo];
  onepass_tile<kOnePassMaxSub>(a, b - begin[lo]);
}

// ---------------------------------------------------------------------------
// FP16 (DT 2) and FP32 (DT 3) input in one pass: the same tile schedule,
// block parameters and decoupled look-back as the BF16 tile above, with the
// other float layouts' fields (FP16: 5 exponent bits, the sign and 10
// mantissa bits kept as an 11-bit field; FP32: 8 exponent bits, a 24-bit
// kept field). A group of 8 values owns exactly 11 or 24 bytes of the kept
// section, so each sub-tile's kept fields are assembled in a zeroed LDS image
// (fixed position in the stream: no look-back needed) and leave with 16-byte
// stores while the codes collect in the workgroup's payload image.
// ---------------------------------------------------------------------------
template <uint32_t DT>
struct WideField {
  static constexpr uint32_t kBytes = DT == 3 ? 4 : 2;     // input bytes per value
  static constexpr uint32_t kSmBits = DT == 3 ? 24 : 11;  // kept bits per value
  static constexpr uint32_t kShift = DT == 3 ? 23 : 10;   // exponent position
  static constexpr uint32_t kExpMask = DT == 3 ? 0xFFu : 0x1Fu;
  static constexpr uint32_t kChunks = DT == 3 ? 2 : 1;    // 16-byte loads per group
};

// Value k of a group loaded as WideField<DT>::kChunks 16-byte pieces.
template <uint32_t DT>
__device__ __forceinline__ uint32_t wide_value(const uint4 (&r)[WideField<DT>::kChunks], uint32_t k) {
  if (DT == 3) {
    const uint4 &c = r[(k >> 2) & (WideField<DT>::kChunks - 1)];
    const uint32_t j = k & 3;
    return j == 0 ? c.x : j == 1 ? c.y : j == 2 ? c.z : c.w;
  }
  const uint32_t j = k >> 1;
  const uint32_t d = j == 0 ? r[0].x : j == 1 ? r[0].y : j == 2 ? r[0].z : r[0].w;
  return (d >> (16 * (k & 1))) & 0xFFFFu;
}

template <uint32_t DT, uint32_t SUB>
__device__ __forceinline__ void onepass_tile_wide(const EncodeArgs &a, uint64_t tile) {
  typedef WideField<DT> F;
  constexpr uint32_t CH = F::kChunks;
  constexpr uint32_t kPayBytes = SUB * kTileGroups * 8 + 16;   // a tile's payload, at most
  constexpr uint32_t kTileSm = kTileGroups * F::kSmBits;       // kept bytes of a sub-tile (x16)
  __shared__ __attribute__((aligned(16))) uint32_t pay[kPayBytes / 4];
  __shared__ __attribute__((aligned(16))) uint32_t smi[kTileSm / 4 + 4];
  __shared__ uint32_t smin[64], smax[64], sblk[64], s_suboff[SUB];
  __shared__ uint64_t s_excl;
  __shared__ uint32_t s_run;
  const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t log2b = a.log2b, log2gpb = log2b - 3;
  const uint32_t bps = (uint32_t)(kTileElems >> log2b);            // blocks per sub-tile
  const uint64_t n = a.n;
  const uint64_t start = tile * SUB * kTileElems;
  const uint64_t left = n - start;
  const uint64_t span_vals = left < SUB * kTileElems ? left : SUB * kTileElems;
  const uint32_t nsub = (uint32_t)((span_vals + kTileElems - 1) / kTileElems);
  const uint32_t span = (1u << log2gpb) < 64 ? (1u << log2gpb) : 64u;   // lanes of one block
  const __amdgpu_buffer_rsrc_t in_rs =
      range_rsrc(reinterpret_cast<const uint8_t *>(a.in) + F::kBytes * start, F::kBytes * span_vals);
  const uint64_t sm_total = (F::kSmBits * n + 7) / 8;                  // bytes of kept fields
  gu64 *const status = (gu64 *)a.status;
  // FP16, n odd: the last value's dword straddles the input's end, so the
  // range check reads it as 0; the value itself comes from this load
  const uint32_t x_last = DT == 2 ? (uint32_t)*(const ENC_GLOBAL uint16_t *)(a.in + n - 1) : 0u;

  if (tid < 64) {
    smin[tid] = 255;
    smax[tid] = 0;
  }
  if (tid == 0) s_run = 0;
  for (uint32_t i = tid; i < kPayBytes / 16; i += kThreads)
    reinterpret_cast<uint4 *>(pay)[i] = make_uint4(0, 0, 0, 0);
  uint64_t lb_first = kFlagPre;   // wave 0: first look-back window, read early
  uint4 g[kGroupsPerThread][CH], gn[kGroupsPerThread][CH];
  uint32_t valid[kGroupsPerThread], vn[kGroupsPerThread];
  // the groups of sub-tile `sub` (offsets from the tile start; past the
  // tile every dword is out of the descriptor's range: zeros, no access)
  auto load = [&](uint32_t sub, uint4 (&dst)[kGroupsPerThread][CH], uint32_t (&v)[kGroupsPerThread]) {
#pragma unroll
    for (uint32_t it = 0; it < kGroupsPerThread; ++it) {
      const uint32_t e0 = (sub * kTileGroups + it * kThreads + tid) * 8;
#pragma unroll
      for (uint32_t c = 0; c < CH; ++c) {
        const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(in_rs, F::kBytes * e0 + 16 * c, 0, 0);
        dst[it][c] = make_uint4(x.x, x.y, x.z, x.w);
      }
      v[it] = e0 < left ? (left - e0 < 8 ? (uint32_t)(left - e0) : 8u) : 0u;
    }
  };
  load(0, g, valid);
#pragma unroll 1
  for (uint32_t sub = 0; sub < nsub; ++sub) {
    const uint64_t st = tile * SUB + sub;                  // global sub-tile index
    const uint64_t blk0 = st * bps;
    load(sub + 1, gn, vn);                                 // next sub-tile, in flight
    lds_barrier();   // previous sub-tile packed and stored (sblk, smi free), min/max reset
    for (uint32_t i = tid; i < kTileSm / 16; i += kThreads)
      reinterpret_cast<uint4 *>(smi)[i] = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (uint32_t it = 0; it < kGroupsPerThread; ++it)
      if (DT == 2 && (valid[it] & 1)) {   // value v - 1 alone in the low half of dword (v - 1) / 2
        const uint32_t j = (valid[it] - 1) >> 1;
        uint4 &c = g[it][0];
        c.x = j == 0 ? x_last : c.x;
        c.y = j == 1 ? x_last : c.y;
        c.z = j == 2 ? x_last : c.z;
        c.w = j == 3 ? x_last : c.w;
      }

    // per-block min / max exponent over the valid values
#pragma unroll
    for (uint32_t it = 0; it < kGroupsPerThread; ++it) {
      uint32_t mn = 255, mx = 0;
#pragma unroll
      for (uint32_t k = 0; k < 8; ++k) {
        const uint32_t e = (wide_value<DT>(g[it], k) >> F::kShift) & F::kExpMask;
        mn = k < valid[it] && e < mn ? e : mn;
        mx = k < valid[it] && e > mx ? e : mx;
      }
      uint32_t key = valid[it] ? ((255u - mn) << 16) | mx : 0u;   // 0: no valid value here
      key = span_max16(key, span);
      const uint32_t q = it * kThreads + tid;
      if ((lane & (span - 1)) == span - 1 && key != 0) {
        atomicMin(&smin[q >> log2gpb], 255u - (key >> 16));
        atomicMax(&smax[q >> log2gpb], key & 0xFFFFu);
      }
    }
    lds_barrier();

    // block parameters, metas, offsets inside the workgroup's payload
    if (wave == 0) {
      const uint64_t blk = blk0 + lane;
      uint32_t P = 0, base = 0, w = 0;
      if (lane < bps && blk < a.nb) {
        base = smin[lane];
        w = block_width(smax[lane] - base, a.pow2);
        const uint32_t L = (blk + 1 == a.nb) ? (uint32_t)(n - ((a.nb - 1) << log2b)) : (1u << log2b);
        P = (((w * L + 7) >> 3) + 15) & ~15u;
      }
      const __amdgpu_buffer_rsrc_t meta_rs = range_rsrc(
          a.out + a.meta_off + 2 * blk0, align_up(2 * (a.nb - blk0 < bps ? a.nb - blk0 : bps), 4));
      const uint32_t mw = base | (w << 8);
      const uint32_t pair = mw | (__shfl_down(mw, 1, 64) << 16);
      if (!(lane & 1)) __builtin_amdgcn_raw_buffer_store_b32(pair, meta_rs, 2 * lane, 0, 0);
      smin[lane] = 255;
      smax[lane] = 0;
      const uint32_t run = s_run;
      const uint32_t incl = wave_incl_scan(P);
      const uint32_t sub_total = __builtin_amdgcn_readlane(incl, 63);
      sblk[lane] = base | (w << 8) | ((run + incl - P) << 16);
      if (lane == 0) {
        s_suboff[sub] = run;
        s_run = run + sub_total;
      }
      if (sub + 1 == nsub) {
        if (lane == 0) publish(status, tile, (tile == 0 ? kFlagPre : kFlagAgg) | (run + sub_total));
        lb_first = window_word(status, (int64_t)tile - 1, lane);
      }
    }
    lds_barrier();

    // codes into the payload image, kept fields into the sub-tile's image
#pragma unroll
    for (uint32_t it = 0; it < kGroupsPerThread; ++it) {
      const uint32_t q = it * kThreads + tid;
      const uint32_t v = valid[it];
      if (!v) continue;
      const uint32_t info = sblk[q >> log2gpb];
      const uint32_t base = info & 0xFFu, w = (info >> 8) & 0xFFu;
      uint32_t f[8];
      unsigned long long codes = 0;
#pragma unroll
      for (uint32_t k = 0; k < 8; ++k) {
        const uint32_t x = wide_value<DT>(g[it], k);
        const uint32_t e = (x >> F::kShift) & F::kExpMask;
        constexpr uint32_t top = F::kBytes * 8 - 1;
        f[k] = k < v ? ((x >> top) << F::kShift) | (x & ((1u << F::kShift) - 1)) : 0u;
        if (k < v) codes |= (unsigned long long)(e - base) << (k * w);
      }
      const uint32_t pos = (info >> 16) + (q & ((1u << log2gpb) - 1)) * w;
      const uint32_t lo = (uint32_t)codes, hi = (uint32_t)(codes >> 32);
      const uint32_t sh = (pos & 3) * 8, d0 = pos >> 2;
      const uint32_t w0 = lo << sh;
      const uint32_t w1 = sh ? (lo >> (32 - sh)) | (hi << sh) : hi;
      const uint32_t w2 = sh ? hi >> (32 - sh) : 0u;
      if (w0) atomicOr(&pay[d0], w0);
      if (w1) atomicOr(&pay[d0 + 1], w1);
      if (w2) atomicOr(&pay[d0 + 2], w2);
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
        // 88 bits at bit 88 q, OR-ed into the four dwords they can touch
        // (the first and last are shared with the neighbouring groups)
        const unsigned long long fl = (unsigned long long)f[0] | (unsigned long long)f[1] << 11 |
                                      (unsigned long long)f[2] << 22 | (unsigned long long)f[3] << 33 |
                                      (unsigned long long)f[4] << 44 | (unsigned long long)f[5] << 55;
        const uint32_t fh = f[5] >> 9 | f[6] << 2 | f[7] << 13;   // bits 64..87
        const uint32_t v0 = (uint32_t)fl, v1 = (uint32_t)(fl >> 32), v2 = fh;
        const uint32_t bit = 88 * q, e0 = bit >> 5, s5 = bit & 31;   // s5 is 0, 8, 16 or 24
        const uint32_t x0 = v0 << s5;
        const uint32_t x1 = s5 ? (v0 >> (32 - s5)) | (v1 << s5) : v1;
        const uint32_t x2 = s5 ? (v1 >> (32 - s5)) | (v2 << s5) : v2;
        const uint32_t x3 = s5 ? v2 >> (32 - s5) : 0u;
        if (x0) atomicOr(&smi[e0], x0);
        if (x1) atomicOr(&smi[e0 + 1], x1);
        if (x2) atomicOr(&smi[e0 + 2], x2);
        if (x3) atomicOr(&smi[e0 + 3], x3);
      }
    }
    lds_barrier();
    // the sub-tile's kept fields (16-byte aligned: 1024 x 11 and 1024 x 24
    // are multiples of 16); bytes past the section's last field are not
    // written
    const uint64_t sm0 = (uint64_t)kTileSm * st;
    const uint32_t len = (uint32_t)(sm_total - sm0 < kTileSm ? sm_total - sm0 : kTileSm);
    uint8_t *sdst = a.out + kHeaderBytes + sm0;
    for (uint32_t i = tid; i < len / 16; i += kThreads) {
      const uint4 d = reinterpret_cast<const uint4 *>(smi)[i];
      store_nt16(sdst + 16 * i, d);
    }
    if (tid < (len & 15)) {
      const uint32_t b = (len & ~15u) + tid;
      sdst[b] = reinterpret_cast<const uint8_t *>(smi)[b];
    }
#pragma unroll
    for (uint32_t it = 0; it < kGroupsPerThread; ++it) {
#pragma unroll
      for (uint32_t c = 0; c < CH; ++c) g[it][c] = gn[it][c];
      valid[it] = vn[it];
    }
  }
  lds_barrier();

  // the workgroup's payload offset
  if (wave == 0) {
    const uint32_t agg = s_run;
    const uint64_t excl = look_back(status, tile, lane, (gu32 *)a.error, a.spin_limit, a.short_sleep,
                                    lb_first);
    if (lane == 0) {
      if (tile > 0) publish(status, tile, kFlagPre | (excl + agg));
      if (tile + 1 == a.ntiles) *(gu64 *)a.ws_total = excl + agg;
      s_excl = excl;
    }
    if (lane < nsub && (((tile * SUB + lane) * bps) & 63) == 0)   // segment starts
      *(gu64 *)(a.out + a.segoff_off + 8 * (((tile * SUB + lane) * bps) >> 6)) = excl + s_suboff[lane];
  }
  lds_barrier();

  // payload out
  const uint64_t dst = a.payload_off + s_excl;
  const __amdgpu_buffer_rsrc_t pay_rs = range_rsrc(a.out + dst, a.cap > dst ? a.cap - dst : 0);
  for (uint32_t i = tid; i < s_run / 16; i += kThreads) {
    const uint4 d = reinterpret_cast<const uint4 *>(pay)[i];
    __builtin_amdgcn_raw_buffer_store_b128((u32x4){d.x, d.y, d.z, d.w}, pay_rs, 16 * i, 0, kStoreNT);
  }
}

template <uint32_t DT, uint32_t SUB>
__global__ __launch_bounds__(kThreads) void k_encw_onepass(EncodeArgs a) {
  onepass_tile_wide<DT, SUB>(a, blockIdx.x);
}

// Many FP16 or FP32 streams (one dtype per launch) in one launch, as
// k_enc_onepass_batch.
template <uint32_t DT>
__global__ __launch_bounds__(kThreads) void k_encw_onepass_batch(const uint8_t *__restrict__ table) {
  const EncBatchHeader *h = reinterpret_cast<const EncBatchHeader *>(table);
  const uint32_t count = h->count;
  const EncodeArgs *items = reinterpret_cast<const EncodeArgs *>(table + sizeof(EncBatchHeader));
  const uint64_t *begin = reinterpret_cast<const uint64_t *>(table + sizeof(EncBatchHeader) +
                                                             count * sizeof(EncodeArgs));
  const uint64_t b = blockIdx.x;
  uint32_t lo = 0, hi = count;
  while (hi - lo > 1) {
    const uint32_t mid = (lo + hi) / 2;
    if (begin[mid] <= b) lo = mid; else hi = mid;
  }
  const EncodeArgs a = items[lo];
  onepass_tile_wide<DT, kOnePassMaxSub>(a, b - begin[lo]);
}

// Header and the zero padding of the sm, meta and segment-offset sections of
// a stream the single pass wrote (threads tid, tid + stride, ...).
__device__ __forceinline__ void pads_body(const EncodeArgs &a, const HeaderImage &h, uint64_t tid,
                                          uint64_t stride) {
  if (tid < 64) reinterpret_cast<uint32_t *>(a.out)[tid] = reinterpret_cast<const uint32_t *>(h.bytes)[tid];
  // the single pass writes BF16 sign+mantissa bytes in whole groups, the
  // wide types' kept fields up to the section's last byte
  const uint64_t sm_from = kHeaderBytes + (a.dtype == 2   ? (11 * a.n + 7) / 8
                                           : a.dtype == 3 ? 3 * a.n
                                                          : align_up(a.n, 8)),
                 sm_to = a.meta_off;
  const uint64_t meta_from = a.meta_off + 2 * a.nb, meta_to = a.segoff_off;
  const uint64_t seg_from = a.segoff_off + 8 * a.nseg, seg_to = a.payload_off;
  const uint64_t l0 = sm_to - sm_from, l1 = meta_to - meta_from, l2 = seg_to - seg_from;
  for (uint64_t i = tid; i < l0 + l1 + l2; i += stride) {
    const uint64_t at = i < l0 ? sm_from + i : i < l0 + l1 ? meta_from + (i - l0) : seg_from + (i - l0 - l1);
    a.out[at] = 0;
  }
}

__global__ __launch_bounds__(kThreads) void k_enc_pads(EncodeArgs a, HeaderImage h) {
  pads_body(a, h, (uint64_t)blockIdx.x * blockDim.x + threadIdx.x, (uint64_t)gridDim.x * blockDim.x);
}

// One workgroup per stream of a PadsItem table.
__global__ __launch_bounds__(kThreads) void k_enc_pads_batch(const PadsItem *__restrict__ items) {
  pads_body(items[blockIdx.x].a, items[blockIdx.x].h, threadIdx.x, blockDim.x);
}

}  // namespace

hipError_t launch_encode_onepass(const EncodeArgs &a, hipStream_t s) {
  switch (onepass_sub(a.n)) {
    case 1: hipLaunchKernelGGL(k_enc_onepass<1>, dim3((uint32_t)a.ntiles), dim3(kThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL(k_enc_onepass<2>, dim3((uint32_t)a.ntiles), dim3(kThreads), 0, s, a); break;
    default: hipLaunchKernelGGL(k_enc_onepass<4>, dim3((uint32_t)a.ntiles), dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_encode_wide_onepass(const EncodeArgs &a, hipStream_t s) {
  const dim3 grid((uint32_t)a.ntiles), block(kThreads);
  const uint32_t sub = onepass_sub(a.n);
  if (a.dtype == 2) {
    if (sub == 1) hipLaunchKernelGGL((k_encw_onepass<2, 1>), grid, block, 0, s, a);
    else if (sub == 2) hipLaunchKernelGGL((k_encw_onepass<2, 2>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_encw_onepass<2, 4>), grid, block, 0, s, a);
  } else {
    if (sub == 1) hipLaunchKernelGGL((k_encw_onepass<3, 1>), grid, block, 0, s, a);
    else if (sub == 2) hipLaunchKernelGGL((k_encw_onepass<3, 2>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_encw_onepass<3, 4>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_encode_wide_onepass_batch(const void *table, uint64_t total_wgs, uint32_t dtype,
                                            hipStream_t s) {
  if (total_wgs == 0) return hipSuccess;
  const dim3 grid((uint32_t)total_wgs), block(kThreads);
  const uint8_t *t = static_cast<const uint8_t *>(table);
  if (dtype == 2)
    hipLaunchKernelGGL(k_encw_onepass_batch<2>, grid, block, 0, s, t);
  else
    hipLaunchKernelGGL(k_encw_onepass_batch<3>, grid, block, 0, s, t);
  return hipGetLastError();
}

hipError_t launch_encode_pads(const EncodeArgs &a, const HeaderImage &h, hipStream_t s) {
  hipLaunchKernelGGL(k_enc_pads, dim3(4), dim3(kThreads), 0, s, a, h);
  return hipGetLastError();
}

hipError_t launch_encode_onepass_batch(const void *table, uint64_t total_wgs, hipStream_t s) {
  if (total_wgs == 0) return hipSuccess;
  hipLaunchKernelGGL(k_enc_onepass_batch, dim3((uint32_t)total_wgs), dim3(kThreads), 0, s,
                     static_cast<const uint8_t *>(table));
  return hipGetLastError();
}

hipError_t launch_encode_pads_batch(const void *items, uint32_t count, hipStream_t s) {
  if (count == 0) return hipSuccess;
  hipLaunchKernelGGL(k_enc_pads_batch, dim3(count), dim3(kThreads), 0, s,
                     static_cast<const PadsItem *>(items));
  return hipGetLastError();
}

}  // namespace enc
