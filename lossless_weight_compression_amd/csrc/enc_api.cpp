// enc_api.cpp -- host side of the C ABI declared in include/enc.h.
//
// Validates every argument on the host before anything is launched, sizes
// workspaces, builds stream headers and launches the gfx950 kernels. No
// exception crosses the ABI; failures return a negative enc_status and leave
// a message in a thread-local buffer (enc_last_error).
#include "enc.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "enc_common.h"
#include "encode_batch.h"

using namespace enc;

namespace {

thread_local char g_err[512];

enc_status fail(enc_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

enc_status hip_fail(hipError_t e, const char *what) {
  return fail(ENC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

void clear_err() { g_err[0] = 0; }

// ENC_DEBUG_SYNC set to anything but "" or "0": every asynchronous entry
// point synchronises its stream after its launches (unless the stream is
// being captured into a graph), so a fault inside a kernel is reported by
// the call that launched it. Read on every call, so it can be toggled.
bool debug_sync() {
  const char *v = getenv("ENC_DEBUG_SYNC");
  return v && v[0] && strcmp(v, "0") != 0;
}

enc_status launched(hipError_t e, hipStream_t s, const char *what) {
  if (e != hipSuccess) return hip_fail(e, what);
  if (debug_sync()) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(s, &cs);
    if (e != hipSuccess) return hip_fail(e, "capture status query");
    if (cs == hipStreamCaptureStatusNone) {
      e = hipStreamSynchronize(s);
      if (e != hipSuccess)
        return fail(ENC_ERR_HIP, "%s, found by ENC_DEBUG_SYNC: %s", what, hipGetErrorString(e));
    }
  }
  return ENC_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int log2_block(uint32_t B) {
  for (uint32_t l = kMinLog2B; l <= kMaxLog2B; ++l)
    if (B == (1u << l)) return (int)l;
  return -1;
}

constexpr uint64_t kMaxElems = 1ull << 40;

// Header element types: 1 BF16, 2 FP16, 3 FP32. Bytes per value, bits of
// the kept sign+mantissa field, and the largest exponent field value.
bool dtype_known(uint32_t dt) { return dt >= 1 && dt <= 3; }
uint32_t elem_bytes(uint32_t dt) { return dt == 3 ? 4u : 2u; }
uint32_t kept_bits(uint32_t dt) { return dt == 2 ? 11u : dt == 3 ? 24u : 8u; }
uint32_t exp_max(uint32_t dt) { return dt == 2 ? 31u : 255u; }

struct Layout {
  uint64_t n, nb, nseg, sm_off, meta_off, segoff_off, payload_off;
};

Layout layout_of(uint64_t n, uint32_t B, uint32_t dtype = 1) {
  Layout L;
  L.n = n;
  L.nb = (n + B - 1) / B;
  L.nseg = (L.nb + kSegBlocks - 1) / kSegBlocks;
  L.sm_off = kHeaderBytes;
  L.meta_off = L.sm_off + align_up((kept_bits(dtype) * n + 7) / 8, kSectionAlign);
  L.segoff_off = L.meta_off + align_up(2 * L.nb, kSectionAlign);
  L.payload_off = L.segoff_off + align_up(8 * L.nseg, kSectionAlign);
  return L;
}

void put_le(uint8_t *p, uint64_t v, int nbytes) {
  for (int i = 0; i < nbytes; ++i) p[i] = (uint8_t)(v >> (8 * i));
}

uint64_t get_le(const uint8_t *p, int nbytes) {
  uint64_t v = 0;
  for (int i = 0; i < nbytes; ++i) v |= (uint64_t)p[i] << (8 * i);
  return v;
}

HeaderImage header_of(const enc_info &i) {
  HeaderImage h;
  memset(h.bytes, 0, sizeof h.bytes);
  memcpy(h.bytes, "ENCB", 4);
  put_le(h.bytes + 4, i.version, 2);
  put_le(h.bytes + 6, i.dtype, 2);
  put_le(h.bytes + 8, i.flags, 4);
  put_le(h.bytes + 12, i.block_size, 4);
  put_le(h.bytes + 16, kSegBlocks, 4);
  const uint64_t f[] = {i.n_elems,    i.n_blocks,    i.n_segments,    i.sm_off,
                        i.meta_off,   i.segoff_off,  i.payload_off,   i.payload_bytes,
                        i.raw_off,    i.total_bytes};
  for (int k = 0; k < 10; ++k) put_le(h.bytes + 24 + 8 * k, f[k], 8);
  return h;
}

enc_info raw_info(uint64_t n, uint32_t B, uint32_t dtype = 1) {
  enc_info i;
  memset(&i, 0, sizeof i);
  i.version = 1;
  i.dtype = dtype;
  i.flags = 1;
  i.block_size = B;
  i.n_elems = n;
  i.raw_off = kHeaderBytes;
  i.total_bytes = kHeaderBytes + elem_bytes(dtype) * n;
  return i;
}

// Consistency of a parsed header with the format (no device data read).
enc_status check_info(const enc_info *i) {
  if (!i) return fail(ENC_ERR_INVALID_ARG, "info is NULL");
  if (i->version != 1 || !dtype_known(i->dtype))
    return fail(ENC_ERR_BAD_STREAM, "version %u / dtype %u not supported", i->version, i->dtype);
  if (i->n_elems > kMaxElems) return fail(ENC_ERR_UNSUPPORTED, "n_elems above 2^40");
  if (i->flags == 1) {
    if (i->n_blocks || i->n_segments || i->sm_off || i->meta_off || i->segoff_off ||
        i->payload_off || i->payload_bytes || i->raw_off != kHeaderBytes ||
        i->total_bytes != kHeaderBytes + elem_bytes(i->dtype) * i->n_elems)
      return fail(ENC_ERR_BAD_STREAM, "inconsistent RAW header");
    return ENC_OK;
  }
  if (i->flags != 0 && i->flags != 2) return fail(ENC_ERR_BAD_STREAM, "unknown flags 0x%x", i->flags);
  if (log2_block(i->block_size) < 0)
    return fail(ENC_ERR_UNSUPPORTED, "block size %u (library supports 128..4096, powers of two)",
                i->block_size);
  if (i->n_elems == 0) return fail(ENC_ERR_BAD_STREAM, "coded stream with zero elements");
  const Layout L = layout_of(i->n_elems, i->block_size, i->dtype);
  if (i->n_blocks != L.nb || i->n_segments != L.nseg || i->sm_off != L.sm_off ||
      i->meta_off != L.meta_off || i->segoff_off != L.segoff_off ||
      i->payload_off != L.payload_off || i->raw_off != 0 ||
      i->total_bytes != i->payload_off + i->payload_bytes ||
      i->payload_bytes > L.nb * (uint64_t)i->block_size + 16 * L.nb || (i->total_bytes & 15))
    return fail(ENC_ERR_BAD_STREAM, "section offsets do not match n=%llu, B=%u",
                (unsigned long long)i->n_elems, i->block_size);
  return ENC_OK;
}

DecodeDesc desc_of(const void *d_comp, const enc_info &i, void *d_out) {
  DecodeDesc d;
  memset(&d, 0, sizeof d);
  d.stream = static_cast<const uint8_t *>(d_comp);
  d.out = d_out;
  d.n = i.n_elems;
  d.total = i.total_bytes;
  d.dtype = i.dtype;
  if (i.flags == 1) {
    d.raw = 1;
    d.log2b = kMinLog2B;
  } else {
    d.nb = i.n_blocks;
    d.meta_off = i.meta_off;
    d.segoff_off = i.segoff_off;
    d.payload_off = i.payload_off;
    d.log2b = (uint32_t)log2_block(i.block_size);
  }
  return d;
}

enc_info coded_info(uint64_t n, uint32_t block_size, const Layout &L, uint64_t payload,
                    uint32_t pow2, uint32_t dtype = 1) {
  enc_info i;
  memset(&i, 0, sizeof i);
  i.version = 1;
  i.dtype = dtype;
  i.flags = pow2 ? 2 : 0;
  i.block_size = block_size;
  i.n_elems = n;
  i.n_blocks = L.nb;
  i.n_segments = L.nseg;
  i.sm_off = L.sm_off;
  i.meta_off = L.meta_off;
  i.segoff_off = L.segoff_off;
  i.payload_off = L.payload_off;
  i.payload_bytes = payload;
  i.raw_off = 0;
  i.total_bytes = L.payload_off + payload;
  return i;
}

// Polls of an unpublished tile before the single pass gives up (about 0.1 s
// at one poll per ~3.4 us of sleep; never reached when workgroups are
// dispatched in order). ENC_LOOKBACK_SPINS overrides it; 0 makes every
// tile after the first give up at once, so tests take the fallback path
// deterministically.
#ifndef ENC_SHORT_SLEEP_TILES
#define ENC_SHORT_SLEEP_TILES 4096
#endif
constexpr uint64_t kShortSleepTiles = ENC_SHORT_SLEEP_TILES;

uint32_t lookback_spin_limit() {
  const char *v = getenv("ENC_LOOKBACK_SPINS");
  if (v && v[0]) return (uint32_t)strtoul(v, nullptr, 10);
  return 1u << 15;
}

// Single pass (reads the input once): used when the output can hold the
// RAW size and the fixed sections fit below it, so no store of the pass can
// land outside the buffer and the RAW fallback can simply overwrite it.
// Returns ENC_ERR_HIP with *gave_up set if a look-back wait gave up; the
// caller then runs the two-pass encoder, which rewrites every byte.
enc_status compress_one_pass(const void *d_in, uint64_t n, uint32_t dtype, uint32_t block_size,
                             uint32_t pow2, const Layout &L, uint8_t *d_out, uint64_t cap,
                             uint8_t *d_ws, hipStream_t s, enc_info *h_info, bool *gave_up) {
  *gave_up = false;
  EncodeArgs a;
  memset(&a, 0, sizeof a);
  a.pow2 = pow2;
  a.dtype = dtype;
  a.in = static_cast<const uint16_t *>(d_in);
  a.out = d_out;
  a.n = n;
  a.nb = L.nb;
  a.nseg = L.nseg;
  a.meta_off = L.meta_off;
  a.segoff_off = L.segoff_off;
  a.payload_off = L.payload_off;
  a.log2b = (uint32_t)log2_block(block_size);
  a.ntiles = onepass_tiles(n);
  a.cap = cap;
  const uint64_t status_bytes = align_up(8 * a.ntiles, kSectionAlign);
  a.status = reinterpret_cast<uint64_t *>(d_ws);
  a.ws_total = reinterpret_cast<uint64_t *>(d_ws + status_bytes);
  a.error = reinterpret_cast<uint32_t *>(d_ws + status_bytes + 12);
  a.spin_limit = lookback_spin_limit();
  // one tensor of at most kShortSleepTiles workgroups: poll after a short
  // sleep (the spin limit scaled so a wait still gives up after ~0.1 s)
  a.short_sleep = a.ntiles <= kShortSleepTiles;
  if (a.short_sleep && a.spin_limit < (1u << 27)) a.spin_limit *= 16;
  hipError_t e = hipMemsetAsync(d_ws, 0, status_bytes + 16, s);
  if (e != hipSuccess) return hip_fail(e, "look-back state initialisation");
  e = dtype == 1 ? launch_encode_onepass(a, s) : launch_encode_wide_onepass(a, s);
  if (e != hipSuccess) return hip_fail(e, "single-pass kernel launch");
  uint64_t back[2] = {0, 0};   // payload bytes; (unused) | error << 32
  e = hipMemcpyAsync(back, a.ws_total, sizeof back, hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return hip_fail(e, "size read-back");
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "stream synchronize");
  if (back[1] >> 32) {
    *gave_up = true;
    return fail(ENC_ERR_HIP, "single-pass encoder: a look-back wait gave up");
  }
  const uint64_t payload = back[0];
  const uint64_t raw_total = kHeaderBytes + elem_bytes(dtype) * n;
  enc_info i;
  enc_status st;
  if (L.payload_off + payload >= raw_total) {
    i = raw_info(n, block_size, dtype);
    // the verbatim copy moves 16-bit units
    st = launched(launch_encode_raw(a.in, d_out, n * (elem_bytes(dtype) / 2), header_of(i), s), s,
                  "raw copy launch");
  } else {
    i = coded_info(n, block_size, L, payload, a.pow2, dtype);
    st = launched(launch_encode_pads(a, header_of(i), s), s, "header kernel launch");
  }
  if (st != ENC_OK) return st;
  *h_info = i;
  return ENC_OK;
}

// FP16 / FP32 input: block parameters, the segment scan, then the pack
// (reads the input twice); RAW when the coded stream would not be smaller.
enc_status compress_wide(const void *d_in, uint64_t n, uint32_t dtype, uint32_t block_size,
                         uint32_t pow2, uint8_t *d_out, uint64_t cap, uint8_t *d_ws,
                         hipStream_t s, enc_info *h_info) {
  const Layout L = layout_of(n, block_size, dtype);
  EncodeArgs a;
  memset(&a, 0, sizeof a);
  a.in = static_cast<const uint16_t *>(d_in);
  a.out = d_out;
  a.ws_meta = d_ws;
  a.ws_segsum = reinterpret_cast<uint64_t *>(a.ws_meta + align_up(2 * L.nb, kSectionAlign));
  a.ws_total = reinterpret_cast<uint64_t *>(reinterpret_cast<uint8_t *>(a.ws_segsum) +
                                            align_up(8 * L.nseg, kSectionAlign));
  a.n = n;
  a.nb = L.nb;
  a.nseg = L.nseg;
  a.meta_off = L.meta_off;
  a.segoff_off = L.segoff_off;
  a.payload_off = L.payload_off;
  a.log2b = (uint32_t)log2_block(block_size);
  a.pow2 = pow2;
  hipError_t e = launch_encode_wide_params(a, dtype, s);
  if (e != hipSuccess) return hip_fail(e, "width kernel launch");
  e = launch_encode_scan(a, s);
  if (e != hipSuccess) return hip_fail(e, "scan kernel launch");
  uint64_t payload = 0;
  e = hipMemcpyAsync(&payload, a.ws_total, sizeof payload, hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return hip_fail(e, "size read-back");
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "stream synchronize");
  const uint64_t raw_total = kHeaderBytes + elem_bytes(dtype) * n;
  const uint64_t coded_total = L.payload_off + payload;
  enc_info i;
  if (coded_total >= raw_total) {
    if (cap < raw_total)
      return fail(ENC_ERR_CAPACITY, "output capacity %llu below stream size %llu",
                  (unsigned long long)cap, (unsigned long long)raw_total);
    i = raw_info(n, block_size, dtype);
    // the verbatim copy moves 16-bit units
    const enc_status st = launched(launch_encode_raw(a.in, d_out, n * (elem_bytes(dtype) / 2),
                                                     header_of(i), s),
                                   s, "raw copy launch");
    if (st != ENC_OK) return st;
  } else {
    if (cap < coded_total)
      return fail(ENC_ERR_CAPACITY, "output capacity %llu below stream size %llu",
                  (unsigned long long)cap, (unsigned long long)coded_total);
    i = coded_info(n, block_size, L, payload, pow2, dtype);
    e = launch_encode_wide_pack(a, dtype, s);
    if (e != hipSuccess) return hip_fail(e, "pack kernel launch");
    const enc_status st = launched(launch_encode_wide_finish(a, dtype, header_of(i), s), s,
                                   "finish kernel launch");
    if (st != ENC_OK) return st;
  }
  *h_info = i;
  return ENC_OK;
}

// Workspace of enc_compress_batch, in order: the single-pass table, the
// header/pads table, one 16-byte result slot per item (payload bytes, then
// the error word in the upper half of the second u64), the per-item status
// words (64-byte aligned runs). The status words and result slots are one
// contiguous range, cleared by one memset.
struct BatchEncLayout {
  uint64_t table, pads, results, status, status_bytes, total;
};

BatchEncLayout batch_enc_layout(const enc_citem *items, int count) {
  BatchEncLayout b;
  b.table = 0;
  b.pads = align_up(sizeof(EncBatchHeader) + (uint64_t)count * sizeof(EncodeArgs) +
                        8 * ((uint64_t)count + 1),
                    kSectionAlign);
  b.results = b.pads + align_up((uint64_t)count * sizeof(PadsItem), kSectionAlign);
  b.status = b.results + align_up(16 * (uint64_t)count, kSectionAlign);
  b.status_bytes = 0;
  for (int k = 0; k < count; ++k)
    if (items[k].n_elems > 0) b.status_bytes += align_up(8 * onepass_batch_tiles(items[k].n_elems), 64);
  b.total = b.status + align_up(b.status_bytes, kSectionAlign);
  return b;
}

// Device layout of a batch table for these items (see BatchHeader).
struct BatchLayout {
  uint64_t tiles, wide_tiles, map_off, wide_map_off, total;
};

BatchLayout batch_layout(const enc_item *items, int count) {
  BatchLayout b;
  b.tiles = b.wide_tiles = 0;
  for (int k = 0; k < count; ++k)
    (items[k].info.dtype == 1 ? b.tiles : b.wide_tiles) +=
        decode_tiles_for(items[k].info.n_elems, items[k].info.dtype);
  b.map_off = align_up(sizeof(BatchHeader) + (uint64_t)count * sizeof(DecodeDesc) +
                           2 * 8 * ((uint64_t)count + 1),
                       256);
  b.wide_map_off = b.map_off + align_up(4 * b.tiles, 256);
  b.total = b.wide_map_off + align_up(4 * b.wide_tiles, 256);
  return b;
}

}  // namespace

enc_status enc::set_error(enc_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

extern "C" {

uint64_t enc_compress_bound(uint64_t n_elems) { return kHeaderBytes + 2 * n_elems; }

uint64_t enc_compress_bound_dt(uint64_t n_elems, uint32_t dtype) {
  return dtype_known(dtype) ? kHeaderBytes + elem_bytes(dtype) * n_elems : 0;
}

uint64_t enc_compress_workspace_bytes(uint64_t n_elems, uint32_t block_size) {
  if (log2_block(block_size) < 0) return 0;
  const Layout L = layout_of(n_elems, block_size);
  const uint64_t two_pass =
      align_up(2 * L.nb, kSectionAlign) + align_up(8 * L.nseg, kSectionAlign) + kSectionAlign;
  const uint64_t one_pass = align_up(8 * onepass_tiles(n_elems), kSectionAlign) + kSectionAlign;
  return two_pass > one_pass ? two_pass : one_pass;
}

enc_status enc_compress(const uint16_t *d_in, uint64_t n, uint32_t block_size, void *d_out,
                        uint64_t out_capacity, void *d_ws, uint64_t ws_bytes, void *stream,
                        enc_info *h_info) {
  return enc_compress_ex(d_in, n, block_size, 0, d_out, out_capacity, d_ws, ws_bytes, stream, h_info);
}

enc_status enc_compress_ex(const uint16_t *d_in, uint64_t n, uint32_t block_size, uint32_t options,
                           void *d_out, uint64_t out_capacity, void *d_ws, uint64_t ws_bytes,
                           void *stream, enc_info *h_info) {
  clear_err();
  if (options & ~(uint32_t)ENC_OPT_POW2_WIDTHS)
    return fail(ENC_ERR_INVALID_ARG, "unknown options 0x%x", options);
  const uint32_t pow2 = (options & ENC_OPT_POW2_WIDTHS) ? 1u : 0u;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!h_info) return fail(ENC_ERR_INVALID_ARG, "h_info is NULL");
  if (!d_out) return fail(ENC_ERR_INVALID_ARG, "d_out is NULL");
  if (n > 0 && !d_in) return fail(ENC_ERR_INVALID_ARG, "d_in is NULL");
  const int lb = log2_block(block_size);
  if (lb < 0)
    return fail(ENC_ERR_UNSUPPORTED, "block size %u (supported: 128..4096, powers of two)",
                block_size);
  if (n > kMaxElems) return fail(ENC_ERR_UNSUPPORTED, "n above 2^40");
  if (!aligned16(d_in) || !aligned16(d_out) || !aligned16(d_ws))
    return fail(ENC_ERR_INVALID_ARG, "device buffers must be 16-byte aligned");
  const uint64_t raw_total = kHeaderBytes + 2 * n;
  if (n == 0) {
    if (out_capacity < raw_total) return fail(ENC_ERR_CAPACITY, "output capacity below 256");
    const enc_info i = raw_info(0, block_size);
    const enc_status st = launched(launch_encode_raw(d_in, static_cast<uint8_t *>(d_out), 0,
                                                     header_of(i), s),
                                   s, "raw header launch");
    if (st != ENC_OK) return st;
    *h_info = i;
    return ENC_OK;
  }
  const uint64_t need_ws = enc_compress_workspace_bytes(n, block_size);
  if (!d_ws || ws_bytes < need_ws)
    return fail(ENC_ERR_CAPACITY, "workspace of %llu bytes needed", (unsigned long long)need_ws);

  const Layout L = layout_of(n, block_size);
  if (out_capacity >= raw_total && L.payload_off <= raw_total) {
    bool gave_up = false;
    const enc_status st = compress_one_pass(d_in, n, 1, block_size, pow2, L,
                                            static_cast<uint8_t *>(d_out), out_capacity,
                                            static_cast<uint8_t *>(d_ws), s, h_info, &gave_up);
    if (!gave_up) return st;
    clear_err();   // fall through to the two-pass encoder
  }
  EncodeArgs a;
  memset(&a, 0, sizeof a);
  a.in = d_in;
  a.out = static_cast<uint8_t *>(d_out);
  a.ws_meta = static_cast<uint8_t *>(d_ws);
  a.ws_segsum = reinterpret_cast<uint64_t *>(a.ws_meta + align_up(2 * L.nb, kSectionAlign));
  a.ws_total = reinterpret_cast<uint64_t *>(reinterpret_cast<uint8_t *>(a.ws_segsum) +
                                            align_up(8 * L.nseg, kSectionAlign));
  a.n = n;
  a.nb = L.nb;
  a.nseg = L.nseg;
  a.meta_off = L.meta_off;
  a.segoff_off = L.segoff_off;
  a.payload_off = L.payload_off;
  a.log2b = (uint32_t)lb;
  a.pow2 = pow2;

  hipError_t e = launch_encode_params(a, s);
  if (e != hipSuccess) return hip_fail(e, "width kernel launch");
  e = launch_encode_scan(a, s);
  if (e != hipSuccess) return hip_fail(e, "scan kernel launch");
  uint64_t payload = 0;
  e = hipMemcpyAsync(&payload, a.ws_total, sizeof payload, hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return hip_fail(e, "size read-back");
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "stream synchronize");

  const uint64_t coded_total = L.payload_off + payload;
  enc_info i;
  if (coded_total >= raw_total) {
    if (out_capacity < raw_total)
      return fail(ENC_ERR_CAPACITY, "output capacity %llu below stream size %llu",
                  (unsigned long long)out_capacity, (unsigned long long)raw_total);
    i = raw_info(n, block_size);
    const enc_status st = launched(launch_encode_raw(d_in, a.out, n, header_of(i), s), s,
                                   "raw copy launch");
    if (st != ENC_OK) return st;
  } else {
    if (out_capacity < coded_total)
      return fail(ENC_ERR_CAPACITY, "output capacity %llu below stream size %llu",
                  (unsigned long long)out_capacity, (unsigned long long)coded_total);
    i = coded_info(n, block_size, L, payload, a.pow2);
    e = launch_encode_pack(a, s);
    if (e != hipSuccess) return hip_fail(e, "pack kernel launch");
    const enc_status st = launched(launch_encode_finish(a, header_of(i), s), s,
                                   "finish kernel launch");
    if (st != ENC_OK) return st;
  }
  *h_info = i;
  return ENC_OK;
}

enc_status enc_compress_dt(const void *d_in, uint64_t n, uint32_t dtype, uint32_t block_size,
                           uint32_t options, void *d_out, uint64_t out_capacity, void *d_ws,
                           uint64_t ws_bytes, void *stream, enc_info *h_info) {
  clear_err();
  if (!dtype_known(dtype)) return fail(ENC_ERR_UNSUPPORTED, "dtype %u (1 BF16, 2 FP16, 3 FP32)", dtype);
  if (dtype == 1)
    return enc_compress_ex(static_cast<const uint16_t *>(d_in), n, block_size, options, d_out,
                           out_capacity, d_ws, ws_bytes, stream, h_info);
  if (options & ~(uint32_t)ENC_OPT_POW2_WIDTHS)
    return fail(ENC_ERR_INVALID_ARG, "unknown options 0x%x", options);
  const uint32_t pow2 = (options & ENC_OPT_POW2_WIDTHS) ? 1u : 0u;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!h_info) return fail(ENC_ERR_INVALID_ARG, "h_info is NULL");
  if (!d_out) return fail(ENC_ERR_INVALID_ARG, "d_out is NULL");
  if (n > 0 && !d_in) return fail(ENC_ERR_INVALID_ARG, "d_in is NULL");
  if (log2_block(block_size) < 0)
    return fail(ENC_ERR_UNSUPPORTED, "block size %u (supported: 128..4096, powers of two)",
                block_size);
  if (n > kMaxElems) return fail(ENC_ERR_UNSUPPORTED, "n above 2^40");
  if (!aligned16(d_in) || !aligned16(d_out) || !aligned16(d_ws))
    return fail(ENC_ERR_INVALID_ARG, "device buffers must be 16-byte aligned");
  if (n == 0) {
    if (out_capacity < kHeaderBytes) return fail(ENC_ERR_CAPACITY, "output capacity below 256");
    const enc_info i = raw_info(0, block_size, dtype);
    const enc_status st = launched(launch_encode_raw(static_cast<const uint16_t *>(d_in),
                                                     static_cast<uint8_t *>(d_out), 0, header_of(i), s),
                                   s, "raw header launch");
    if (st != ENC_OK) return st;
    *h_info = i;
    return ENC_OK;
  }
  const uint64_t need_ws = enc_compress_workspace_bytes(n, block_size);
  if (!d_ws || ws_bytes < need_ws)
    return fail(ENC_ERR_CAPACITY, "workspace of %llu bytes needed", (unsigned long long)need_ws);
  // single pass when the output can hold the RAW size (as for BF16); the
  // two-pass encoder when it cannot, or when a look-back wait gave up
  const Layout L = layout_of(n, block_size, dtype);
  const uint64_t raw_total = kHeaderBytes + elem_bytes(dtype) * n;
  if (out_capacity >= raw_total && L.payload_off <= raw_total) {
    bool gave_up = false;
    const enc_status st = compress_one_pass(d_in, n, dtype, block_size, pow2, L,
                                            static_cast<uint8_t *>(d_out), out_capacity,
                                            static_cast<uint8_t *>(d_ws), s, h_info, &gave_up);
    if (!gave_up) return st;
    clear_err();
  }
  return compress_wide(d_in, n, dtype, block_size, pow2, static_cast<uint8_t *>(d_out),
                       out_capacity, static_cast<uint8_t *>(d_ws), s, h_info);
}

uint64_t enc_compress_batch_workspace_bytes(const enc_citem *h_items, int count,
                                            uint32_t block_size) {
  if (log2_block(block_size) < 0 || count < 0 || (count > 0 && !h_items)) return 0;
  uint64_t need = batch_enc_layout(h_items, count).total;
  for (int k = 0; k < count; ++k) {
    const uint64_t one = enc_compress_workspace_bytes(h_items[k].n_elems, block_size);
    if (one > need) need = one;
  }
  return need;
}

enc_status enc_compress_batch_dt(const enc_citem *h_items, int count, uint32_t dtype,
                                 uint32_t block_size, uint32_t options, void *d_ws, uint64_t ws_bytes,
                                 void *stream, enc_info *h_infos) {
  clear_err();
  if (!dtype_known(dtype)) return fail(ENC_ERR_UNSUPPORTED, "dtype %u (1 BF16, 2 FP16, 3 FP32)", dtype);
  const uint64_t eb = elem_bytes(dtype);
  if (options & ~(uint32_t)ENC_OPT_POW2_WIDTHS)
    return fail(ENC_ERR_INVALID_ARG, "unknown options 0x%x", options);
  const uint32_t pow2 = (options & ENC_OPT_POW2_WIDTHS) ? 1u : 0u;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (count < 0) return fail(ENC_ERR_INVALID_ARG, "count %d", count);
  if (count == 0) return ENC_OK;
  if (!h_items || !h_infos) return fail(ENC_ERR_INVALID_ARG, "h_items or h_infos is NULL");
  const int lb = log2_block(block_size);
  if (lb < 0)
    return fail(ENC_ERR_UNSUPPORTED, "block size %u (supported: 128..4096, powers of two)",
                block_size);
  uint64_t total_wgs = 0;
  for (int k = 0; k < count; ++k) {
    const enc_citem &it = h_items[k];
    if (!it.d_out) return fail(ENC_ERR_INVALID_ARG, "item %d: d_out is NULL", k);
    if (it.n_elems > 0 && !it.d_in) return fail(ENC_ERR_INVALID_ARG, "item %d: d_in is NULL", k);
    if (it.n_elems > kMaxElems) return fail(ENC_ERR_UNSUPPORTED, "item %d: n above 2^40", k);
    if (!aligned16(it.d_in) || !aligned16(it.d_out))
      return fail(ENC_ERR_INVALID_ARG, "item %d: device buffers must be 16-byte aligned", k);
    if (it.out_capacity < kHeaderBytes + eb * it.n_elems)
      return fail(ENC_ERR_CAPACITY, "item %d: output capacity %llu below the RAW size %llu", k,
                  (unsigned long long)it.out_capacity,
                  (unsigned long long)(kHeaderBytes + eb * it.n_elems));
    total_wgs += onepass_batch_tiles(it.n_elems);
  }
  // one launch: the grid's work-item count (256 per workgroup) is a u32
  if (total_wgs >= (1ull << 24)) return fail(ENC_ERR_UNSUPPORTED, "batch above 2^24 tiles");
  if (!aligned16(d_ws)) return fail(ENC_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  const uint64_t need_ws = enc_compress_batch_workspace_bytes(h_items, count, block_size);
  if (!d_ws || ws_bytes < need_ws)
    return fail(ENC_ERR_CAPACITY, "workspace of %llu bytes needed", (unsigned long long)need_ws);

  // Items the single pass takes; the others (empty, or fixed sections past
  // the RAW size, which always ends RAW) get their RAW stream directly.
  uint8_t *ws = static_cast<uint8_t *>(d_ws);
  const BatchEncLayout W = batch_enc_layout(h_items, count);
  std::vector<uint8_t> table(W.pads, 0);
  EncBatchHeader *th = reinterpret_cast<EncBatchHeader *>(table.data());
  EncodeArgs *targs = reinterpret_cast<EncodeArgs *>(table.data() + sizeof(EncBatchHeader));
  std::vector<int> coded_items, raw_items;
  const uint32_t spins = lookback_spin_limit();
  uint64_t status_at = W.status, wgs = 0;
  std::vector<uint64_t> begin;
  for (int k = 0; k < count; ++k) {
    const enc_citem &it = h_items[k];
    const uint64_t n = it.n_elems;
    if (n == 0) {
      raw_items.push_back(k);
      continue;
    }
    const Layout L = layout_of(n, block_size, dtype);
    if (L.payload_off > kHeaderBytes + eb * n) {
      raw_items.push_back(k);
      continue;
    }
    EncodeArgs &a = targs[coded_items.size()];
    memset(&a, 0, sizeof a);
    a.pow2 = pow2;
    a.dtype = dtype;
    a.in = it.d_in;
    a.out = static_cast<uint8_t *>(it.d_out);
    a.n = n;
    a.nb = L.nb;
    a.nseg = L.nseg;
    a.meta_off = L.meta_off;
    a.segoff_off = L.segoff_off;
    a.payload_off = L.payload_off;
    a.log2b = (uint32_t)lb;
    a.ntiles = onepass_batch_tiles(n);
    a.cap = it.out_capacity;
    a.status = reinterpret_cast<uint64_t *>(ws + status_at);
    a.ws_total = reinterpret_cast<uint64_t *>(ws + W.results + 16 * coded_items.size());
    a.error = reinterpret_cast<uint32_t *>(ws + W.results + 16 * coded_items.size() + 12);
    a.spin_limit = spins;
    status_at += align_up(8 * a.ntiles, 64);
    begin.push_back(wgs);
    wgs += a.ntiles;
    coded_items.push_back(k);
  }
  const uint32_t nc = (uint32_t)coded_items.size();
  begin.push_back(wgs);
  th->total_wgs = wgs;
  th->count = nc;
  th->magic = kEncBatchMagic;
  // the prefix list follows the nc argument records actually used
  memcpy(table.data() + sizeof(EncBatchHeader) + nc * sizeof(EncodeArgs), begin.data(),
         8 * begin.size());

  hipError_t e;
  std::vector<uint64_t> back(2 * (size_t)nc, 0);
  if (nc > 0) {
    e = hipMemsetAsync(ws + W.results, 0, W.total - W.results, s);
    if (e != hipSuccess) return hip_fail(e, "look-back state initialisation");
    e = hipMemcpyAsync(ws + W.table, table.data(), table.size(), hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_fail(e, "batch table upload");
    e = dtype == 1 ? launch_encode_onepass_batch(ws + W.table, wgs, s)
                   : launch_encode_wide_onepass_batch(ws + W.table, wgs, dtype, s);
    if (e != hipSuccess) return hip_fail(e, "batched single-pass kernel launch");
    e = hipMemcpyAsync(back.data(), ws + W.results, 16 * (uint64_t)nc, hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return hip_fail(e, "size read-back");
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "stream synchronize");
  }

  // Headers and pads of the coded results, one launch; RAW copies and the
  // items whose look-back gave up (two-pass encoder) one by one.
  std::vector<PadsItem> pads;
  std::vector<int> retry;
  for (uint32_t c = 0; c < nc; ++c) {
    const int k = coded_items[c];
    const uint64_t n = h_items[k].n_elems;
    if (back[2 * c + 1] >> 32) {
      retry.push_back(k);
      continue;
    }
    const uint64_t payload = back[2 * c];
    const Layout L = layout_of(n, block_size, dtype);
    if (L.payload_off + payload >= kHeaderBytes + eb * n) {
      raw_items.push_back(k);
      continue;
    }
    h_infos[k] = coded_info(n, block_size, L, payload, pow2, dtype);
    PadsItem p;
    p.a = targs[c];
    p.h = header_of(h_infos[k]);
    pads.push_back(p);
  }
  if (!pads.empty()) {
    e = hipMemcpyAsync(ws + W.pads, pads.data(), pads.size() * sizeof(PadsItem),
                       hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_fail(e, "pads table upload");
    const enc_status st = launched(launch_encode_pads_batch(ws + W.pads, (uint32_t)pads.size(), s),
                                   s, "header kernel launch");
    if (st != ENC_OK) return st;
  }
  for (const int k : raw_items) {
    const enc_citem &it = h_items[k];
    const enc_info i = raw_info(it.n_elems, block_size, dtype);
    // the verbatim copy moves 16-bit units
    const enc_status st = launched(launch_encode_raw(it.d_in, static_cast<uint8_t *>(it.d_out),
                                                     it.n_elems * (eb / 2), header_of(i), s),
                                   s, "raw copy launch");
    if (st != ENC_OK) return st;
    h_infos[k] = i;
  }
  // The host tables above must outlive their uploads.
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "stream synchronize");
  for (const int k : retry) {
    const enc_citem &it = h_items[k];
    const enc_status st = enc_compress_dt(it.d_in, it.n_elems, dtype, block_size, options, it.d_out,
                                          it.out_capacity, d_ws, ws_bytes, stream, &h_infos[k]);
    if (st != ENC_OK) return st;
  }
  return ENC_OK;
}

enc_status enc_compress_batch(const enc_citem *h_items, int count, uint32_t block_size,
                              uint32_t options, void *d_ws, uint64_t ws_bytes, void *stream,
                              enc_info *h_infos) {
  return enc_compress_batch_dt(h_items, count, 1, block_size, options, d_ws, ws_bytes, stream,
                               h_infos);
}

enc_status enc_parse_header(const void *h_header, uint64_t header_bytes, uint64_t comp_bytes,
                            enc_info *h_info) {
  clear_err();
  if (!h_header || !h_info) return fail(ENC_ERR_INVALID_ARG, "NULL argument");
  if (header_bytes < kHeaderBytes) return fail(ENC_ERR_INVALID_ARG, "header needs 256 bytes");
  const uint8_t *h = static_cast<const uint8_t *>(h_header);
  if (memcmp(h, "ENCB", 4) != 0) return fail(ENC_ERR_BAD_STREAM, "bad magic");
  if (get_le(h + 16, 4) != kSegBlocks || get_le(h + 20, 4) != 0)
    return fail(ENC_ERR_BAD_STREAM, "segment size field is not 64");
  for (uint32_t k = 104; k < kHeaderBytes; ++k)
    if (h[k]) return fail(ENC_ERR_BAD_STREAM, "reserved header byte %u is not zero", k);
  enc_info i;
  i.version = (uint32_t)get_le(h + 4, 2);
  i.dtype = (uint32_t)get_le(h + 6, 2);
  i.flags = (uint32_t)get_le(h + 8, 4);
  i.block_size = (uint32_t)get_le(h + 12, 4);
  uint64_t *f[] = {&i.n_elems,  &i.n_blocks,    &i.n_segments,    &i.sm_off,  &i.meta_off,
                   &i.segoff_off, &i.payload_off, &i.payload_bytes, &i.raw_off, &i.total_bytes};
  for (int k = 0; k < 10; ++k) *f[k] = get_le(h + 24 + 8 * k, 8);
  if (i.flags == 1 && log2_block(i.block_size) < 0 && (i.block_size < 8 || i.block_size > 4096 ||
                                                       i.block_size % 8))
    return fail(ENC_ERR_BAD_STREAM, "block size %u", i.block_size);
  const enc_status st = check_info(&i);
  if (st != ENC_OK) return st;
  if (i.total_bytes > comp_bytes)
    return fail(ENC_ERR_BAD_STREAM, "stream claims %llu bytes, buffer holds %llu",
                (unsigned long long)i.total_bytes, (unsigned long long)comp_bytes);
  *h_info = i;
  return ENC_OK;
}

enc_status enc_read_info(const void *d_comp, uint64_t comp_bytes, void *stream, enc_info *h_info) {
  clear_err();
  if (!d_comp || !h_info) return fail(ENC_ERR_INVALID_ARG, "NULL argument");
  if (comp_bytes < kHeaderBytes) return fail(ENC_ERR_BAD_STREAM, "stream shorter than its header");
  uint8_t h[kHeaderBytes];
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(h, d_comp, kHeaderBytes, hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return hip_fail(e, "header read-back");
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "stream synchronize");
  return enc_parse_header(h, kHeaderBytes, comp_bytes, h_info);
}

enc_status enc_decompress(const void *d_comp, const enc_info *h_info, void *d_out,
                          uint64_t out_elems, void *stream) {
  clear_err();
  const enc_status st = check_info(h_info);
  if (st != ENC_OK) return st;
  if (!d_comp) return fail(ENC_ERR_INVALID_ARG, "d_comp is NULL");
  if (out_elems != h_info->n_elems)
    return fail(ENC_ERR_SHAPE, "out_elems %llu != stream elements %llu",
                (unsigned long long)out_elems, (unsigned long long)h_info->n_elems);
  if (out_elems > 0 && !d_out) return fail(ENC_ERR_INVALID_ARG, "d_out is NULL");
  if (!aligned16(d_comp) || !aligned16(d_out))
    return fail(ENC_ERR_INVALID_ARG, "device buffers must be 16-byte aligned");
  if (out_elems == 0) return ENC_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return launched(launch_decode(desc_of(d_comp, *h_info, d_out), s), s, "decode launch");
}

uint64_t enc_batch_table_bytes(const enc_item *h_items, int count) {
  if (count < 0 || (count > 0 && !h_items)) return 0;
  return batch_layout(h_items, count).total;
}

enc_status enc_batch_prepare(const enc_item *h_items, int count, void *d_table, uint64_t table_bytes,
                             void *stream, enc_batch_plan *h_plan) {
  clear_err();
  if (count < 0) return fail(ENC_ERR_INVALID_ARG, "negative count");
  if (count > 0 && !h_items) return fail(ENC_ERR_INVALID_ARG, "h_items is NULL");
  if (!h_plan) return fail(ENC_ERR_INVALID_ARG, "h_plan is NULL");
  if (!d_table || !aligned16(d_table)) return fail(ENC_ERR_INVALID_ARG, "d_table NULL or unaligned");
  for (int k = 0; k < count; ++k) {
    const enc_item &it = h_items[k];
    const enc_status st = check_info(&it.info);
    if (st != ENC_OK) {
      char why[sizeof g_err];
      memcpy(why, g_err, sizeof why);
      return fail(st, "item %d: %s", k, why);
    }
    if (!it.d_comp || (it.info.n_elems && !it.d_out))
      return fail(ENC_ERR_INVALID_ARG, "item %d: NULL pointer", k);
    if (!aligned16(it.d_comp) || !aligned16(it.d_out))
      return fail(ENC_ERR_INVALID_ARG, "item %d: unaligned pointer", k);
  }
  const BatchLayout lay = batch_layout(h_items, count);
  const uint64_t need = lay.total;
  if (table_bytes < need)
    return fail(ENC_ERR_CAPACITY, "table needs %llu bytes", (unsigned long long)need);
  std::vector<uint8_t> host(need, 0);
  BatchHeader hdr;
  memset(&hdr, 0, sizeof hdr);
  hdr.count = (uint32_t)count;
  hdr.magic = kBatchMagic;
  DecodeDesc *descs = reinterpret_cast<DecodeDesc *>(host.data() + sizeof(BatchHeader));
  uint64_t *tiles = reinterpret_cast<uint64_t *>(host.data() + sizeof(BatchHeader) +
                                                 (uint64_t)count * sizeof(DecodeDesc));
  uint64_t *wide = tiles + count + 1;   // the FP16 / FP32 items' tile list
  uint32_t *map = reinterpret_cast<uint32_t *>(host.data() + lay.map_off);
  uint32_t *wide_map = reinterpret_cast<uint32_t *>(host.data() + lay.wide_map_off);
  uint64_t t = 0, tw = 0;
  for (int k = 0; k < count; ++k) {
    const enc_item &it = h_items[k];
    descs[k] = desc_of(it.d_comp, it.info, it.d_out);
    tiles[k] = t;
    wide[k] = tw;
    const uint64_t nt = decode_tiles_for(it.info.n_elems, it.info.dtype);
    uint64_t &at = it.info.dtype == 1 ? t : tw;
    uint32_t *m = it.info.dtype == 1 ? map : wide_map;
    for (uint64_t x = 0; x < nt; ++x) m[at + x] = (uint32_t)k;
    at += nt;
  }
  tiles[count] = t;
  wide[count] = tw;
  hdr.total_tiles = t;
  hdr.wide_tiles = tw;
  hdr.map_off = lay.map_off;
  hdr.wide_map_off = lay.wide_map_off;
  memcpy(host.data(), &hdr, sizeof hdr);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(d_table, host.data(), need, hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return hip_fail(e, "table upload");
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "stream synchronize");
  memset(h_plan, 0, sizeof *h_plan);
  h_plan->tiles = t;
  h_plan->wide_tiles = tw;
  h_plan->d_table = d_table;
  h_plan->count = count;
  return ENC_OK;
}

enc_status enc_decompress_batch(const void *d_table, int count, const enc_batch_plan *h_plan,
                                void *stream) {
  clear_err();
  if (count < 0) return fail(ENC_ERR_INVALID_ARG, "negative count");
  if (!d_table || !aligned16(d_table)) return fail(ENC_ERR_INVALID_ARG, "d_table NULL or unaligned");
  if (!h_plan) return fail(ENC_ERR_INVALID_ARG, "h_plan is NULL");
  if (h_plan->d_table != d_table || h_plan->count != count)
    return fail(ENC_ERR_INVALID_ARG, "the plan was made for another table or count");
  if (count == 0) return ENC_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return launched(launch_decode_batch(d_table, h_plan->tiles, h_plan->wide_tiles, s), s,
                  "batch decode launch");
}

uint64_t enc_gemm_workspace_bytes(uint32_t M, uint32_t K, uint32_t N, uint32_t block_size) {
  // 0 for a shape enc_decompress_gemm rejects (the plan divides by the
  // number of 512-column strips)
  if (log2_block(block_size) < 0 || M == 0 || M > 4096 || K == 0 || N == 0 || N % 512 || K % 8)
    return 0;
  return gemm_workspace_bytes(M, K, N);
}

static enc_status gemm_common(const uint16_t *d_x, uint32_t M, uint32_t K, uint32_t N, float *d_y,
                              void *d_ws, uint64_t ws_bytes, GemmArgs *a) {
  if (!d_x || !d_y || !d_ws) return fail(ENC_ERR_INVALID_ARG, "NULL device pointer");
  if (!aligned16(d_x) || !aligned16(d_y) || !aligned16(d_ws))
    return fail(ENC_ERR_INVALID_ARG, "device buffers must be 16-byte aligned");
  if (M == 0 || M > 4096 || K == 0 || N == 0)
    return fail(ENC_ERR_SHAPE, "M=%u K=%u N=%u out of range", M, K, N);
  if (N % 512) return fail(ENC_ERR_UNSUPPORTED, "N=%u must be a multiple of 512", N);
  if (K % 8) return fail(ENC_ERR_UNSUPPORTED, "K=%u must be a multiple of 8", K);
  const uint64_t need = gemm_workspace_bytes(M, K, N);
  if (ws_bytes < need)
    return fail(ENC_ERR_CAPACITY, "GEMM workspace of %llu bytes needed", (unsigned long long)need);
  memset(a, 0, sizeof *a);
  a->x = d_x;
  a->y = d_y;
  a->M = M;
  a->K = K;
  a->N = N;
  gemm_plan(M, K, N, &a->ksplit, &a->krows);
  a->counters = static_cast<uint32_t *>(d_ws);
  a->partial = reinterpret_cast<float *>(static_cast<uint8_t *>(d_ws) + gemm_counter_bytes(N));
  return ENC_OK;
}

enc_status enc_decompress_gemm(const uint16_t *d_x, uint32_t M, uint32_t K, const void *d_wcomp,
                               const enc_info *h_winfo, uint32_t N, float *d_y, void *d_ws,
                               uint64_t ws_bytes, void *stream) {
  clear_err();
  enc_status st = check_info(h_winfo);
  if (st != ENC_OK) return st;
  if (h_winfo->dtype != 1) return fail(ENC_ERR_UNSUPPORTED, "the GEMM takes BF16 weights only");
  if (!d_wcomp || !aligned16(d_wcomp)) return fail(ENC_ERR_INVALID_ARG, "d_wcomp NULL or unaligned");
  if ((uint64_t)K * N != h_winfo->n_elems)
    return fail(ENC_ERR_SHAPE, "K*N=%llu but the stream holds %llu elements",
                (unsigned long long)K * N, (unsigned long long)h_winfo->n_elems);
  if (h_winfo->flags != 1 && N % h_winfo->block_size)
    return fail(ENC_ERR_UNSUPPORTED, "N=%u not a multiple of the block size %u", N,
                h_winfo->block_size);
  GemmArgs a;
  st = gemm_common(d_x, M, K, N, d_y, d_ws, ws_bytes, &a);
  if (st != ENC_OK) return st;
  const uint8_t *w = static_cast<const uint8_t *>(d_wcomp);
  if (h_winfo->flags == 1) {
    a.wdense = reinterpret_cast<const uint16_t *>(w + kHeaderBytes);
  } else {
    a.wstream = w;
    a.log2b = (uint32_t)log2_block(h_winfo->block_size);
    a.nb = h_winfo->n_blocks;
    a.meta_off = h_winfo->meta_off;
    a.segoff_off = h_winfo->segoff_off;
    a.payload_off = h_winfo->payload_off;
    a.total = h_winfo->total_bytes;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  return launched(launch_gemm(a, s), s, "GEMM launch");
}

enc_status enc_gemm_dense(const uint16_t *d_x, uint32_t M, uint32_t K, const uint16_t *d_w,
                          uint32_t N, float *d_y, void *d_ws, uint64_t ws_bytes, void *stream) {
  clear_err();
  if (!d_w || !aligned16(d_w)) return fail(ENC_ERR_INVALID_ARG, "d_w NULL or unaligned");
  GemmArgs a;
  const enc_status st = gemm_common(d_x, M, K, N, d_y, d_ws, ws_bytes, &a);
  if (st != ENC_OK) return st;
  a.wdense = d_w;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return launched(launch_gemm(a, s), s, "GEMM launch");
}

uint64_t enc_gemm_nt_workspace_bytes(uint32_t M, uint32_t K, uint32_t N, uint32_t block_size) {
  const int lb = log2_block(block_size);
  // 0 for a shape enc_decompress_gemm_nt rejects (the plan divides by the
  // number of 64-column tiles)
  if (lb < 0 || M == 0 || M > 4096 || K == 0 || N == 0 || N % 64 || K % 32) return 0;
  return gemm_nt_workspace_bytes(M, K, N, (uint32_t)lb);
}

static enc_status gemm_nt_common(const uint16_t *d_x, uint32_t M, uint32_t K, uint32_t N,
                                 uint32_t log2b, float *d_y, void *d_ws, uint64_t ws_bytes,
                                 GemmArgs *a) {
  if (!d_x || !d_y || !d_ws) return fail(ENC_ERR_INVALID_ARG, "NULL device pointer");
  if (!aligned16(d_x) || !aligned16(d_y) || !aligned16(d_ws))
    return fail(ENC_ERR_INVALID_ARG, "device buffers must be 16-byte aligned");
  if (M == 0 || M > 4096 || K == 0 || N == 0)
    return fail(ENC_ERR_SHAPE, "M=%u K=%u N=%u out of range", M, K, N);
  if (N % 64) return fail(ENC_ERR_UNSUPPORTED, "N=%u must be a multiple of 64", N);
  if (K % 32) return fail(ENC_ERR_UNSUPPORTED, "K=%u must be a multiple of 32", K);
  const uint64_t need = gemm_nt_workspace_bytes(M, K, N, log2b);
  if (ws_bytes < need)
    return fail(ENC_ERR_CAPACITY, "GEMM workspace of %llu bytes needed", (unsigned long long)need);
  memset(a, 0, sizeof *a);
  a->x = d_x;
  a->y = d_y;
  a->M = M;
  a->K = K;
  a->N = N;
  a->log2b = log2b;
  a->partial = static_cast<float *>(d_ws);
  return ENC_OK;
}

enc_status enc_decompress_gemm_nt(const uint16_t *d_x, uint32_t M, uint32_t K, const void *d_wcomp,
                                  const enc_info *h_winfo, uint32_t N, float *d_y, void *d_ws,
                                  uint64_t ws_bytes, void *stream) {
  clear_err();
  enc_status st = check_info(h_winfo);
  if (st != ENC_OK) return st;
  if (h_winfo->dtype != 1) return fail(ENC_ERR_UNSUPPORTED, "the GEMM takes BF16 weights only");
  if (!d_wcomp || !aligned16(d_wcomp)) return fail(ENC_ERR_INVALID_ARG, "d_wcomp NULL or unaligned");
  if ((uint64_t)K * N != h_winfo->n_elems)
    return fail(ENC_ERR_SHAPE, "K*N=%llu but the stream holds %llu elements",
                (unsigned long long)K * N, (unsigned long long)h_winfo->n_elems);
  const bool raw = h_winfo->flags == 1;
  const int lb = log2_block(h_winfo->block_size);
  if (!raw && K % h_winfo->block_size)
    return fail(ENC_ERR_UNSUPPORTED, "K=%u not a multiple of the block size %u", K,
                h_winfo->block_size);
  if (!raw && h_winfo->total_bytes >= (1ull << 31))
    return fail(ENC_ERR_UNSUPPORTED, "coded stream above 2 GiB (32-bit buffer offsets)");
  GemmArgs a;
  st = gemm_nt_common(d_x, M, K, N, raw ? 9u : (uint32_t)lb, d_y, d_ws, ws_bytes, &a);
  if (st != ENC_OK) return st;
  const uint8_t *w = static_cast<const uint8_t *>(d_wcomp);
  if (raw) {
    a.wdense = reinterpret_cast<const uint16_t *>(w + kHeaderBytes);
  } else {
    a.wstream = w;
    a.nb = h_winfo->n_blocks;
    a.meta_off = h_winfo->meta_off;
    a.segoff_off = h_winfo->segoff_off;
    a.payload_off = h_winfo->payload_off;
    a.total = h_winfo->total_bytes;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  return launched(launch_gemm_nt(a, s), s, "GEMM launch");
}

enc_status enc_gemm_dense_nt(const uint16_t *d_x, uint32_t M, uint32_t K, const uint16_t *d_w,
                             uint32_t N, float *d_y, void *d_ws, uint64_t ws_bytes, void *stream) {
  clear_err();
  if (!d_w || !aligned16(d_w)) return fail(ENC_ERR_INVALID_ARG, "d_w NULL or unaligned");
  GemmArgs a;
  const enc_status st = gemm_nt_common(d_x, M, K, N, 9u, d_y, d_ws, ws_bytes, &a);
  if (st != ENC_OK) return st;
  a.wdense = d_w;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return launched(launch_gemm_nt(a, s), s, "GEMM launch");
}

enc_status enc_stream_probe(const void *d_src, uint64_t src_bytes, void *d_dst, uint64_t dst_bytes,
                            uint32_t items_per_thread, uint32_t threads_per_workgroup, void *stream) {
  clear_err();
  if (!d_src || !d_dst) return fail(ENC_ERR_INVALID_ARG, "NULL device pointer");
  if (!aligned16(d_src) || !aligned16(d_dst)) return fail(ENC_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  if (src_bytes == 0 || dst_bytes == 0 || src_bytes % 16 || dst_bytes % 16)
    return fail(ENC_ERR_INVALID_ARG, "sizes must be nonzero multiples of 16 bytes");
  if (items_per_thread != 1 && items_per_thread != 2 && items_per_thread != 4)
    return fail(ENC_ERR_INVALID_ARG, "items_per_thread must be 1, 2 or 4");
  const uint32_t T = threads_per_workgroup;
  if (T != 64 && T != 128 && T != 256)
    return fail(ENC_ERR_INVALID_ARG, "threads_per_workgroup must be 64, 128 or 256");
  const uintptr_t s0 = (uintptr_t)d_src, d0 = (uintptr_t)d_dst;
  if (s0 < d0 + dst_bytes && d0 < s0 + src_bytes) return fail(ENC_ERR_INVALID_ARG, "buffers overlap");
  const uint64_t nwg = (dst_bytes / 16 + (uint64_t)T * items_per_thread - 1) / ((uint64_t)T * items_per_thread);
  const uint64_t si = src_bytes / 16;
  // 32.32 fixed-point source run per workgroup: (workgroups x ratio) < 2^64
  if (nwg > (1ull << 30) || si >= (1ull << 31) || si / nwg + 1 >= (1ull << 31))
    return fail(ENC_ERR_UNSUPPORTED, "sizes too large for the probe's index arithmetic");
  hipStream_t s = static_cast<hipStream_t>(stream);
  return launched(launch_stream_probe(d_src, src_bytes, d_dst, dst_bytes, items_per_thread, T, s), s,
                  "probe launch");
}

uint64_t enc_validate_workspace_bytes(void) { return 256; }

enc_status enc_validate(const void *d_comp, const enc_info *h_info, void *d_ws, uint64_t ws_bytes,
                        void *stream, enc_check *h_check) {
  clear_err();
  enc_status st = check_info(h_info);
  if (st != ENC_OK) return st;
  if (!d_comp || !aligned16(d_comp)) return fail(ENC_ERR_INVALID_ARG, "d_comp NULL or unaligned");
  if (h_check) memset(h_check, 0, sizeof *h_check);
  if (h_info->flags == 1) return ENC_OK;   // RAW: the header is the whole structure
  if (!d_ws || !aligned16(d_ws) || ws_bytes < enc_validate_workspace_bytes())
    return fail(ENC_ERR_CAPACITY, "validation workspace of %llu bytes needed",
                (unsigned long long)enc_validate_workspace_bytes());
  hipStream_t s = static_cast<hipStream_t>(stream);
  ValidateArgs a;
  memset(&a, 0, sizeof a);
  a.stream = static_cast<const uint8_t *>(d_comp);
  a.result = static_cast<unsigned long long *>(d_ws);
  a.n = h_info->n_elems;
  a.nb = h_info->n_blocks;
  a.nseg = h_info->n_segments;
  a.meta_off = h_info->meta_off;
  a.segoff_off = h_info->segoff_off;
  a.payload_off = h_info->payload_off;
  a.payload_bytes = h_info->payload_bytes;
  a.log2b = (uint32_t)log2_block(h_info->block_size);
  a.pow2 = h_info->flags == 2;
  a.emax = exp_max(h_info->dtype);
  hipError_t e = hipMemsetAsync(d_ws, 0xFF, 3 * sizeof(unsigned long long), s);
  if (e != hipSuccess) return hip_fail(e, "result initialisation");
  e = launch_validate(a, s);
  if (e != hipSuccess) return hip_fail(e, "validation launch");
  unsigned long long r[3];
  e = hipMemcpyAsync(r, d_ws, sizeof r, hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return hip_fail(e, "result read-back");
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "stream synchronize");
  static const char *const what[3] = {"block %llu has a width above 8 (or not a power of two "
                                      "in a stream that declares power-of-two widths)",
                                      "stored segment offset %llu is not the prefix sum of the "
                                      "block sizes (index n_segments = payload_bytes)",
                                      "block %llu decodes an exponent above the field's maximum"};
  for (int k = 0; k < 3; ++k) {
    if (r[k] != ~0ull) {
      if (h_check) {
        h_check->kind = (uint32_t)(k + 1);
        h_check->index = r[k];
      }
      return fail(ENC_ERR_BAD_STREAM, what[k], r[k]);
    }
  }
  return ENC_OK;
}

const char *enc_status_string(enc_status s) {
  switch (s) {
    case ENC_OK: return "ok";
    case ENC_ERR_INVALID_ARG: return "invalid argument";
    case ENC_ERR_UNSUPPORTED: return "unsupported";
    case ENC_ERR_CAPACITY: return "buffer too small";
    case ENC_ERR_BAD_STREAM: return "bad stream";
    case ENC_ERR_SHAPE: return "shape mismatch";
    case ENC_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char *enc_last_error(void) { return g_err; }

}  // extern "C"
