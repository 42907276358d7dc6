/*
 * enc_oracle.c -- CPU oracle for lossless block-based fixed-length coding of
 * BF16 weights.
 *
 * TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT. Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg load this library. It shares no
 * code, header, table or constant with the GPU library: it redeclares the
 * stream layout itself from the written format definition.
 *
 * Plain, scalar, single-threaded C. Every loop follows the definition of the
 * stream step by step; nothing is blocked, fused or vectorised by hand. Bits
 * are set and read one at a time.
 *
 * Sources (the pages are abstracts; where they are silent the plainest reading
 * is taken and listed with the design notes):
 *  - "ENEC: A Lossless AI Model Compression Method Enabling Fast Inference on
 *    Ascend NPUs", Abstract: block-based fixed-length encoding; bit-width
 *    quantization with bit-packing; branch-free integer transformation;
 *    intra-segment scan for the prefix sums of block sizes.
 *  - "ZipServ: Fast and Memory-Efficient LLM Inference with Hardware-Aware
 *    Lossless Compression", Abstract: a fixed-length format decodable in
 *    constant time and in parallel; a fused decompress-GEMM.
 *
 * Readings used here (the pages give no layout):
 *  - a BF16 value x splits into an exponent byte E = (x >> 7) & 0xFF and a
 *    sign+mantissa byte SM = (sign << 7) | mantissa; FP16 and FP32 values
 *    split the same way into their exponent field (5 / 8 bits) and a
 *    sign+mantissa field (11 / 24 bits), the latter packed LSB first
 *    (header dtype 2 / 3);
 *  - the branch-free transform is d = E - base, base = the block minimum;
 *  - the block width is the number of bits of (max E - base), 0..8, with no
 *    further rounding of the width;
 *  - fields are packed LSB first, consecutively, within each block;
 *  - stored offsets: one u64 per 64-block segment (exclusive prefix sum of
 *    padded block payload sizes); offsets inside a segment are re-derived by
 *    the decoder from the widths.
 *
 * Parity status of each function is given in its comment; all are pinned by
 * the CPU tests (round trip, closed-form size, exhaustive width search,
 * brute-force bit layout, hand-derived blocks, exact GEMM special cases).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ----- stream layout constants (the format definition, restated here) ----- */
#define ORC_HEADER_BYTES 256u
#define ORC_SEG_BLOCKS 64u
#define ORC_SECTION_ALIGN 256u
#define ORC_PAYLOAD_ALIGN 16u
#define ORC_VERSION 1u
#define ORC_DTYPE_BF16 1u
#define ORC_FLAG_RAW 1u
#define ORC_FLAG_POW2 2u   /* coded stream whose widths are powers of two */
#define ORC_OPT_POW2 1u    /* encoder option: round widths up to 0, 1, 2, 4 or 8 */

/* status codes returned by the oracle (negative = failure) */
#define ORC_OK 0
#define ORC_E_ARG (-1)
#define ORC_E_CAPACITY (-3)
#define ORC_E_STREAM (-4)
#define ORC_E_NOMEM (-7)

static uint64_t round_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

static void put_le(uint8_t *p, uint64_t v, int nbytes) {
  for (int i = 0; i < nbytes; i++) p[i] = (uint8_t)(v >> (8 * i));
}

static uint64_t get_le(const uint8_t *p, int nbytes) {
  uint64_t v = 0;
  for (int i = 0; i < nbytes; i++) v |= (uint64_t)p[i] << (8 * i);
  return v;
}

/* ---------------------------------------------------------------------------
 * Field split (ENEC Abstract, "block-based fixed-length encoding" of the
 * exponent; reading: exponent byte plus a raw sign+mantissa byte).
 * ------------------------------------------------------------------------- */
unsigned orc_exponent(uint16_t x) { return (x >> 7) & 0xFFu; }

unsigned orc_signmant(uint16_t x) {
  unsigned sign = (x >> 15) & 1u;
  unsigned mant = x & 0x7Fu;
  return (sign << 7) | mant;
}

uint16_t orc_join(unsigned sm, unsigned e) {
  unsigned sign = (sm >> 7) & 1u;
  unsigned mant = sm & 0x7Fu;
  return (uint16_t)((sign << 15) | ((e & 0xFFu) << 7) | mant);
}

/* Element types. A value of `bits` bits is a sign (top bit), an exponent
 * field of exp_bits bits from bit exp_shift up, and the mantissa below it
 * (BF16 16/8/7, FP16 16/5/10, FP32 32/8/23). The coded field is always the
 * exponent; the rest -- sign and mantissa, exp_shift + 1 bits, read as
 * mantissa | sign << exp_shift -- is kept verbatim, packed LSB first. For
 * BF16 that rest is exactly the sign+mantissa byte of orc_signmant. */
#define ORC_DTYPE_FP16 2u
#define ORC_DTYPE_FP32 3u

typedef struct {
  unsigned bytes, bits, exp_shift, exp_bits;
} orc_dt;

static int dt_of(uint32_t dtype, orc_dt *t) {
  if (dtype == ORC_DTYPE_BF16) {
    t->bytes = 2; t->bits = 16; t->exp_shift = 7; t->exp_bits = 8;
  } else if (dtype == ORC_DTYPE_FP16) {
    t->bytes = 2; t->bits = 16; t->exp_shift = 10; t->exp_bits = 5;
  } else if (dtype == ORC_DTYPE_FP32) {
    t->bytes = 4; t->bits = 32; t->exp_shift = 23; t->exp_bits = 8;
  } else {
    return 0;
  }
  return 1;
}

static unsigned sm_bits_of(const orc_dt *t) { return t->exp_shift + 1; }

static uint32_t exponent_dt(uint32_t x, const orc_dt *t) {
  return (x >> t->exp_shift) & ((1u << t->exp_bits) - 1u);
}

static uint32_t signmant_dt(uint32_t x, const orc_dt *t) {
  uint32_t mant = x & ((1u << t->exp_shift) - 1u);
  uint32_t sign = (x >> (t->bits - 1)) & 1u;
  return mant | (sign << t->exp_shift);
}

static uint32_t join_dt(uint32_t sm, uint32_t e, const orc_dt *t) {
  uint32_t mant = sm & ((1u << t->exp_shift) - 1u);
  uint32_t sign = (sm >> t->exp_shift) & 1u;
  return (sign << (t->bits - 1)) | ((e & ((1u << t->exp_bits) - 1u)) << t->exp_shift) | mant;
}

uint32_t orc_exponent_dt(uint32_t x, uint32_t dtype) {
  orc_dt t;
  return dt_of(dtype, &t) ? exponent_dt(x, &t) : 0;
}

uint32_t orc_signmant_dt(uint32_t x, uint32_t dtype) {
  orc_dt t;
  return dt_of(dtype, &t) ? signmant_dt(x, &t) : 0;
}

uint32_t orc_join_dt(uint32_t sm, uint32_t e, uint32_t dtype) {
  orc_dt t;
  return dt_of(dtype, &t) ? join_dt(sm, e, &t) : 0;
}

static uint32_t elem(const void *x, uint64_t j, const orc_dt *t) {
  if (t->bytes == 2) return ((const uint16_t *)x)[j];
  return ((const uint32_t *)x)[j];
}

static void put_elem(void *out, uint64_t j, uint32_t v, const orc_dt *t) {
  if (t->bytes == 2)
    ((uint16_t *)out)[j] = (uint16_t)v;
  else
    ((uint32_t *)out)[j] = v;
}

/* Number of bits needed to write r (0 for r == 0): the smallest w with
 * r < 2^w ("bit-width quantization", ENEC Abstract, read as the minimal
 * width). Counted by repeated halving. */
unsigned orc_bit_width(unsigned r) {
  unsigned w = 0;
  while (r != 0) {
    w++;
    r >>= 1;
  }
  return w;
}

/* The width variant that keeps only powers of two ("bit-width quantization"
 * with "hierarchical halving bit-packing", ENEC Abstract, read as: the width
 * of a block is rounded up to the next of 0, 1, 2, 4, 8, so that a byte holds
 * exactly 8, 4, 2 or 1 codes). Found by doubling from 1. */
unsigned orc_pow2_width(unsigned r) {
  unsigned w = orc_bit_width(r);
  if (w == 0) return 0;
  unsigned p = 1;
  while (p < w) p *= 2;
  return p;
}

static int width_allowed(unsigned w, uint32_t flags) {
  if (w > 8) return 0;
  if ((flags & ORC_FLAG_POW2) && w != 0 && w != 1 && w != 2 && w != 4 && w != 8) return 0;
  return 1;
}

/* ---------------------------------------------------------------------------
 * Layout of a non-RAW stream for n elements and block size B.
 * ------------------------------------------------------------------------- */
typedef struct {
  uint64_t n, nb, nseg;
  uint64_t sm_off, meta_off, segoff_off, payload_off;
} orc_layout;

static orc_layout layout_of(uint64_t n, uint32_t B, const orc_dt *t) {
  orc_layout L;
  L.n = n;
  L.nb = (n + B - 1) / B;
  L.nseg = (L.nb + ORC_SEG_BLOCKS - 1) / ORC_SEG_BLOCKS;
  L.sm_off = ORC_HEADER_BYTES;
  L.meta_off = L.sm_off + round_up((sm_bits_of(t) * n + 7) / 8, ORC_SECTION_ALIGN);
  L.segoff_off = L.meta_off + round_up(2 * L.nb, ORC_SECTION_ALIGN);
  L.payload_off = L.segoff_off + round_up(8 * L.nseg, ORC_SECTION_ALIGN);
  return L;
}

/* Length of block i (the last block may be shorter). */
static uint64_t block_len(uint64_t n, uint32_t B, uint64_t i) {
  uint64_t start = i * B;
  uint64_t end = start + B;
  if (end > n) end = n;
  return end - start;
}

/* Padded payload bytes of a block of L codes of w bits. */
uint64_t orc_block_payload_bytes(unsigned w, uint64_t L) {
  uint64_t bits = (uint64_t)w * L;
  uint64_t bytes = (bits + 7) / 8;
  return round_up(bytes, ORC_PAYLOAD_ALIGN);
}

static int block_size_ok(uint32_t B) { return B >= 8 && B <= 4096 && B % 8 == 0; }

/* ---------------------------------------------------------------------------
 * Per-block base and width (ENEC Abstract: "branch-free integer
 * transformation" read as subtraction of the block minimum exponent; "bit-width
 * quantization" read as the minimal width of the transformed values).
 * Writes base[nb], width[nb]. Returns nb, or a negative status.
 * ------------------------------------------------------------------------- */
int64_t orc_block_params_dt(const void *x, uint64_t n, uint32_t dtype, uint32_t B, uint32_t opts,
                            uint8_t *base, uint8_t *width) {
  orc_dt dt;
  if (!block_size_ok(B) || !dt_of(dtype, &dt)) return ORC_E_ARG;
  uint64_t nb = (n + B - 1) / B;
  for (uint64_t i = 0; i < nb; i++) {
    uint64_t L = block_len(n, B, i);
    unsigned lo = 255, hi = 0;
    for (uint64_t t = 0; t < L; t++) {
      unsigned e = exponent_dt(elem(x, i * B + t, &dt), &dt);
      if (e < lo) lo = e;
      if (e > hi) hi = e;
    }
    base[i] = (uint8_t)lo;
    width[i] = (uint8_t)((opts & ORC_OPT_POW2) ? orc_pow2_width(hi - lo) : orc_bit_width(hi - lo));
  }
  return (int64_t)nb;
}

int64_t orc_block_params_opts(const uint16_t *x, uint64_t n, uint32_t B, uint32_t opts,
                              uint8_t *base, uint8_t *width) {
  return orc_block_params_dt(x, n, ORC_DTYPE_BF16, B, opts, base, width);
}

int64_t orc_block_params(const uint16_t *x, uint64_t n, uint32_t B, uint8_t *base,
                         uint8_t *width) {
  return orc_block_params_opts(x, n, B, 0, base, width);
}

/* Size in bytes of the stream that orc_encode writes for x (RAW fallback
 * included). Closed form of the layout: header + aligned sections + sum of
 * padded block payloads; RAW when that is not smaller than header + 2n. */
int64_t orc_stream_size_dt(const void *x, uint64_t n, uint32_t dtype, uint32_t B, uint32_t opts) {
  orc_dt dt;
  if (!block_size_ok(B) || !dt_of(dtype, &dt)) return ORC_E_ARG;
  uint64_t raw_total = ORC_HEADER_BYTES + dt.bytes * n;
  if (n == 0) return (int64_t)raw_total;
  orc_layout L = layout_of(n, B, &dt);
  uint8_t *base = (uint8_t *)malloc(L.nb), *w = (uint8_t *)malloc(L.nb);
  if (!base || !w) {
    free(base);
    free(w);
    return ORC_E_NOMEM;
  }
  orc_block_params_dt(x, n, dtype, B, opts, base, w);
  uint64_t payload = 0;
  for (uint64_t i = 0; i < L.nb; i++) payload += orc_block_payload_bytes(w[i], block_len(n, B, i));
  free(base);
  free(w);
  uint64_t total = L.payload_off + payload;
  return (int64_t)(total >= raw_total ? raw_total : total);
}

int64_t orc_stream_size_opts(const uint16_t *x, uint64_t n, uint32_t B, uint32_t opts) {
  return orc_stream_size_dt(x, n, ORC_DTYPE_BF16, B, opts);
}

int64_t orc_stream_size(const uint16_t *x, uint64_t n, uint32_t B) {
  return orc_stream_size_opts(x, n, B, 0);
}

static void write_header(uint8_t *h, uint32_t dtype, uint32_t flags, uint32_t B, uint64_t n, uint64_t nb,
                         uint64_t nseg, uint64_t sm_off, uint64_t meta_off, uint64_t segoff_off,
                         uint64_t payload_off, uint64_t payload_bytes, uint64_t raw_off,
                         uint64_t total) {
  memset(h, 0, ORC_HEADER_BYTES);
  h[0] = 'E';
  h[1] = 'N';
  h[2] = 'C';
  h[3] = 'B';
  put_le(h + 4, ORC_VERSION, 2);
  put_le(h + 6, dtype, 2);
  put_le(h + 8, flags, 4);
  put_le(h + 12, B, 4);
  put_le(h + 16, ORC_SEG_BLOCKS, 4);
  put_le(h + 20, 0, 4);
  put_le(h + 24, n, 8);
  put_le(h + 32, nb, 8);
  put_le(h + 40, nseg, 8);
  put_le(h + 48, sm_off, 8);
  put_le(h + 56, meta_off, 8);
  put_le(h + 64, segoff_off, 8);
  put_le(h + 72, payload_off, 8);
  put_le(h + 80, payload_bytes, 8);
  put_le(h + 88, raw_off, 8);
  put_le(h + 96, total, 8);
}

/* Set bit k of the byte array q (bit k = bit (k mod 8) of byte k / 8). */
static void set_bit(uint8_t *q, uint64_t k) { q[k >> 3] |= (uint8_t)(1u << (k & 7)); }

static unsigned get_bit(const uint8_t *q, uint64_t k) { return (q[k >> 3] >> (k & 7)) & 1u; }

/* ---------------------------------------------------------------------------
 * Encoder. Writes the whole stream into out[0..cap). Returns the stream size
 * or a negative status. Steps, in order:
 *  1. split every value into its exponent field and the rest (sign and
 *     mantissa; for BF16 the sign+mantissa byte);
 *  2. per block: base = min exponent, width = bits of (max - base);
 *  3. per block: transformed codes d = exponent - base;
 *  4. per block: padded payload size; per segment of 64 blocks: exclusive
 *     prefix sum of the payload sizes (ENEC Abstract, intra-segment scan);
 *  5. pack each block's codes at its fixed width, LSB first;
 *  6. fall back to a verbatim (RAW) stream when that is not larger.
 * ------------------------------------------------------------------------- */
int64_t orc_encode_dt(const void *x, uint64_t n, uint32_t dtype, uint32_t B, uint32_t opts,
                      uint8_t *out, uint64_t cap) {
  orc_dt dt;
  if (!block_size_ok(B) || !dt_of(dtype, &dt)) return ORC_E_ARG;
  if (n > 0 && x == NULL) return ORC_E_ARG;
  if (opts & ~ORC_OPT_POW2) return ORC_E_ARG;
  int64_t size = orc_stream_size_dt(x, n, dtype, B, opts);
  if (size < 0) return size;
  if ((uint64_t)size > cap) return ORC_E_CAPACITY;
  uint64_t raw_total = ORC_HEADER_BYTES + dt.bytes * n;

  if ((uint64_t)size == raw_total) {
    /* RAW: header, then the input values verbatim, little-endian. */
    memset(out, 0, (size_t)size);
    write_header(out, dtype, ORC_FLAG_RAW, B, n, 0, 0, 0, 0, 0, 0, 0, ORC_HEADER_BYTES, raw_total);
    for (uint64_t j = 0; j < n; j++)
      put_le(out + ORC_HEADER_BYTES + dt.bytes * j, elem(x, j, &dt), (int)dt.bytes);
    return size;
  }

  orc_layout L = layout_of(n, B, &dt);
  uint8_t *base = (uint8_t *)malloc(L.nb), *w = (uint8_t *)malloc(L.nb);
  uint64_t *psize = (uint64_t *)malloc(L.nb * sizeof(uint64_t));
  if (!base || !w || !psize) {
    free(base);
    free(w);
    free(psize);
    return ORC_E_NOMEM;
  }
  orc_block_params_dt(x, n, dtype, B, opts, base, w);
  for (uint64_t i = 0; i < L.nb; i++) psize[i] = orc_block_payload_bytes(w[i], block_len(n, B, i));

  memset(out, 0, (size_t)size);

  /* sign+mantissa plane: field j = bits [j S, j S + S), LSB first */
  const unsigned S = sm_bits_of(&dt);
  for (uint64_t j = 0; j < n; j++) {
    uint32_t sm = signmant_dt(elem(x, j, &dt), &dt);
    for (unsigned b = 0; b < S; b++)
      if ((sm >> b) & 1u) set_bit(out + L.sm_off, (uint64_t)j * S + b);
  }

  /* meta: {base, width} per block */
  for (uint64_t i = 0; i < L.nb; i++) {
    out[L.meta_off + 2 * i] = base[i];
    out[L.meta_off + 2 * i + 1] = w[i];
  }

  /* segment offsets: exclusive prefix sum of payload sizes, one per segment */
  uint64_t running = 0;
  for (uint64_t i = 0; i < L.nb; i++) {
    if (i % ORC_SEG_BLOCKS == 0) put_le(out + L.segoff_off + 8 * (i / ORC_SEG_BLOCKS), running, 8);
    running += psize[i];
  }
  uint64_t payload_bytes = running;

  /* payloads, concatenated in block order */
  uint64_t pos = L.payload_off;
  for (uint64_t i = 0; i < L.nb; i++) {
    uint64_t len = block_len(n, B, i);
    uint8_t *q = out + pos;
    for (uint64_t t = 0; t < len; t++) {
      unsigned d = exponent_dt(elem(x, i * B + t, &dt), &dt) - base[i];
      for (unsigned b = 0; b < w[i]; b++)
        if ((d >> b) & 1u) set_bit(q, (uint64_t)t * w[i] + b);
    }
    pos += psize[i];
  }

  write_header(out, dtype, (opts & ORC_OPT_POW2) ? ORC_FLAG_POW2 : 0, B, n, L.nb, L.nseg,
               L.sm_off, L.meta_off, L.segoff_off, L.payload_off, payload_bytes, 0,
               L.payload_off + payload_bytes);
  free(base);
  free(w);
  free(psize);
  return size;
}

int64_t orc_encode_opts(const uint16_t *x, uint64_t n, uint32_t B, uint32_t opts, uint8_t *out,
                        uint64_t cap) {
  return orc_encode_dt(x, n, ORC_DTYPE_BF16, B, opts, out, cap);
}

int64_t orc_encode(const uint16_t *x, uint64_t n, uint32_t B, uint8_t *out, uint64_t cap) {
  return orc_encode_opts(x, n, B, 0, out, cap);
}

/* ---------------------------------------------------------------------------
 * Header parsing and full validation. Fills the fields the decoder needs.
 * ------------------------------------------------------------------------- */
typedef struct {
  uint32_t dtype, flags, B;
  orc_dt dt;
  uint64_t n, nb, nseg, sm_off, meta_off, segoff_off, payload_off, payload_bytes, raw_off, total;
} orc_header;

static int parse_header_fields(const uint8_t *s, uint64_t bytes, orc_header *h) {
  if (s == NULL || bytes < ORC_HEADER_BYTES) return ORC_E_STREAM;
  if (s[0] != 'E' || s[1] != 'N' || s[2] != 'C' || s[3] != 'B') return ORC_E_STREAM;
  if (get_le(s + 4, 2) != ORC_VERSION) return ORC_E_STREAM;
  h->dtype = (uint32_t)get_le(s + 6, 2);
  if (!dt_of(h->dtype, &h->dt)) return ORC_E_STREAM;
  h->flags = (uint32_t)get_le(s + 8, 4);
  h->B = (uint32_t)get_le(s + 12, 4);
  if (get_le(s + 16, 4) != ORC_SEG_BLOCKS || get_le(s + 20, 4) != 0) return ORC_E_STREAM;
  h->n = get_le(s + 24, 8);
  h->nb = get_le(s + 32, 8);
  h->nseg = get_le(s + 40, 8);
  h->sm_off = get_le(s + 48, 8);
  h->meta_off = get_le(s + 56, 8);
  h->segoff_off = get_le(s + 64, 8);
  h->payload_off = get_le(s + 72, 8);
  h->payload_bytes = get_le(s + 80, 8);
  h->raw_off = get_le(s + 88, 8);
  h->total = get_le(s + 96, 8);
  for (int k = 104; k < 256; k++)
    if (s[k] != 0) return ORC_E_STREAM;
  if (!block_size_ok(h->B)) return ORC_E_STREAM;
  if (h->total > bytes) return ORC_E_STREAM;
  if (h->flags == ORC_FLAG_RAW) {
    if (h->nb || h->nseg || h->sm_off || h->meta_off || h->segoff_off || h->payload_off ||
        h->payload_bytes || h->raw_off != ORC_HEADER_BYTES ||
        h->total != ORC_HEADER_BYTES + h->dt.bytes * h->n)
      return ORC_E_STREAM;
    return ORC_OK;
  }
  if ((h->flags != 0 && h->flags != ORC_FLAG_POW2) || h->n == 0) return ORC_E_STREAM;
  orc_layout L = layout_of(h->n, h->B, &h->dt);
  if (h->nb != L.nb || h->nseg != L.nseg || h->sm_off != L.sm_off || h->meta_off != L.meta_off ||
      h->segoff_off != L.segoff_off || h->payload_off != L.payload_off || h->raw_off != 0 ||
      h->total != h->payload_off + h->payload_bytes)
    return ORC_E_STREAM;
  return ORC_OK;
}

/* The two structural conditions on the data sections of a coded stream with
 * a consistent header: every width is at most 8, and a power of two in a
 * stream flagged so (kind 1, index = first other block), and each stored
 * segment offset equals the sum of the padded
 * payload sizes of all earlier blocks, with payload_bytes equal to the sum
 * over all blocks (kind 2, index = first wrong stored offset; index nseg
 * stands for payload_bytes). Returns 0 when both hold. */
static int check_widths_offsets(const uint8_t *s, const orc_header *h, uint64_t *index) {
  for (uint64_t i = 0; i < h->nb; i++) {
    if (!width_allowed(s[h->meta_off + 2 * i + 1], h->flags)) {
      *index = i;
      return 1;
    }
  }
  uint64_t running = 0;
  for (uint64_t i = 0; i < h->nb; i++) {
    if (i % ORC_SEG_BLOCKS == 0 &&
        get_le(s + h->segoff_off + 8 * (i / ORC_SEG_BLOCKS), 8) != running) {
      *index = i / ORC_SEG_BLOCKS;
      return 2;
    }
    running += orc_block_payload_bytes(s[h->meta_off + 2 * i + 1], block_len(h->n, h->B, i));
  }
  if (running != h->payload_bytes) {
    *index = h->nseg;
    return 2;
  }
  return 0;
}

static int parse_header(const uint8_t *s, uint64_t bytes, orc_header *h) {
  int st = parse_header_fields(s, bytes, h);
  if (st != ORC_OK || h->flags == ORC_FLAG_RAW) return st;
  uint64_t index;
  return check_widths_offsets(s, h, &index) == 0 ? ORC_OK : ORC_E_STREAM;
}

/* Validates a stream; returns its element count or a negative status. */
int64_t orc_stream_elements(const uint8_t *s, uint64_t bytes) {
  orc_header h;
  int st = parse_header(s, bytes, &h);
  if (st != ORC_OK) return st;
  return (int64_t)h.n;
}

/* Payload start of block i, found the way a parallel decoder finds it: the
 * stored offset of its segment plus the sizes of the earlier blocks of the
 * same segment (ZipServ Abstract: every block is located in the same, fixed
 * number of steps, so all blocks decode in parallel; ENEC Abstract: the scan
 * within a segment). */
static uint64_t block_payload_start(const uint8_t *s, const orc_header *h, uint64_t i) {
  uint64_t seg = i / ORC_SEG_BLOCKS;
  uint64_t off = get_le(s + h->segoff_off + 8 * seg, 8);
  for (uint64_t k = seg * ORC_SEG_BLOCKS; k < i; k++)
    off += orc_block_payload_bytes(s[h->meta_off + 2 * k + 1], block_len(h->n, h->B, k));
  return h->payload_off + off;
}

/* Bits [k, k + nbits) of the byte array q, LSB first. */
static uint32_t get_bits(const uint8_t *q, uint64_t k, unsigned nbits) {
  uint32_t v = 0;
  for (unsigned b = 0; b < nbits; b++) v |= get_bit(q, k + b) << b;
  return v;
}

/* Decoder for one element j of a validated non-RAW stream (the per-element
 * definition: locate block, read the w-bit field, add the base, rejoin with
 * the element's sign+mantissa field). */
static uint32_t decode_one(const uint8_t *s, const orc_header *h, uint64_t j, uint64_t qstart) {
  uint64_t i = j / h->B, t = j - i * h->B;
  unsigned base = s[h->meta_off + 2 * i];
  unsigned w = s[h->meta_off + 2 * i + 1];
  unsigned d = get_bits(s + qstart, (uint64_t)t * w, w);
  const unsigned S = sm_bits_of(&h->dt);
  uint32_t sm = get_bits(s + h->sm_off, (uint64_t)j * S, S);
  return join_dt(sm, base + d, &h->dt);
}

/* Full decoder. out must hold n elements of the stream's type (2 bytes for
 * BF16 and FP16, 4 for FP32; n = the stream's element count). Returns ORC_OK
 * or a negative status. */
int orc_decode_dt(const uint8_t *s, uint64_t bytes, void *out, uint64_t n) {
  orc_header h;
  int st = parse_header(s, bytes, &h);
  if (st != ORC_OK) return st;
  if (n != h.n) return ORC_E_ARG;
  if (h.flags == ORC_FLAG_RAW) {
    for (uint64_t j = 0; j < n; j++)
      put_elem(out, j, (uint32_t)get_le(s + h.raw_off + h.dt.bytes * j, (int)h.dt.bytes), &h.dt);
    return ORC_OK;
  }
  for (uint64_t i = 0; i < h.nb; i++) {
    uint64_t q = block_payload_start(s, &h, i);
    uint64_t len = block_len(h.n, h.B, i);
    for (uint64_t t = 0; t < len; t++) put_elem(out, i * h.B + t, decode_one(s, &h, i * h.B + t, q), &h.dt);
  }
  return ORC_OK;
}

/* The stream's element type (1 BF16, 2 FP16, 3 FP32) or a negative status. */
int64_t orc_stream_dtype(const uint8_t *s, uint64_t bytes) {
  orc_header h;
  int st = parse_header(s, bytes, &h);
  if (st != ORC_OK) return st;
  return (int64_t)h.dtype;
}

/* BF16 (and FP16) streams into 16-bit outputs. */
int orc_decode(const uint8_t *s, uint64_t bytes, uint16_t *out, uint64_t n) {
  int64_t dt = orc_stream_dtype(s, bytes);
  if (dt < 0) return (int)dt;
  if (dt == ORC_DTYPE_FP32) return ORC_E_ARG;
  return orc_decode_dt(s, bytes, out, n);
}

/* Decoder for elements [first, first + count) only (for sampled checks of
 * large tensors). Same definition as orc_decode_dt. */
int orc_decode_range_dt(const uint8_t *s, uint64_t bytes, uint64_t first, uint64_t count,
                        void *out) {
  orc_header h;
  int st = parse_header(s, bytes, &h);
  if (st != ORC_OK) return st;
  if (first > h.n || count > h.n - first) return ORC_E_ARG;
  for (uint64_t j = first; j < first + count; j++) {
    if (h.flags == ORC_FLAG_RAW) {
      put_elem(out, j - first, (uint32_t)get_le(s + h.raw_off + h.dt.bytes * j, (int)h.dt.bytes), &h.dt);
    } else {
      uint64_t i = j / h.B;
      put_elem(out, j - first, decode_one(s, &h, j, block_payload_start(s, &h, i)), &h.dt);
    }
  }
  return ORC_OK;
}

int orc_decode_range(const uint8_t *s, uint64_t bytes, uint64_t first, uint64_t count,
                     uint16_t *out) {
  int64_t dt = orc_stream_dtype(s, bytes);
  if (dt < 0) return (int)dt;
  if (dt == ORC_DTYPE_FP32) return ORC_E_ARG;
  return orc_decode_range_dt(s, bytes, first, count, out);
}

/* Deep validity of a stream whose header is consistent. Returns the kind of
 * the first failing condition, in this order: 1 = a width above 8, 2 = a
 * stored segment offset (or payload_bytes) that is not the prefix sum of the
 * padded block sizes, 3 = an element whose base + code exceeds the largest
 * exponent field value (255; 31 for FP16): the transform subtracts the block
 * minimum, so a stream written from real input never has one (ENEC
 * Abstract: branch-free integer transformation). *index receives the first
 * failing block (1, 3) or stored offset (2). 0 = valid (RAW streams always
 * are). Negative = bad header. */
int orc_validate(const uint8_t *s, uint64_t bytes, uint64_t *index) {
  orc_header h;
  *index = 0;
  int st = parse_header_fields(s, bytes, &h);
  if (st != ORC_OK) return st;
  if (h.flags == ORC_FLAG_RAW) return 0;
  int kind = check_widths_offsets(s, &h, index);
  if (kind != 0) return kind;
  const unsigned emax = (1u << h.dt.exp_bits) - 1u;
  for (uint64_t i = 0; i < h.nb; i++) {
    uint64_t q = block_payload_start(s, &h, i);
    unsigned base = s[h.meta_off + 2 * i];
    unsigned w = s[h.meta_off + 2 * i + 1];
    uint64_t len = block_len(h.n, h.B, i);
    for (uint64_t t = 0; t < len; t++) {
      unsigned d = get_bits(s + q, t * w, w);
      if (base + d > emax) {
        *index = i;
        return 3;
      }
    }
  }
  return 0;
}

/* ---------------------------------------------------------------------------
 * GEMM oracle (ZipServ Abstract: the fused decompress-GEMM computes the same
 * product as decompression followed by a GEMM). Y[m][n] = sum_k X[m][k] *
 * W[k][n] in double precision, k ascending for every output; absb[m][n] =
 * sum_k |X[m][k] * W[k][n]|. X is [M,K], W is [K,N], both BF16 row-major.
 * Products of two BF16 values are exact in double.
 * ------------------------------------------------------------------------- */
double orc_bf16_to_double(uint16_t v) {
  uint32_t u = (uint32_t)v << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

void orc_gemm_f64(const uint16_t *X, uint32_t M, uint32_t K, const uint16_t *W, uint32_t N,
                  double *Y, double *absb) {
  for (uint64_t i = 0; i < (uint64_t)M * N; i++) {
    Y[i] = 0.0;
    if (absb) absb[i] = 0.0;
  }
  for (uint32_t m = 0; m < M; m++) {
    for (uint32_t k = 0; k < K; k++) {
      double xv = orc_bf16_to_double(X[(uint64_t)m * K + k]);
      const uint16_t *wrow = W + (uint64_t)k * N;
      double *yrow = Y + (uint64_t)m * N;
      double *arow = absb ? absb + (uint64_t)m * N : NULL;
      for (uint32_t n = 0; n < N; n++) {
        double p = xv * orc_bf16_to_double(wrow[n]);
        yrow[n] += p;
        if (arow) arow[n] += p < 0 ? -p : p;
      }
    }
  }
}

/* Same product for a chosen set of columns only: Y[m][c], absb[m][c] for
 * c in [0, ncols), column index cols[c]. */
void orc_gemm_f64_cols(const uint16_t *X, uint32_t M, uint32_t K, const uint16_t *W, uint32_t N,
                       const uint32_t *cols, uint32_t ncols, double *Y, double *absb) {
  for (uint32_t m = 0; m < M; m++) {
    for (uint32_t c = 0; c < ncols; c++) {
      double acc = 0.0, aacc = 0.0;
      for (uint32_t k = 0; k < K; k++) {
        double p = orc_bf16_to_double(X[(uint64_t)m * K + k]) *
                   orc_bf16_to_double(W[(uint64_t)k * N + cols[c]]);
        acc += p;
        aacc += p < 0 ? -p : p;
      }
      Y[(uint64_t)m * ncols + c] = acc;
      if (absb) absb[(uint64_t)m * ncols + c] = aacc;
    }
  }
}
