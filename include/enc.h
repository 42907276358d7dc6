/*
 * enc.h -- C ABI of libenc.so: lossless block-based fixed-length coding of
 * BF16 weights on MI355X (gfx950), with a fused decompress-GEMM.
 *
 * What the operations are (the pages give abstracts, no interface):
 *  - "ENEC: A Lossless AI Model Compression Method Enabling Fast Inference on
 *    Ascend NPUs", Abstract: weights are compressed losslessly with a
 *    block-based fixed-length code (per-block bit width, bit-packing, a
 *    branch-free integer transform, an intra-segment prefix scan of block
 *    sizes) so that less weight data has to be moved at inference time.
 *  - "ZipServ: Fast and Memory-Efficient LLM Inference with Hardware-Aware
 *    Lossless Compression", Abstract: a fixed-length format decodes in
 *    constant time and in parallel, and a fused decompress-GEMM consumes the
 *    compressed weights directly, with no intermediate decompressed buffer.
 *  - "MINE: Entropy-coded Memory-efficient Inference for Large Language
 *    Models", Abstract: single-stream decoding is memory-bound because every
 *    weight is streamed once per generated token.
 *
 * Stream format (little-endian; all pad bytes zero):
 *   [0, 256)            header: "ENCB", u16 version=1, u16 dtype (1 BF16,
 *                       2 FP16, 3 FP32),
 *                       u32 flags (0 = coded, 1 = RAW, 2 = coded with
 *                       power-of-two widths), u32 block_size, u32 64,
 *                       u32 0, then u64 n_elems, n_blocks, n_segments, sm_off,
 *                       meta_off, segoff_off, payload_off, payload_bytes,
 *                       raw_off, total_bytes; bytes 104..255 zero.
 *   sm_off = 256        the kept field of each value: sign on top of the
 *                       mantissa, S bits (S = 8 for BF16: sign in bit 7,
 *                       mantissa in bits 6..0; 11 for FP16; 24 for FP32),
 *                       packed LSB first in element order (for BF16 one
 *                       byte per value), ceil(S n / 8) bytes, section padded
 *                       to a multiple of 256.
 *   meta_off            u8[2 * n_blocks]: {base, width} per block, padded.
 *   segoff_off          u64[n_segments]: exclusive prefix sum of padded block
 *                       payload sizes at each 64-block segment start, padded.
 *   payload_off         per block, ceil(width * len / 8) bytes rounded up to
 *                       16: the codes exponent - base, width bits each, packed
 *                       LSB first in element order. The exponent field is 8
 *                       bits for BF16 and FP32, 5 bits for FP16.
 *   RAW streams (flags 1): header, then the n input values verbatim at
 *   raw_off = 256 (2 or 4 bytes each); chosen when the coded stream would not
 *   be smaller.
 *   Flags 2: the widths were rounded up to 0, 1, 2, 4 or 8 (ENEC Abstract:
 *   bit-width quantization with hierarchical halving bit-packing, read as
 *   power-of-two widths, so a byte holds exactly 8, 4, 2 or 1 codes); the
 *   layout is otherwise identical and every entry point reads such streams.
 *   A stream is valid only if every decoded exponent base + code fits the
 *   exponent field (<= 255, or <= 31 for FP16; always true for a stream
 *   written by these rules).
 *   FP16 and FP32 streams (the same code applied to the other float layouts)
 *   are written by enc_compress_dt and read by enc_decompress, the batched
 *   decode, enc_read_info, enc_parse_header and enc_validate; the GEMMs take
 *   BF16 streams only (ENC_ERR_UNSUPPORTED otherwise).
 *
 * Conventions for every entry point:
 *  - d_ pointers are device (HBM) pointers, h_ pointers are host pointers.
 *    The caller owns every buffer; the library never allocates or frees
 *    device memory, and keeps no state between calls.
 *  - Device buffers holding streams, value arrays and float arrays must be
 *    16-byte aligned; inputs and outputs must not overlap.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Calls are asynchronous on that stream unless stated otherwise; a fault
 *    inside a kernel surfaces at the caller's next synchronisation.
 *  - Every entry point checks its arguments on the host before launching
 *    anything; failures return a negative enc_status and set a thread-local
 *    message readable with enc_last_error(). Nothing is launched on failure.
 *  - With the environment variable ENC_DEBUG_SYNC set (to anything but "" or
 *    "0"), the asynchronous entry points synchronise their stream after
 *    launching (except while it is being captured into a graph), so a kernel
 *    fault is returned as ENC_ERR_HIP by the call that caused it.
 *  - Two more variables exist for tests: ENC_LOOKBACK_SPINS (polls of an
 *    unpublished tile before the single-pass encoder gives up and the
 *    two-pass encoder takes over; 0 makes every tile after the first give
 *    up at once, so that path always runs) and
 *    ENC_DECODE_MAX_GRID (workgroups per decode launch, below the default
 *    2^23, to run the several-launch path on small inputs). Results do not
 *    depend on either.
 */
#ifndef ENC_H
#define ENC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum enc_status {
  ENC_OK = 0,
  ENC_ERR_INVALID_ARG = -1, /* null pointer, misalignment, bad size or block size */
  ENC_ERR_UNSUPPORTED = -2, /* valid request outside what the kernels implement */
  ENC_ERR_CAPACITY = -3,    /* output or workspace buffer too small */
  ENC_ERR_BAD_STREAM = -4,  /* header or layout of a stream is inconsistent */
  ENC_ERR_SHAPE = -5,       /* GEMM shapes do not match the stream */
  ENC_ERR_HIP = -6          /* a HIP runtime call or a launch failed */
} enc_status;

/* Parsed header of a stream (field meanings as in the format above). */
typedef struct enc_info {
  uint32_t version, dtype, flags, block_size;
  uint64_t n_elems, n_blocks, n_segments;
  uint64_t sm_off, meta_off, segoff_off, payload_off, payload_bytes, raw_off, total_bytes;
} enc_info;

/* Largest stream any n-element input can produce: 256 + 2 n (the RAW size). */
uint64_t enc_compress_bound(uint64_t n_elems);

/* Device workspace bytes enc_compress needs for n elements at block size B
 * (per-block {base, width}, per-segment sums and offsets, a size slot).
 * Returns 0 for an unsupported block size. */
uint64_t enc_compress_workspace_bytes(uint64_t n_elems, uint32_t block_size);

/* Compress n BF16 values (bit patterns) d_in into d_out (ENEC Abstract).
 * Block size: 128, 256, 512, 1024, 2048 or 4096. Launches the width/segment
 * kernel, the scan of segment sizes and the pack kernel on `stream`; then
 * synchronises `stream` once to read back the stream size (the only blocking
 * point of the library), and fills *h_info. The bytes written are exactly
 * the ones the format above prescribes (the stream is unique for a given
 * input and block size). out_capacity must be
 * at least the final stream size (enc_compress_bound(n) always suffices). */
enc_status enc_compress(const uint16_t *d_in, uint64_t n_elems, uint32_t block_size, void *d_out,
                        uint64_t out_capacity, void *d_ws, uint64_t ws_bytes, void *stream,
                        enc_info *h_info);

/* enc_compress with options (bitwise or; 0 = enc_compress):
 *   ENC_OPT_POW2_WIDTHS  round every block width up to 0, 1, 2, 4 or 8 and
 *                        write flags 2 (if the result is RAW, flags 1).
 * Unknown option bits: ENC_ERR_INVALID_ARG. */
enum { ENC_OPT_POW2_WIDTHS = 1 };
enc_status enc_compress_ex(const uint16_t *d_in, uint64_t n_elems, uint32_t block_size,
                           uint32_t options, void *d_out, uint64_t out_capacity, void *d_ws,
                           uint64_t ws_bytes, void *stream, enc_info *h_info);

/* Largest stream an n-element input of the given dtype (1 BF16, 2 FP16,
 * 3 FP32) can produce: 256 + element bytes x n (the RAW size); 0 for an
 * unknown dtype. */
uint64_t enc_compress_bound_dt(uint64_t n_elems, uint32_t dtype);

/* Compress n values of the given dtype (bit patterns, 2 bytes each for BF16
 * and FP16, 4 for FP32) -- the block code above with the element type's
 * exponent and kept fields. dtype 1 is enc_compress_ex. FP16 and FP32 take
 * the same single pass (decoupled look-back) as BF16 when out_capacity holds
 * the RAW size (enc_compress_bound_dt), with one synchronisation of `stream`
 * to read back the size; otherwise, or should a look-back wait give up, a
 * width kernel, the scan of segment sizes, the synchronisation, then the
 * pack kernel (the input read twice). Either way the bytes are the ones the
 * format prescribes. Same block sizes, options, workspace size
 * (enc_compress_workspace_bytes) and capacity rule (the final stream size;
 * enc_compress_bound_dt always suffices). Unknown dtype:
 * ENC_ERR_UNSUPPORTED. */
enc_status enc_compress_dt(const void *d_in, uint64_t n_elems, uint32_t dtype, uint32_t block_size,
                           uint32_t options, void *d_out, uint64_t out_capacity, void *d_ws,
                           uint64_t ws_bytes, void *stream, enc_info *h_info);

/* Batched compression of BF16 tensors (ENEC Abstract: the same per-block
 * code and decoupled prefix scan as enc_compress_ex; one kernel launch
 * covers every tensor, which matters for a model's many small tensors).
 * Each item's stream is byte-identical to what enc_compress_ex writes for
 * it with the same block size and options. */
typedef struct enc_citem {
  const uint16_t *d_in;  /* device BF16 bit patterns, 16-byte aligned (NULL allowed if n_elems is 0) */
  uint64_t n_elems;      /* values */
  void *d_out;           /* device output, 16-byte aligned */
  uint64_t out_capacity; /* bytes of d_out: at least enc_compress_bound(n_elems) */
} enc_citem;

/* Device workspace bytes for enc_compress_batch over these items: the batch
 * tables, per-item look-back state, and room for enc_compress_ex of the
 * largest item. Returns 0 for an unsupported block size, a negative count or
 * NULL items with count > 0. */
uint64_t enc_compress_batch_workspace_bytes(const enc_citem *h_items, int count,
                                            uint32_t block_size);

/* Compress `count` items: one single-pass launch over all of them, one
 * synchronisation of `stream` to read back their sizes, one launch that
 * writes the coded headers and section padding, a RAW copy launch per item
 * whose coded stream would not be smaller (and for empty items), then a
 * second synchronisation (the host tables live only for the call). Items
 * whose look-back wait gave up are re-encoded with enc_compress_ex. Fills
 * h_infos[k] for each item. Errors: an item's capacity below its RAW size
 * is ENC_ERR_CAPACITY, as is a short workspace; all argument checks run
 * before any launch. A HIP error after the first launch returns
 * ENC_ERR_HIP, and then the items' outputs and h_infos are unspecified.
 * Options as enc_compress_ex. count 0 does nothing. Items must not share
 * output buffers, and the input and output of an item must not overlap. */
enc_status enc_compress_batch(const enc_citem *h_items, int count, uint32_t block_size,
                              uint32_t options, void *d_ws, uint64_t ws_bytes, void *stream,
                              enc_info *h_infos);

/* enc_compress_batch for items of one dtype (1 BF16 -- enc_compress_batch
 * --, 2 FP16, 3 FP32; ENEC Abstract, as enc_compress_dt): each item's d_in
 * holds n_elems values of that dtype and its out_capacity at least
 * enc_compress_bound_dt(n_elems, dtype); the workspace is
 * enc_compress_batch_workspace_bytes of the same items. Each item's stream
 * is byte-identical to what enc_compress_dt writes for it; items whose
 * look-back wait gave up are re-encoded with enc_compress_dt. Unknown dtype:
 * ENC_ERR_UNSUPPORTED. */
enc_status enc_compress_batch_dt(const enc_citem *h_items, int count, uint32_t dtype,
                                 uint32_t block_size, uint32_t options, void *d_ws, uint64_t ws_bytes,
                                 void *stream, enc_info *h_infos);

/* Parse and check a stream header held in host memory (header_bytes >= 256)
 * for a stream of comp_bytes bytes. Checks magic, version, dtype, flags,
 * block size, section offsets against n, and total <= comp_bytes. Host only;
 * launches nothing. */
enc_status enc_parse_header(const void *h_header, uint64_t header_bytes, uint64_t comp_bytes,
                            enc_info *h_info);

/* Copy the 256-byte header of a device stream to the host (synchronous on
 * `stream`) and parse it with enc_parse_header. */
enc_status enc_read_info(const void *d_comp, uint64_t comp_bytes, void *stream, enc_info *h_info);

/* Decompress a whole stream into out_elems values of the stream's dtype
 * (2 bytes each for BF16 and FP16, 4 for FP32; ZipServ Abstract: each
 * block is found in a fixed number of steps and all decode in parallel). One kernel launch; asynchronous;
 * allocates nothing. h_info must describe d_comp (enc_read_info or the
 * enc_info enc_compress returned); out_elems must equal its n_elems. */
enc_status enc_decompress(const void *d_comp, const enc_info *h_info, void *d_out,
                          uint64_t out_elems, void *stream);

/* Batched decompression: many streams, one launch (a model's whole weight
 * set decoded per step, as single-stream inference streams every weight
 * once per token -- MINE Abstract). */
typedef struct enc_item {
  const void *d_comp; /* device stream (any dtype; items may mix them) */
  void *d_out;        /* device output, info.n_elems values of the stream's dtype */
  enc_info info;      /* parsed header of d_comp */
} enc_item;

/* Device bytes of the batch table for these items: descriptors, tile
 * prefixes and a 4-byte item index per decoder tile (about 0.001 byte per
 * value). Reads only info.dtype and info.n_elems of each item. Returns 0
 * for a negative count or NULL items with count > 0. */
uint64_t enc_batch_table_bytes(const enc_item *h_items, int count);

/* Launch sizes of a prepared batch, filled by enc_batch_prepare: the decoder
 * runs one workgroup per tile (4096 values of a BF16 or FP32 stream, 8192
 * of an FP16 one), and the grid size has to be known on the host when the
 * kernel is launched. */
typedef struct enc_batch_plan {
  uint64_t tiles;      /* tiles of the BF16 items */
  uint64_t wide_tiles; /* tiles of the FP16 and FP32 items */
  const void *d_table; /* the table the plan belongs to */
  int32_t count;       /* its item count */
  uint32_t reserved;
} enc_batch_plan;

/* Validate the items, write the batch table into d_table (device, at least
 * enc_batch_table_bytes(h_items, count) bytes) and fill *h_plan.
 * Synchronous: returns after the table has been copied. The table stays
 * valid while the streams and outputs do. */
enc_status enc_batch_prepare(const enc_item *h_items, int count, void *d_table,
                             uint64_t table_bytes, void *stream, enc_batch_plan *h_plan);

/* Decode every item of a prepared table: one kernel launch for the BF16
 * items and one for the FP16 / FP32 items (each only if there are any;
 * inputs past 2^23 tiles take one more launch per 2^23 tiles).
 * Asynchronous. h_plan must be the plan enc_batch_prepare filled for this
 * table and count (else ENC_ERR_INVALID_ARG). */
enc_status enc_decompress_batch(const void *d_table, int count, const enc_batch_plan *h_plan,
                                void *stream);

/* Device workspace bytes for enc_decompress_gemm / enc_gemm_dense: a small
 * area of per-strip arrival counters, then the split-K partial sums (fp32,
 * one slice per K range). Returns 0 for an unsupported block size or a
 * shape those calls reject (M outside 1..4096, N % 512, K % 8, a zero). */
uint64_t enc_gemm_workspace_bytes(uint32_t M, uint32_t K, uint32_t N, uint32_t block_size);

/* Fused decompress-GEMM (ZipServ Abstract: decompress on the fly into the
 * matrix units, no intermediate decompressed weights in HBM):
 *   Y[M,N] (fp32, overwritten) = X[M,K] (BF16 row-major) * W[K,N]
 * where W is the row-major BF16 matrix compressed in d_wcomp (n_elems = K*N).
 * Requirements: K*N == n_elems, N % 512 == 0 and N % block_size == 0,
 * K % 8 == 0, 1 <= M <= 4096, else ENC_ERR_SHAPE / ENC_ERR_UNSUPPORTED. A RAW
 * stream is multiplied directly from its verbatim values. The workspace must
 * be at least enc_gemm_workspace_bytes(M, K, N, block_size) bytes and must be
 * zero-filled before its first use with these two entry points: it starts
 * with per-strip arrival counters, which every call leaves at zero again
 * (the rest is scratch). When the K dimension is split, the fp32 partial
 * slices are added in K order -- by the last workgroup of each strip to
 * finish (M = 1, coded W with B >= 512) or by a second kernel on the same
 * stream -- so the result is deterministic; calls sharing one workspace must
 * not overlap. Accumulation is fp32. Asynchronous; allocates nothing. */
enc_status enc_decompress_gemm(const uint16_t *d_x, uint32_t M, uint32_t K, const void *d_wcomp,
                               const enc_info *h_winfo, uint32_t N, float *d_y, void *d_ws,
                               uint64_t ws_bytes, void *stream);

/* enc_decompress_gemm for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation). Same arguments, requirements and results, without the
 * workspace: it comes from a fixed-size device array inside the library,
 * enc_gemm_noalloc_scratch_bytes() bytes on every device the library runs on,
 * zero-filled at load and held until the process ends. A shape whose
 * workspace (enc_gemm_workspace_bytes) exceeds it returns ENC_ERR_CAPACITY
 * before anything is launched. Calls on one device share the array: calls
 * that overlap in time on one device race. Uses the current device.
 * Asynchronous; allocates nothing. */
uint64_t enc_gemm_noalloc_scratch_bytes(void);
enc_status enc_decompress_gemm_noalloc(const uint16_t *d_x, uint32_t M, uint32_t K,
                                       const void *d_wcomp, const enc_info *h_winfo, uint32_t N,
                                       float *d_y, void *stream);

/* The same GEMM on an uncompressed BF16 W[K,N] (same kernels with the decode
 * stage replaced by plain loads): the baseline the fused path is compared
 * with. Same workspace rules, with block_size 512. */
enc_status enc_gemm_dense(const uint16_t *d_x, uint32_t M, uint32_t K, const uint16_t *d_w,
                          uint32_t N, float *d_y, void *d_ws, uint64_t ws_bytes, void *stream);

/* Fused decompress-GEMM with W in the layout of a linear layer's weight
 * (output features x input features):
 *   Y[M,N] (fp32, overwritten) = X[M,K] (BF16 row-major) * W^T
 * where W is the row-major BF16 matrix [N, K] compressed in d_wcomp
 * (n_elems = N*K), so each block holds consecutive k of one output column and
 * decodes straight into matrix-core operands (ZipServ Abstract: decompression
 * fused into the GEMM, no intermediate decompressed weights). Requirements:
 * N*K == n_elems, N % 64 == 0, K % 32 == 0, K % block_size == 0 for a coded
 * stream, coded stream below 2 GiB, 1 <= M <= 4096; else ENC_ERR_SHAPE /
 * ENC_ERR_UNSUPPORTED. A RAW stream is multiplied from its verbatim values.
 * Workspace: at least enc_gemm_nt_workspace_bytes(M, K, N, block_size) bytes
 * (split-K partial sums; no initialisation needed). A second kernel on the
 * same stream adds the partial slices in K order (deterministic); calls
 * sharing a workspace must not overlap. Accumulation is fp32. Asynchronous;
 * allocates nothing. */
/* (Returns 0 for an unsupported block size or a shape the call rejects: M
 * outside 1..4096, N % 64, K % 32, a zero.) */
uint64_t enc_gemm_nt_workspace_bytes(uint32_t M, uint32_t K, uint32_t N, uint32_t block_size);
enc_status enc_decompress_gemm_nt(const uint16_t *d_x, uint32_t M, uint32_t K, const void *d_wcomp,
                                  const enc_info *h_winfo, uint32_t N, float *d_y, void *d_ws,
                                  uint64_t ws_bytes, void *stream);

/* The same GEMM on an uncompressed BF16 W[N, K] (same kernel, plain loads):
 * the baseline the fused [N, K] path is compared with. Workspace rules as
 * above with block_size 512. */
enc_status enc_gemm_dense_nt(const uint16_t *d_x, uint32_t M, uint32_t K, const uint16_t *d_w,
                             uint32_t N, float *d_y, void *d_ws, uint64_t ws_bytes, void *stream);

/* Deep check of a stream's device data (the header is checked on the host
 * by enc_parse_header / enc_read_info). In this order of precedence:
 *   ENC_CHECK_WIDTH    some block width is above 8 (or, in a flags-2
 *                      stream, not a power of two);
 *   ENC_CHECK_OFFSETS  a stored segment offset differs from the exclusive
 *                      prefix sum of the padded block payload sizes, or
 *                      payload_bytes differs from their total (ENEC
 *                      Abstract: block offsets come from a prefix scan);
 *   ENC_CHECK_EXPONENT some base + code exceeds the exponent field's
 *                      maximum (255; 31 for FP16): the transform subtracts
 *                      the block minimum, so a valid code never does.
 * index = the first failing block (width, exponent) or the first wrong stored
 * offset (offsets; index n_segments stands for payload_bytes). A RAW stream
 * has no device structure and always passes. d_ws: device workspace of at
 * least enc_validate_workspace_bytes() bytes, 16-byte aligned. Synchronous
 * on `stream` (so it cannot be captured in a graph). Returns ENC_OK, or
 * ENC_ERR_BAD_STREAM with *h_check (may be NULL) naming the failure.
 * Decoding never reads outside a stream, valid or not; this check says
 * whether its output is meaningful. */
enum { ENC_CHECK_OK = 0, ENC_CHECK_WIDTH = 1, ENC_CHECK_OFFSETS = 2, ENC_CHECK_EXPONENT = 3 };
typedef struct enc_check {
  uint32_t kind;     /* ENC_CHECK_* */
  uint32_t reserved; /* 0 */
  uint64_t index;    /* first failing block or stored offset */
} enc_check;

uint64_t enc_validate_workspace_bytes(void);
enc_status enc_validate(const void *d_comp, const enc_info *h_info, void *d_ws, uint64_t ws_bytes,
                        void *stream, enc_check *h_check);

/* Measurement helper, not part of the codec: a streaming kernel with the
 * decoder's access shape and no decoding, so a benchmark can state the HBM
 * rate the device reaches for that shape beside the decoder's (the
 * decoder's roofline is memory bandwidth: every stream byte is read once and
 * every output byte written once, as the MINE Abstract describes for
 * single-stream inference). Reads src_bytes from d_src and writes dst_bytes
 * to d_dst (16-byte items, non-temporal stores): workgroup b (of
 * threads_per_workgroup threads: 64, 128 or 256) writes the b-th run of
 * threads_per_workgroup x items_per_thread output items and reads the b-th
 * proportional run of the source; the output holds copies of source items
 * (which ones is unspecified). Sizes: nonzero multiples of 16;
 * items_per_thread 1, 2 or 4; buffers 16-byte aligned, not overlapping.
 * Asynchronous; allocates nothing. Errors: ENC_ERR_INVALID_ARG,
 * ENC_ERR_UNSUPPORTED (sizes past the index arithmetic), ENC_ERR_HIP. */
enc_status enc_stream_probe(const void *d_src, uint64_t src_bytes, void *d_dst, uint64_t dst_bytes,
                            uint32_t items_per_thread, uint32_t threads_per_workgroup, void *stream);

/* Static text for a status code. */
const char *enc_status_string(enc_status s);

/* Thread-local text describing the last failure on this thread ("" if none). */
const char *enc_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ENC_H */
