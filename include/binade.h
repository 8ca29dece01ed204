/*
 * binade.h -- C ABI of libbinade, the Binade hot path on MI355X (gfx950).
 *
 * What it computes (the pages):
 *   "Binade" package page (pypi.org/project/binade), intro: each BF16
 *   weight is stored as a byte of its sign and mantissa bits, unchanged,
 *   plus its exponent's rank among the tensor's exponents ordered by
 *   frequency; the ranks are Rice-coded on disk and rewritten at load into
 *   a 4-bit form that the kernels read directly, with bit-identical outputs.
 *   Same page, "How it works": a single table per tensor, because nearby
 *   weights do not share exponents; format 2 = Rice codes; runtime layout
 *   R4 = 4-bit rank codes with the few large ranks in a side list, produced
 *   by a GPU kernel at load; the matvec, the MoE expert gather and the GEMM
 *   each add their products in one fixed order.
 *
 * Conventions
 *   - Every function returns a binade_status (0 = OK). Nothing aborts or
 *     throws across this ABI.
 *   - The caller owns every buffer. Host functions take host pointers;
 *     device functions take device pointers (e.g. torch tensors' data_ptr())
 *     inside the descriptors and never allocate device memory.
 *   - Device functions check their arguments on the host, enqueue kernels on
 *     the given hipStream_t (NULL = the default stream) and return; results
 *     and the device status word are valid after the stream is synchronised.
 *   - Matrices are row-major [rows = N outputs, cols = K inputs], like a
 *     linear layer's weight. The device paths require cols % 32 == 0 and
 *     16-byte aligned planes, else BINADE_EUNSUPPORTED.
 *   - Row-chunks: each row is cut into chunks of BINADE_CHUNK columns (the
 *     last one of a row may be shorter); chunk c of row i has flat index
 *     i * ceil(cols / BINADE_CHUNK) + c. Format 2 stores one unary-bit anchor
 *     and one escape prefix per row-chunk; R4 reuses the escape prefix.
 *
 * Format 2 (on-disk layout; the pages give no byte layout, so these are this
 * library's readings):
 *   sm      u8[rows*cols]   (sign << 7) | mantissa
 *   unary   u32 words       per weight in row-major order: q = rank >> k zero
 *                           bits, then a one; bit p is bit p%32 of word p/32
 *   rem     u32 words       the k low bits of the rank of weight i at bits
 *                           i*k .. i*k+k-1, least significant first
 *   anchor  u64[chunks+1]   unary bit position of each row-chunk's first
 *                           weight; the last entry = total unary bits
 *   esc_pre u32[chunks+1]   weights with rank >= 15 before each row-chunk;
 *                           the last entry = total
 * R4 (runtime layout):
 *   sm      the same plane as format 2 (shared, never copied)
 *   nib     u8[rows*cols/2] min(rank, 15); in each row the columns go in
 *                           groups of 8; group g owns bytes 4g..4g+3 of the
 *                           row, byte b = col 8g+b (low nibble) | col 8g+4+b
 *                           (high nibble) << 4
 *   lut     u8[16]          exponent of ranks 0..14; lut[15] unused
 *   esc     u32[n_esc]      one entry per weight of rank >= 15, row-major:
 *                           (exponent << 16) | (column - BINADE_CHUNK*chunk)
 *   esc_pre the same array as format 2's
 */
#ifndef BINADE_H
#define BINADE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BINADE_CHUNK 2048

typedef enum binade_status {
  BINADE_OK = 0,
  BINADE_EINVAL = -1,       /* bad argument: null pointer, size, shape */
  BINADE_ECORRUPT = -2,     /* inconsistent planes found on the host */
  BINADE_EUNSUPPORTED = -3, /* shape or alignment the kernels do not take */
  BINADE_EHIP = -4,         /* a HIP runtime call failed */
  BINADE_ENOSPACE = -5      /* an output buffer is smaller than needed */
} binade_status;

/* Output element type of the products. */
typedef enum binade_dtype {
  BINADE_F32 = 0,     /* fp32 as accumulated */
  BINADE_BF16 = 1     /* the fp32 result rounded to bf16, nearest-even */
} binade_dtype;

/* Device status word bits (set with atomic OR by the kernels; the caller
 * clears the word before the call and reads it after synchronising). */
#define BINADE_DEV_CORRUPT_STREAM 0x1u  /* a chunk's unary bits do not hold
                                            its weight count, or a rank is not
                                            in the table */
#define BINADE_DEV_BAD_INDEX 0x2u       /* an expert index is out of range */
#define BINADE_DEV_CORRUPT_ESC 0x4u     /* escape prefix / entries disagree */

/* Per-tensor exponent table. */
typedef struct binade_table {
  uint32_t n;                /* distinct exponents present, 1..256 */
  uint32_t k;                /* Rice parameter for this table, 0..7 */
  uint8_t exp_of_rank[256];  /* exponent of rank r (r < n); 0 beyond n */
  uint16_t rank_of_exp[256]; /* rank of exponent e; 0xFFFF if absent */
  uint64_t count_of_rank[256];
} binade_table;

/* Format 2 descriptor. Pointers are host memory for binade_pack_rice and
 * device memory for binade_rice_to_r4. */
typedef struct binade_rice {
  int64_t rows, cols;
  uint32_t k, n;
  uint8_t exp_of_rank[256];
  uint8_t *sm;
  uint32_t *unary;
  uint64_t unary_bits;
  uint64_t unary_words;   /* words the buffer holds (>= binade_sizes_of's) */
  uint32_t *rem;
  uint64_t rem_words;
  uint64_t *anchor;       /* chunks + 1 */
  uint32_t *esc_pre;      /* chunks + 1 */
  uint64_t n_esc;
} binade_rice;

/* Sizes a caller allocates for format 2 and R4. */
typedef struct binade_sizes {
  uint64_t n_weights;     /* rows * cols */
  uint64_t n_chunks;      /* rows * ceil(cols / BINADE_CHUNK) */
  uint64_t unary_bits;    /* sum over ranks of count * ((r >> k) + 1) */
  uint64_t unary_words;   /* u32 words to allocate (bits rounded up + 2) */
  uint64_t rem_words;     /* u32 words to allocate (rows*cols*k bits + 2) */
  uint64_t n_esc;         /* weights with rank >= 15 */
  uint64_t nib_bytes;     /* rows * cols / 2 */
} binade_sizes;

/* R4 descriptor (device pointers). */
typedef struct binade_r4 {
  int64_t rows, cols;
  uint8_t lut[16];
  const uint8_t *sm;
  uint8_t *nib;
  const uint32_t *esc_pre;
  uint32_t *esc;
  uint64_t n_esc;
} binade_r4;

/* Format 1 descriptor ("Binade" package page, "How it works": a fixed code
 * width per 128-weight tile with escapes). Layout (this library's reading;
 * the pages give none): a tile is 128 consecutive columns of a row, a row's
 * last tile may be shorter. Each tile has a width w in 0..8; for w >= 1 a
 * rank r < 2^w - 1 is the w-bit code r and a larger rank is the escape code
 * 2^w - 1 with the rank appended, as a byte, to the escape list (row-major);
 * w = 0 stores nothing (every rank of the tile is 0). A tile takes the width
 * with the fewest bits, len * w + 8 * escapes, ties to the smaller width.
 *   sm       u8[rows*cols]     as in format 2 (the same plane)
 *   width    u8[tiles]          per tile, row-major (tiles = rows *
 *                               ceil(cols / 128))
 *   codes    u32 words          the tiles' codes in row-major order, code i
 *                               of a tile at bits base + i*w, least
 *                               significant bit first
 *   esc_rank u8[n_f1esc]        ranks of the escaped weights, row-major
 *   anchor   u64[chunks+1]      code bit position of each row-chunk's first
 *                               code; the last entry = total code bits
 *   f1_pre   u32[chunks+1]      format 1 escapes before each row-chunk
 *   esc_pre  u32[chunks+1]      weights of rank >= 15 before each row-chunk
 *                               (R4's escape prefix, as in format 2)
 * Pointers are host memory for binade_pack_f1, device memory for
 * binade_f1_to_r4. */
typedef struct binade_f1 {
  int64_t rows, cols;
  uint32_t n;
  uint8_t exp_of_rank[256];
  uint8_t *sm;
  uint8_t *width;
  uint32_t *codes;
  uint64_t code_bits;
  uint64_t code_words;    /* words the buffer holds */
  uint8_t *esc_rank;
  uint64_t n_f1esc;
  uint64_t esc_cap;       /* entries the esc_rank buffer holds */
  uint64_t *anchor;
  uint32_t *f1_pre;
  uint32_t *esc_pre;
  uint64_t n_esc;         /* weights of rank >= 15 */
} binade_f1;

/* Buffer capacities a caller allocates for format 1 of a rows x cols
 * tensor (widths depend on the data, so codes and escapes are bounded by
 * 8 bits and one escape per weight). */
typedef struct binade_f1_sizes {
  uint64_t n_weights;     /* rows * cols */
  uint64_t n_tiles;       /* rows * ceil(cols / 128) */
  uint64_t n_chunks;      /* rows * ceil(cols / BINADE_CHUNK) */
  uint64_t code_words;    /* u32 words: 8 bits per weight + 2 */
  uint64_t esc_cap;       /* rows * cols */
} binade_f1_sizes;

/* Huffman comparison codec ("Lossless BF16 weight compression" page, intro
 * and "Best measured configuration": the exponent field in canonical Huffman
 * codes, blocks of 64 symbols whose 8-bit byte lengths a prefix sum turns
 * into offsets, sign and mantissa raw). Layout (this library's reading): the
 * symbol is each weight's exponent byte, row-major; code lengths from
 * Huffman's construction (merge the two nodes of least (count, id), leaves
 * id = exponent, merged nodes 256, 257, ... in order; one present exponent
 * gets length 1; lengths <= 31); canonical codes in (length, exponent)
 * order; each block of BINADE_HUFF_BLOCK symbols MSB-first, padded to a
 * byte.
 *   sm         u8[n]                 as in format 2
 *   stream     u8[stream_cap]        the blocks' codes (stream 4-byte
 *                                    aligned for the decoder, stream_cap >=
 *                                    stream_bytes + 8)
 *   block_len  u8[ceil(n/64)]        bytes of each block
 *   group_off  u64[ceil(n/8192)+1]   byte offset of every 128th block; the
 *                                    last entry = stream_bytes
 * Pointers are host memory for binade_huff_pack, device memory for
 * binade_huff_decode. */
#define BINADE_HUFF_BLOCK 64
#define BINADE_HUFF_GROUP 128
typedef struct binade_huff {
  int64_t n;
  uint8_t len[256];
  uint8_t *sm;
  uint8_t *stream;
  uint64_t stream_bytes;
  uint64_t stream_cap;
  uint8_t *block_len;
  uint64_t *group_off;
} binade_huff;

/* Text for a status code (static storage). */
const char *binade_status_str(int32_t status);
/* The last HIP error code seen by a device call on this thread (0 if none). */
int32_t binade_last_hip_error(void);

/* ---------------------------------------------------------------- host */

/* Histogram of the exponent field of n bf16 values (host), ranks ordered by
 * count descending and exponent ascending on ties, and the Rice k with the
 * fewest bits (ties to the smaller k). "Binade" package page, intro and
 * "How it works" (one frequency-rank table per tensor).
 * EINVAL: w or out null, n <= 0. */
int32_t binade_build_table(const uint16_t *w, int64_t n, binade_table *out);

/* Buffer sizes for a rows x cols tensor under table t (host, closed form).
 * EINVAL: null pointers, rows/cols <= 0, table n or k out of range. */
int32_t binade_sizes_of(const binade_table *t, int64_t rows, int64_t cols,
                        binade_sizes *out);

/* Format 2 pack of the bf16 matrix w [rows, cols] (host). out->sm, unary,
 * rem (if t->k > 0), anchor and esc_pre point at caller buffers of at least
 * binade_sizes_of() entries, with out->unary_words / rem_words giving their
 * capacity; fills the scalar fields. Byte-identical to the oracle's pack.
 * "Binade" package page, intro and "How it works" (format 2 = Rice codes).
 * EINVAL: bad pointers or shape, or a weight whose exponent is not in t.
 * ENOSPACE: a plane's capacity is too small. */
int32_t binade_pack_rice(const uint16_t *w, int64_t rows, int64_t cols,
                         const binade_table *t, binade_rice *out);

/* Capacities for format 1 of a rows x cols tensor (host). EINVAL: null out
 * or rows/cols <= 0. */
int32_t binade_f1_sizes_of(int64_t rows, int64_t cols, binade_f1_sizes *out);

/* Format 1 pack of the bf16 matrix w [rows, cols] (host) under table t.
 * out->sm, width, codes, esc_rank, anchor, f1_pre and esc_pre point at
 * caller buffers of binade_f1_sizes_of() entries; out->code_words and
 * out->esc_cap give the codes' and escapes' capacities. Fills the scalar
 * fields; byte-identical to the oracle's pack. "Binade" package page, "How
 * it works" (format 1). EINVAL: bad pointers or shape, or a weight whose
 * exponent is not in t. ENOSPACE: a capacity is too small. */
int32_t binade_pack_f1(const uint16_t *w, int64_t rows, int64_t cols,
                       const binade_table *t, binade_f1 *out);

/* Huffman code lengths of the exponents of w[n] (host) and the stream
 * capacity a pack needs (its code bytes plus one byte per block and 8 bytes
 * of look-ahead). EUNSUPPORTED: a code longer than 31 bits. */
int32_t binade_huff_lengths(const uint16_t *w, int64_t n, uint8_t len[256],
                            uint64_t *stream_cap);

/* Huffman pack of w[out->n] (host) with the lengths in out->len; fills
 * sm, stream (zero padded to stream_cap), block_len, group_off and
 * stream_bytes; byte-identical to the oracle's pack. EINVAL: an exponent
 * with no code, bad pointers. ENOSPACE: stream_cap too small. */
int32_t binade_huff_pack(const uint16_t *w, binade_huff *out);

/* -------------------------------------------------------------- device */

/* The exponent table on the GPU: the same table binade_build_table makes
 * ("Binade" package page, intro and "How it works": one table per tensor,
 * exponents ranked by frequency; ties to the smaller exponent; the Rice k
 * with the fewest bits, ties to the smaller k). w: device bf16[n], 16-byte
 * aligned. workspace: device, >= 2048 bytes, 8-byte aligned (the histogram;
 * cleared by the call). table: device binade_table, written by the call.
 * Calls on one stream that share a workspace are ordered; calls that overlap
 * on different streams need their own. */
int32_t binade_build_table_gpu(const uint16_t *w, int64_t n, void *workspace,
                               binade_table *table, void *stream);

/* Workspace bytes binade_pack_rice_gpu needs for a rows x cols tensor
 * (8 per row-chunk and 12 per 1024 chunks; at least the table's 2048). */
int64_t binade_pack_gpu_workspace_bytes(int64_t rows, int64_t cols);

/* Format 2 pack on the GPU: the same planes, byte for byte, as
 * binade_pack_rice (padding words included). w: device bf16 [rows, cols],
 * cols % 32 == 0. t: the tensor's table in HOST memory (binade_build_table,
 * or binade_build_table_gpu copied back). out: device planes with host
 * capacities as for binade_pack_rice; the scalar fields are filled from the
 * table. dev_status (device u32 or NULL) gets BINADE_DEV_CORRUPT_STREAM when
 * a weight's exponent is not in t or the bits disagree with t's counts (the
 * planes are then unspecified; no write leaves the buffers).
 * EUNSUPPORTED: cols % 32 != 0, misaligned pointers. ENOSPACE: capacities. */
int32_t binade_pack_rice_gpu(const uint16_t *w, int64_t rows, int64_t cols,
                             const binade_table *t, binade_rice *out,
                             void *workspace, uint32_t *dev_status,
                             void *stream);


/* Format 2 -> R4 on the GPU ("Binade" package page, "How it works": a GPU
 * kernel turns the file format into R4 at load). in: device planes of a
 * format 2 tensor (all of in's fields filled as binade_pack_rice leaves
 * them, unary/rem buffers at least binade_sizes_of() words). out: rows, cols
 * are set from in; out->sm and out->esc_pre are set to in->sm and
 * in->esc_pre; lut is filled; the kernel writes out->nib (nib_bytes) and
 * out->esc (n_esc entries), which the caller allocates. dev_status: device
 * u32 or NULL; the kernel ORs BINADE_DEV_CORRUPT_* into it when a chunk's
 * bits are inconsistent (its outputs are then unspecified).
 * EUNSUPPORTED: cols % 32 != 0 or misaligned planes. */
int32_t binade_rice_to_r4(const binade_rice *in, binade_r4 *out,
                          uint32_t *dev_status, void *stream);

/* Format 2 -> R4 for count tensors, up to 16 per launch (a model's load-time
 * decode): in[i] and out[i] as for binade_rice_to_r4; the same kernel and
 * results. The argument checks of every tensor run before its launch. */
int32_t binade_rice_to_r4_batch(const binade_rice *in, binade_r4 *out,
                                int32_t count, uint32_t *dev_status,
                                void *stream);

/* Format 2 -> R4 for a whole model in one launch ("Binade" package page,
 * "How it works": at load a GPU kernel turns the file format into R4). A
 * plan is written once on the host, copied to device memory by the caller
 * and run any number of times; each run decodes every tensor of the plan in
 * a single launch, with the results of binade_rice_to_r4 bit for bit.
 *
 * binade_rice_plan_bytes: bytes a plan of count tensors may take (count in
 * 0 .. 65536; BINADE_EINVAL otherwise).
 *
 * binade_rice_to_r4_plan: checks in[i] and fills out[i]'s host-visible
 * fields exactly as binade_rice_to_r4_batch does, and writes the plan into
 * HOST memory plan (plan_bytes >= binade_rice_plan_bytes(count), else
 * BINADE_EINVAL). The plan records the device addresses of in[i]'s planes
 * and of out[i].nib / out[i].esc: those buffers must stay allocated while
 * the plan is used. Every tensor must take the streamed decoder: Rice
 * k = 1, a table of at least 15 ranks, at least 1024 columns, a last
 * row-chunk of 0 or at least 128 columns and fewer than 2^31 weights
 * (together fewer than 2^31 spans of 32768 weights); otherwise
 * BINADE_EUNSUPPORTED and the plan is not usable (binade_rice_to_r4_batch
 * takes any tensor).
 *
 * binade_rice_to_r4_run: host_plan is the plan as written (its header is
 * read); dev_plan is a byte-for-byte copy of it in device memory, 8-byte
 * aligned, which the launch reads (the caller owns it and keeps it until
 * the launch has run). dev_status: device u32 or NULL, as for
 * binade_rice_to_r4. BINADE_EINVAL for a header that is not a plan's. */
int64_t binade_rice_plan_bytes(int32_t count);
int32_t binade_rice_to_r4_plan(const binade_rice *in, binade_r4 *out,
                               int32_t count, void *plan, int64_t plan_bytes);
int32_t binade_rice_to_r4_run(const void *host_plan, const void *dev_plan,
                              uint32_t *dev_status, void *stream);

/* Format 1 -> R4 on the GPU ("Binade" package page, "How it works": at load
 * a GPU kernel turns either file format into R4). in: device planes of a
 * format 1 tensor as binade_pack_f1 leaves them (code_words and esc_cap the
 * buffers' entries). out: as for binade_rice_to_r4 (rows, cols, sm, esc_pre
 * set from in; lut filled; the kernel writes out->nib and out->esc, which
 * the caller allocates). dev_status: device u32 or NULL; the kernel ORs
 * BINADE_DEV_CORRUPT_* into it when a chunk's planes are inconsistent (its
 * outputs are then unspecified). EUNSUPPORTED: cols % 32 != 0 or misaligned
 * planes. The R4 result equals binade_rice_to_r4's on the same weights. */
int32_t binade_f1_to_r4(const binade_f1 *in, binade_r4 *out,
                        uint32_t *dev_status, void *stream);

/* Workspace bytes binade_huff_decode needs (its decode tables). */
int64_t binade_huff_workspace_bytes(void);

/* Huffman stream -> bf16 weights on the GPU: the comparison decoder of the
 * "Lossless BF16 weight compression" page ("Best measured configuration":
 * one thread per block of 64 symbols, offsets from a prefix sum over the
 * 8-bit block lengths of 128 blocks, a lookup table for the codes). in:
 * device planes as binade_huff_pack leaves them. out: device bf16[n],
 * 16-byte aligned. workspace: device, binade_huff_workspace_bytes(), 16-byte
 * aligned (rebuilt by each call; calls overlapping on different streams need
 * their own). dev_status: BINADE_DEV_CORRUPT_STREAM when a block's codes,
 * padding or a group offset disagree with the index (outputs then
 * unspecified). */
int32_t binade_huff_decode(const binade_huff *in, uint16_t *out,
                           void *workspace, uint32_t *dev_status,
                           void *stream);

/* R4 -> bf16 bits [rows, cols] on the GPU (the rebuild path; "Binade"
 * package page, "Use": unpack restores the original BF16 bit for bit). */
int32_t binade_unpack(const binade_r4 *w, uint16_t *out, void *stream);

/* Batch-1 product y[N] = W[N,K] x[K] with W in R4, every weight rebuilt in
 * registers ("Binade" package page, "Results" and "How it works": the R4
 * matvec). x: device bf16[K]. y: device fp32[N] or bf16[N] per y_dtype.
 * Summation order (fixed, independent of launch shape): K is cut into tiles
 * of 32; tile j goes to slot j mod 64; each slot keeps fp32 sums a0 (even
 * columns) and a1 (odd columns) from +0.0, fused multiply-adding its tiles
 * in increasing j and columns in increasing order; slot value a0 + a1; then
 * p[l] += p[l+s] for s = 32, 16, 8, 4, 2, 1; y = p[0]. */
int32_t binade_r4_gemv(const binade_r4 *w, const uint16_t *x, void *y,
                       int32_t y_dtype, void *stream);

/* count independent products y_i = W_i x_i (ws[i], xs[i], ys[i] as for
 * binade_r4_gemv), up to 16 per launch: the products a decode step issues
 * together, such as one layer's q, k and v projections or its gate and up
 * projections. Every y_i is bit-identical to binade_r4_gemv's. */
int32_t binade_r4_gemv_batch(const binade_r4 *ws, const uint16_t *const *xs,
                             void *const *ys, int32_t count, int32_t y_dtype,
                             void *stream);

/* The batched twin: count products y_i = W_i x_i with plain bf16 W_i
 * [rows[i], cols[i]] (device), up to 16 per launch, in the same order. */
int32_t binade_bf16_gemv_batch(const uint16_t *const *ws, const int64_t *rows,
                               const int64_t *cols, const uint16_t *const *xs,
                               void *const *ys, int32_t count, int32_t y_dtype,
                               void *stream);

/* The same product and order with W given as plain bf16 [N, K] (device):
 * the exactness twin and the speed reference. */
int32_t binade_bf16_gemv(const uint16_t *w, int64_t rows, int64_t cols,
                         const uint16_t *x, void *y, int32_t y_dtype,
                         void *stream);

/* The decode step of 2..8 sequences: Y[b, :] = W x_b for b < m, m in 1..8
 * ("Binade" package page, "Limitations": the fused kernels cover small dense
 * products; "Results": the per-token matvec). Each row of Y is bit-identical
 * to binade_r4_gemv of that row of X (the same order per output), and W is
 * read once for all m rows. x: device bf16, row b at x + b*ldx (ldx >= K, a
 * multiple of 8, x 16-byte aligned). y: device fp32 or bf16 per y_dtype,
 * row b at y + b*ldy (ldy >= N). EINVAL: m outside 1..8, bad strides or
 * pointers. */
int32_t binade_r4_gemv_rows(const binade_r4 *w, const uint16_t *x, int64_t ldx,
                            int32_t m, void *y, int64_t ldy, int32_t y_dtype,
                            void *stream);

/* The same with plain bf16 W [rows, cols] (device): the twin. */
int32_t binade_bf16_gemv_rows(const uint16_t *w, int64_t rows, int64_t cols,
                              const uint16_t *x, int64_t ldx, int32_t m,
                              void *y, int64_t ldy, int32_t y_dtype,
                              void *stream);

/* Prompt GEMM Y[M,N] = X[M,K] W[N,K]^T with W in R4, tiles decoded into LDS
 * and multiplied on bf16 MFMA with fp32 accumulation ("Binade" package page,
 * "Results" and "Limitations": prompt processing with fused GEMM). X: device
 * bf16 with row stride ldx (elements, a multiple of 8); Y: fp32 or bf16 with
 * row stride ldy. K must be a multiple of 32.
 * Order (depends on K only, never on M, the workspace or the launch shape):
 * K is cut into nsb = K/128 super-blocks of 128 columns, then (K%128)/32
 * tail blocks of 32. Super-block u is four v_mfma_f32_16x16x32_bf16 steps;
 * in step j, lanes 16g..16g+15 carry columns 128u + 32g + 8j .. +7. A tail
 * block is one step with columns 8g .. 8g+7 of the block. The super-blocks
 * form S = min(8, ceil(K/1024)) slices, slice s = [s*nsb/S, (s+1)*nsb/S),
 * the last one also taking the tail blocks. Per output and slice one fp32
 * accumulator from +0.0 takes the slice's steps in order; the output adds
 * the slices' accumulators in slice order.
 * workspace: optional device memory (16-byte aligned, caller-owned, not
 * read before written) of workspace_bytes; with at least
 * binade_gemm_workspace_bytes(M, N, K) bytes the slices of a shape with few
 * tiles run in separate blocks, otherwise in one. NULL/0 is always valid.
 * Calls that share a workspace must not overlap. */
int32_t binade_r4_gemm(const binade_r4 *w, const uint16_t *x, int64_t m,
                       int64_t ldx, void *y, int64_t ldy, int32_t y_dtype,
                       void *workspace, int64_t workspace_bytes, void *stream);

/* The same GEMM with plain bf16 W [N, K] (device). */
int32_t binade_bf16_gemm(const uint16_t *w, int64_t rows, int64_t cols,
                         const uint16_t *x, int64_t m, int64_t ldx, void *y,
                         int64_t ldy, int32_t y_dtype, void *workspace,
                         int64_t workspace_bytes, void *stream);

/* binade_r4_gemm without a workspace argument and without allocating, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc). The split slices'
 * partial sums go to a fixed scratch array inside the library, one per
 * device, of binade_gemm_scratch_bytes() bytes (32 MiB), held until the
 * process ends. Same arguments, results and order as binade_r4_gemm (the
 * same bits whether or not it splits). Returns BINADE_ENOSPACE, launching
 * nothing, when the shape's partial sums (binade_gemm_workspace_bytes)
 * exceed the scratch. Calls are stream-ordered but share the device's
 * scratch: calls that overlap on one device (different streams or host
 * threads) race and must not be issued. Nothing in the scratch is read before
 * the same call writes it. */
int32_t binade_r4_gemm_noalloc(const binade_r4 *w, const uint16_t *x,
                               int64_t m, int64_t ldx, void *y, int64_t ldy,
                               int32_t y_dtype, void *stream);

/* Size in bytes of binade_r4_gemm_noalloc's per-device scratch. */
int64_t binade_gemm_scratch_bytes(void);

/* Workspace bytes with which binade_r4_gemm / binade_bf16_gemm split the
 * slices of an M x N x K product over blocks (0: that shape never splits;
 * also 0 for invalid sizes). Pure host function. */
int64_t binade_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k);

/* MoE expert-gather GEMV ("Binade" package page, "How it works": the MoE
 * expert gather in the matvec's order; "Limitations": fused kernels cover
 * every expert product). experts: R4 stack of n_experts matrices [N, K]
 * stored as one [n_experts*N, K] tensor with one table. idx: device
 * int32[n_tokens*top_k]. x: device bf16 [n_tokens, K] (x_per_slot = 0) or
 * [n_tokens*top_k, K] (x_per_slot = 1). y: [n_tokens*top_k, N], row p =
 * expert idx[p] times its input, in the binade_r4_gemv order. Experts no
 * pair chose are not read; a wave that serves several pairs of one expert
 * re-reads its rows from cache. An index outside
 * [0, n_experts) sets BINADE_DEV_BAD_INDEX in dev_status (if not NULL) and
 * leaves that output row as zeros. */
int32_t binade_r4_moe_gemv(const binade_r4 *experts, int32_t n_experts,
                           const uint16_t *x, int32_t x_per_slot,
                           const int32_t *idx, int64_t n_tokens,
                           int32_t top_k, void *y, int32_t y_dtype,
                           uint32_t *dev_status, void *stream);

/* The same gather with plain bf16 experts [n_experts*N, K] (device). */
int32_t binade_bf16_moe_gemv(const uint16_t *experts, int32_t n_experts,
                             int64_t rows_per_expert, int64_t cols,
                             const uint16_t *x, int32_t x_per_slot,
                             const int32_t *idx, int64_t n_tokens,
                             int32_t top_k, void *y, int32_t y_dtype,
                             uint32_t *dev_status, void *stream);

/* MoE epilogue, gate.up activation ("Binade" package page, "How it works"
 * and "Limitations": the expert products of a MoE layer, whose gate and up
 * outputs meet in an activation before the down product). h[i] = silu(g[i])
 * * u[i] for i < n, silu(g) = g / (1 + exp(-g)), evaluated in fp64 from the
 * fp32 inputs and rounded once to fp32 (then to bf16, nearest-even, when
 * h_dtype is BF16). gate, up: device fp32[n]; h: device fp32 or bf16 [n].
 * g = -inf gives NaN, as the formula does. */
int32_t binade_moe_silu_mul(const float *gate, const float *up, int64_t n,
                            void *h, int32_t h_dtype, void *stream);

/* MoE epilogue, top-k weighted combine. y: device fp32 [n_tokens*top_k, N]
 * (the down product per (token, slot) pair, as binade_r4_moe_gemv writes
 * it); weights: device fp32 [n_tokens*top_k]. out[t, j] = acc after
 * acc = +0.0; acc = fma(weights[t*top_k + s], y[t*top_k + s, j], acc) for
 * s = 0 .. top_k-1, in fp32 (then bf16, nearest-even, when out_dtype is
 * BF16). out: device [n_tokens, N]. EINVAL: top_k outside 1..64, sizes. */
int32_t binade_moe_combine(const float *y, const float *weights,
                           int64_t n_tokens, int32_t top_k, int64_t n,
                           void *out, int32_t out_dtype, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* BINADE_H */
