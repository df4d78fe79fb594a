/*
 * q8moe.h -- C ABI of the MI355X (gfx950) Q8_0 decode library (libq8moe.so).
 *
 * The operations are the hot path of token-by-token LLM decode with Q8_0
 * weights: activation quantization, the Q8_0 x Q8_0 matrix-vector product, its
 * small-batch and prefill forms, and the mixture-of-experts expert FFN
 * (mul_mat_id over a combined up_gate tensor, SwiGLU, down projection and the
 * weighted combine over a token's active experts).
 *
 * Sources (web pages, cited by title and section):
 *  [XEON]  "GPUなしで13年前のXeon上でGemma 4 26Bを毎秒5トークンで実行する"
 *          (Gemma 4 26B-A4B Q8_0 on a 2013 dual Xeon, ja.news.hada.io).
 *  [NARR]  "narray-llm" README (Llama 2 110M int8 (Q8_0) table; kernels per
 *          token table).
 *
 * ---------------------------------------------------------------------------
 * Data format.  A Q8_0 block holds 32 values: an IEEE binary16 scale d
 * (little-endian, first) followed by 32 signed 8-bit codes q[j]; value j is
 * d*q[j].  A block is 34 bytes with 2-byte alignment.  A row of k values is
 * k/32 blocks back to back; a matrix [n][k] is n such rows back to back.  This
 * is the plain reading of the format the pages name but do not print
 * ([XEON] summary and the section on the broken op paths; [NARR] Llama 2 110M
 * int8 table).
 *
 * Quantization rule (per 32-block, fp32): d = max|x| / 127 (IEEE division),
 * q = round(x / d) with ties away from zero (codes saturate at +-127, which is
 * reachable only when d is an fp32 subnormal), d stored rounded to nearest-even
 * binary16; an all-zero block stores d = +0 and zero codes.
 *
 * Block dot product: s = sum_j qw[j]*qx[j] is exact in int32; the fp32 result
 * is sum_b (f32(dw_b) * f32(dx_b)) * s_b (the product of the two scales is
 * exact in fp32).  The order of the fp32 sum over blocks is fixed per launch
 * shape (results are deterministic run to run) but is not the sequential
 * order; results agree with the exact sum within a few fp32 ulps.
 *
 * ---------------------------------------------------------------------------
 * Conventions for every entry point.
 *  - Pointers are DEVICE pointers owned by the caller (the library never
 *    allocates, frees or synchronizes).  Matrices of blocks must start on a
 *    16-byte boundary; fp32 arrays on a 4-byte boundary, and the fp32 input of
 *    q8_0_quantize_rows on a 16-byte boundary with a row stride that is a
 *    multiple of 4 floats.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work
 *    is enqueued asynchronously on it and ordered with everything else on it.
 *  - Return value: Q8_OK (0), or a negative q8_status.  On a negative status
 *    nothing has been enqueued and no output has been touched.  Arguments are
 *    checked on the host before any HIP call, so argument errors are reported
 *    the same way with or without a GPU.
 *  - Outputs are always fully overwritten, never accumulated into.  No
 *    operation is skipped silently: an unsupported shape is an error.
 *  - Sizes are int64_t; k, n_embd and n_ff must be multiples of 32.
 *  - Calls are reentrant; two calls that write the same output or the same
 *    workspace race unless they are ordered on one stream.
 */
#ifndef Q8MOE_H
#define Q8MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* One Q8_0 block: 34 bytes, 2-byte aligned (no padding). */
typedef struct q8_0_block {
    uint16_t d;       /* binary16 bits of the scale */
    int8_t qs[32];    /* codes */
} q8_0_block;

typedef enum q8_status {
    Q8_OK = 0,
    Q8_E_NULL = -1,         /* a required pointer is NULL */
    Q8_E_SHAPE = -2,        /* a size is <= 0 (or < 0 where 0 is allowed), or not a multiple of 32 */
    Q8_E_ALIGN = -3,        /* a pointer or stride breaks the alignment rules above */
    Q8_E_UNSUPPORTED = -4,  /* valid but outside what this build supports (stated per call) */
    Q8_E_WORKSPACE = -5,    /* workspace missing or smaller than the ..._workspace_bytes() value */
    Q8_E_HIP = -6           /* the HIP runtime reported an error when enqueuing */
} q8_status;

/* Human-readable name of a status; never NULL. */
const char *q8_status_str(int status);

/* Library version string. */
const char *q8_version(void);

/* ---------------------------------------------------------------------------
 * q8_0_quantize_rows -- activation quantization (the role of
 * quantize_row_q8_0 / quantize_row_q8_0_x4, [XEON] three-part fix, compile-fix
 * part).
 *   x      fp32 [n_rows][x_row_stride], the first k values of each row are used
 *   y      Q8_0 [n_rows][k/32] blocks, written
 * n_rows >= 0 (0 is a no-op), k > 0 and k % 32 == 0, x_row_stride >= k.
 * The bytes written are identical to the quantization rule above, bit for bit.
 */
int q8_0_quantize_rows(const float *x, int64_t x_row_stride, q8_0_block *y,
                       int64_t n_rows, int64_t k, void *stream);

/* ---------------------------------------------------------------------------
 * q8_0_matvec -- y[n] = W[n][k] . x[k]: the batch-1 decode product (the Q8_0
 * mul_mat whose plain fallback worked on the old Xeon, [XEON] section on the
 * broken op paths; the block dot of ggml_vec_dot_q8_0_q8_0, [XEON] section on
 * narrowing down the cause).
 *   w  Q8_0 [n][k/32] (16-byte aligned), x  Q8_0 [k/32], y  fp32 [n] (written)
 * n >= 0, k > 0, k % 32 == 0.
 */
int q8_0_matvec(const q8_0_block *w, const q8_0_block *x, float *y,
                int64_t n, int64_t k, void *stream);

/* ---------------------------------------------------------------------------
 * q8_0_matmul -- Y[m][n] = X[m][k] . W[n][k]^T for m token rows: batched decode
 * (small m, weights streamed once for all rows: the batch-of-8 decode of the
 * [NARR] GPT-2 124M table) and prefill (large m, int8 matrix cores: prompt
 * evaluation, which [XEON] reports apart from decode in its summary, and
 * which a matrix library speeds up where sequential decode gains little: the
 * ARM page, section on build optimisation, OpenBLAS offload).  Same
 * arithmetic as q8_0_matvec for every (m, n): the block dot of
 * ggml_vec_dot_q8_0_q8_0 ([XEON] section on narrowing down the cause).
 *   w  Q8_0 [n][k/32], x  Q8_0 [m][k/32], y  fp32 [m][n] (written)
 * m >= 0, n >= 0, k > 0, k % 32 == 0.
 */
int q8_0_matmul(const q8_0_block *w, const q8_0_block *x, float *y,
                int64_t n, int64_t k, int64_t m, void *stream);

/* ---------------------------------------------------------------------------
 * Row-interleaved weights (R8).  The [XEON] section on the fallback's cost and
 * the repacking bug describes a startup option that reorders quantized weights
 * into an interleaved form, Q8_0_R8; the page gives no byte layout.  This
 * library's layout (same bytes as the native rows, moved once at load time):
 * rows in groups of 8, the last group padded with zero rows; group g takes
 * 272*(k/32) bytes at g*272*(k/32):
 *   bytes [0, 16*(k/32))     the binary16 scales, little-endian, the one of
 *                            row 8g+r at block b at index 8*b + r
 *   then the codes           the 32 codes of row 8g+r at block b at byte
 *                            16*(k/32) + 32*(8*b + r)
 *
 * q8_0_r8_bytes -- the size of that layout for n rows of k values (a negative
 * status for a bad shape).
 *
 * q8_0_repack_r8 -- writes the layout of native rows w (Q8_0 [n][k/32]) to
 * w_r8 (q8_0_r8_bytes(n, k) bytes, 16-byte aligned, written in full,
 * padding included).  w and w_r8 must not overlap.
 *
 * q8_0_matvec_r8 -- y[n] = W[n][k] . x[k] with W in the R8 layout: the
 * arithmetic of q8_0_matvec (exact int32 block sums, (d_w*d_x)*s in fp32).
 *   w_r8 (16-byte aligned), x  Q8_0 [k/32], y  fp32 [n] (written)
 * n >= 0, k > 0, k % 32 == 0, k <= 32768 (Q8_E_UNSUPPORTED above).
 */
int64_t q8_0_r8_bytes(int64_t n, int64_t k);
int q8_0_repack_r8(const q8_0_block *w, void *w_r8, int64_t n, int64_t k, void *stream);
int q8_0_matvec_r8(const void *w_r8, const q8_0_block *x, float *y, int64_t n, int64_t k,
                   void *stream);

/* q8_0_matvec_r8_batched -- several R8 products in one launch (a decode step's
 * matrices).  Descriptor i computes, for every b < batch:
 *   y + b*y_batch_stride  =  W_b . (x + b*x_batch_stride)
 * with W_b the R8 layout at w_r8 + b*w_batch_stride BYTES (a multiple of 16,
 * at least q8_0_r8_bytes(n, k) when batch > 1), x_batch_stride in blocks,
 * y_batch_stride in floats (>= n when batch > 1).  Same limits as
 * q8_0_matvec_r8 per descriptor; n_desc <= 32.  descs is a HOST array.
 */
typedef struct q8_0_r8_desc {
    const void *w_r8;
    const q8_0_block *x;
    float *y;
    int64_t n, k, batch;
    int64_t w_batch_stride;   /* bytes */
    int64_t x_batch_stride;   /* blocks */
    int64_t y_batch_stride;   /* floats */
} q8_0_r8_desc;

int q8_0_matvec_r8_batched(const q8_0_r8_desc *descs, int64_t n_desc, void *stream);

/* q8_0_matvec_r8_f32_batched -- the same products from fp32 activation rows:
 * every row is quantized inside the launch by the rule above (the bytes of
 * q8_0_quantize_rows), so a decode step is one launch.  x + b*x_batch_stride
 * (floats; x 16-byte aligned, x_batch_stride a multiple of 4) is the fp32 row
 * of matrix b.  Results are bitwise those of q8_0_quantize_rows followed by
 * q8_0_matvec_r8_batched.  Same limits otherwise.
 */
typedef struct q8_0_r8_f32_desc {
    const void *w_r8;
    const float *x;
    float *y;
    int64_t n, k, batch;
    int64_t w_batch_stride;   /* bytes */
    int64_t x_batch_stride;   /* floats */
    int64_t y_batch_stride;   /* floats */
} q8_0_r8_f32_desc;

int q8_0_matvec_r8_f32_batched(const q8_0_r8_f32_desc *descs, int64_t n_desc, void *stream);

/* q8_0_matmul_r8_batched -- batched small-batch decode over R8 weights (the
 * products of a decode step at 1..16 token rows, on the int8 matrix cores).
 * Descriptor i computes, for every b < batch and token row t < m:
 *   y_b[t][0..n) = W_b . X_b[t]
 * with W_b the R8 layout at w_r8 + b*w_batch_stride BYTES (a multiple of 16,
 * >= q8_0_r8_bytes(n, k) when batch > 1), X_b[t] = x + b*x_batch_stride +
 * t*x_row_stride (Q8_0 blocks; x_row_stride >= k/32 when m > 1), y_b[t] = y +
 * b*y_batch_stride + t*y_row_stride (floats; y_row_stride >= n when m > 1,
 * y_batch_stride >= n when batch > 1).  Arithmetic of q8_0_matmul (exact int32
 * block sums, (d_w*d_x)*s in fp32).  m <= 16 (Q8_E_UNSUPPORTED above, and when
 * 36*m'*k/32 bytes of staged activations exceed the workgroup's LDS, m' = 8
 * for m <= 8 else 16); n_desc <= 32.  descs is a HOST array.
 */
typedef struct q8_0_r8_mm_desc {
    const void *w_r8;
    const q8_0_block *x;
    float *y;
    int64_t n, k, m, batch;
    int64_t w_batch_stride;   /* bytes */
    int64_t x_row_stride;     /* blocks */
    int64_t x_batch_stride;   /* blocks */
    int64_t y_row_stride;     /* floats */
    int64_t y_batch_stride;   /* floats */
} q8_0_r8_mm_desc;

int q8_0_matmul_r8_batched(const q8_0_r8_mm_desc *descs, int64_t n_desc, void *stream);

/* ---------------------------------------------------------------------------
 * Q8_1 activations and 4/5-bit K-quant weights.  [XEON] (three-part fix,
 * compile fix) names a Q8_1 activation quantizer beside the Q8_0 one; the
 * other pages serve Q4_K_M / Q5_K_M model files ([NEMO] closing section; the
 * ARM page's server commands).  No page prints a layout; this library reads:
 *   Q8_1 block, 36 bytes: binary16 d, binary16 s, 32 int8 codes.  d and the
 *     codes follow the Q8_0 rule; s = binary16(d32 * sum of the codes), d32 =
 *     amax/127 unrounded, the product in fp32.
 *   Super-block of 256 values, 8 sub-blocks of 32:
 *     Q4_K (type 4), 144 bytes: binary16 d, binary16 dmin, 12 bytes of 6-bit
 *       sub-block scales sc[8] and mins m[8] (j < 4: sc = byte j & 63,
 *       m = byte j+4 & 63; j >= 4: low 4 bits from the low / high nibble of
 *       byte j+4, top 2 bits from the top bits of byte j-4 / byte j), then
 *       128 bytes of 4-bit codes (byte 32c+l: low nibble = value l of
 *       sub-block 2c, high nibble = value l of sub-block 2c+1);
 *     Q5_K (type 5), 176 bytes: the same 16-byte header, 32 bytes of high bits
 *       (bit j of byte l adds 16 to value l of sub-block j), then the 128
 *       bytes of low 4-bit codes.
 *   Value l of sub-block j = d * sc[j] * q - dmin * m[j].
 *
 * q8_1_quantize_rows -- fp32 rows (16-byte aligned, row stride a multiple of
 * 4 floats, >= k) -> Q8_1 [n_rows][k/32] blocks (4-byte aligned).
 *
 * kq_matvec_batched -- y + b*y_batch_stride = W_b . x_b for every descriptor
 * and b < batch: W_b = w + b*w_batch_stride SUPER-BLOCKS of K-quant `type`
 * ([n][k/256], 16-byte aligned), x_b = x + b*x_batch_stride Q8_1 blocks (one
 * row of k/32), y fp32 [n] (written); per sub-block the exact int32 sums of
 * code products and of activation codes, then (d*sc*d_x)*S - (dmin*m*d_x)*Q
 * in fp32 (s of the Q8_1 blocks is not read).  k % 256 == 0, k <= 8192
 * (Q8_E_UNSUPPORTED above, and for a type other than 4 or 5); n_desc <= 32;
 * with batch > 1 the strides must separate matrices and outputs (Q8_E_SHAPE).
 * q4_k_matvec / q5_k_matvec -- one product.
 */
int q8_1_quantize_rows(const float *x, int64_t x_row_stride, void *y, int64_t n_rows,
                       int64_t k, void *stream);

typedef struct kq_matvec_desc {
    const void *w;
    const void *x;
    float *y;
    int64_t n, k, batch;
    int64_t w_batch_stride;   /* super-blocks */
    int64_t x_batch_stride;   /* Q8_1 blocks */
    int64_t y_batch_stride;   /* floats */
} kq_matvec_desc;

int kq_matvec_batched(int type, const kq_matvec_desc *descs, int64_t n_desc, void *stream);
int q4_k_matvec(const void *w, const void *x, float *y, int64_t n, int64_t k, void *stream);
int q5_k_matvec(const void *w, const void *x, float *y, int64_t n, int64_t k, void *stream);

/* ---------------------------------------------------------------------------
 * q8_0_matmul_batched -- several independent products in one launch, for
 * sequencing a decode step with few kernel launches (launch count per token
 * is the cost the [NARR] kernels-per-token table tracks).  Descriptor i
 * computes, for every b < batch:
 *   Y_b[m][n] = X_b[m][k] . W_b[n][k]^T
 * with W_b = w + b*w_batch_stride (blocks), X_b row r = x + b*x_batch_stride +
 * r*x_row_stride (blocks), Y_b row r = y + b*y_batch_stride + r*y_row_stride
 * (floats).  All outputs of all descriptors must be disjoint; with batch > 1
 * the call rejects y_batch_stride < n and w_batch_stride < n*k/32 (Q8_E_SHAPE).
 * descs is a HOST array, read before the call returns.
 * Limits: n_desc <= 32 per call (Q8_E_UNSUPPORTED above), m <= 16 for every
 * descriptor (larger m: use q8_0_matmul).  W_b must be 16-byte aligned.
 */
typedef struct q8_0_matmul_desc {
    const q8_0_block *w;
    const q8_0_block *x;
    float *y;
    int64_t n, k, m, batch;
    int64_t w_batch_stride;   /* blocks */
    int64_t x_row_stride;     /* blocks, >= k/32 when m > 1 */
    int64_t x_batch_stride;   /* blocks */
    int64_t y_row_stride;     /* floats, >= n when m > 1 */
    int64_t y_batch_stride;   /* floats */
} q8_0_matmul_desc;

int q8_0_matmul_batched(const q8_0_matmul_desc *descs, int64_t n_desc, void *stream);

/* q8_0_matmul_f32_batched: the same products with fp32 activations, quantized
 * inside the launch by the activation rule (quantize_row_q8_0, [XEON] section
 * on narrowing down the cause; the bytes equal q8_0_quantize_rows of the rows),
 * so a decode step is one launch instead of a quantize launch and a product
 * launch.  Results are bitwise equal to q8_0_quantize_rows followed by
 * q8_0_matmul_batched on the same descriptors.
 *   x  fp32 rows, 16-byte aligned; x_row_stride and x_batch_stride in floats,
 *      multiples of 4 (x_row_stride >= k when m > 1)
 *   w  16-byte aligned, w_batch_stride (blocks) a multiple of 8
 * Streaming engines only: k % 256 == 0 and k <= 8192 (else Q8_E_UNSUPPORTED;
 * quantize with q8_0_quantize_rows and use q8_0_matmul_batched), m <= 16.
 * Other rules as q8_0_matmul_batched. */
typedef struct {
    const q8_0_block *w;
    const float *x;
    float *y;
    int64_t n, k, m, batch;
    int64_t w_batch_stride;   /* blocks */
    int64_t x_row_stride;     /* floats */
    int64_t x_batch_stride;   /* floats */
    int64_t y_row_stride;     /* floats */
    int64_t y_batch_stride;   /* floats */
} q8_0_matmul_f32_desc;

int q8_0_matmul_f32_batched(const q8_0_matmul_f32_desc *descs, int64_t n_desc, void *stream);

/* q8_0_matmul_f32_step: the products of q8_0_matmul_f32_batched (same
 * descriptors and rules) for m <= 2, as one launch in which every activation
 * row is quantized once: the first workgroups quantize the rows into the
 * workspace, and each product tile waits for the rows it reads.  Protocol:
 * every batch entry's quantizer parts count themselves on a per-entry part
 * counter; the entry's last part resets that counter and sets one flag per
 * product tile of the entry; a tile takes its flag with one atomic exchange
 * (read and clear in one access) and polls until it reads 1, so every flag
 * and counter is zero again at the end of a call that completes.  Ordering
 * rests on agent-scope accesses, not on release/acquire fences: the
 * quantized rows are written with agent-scope stores and read with
 * agent-scope loads (each coherent across the device's L2 caches by itself),
 * counters and flags are relaxed agent-scope atomics, a quantizer waits for
 * its stores to complete (s_waitcnt on the store counter) before it counts
 * itself, and a tile issues its row loads only after its poll has returned
 * 1.  The wait is bounded (see the error word below).  This is the whole decode step of the
 * narray-llm README's Llama 2 110M int8 table (every matvec's input
 * re-quantized, [NARR] sections on the measurement and on kernels per token)
 * in one launch.  Results are bitwise equal to q8_0_quantize_rows followed by
 * q8_0_matmul_batched.
 *   m > 2 for any descriptor: Q8_E_UNSUPPORTED (use q8_0_matmul_f32_batched).
 * Workspace: device memory of at least q8_0_matmul_f32_step_ws_bytes(descs,
 * n_desc) bytes, 256-byte aligned, ZERO-FILLED before its first use.  Every
 * call that completes leaves its counters at zero again, so it can be reused
 * (also across replays of a captured graph) without clearing.  After a call:
 *   - int32 at byte 0 is the error word: 1 if a tile's bounded wait for its
 *     rows ran out (the outputs of that call are then invalid); the library
 *     never clears it (zero-fill the workspace again after reading 1);
 *   - the quantized rows of descriptor i start at byte
 *     256 + sum over j < i of align256(batch_j * m_j * k_j/32 * 34), batch
 *     entry b at b * m_i * k_i/32 * 34 within them (the bytes of
 *     q8_0_quantize_rows); the counters and flags follow the rows.
 * One workspace must not be shared by calls that may run concurrently.
 * q8_0_matmul_f32_step_ws_bytes returns the byte count, or a negative status
 * for descriptors q8_0_matmul_f32_step would reject. */
int64_t q8_0_matmul_f32_step_ws_bytes(const q8_0_matmul_f32_desc *descs, int64_t n_desc);

int q8_0_matmul_f32_step(const q8_0_matmul_f32_desc *descs, int64_t n_desc, void *ws,
                         int64_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * q8_0_up_gate_swiglu_batched -- the dense FFN up_gate with SwiGLU in one pass
 * (FUSED_UP_GATE, named beside MOE_FUSED_UP_GATE in the [XEON] section on the
 * broken op paths; the split form two products + silu(gate)*up is the one the
 * [XEON] three-part fix, runtime graph fallback, builds).  Descriptor i
 * computes, for every b < batch and token row t < m:
 *   h_b[t][j] = silu(W_b[j] . X_b[t]) * (W_b[n_ff + j] . X_b[t]),  j < n_ff
 * with silu(g) = g / (1 + exp(-g)) in fp32, W_b = w + b*w_batch_stride (blocks),
 * the combined weight [2*n_ff][n_embd/32] with the gate rows first (16-byte
 * aligned), X_b row t = x + b*x_batch_stride + t*x_row_stride (Q8_0 blocks, as
 * q8_0_quantize_rows writes them), h_b row t = h + b*h_batch_stride +
 * t*h_row_stride (floats, written).  Each gate and up sum is bitwise the
 * q8_0_matmul_batched result for that row.
 * Limits: m <= 2 (Q8_E_UNSUPPORTED above); n_embd/32 a multiple of 8 and
 * n_embd <= 8192, w_batch_stride*34 a multiple of 16 (else Q8_E_UNSUPPORTED /
 * Q8_E_ALIGN); n_desc <= 32.  With batch > 1: w_batch_stride >= 2*n_ff*n_embd/32
 * and h_batch_stride >= n_ff (Q8_E_SHAPE).  descs is a HOST array.
 */
typedef struct q8_0_up_gate_desc {
    const q8_0_block *w;
    const q8_0_block *x;
    float *h;
    int64_t n_ff, n_embd, m, batch;
    int64_t w_batch_stride;   /* blocks */
    int64_t x_row_stride;     /* blocks, >= n_embd/32 when m > 1 */
    int64_t x_batch_stride;   /* blocks */
    int64_t h_row_stride;     /* floats, >= n_ff when m > 1 */
    int64_t h_batch_stride;   /* floats */
} q8_0_up_gate_desc;

int q8_0_up_gate_swiglu_batched(const q8_0_up_gate_desc *descs, int64_t n_desc, void *stream);

/* ---------------------------------------------------------------------------
 * Mixture-of-experts expert FFN ([XEON] sections on the broken op paths and on
 * the three-part fix, runtime graph fallback).  Per token t and active slot
 * u < n_used with expert e = ids[t][u]:
 *   g  = W_ug[e][j]        . q(x_t)   (gate rows j < n_ff, the first half)
 *   up = W_ug[e][n_ff + j] . q(x_t)   (up rows, the second half)
 *   h[t][u][j] = silu(g) * up = g / (1 + exp(-g)) * up        (fp32)
 *   out[t] = sum over u ascending of cw[t][u] * (W_d[e] . q(h[t][u]))
 * where q() is the quantization rule above, applied to each token row x_t and
 * to each h row inside the calls (the bytes equal q8_0_quantize_rows of those
 * rows), as the activations reach mul_mat_id in fp32.  The gate
 * and up products use the same quantized token row; the fused computation
 * gives the numbers of the split form (two mul_mat_id on row views + silu*up).
 * Each active expert's weight rows are streamed once per call, for all of the
 * slots routed to it.
 *
 * ids: int32 [n_tok][n_used], each in [0, n_expert).  An id outside that range
 * cannot be seen on the host; the kernels skip such a slot's products, write
 * NaN to its h row (up_gate) or to the output rows of its token (down), and set
 * the int32 error word at the start of the workspace to 1.  The word is cleared
 * at the start of every call; read it after the call to check.
 *
 * Workspace: caller-owned device memory of at least moe_workspace_bytes(...)
 * bytes, 256-byte aligned; contents need not be initialised and are
 * overwritten.  One workspace must not be shared by calls that may run
 * concurrently.
 */
size_t moe_workspace_bytes(int64_t n_tok, int64_t n_embd, int64_t n_ff,
                           int64_t n_expert, int64_t n_used);

/*   w_up_gate  Q8_0 [n_expert][2*n_ff][n_embd/32]  (ggml [n_embd, 2*n_ff, n_expert])
 *   x          fp32 [n_tok][n_embd], 16-byte aligned (token activations)
 *   ids        int32 [n_tok][n_used]
 *   h          fp32 [n_tok][n_used][n_ff]          (written)
 * n_tok >= 0, n_embd % 32 == 0, n_ff % 32 == 0, 1 <= n_used <= 16,
 * n_expert <= 1024.
 * Up to 16 tokens per call (decode) the expert-major streaming kernels run.
 * With more tokens (prompt evaluation) the call routes the slots into tiles of
 * at most 32 per expert and runs grouped GEMMs on the int8 matrix cores; that
 * path needs n_embd % 128 == 0 and n_ff % 128 == 0, n_tok <= 8192 and
 * n_tok*n_used <= 65536.  Other shapes with more than 16 tokens run on the
 * streaming kernels up to n_tok*n_used = 1024, else Q8_E_UNSUPPORTED.  Both
 * paths compute the same quantities; their fp32 sums may differ in the last
 * bits (different summation order), each within the stated tolerance.
 * x is taken in fp32, not as Q8_0 rows: activations reach mul_mat_id in fp32
 * and are quantized for the Q8_0 x Q8_0 product ([XEON] three-part fix, where
 * the compile fix names the activation quantizer), so the call quantizes each
 * token row inside its own launch (the bytes of q8_0_quantize_rows) instead of
 * needing a separate quantize launch and a Q8_0 buffer; every block sum and h
 * value is that of q8_0_quantize_rows(x) against the weights. */
int moe_up_gate_swiglu(const q8_0_block *w_up_gate, const float *x,
                       const int32_t *ids, float *h,
                       int64_t n_tok, int64_t n_embd, int64_t n_ff,
                       int64_t n_expert, int64_t n_used,
                       void *ws, size_t ws_bytes, void *stream);

/*   w_down  Q8_0 [n_expert][n_embd][n_ff/32]  (ggml [n_ff, n_embd, n_expert])
 *   h       fp32 [n_tok][n_used][n_ff]        (quantized inside, rule above)
 *   ids     int32 [n_tok][n_used];  cw  fp32 [n_tok][n_used] combine weights
 *   out     fp32 [n_tok][n_embd]              (written)
 * Same limits as moe_up_gate_swiglu. */
int moe_down_combine(const q8_0_block *w_down, const float *h,
                     const int32_t *ids, const float *cw, float *out,
                     int64_t n_tok, int64_t n_ff, int64_t n_embd,
                     int64_t n_expert, int64_t n_used,
                     void *ws, size_t ws_bytes, void *stream);

/* Grouped forms: n_desc independent layers (or micro-batches) of the same
 * shape in one launch per 32 descriptors, each with its own weights, inputs,
 * outputs and workspace; per layer the results are those of the single-layer
 * call (same kernels, same bits).  For a layer stack whose layers do not feed
 * each other within the call, e.g. layers of separate requests, or synthetic
 * per-layer inputs.  Workspaces of different descriptors must not overlap;
 * every other rule and limit is that of the single-layer call.  n_desc == 0
 * does nothing; a descriptor that fails a check fails the whole call before
 * anything is enqueued. */
typedef struct {
    const q8_0_block *w_up_gate;
    const float *x;
    const int32_t *ids;
    float *h;
    void *ws;
    size_t ws_bytes;
} moe_up_gate_desc;

int moe_up_gate_swiglu_batched(const moe_up_gate_desc *descs, int64_t n_desc,
                               int64_t n_tok, int64_t n_embd, int64_t n_ff,
                               int64_t n_expert, int64_t n_used, void *stream);

typedef struct {
    const q8_0_block *w_down;
    const float *h;
    const int32_t *ids;
    const float *cw;
    float *out;
    void *ws;
    size_t ws_bytes;
} moe_down_desc;

int moe_down_combine_batched(const moe_down_desc *descs, int64_t n_desc,
                             int64_t n_tok, int64_t n_ff, int64_t n_embd,
                             int64_t n_expert, int64_t n_used, void *stream);

/* ---------------------------------------------------------------------------
 * moe_r8_ffn_batched -- the whole expert FFN (the moe_up_gate_swiglu and
 * moe_down_combine arithmetic, same h and out) over expert weights repacked
 * once into the R8 layout (q8_0_repack_r8): w_up_gate_r8 = the combined tensor
 * as n_expert*2*n_ff rows of n_embd values, w_down_r8 = the down tensor as
 * n_expert*n_embd rows of n_ff values.  h [n_tok][n_used][n_ff] and out
 * [n_tok][n_embd] are written; x, ids, cw as for the native calls.
 * Up to 16 tokens (decode), several layers of one shape per launch: at one
 * token two launches per call, each slot streaming its expert's rows; at 2..16
 * tokens three (up_gate, down, the combine of the native path), each active
 * expert's rows streamed once per call for all of its slots (4 slots per pass
 * over the rows).  h and out are the same bits either way: per slot the
 * arithmetic and its order do not depend on how slots are grouped.
 * More than 16 tokens (prompt evaluation), where n_embd % 128 == 0 and
 * n_ff % 128 == 0 and the limits of the native prefill path hold: per layer
 * routing into tiles of up to 32 slots, then the two products on the int8
 * matrix cores, each expert's rows read once per tile; h and out are bit for
 * bit those of the native calls on the same weights; h must be 16-byte
 * aligned on this path.
 * Limits otherwise: n_embd % 32 == 0, n_ff % 32 == 0, n_ff <= 2048,
 * n_embd <= 32768, n_tok*n_used <= 1024, n_used <= 16, n_expert <= 1024
 * (Q8_E_UNSUPPORTED).
 * Out-of-range ids: the error word (first int32 of ws, set every call), NaN
 * h rows for such slots and NaN output rows for their tokens.
 * Workspace: moe_r8_workspace_bytes(...) bytes, 256-byte aligned (0 for an
 * unsupported shape); one workspace per layer, not shared by concurrent calls.
 */
typedef struct moe_r8_ffn_desc {
    const void *w_up_gate_r8;
    const void *w_down_r8;
    const float *x;
    const int32_t *ids;
    const float *cw;
    float *h;
    float *out;
    void *ws;
    size_t ws_bytes;
} moe_r8_ffn_desc;

size_t moe_r8_workspace_bytes(int64_t n_tok, int64_t n_embd, int64_t n_ff, int64_t n_expert,
                              int64_t n_used);
int moe_r8_ffn_batched(const moe_r8_ffn_desc *descs, int64_t n_desc, int64_t n_tok,
                       int64_t n_embd, int64_t n_ff, int64_t n_expert, int64_t n_used,
                       void *stream);

/* moe_r8_ffn_fused -- one token through one layer of the expert FFN over R8
 * expert weights in ONE launch: the form for a model whose layers run one
 * after another (each layer's input is the previous layer's output), where
 * moe_r8_ffn_batched takes two launches per layer.  Same inputs and outputs
 * as moe_r8_ffn_batched with n_tok = 1 and one descriptor (Gemma-4-on-Xeon
 * page, "GPUなしで13年前のXeon上でGemma 4 26Bを毎秒5トークンで実行する", section
 * on the broken op paths: the expert FFN with mul_mat_id and the combine).
 * h is the same bits as moe_r8_ffn_batched's; out is the same sums of the
 * same block terms (d_w * d_h) * s, added in another order (per slot over
 * the blocks of h ascending, then over the slots ascending with cw), so it
 * matches within rounding, not bit for bit.
 * Measured on the Gemma-4-26B-A4B expert shape (30 layers, one after
 * another): slower than moe_r8_ffn_batched per layer, 562 against 445 us per
 * step.  The launch it saves costs less than the in-kernel summation: every
 * workgroup's terms reach agent scope, a ticket, the last workgroups' wait,
 * and their agent-scope reads are one chain of memory round trips.
 * Limits: n_embd % 256 == 0 and those of moe_r8_ffn_batched's one-token path
 * (Q8_E_UNSUPPORTED otherwise).
 * Workspace: moe_r8_fused_workspace_bytes(...) bytes (0 for an unsupported
 * shape), 256-byte aligned; its first 256 bytes must be zero before the
 * first call (every call leaves them zero).  Word 0 is the error word: bit 0
 * set when an id is out of range (then that slot's h row and every out row
 * are NaN), bit 1 when the launch's final summation gave up waiting for its
 * workgroups (out is then invalid).  One workspace per stream: two calls
 * that may run at the same time must not share it. */
size_t moe_r8_fused_workspace_bytes(int64_t n_embd, int64_t n_ff, int64_t n_expert, int64_t n_used);
int moe_r8_ffn_fused(const moe_r8_ffn_desc *desc, int64_t n_embd, int64_t n_ff, int64_t n_expert,
                     int64_t n_used, void *stream);

/* moe_r8_ffn_batched_noalloc -- moe_r8_ffn_batched for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same kernels, h and out bit for bit,
 * with the workspaces taken from an array the library holds on each device
 * (48 MiB per device, held until the process ends; looked up once per device
 * at the first call on it, which is the only call that can return Q8_E_HIP
 * for that lookup).  The call allocates and frees nothing.
 *   descs  as for moe_r8_ffn_batched; ws and ws_bytes are ignored.
 * Decode shapes only: n_tok <= 16 (more tokens: Q8_E_UNSUPPORTED).  Layer i
 * uses the i-th slice of moe_r8_workspace_bytes(...) rounded up to 256 bytes;
 * n_desc slices beyond 48 MiB: Q8_E_WORKSPACE (split the call).  Every call on
 * a device shares that device's array and leaves its contents behind: two
 * calls that may run at the same time on one device race (order them on one
 * stream).  Nothing in the array needs clearing: every call rewrites what it
 * reads.  The error word of the workspace is not visible to the caller; an
 * out-of-range id shows as NaN h rows for its slot and NaN output rows for
 * its token, as in moe_r8_ffn_batched. */
int moe_r8_ffn_batched_noalloc(const moe_r8_ffn_desc *descs, int64_t n_desc, int64_t n_tok,
                               int64_t n_embd, int64_t n_ff, int64_t n_expert, int64_t n_used,
                               void *stream);

/* ---------------------------------------------------------------------------
 * Validation exports, for testing: the kernels of the product path, built
 * with an extra output (a compile-time flag, so the product path itself is
 * unchanged), that write the exact int32 block sums s = sum_j qw[j]*qx[j] of
 * every (token row, weight row, block) they form -- the quantity the block
 * dot of ggml_vec_dot_q8_0_q8_0 computes ([XEON] section on narrowing down
 * the cause) -- and, for the expert FFN, the routing and the quantized h rows
 * they used.  Each takes the arguments of its product call plus the extra
 * outputs, computes the same fp32 results, and follows the same kernel
 * selection (so a shape is checked on the kernel the product call runs).
 *
 * q8_0_matmul_blocksums: the sums s[m][n][b] of q8_0_matmul for W[n][k],
 * X[m][k] (any m: the streaming engines up to 16 rows, the matrix-core
 * kernel above), written to sums (int32 [m][n][k/32]); y receives the usual
 * fp32 result.
 */
int q8_0_matmul_blocksums(const q8_0_block *w, const q8_0_block *x, float *y,
                          int32_t *sums, int64_t n, int64_t k, int64_t m,
                          void *stream);

/* q8v_matvec_r8_batched_blocksums / q8v_matvec_r8_f32_batched_blocksums: the
 * products of q8_0_matvec_r8_batched / q8_0_matvec_r8_f32_batched (same
 * descriptors, same kernel) and, for descriptor i, the block sums in sums[i]
 * (int32 [batch][n][k/32]; sums is a HOST array of n_desc device pointers).
 * The f32 form's sums are those of the activation row quantized inside the
 * launch. */
int q8v_matvec_r8_batched_blocksums(const q8_0_r8_desc *descs, int64_t n_desc,
                                    int32_t *const *sums, void *stream);
int q8v_matvec_r8_f32_batched_blocksums(const q8_0_r8_f32_desc *descs, int64_t n_desc,
                                        int32_t *const *sums, void *stream);

/* q8v_matmul_r8_batched_blocksums: q8_0_matmul_r8_batched with the block sums
 * of descriptor i in sums[i] (int32 [batch][m][n][k/32]). */
int q8v_matmul_r8_batched_blocksums(const q8_0_r8_mm_desc *descs, int64_t n_desc,
                                    int32_t *const *sums, void *stream);

/* q8v_moe_up_gate: moe_up_gate_swiglu (same arguments, same path and
 * kernels for the shape: the decode kernels up to 16 tokens, the grouped
 * matrix-core path above) with validation outputs, each optional (NULL):
 *   sums    int32 [n_tok*n_used][2*n_ff][n_embd/32]: the block sums of every
 *           gate row (index j) and up row (n_ff + j) of each slot's expert
 *           against its token's quantized row (slots with an out-of-range id
 *           are not written);
 *   counts  int32 [n_expert], offsets int32 [n_expert + 1], pairs int32
 *           [n_tok*n_used]: the expert-major grouping the kernels served
 *           (slot t*n_used+u listed under its expert, experts ascending,
 *           slots ascending within an expert; out-of-range ids left out) --
 *           written by the kernels that group the slots (the ownership scan
 *           of the decode kernels, the routing tables of the grouped path);
 *           all three or none, and Q8_E_UNSUPPORTED for the shapes that run
 *           on the generic kernels, which serve every slot on its own.
 * h and the workspace are written as by moe_up_gate_swiglu. */
int q8v_moe_up_gate(const q8_0_block *w_up_gate, const float *x, const int32_t *ids, float *h,
                    int32_t *sums, int32_t *counts, int32_t *offsets, int32_t *pairs,
                    int64_t n_tok, int64_t n_embd, int64_t n_ff, int64_t n_expert, int64_t n_used,
                    void *ws, size_t ws_bytes, void *stream);

/* q8v_moe_hq: moe_down_combine (same arguments and kernels) with validation
 * outputs, each optional (NULL):
 *   hq    Q8_0 [n_tok*n_used][n_ff/32]: the quantized h rows the down
 *         products used (the bytes of q8_0_quantize_rows of the h rows; rows
 *         of slots with an out-of-range id are unspecified);
 *   sums  int32 [n_tok*n_used][n_embd][n_ff/32]: the block sums of every
 *         down row of each slot's expert against that slot's q(h) row.
 * out and the workspace are written as by moe_down_combine. */
int q8v_moe_hq(const q8_0_block *w_down, const float *h, const int32_t *ids, const float *cw,
               float *out, q8_0_block *hq, int32_t *sums, int64_t n_tok, int64_t n_ff,
               int64_t n_embd, int64_t n_expert, int64_t n_used, void *ws, size_t ws_bytes,
               void *stream);

/* q8v_moe_r8_ffn: moe_r8_ffn_batched for one layer (desc, with its
 * workspace) with the validation outputs of both products: ug_sums and
 * dn_sums laid out as the sums of q8v_moe_up_gate and q8v_moe_hq, hq the
 * quantized h rows the down product used, and the routing (counts, offsets,
 * pairs as in q8v_moe_up_gate) the kernels grouped the slots by (2 tokens or
 * more; at one token each slot streams its expert on its own:
 * Q8_E_UNSUPPORTED there).  Each output optional (NULL). */
int q8v_moe_r8_ffn(const moe_r8_ffn_desc *desc, int64_t n_tok, int64_t n_embd, int64_t n_ff,
                   int64_t n_expert, int64_t n_used, int32_t *ug_sums, int32_t *dn_sums,
                   q8_0_block *hq, int32_t *counts, int32_t *offsets, int32_t *pairs,
                   void *stream);

/* moe_route: the grouping of (t,u) slots by expert that the MoE kernels use:
 * counts[e] (int32 [n_expert]), offsets[e] (int32 [n_expert+1], exclusive
 * prefix of counts), pairs (int32 [n_tok*n_used]): t*n_used+u of every slot,
 * grouped by ascending expert, ascending (t,u) within an expert.  Slots with
 * an out-of-range id are left out (offsets[n_expert] then counts the rest)
 * and set the error word in ws.  Same limits as moe_up_gate_swiglu. */
int moe_route(const int32_t *ids, int32_t *counts, int32_t *offsets,
              int32_t *pairs, int64_t n_tok, int64_t n_expert, int64_t n_used,
              void *ws, size_t ws_bytes, void *stream);

/* q8_read_probe: a plain streaming read of `bytes` bytes at p (16-byte
 * aligned, a multiple of 16) with the engines' load pattern, the device
 * analogue of a host memory-bandwidth probe, for reporting the achievable
 * read rate beside the datasheet peak.  Writes one word per workgroup to sink
 * (at most 4096 words are used; Q8_E_WORKSPACE if sink_words is too small). */
int q8_read_probe(const void *p, int64_t bytes, uint32_t *sink, int64_t sink_words,
                  void *stream);

#ifdef __cplusplus
}
#endif

#endif /* Q8MOE_H */
