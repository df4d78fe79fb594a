/*
 * q8_oracle.c -- the CPU oracle for the Q8_0 decode path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  The product path (the
 * HIP library under moe_expert_ffn_q8_amd/) never calls it, and the two share
 * no code: this file has its own block parser, its own fp16 codec and its own
 * loops.
 *
 * It is plain scalar C, compiled with -O2 -ffp-contract=off and without
 * -ffast-math, so every float operation below is one IEEE operation in the
 * order written.
 *
 * What it computes, and where that comes from (sources are web pages, cited by
 * title and section):
 *
 *  - The Q8_0 format.  The page "GPUなしで13年前のXeon上でGemma 4 26Bを毎秒5
 *    トークンで実行する" (Gemma 4 26B-A4B Q8_0 on a 2013 dual Xeon) names the
 *    format in its summary and in the section on the broken op paths, and names
 *    the activation quantizer quantize_row_q8_0_x4 in the section on the
 *    three-part fix (compile fix).  The narray-llm README names "int8 (Q8_0)"
 *    in its Llama 2 110M table.  None of the pages prints the bytes, so this
 *    file uses the plain reading of the format: a block is 32 signed 8-bit
 *    codes q[j] and one IEEE binary16 scale d; it is stored as 34 bytes, the
 *    scale first (little-endian) then the 32 codes; its value is d*q[j].
 *    Quantization of 32 fp32 values: d = max|x| / 127 (fp32), q = round(x/d)
 *    with ties away from zero, d stored rounded to binary16.
 *
 *  - The block dot product behind ggml_vec_dot_q8_0_q8_0 (same page, section
 *    on how the cause was narrowed down): the exact integer sum of the 32
 *    products q_w*q_x, scaled by d_w*d_x.  Here the scaling and the sum over
 *    blocks are done in fp64; every product d_w*d_x*s is exact in fp64 (at
 *    most 11+11+20 significant bits), so the only rounding is in the sum.
 *
 *  - mul_mat_id over the combined up_gate tensor [n_embd, 2*n_ff, n_experts],
 *    gate rows first and up rows second, followed by silu(gate)*up (same page,
 *    section on the three-part fix, runtime graph fallback).  The fallback
 *    there splits the tensor into two views, runs mul_mat_id on each and
 *    combines with fused_mul_unary(SILU); the fused form must give the same
 *    numbers.  Both forms are written out below so that the identity can be
 *    checked.
 *
 *  - The expert down projection and the weighted combine over the active
 *    experts of a token: out[t] = sum_k w[t][k] * down_{e(t,k)}(q(h[t][k])),
 *    with h quantized per row by the same Q8_0 rule.  The pages show the expert
 *    FFN and its 8 active experts per token (same page, section on the broken
 *    op paths) but not the down/combine arithmetic; this is the plain reading.
 *
 * Layouts (C order, rows of blocks back to back):
 *   weights  [n_rows][k/32] blocks          (ggml [k, n_rows])
 *   up_gate  [n_expert][2*n_ff][n_embd/32]  (ggml [n_embd, 2*n_ff, n_expert])
 *   down     [n_expert][n_embd][n_ff/32]    (ggml [n_ff, n_embd, n_expert])
 *   ids, combine weights [n_tok][n_used]
 *
 * Every function returns 0 on success and a negative value on a bad argument.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define OQK 32          /* values per block */
#define OBLK 34         /* bytes per block: 2 scale bytes + 32 codes */

/* ------------------------------------------------------------------------ */
/* binary16 codec, by bit manipulation (IEEE 754-2008 binary16).             */
/* ------------------------------------------------------------------------ */

/* fp32 -> binary16, round to nearest, ties to even; gradual underflow;
   overflow to +-inf; NaN stays NaN (quiet). */
uint16_t or_f32_to_f16(float f)
{
    uint32_t x;
    memcpy(&x, &f, 4);
    uint32_t sign = (x >> 16) & 0x8000u;
    uint32_t e32 = (x >> 23) & 0xffu;
    uint32_t m32 = x & 0x7fffffu;

    if (e32 == 0xffu) {                       /* inf or NaN */
        if (m32 == 0) return (uint16_t)(sign | 0x7c00u);
        return (uint16_t)(sign | 0x7e00u | (m32 >> 13));
    }
    int e16 = (int)e32 - 127 + 15;            /* biased binary16 exponent */
    if (e16 >= 31) return (uint16_t)(sign | 0x7c00u);

    if (e16 >= 1) {                           /* normal range before rounding */
        uint32_t base = ((uint32_t)e16 << 10) | (m32 >> 13);
        uint32_t rest = m32 & 0x1fffu;        /* the 13 bits dropped */
        if (rest > 0x1000u || (rest == 0x1000u && (base & 1u))) base += 1;
        /* a carry out of the mantissa bumps the exponent; 0x7c00 is inf */
        return (uint16_t)(sign | base);
    }

    /* result is subnormal (or zero): value in units of 2^-24 is
       (2^23 + m32) * 2^(e32 - 126 - 23) ... i.e. sig >> shift below */
    if (e32 == 0) return (uint16_t)sign;      /* fp32 zero or subnormal: < 2^-126 */
    uint32_t sig = 0x800000u | m32;           /* 24-bit significand */
    int shift = 126 - (int)e32;               /* >= 14 here */
    if (shift > 24) return (uint16_t)sign;    /* below half of 2^-24 */
    uint32_t q = sig >> shift;
    uint32_t rest = sig & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (rest > half || (rest == half && (q & 1u))) q += 1;
    return (uint16_t)(sign | q);              /* q == 0x400 is the smallest normal */
}

/* binary16 -> fp32, exact, written as arithmetic on the fields. */
float or_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)m, -24);                     /* zero or subnormal */
    } else if (e == 31) {
        if (m == 0) v = INFINITY;
        else return sign ? -NAN : NAN;
    } else {
        v = ldexp((double)(1024 + m), e - 25);          /* (1 + m/1024) * 2^(e-15) */
    }
    return (float)(sign ? -v : v);                      /* exact in fp32 */
}

/* ------------------------------------------------------------------------ */
/* Q8_0 block access                                                         */
/* ------------------------------------------------------------------------ */

static float blk_scale(const uint8_t *blk)
{
    uint16_t h = (uint16_t)(blk[0] | ((uint16_t)blk[1] << 8));
    return or_f16_to_f32(h);
}

static int blk_code(const uint8_t *blk, int j)
{
    return (int)(int8_t)blk[2 + j];
}

/* Quantize 32 fp32 values into one 34-byte block.
   amax is exact; d = amax/127 is one fp32 division; each code is
   roundf(x/d) (fp32 division, then rounding half away from zero).  For a
   normal d the code is within [-127, 127] by construction; a subnormal d
   can push the ratio past 127.5, and the code saturates at +-127 there.
   An all-zero block stores d = +0 and all codes 0. */
void or_quantize_block(const float *x, uint8_t *out)
{
    float amax = 0.0f;
    for (int j = 0; j < OQK; j++) {
        float a = fabsf(x[j]);
        if (a > amax) amax = a;
    }
    float d = amax / 127.0f;
    uint16_t dh = or_f32_to_f16(d);
    out[0] = (uint8_t)(dh & 0xff);
    out[1] = (uint8_t)(dh >> 8);
    for (int j = 0; j < OQK; j++) {
        int q = 0;
        if (d != 0.0f) {
            float r = roundf(x[j] / d);
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            q = (int)r;
        }
        out[2 + j] = (uint8_t)(int8_t)q;
    }
}

/* x: [n_rows][row_stride] fp32 (row_stride >= k), out: [n_rows][k/32] blocks */
int or_quantize_rows(const float *x, int64_t row_stride, uint8_t *out,
                     int64_t n_rows, int64_t k)
{
    if (k <= 0 || k % OQK != 0 || n_rows < 0 || row_stride < k) return -2;
    int64_t nb = k / OQK;
    for (int64_t r = 0; r < n_rows; r++)
        for (int64_t b = 0; b < nb; b++)
            or_quantize_block(x + r * row_stride + b * OQK,
                              out + (r * nb + b) * OBLK);
    return 0;
}

/* Integer dot product of the codes of two blocks (exact). */
int32_t or_block_dot(const uint8_t *wb, const uint8_t *xb)
{
    int32_t s = 0;
    for (int j = 0; j < OQK; j++) s += blk_code(wb, j) * blk_code(xb, j);
    return s;
}

/* One output: sum over the nb blocks of d_w*d_x*s_b, in fp64. */
static double row_dot(const uint8_t *wrow, const uint8_t *xrow, int64_t nb)
{
    double acc = 0.0;
    for (int64_t b = 0; b < nb; b++) {
        const uint8_t *wb = wrow + b * OBLK;
        const uint8_t *xb = xrow + b * OBLK;
        double s = (double)or_block_dot(wb, xb);
        acc += ((double)blk_scale(wb) * (double)blk_scale(xb)) * s;
    }
    return acc;
}

/* Y[m][n] = sum_b d_w[n][b] d_x[m][b] s[m][n][b]; y: [m][n] fp64.
   Only rows n in [n_begin, n_end) are written (the rest of y is untouched). */
int or_matmul(const uint8_t *w, const uint8_t *x, double *y,
              int64_t n, int64_t k, int64_t m, int64_t n_begin, int64_t n_end)
{
    if (k <= 0 || k % OQK != 0 || n < 0 || m < 0) return -2;
    if (n_begin < 0 || n_end > n || n_begin > n_end) return -2;
    int64_t nb = k / OQK;
    for (int64_t mi = 0; mi < m; mi++)
        for (int64_t ni = n_begin; ni < n_end; ni++)
            y[mi * n + ni] = row_dot(w + ni * nb * OBLK, x + mi * nb * OBLK, nb);
    return 0;
}

/* Selected outputs only: y_sel[i] = Y[sel_m[i]][sel_n[i]]. */
int or_matmul_select(const uint8_t *w, const uint8_t *x, int64_t n, int64_t k,
                     int64_t m, const int64_t *sel_m, const int64_t *sel_n,
                     int64_t n_sel, double *y_sel)
{
    if (k <= 0 || k % OQK != 0) return -2;
    int64_t nb = k / OQK;
    for (int64_t i = 0; i < n_sel; i++) {
        if (sel_m[i] < 0 || sel_m[i] >= m || sel_n[i] < 0 || sel_n[i] >= n) return -2;
        y_sel[i] = row_dot(w + sel_n[i] * nb * OBLK, x + sel_m[i] * nb * OBLK, nb);
    }
    return 0;
}

/* Per-block integer sums s[m][n][b] (exact). */
int or_matmul_blocksums(const uint8_t *w, const uint8_t *x, int32_t *s,
                        int64_t n, int64_t k, int64_t m)
{
    if (k <= 0 || k % OQK != 0 || n < 0 || m < 0) return -2;
    int64_t nb = k / OQK;
    for (int64_t mi = 0; mi < m; mi++)
        for (int64_t ni = 0; ni < n; ni++)
            for (int64_t b = 0; b < nb; b++)
                s[(mi * n + ni) * nb + b] =
                    or_block_dot(w + (ni * nb + b) * OBLK, x + (mi * nb + b) * OBLK);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Mixture-of-experts pieces                                                 */
/* ------------------------------------------------------------------------ */

static int check_ids(const int32_t *ids, int64_t n_tok, int64_t n_used, int64_t n_expert)
{
    for (int64_t i = 0; i < n_tok * n_used; i++)
        if (ids[i] < 0 || ids[i] >= n_expert) return -7;
    return 0;
}

/* mul_mat_id on a 3-D weight [n_expert][rows_per_expert][nb], restricted to
   the row window [row_off, row_off + n_rows) of every expert (a view):
   out[t][u][r] = row_dot(W[ids[t][u]][row_off + r], x[t]), x: [n_tok][nb]. */
int or_mul_mat_id(const uint8_t *w, int64_t rows_per_expert, int64_t row_off,
                  int64_t n_rows, const uint8_t *x, const int32_t *ids,
                  double *out, int64_t n_tok, int64_t k, int64_t n_expert,
                  int64_t n_used)
{
    if (k <= 0 || k % OQK != 0 || row_off < 0 || n_rows < 0 ||
        row_off + n_rows > rows_per_expert) return -2;
    if (check_ids(ids, n_tok, n_used, n_expert)) return -7;
    int64_t nb = k / OQK;
    for (int64_t t = 0; t < n_tok; t++)
        for (int64_t u = 0; u < n_used; u++) {
            int64_t e = ids[t * n_used + u];
            const uint8_t *we = w + e * rows_per_expert * nb * OBLK;
            for (int64_t r = 0; r < n_rows; r++)
                out[(t * n_used + u) * n_rows + r] =
                    row_dot(we + (row_off + r) * nb * OBLK, x + t * nb * OBLK, nb);
        }
    return 0;
}

/* silu(g) * u elementwise in fp64: g / (1 + exp(-g)) * u. */
void or_fused_mul_silu(const double *g, const double *u, double *h, int64_t n)
{
    for (int64_t i = 0; i < n; i++) h[i] = g[i] / (1.0 + exp(-g[i])) * u[i];
}

/* Fused form: for every slot (t,u) with e = ids[t][u] and every j < n_ff,
   g = row j of up_gate[e], up = row n_ff + j of up_gate[e], both against the
   token's quantized activation row x[t]; h[t][u][j] = silu(g) * up. */
int or_moe_up_gate_swiglu(const uint8_t *w_ug, const uint8_t *x, const int32_t *ids,
                          double *h, int64_t n_tok, int64_t n_embd, int64_t n_ff,
                          int64_t n_expert, int64_t n_used)
{
    if (n_embd <= 0 || n_embd % OQK != 0 || n_ff <= 0) return -2;
    if (check_ids(ids, n_tok, n_used, n_expert)) return -7;
    int64_t nb = n_embd / OQK;
    for (int64_t t = 0; t < n_tok; t++)
        for (int64_t u = 0; u < n_used; u++) {
            int64_t e = ids[t * n_used + u];
            const uint8_t *we = w_ug + e * 2 * n_ff * nb * OBLK;
            for (int64_t j = 0; j < n_ff; j++) {
                double g = row_dot(we + j * nb * OBLK, x + t * nb * OBLK, nb);
                double up = row_dot(we + (n_ff + j) * nb * OBLK, x + t * nb * OBLK, nb);
                h[(t * n_used + u) * n_ff + j] = g / (1.0 + exp(-g)) * up;
            }
        }
    return 0;
}

/* Routing: the (t,u) slots grouped by expert.  counts[e] = number of slots
   routed to e; offsets[e] = sum of counts below e (offsets[n_expert] = total);
   pairs[offsets[e] + i] = t*n_used + u of the i-th slot of expert e, in
   ascending (t, u) order. */
int or_moe_route(const int32_t *ids, int64_t n_tok, int64_t n_used, int64_t n_expert,
                 int32_t *counts, int32_t *offsets, int32_t *pairs)
{
    if (check_ids(ids, n_tok, n_used, n_expert)) return -7;
    int64_t pos = 0;
    for (int64_t e = 0; e < n_expert; e++) {
        offsets[e] = (int32_t)pos;
        int32_t c = 0;
        for (int64_t t = 0; t < n_tok; t++)
            for (int64_t u = 0; u < n_used; u++)
                if (ids[t * n_used + u] == e) {
                    pairs[pos++] = (int32_t)(t * n_used + u);
                    c++;
                }
        counts[e] = c;
    }
    offsets[n_expert] = (int32_t)pos;
    return 0;
}

/* Down projection and combine.
   h: [n_tok][n_used][n_ff] fp32 (the activation of every slot); each h row is
   quantized with the Q8_0 rule (in fp32, the precision it arrives in);
   y[t][u][n] = row_dot(down[e][n], q(h[t][u])) for e = ids[t][u];
   out[t][n] = sum over u ascending of cw[t][u] * y[t][u][n], in fp64.
   hq (optional, may be NULL): [n_tok][n_used][n_ff/32] blocks of q(h).
   sel (optional): only the listed output columns n are computed; out is then
   [n_tok][n_sel]. */
int or_moe_down_combine(const uint8_t *w_d, const float *h, const int32_t *ids,
                        const float *cw, double *out, uint8_t *hq,
                        int64_t n_tok, int64_t n_ff, int64_t n_embd,
                        int64_t n_expert, int64_t n_used,
                        const int64_t *sel, int64_t n_sel,
                        uint8_t *scratch_hq /* [n_used][n_ff/32] blocks */)
{
    if (n_ff <= 0 || n_ff % OQK != 0 || n_embd <= 0) return -2;
    if (check_ids(ids, n_tok, n_used, n_expert)) return -7;
    int64_t nb = n_ff / OQK;
    int64_t n_out = sel ? n_sel : n_embd;
    for (int64_t t = 0; t < n_tok; t++) {
        for (int64_t u = 0; u < n_used; u++) {
            uint8_t *q = scratch_hq + u * nb * OBLK;
            for (int64_t b = 0; b < nb; b++)
                or_quantize_block(h + (t * n_used + u) * n_ff + b * OQK, q + b * OBLK);
            if (hq) memcpy(hq + (t * n_used + u) * nb * OBLK, q, (size_t)(nb * OBLK));
        }
        for (int64_t i = 0; i < n_out; i++) {
            int64_t n = sel ? sel[i] : i;
            if (n < 0 || n >= n_embd) return -2;
            double acc = 0.0;
            for (int64_t u = 0; u < n_used; u++) {
                int64_t e = ids[t * n_used + u];
                const uint8_t *wrow = w_d + (e * n_embd + n) * nb * OBLK;
                double y = row_dot(wrow, scratch_hq + u * nb * OBLK, nb);
                acc += (double)cw[t * n_used + u] * y;
            }
            out[t * n_out + i] = acc;
        }
    }
    return 0;
}

/* Array forms of the codec (used by the exhaustive codec tests). */
void or_f32_to_f16_array(const float *x, uint16_t *h, int64_t n)
{
    for (int64_t i = 0; i < n; i++) h[i] = or_f32_to_f16(x[i]);
}

void or_f16_to_f32_array(const uint16_t *h, float *x, int64_t n)
{
    for (int64_t i = 0; i < n; i++) x[i] = or_f16_to_f32(h[i]);
}

/* ------------------------------------------------------------------------ */
/* Row-interleaved weight layout (R8)                                        */
/* ------------------------------------------------------------------------ */

/* The Gemma-4-on-Xeon page (section on the fallback's cost and the repacking
   bug) describes an option that, at startup, reorders the quantized weights
   into an interleaved form named Q8_0_R8, built for one instruction set.  The
   page gives no byte layout.  This library's reading, used for GPU streaming:
   rows are taken in groups of 8 (the last group padded with rows whose
   scale and codes are all zero); a group of 8 rows of nb blocks is 272*nb
   bytes, the 8*nb binary16 scales first, ordered by (block, row), then the
   codes, ordered by (block, row, position).  Group g starts at byte
   g*272*nb.  The data are the same bytes as the native rows, moved. */

#define OR8 8

static int64_t r8_group_bytes(int64_t nb) { return (int64_t)OR8 * OBLK * nb; }

/* Byte offset, inside its group, of the scale of row r (0..7) at block b. */
static int64_t r8_scale_at(int64_t b, int r) { return 2 * (b * OR8 + r); }

/* Byte offset, inside its group, of code j of row r at block b. */
static int64_t r8_code_at(int64_t nb, int64_t b, int r, int j)
{
    return 2 * OR8 * nb + (b * OR8 + r) * OQK + j;
}

int64_t or_r8_bytes(int64_t n, int64_t k)
{
    if (n < 0 || k <= 0 || k % OQK != 0) return -2;
    return (n + OR8 - 1) / OR8 * r8_group_bytes(k / OQK);
}

/* Native rows [n][k/32] blocks -> the R8 layout (or_r8_bytes(n, k) bytes). */
int or_repack_r8(const uint8_t *w, uint8_t *out, int64_t n, int64_t k)
{
    if (n < 0 || k <= 0 || k % OQK != 0) return -2;
    int64_t nb = k / OQK;
    int64_t groups = (n + OR8 - 1) / OR8;
    for (int64_t g = 0; g < groups; g++) {
        uint8_t *gp = out + g * r8_group_bytes(nb);
        for (int r = 0; r < OR8; r++) {
            int64_t row = g * OR8 + r;
            for (int64_t b = 0; b < nb; b++) {
                const uint8_t *blk = row < n ? w + (row * nb + b) * OBLK : NULL;
                gp[r8_scale_at(b, r)] = blk ? blk[0] : 0;
                gp[r8_scale_at(b, r) + 1] = blk ? blk[1] : 0;
                for (int j = 0; j < OQK; j++)
                    gp[r8_code_at(nb, b, r, j)] = blk ? blk[2 + j] : 0;
            }
        }
    }
    return 0;
}

/* y[i] (fp64) = sum over blocks, ascending, of d_w*d_x*s for row i read from
   the R8 layout; the same sum, in the same order, as or_matmul on the native
   rows. */
int or_matvec_r8(const uint8_t *w_r8, const uint8_t *x, double *y, int64_t n, int64_t k)
{
    if (n < 0 || k <= 0 || k % OQK != 0) return -2;
    int64_t nb = k / OQK;
    for (int64_t i = 0; i < n; i++) {
        const uint8_t *gp = w_r8 + (i / OR8) * r8_group_bytes(nb);
        int r = (int)(i % OR8);
        double acc = 0.0;
        for (int64_t b = 0; b < nb; b++) {
            const uint8_t *xb = x + b * OBLK;
            uint16_t dh = (uint16_t)(gp[r8_scale_at(b, r)] |
                                     ((uint16_t)gp[r8_scale_at(b, r) + 1] << 8));
            int32_t s = 0;
            for (int j = 0; j < OQK; j++)
                s += (int)(int8_t)gp[r8_code_at(nb, b, r, j)] * blk_code(xb, j);
            acc += ((double)or_f16_to_f32(dh) * (double)blk_scale(xb)) * (double)s;
        }
        y[i] = acc;
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Q8_1 activations and the 4/5-bit K-quant weight formats                  */
/* ------------------------------------------------------------------------ */

/* The Gemma-4-on-Xeon page names a second activation quantizer,
   quantize_row_q8_1_x4_T, beside the Q8_0 one (section on the three-part fix,
   compile fix), and the other pages run models stored as Q4_K_M and Q5_K_M
   (the Nemotron review's closing section; the ARM page's server commands).
   None of them prints a layout.  Readings used here:

   Q8_1 block, 36 bytes: binary16 d, binary16 s, 32 int8 codes.  d and the
   codes follow the Q8_0 rule exactly; s = binary16(d32 * sum of the codes),
   with d32 = amax/127 the unrounded fp32 scale, the product in fp32.

   K-quant super-block of 256 values = 8 sub-blocks of 32:
     Q4_K, 144 bytes: binary16 d, binary16 dmin, 12 bytes of 6-bit sub-block
       scales sc[8] and mins m[8], 128 bytes of 4-bit codes.
     Q5_K, 176 bytes: the same 16-byte header, 32 bytes of high bits, then the
       128 bytes of low 4-bit codes.
   6-bit fields: for j < 4, sc[j] = b[j] & 63 and m[j] = b[j+4] & 63; for
   j >= 4, the low 4 bits of sc[j] and m[j] are the low and high nibble of
   b[j+4], and their top 2 bits are the top 2 bits of b[j-4] and b[j].
   4-bit codes: sub-blocks 2c and 2c+1 share the 32 bytes at 32c: the low
   nibble of byte 32c+l is value l of sub-block 2c, the high nibble value l of
   sub-block 2c+1.  Q5_K adds 16 * bit j of high-bit byte l to value l of
   sub-block j.
   Value l of sub-block j: d * sc[j] * q - dmin * m[j]. */

#define OBLK81 36
#define OQKK 256
#define OBLK_Q4K 144
#define OBLK_Q5K 176

void or_quantize_block_q8_1(const float *x, uint8_t *out)
{
    uint8_t q0[OBLK];
    or_quantize_block(x, q0);                 /* d and codes by the Q8_0 rule */
    float amax = 0.0f;
    for (int j = 0; j < OQK; j++) {
        float a = fabsf(x[j]);
        if (a > amax) amax = a;
    }
    float d32 = amax / 127.0f;
    int sum = 0;
    for (int j = 0; j < OQK; j++) sum += blk_code(q0, j);
    uint16_t sh = or_f32_to_f16(d32 * (float)sum);
    out[0] = q0[0];
    out[1] = q0[1];
    out[2] = (uint8_t)(sh & 0xff);
    out[3] = (uint8_t)(sh >> 8);
    memcpy(out + 4, q0 + 2, OQK);
}

int or_quantize_rows_q8_1(const float *x, int64_t row_stride, uint8_t *out,
                          int64_t n_rows, int64_t k)
{
    if (k <= 0 || k % OQK != 0 || n_rows < 0 || row_stride < k) return -2;
    int64_t nb = k / OQK;
    for (int64_t r = 0; r < n_rows; r++)
        for (int64_t b = 0; b < nb; b++)
            or_quantize_block_q8_1(x + r * row_stride + b * OQK, out + (r * nb + b) * OBLK81);
    return 0;
}

static int kq_block_bytes(int type)
{
    return type == 4 ? OBLK_Q4K : type == 5 ? OBLK_Q5K : -1;
}

/* The 6-bit scale and min of sub-block j (0..7) from the 12 packed bytes. */
void or_kq_scale_min(const uint8_t *b, int j, int *sc, int *m)
{
    if (j < 4) {
        *sc = b[j] & 63;
        *m = b[j + 4] & 63;
    } else {
        *sc = (b[j + 4] & 15) | ((b[j - 4] >> 6) << 4);
        *m = (b[j + 4] >> 4) | ((b[j] >> 6) << 4);
    }
}

/* Unsigned code (0..15 or 0..31) of value l of sub-block j. */
static int kq_code(int type, const uint8_t *blk, int j, int l)
{
    const uint8_t *qs = blk + (type == 4 ? 16 : 48);
    int byte = qs[32 * (j / 2) + l];
    int q = (j % 2) ? (byte >> 4) : (byte & 15);
    if (type == 5) q += 16 * ((blk[16 + l] >> j) & 1);
    return q;
}

/* Value l of sub-block j in fp64 (exact: at most 22 significant bits each side). */
static double kq_value(int type, const uint8_t *blk, int j, int l)
{
    double d = or_f16_to_f32((uint16_t)(blk[0] | (blk[1] << 8)));
    double dmin = or_f16_to_f32((uint16_t)(blk[2] | (blk[3] << 8)));
    int sc, m;
    or_kq_scale_min(blk + 4, j, &sc, &m);
    return d * sc * kq_code(type, blk, j, l) - dmin * m;
}

/* w: [n][k/256] super-blocks -> out fp64 [n][k]. */
int or_kq_dequantize_rows(int type, const uint8_t *w, double *out, int64_t n, int64_t k)
{
    int bb = kq_block_bytes(type);
    if (bb < 0 || k <= 0 || k % OQKK != 0 || n < 0) return -2;
    int64_t ns = k / OQKK;
    for (int64_t i = 0; i < n; i++)
        for (int64_t s = 0; s < ns; s++)
            for (int j = 0; j < 8; j++)
                for (int l = 0; l < OQK; l++)
                    out[i * k + s * OQKK + j * OQK + l] =
                        kq_value(type, w + (i * ns + s) * bb, j, l);
    return 0;
}

/* y[i] (fp64) = sum over the k values, ascending, of the dequantized weight
   times the dequantized Q8_1 activation d_x * q_x. */
int or_kq_matvec(int type, const uint8_t *w, const uint8_t *x, double *y, int64_t n, int64_t k)
{
    int bb = kq_block_bytes(type);
    if (bb < 0 || k <= 0 || k % OQKK != 0 || n < 0) return -2;
    int64_t ns = k / OQKK;
    for (int64_t i = 0; i < n; i++) {
        double acc = 0.0;
        for (int64_t s = 0; s < ns; s++) {
            const uint8_t *blk = w + (i * ns + s) * bb;
            for (int j = 0; j < 8; j++) {
                const uint8_t *xb = x + (s * 8 + j) * OBLK81;
                double dx = or_f16_to_f32((uint16_t)(xb[0] | (xb[1] << 8)));
                for (int l = 0; l < OQK; l++)
                    acc += kq_value(type, blk, j, l) * (dx * (double)(int8_t)xb[4 + l]);
            }
        }
        y[i] = acc;
    }
    return 0;
}
