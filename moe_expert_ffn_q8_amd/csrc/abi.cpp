// abi.cpp -- the extern "C" entry points of libq8moe.so (see include/q8moe.h).
//
// Every entry point validates its arguments on the host, before any HIP call,
// and returns a negative status without enqueuing anything when they are
// wrong.  Nothing here allocates, frees or synchronizes.
#include "q8moe.h"

#include <string.h>

#include <algorithm>

#include "q8_internal.h"
#include "q8_moe.h"

namespace {

constexpr int64_t kQK = 32;
constexpr int64_t kBB = 34;

inline bool aligned(const void *p, uintptr_t a) { return (((uintptr_t)p) % a) == 0; }

inline hipStream_t as_stream(void *s) { return (hipStream_t)s; }

inline int hip_status(int rc) { return rc == 0 ? Q8_OK : (rc < 0 ? rc : Q8_E_HIP); }

int check_k(int64_t k)
{
    if (k <= 0 || k % kQK != 0) return Q8_E_SHAPE;
    return Q8_OK;
}

// validation calls: every descriptor needs its block-sum array
bool sums_required(int32_t *const *sums, int64_t n_desc)
{
    if (!sums) return false;
    for (int64_t i = 0; i < n_desc; ++i)
        if (!sums[i]) return true;
    return false;
}

}  // namespace

extern "C" {

const char *q8_status_str(int status)
{
    switch (status) {
        case Q8_OK: return "ok";
        case Q8_E_NULL: return "null pointer";
        case Q8_E_SHAPE: return "bad shape";
        case Q8_E_ALIGN: return "misaligned pointer or stride";
        case Q8_E_UNSUPPORTED: return "unsupported by this build";
        case Q8_E_WORKSPACE: return "workspace missing or too small";
        case Q8_E_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char *q8_version(void) { return "q8moe 0.1 gfx950"; }

int q8_0_quantize_rows(const float *x, int64_t x_row_stride, q8_0_block *y, int64_t n_rows,
                       int64_t k, void *stream)
{
    if (int rc = check_k(k)) return rc;
    if (n_rows < 0 || x_row_stride < k) return Q8_E_SHAPE;
    if (n_rows == 0) return Q8_OK;
    if (!x || !y) return Q8_E_NULL;
    if (!aligned(x, 16) || x_row_stride % 4 != 0 || !aligned(y, 2)) return Q8_E_ALIGN;
    return hip_status(q8::launch_quantize_rows(x, x_row_stride, y, n_rows, k, as_stream(stream)));
}

static int matmul_impl(const q8_0_block *w, const q8_0_block *x, float *y, int32_t *sums,
                       int64_t n, int64_t k, int64_t m, void *stream)
{
    if (int rc = check_k(k)) return rc;
    if (n < 0 || m < 0) return Q8_E_SHAPE;
    if (n == 0 || m == 0) return Q8_OK;
    if (!w || !x || !y) return Q8_E_NULL;
    if (!aligned(w, 2) || !aligned(x, 2) || !aligned(y, 4) || (sums && !aligned(sums, 4)))
        return Q8_E_ALIGN;
    const int64_t nb = k / kQK;
    // many token rows: the matrix-core kernel (weights read once per 128 rows)
    if (m > q8::kStreamMaxM && aligned(w, 16) && aligned(x, 16) && q8::gemm_ok(n, nb, m))
        return hip_status(q8::launch_gemm((const uint8_t *)w, (const uint8_t *)x, y, n, nb, m, n,
                                          as_stream(stream), sums));
    for (int64_t m0 = 0; m0 < m; m0 += q8::kStreamMaxM) {
        const int64_t mc = (m - m0) < q8::kStreamMaxM ? (m - m0) : q8::kStreamMaxM;
        q8::StreamDesc d;
        memset(&d, 0, sizeof(d));
        d.w = (const uint8_t *)w;
        d.x = (const uint8_t *)x + m0 * nb * kBB;
        d.y = y + m0 * n;
        d.sums = sums ? sums + m0 * n * nb : nullptr;
        d.n = n; d.nb = nb; d.m = mc; d.batch = 1;
        d.w_bstride = 0; d.x_bstride = 0; d.y_bstride = 0;
        d.x_rstride = nb * kBB;
        d.y_rstride = n;
        int rc = q8::launch_stream(&d, 1, as_stream(stream));
        if (rc) return hip_status(rc);
    }
    return Q8_OK;
}

int q8_0_matvec(const q8_0_block *w, const q8_0_block *x, float *y, int64_t n, int64_t k,
                void *stream)
{
    return matmul_impl(w, x, y, nullptr, n, k, 1, stream);
}

int q8_0_matmul(const q8_0_block *w, const q8_0_block *x, float *y, int64_t n, int64_t k,
                int64_t m, void *stream)
{
    return matmul_impl(w, x, y, nullptr, n, k, m, stream);
}

int q8_0_matmul_blocksums(const q8_0_block *w, const q8_0_block *x, float *y, int32_t *sums,
                          int64_t n, int64_t k, int64_t m, void *stream)
{
    if (!sums && n > 0 && m > 0) return Q8_E_NULL;
    return matmul_impl(w, x, y, sums, n, k, m, stream);
}

int q8_0_matmul_batched(const q8_0_matmul_desc *descs, int64_t n_desc, void *stream)
{
    if (n_desc < 0) return Q8_E_SHAPE;
    if (n_desc == 0) return Q8_OK;
    if (!descs) return Q8_E_NULL;
    if (n_desc > q8::kStreamMaxJobs) return Q8_E_UNSUPPORTED;
    q8::StreamDesc d[q8::kStreamMaxJobs];
    int nd = 0;
    for (int64_t i = 0; i < n_desc; ++i) {
        const q8_0_matmul_desc &s = descs[i];
        if (int rc = check_k(s.k)) return rc;
        if (s.n < 0 || s.m < 0 || s.batch < 0) return Q8_E_SHAPE;
        if (s.m > q8::kStreamMaxM) return Q8_E_UNSUPPORTED;
        if (s.n == 0 || s.m == 0 || s.batch == 0) continue;
        if (!s.w || !s.x || !s.y) return Q8_E_NULL;
        const int64_t nb = s.k / kQK;
        if (s.m > 1 && (s.x_row_stride < nb || s.y_row_stride < s.n)) return Q8_E_SHAPE;
        // batch entries must not write the same outputs (a common mistake: a
        // zero output batch stride)
        if (s.batch > 1 && (s.w_batch_stride < s.n * nb || s.x_batch_stride < 0 ||
                            s.y_batch_stride < s.n))
            return Q8_E_SHAPE;
        if (!aligned(s.w, 2) || !aligned(s.x, 2) || !aligned(s.y, 4)) return Q8_E_ALIGN;
        q8::StreamDesc &o = d[nd++];
        memset(&o, 0, sizeof(o));
        o.w = (const uint8_t *)s.w;
        o.x = (const uint8_t *)s.x;
        o.y = s.y;
        o.n = s.n; o.nb = nb; o.m = s.m; o.batch = s.batch;
        o.w_bstride = s.w_batch_stride * kBB;
        o.x_rstride = s.x_row_stride * kBB;
        o.x_bstride = s.x_batch_stride * kBB;
        o.y_rstride = s.y_row_stride;
        o.y_bstride = s.y_batch_stride;
    }
    return hip_status(q8::launch_stream(d, nd, as_stream(stream)));
}

}  // extern "C"

// Validation shared by the fp32-activation entry points: fills d[0..nd) with
// the descriptors that have work; step = the one-launch step form (m <= 2).
static int f32_descs(const q8_0_matmul_f32_desc *descs, int64_t n_desc, bool step,
                     q8::StreamDesc *d, int &nd)
{
    nd = 0;
    if (n_desc < 0) return Q8_E_SHAPE;
    if (n_desc == 0) return Q8_OK;
    if (!descs) return Q8_E_NULL;
    if (n_desc > q8::kStreamMaxJobs) return Q8_E_UNSUPPORTED;
    for (int64_t i = 0; i < n_desc; ++i) {
        const q8_0_matmul_f32_desc &s = descs[i];
        if (int rc = check_k(s.k)) return rc;
        if (s.n < 0 || s.m < 0 || s.batch < 0) return Q8_E_SHAPE;
        if (s.m > (step ? 2 : q8::kStreamMaxM)) return Q8_E_UNSUPPORTED;
        if (s.n == 0 || s.m == 0 || s.batch == 0) continue;
        if (!s.w || !s.x || !s.y) return Q8_E_NULL;
        const int64_t nb = s.k / kQK;
        if (s.m > 1 && (s.x_row_stride < s.k || s.y_row_stride < s.n)) return Q8_E_SHAPE;
        if (s.batch > 1 && (s.w_batch_stride < s.n * nb || s.x_batch_stride < 0 ||
                            s.y_batch_stride < s.n))
            return Q8_E_SHAPE;
        if (!aligned(s.w, 16) || !aligned(s.x, 16) || !aligned(s.y, 4) ||
            (s.m > 1 && s.x_row_stride % 4 != 0) || (s.batch > 1 && s.x_batch_stride % 4 != 0))
            return Q8_E_ALIGN;
        q8::StreamDesc &o = d[nd++];
        memset(&o, 0, sizeof(o));
        o.w = (const uint8_t *)s.w;
        o.x = (const uint8_t *)s.x;
        o.y = s.y;
        o.n = s.n; o.nb = nb; o.m = s.m; o.batch = s.batch;
        o.w_bstride = s.w_batch_stride * kBB;
        o.x_rstride = (s.m > 1 ? s.x_row_stride : s.k) * 4;
        o.x_bstride = s.x_batch_stride * 4;
        o.y_rstride = s.y_row_stride;
        o.y_bstride = s.y_batch_stride;
        o.x_f32 = 1;
        // the fused quantization exists in the streaming engines only
        if (step ? !q8::step_ok(o) : !q8::stream_fast_ok(o)) return Q8_E_UNSUPPORTED;
    }
    return Q8_OK;
}

extern "C" {

int q8_0_matmul_f32_batched(const q8_0_matmul_f32_desc *descs, int64_t n_desc, void *stream)
{
    q8::StreamDesc d[q8::kStreamMaxJobs];
    int nd = 0;
    if (int rc = f32_descs(descs, n_desc, false, d, nd)) return rc;
    if (nd == 0) return Q8_OK;
    return hip_status(q8::launch_stream(d, nd, as_stream(stream)));
}

int64_t q8_0_matmul_f32_step_ws_bytes(const q8_0_matmul_f32_desc *descs, int64_t n_desc)
{
    q8::StreamDesc d[q8::kStreamMaxJobs];
    int nd = 0;
    if (int rc = f32_descs(descs, n_desc, true, d, nd)) return rc;
    return (int64_t)q8::step_ws_bytes(d, nd);
}

int q8_0_matmul_f32_step(const q8_0_matmul_f32_desc *descs, int64_t n_desc, void *ws,
                         int64_t ws_bytes, void *stream)
{
    q8::StreamDesc d[q8::kStreamMaxJobs];
    int nd = 0;
    if (int rc = f32_descs(descs, n_desc, true, d, nd)) return rc;
    if (nd == 0) return Q8_OK;
    if (!ws) return Q8_E_WORKSPACE;
    if (!aligned(ws, 256)) return Q8_E_ALIGN;
    if (ws_bytes < 0 || (uint64_t)ws_bytes < q8::step_ws_bytes(d, nd)) return Q8_E_WORKSPACE;
    return hip_status(q8::launch_step(d, nd, ws, as_stream(stream)));
}

int q8_0_up_gate_swiglu_batched(const q8_0_up_gate_desc *descs, int64_t n_desc, void *stream)
{
    if (n_desc < 0) return Q8_E_SHAPE;
    if (n_desc == 0) return Q8_OK;
    if (!descs) return Q8_E_NULL;
    if (n_desc > q8::kStreamMaxJobs) return Q8_E_UNSUPPORTED;
    q8::StreamDesc d[q8::kStreamMaxJobs];
    int nd = 0;
    for (int64_t i = 0; i < n_desc; ++i) {
        const q8_0_up_gate_desc &s = descs[i];
        if (int rc = check_k(s.n_embd)) return rc;
        if (s.n_ff < 0 || s.m < 0 || s.batch < 0) return Q8_E_SHAPE;
        if (s.m > 2) return Q8_E_UNSUPPORTED;
        if (s.n_ff == 0 || s.m == 0 || s.batch == 0) continue;
        if (!s.w || !s.x || !s.h) return Q8_E_NULL;
        const int64_t nb = s.n_embd / kQK;
        if (s.m > 1 && (s.x_row_stride < nb || s.h_row_stride < s.n_ff)) return Q8_E_SHAPE;
        if (s.batch > 1 && (s.w_batch_stride < 2 * s.n_ff * nb || s.x_batch_stride < 0 ||
                            s.h_batch_stride < s.n_ff))
            return Q8_E_SHAPE;
        if (!aligned(s.w, 16) || !aligned(s.x, 2) || !aligned(s.h, 4) ||
            (s.batch > 1 && (s.w_batch_stride * kBB) % 16 != 0))
            return Q8_E_ALIGN;
        q8::StreamDesc &o = d[nd++];
        memset(&o, 0, sizeof(o));
        o.w = (const uint8_t *)s.w;
        o.x = (const uint8_t *)s.x;
        o.y = s.h;
        o.n = s.n_ff; o.nb = nb; o.m = s.m; o.batch = s.batch;
        o.w_bstride = s.w_batch_stride * kBB;
        o.x_rstride = s.x_row_stride * kBB;
        o.x_bstride = s.x_batch_stride * kBB;
        o.y_rstride = s.h_row_stride;
        o.y_bstride = s.h_batch_stride;
        if (!q8::stream_fast_ok(o)) return Q8_E_UNSUPPORTED;
    }
    if (nd == 0) return Q8_OK;
    return hip_status(q8::launch_dense_up_gate(d, nd, as_stream(stream)));
}

// ---------------------------------------------------------------------------
// Mixture of experts

// Shape checks shared by the expert-FFN calls.  Up to 1024 slots any shape
// runs (decode kernels); more tokens take the prefill path, which needs
// n_embd/32 and n_ff/32 to be multiples of 4.
static int moe_check(int64_t n_tok, int64_t n_embd, int64_t n_ff, int64_t n_expert,
                     int64_t n_used)
{
    if (n_tok < 0 || n_expert <= 0 || n_used <= 0) return Q8_E_SHAPE;
    if (check_k(n_embd) || check_k(n_ff)) return Q8_E_SHAPE;
    if (n_used > q8::kMoeMaxUsed) return Q8_E_UNSUPPORTED;
    if (n_expert > q8::kMoeMaxExperts) return Q8_E_UNSUPPORTED;
    if (n_tok * n_used > q8::kMoeMaxSlots && !q8::moe_prefill_ok(n_tok, n_embd, n_ff, n_expert, n_used))
        return Q8_E_UNSUPPORTED;
    return Q8_OK;
}

size_t moe_workspace_bytes(int64_t n_tok, int64_t n_embd, int64_t n_ff, int64_t n_expert,
                           int64_t n_used)
{
    if (moe_check(n_tok, n_embd, n_ff, n_expert, n_used)) return 0;
    return q8::moe_ws_bytes(n_tok, n_embd, n_ff, n_expert, n_used);
}

static int check_up_gate_desc(const moe_up_gate_desc &d, int64_t n_tok, int64_t n_embd,
                              int64_t n_ff, int64_t n_expert, int64_t n_used)
{
    if (!d.ws) return Q8_E_WORKSPACE;
    if (d.ws_bytes < q8::moe_ws_bytes(n_tok, n_embd, n_ff, n_expert, n_used)) return Q8_E_WORKSPACE;
    if (!aligned(d.ws, 256)) return Q8_E_ALIGN;
    if (n_tok > 0 && (!d.w_up_gate || !d.x || !d.ids || !d.h)) return Q8_E_NULL;
    if (!aligned(d.w_up_gate, 16) || !aligned(d.x, 16) || !aligned(d.ids, 4) || !aligned(d.h, 4))
        return Q8_E_ALIGN;
    return Q8_OK;
}

static int check_down_desc(const moe_down_desc &d, int64_t n_tok, int64_t n_embd, int64_t n_ff,
                           int64_t n_expert, int64_t n_used)
{
    if (!d.ws) return Q8_E_WORKSPACE;
    if (d.ws_bytes < q8::moe_ws_bytes(n_tok, n_embd, n_ff, n_expert, n_used)) return Q8_E_WORKSPACE;
    if (!aligned(d.ws, 256)) return Q8_E_ALIGN;
    if (n_tok > 0 && (!d.w_down || !d.h || !d.ids || !d.cw || !d.out)) return Q8_E_NULL;
    if (!aligned(d.w_down, 16) || !aligned(d.h, 16) || !aligned(d.ids, 4) || !aligned(d.cw, 4) ||
        !aligned(d.out, 4))
        return Q8_E_ALIGN;
    return Q8_OK;
}

int moe_up_gate_swiglu_batched(const moe_up_gate_desc *descs, int64_t n_desc, int64_t n_tok,
                               int64_t n_embd, int64_t n_ff, int64_t n_expert, int64_t n_used,
                               void *stream)
{
    if (n_desc < 0) return Q8_E_SHAPE;
    if (n_desc == 0) return Q8_OK;
    if (!descs) return Q8_E_NULL;
    if (int rc = moe_check(n_tok, n_embd, n_ff, n_expert, n_used)) return rc;
    for (int64_t i = 0; i < n_desc; ++i)
        if (int rc = check_up_gate_desc(descs[i], n_tok, n_embd, n_ff, n_expert, n_used)) return rc;
    for (int64_t i0 = 0; i0 < n_desc; i0 += q8::kMoeMaxLayers) {
        q8::MoeUpGateArgs a;
        a.n_layers = (int)std::min<int64_t>(q8::kMoeMaxLayers, n_desc - i0);
        for (int l = 0; l < a.n_layers; ++l) {
            const moe_up_gate_desc &d = descs[i0 + l];
            a.layer[l] = {(const uint8_t *)d.w_up_gate, d.x, d.ids, d.h, d.ws};
        }
        a.n_tok = n_tok; a.n_embd = n_embd; a.n_ff = n_ff; a.n_expert = n_expert;
        a.n_used = n_used;
        if (int rc = hip_status(q8::launch_moe_up_gate(a, as_stream(stream)))) return rc;
    }
    return Q8_OK;
}

int moe_up_gate_swiglu(const q8_0_block *w_up_gate, const float *x, const int32_t *ids,
                       float *h, int64_t n_tok, int64_t n_embd, int64_t n_ff,
                       int64_t n_expert, int64_t n_used, void *ws, size_t ws_bytes,
                       void *stream)
{
    if (int rc = moe_check(n_tok, n_embd, n_ff, n_expert, n_used)) return rc;
    const moe_up_gate_desc d = {w_up_gate, x, ids, h, ws, ws_bytes};
    return moe_up_gate_swiglu_batched(&d, 1, n_tok, n_embd, n_ff, n_expert, n_used, stream);
}

int moe_down_combine_batched(const moe_down_desc *descs, int64_t n_desc, int64_t n_tok,
                             int64_t n_ff, int64_t n_embd, int64_t n_expert, int64_t n_used,
                             void *stream)
{
    if (n_desc < 0) return Q8_E_SHAPE;
    if (n_desc == 0) return Q8_OK;
    if (!descs) return Q8_E_NULL;
    if (int rc = moe_check(n_tok, n_embd, n_ff, n_expert, n_used)) return rc;
    for (int64_t i = 0; i < n_desc; ++i)
        if (int rc = check_down_desc(descs[i], n_tok, n_embd, n_ff, n_expert, n_used)) return rc;
    for (int64_t i0 = 0; i0 < n_desc; i0 += q8::kMoeMaxLayers) {
        q8::MoeDownArgs a;
        a.n_layers = (int)std::min<int64_t>(q8::kMoeMaxLayers, n_desc - i0);
        for (int l = 0; l < a.n_layers; ++l) {
            const moe_down_desc &d = descs[i0 + l];
            a.layer[l] = {(const uint8_t *)d.w_down, d.h, d.ids, d.cw, d.out, d.ws};
        }
        a.n_tok = n_tok; a.n_embd = n_embd; a.n_ff = n_ff; a.n_expert = n_expert;
        a.n_used = n_used;
        if (int rc = hip_status(q8::launch_moe_down(a, as_stream(stream)))) return rc;
    }
    return Q8_OK;
}

int moe_down_combine(const q8_0_block *w_down, const float *h, const int32_t *ids,
                     const float *cw, float *out, int64_t n_tok, int64_t n_ff, int64_t n_embd,
                     int64_t n_expert, int64_t n_used, void *ws, size_t ws_bytes, void *stream)
{
    if (int rc = moe_check(n_tok, n_embd, n_ff, n_expert, n_used)) return rc;
    const moe_down_desc d = {w_down, h, ids, cw, out, ws, ws_bytes};
    return moe_down_combine_batched(&d, 1, n_tok, n_ff, n_embd, n_expert, n_used, stream);
}

// The routing outputs of a validation call: all three or none.
static int route_outputs(const int32_t *counts, const int32_t *offsets, const int32_t *pairs)
{
    const int given = (counts != nullptr) + (offsets != nullptr) + (pairs != nullptr);
    if (given != 0 && given != 3) return Q8_E_NULL;
    if (!aligned(counts, 4) || !aligned(offsets, 4) || !aligned(pairs, 4)) return Q8_E_ALIGN;
    return Q8_OK;
}

int q8v_moe_up_gate(const q8_0_block *w_up_gate, const float *x, const int32_t *ids, float *h,
                    int32_t *sums, int32_t *counts, int32_t *offsets, int32_t *pairs,
                    int64_t n_tok, int64_t n_embd, int64_t n_ff, int64_t n_expert, int64_t n_used,
                    void *ws, size_t ws_bytes, void *stream)
{
    if (int rc = moe_check(n_tok, n_embd, n_ff, n_expert, n_used)) return rc;
    const moe_up_gate_desc d = {w_up_gate, x, ids, h, ws, ws_bytes};
    if (int rc = check_up_gate_desc(d, n_tok, n_embd, n_ff, n_expert, n_used)) return rc;
    if (int rc = route_outputs(counts, offsets, pairs)) return rc;
    if (!aligned(sums, 4)) return Q8_E_ALIGN;
    if (n_tok == 0) return Q8_OK;
    q8::MoeEmit e = {sums, nullptr, counts, offsets, pairs};
    q8::MoeUpGateArgs a;
    a.n_layers = 1;
    a.layer[0] = {(const uint8_t *)w_up_gate, x, ids, h, ws};
    a.n_tok = n_tok; a.n_embd = n_embd; a.n_ff = n_ff; a.n_expert = n_expert; a.n_used = n_used;
    a.emit = &e;
    return hip_status(q8::launch_moe_up_gate(a, as_stream(stream)));
}

int q8v_moe_hq(const q8_0_block *w_down, const float *h, const int32_t *ids, const float *cw,
               float *out, q8_0_block *hq, int32_t *sums, int64_t n_tok, int64_t n_ff,
               int64_t n_embd, int64_t n_expert, int64_t n_used, void *ws, size_t ws_bytes,
               void *stream)
{
    if (int rc = moe_check(n_tok, n_embd, n_ff, n_expert, n_used)) return rc;
    const moe_down_desc d = {w_down, h, ids, cw, out, ws, ws_bytes};
    if (int rc = check_down_desc(d, n_tok, n_embd, n_ff, n_expert, n_used)) return rc;
    if (!aligned(hq, 2) || !aligned(sums, 4)) return Q8_E_ALIGN;
    if (n_tok == 0) return Q8_OK;
    q8::MoeEmit e = {sums, hq, nullptr, nullptr, nullptr};
    q8::MoeDownArgs a;
    a.n_layers = 1;
    a.layer[0] = {(const uint8_t *)w_down, h, ids, cw, out, ws};
    a.n_tok = n_tok; a.n_embd = n_embd; a.n_ff = n_ff; a.n_expert = n_expert; a.n_used = n_used;
    a.emit = &e;
    return hip_status(q8::launch_moe_down(a, as_stream(stream)));
}

int64_t q8_0_r8_bytes(int64_t n, int64_t k)
{
    if (int rc = check_k(k)) return rc;
    if (n < 0) return Q8_E_SHAPE;
    return q8::r8_bytes(n, k / kQK);
}

int q8_0_repack_r8(const q8_0_block *w, void *w_r8, int64_t n, int64_t k, void *stream)
{
    if (int rc = check_k(k)) return rc;
    if (n < 0) return Q8_E_SHAPE;
    if (n == 0) return Q8_OK;
    if (!w || !w_r8) return Q8_E_NULL;
    if (!aligned(w, 2) || !aligned(w_r8, 16)) return Q8_E_ALIGN;
    return hip_status(q8::launch_r8_repack((const uint8_t *)w, (uint8_t *)w_r8, n, k / kQK,
                                           as_stream(stream)));
}

}  // extern "C"

// Validation shared by the R8 entry points; x_f32: activation rows are fp32
// (x_batch_stride in floats) instead of Q8_0 blocks.
static int r8_launch(const void *const *w, const void *const *x, float *const *y,
                     const int64_t *n, const int64_t *k, const int64_t *batch, const int64_t *ws,
                     const int64_t *xs, const int64_t *ys, int64_t n_desc, bool x_f32,
                     int32_t *const *sums, void *stream)
{
    q8::R8Desc d[q8::kStreamMaxJobs];
    int nd = 0;
    for (int64_t i = 0; i < n_desc; ++i) {
        if (int rc = check_k(k[i])) return rc;
        if (n[i] < 0 || batch[i] < 0) return Q8_E_SHAPE;
        if (n[i] == 0 || batch[i] == 0) continue;
        if (!w[i] || !x[i] || !y[i] || (sums && !sums[i])) return Q8_E_NULL;
        const int64_t nb = k[i] / kQK;
        if (batch[i] > 1 && (ws[i] < q8::r8_bytes(n[i], nb) || xs[i] < 0 || ys[i] < n[i]))
            return Q8_E_SHAPE;
        if (sums && !aligned(sums[i], 4)) return Q8_E_ALIGN;
        if (!aligned(w[i], 16) || !aligned(x[i], x_f32 ? 16 : 2) || !aligned(y[i], 4) ||
            (batch[i] > 1 && (ws[i] % 16 != 0 || (x_f32 && xs[i] % 4 != 0))))
            return Q8_E_ALIGN;
        if (!q8::r8_matvec_ok(n[i], nb, batch[i])) return Q8_E_UNSUPPORTED;
        q8::R8Desc &o = d[nd++];
        o.w = (const uint8_t *)w[i];
        o.x = (const uint8_t *)x[i];
        o.y = y[i];
        o.n = n[i]; o.nb = nb; o.batch = batch[i];
        o.w_bstride = batch[i] > 1 ? ws[i] : 0;
        o.x_bstride = batch[i] > 1 ? xs[i] * (x_f32 ? 4 : kBB) : 0;
        o.y_bstride = batch[i] > 1 ? ys[i] : 0;
        o.sums = sums ? sums[i] : nullptr;
    }
    if (nd == 0) return Q8_OK;
    return hip_status(q8::launch_r8_matvec(d, nd, x_f32, as_stream(stream)));
}

template <class Desc>
static int r8_batched(const Desc *descs, int64_t n_desc, bool x_f32, int32_t *const *sums,
                      void *stream)
{
    if (n_desc < 0) return Q8_E_SHAPE;
    if (n_desc == 0) return Q8_OK;
    if (!descs) return Q8_E_NULL;
    if (n_desc > q8::kStreamMaxJobs) return Q8_E_UNSUPPORTED;
    if (sums_required(sums, n_desc)) return Q8_E_NULL;
    const void *w[q8::kStreamMaxJobs], *x[q8::kStreamMaxJobs];
    float *y[q8::kStreamMaxJobs];
    int64_t n[q8::kStreamMaxJobs], k[q8::kStreamMaxJobs], b[q8::kStreamMaxJobs];
    int64_t ws[q8::kStreamMaxJobs], xs[q8::kStreamMaxJobs], ys[q8::kStreamMaxJobs];
    for (int64_t i = 0; i < n_desc; ++i) {
        w[i] = descs[i].w_r8; x[i] = descs[i].x; y[i] = descs[i].y;
        n[i] = descs[i].n; k[i] = descs[i].k; b[i] = descs[i].batch;
        ws[i] = descs[i].w_batch_stride; xs[i] = descs[i].x_batch_stride;
        ys[i] = descs[i].y_batch_stride;
    }
    return r8_launch(w, x, y, n, k, b, ws, xs, ys, n_desc, x_f32, sums, stream);
}

extern "C" {

int q8_0_matvec_r8_batched(const q8_0_r8_desc *descs, int64_t n_desc, void *stream)
{
    return r8_batched(descs, n_desc, false, nullptr, stream);
}

int q8_0_matvec_r8_f32_batched(const q8_0_r8_f32_desc *descs, int64_t n_desc, void *stream)
{
    return r8_batched(descs, n_desc, true, nullptr, stream);
}

int q8v_matvec_r8_batched_blocksums(const q8_0_r8_desc *descs, int64_t n_desc,
                                    int32_t *const *sums, void *stream)
{
    if (n_desc > 0 && !sums) return Q8_E_NULL;
    return r8_batched(descs, n_desc, false, sums, stream);
}

int q8v_matvec_r8_f32_batched_blocksums(const q8_0_r8_f32_desc *descs, int64_t n_desc,
                                        int32_t *const *sums, void *stream)
{
    if (n_desc > 0 && !sums) return Q8_E_NULL;
    return r8_batched(descs, n_desc, true, sums, stream);
}

}  // extern "C"

static int r8_mm_batched(const q8_0_r8_mm_desc *descs, int64_t n_desc, int32_t *const *sums,
                         void *stream)
{
    if (n_desc < 0) return Q8_E_SHAPE;
    if (n_desc == 0) return Q8_OK;
    if (!descs) return Q8_E_NULL;
    if (n_desc > q8::kStreamMaxJobs) return Q8_E_UNSUPPORTED;
    if (sums_required(sums, n_desc)) return Q8_E_NULL;
    q8::R8MmDesc d[q8::kStreamMaxJobs];
    int nd = 0;
    for (int64_t i = 0; i < n_desc; ++i) {
        const q8_0_r8_mm_desc &s = descs[i];
        if (int rc = check_k(s.k)) return rc;
        if (s.n < 0 || s.m < 0 || s.batch < 0) return Q8_E_SHAPE;
        if (s.m > q8::kStreamMaxM) return Q8_E_UNSUPPORTED;
        if (s.n == 0 || s.m == 0 || s.batch == 0) continue;
        if (!s.w_r8 || !s.x || !s.y) return Q8_E_NULL;
        if (sums && !aligned(sums[i], 4)) return Q8_E_ALIGN;
        const int64_t nb = s.k / kQK;
        if (s.m > 1 && (s.x_row_stride < nb || s.y_row_stride < s.n)) return Q8_E_SHAPE;
        if (s.batch > 1 && (s.w_batch_stride < q8::r8_bytes(s.n, nb) || s.x_batch_stride < 0 ||
                            s.y_batch_stride < s.n))
            return Q8_E_SHAPE;
        if (!aligned(s.w_r8, 16) || !aligned(s.x, 2) || !aligned(s.y, 4) ||
            (s.batch > 1 && s.w_batch_stride % 16 != 0))
            return Q8_E_ALIGN;
        if (!q8::r8_mm_ok(s.n, nb, s.m, s.batch)) return Q8_E_UNSUPPORTED;
        q8::R8MmDesc &o = d[nd++];
        o.w = (const uint8_t *)s.w_r8;
        o.x = (const uint8_t *)s.x;
        o.y = s.y;
        o.n = s.n; o.nb = nb; o.m = s.m; o.batch = s.batch;
        o.w_bstride = s.batch > 1 ? s.w_batch_stride : 0;
        o.x_rstride = (s.m > 1 ? s.x_row_stride : nb) * kBB;
        o.x_bstride = s.batch > 1 ? s.x_batch_stride * kBB : 0;
        o.y_rstride = s.m > 1 ? s.y_row_stride : s.n;
        o.y_bstride = s.batch > 1 ? s.y_batch_stride : 0;
        o.sums = sums ? sums[i] : nullptr;
    }
    if (nd == 0) return Q8_OK;
    return hip_status(q8::launch_r8_mm(d, nd, as_stream(stream)));
}

extern "C" {

int q8_0_matmul_r8_batched(const q8_0_r8_mm_desc *descs, int64_t n_desc, void *stream)
{
    return r8_mm_batched(descs, n_desc, nullptr, stream);
}

int q8v_matmul_r8_batched_blocksums(const q8_0_r8_mm_desc *descs, int64_t n_desc,
                                    int32_t *const *sums, void *stream)
{
    if (n_desc > 0 && !sums) return Q8_E_NULL;
    return r8_mm_batched(descs, n_desc, sums, stream);
}

int q8_0_matvec_r8(const void *w_r8, const q8_0_block *x, float *y, int64_t n, int64_t k,
                   void *stream)
{
    const q8_0_r8_desc d = {w_r8, x, y, n, k, 1, 0, 0, 0};
    return q8_0_matvec_r8_batched(&d, 1, stream);
}

int q8_1_quantize_rows(const float *x, int64_t x_row_stride, void *y, int64_t n_rows, int64_t k,
                       void *stream)
{
    if (int rc = check_k(k)) return rc;
    if (n_rows < 0 || x_row_stride < k) return Q8_E_SHAPE;
    if (n_rows == 0) return Q8_OK;
    if (!x || !y) return Q8_E_NULL;
    if (!aligned(x, 16) || x_row_stride % 4 != 0 || !aligned(y, 4)) return Q8_E_ALIGN;
    return hip_status(q8::launch_q8_1_quantize_rows(x, x_row_stride, y, n_rows, k,
                                                    as_stream(stream)));
}

int kq_matvec_batched(int type, const kq_matvec_desc *descs, int64_t n_desc, void *stream)
{
    if (type != 4 && type != 5) return Q8_E_UNSUPPORTED;
    if (n_desc < 0) return Q8_E_SHAPE;
    if (n_desc == 0) return Q8_OK;
    if (!descs) return Q8_E_NULL;
    if (n_desc > q8::kStreamMaxJobs) return Q8_E_UNSUPPORTED;
    const int64_t bb = type == 4 ? 144 : 176;
    q8::KqDesc d[q8::kStreamMaxJobs];
    int nd = 0;
    for (int64_t i = 0; i < n_desc; ++i) {
        const kq_matvec_desc &s = descs[i];
        if (s.k <= 0 || s.k % 256 != 0 || s.n < 0 || s.batch < 0) return Q8_E_SHAPE;
        if (s.n == 0 || s.batch == 0) continue;
        if (!s.w || !s.x || !s.y) return Q8_E_NULL;
        if (s.batch > 1 && (s.w_batch_stride < s.n * (s.k / 256) || s.x_batch_stride < 0 ||
                            s.y_batch_stride < s.n))
            return Q8_E_SHAPE;
        if (!aligned(s.w, 16) || !aligned(s.x, 4) || !aligned(s.y, 4)) return Q8_E_ALIGN;
        if (!q8::kq_matvec_ok(type, s.n, s.k, s.batch)) return Q8_E_UNSUPPORTED;
        q8::KqDesc &o = d[nd++];
        o.w = (const uint8_t *)s.w;
        o.x = (const uint8_t *)s.x;
        o.y = s.y;
        o.n = s.n; o.k = s.k; o.batch = s.batch;
        o.w_bstride = s.batch > 1 ? s.w_batch_stride * bb : 0;
        o.x_bstride = s.batch > 1 ? s.x_batch_stride * 36 : 0;
        o.y_bstride = s.batch > 1 ? s.y_batch_stride : 0;
    }
    if (nd == 0) return Q8_OK;
    return hip_status(q8::launch_kq_matvec(type, d, nd, as_stream(stream)));
}

int q4_k_matvec(const void *w, const void *x, float *y, int64_t n, int64_t k, void *stream)
{
    const kq_matvec_desc d = {w, x, y, n, k, 1, 0, 0, 0};
    return kq_matvec_batched(4, &d, 1, stream);
}

int q5_k_matvec(const void *w, const void *x, float *y, int64_t n, int64_t k, void *stream)
{
    const kq_matvec_desc d = {w, x, y, n, k, 1, 0, 0, 0};
    return kq_matvec_batched(5, &d, 1, stream);
}

size_t moe_r8_workspace_bytes(int64_t n_tok, int64_t n_embd, int64_t n_ff, int64_t n_expert,
                              int64_t n_used)
{
    if (n_tok < 0 || n_expert <= 0 || n_used <= 0 || check_k(n_embd) || check_k(n_ff)) return 0;
    if (!q8::moe_r8_ok(n_tok, n_embd, n_ff, n_expert, n_used)) return 0;
    return q8::moe_r8_ws_bytes(n_tok, n_embd, n_ff, n_expert, n_used);
}

}  // extern "C"

// Checks shared by moe_r8_ffn_batched and its no-alloc variant: the shape,
// every descriptor (its workspace too when with_ws) and the launch-shape
// limits, before anything is enqueued.
static int r8_ffn_checks(const moe_r8_ffn_desc *descs, int64_t n_desc, int64_t n_tok,
                         int64_t n_embd, int64_t n_ff, int64_t n_expert, int64_t n_used,
                         bool with_ws)
{
    if (n_desc < 0 || n_tok < 0 || n_expert <= 0 || n_used <= 0) return Q8_E_SHAPE;
    if (check_k(n_embd) || check_k(n_ff)) return Q8_E_SHAPE;
    if (!q8::moe_r8_ok(n_tok, n_embd, n_ff, n_expert, n_used)) return Q8_E_UNSUPPORTED;
    if (n_desc == 0) return Q8_OK;
    if (!descs) return Q8_E_NULL;
    if (n_desc > 4096) return Q8_E_UNSUPPORTED;
    const size_t need = q8::moe_r8_ws_bytes(n_tok, n_embd, n_ff, n_expert, n_used);
    // more than 16 tokens: h rows are read back with 16-byte loads
    const uintptr_t h_align =
        q8::moe_r8_prefill_path(n_tok, n_embd, n_ff, n_expert, n_used) ? 16 : 4;
    for (int64_t i = 0; i < n_desc; ++i) {
        const moe_r8_ffn_desc &d = descs[i];
        if (with_ws) {
            if (!d.ws) return Q8_E_WORKSPACE;
            if (d.ws_bytes < need) return Q8_E_WORKSPACE;
            if (!aligned(d.ws, 256)) return Q8_E_ALIGN;
        }
        if (n_tok > 0 && (!d.w_up_gate_r8 || !d.w_down_r8 || !d.x || !d.ids || !d.cw || !d.h ||
                          !d.out))
            return Q8_E_NULL;
        if (!aligned(d.w_up_gate_r8, 16) || !aligned(d.w_down_r8, 16) || !aligned(d.x, 16) ||
            !aligned(d.ids, 4) || !aligned(d.cw, 4) || !aligned(d.h, h_align) || !aligned(d.out, 4))
            return Q8_E_ALIGN;
    }
    return q8::moe_r8_ffn_check(n_tok, n_embd, n_ff, n_expert, n_used);
}

// Launches in groups of 64 layers; layer i's workspace is ws_of(i).
template <class WsOf>
static int r8_ffn_launch(const moe_r8_ffn_desc *descs, int64_t n_desc, int64_t n_tok,
                         int64_t n_embd, int64_t n_ff, int64_t n_expert, int64_t n_used,
                         WsOf ws_of, void *stream)
{
    q8::MoeR8Layer l[64];
    for (int64_t i0 = 0; i0 < n_desc; i0 += 64) {
        const int nl = (int)std::min<int64_t>(64, n_desc - i0);
        for (int i = 0; i < nl; ++i) {
            const moe_r8_ffn_desc &d = descs[i0 + i];
            l[i] = {d.w_up_gate_r8, d.w_down_r8, d.x, d.ids, d.cw, d.h, d.out, ws_of(i0 + i)};
        }
        if (int rc = hip_status(q8::launch_moe_r8_ffn(l, nl, n_tok, n_embd, n_ff, n_expert, n_used,
                                                      as_stream(stream))))
            return rc;
    }
    return Q8_OK;
}

extern "C" {

int moe_r8_ffn_batched(const moe_r8_ffn_desc *descs, int64_t n_desc, int64_t n_tok,
                       int64_t n_embd, int64_t n_ff, int64_t n_expert, int64_t n_used,
                       void *stream)
{
    if (int rc = r8_ffn_checks(descs, n_desc, n_tok, n_embd, n_ff, n_expert, n_used, true))
        return rc;
    if (n_desc == 0) return Q8_OK;
    return r8_ffn_launch(descs, n_desc, n_tok, n_embd, n_ff, n_expert, n_used,
                         [&](int64_t i) { return descs[i].ws; }, stream);
}

size_t moe_r8_fused_workspace_bytes(int64_t n_embd, int64_t n_ff, int64_t n_expert, int64_t n_used)
{
    if (n_expert <= 0 || n_used <= 0 || check_k(n_embd) || check_k(n_ff)) return 0;
    if (q8::moe_r8_fused_check(n_embd, n_ff, n_expert, n_used)) return 0;
    return q8::moe_r8_fused_ws_bytes(n_embd, n_ff, n_used);
}

int moe_r8_ffn_fused(const moe_r8_ffn_desc *desc, int64_t n_embd, int64_t n_ff, int64_t n_expert,
                     int64_t n_used, void *stream)
{
    if (n_expert <= 0 || n_used <= 0 || check_k(n_embd) || check_k(n_ff)) return Q8_E_SHAPE;
    if (q8::moe_r8_fused_check(n_embd, n_ff, n_expert, n_used)) return Q8_E_UNSUPPORTED;
    if (!desc) return Q8_E_NULL;
    const moe_r8_ffn_desc &d = *desc;
    if (!d.w_up_gate_r8 || !d.w_down_r8 || !d.x || !d.ids || !d.cw || !d.h || !d.out) return Q8_E_NULL;
    if (!d.ws || d.ws_bytes < q8::moe_r8_fused_ws_bytes(n_embd, n_ff, n_used)) return Q8_E_WORKSPACE;
    if (!aligned(d.ws, 256) || !aligned(d.w_up_gate_r8, 16) || !aligned(d.w_down_r8, 16) ||
        !aligned(d.x, 16) || !aligned(d.ids, 4) || !aligned(d.cw, 4) || !aligned(d.h, 4) ||
        !aligned(d.out, 4))
        return Q8_E_ALIGN;
    const q8::MoeR8Layer l = {d.w_up_gate_r8, d.w_down_r8, d.x, d.ids, d.cw, d.h, d.out, d.ws};
    return hip_status(q8::launch_moe_r8_fused(l, n_embd, n_ff, n_expert, n_used, as_stream(stream)));
}

int q8v_moe_r8_ffn(const moe_r8_ffn_desc *desc, int64_t n_tok, int64_t n_embd, int64_t n_ff,
                   int64_t n_expert, int64_t n_used, int32_t *ug_sums, int32_t *dn_sums,
                   q8_0_block *hq, int32_t *counts, int32_t *offsets, int32_t *pairs,
                   void *stream)
{
    if (int rc = r8_ffn_checks(desc, 1, n_tok, n_embd, n_ff, n_expert, n_used, true)) return rc;
    if (int rc = route_outputs(counts, offsets, pairs)) return rc;
    if (!aligned(ug_sums, 4) || !aligned(dn_sums, 4) || !aligned(hq, 2)) return Q8_E_ALIGN;
    // one token: every slot is served on its own, no grouping to report
    if (counts && n_tok == 1) return Q8_E_UNSUPPORTED;
    if (n_tok == 0) return Q8_OK;
    q8::MoeEmit eu = {ug_sums, nullptr, counts, offsets, pairs};
    q8::MoeEmit ed = {dn_sums, hq, nullptr, nullptr, nullptr};
    const q8::MoeR8Layer l = {desc->w_up_gate_r8, desc->w_down_r8, desc->x, desc->ids, desc->cw,
                              desc->h, desc->out, desc->ws};
    return hip_status(q8::launch_moe_r8_ffn(&l, 1, n_tok, n_embd, n_ff, n_expert, n_used,
                                            as_stream(stream), &eu, &ed));
}

int moe_r8_ffn_batched_noalloc(const moe_r8_ffn_desc *descs, int64_t n_desc, int64_t n_tok,
                               int64_t n_embd, int64_t n_ff, int64_t n_expert, int64_t n_used,
                               void *stream)
{
    if (int rc = r8_ffn_checks(descs, n_desc, n_tok, n_embd, n_ff, n_expert, n_used, false))
        return rc;
    if (n_desc == 0 || n_tok == 0) return Q8_OK;
    // decode shapes only: the prefill path's workspace is far larger
    if (q8::moe_r8_prefill_path(n_tok, n_embd, n_ff, n_expert, n_used)) return Q8_E_UNSUPPORTED;
    const size_t per = (q8::moe_r8_ws_bytes(n_tok, n_embd, n_ff, n_expert, n_used) + 255) &
                       ~(size_t)255;
    if ((uint64_t)n_desc * per > q8::kMoeR8ScratchBytes) return Q8_E_WORKSPACE;
    uint8_t *base = nullptr;
    if (q8::moe_r8_scratch(&base)) return Q8_E_HIP;
    return r8_ffn_launch(descs, n_desc, n_tok, n_embd, n_ff, n_expert, n_used,
                         [&](int64_t i) { return (void *)(base + i * per); }, stream);
}

int q8_read_probe(const void *p, int64_t bytes, uint32_t *sink, int64_t sink_words, void *stream)
{
    if (bytes < 0 || sink_words < 0) return Q8_E_SHAPE;
    if (bytes == 0) return Q8_OK;
    if (!p || !sink) return Q8_E_NULL;
    if (!aligned(p, 16) || bytes % 16 != 0 || !aligned(sink, 4)) return Q8_E_ALIGN;
    return hip_status(q8::launch_read_probe(p, bytes, sink, sink_words, as_stream(stream)));
}

int moe_route(const int32_t *ids, int32_t *counts, int32_t *offsets, int32_t *pairs,
              int64_t n_tok, int64_t n_expert, int64_t n_used, void *ws, size_t ws_bytes,
              void *stream)
{
    if (n_tok < 0 || n_expert <= 0 || n_used <= 0) return Q8_E_SHAPE;
    if (n_used > q8::kMoeMaxUsed || n_tok * n_used > q8::kMoeMaxSlots ||
        n_expert > q8::kMoeMaxExperts)
        return Q8_E_UNSUPPORTED;
    if (!ws) return Q8_E_WORKSPACE;
    if (ws_bytes < 256) return Q8_E_WORKSPACE;
    if (!aligned(ws, 256)) return Q8_E_ALIGN;
    if (!counts || !offsets || (n_tok > 0 && (!ids || !pairs))) return Q8_E_NULL;
    if (!aligned(ids, 4) || !aligned(counts, 4) || !aligned(offsets, 4) || !aligned(pairs, 4))
        return Q8_E_ALIGN;
    return hip_status(q8::launch_moe_route(ids, counts, offsets, pairs, n_tok, n_expert, n_used,
                                           ws, as_stream(stream)));
}

}  // extern "C"
