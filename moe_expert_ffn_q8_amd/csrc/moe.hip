// moe.hip -- the expert FFN of a mixture-of-experts layer on gfx950.
//
// What is computed (Gemma-4-on-Xeon page, "GPUなしで13年前のXeon上でGemma 4
// 26Bを毎秒5トークンで実行する": the section on the broken op paths shows the
// expert FFN with 8 active experts per token; the three-part fix, runtime graph
// fallback, gives the combined up_gate tensor [n_embd, 2*n_ff, n_expert] with
// the gate half first, its split into two mul_mat_id products, and
// fused_mul_unary(gate, up, SILU)):
//   h[t][u][j] = silu(W_ug[e][j] . x_t) * (W_ug[e][n_ff+j] . x_t),  e = ids[t][u]
//   out[t]     = sum_u cw[t][u] * (W_d[e] . q(h[t][u]))
//
// Design:
//  * Expert-major gather.  Workgroups are laid out as (slot, part).  The
//    workgroup of slot s reads e = ids[s], issues its first weight loads at
//    once, and with one ballot pass over the ids decides whether s is the first
//    slot naming e; if so it serves every slot routed to e (ascending (t,u)
//    order), otherwise it exits.  So no routing kernel and no host sync are
//    needed, and each active expert's rows are streamed from HBM once per call
//    for all of its slots.
//  * The weight tiles go through the same engine as the decode products
//    (coalesced 16-byte loads -> per-wave LDS slot -> one 4-block quad per
//    lane, v_dot4 against a masked activation image).
//  * up_gate: a wave-tile pairs R gate rows with the same R up rows, so SwiGLU
//    is applied in the epilogue on the reduced dot products; no second pass.
//  * down: the workgroup quantizes the h rows of its expert's slots straight
//    into the masked image (same rule and code as the activation quantizer),
//    writes per-slot outputs to the workspace, and a small kernel combines the
//    n_used slot outputs of each token in ascending u order (deterministic).
//    For few slots (decode at one or two tokens) a row-major kernel instead
//    streams a row band of every slot's expert and combines in LDS: one launch.
//  * Ids outside [0, n_expert) never match an expert; workgroup 0 records them
//    in the error word of the workspace and writes NaN into what they would
//    have produced.
#include "q8_device.h"
#include "q8_internal.h"
#include "q8_moe.h"

namespace q8 {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;

struct PickShared {
    int invalid;
    int expert;
    int count;
    int pad;
    int slots[kMoeMaxSlots];
};

// Build the ascending list of slots routed to expert e with one wave (ballot
// compaction in slot order).  Returns the count (valid in that wave).
__device__ int build_slot_list(const int32_t *ids, int n_slots, int e, int *list, int lane)
{
    int cnt = 0;
    for (int base = 0; base < n_slots; base += kWave) {
        const int s = base + lane;
        const bool pred = s < n_slots && ids[s] == e;
        const uint64_t mask = __ballot(pred);
        if (pred) list[cnt + __popcll(mask & __lanemask_lt())] = s;
        cnt += __popcll(mask);
    }
    return cnt;
}

// Workgroup for slot s with expert e = ids[s]: the workgroup owns the expert
// when e is in range and s is the first slot that names it; it then serves
// every slot routed to e (listed in ascending (t,u) order).  One ballot pass
// of wave 0 over the ids finds ownership, the slot list and whether any id is
// out of range.  Sets ps.expert (-1: nothing to do), ps.count, ps.slots,
// ps.invalid; ends with a workgroup barrier.
__device__ void pick_by_slot(const int32_t *ids, int n_slots, int n_expert, int s, int e,
                             PickShared &ps)
{
    const int tid = threadIdx.x;
    if (tid < kWave) {
        int cnt = 0;
        bool first = true, bad = false;
        for (int base = 0; base < n_slots; base += kWave) {
            const int i = base + tid;
            const bool in = i < n_slots;
            const int v = in ? ids[i] : 0;
            bad |= __ballot(in && (v < 0 || v >= n_expert)) != 0;
            const bool hit = in && v == e;
            const uint64_t m = __ballot(hit);
            first &= __ballot(hit && i < s) == 0;
            if (hit) ps.slots[cnt + __popcll(m & __lanemask_lt())] = i;
            cnt += __popcll(m);
        }
        if (tid == 0) {
            ps.invalid = bad ? 1 : 0;
            ps.expert = (e >= 0 && e < n_expert && first) ? e : -1;
            ps.count = cnt;
        }
    }
    __syncthreads();
}

// Quantize mc fp32 rows (row m starts at base + row_index[m] * row_floats)
// into the masked image (nb*34 bytes per row, scale bytes zero) plus fp32
// scales, with the activation quantization rule (same code as the quantizer:
// the bytes equal q8_0_quantize_rows of those rows).  All threads of the
// workgroup take part; 8 lanes per block.
__device__ void quantize_rows_to_image(const float *base, int64_t row_floats, const int *row_index,
                                       int mc, int nb, uint8_t *ximg, float *xsc)
{
    const int tid = threadIdx.x;
    const int li = tid & 7;
    const int img_row = nb * kBlockBytes;
    const int step = (int)blockDim.x / 8;
    for (int bi = tid >> 3; bi < mc * nb; bi += step) {
        const int m = bi / nb;
        const int b = bi - m * nb;
        const float4 v = *(const float4 *)(base + (int64_t)row_index[m] * row_floats + b * kQK + 4 * li);
        uint32_t codes, dbits;
        quantize_block8(v.x, v.y, v.z, v.w, codes, dbits);
        uint16_t *img16 = (uint16_t *)(ximg + m * img_row);
        if (li == 0) {
            img16[b * 17] = 0;
            xsc[m * nb + b] = half_bits_to_float(dbits);
        }
        img16[b * 17 + 1 + 2 * li] = (uint16_t)(codes & 0xffffu);
        img16[b * 17 + 2 + 2 * li] = (uint16_t)(codes >> 16);
    }
}

struct UgParams {
    const uint8_t *w;
    const float *x;        // fp32 [n_tok][n_embd]
    const int32_t *ids;
    float *h;
    int32_t *err;
    int n_slots, n_used, n_expert, nb, n_ff;
    int R;                 // rows per wave-tile
    int tiles_per_expert;  // ceil(n_ff / R)
    int wgs_per_expert;
    int tiles_per_wg;
};

template <int MT>
__global__ __launch_bounds__(kThreads) void moe_up_gate_kernel(const UgParams p)
{
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int nb = p.nb;
    const int Q = nb >> 2;
    const int img_row = nb * kBlockBytes;

    uint8_t *stage = smem + wave * kStageBytes;
    float *redg = (float *)(smem + kWaves * kStageBytes) + wave * 2 * MT * kWave;
    float *redu = redg + MT * kWave;
    uint8_t *ximg = smem + kWaves * kStageBytes + kWaves * 2 * MT * kWave * 4;
    float *xsc = (float *)(ximg + MT * img_row);
    PickShared &ps = *(PickShared *)(xsc + MT * nb);
    int *rows_of = (int *)(&ps + 1);     // MT token rows of the current chunk

    const int slot = blockIdx.x / p.wgs_per_expert;
    const int part = blockIdx.x - slot * p.wgs_per_expert;
    const int e0 = p.ids[slot];
    const bool e0_ok = e0 >= 0 && e0 < p.n_expert;
    const int64_t row_bytes = (int64_t)nb * kBlockBytes;
    const uint8_t *We = p.w + (int64_t)(e0_ok ? e0 : 0) * 2 * p.n_ff * row_bytes;
    const int t0 = part * p.tiles_per_wg;
    const int t1 = min(t0 + p.tiles_per_wg, p.tiles_per_expert);
    const int c = lane % Q;

    // The wave walks a sequence of half-tiles (gate rows of tile t, up rows of
    // tile t, gate rows of tile t+4, ...) with one half-tile of loads in
    // flight ahead of the one being computed.
    u32x4 g[kTileLoads];
    auto issue = [&](int tt, bool up) {
        const int j0 = tt * p.R;
        const int rows = min(p.R, p.n_ff - j0);
        tile_issue(We + (int64_t)((up ? p.n_ff : 0) + j0) * row_bytes, rows * nb * 17 / 8, lane, g);
    };
    // the first half-tile depends only on ids[slot]: issue it before the scan
    // and the activation round trip (dropped if another slot owns the expert)
    if (e0_ok && t0 + wave < t1) issue(t0 + wave, false);
    pick_by_slot(p.ids, p.n_slots, p.n_expert, slot, e0, ps);

    if (blockIdx.x == 0) {
        if (tid == 0) *p.err = ps.invalid ? 1 : 0;
        if (ps.invalid) {
            for (int s = 0; s < p.n_slots; ++s) {
                const int e = p.ids[s];
                if (e < 0 || e >= p.n_expert)
                    for (int j = tid; j < p.n_ff; j += kThreads)
                        p.h[(int64_t)s * p.n_ff + j] = __builtin_nanf("");
            }
        }
    }
    if (ps.expert < 0) return;
    const int count = ps.count;

    for (int c0 = 0; c0 < count; c0 += MT) {
        const int mc = min(MT, count - c0);
        __syncthreads();
        if (tid < mc) rows_of[tid] = ps.slots[c0 + tid] / p.n_used;
        // later chunks restart the tile walk: issue its first half-tile now
        if (c0 > 0 && t0 + wave < t1) issue(t0 + wave, false);
        __syncthreads();
        quantize_rows_to_image(p.x, (int64_t)nb * kQK, rows_of, mc, nb, ximg, xsc);
        __syncthreads();

        uint32_t xr[kQuadDwords];
        float4 xd1 = make_float4(0.f, 0.f, 0.f, 0.f);
        if (MT == 1) {
            lds_quad(ximg + kQuadBytes * c, xr);
            xd1 = *(const float4 *)(xsc + 4 * c);
        }

        for (int t = t0 + wave; t < t1; t += kWaves) {
            const int j0 = t * p.R;
            const int rows = min(p.R, p.n_ff - j0);
            const int live = rows * Q;
#pragma unroll 1
            for (int half = 0; half < 2; ++half) {
                uint32_t wq[kQuadDwords];
                tile_to_quad(stage, g, lane, live, wq);
                if (half == 0) issue(t, true);
                else if (t + kWaves < t1) issue(t + kWaves, false);
                float dw0, dw1, dw2, dw3;
                quad_scales(wq, dw0, dw1, dw2, dw3);
                float *red = half == 0 ? redg : redu;
#pragma unroll 1
                for (int m = 0; m < mc; ++m) {
                    uint32_t xt[kQuadDwords];
                    const uint32_t *xq = xr;
                    float4 dx = xd1;
                    if (MT != 1) {
                        lds_quad(ximg + m * img_row + kQuadBytes * c, xt);
                        xq = xt;
                        dx = *(const float4 *)(xsc + m * nb + 4 * c);
                    }
                    int sb[4];
                    const float acc = quad_dot(wq, xq, dw0, dw1, dw2, dw3, dx, sb);
                    red[m * kWave + lane] = (lane < live) ? acc : 0.0f;
                }
            }
            wave_lds_sync();
            for (int i = lane; i < rows * mc; i += kWave) {
                const int m = i / rows;
                const int r = i - m * rows;
                const float *pg = redg + m * kWave + r * Q;
                const float *pu = redu + m * kWave + r * Q;
                float gs = pg[0], us = pu[0];
                for (int cc = 1; cc < Q; ++cc) {
                    gs += pg[cc];
                    us += pu[cc];
                }
                const float hv = gs / (1.0f + expf(-gs)) * us;
                p.h[(int64_t)ps.slots[c0 + m] * p.n_ff + j0 + r] = hv;
            }
            wave_lds_sync();
        }
    }
}

struct DnParams {
    const uint8_t *w;
    const float *h;
    const int32_t *ids;
    float *yslot;        // [n_slots][n_rows]
    int32_t *err;
    int n_slots, n_used, n_expert, nb, n_ff, n_rows;
    int R, tiles_per_expert, wgs_per_expert, tiles_per_wg;
};

template <int MT>
__global__ __launch_bounds__(kThreads) void moe_down_kernel(const DnParams p)
{
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int nb = p.nb;
    const int Q = nb >> 2;
    const int img_row = nb * kBlockBytes;

    uint8_t *stage = smem + wave * kStageBytes;
    float *red = (float *)(smem + kWaves * kStageBytes) + wave * MT * kWave;
    uint8_t *ximg = smem + kWaves * kStageBytes + kWaves * MT * kWave * 4;
    float *xsc = (float *)(ximg + MT * img_row);
    PickShared &ps = *(PickShared *)(xsc + MT * nb);

    const int slot = blockIdx.x / p.wgs_per_expert;
    const int part = blockIdx.x - slot * p.wgs_per_expert;
    const int e0 = p.ids[slot];
    const bool e0_ok = e0 >= 0 && e0 < p.n_expert;
    const int64_t row_bytes = (int64_t)nb * kBlockBytes;
    const uint8_t *We = p.w + (int64_t)(e0_ok ? e0 : 0) * p.n_rows * row_bytes;
    const int t0 = part * p.tiles_per_wg;
    const int t1 = min(t0 + p.tiles_per_wg, p.tiles_per_expert);
    const int c = lane % Q;

    u32x4 g[kTileLoads];
    auto issue = [&](int tt) {
        const int r0 = tt * p.R;
        tile_issue(We + (int64_t)r0 * row_bytes, min(p.R, p.n_rows - r0) * nb * 17 / 8, lane, g);
    };
    // depends only on ids[slot]: issue before the scan and the h round trip
    if (e0_ok && t0 + wave < t1) issue(t0 + wave);
    pick_by_slot(p.ids, p.n_slots, p.n_expert, slot, e0, ps);
    if (blockIdx.x == 0 && tid == 0) *p.err = ps.invalid ? 1 : 0;
    if (ps.expert < 0) return;
    const int count = ps.count;

    for (int c0 = 0; c0 < count; c0 += MT) {
        const int mc = min(MT, count - c0);
        int t = t0 + wave;
        if (c0 > 0 && t < t1) issue(t);
        __syncthreads();
        // quantize the h rows of this chunk's slots into the masked image
        quantize_rows_to_image(p.h, p.n_ff, ps.slots + c0, mc, nb, ximg, xsc);
        __syncthreads();

        uint32_t xr[kQuadDwords];
        float4 xd1 = make_float4(0.f, 0.f, 0.f, 0.f);
        if (MT == 1) {
            lds_quad(ximg + kQuadBytes * c, xr);
            xd1 = *(const float4 *)(xsc + 4 * c);
        }

        for (; t < t1; t += kWaves) {
            const int row0 = t * p.R;
            const int rows = min(p.R, p.n_rows - row0);
            const int live = rows * Q;
            uint32_t wq[kQuadDwords];
            tile_to_quad(stage, g, lane, live, wq);
            if (t + kWaves < t1) issue(t + kWaves);
            float dw0, dw1, dw2, dw3;
            quad_scales(wq, dw0, dw1, dw2, dw3);
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                if (m < mc) {
                    uint32_t xt[kQuadDwords];
                    const uint32_t *xq = xr;
                    float4 dx = xd1;
                    if (MT != 1) {
                        lds_quad(ximg + m * img_row + kQuadBytes * c, xt);
                        xq = xt;
                        dx = *(const float4 *)(xsc + m * nb + 4 * c);
                    }
                    int s[4];
                    const float acc = quad_dot(wq, xq, dw0, dw1, dw2, dw3, dx, s);
                    red[m * kWave + lane] = (lane < live) ? acc : 0.0f;
                }
            }
            wave_lds_sync();
            for (int i = lane; i < rows * mc; i += kWave) {
                const int m = i / rows;
                const int r = i - m * rows;
                const float *pr = red + m * kWave + r * Q;
                float acc = pr[0];
                for (int cc = 1; cc < Q; ++cc) acc += pr[cc];
                p.yslot[(int64_t)ps.slots[c0 + m] * p.n_rows + row0 + r] = acc;
            }
            wave_lds_sync();
        }
    }
}

// Row-major down projection with the combine fused in (small slot counts,
// i.e. decode at one or two tokens).  A workgroup owns R output rows for all
// slots: wave w streams those rows of the experts of slots w, w + kRowWaves,
// ..., the per-slot results meet in LDS and the workgroup writes
//   out[t][row] = sum over u ascending of cw[t][u] * y[t*n_used+u][row]
// directly: no workspace round trip and no combine launch.  Every workgroup
// quantizes all slots' h rows into its LDS image (same rule as the quantizer).
constexpr int kRowWaves = 8;
constexpr int kRowThreads = kRowWaves * kWave;
constexpr int kRowsMaxSlots = 16;

struct DrParams {
    const uint8_t *w;
    const float *h;
    const int32_t *ids;
    const float *cw;
    float *out;
    int32_t *err;
    int n_used, n_slots, n_expert, nb, n_ff, n_rows, R;
};

__global__ __launch_bounds__(kRowThreads) void moe_down_rows_kernel(const DrParams p)
{
    extern __shared__ __align__(16) uint8_t smem[];
    __shared__ int s_e[kRowsMaxSlots];
    __shared__ int s_rows[kRowsMaxSlots];
    __shared__ float ys[kRowsMaxSlots][kWave];
    __shared__ float red[kRowWaves][kWave];
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int nb = p.nb;
    const int Q = nb >> 2;
    const int img_row = nb * kBlockBytes;
    uint8_t *stage = smem + wave * kStageBytes;
    uint8_t *ximg = smem + kRowWaves * kStageBytes;
    float *xsc = (float *)(ximg + kRowsMaxSlots * img_row);

    const int row0 = blockIdx.x * p.R;
    const int rows = min(p.R, p.n_rows - row0);
    const int live = rows * Q;
    const int c = lane % Q;
    const int64_t row_bytes = (int64_t)nb * kBlockBytes;

    u32x4 g[kTileLoads];
    auto issue_e = [&](int e) {
        const uint8_t *base = p.w + ((int64_t)e * p.n_rows + row0) * row_bytes;
        tile_issue(base, rows * nb * 17 / 8, lane, g);
    };
    // this wave's first slot's weights depend only on its id: issue them before
    // anything else
    const int e_first = wave < p.n_slots ? p.ids[wave] : -1;
    const bool first_ok = e_first >= 0 && e_first < p.n_expert;
    if (first_ok) issue_e(e_first);

    if (tid < p.n_slots) {
        const int e = p.ids[tid];
        s_e[tid] = (e >= 0 && e < p.n_expert) ? e : -1;
        s_rows[tid] = tid;
    }
    __syncthreads();
    if (blockIdx.x == 0 && tid == 0) {
        int bad = 0;
        for (int s = 0; s < p.n_slots; ++s) bad |= (s_e[s] < 0);
        *p.err = bad;
    }

    auto next_slot = [&](int s) {
        while (s < p.n_slots && s_e[s] < 0) s += kRowWaves;
        return s;
    };
    int s = next_slot(wave);
    if (!first_ok && s < p.n_slots) issue_e(s_e[s]);

    quantize_rows_to_image(p.h, p.n_ff, s_rows, p.n_slots, nb, ximg, xsc);
    __syncthreads();

    while (s < p.n_slots) {
        uint32_t wq[kQuadDwords];
        tile_to_quad(stage, g, lane, live, wq);
        const int sn = next_slot(s + kRowWaves);
        if (sn < p.n_slots) issue_e(s_e[sn]);
        float dw0, dw1, dw2, dw3;
        quad_scales(wq, dw0, dw1, dw2, dw3);
        uint32_t xq[kQuadDwords];
        lds_quad(ximg + s * img_row + kQuadBytes * c, xq);
        const float4 dx = *(const float4 *)(xsc + s * nb + 4 * c);
        int sb[4];
        const float acc = quad_dot(wq, xq, dw0, dw1, dw2, dw3, dx, sb);
        red[wave][lane] = (lane < live) ? acc : 0.0f;
        wave_lds_sync();
        if (lane < rows) {
            const float *pr = &red[wave][lane * Q];
            float y = pr[0];
            for (int cc = 1; cc < Q; ++cc) y += pr[cc];
            ys[s][lane] = y;
        }
        wave_lds_sync();
        s = sn;
    }
    __syncthreads();

    const int n_tok = p.n_slots / p.n_used;
    for (int i = tid; i < n_tok * rows; i += kRowThreads) {
        const int t = i / rows;
        const int r = i - t * rows;
        bool bad = false;
        for (int u = 0; u < p.n_used; ++u) bad |= (s_e[t * p.n_used + u] < 0);
        float acc;
        if (bad) {
            acc = __builtin_nanf("");
        } else {
            acc = p.cw[t * p.n_used] * ys[t * p.n_used][r];
            for (int u = 1; u < p.n_used; ++u)
                acc = fmaf(p.cw[t * p.n_used + u], ys[t * p.n_used + u][r], acc);
        }
        p.out[(int64_t)t * p.n_rows + row0 + r] = acc;
    }
}

// out[t][n] = sum over u ascending of cw[t][u] * yslot[t*n_used+u][n]; a token
// with an out-of-range id gets NaN.
__global__ __launch_bounds__(256) void moe_combine_kernel(const float *__restrict__ yslot,
                                                          const int32_t *__restrict__ ids,
                                                          const float *__restrict__ cw,
                                                          float *__restrict__ out, int n_rows,
                                                          int n_used, int n_expert)
{
    const int t = blockIdx.y;
    const int n = blockIdx.x * 256 + threadIdx.x;
    if (n >= n_rows) return;
    bool bad = false;
    for (int u = 0; u < n_used; ++u) {
        const int e = ids[t * n_used + u];
        bad |= (e < 0 || e >= n_expert);
    }
    float acc;
    if (bad) {
        acc = __builtin_nanf("");
    } else {
        const float *y = yslot + (int64_t)t * n_used * n_rows + n;
        acc = cw[t * n_used] * y[0];
        for (int u = 1; u < n_used; ++u) acc = fmaf(cw[t * n_used + u], y[(int64_t)u * n_rows], acc);
    }
    out[(int64_t)t * n_rows + n] = acc;
}

__global__ __launch_bounds__(kThreads) void moe_route_kernel(const int32_t *ids, int32_t *counts,
                                                             int32_t *offsets, int32_t *pairs,
                                                             int n_slots, int n_expert,
                                                             int32_t *err)
{
    __shared__ int invalid;
    const int tid = threadIdx.x;
    if (tid == 0) invalid = 0;
    __syncthreads();
    for (int s = tid; s < n_slots; s += kThreads) {
        const int e = ids[s];
        if (e < 0 || e >= n_expert) atomicOr(&invalid, 1);
    }
    __syncthreads();
    if (tid == 0) *err = invalid ? 1 : 0;
    if (tid >= kWave) return;
    int pos = 0;
    for (int e = 0; e < n_expert; ++e) {
        const int cnt = build_slot_list(ids, n_slots, e, pairs + pos, tid);
        if (tid == 0) {
            counts[e] = cnt;
            offsets[e] = pos;
        }
        pos += cnt;
    }
    if (tid == 0) offsets[n_expert] = pos;
}

// ---------------------------------------------------------------------------
// Generic expert kernels: any n_embd, n_ff that are multiples of 32 (used when
// the block count per row is not a multiple of 8 or exceeds the fast path's
// limit).  One wave per (slot, row); lanes stride over blocks with 2-byte
// loads; fixed-order xor-tree reduction.

__device__ __forceinline__ float generic_row_dot(const uint8_t *w, const uint8_t *x, int nb,
                                                 int lane)
{
    float acc = 0.0f;
    for (int b = lane; b < nb; b += kWave) {
        const uint8_t *wb = w + b * kBlockBytes;
        const uint8_t *xb = x + b * kBlockBytes;
        int s = 0;
        for (int hh = 1; hh < 17; ++hh) {
            const uint32_t wv = load_u16(wb + 2 * hh);
            const uint32_t xv = load_u16(xb + 2 * hh);
            s += (int)(int8_t)(wv & 0xff) * (int)(int8_t)(xv & 0xff);
            s += (int)(int8_t)(wv >> 8) * (int)(int8_t)(xv >> 8);
        }
        acc = fmaf(half_bits_to_float(load_u16(wb)) * half_bits_to_float(load_u16(xb)),
                   (float)s, acc);
    }
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    return acc;
}

__device__ __forceinline__ void generic_flag_invalid(const int32_t *ids, int n_slots,
                                                     int n_expert, int32_t *err)
{
    if (blockIdx.x != 0 || blockIdx.y != 0 || threadIdx.x != 0) return;
    int bad = 0;
    for (int s = 0; s < n_slots; ++s) bad |= (ids[s] < 0 || ids[s] >= n_expert);
    *err = bad;
}

// grid (n_slots, ceil(n_ff / 4)); 4 waves, one j each.  The slot's token row
// is quantized into LDS first (same rule and code as the quantizer).
__device__ void quantize_row_to_blocks(const float *src, int nb, uint8_t *dst)
{
    const int tid = threadIdx.x;
    for (int bi = tid >> 3; bi < nb; bi += kThreads / 8) {
        const int li = tid & 7;
        const float4 v = *(const float4 *)(src + bi * kQK + 4 * li);
        uint32_t codes, dbits;
        quantize_block8(v.x, v.y, v.z, v.w, codes, dbits);
        uint16_t *b16 = (uint16_t *)(dst + bi * kBlockBytes);
        if (li == 0) b16[0] = (uint16_t)dbits;
        b16[1 + 2 * li] = (uint16_t)(codes & 0xffffu);
        b16[2 + 2 * li] = (uint16_t)(codes >> 16);
    }
}

__global__ __launch_bounds__(kThreads) void moe_up_gate_generic_kernel(UgParams p)
{
    extern __shared__ __align__(16) uint8_t xq[];      // nb blocks of 34 B
    generic_flag_invalid(p.ids, p.n_slots, p.n_expert, p.err);
    const int s = blockIdx.x;
    const int e = p.ids[s];
    quantize_row_to_blocks(p.x + (int64_t)(s / p.n_used) * p.nb * kQK, p.nb, xq);
    __syncthreads();
    const int j = blockIdx.y * kWaves + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (j >= p.n_ff) return;
    float *dst = p.h + (int64_t)s * p.n_ff + j;
    if (e < 0 || e >= p.n_expert) {
        if (lane == 0) *dst = __builtin_nanf("");
        return;
    }
    const int64_t row_bytes = (int64_t)p.nb * kBlockBytes;
    const uint8_t *We = p.w + (int64_t)e * 2 * p.n_ff * row_bytes;
    const uint8_t *xr = xq;
    const float g = generic_row_dot(We + (int64_t)j * row_bytes, xr, p.nb, lane);
    const float u = generic_row_dot(We + (int64_t)(p.n_ff + j) * row_bytes, xr, p.nb, lane);
    if (lane == 0) *dst = g / (1.0f + expf(-g)) * u;
}

// grid (n_slots, ceil(n_rows / 4)); the slot's h row is quantized into LDS
// first (same rule and code as the activation quantizer).
__global__ __launch_bounds__(kThreads) void moe_down_generic_kernel(DnParams p)
{
    extern __shared__ __align__(16) uint8_t hq[];      // nb blocks of 34 B
    generic_flag_invalid(p.ids, p.n_slots, p.n_expert, p.err);
    const int s = blockIdx.x;
    const int e = p.ids[s];
    if (e < 0 || e >= p.n_expert) return;              // the combine writes NaN
    const int tid = threadIdx.x;
    quantize_row_to_blocks(p.h + (int64_t)s * p.n_ff, p.nb, hq);
    __syncthreads();
    const int row = blockIdx.y * kWaves + (tid >> 6);
    const int lane = tid & 63;
    if (row >= p.n_rows) return;
    const int64_t row_bytes = (int64_t)p.nb * kBlockBytes;
    const uint8_t *wr = p.w + ((int64_t)e * p.n_rows + row) * row_bytes;
    const float y = generic_row_dot(wr, hq, p.nb, lane);
    if (lane == 0) p.yslot[(int64_t)s * p.n_rows + row] = y;
}

int pick_mt(int64_t n_tok)
{
    if (n_tok <= 1) return 1;
    if (n_tok <= 2) return 2;
    return 4;
}

}  // namespace

size_t moe_ws_bytes(int64_t n_tok, int64_t n_embd, int64_t n_ff, int64_t n_expert,
                    int64_t n_used)
{
    (void)n_ff;
    (void)n_expert;
    const size_t slots = (size_t)(n_tok * n_used);
    const size_t y = slots * (size_t)n_embd * 4;
    return 256 + ((y + 255) / 256) * 256;
}

template <int MT>
static int launch_ug_mt(const UgParams &p, int grid, hipStream_t stream)
{
    const size_t lds = (size_t)kWaves * kStageBytes + (size_t)kWaves * 2 * MT * kWave * 4 +
                       (size_t)MT * p.nb * kBlockBytes + (size_t)MT * p.nb * 4 +
                       sizeof(PickShared) + MT * sizeof(int);
    if (lds > (size_t)max_lds_bytes()) return -4;
    hipLaunchKernelGGL(moe_up_gate_kernel<MT>, dim3(grid), dim3(kThreads), lds, stream, p);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

static int tiles_per_wg_for(int64_t active, int64_t tiles_per_expert)
{
    const int64_t total = active * tiles_per_expert;
    int64_t per_wave = total / (256 * 8 * kWaves);
    if (per_wave < 1) per_wave = 1;
    if (per_wave > 8) per_wave = 8;
    int64_t tpw = per_wave * kWaves;
    if (tpw > tiles_per_expert) tpw = tiles_per_expert;
    return (int)tpw;
}

int launch_moe_up_gate(const MoeUpGateArgs &a, hipStream_t stream)
{
    if (a.n_tok == 0) return 0;
    const int64_t nb = a.n_embd / kQK;
    const bool fast = (nb % 8 == 0) && nb <= kStreamMaxNb;
    UgParams p;
    p.w = a.w; p.x = a.x; p.ids = a.ids; p.h = a.h; p.err = (int32_t *)a.ws;
    p.n_slots = (int)(a.n_tok * a.n_used);
    p.n_used = (int)a.n_used;
    p.n_expert = (int)a.n_expert;
    p.nb = (int)nb;
    p.n_ff = (int)a.n_ff;
    p.R = fast ? (int)(64 / (nb / 4)) : 1;
    p.tiles_per_expert = (p.n_ff + p.R - 1) / p.R;
    const int64_t active = a.n_expert < p.n_slots ? a.n_expert : p.n_slots;
    p.tiles_per_wg = tiles_per_wg_for(active, p.tiles_per_expert);
    p.wgs_per_expert = (p.tiles_per_expert + p.tiles_per_wg - 1) / p.tiles_per_wg;
    const int64_t grid = (int64_t)p.n_slots * p.wgs_per_expert;
    if (!fast) {
        const size_t lds = (size_t)nb * kBlockBytes;
        if (lds > (size_t)max_lds_bytes()) return -4;
        dim3 g((unsigned)p.n_slots, (unsigned)((p.n_ff + kWaves - 1) / kWaves));
        hipLaunchKernelGGL(moe_up_gate_generic_kernel, g, dim3(kThreads), lds, stream, p);
        return hipGetLastError() == hipSuccess ? 0 : -6;
    }
    if (grid > 0x7fffffff) return -4;
    switch (pick_mt(a.n_tok)) {
        case 1: return launch_ug_mt<1>(p, (int)grid, stream);
        case 2: return launch_ug_mt<2>(p, (int)grid, stream);
        default: return launch_ug_mt<4>(p, (int)grid, stream);
    }
}

template <int MT>
static int launch_dn_mt(const DnParams &p, int grid, hipStream_t stream)
{
    const size_t lds = (size_t)kWaves * kStageBytes + (size_t)kWaves * MT * kWave * 4 +
                       (size_t)MT * p.nb * kBlockBytes + (size_t)MT * p.nb * 4 +
                       sizeof(PickShared);
    if (lds > (size_t)max_lds_bytes()) return -4;
    hipLaunchKernelGGL(moe_down_kernel<MT>, dim3(grid), dim3(kThreads), lds, stream, p);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

int launch_moe_down(const MoeDownArgs &a, hipStream_t stream)
{
    if (a.n_tok == 0) return 0;
    const int64_t nb = a.n_ff / kQK;
    const bool fast = (nb % 8 == 0) && nb <= kStreamMaxNb;
    const int64_t n_slots = a.n_tok * a.n_used;
    if (fast && n_slots <= kRowsMaxSlots) {
        DrParams r;
        r.w = a.w; r.h = a.h; r.ids = a.ids; r.cw = a.cw; r.out = a.out;
        r.err = (int32_t *)a.ws;
        r.n_used = (int)a.n_used; r.n_slots = (int)n_slots; r.n_expert = (int)a.n_expert;
        r.nb = (int)nb; r.n_ff = (int)a.n_ff; r.n_rows = (int)a.n_embd;
        r.R = (int)(64 / (nb / 4));
        const size_t lds = (size_t)kRowWaves * kStageBytes + (size_t)kRowsMaxSlots * nb * kBlockBytes +
                           (size_t)kRowsMaxSlots * nb * 4;
        if (lds > (size_t)max_lds_bytes()) return -4;
        const unsigned grid = (unsigned)((a.n_embd + r.R - 1) / r.R);
        hipLaunchKernelGGL(moe_down_rows_kernel, dim3(grid), dim3(kRowThreads), lds, stream, r);
        return hipGetLastError() == hipSuccess ? 0 : -6;
    }
    DnParams p;
    p.w = a.w; p.h = a.h; p.ids = a.ids;
    p.yslot = (float *)((uint8_t *)a.ws + 256);
    p.err = (int32_t *)a.ws;
    p.n_slots = (int)(a.n_tok * a.n_used);
    p.n_used = (int)a.n_used;
    p.n_expert = (int)a.n_expert;
    p.nb = (int)nb;
    p.n_ff = (int)a.n_ff;
    p.n_rows = (int)a.n_embd;
    p.R = fast ? (int)(64 / (nb / 4)) : 1;
    p.tiles_per_expert = (p.n_rows + p.R - 1) / p.R;
    const int64_t active = a.n_expert < p.n_slots ? a.n_expert : p.n_slots;
    p.tiles_per_wg = tiles_per_wg_for(active, p.tiles_per_expert);
    p.wgs_per_expert = (p.tiles_per_expert + p.tiles_per_wg - 1) / p.tiles_per_wg;
    const int64_t grid = (int64_t)p.n_slots * p.wgs_per_expert;
    int rc;
    if (fast && grid > 0x7fffffff) return -4;
    if (!fast) {
        const size_t lds = (size_t)nb * kBlockBytes;
        if (lds > (size_t)max_lds_bytes()) return -4;
        dim3 g((unsigned)p.n_slots, (unsigned)((p.n_rows + kWaves - 1) / kWaves));
        hipLaunchKernelGGL(moe_down_generic_kernel, g, dim3(kThreads), lds, stream, p);
        rc = hipGetLastError() == hipSuccess ? 0 : -6;
    } else switch (pick_mt(a.n_tok)) {
        case 1: rc = launch_dn_mt<1>(p, (int)grid, stream); break;
        case 2: rc = launch_dn_mt<2>(p, (int)grid, stream); break;
        default: rc = launch_dn_mt<4>(p, (int)grid, stream); break;
    }
    if (rc) return rc;
    dim3 cgrid((unsigned)((a.n_embd + 255) / 256), (unsigned)a.n_tok);
    hipLaunchKernelGGL(moe_combine_kernel, cgrid, dim3(256), 0, stream, p.yslot, a.ids, a.cw,
                       a.out, (int)a.n_embd, (int)a.n_used, (int)a.n_expert);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

int launch_moe_route(const int32_t *ids, int32_t *counts, int32_t *offsets, int32_t *pairs,
                     int64_t n_tok, int64_t n_expert, int64_t n_used, void *ws,
                     hipStream_t stream)
{
    hipLaunchKernelGGL(moe_route_kernel, dim3(1), dim3(kThreads), 0, stream, ids, counts,
                       offsets, pairs, (int)(n_tok * n_used), (int)n_expert, (int32_t *)ws);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // namespace q8
