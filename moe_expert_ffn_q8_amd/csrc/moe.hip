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
//  * Expert-major gather.  Workgroups are laid out as (active-expert rank,
//    part); every workgroup scans the ids itself (an LDS bitmap of the active
//    experts, then a ballot compaction of the slots routed to its expert in
//    ascending (t,u) order), so no routing kernel and no host sync are needed,
//    and each active expert's rows are streamed from HBM once per call for all
//    of its slots.  Workgroups whose rank is past the number of active experts
//    exit after the scan.
//  * The weight tiles go through the same engine as the decode products
//    (coalesced 16-byte loads -> per-wave LDS slot -> one 4-block quad per
//    lane, v_dot4 against a masked activation image).
//  * up_gate: a wave-tile pairs R gate rows with the same R up rows, so SwiGLU
//    is applied in the epilogue on the reduced dot products; no second pass.
//  * down: the workgroup quantizes the h rows of its expert's slots straight
//    into the masked image (same rule and code as the activation quantizer),
//    writes per-slot outputs to the workspace, and a small kernel combines the
//    n_used slot outputs of each token in ascending u order (deterministic).
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
constexpr int kBitmapWords = kMoeMaxExperts / 32;

struct PickShared {
    uint32_t bitmap[kBitmapWords];
    int invalid;
    int expert;
    int count;
    int pad;
    int slots[kMoeMaxSlots];
};

// Build the ascending list of slots routed to expert e with wave 0 (ballot
// compaction in slot order).  Returns the count (valid in wave 0).
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

// All threads of the workgroup: find the expert of rank `rank` among the
// active experts (ascending id) and its slot list.  Sets ps.expert (-1 when
// the rank is past the active count), ps.count and ps.slots, and ps.invalid.
__device__ void pick_expert(const int32_t *ids, int n_slots, int n_expert, int rank,
                            PickShared &ps)
{
    const int tid = threadIdx.x;
    for (int i = tid; i < kBitmapWords; i += kThreads) ps.bitmap[i] = 0u;
    if (tid == 0) ps.invalid = 0;
    __syncthreads();
    for (int s = tid; s < n_slots; s += kThreads) {
        const int e = ids[s];
        if (e >= 0 && e < n_expert) atomicOr(&ps.bitmap[e >> 5], 1u << (e & 31));
        else atomicOr(&ps.invalid, 1);
    }
    __syncthreads();
    if (tid == 0) {
        int e = -1, cum = 0;
        const int words = (n_expert + 31) >> 5;
        for (int w = 0; w < words; ++w) {
            const int c = __popc(ps.bitmap[w]);
            if (rank < cum + c) {
                uint32_t bits = ps.bitmap[w];
                for (int k = 0; k < rank - cum; ++k) bits &= bits - 1u;
                e = 32 * w + (__ffs(bits) - 1);
                break;
            }
            cum += c;
        }
        ps.expert = e;
    }
    __syncthreads();
    const int e = ps.expert;
    if (e >= 0 && tid < kWave) {
        const int cnt = build_slot_list(ids, n_slots, e, ps.slots, tid);
        if (tid == 0) ps.count = cnt;
    }
    __syncthreads();
}

// Copy Q8_0 token rows into the masked image (scale bytes zeroed) + fp32 scales.
__device__ void stage_rows_q8(const uint8_t *x, int64_t row_bytes_src, const int *rows_of,
                              int mc, int nb, uint8_t *ximg, float *xsc)
{
    const int img_row = nb * kBlockBytes;
    const int halves = mc * nb * 17;
    for (int i = threadIdx.x; i < halves; i += kThreads) {
        const int m = i / (nb * 17);
        const int rem = i - m * nb * 17;
        const int b = rem / 17;
        const int hh = rem - b * 17;
        const uint32_t v = load_u16(x + (int64_t)rows_of[m] * row_bytes_src + b * kBlockBytes + 2 * hh);
        uint16_t *img16 = (uint16_t *)(ximg + m * img_row);
        if (hh == 0) {
            xsc[m * nb + b] = half_bits_to_float(v);
            img16[b * 17] = 0;
        } else {
            img16[b * 17 + hh] = (uint16_t)v;
        }
    }
}

struct UgParams {
    const uint8_t *w;
    const uint8_t *x;
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

    const int rank = blockIdx.x / p.wgs_per_expert;
    const int part = blockIdx.x - rank * p.wgs_per_expert;
    pick_expert(p.ids, p.n_slots, p.n_expert, rank, ps);

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
    const int e = ps.expert;
    if (e < 0) return;
    const int count = ps.count;

    const int64_t row_bytes = (int64_t)nb * kBlockBytes;
    const uint8_t *We = p.w + (int64_t)e * 2 * p.n_ff * row_bytes;
    const int t0 = part * p.tiles_per_wg;
    const int t1 = min(t0 + p.tiles_per_wg, p.tiles_per_expert);
    const int c = lane % Q;

    for (int c0 = 0; c0 < count; c0 += MT) {
        const int mc = min(MT, count - c0);
        __syncthreads();
        if (tid < mc) rows_of[tid] = ps.slots[c0 + tid] / p.n_used;
        __syncthreads();
        stage_rows_q8(p.x, row_bytes, rows_of, mc, nb, ximg, xsc);
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
            const int chunks = rows * nb * 17 / 8;
            const int live = rows * Q;
            u32x4 gg[kTileLoads], gu[kTileLoads];
            tile_issue(We + (int64_t)j0 * row_bytes, chunks, lane, gg);
            tile_issue(We + (int64_t)(p.n_ff + j0) * row_bytes, chunks, lane, gu);
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                uint32_t wq[kQuadDwords];
                tile_to_quad(stage, half == 0 ? gg : gu, lane, live, wq);
                float dw0, dw1, dw2, dw3;
                quad_scales(wq, dw0, dw1, dw2, dw3);
                float *red = half == 0 ? redg : redu;
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
            }
            wave_lds_sync();
            for (int i = lane; i < rows * mc; i += kWave) {
                const int m = i / rows;
                const int r = i - m * rows;
                const float *pg = redg + m * kWave + r * Q;
                const float *pu = redu + m * kWave + r * Q;
                float g = pg[0], u = pu[0];
                for (int cc = 1; cc < Q; ++cc) {
                    g += pg[cc];
                    u += pu[cc];
                }
                const float hv = g / (1.0f + expf(-g)) * u;
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

    const int rank = blockIdx.x / p.wgs_per_expert;
    const int part = blockIdx.x - rank * p.wgs_per_expert;
    pick_expert(p.ids, p.n_slots, p.n_expert, rank, ps);
    if (blockIdx.x == 0 && tid == 0) *p.err = ps.invalid ? 1 : 0;
    const int e = ps.expert;
    if (e < 0) return;
    const int count = ps.count;

    const int64_t row_bytes = (int64_t)nb * kBlockBytes;
    const uint8_t *We = p.w + (int64_t)e * p.n_rows * row_bytes;
    const int t0 = part * p.tiles_per_wg;
    const int t1 = min(t0 + p.tiles_per_wg, p.tiles_per_expert);
    const int c = lane % Q;

    for (int c0 = 0; c0 < count; c0 += MT) {
        const int mc = min(MT, count - c0);
        __syncthreads();
        // quantize the h rows of this chunk's slots into the masked image
        for (int bi = tid >> 3; bi < mc * nb; bi += kThreads / 8) {
            const int m = bi / nb;
            const int b = bi - m * nb;
            const int li = tid & 7;
            const float4 v = *(const float4 *)(p.h + (int64_t)ps.slots[c0 + m] * p.n_ff +
                                                b * kQK + 4 * li);
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
        __syncthreads();

        uint32_t xr[kQuadDwords];
        float4 xd1 = make_float4(0.f, 0.f, 0.f, 0.f);
        if (MT == 1) {
            lds_quad(ximg + kQuadBytes * c, xr);
            xd1 = *(const float4 *)(xsc + 4 * c);
        }

        u32x4 g[kTileLoads];
        int t = t0 + wave;
        if (t < t1) {
            const int r0 = t * p.R;
            tile_issue(We + (int64_t)r0 * row_bytes, min(p.R, p.n_rows - r0) * nb * 17 / 8, lane, g);
        }
        for (; t < t1; t += kWaves) {
            const int row0 = t * p.R;
            const int rows = min(p.R, p.n_rows - row0);
            const int live = rows * Q;
            uint32_t wq[kQuadDwords];
            tile_to_quad(stage, g, lane, live, wq);
            if (t + kWaves < t1) {
                const int r0 = (t + kWaves) * p.R;
                tile_issue(We + (int64_t)r0 * row_bytes, min(p.R, p.n_rows - r0) * nb * 17 / 8,
                           lane, g);
            }
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
    if (nb % 8 != 0 || nb > kStreamMaxNb) return -4;
    UgParams p;
    p.w = a.w; p.x = a.x; p.ids = a.ids; p.h = a.h; p.err = (int32_t *)a.ws;
    p.n_slots = (int)(a.n_tok * a.n_used);
    p.n_used = (int)a.n_used;
    p.n_expert = (int)a.n_expert;
    p.nb = (int)nb;
    p.n_ff = (int)a.n_ff;
    p.R = (int)(64 / (nb / 4));
    p.tiles_per_expert = (p.n_ff + p.R - 1) / p.R;
    const int64_t active = a.n_expert < p.n_slots ? a.n_expert : p.n_slots;
    p.tiles_per_wg = tiles_per_wg_for(active, p.tiles_per_expert);
    p.wgs_per_expert = (p.tiles_per_expert + p.tiles_per_wg - 1) / p.tiles_per_wg;
    const int64_t grid = active * p.wgs_per_expert;
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
    if (nb % 8 != 0 || nb > kStreamMaxNb) return -4;
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
    p.R = (int)(64 / (nb / 4));
    p.tiles_per_expert = (p.n_rows + p.R - 1) / p.R;
    const int64_t active = a.n_expert < p.n_slots ? a.n_expert : p.n_slots;
    p.tiles_per_wg = tiles_per_wg_for(active, p.tiles_per_expert);
    p.wgs_per_expert = (p.tiles_per_expert + p.tiles_per_wg - 1) / p.tiles_per_wg;
    const int64_t grid = active * p.wgs_per_expert;
    if (grid > 0x7fffffff) return -4;
    int rc;
    switch (pick_mt(a.n_tok)) {
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
