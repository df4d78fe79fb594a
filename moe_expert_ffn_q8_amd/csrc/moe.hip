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
#include <string.h>

#include "q8_device.h"
#include "q8_internal.h"
#include "q8_moe.h"

namespace q8 {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;

// Loads complete in issue order (one counter per wave), so a small load issued
// after a tile's weight loads can only be used once those weights have
// arrived.  The kernels below therefore issue their latency-critical small
// loads (the ids for the ownership scan, activation or h rows) before the
// weights.
constexpr int kPickRegs = 4;          // slots 0..255: ids preloaded in registers
constexpr int kPrePass = 4;           // prefetched row blocks per thread (256 threads)
constexpr int kDnPrePass = 8;         // the same for the 512-thread down kernel
// With one token (MT == 1 below) the slots name distinct experts, every
// workgroup owns its slot's expert, and its first weight tile is issued before
// the ownership scan.  With several tokens a large share of the slots repeat an
// expert named by an earlier slot (at 16 tokens over 128 experts with 8 per
// token about a third of them): those workgroups exit after the scan, so the
// first tile is issued only once ownership is known and the activation image
// is built (the small loads then also run ahead of the weights).  Measured on
// 30 layers at 16 tokens: 1975 us per step against 2042 us with the early
// issue; at one token the early issue is 1% faster.
template <int MT>
constexpr bool issue_after_pick()
{
    return MT > 1;
}

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

// The ids of slots 0 .. 64*kPickRegs-1, one per lane of wave 0 (issued
// before the weight loads).
struct IdsPre {
    int v[kPickRegs];
};

// Every lane loads (from a clamped in-range index, n_slots >= 1): the loads are
// unconditional, so the wait for them never has to cover later loads.
__device__ __forceinline__ void preload_ids(const int32_t *ids, int n_slots, IdsPre &ip)
{
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int c = 0; c < kPickRegs; ++c) ip.v[c] = ids[min(c * kWave + lane, n_slots - 1)];
}

// Workgroup for slot s with expert e = ids[s]: the workgroup owns the expert
// when e is in range and s is the first slot that names it; it then serves
// every slot routed to e (listed in ascending (t,u) order).  One ballot pass
// of wave 0 over the ids finds ownership, the slot list and whether any id is
// out of range.  Sets ps.expert (-1: nothing to do), ps.count, ps.slots,
// ps.invalid (LESS: also ps.pad = the number of in-range slots with an id
// below e, the start of e's group in the expert-major slot order); ends with
// a workgroup barrier.
template <bool LESS>
__device__ void pick_by_slot(const int32_t *ids, int n_slots, int n_expert, int s, int e,
                             const IdsPre &ip, PickShared &ps)
{
    const int tid = threadIdx.x;
    if (tid < kWave) {
        int cnt = 0, less = 0;
        bool first = true, bad = false;
        auto step = [&](int i, int v) {
            const bool in = i < n_slots;
            bad |= __ballot(in && (v < 0 || v >= n_expert)) != 0;
            if (LESS) less += __popcll(__ballot(in && v >= 0 && v < e));
            const bool hit = in && v == e;
            const uint64_t m = __ballot(hit);
            first &= __ballot(hit && i < s) == 0;
            if (hit) ps.slots[cnt + __popcll(m & __lanemask_lt())] = i;
            cnt += __popcll(m);
        };
#pragma unroll
        for (int c = 0; c < kPickRegs; ++c)
            if (c * kWave < n_slots) step(c * kWave + tid, ip.v[c]);
        for (int base = kPickRegs * kWave; base < n_slots; base += kWave) {
            const int i = base + tid;
            step(i, i < n_slots ? ids[i] : 0);
        }
        if (tid == 0) {
            ps.invalid = bad ? 1 : 0;
            ps.expert = (e >= 0 && e < n_expert && first) ? e : -1;
            ps.count = cnt;
            if (LESS) ps.pad = less;
        }
    }
    __syncthreads();
}

// Validation outputs of the expert kernels (null in the product path): the
// exact int32 block sums [slot][weight row][block], the Q8_0 bytes of the h
// rows the down kernels used [slot][n_ff/32], and the expert-major grouping
// the up_gate kernels served (counts per expert, slots at their group's
// start).  Written only by the EMIT instances of the kernels.
struct MoeEmitPtrs {
    int32_t *sums;
    uint8_t *hq;
    int32_t *counts;
    int32_t *pairs;
};

// Write the Q8_0 bytes of image rows [0, mc) (masked image + fp32 scales, as
// quantize_rows_to_image leaves them) to hq rows slot_of(m): the scale bits
// are those of the fp32 scale (a binary16 value, converted exactly).
template <class SlotOf>
__device__ void emit_hq_rows(const uint8_t *ximg, const float *xsc, int mc, int nb, uint8_t *hq,
                             SlotOf slot_of)
{
    for (int i = threadIdx.x; i < mc * nb * 17; i += blockDim.x) {
        const int m = i / (nb * 17);
        const int r = i - m * nb * 17;
        const int b = r / 17, w = r - b * 17;
        uint16_t v = ((const uint16_t *)(ximg + (m * nb + b) * kBlockBytes))[w];
        if (w == 0) v = __builtin_bit_cast(uint16_t, (_Float16)xsc[m * nb + b]);
        ((uint16_t *)(hq + ((int64_t)slot_of(m) * nb + b) * kBlockBytes))[w] = v;
    }
}

// Quantize one 32-value block held as 4 values by each of 8 lanes into image
// row m (scale bytes zero) and the fp32 scale array.
__device__ __forceinline__ void quantize_to_image(float4 v, int m, int b, int nb, uint8_t *ximg,
                                                  float *xsc)
{
    quantize8_to_image(v, ximg + m * nb * kBlockBytes, xsc + m * nb, b, threadIdx.x & 7);
}

// Quantize fp32 rows m_begin..mc-1 (row m starts at base + row_index[m] *
// row_floats) into the masked image (nb*34 bytes per row, scale bytes zero)
// plus fp32 scales, with the activation quantization rule (same code as the
// quantizer: the bytes equal q8_0_quantize_rows of those rows).  All threads
// of the workgroup take part; 8 lanes per block.
__device__ void quantize_rows_to_image(const float *base, int64_t row_floats, const int *row_index,
                                       int m_begin, int mc, int nb, uint8_t *ximg, float *xsc)
{
    const int tid = threadIdx.x;
    const int li = tid & 7;
    const int step = (int)blockDim.x / 8;
    for (int bi = m_begin * nb + (tid >> 3); bi < mc * nb; bi += step) {
        const int m = bi / nb;
        const int b = bi - m * nb;
        const float4 v = *(const float4 *)(base + (int64_t)row_index[m] * row_floats + b * kQK + 4 * li);
        quantize_to_image(v, m, b, nb, ximg, xsc);
    }
}

// Two-step form for rows known before the weights are issued: prefetch_rows
// loads the blocks of rows 0..mc-1 (row m at rows0 + m * row_floats) into
// registers, quantize_prefetched writes them into image rows m_out+m.  Needs
// mc * nb <= P * blockDim.x / 8.
// The loads are unconditional (indices past the rows are clamped to the last
// block), so that later waits are exact counts.
template <int P>
__device__ __forceinline__ void prefetch_rows(const float *rows0, int64_t row_floats, int mc, int nb,
                                              float4 (&v)[P])
{
    const int tid = threadIdx.x;
    const int step = (int)blockDim.x / 8;
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const int bi = min((tid >> 3) + i * step, mc * nb - 1);
        const int m = bi / nb;
        const int b = bi - m * nb;
        v[i] = *(const float4 *)(rows0 + (int64_t)m * row_floats + b * kQK + 4 * (tid & 7));
    }
}

template <int P>
__device__ __forceinline__ void quantize_prefetched(const float4 (&v)[P], int mc, int nb, int m_out,
                                                    uint8_t *ximg, float *xsc)
{
    const int step = (int)blockDim.x / 8;
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const int bi = ((int)threadIdx.x >> 3) + i * step;
        if (bi < mc * nb) {
            const int m = bi / nb;
            quantize_to_image(v[i], m_out + m, bi - m * nb, nb, ximg, xsc);
        }
    }
}

// Per-layer pointers of a launch (up to kMoeMaxLayers independent layers of
// the same shape in one grid).
struct UgLayer {
    const uint8_t *w;
    const float *x;        // fp32 [n_tok][n_embd]
    const int32_t *ids;
    float *h;
    int32_t *err;
};

struct UgParams {
    UgLayer layer[kMoeMaxLayers];
    MoeEmitPtrs emit;
    int n_layers;
    int wgs_per_layer;     // n_slots * wgs_per_expert
    int n_slots, n_used, n_expert, nb, n_ff;
    int R;                 // rows per wave-tile
    int tiles_per_expert;  // ceil(n_ff / R)
    int wgs_per_expert;
    int tiles_per_wg;
};

static_assert(sizeof(UgParams) <= 4000, "kernel arguments must stay below 4 KB");

// EMIT (validation builds of the same kernel): p.emit's block sums and
// routing are written as well.
template <int MT, bool EMIT>
__global__ __launch_bounds__(kThreads) void moe_up_gate_kernel(const UgParams p)
{
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x;
    const int wave = wave_uniform(tid >> 6);
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

    const int li = blockIdx.x / p.wgs_per_layer;
    const int wl = blockIdx.x - li * p.wgs_per_layer;      // workgroup within the layer
    const UgLayer &L = p.layer[li];
    const int slot = wl / p.wgs_per_expert;
    const int part = wl - slot * p.wgs_per_expert;
    const int e0 = L.ids[slot];
    const bool e0_ok = e0 >= 0 && e0 < p.n_expert;
    const int64_t row_bytes = (int64_t)nb * kBlockBytes;
    const uint8_t *We = L.w + (int64_t)(e0_ok ? e0 : 0) * 2 * p.n_ff * row_bytes;
    const int t0 = part * p.tiles_per_wg;
    const int t1 = min(t0 + p.tiles_per_wg, p.tiles_per_expert);
    const int c = lane % Q;

    // Small loads first: the ids for the ownership scan and the token row of
    // this workgroup's own slot (the first row of its first chunk when it owns
    // the expert).
    IdsPre ip;
    preload_ids(L.ids, p.n_slots, ip);
    const bool x_pre = nb <= kPrePass * (kThreads / 8);
    float4 xv[kPrePass];
    prefetch_rows<kPrePass>(L.x + (int64_t)(slot / p.n_used) * nb * kQK, 0, 1, nb, xv);

    // The gate and up rows of a tile are loaded together (two register sets);
    // the wave's next pair is issued once both are staged.  The first pair
    // depends only on ids[slot] (dropped if another slot owns the expert).
    // Issues are unconditional: a tile that does not exist gets a zero-length
    // buffer (zeros, no memory traffic), so every wait is an exact count.
    u32x4 gg[kTileLoads], gu[kTileLoads];
    auto issue = [&](int tt, bool real) {
        const int j0 = tt * p.R;
        const int chunks = real ? min(p.R, p.n_ff - j0) * nb * 17 / 8 : 0;
        tile_issue(We + (int64_t)(real ? j0 : 0) * row_bytes, chunks, lane, gg);
        tile_issue(We + (int64_t)(real ? p.n_ff + j0 : 0) * row_bytes, chunks, lane, gu);
    };
    if (!issue_after_pick<MT>()) issue(t0 + wave, e0_ok && t0 + wave < t1);
    pick_by_slot<EMIT>(L.ids, p.n_slots, p.n_expert, slot, e0, ip, ps);
    if (EMIT && ps.expert >= 0 && part == 0 && p.emit.counts) {
        if (tid == 0) p.emit.counts[ps.expert] = ps.count;
        for (int i = tid; i < ps.count; i += kThreads) p.emit.pairs[ps.pad + i] = ps.slots[i];
    }

    if (wl == 0) {
        if (tid == 0) *L.err = ps.invalid ? 1 : 0;
        if (ps.invalid) {
            for (int s = 0; s < p.n_slots; ++s) {
                const int e = L.ids[s];
                if (e < 0 || e >= p.n_expert)
                    for (int j = tid; j < p.n_ff; j += kThreads)
                        L.h[(int64_t)s * p.n_ff + j] = __builtin_nanf("");
            }
        }
    }
    if (ps.expert < 0) return;
    const int count = ps.count;

    for (int c0 = 0; c0 < count; c0 += MT) {
        const int mc = min(MT, count - c0);
        __syncthreads();
        if (tid < mc) rows_of[tid] = ps.slots[c0 + tid] / p.n_used;
        // later chunks restart the tile walk: issue its first pair now
        if (c0 > 0) issue(t0 + wave, t0 + wave < t1);
        __syncthreads();
        int m_begin = 0;
        if (c0 == 0 && x_pre) {      // ps.slots[0] is this slot: its row is in registers
            quantize_prefetched<kPrePass>(xv, 1, nb, 0, ximg, xsc);
            m_begin = 1;
        }
        quantize_rows_to_image(L.x, (int64_t)nb * kQK, rows_of, m_begin, mc, nb, ximg, xsc);
        __syncthreads();
        if (issue_after_pick<MT>() && c0 == 0) issue(t0 + wave, t0 + wave < t1);

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
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                uint32_t wq[kQuadDwords];
                tile_to_quad(stage, half == 0 ? gg : gu, lane, live, wq);
                if (half == 1) issue(t + kWaves, t + kWaves < t1);
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
                    if (EMIT && p.emit.sums && lane < live) {
                        const int64_t wrow = (int64_t)half * p.n_ff + j0 + lane / Q;
                        int32_t *o = p.emit.sums +
                                     ((int64_t)ps.slots[c0 + m] * 2 * p.n_ff + wrow) * nb + 4 * c;
                        o[0] = sb[0]; o[1] = sb[1]; o[2] = sb[2]; o[3] = sb[3];
                    }
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
                L.h[(int64_t)ps.slots[c0 + m] * p.n_ff + j0 + r] = hv;
            }
            wave_lds_sync();
        }
    }
}

struct DnLayer {
    const uint8_t *w;
    const float *h;
    const int32_t *ids;
    float *yslot;        // [n_slots][n_rows]
    int32_t *err;
};

struct DnParams {
    DnLayer layer[kMoeMaxLayers];
    MoeEmitPtrs emit;
    int n_layers;
    int wgs_per_layer;
    int n_slots, n_used, n_expert, nb, n_ff, n_rows;
    int R, tiles_per_expert, wgs_per_expert, tiles_per_wg;
};

static_assert(sizeof(DnParams) <= 4000, "kernel arguments must stay below 4 KB");

template <int MT, bool EMIT>
__global__ __launch_bounds__(kThreads) void moe_down_kernel(const DnParams p)
{
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x;
    const int wave = wave_uniform(tid >> 6);
    const int lane = tid & 63;
    const int nb = p.nb;
    const int Q = nb >> 2;
    const int img_row = nb * kBlockBytes;

    uint8_t *stage = smem + wave * kStageBytes;
    float *red = (float *)(smem + kWaves * kStageBytes) + wave * MT * kWave;
    uint8_t *ximg = smem + kWaves * kStageBytes + kWaves * MT * kWave * 4;
    float *xsc = (float *)(ximg + MT * img_row);
    PickShared &ps = *(PickShared *)(xsc + MT * nb);

    const int li = blockIdx.x / p.wgs_per_layer;
    const int wl = blockIdx.x - li * p.wgs_per_layer;      // workgroup within the layer
    const DnLayer &L = p.layer[li];
    const int slot = wl / p.wgs_per_expert;
    const int part = wl - slot * p.wgs_per_expert;
    const int e0 = L.ids[slot];
    const bool e0_ok = e0 >= 0 && e0 < p.n_expert;
    const int64_t row_bytes = (int64_t)nb * kBlockBytes;
    const uint8_t *We = L.w + (int64_t)(e0_ok ? e0 : 0) * p.n_rows * row_bytes;
    const int t0 = part * p.tiles_per_wg;
    const int t1 = min(t0 + p.tiles_per_wg, p.tiles_per_expert);
    const int c = lane % Q;

    // Unconditional issues (a tile that does not exist is a zero-length
    // buffer), so every wait is an exact count.
    u32x4 g[kTileLoads];
    auto issue = [&](int tt, bool real) {
        const int r0 = real ? tt * p.R : 0;
        tile_issue(We + (int64_t)r0 * row_bytes, real ? min(p.R, p.n_rows - r0) * nb * 17 / 8 : 0,
                   lane, g);
    };
    IdsPre ip;
    preload_ids(L.ids, p.n_slots, ip);
    // depends only on ids[slot]: issue before the scan and the h round trip
    if (!issue_after_pick<MT>()) issue(t0 + wave, e0_ok && t0 + wave < t1);
    pick_by_slot<false>(L.ids, p.n_slots, p.n_expert, slot, e0, ip, ps);
    if (wl == 0 && tid == 0) *L.err = ps.invalid ? 1 : 0;
    if (ps.expert < 0) return;
    const int count = ps.count;

    for (int c0 = 0; c0 < count; c0 += MT) {
        const int mc = min(MT, count - c0);
        int t = t0 + wave;
        if (c0 > 0) issue(t, t < t1);
        __syncthreads();
        // quantize the h rows of this chunk's slots into the masked image
        quantize_rows_to_image(L.h, p.n_ff, ps.slots + c0, 0, mc, nb, ximg, xsc);
        __syncthreads();
        if (EMIT && p.emit.hq && part == 0)
            emit_hq_rows(ximg, xsc, mc, nb, p.emit.hq, [&](int m) { return ps.slots[c0 + m]; });
        if (issue_after_pick<MT>() && c0 == 0) issue(t, t < t1);

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
            issue(t + kWaves, t + kWaves < t1);
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
                    if (EMIT && p.emit.sums && lane < live) {
                        int32_t *o = p.emit.sums + ((int64_t)ps.slots[c0 + m] * p.n_rows + row0 +
                                                    lane / Q) * nb + 4 * c;
                        o[0] = s[0]; o[1] = s[1]; o[2] = s[2]; o[3] = s[3];
                    }
                }
            }
            wave_lds_sync();
            for (int i = lane; i < rows * mc; i += kWave) {
                const int m = i / rows;
                const int r = i - m * rows;
                const float *pr = red + m * kWave + r * Q;
                float acc = pr[0];
                for (int cc = 1; cc < Q; ++cc) acc += pr[cc];
                L.yslot[(int64_t)ps.slots[c0 + m] * p.n_rows + row0 + r] = acc;
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

struct DrLayer {
    const uint8_t *w;
    const float *h;
    const int32_t *ids;
    const float *cw;
    float *out;
    int32_t *err;
};

struct DrParams {
    DrLayer layer[kMoeMaxLayers];
    MoeEmitPtrs emit;
    int n_layers;
    int wgs_per_layer;     // ceil(n_rows / R)
    int n_used, n_slots, n_expert, nb, n_ff, n_rows, R;
};

static_assert(sizeof(DrParams) <= 4000, "kernel arguments must stay below 4 KB");

template <bool EMIT>
__global__ __launch_bounds__(kRowThreads) void moe_down_rows_kernel(const DrParams p)
{
    extern __shared__ __align__(16) uint8_t smem[];
    __shared__ int s_e[kRowsMaxSlots];
    __shared__ int s_rows[kRowsMaxSlots];
    __shared__ float ys[kRowsMaxSlots][kWave];
    __shared__ float red[kRowWaves][kWave];
    const int tid = threadIdx.x;
    const int wave = wave_uniform(tid >> 6);
    const int lane = tid & 63;
    const int nb = p.nb;
    const int Q = nb >> 2;
    const int img_row = nb * kBlockBytes;
    uint8_t *stage = smem + wave * kStageBytes;
    uint8_t *ximg = smem + kRowWaves * kStageBytes;
    float *xsc = (float *)(ximg + kRowsMaxSlots * img_row);

    const int li = blockIdx.x / p.wgs_per_layer;
    const int wl = blockIdx.x - li * p.wgs_per_layer;      // row band within the layer
    const DrLayer &L = p.layer[li];
    const int row0 = wl * p.R;
    const int rows = min(p.R, p.n_rows - row0);
    const int live = rows * Q;
    const int c = lane % Q;
    const int64_t row_bytes = (int64_t)nb * kBlockBytes;

    u32x4 g[kTileLoads];
    // e < 0: a zero-length buffer (zeros, no memory traffic), so that the
    // issue is unconditional and later waits are exact counts
    auto issue_e = [&](int e) {
        const uint8_t *base = L.w + ((int64_t)(e < 0 ? 0 : e) * p.n_rows + row0) * row_bytes;
        tile_issue(base, e < 0 ? 0 : rows * nb * 17 / 8, lane, g);
    };
    // Small loads before the weights: every slot's id and, when they fit in
    // registers, every slot's h row.  This wave's first weights depend only on
    // its slot's id (a scalar load).
    const int e_first = wave < p.n_slots ? L.ids[wave] : -1;
    const bool first_ok = e_first >= 0 && e_first < p.n_expert;
    const int e_mine = L.ids[min(tid, p.n_slots - 1)];
    const bool h_pre = p.n_slots * nb <= kDnPrePass * (kRowThreads / 8);
    float4 hv[kDnPrePass];
    prefetch_rows<kDnPrePass>(L.h, p.n_ff, p.n_slots, nb, hv);
    issue_e(first_ok ? e_first : -1);

    if (tid < p.n_slots) {
        s_e[tid] = (e_mine >= 0 && e_mine < p.n_expert) ? e_mine : -1;
        s_rows[tid] = tid;
    }
    __syncthreads();
    if (wl == 0 && tid == 0) {
        int bad = 0;
        for (int s = 0; s < p.n_slots; ++s) bad |= (s_e[s] < 0);
        *L.err = bad;
    }

    auto next_slot = [&](int s) {
        while (s < p.n_slots && s_e[s] < 0) s += kRowWaves;
        return s;
    };
    int s = next_slot(wave);
    if (!first_ok && s < p.n_slots) issue_e(s_e[s]);

    if (h_pre) quantize_prefetched<kDnPrePass>(hv, p.n_slots, nb, 0, ximg, xsc);
    else quantize_rows_to_image(L.h, p.n_ff, s_rows, 0, p.n_slots, nb, ximg, xsc);
    __syncthreads();
    if (EMIT && p.emit.hq && wl == 0)
        emit_hq_rows(ximg, xsc, p.n_slots, nb, p.emit.hq, [](int m) { return m; });

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
        if (EMIT && p.emit.sums && lane < live) {
            int32_t *o = p.emit.sums + ((int64_t)s * p.n_rows + row0 + lane / Q) * nb + 4 * c;
            o[0] = sb[0]; o[1] = sb[1]; o[2] = sb[2]; o[3] = sb[3];
        }
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
            acc = L.cw[t * p.n_used] * ys[t * p.n_used][r];
            for (int u = 1; u < p.n_used; ++u)
                acc = fmaf(L.cw[t * p.n_used + u], ys[t * p.n_used + u][r], acc);
        }
        L.out[(int64_t)t * p.n_rows + row0 + r] = acc;
    }
}

// out[t][n] = sum over u ascending of cw[t][u] * yslot[t*n_used+u][n]; a token
// with an out-of-range id gets NaN.  grid (ceil(n_rows/256), n_tok, n_layers).
struct CbLayer {
    const float *yslot;
    const int32_t *ids;
    const float *cw;
    float *out;
};

struct CbParams {
    CbLayer layer[kMoeMaxLayers];
    int n_rows, n_used, n_expert;
};

static_assert(sizeof(CbParams) <= 4000, "kernel arguments must stay below 4 KB");

__global__ __launch_bounds__(256) void moe_combine_kernel(const CbParams p)
{
    const CbLayer &L = p.layer[blockIdx.z];
    const int t = blockIdx.y;
    const int n = blockIdx.x * 256 + threadIdx.x;
    if (n >= p.n_rows) return;
    bool bad = false;
    for (int u = 0; u < p.n_used; ++u) {
        const int e = L.ids[t * p.n_used + u];
        bad |= (e < 0 || e >= p.n_expert);
    }
    float acc;
    if (bad) {
        acc = __builtin_nanf("");
    } else {
        const float *y = L.yslot + (int64_t)t * p.n_used * p.n_rows + n;
        acc = L.cw[t * p.n_used] * y[0];
        for (int u = 1; u < p.n_used; ++u)
            acc = fmaf(L.cw[t * p.n_used + u], y[(int64_t)u * p.n_rows], acc);
    }
    L.out[(int64_t)t * p.n_rows + n] = acc;
}

// The same with four consecutive outputs per thread (n_rows % 4 == 0, out
// 16-byte aligned): one 16-byte load per slot row, the same arithmetic per
// output.  grid (ceil(n_rows/1024), n_tok, n_layers).
__global__ __launch_bounds__(256) void moe_combine4_kernel(const CbParams p)
{
    const CbLayer &L = p.layer[blockIdx.z];
    const int t = blockIdx.y;
    const int n = 4 * (blockIdx.x * 256 + threadIdx.x);
    if (n >= p.n_rows) return;
    bool bad = false;
    for (int u = 0; u < p.n_used; ++u) {
        const int e = L.ids[t * p.n_used + u];
        bad |= (e < 0 || e >= p.n_expert);
    }
    float4 acc;
    if (bad) {
        acc = make_float4(__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""),
                          __builtin_nanf(""));
    } else {
        const float *y = L.yslot + (int64_t)t * p.n_used * p.n_rows + n;
        const float c0 = L.cw[t * p.n_used];
        const float4 y0 = *(const float4 *)y;
        acc = make_float4(c0 * y0.x, c0 * y0.y, c0 * y0.z, c0 * y0.w);
        for (int u = 1; u < p.n_used; ++u) {
            const float c = L.cw[t * p.n_used + u];
            const float4 v = *(const float4 *)(y + (int64_t)u * p.n_rows);
            acc.x = fmaf(c, v.x, acc.x);
            acc.y = fmaf(c, v.y, acc.y);
            acc.z = fmaf(c, v.z, acc.z);
            acc.w = fmaf(c, v.w, acc.w);
        }
    }
    *(float4 *)(L.out + (int64_t)t * p.n_rows + n) = acc;
}

// Either combine kernel for cb (the four-wide one where rows and outputs allow).
int launch_combine(const CbParams &cb, int n_layers, int64_t n_tok, hipStream_t stream)
{
    bool four = cb.n_rows % 4 == 0;
    for (int i = 0; i < n_layers; ++i) four = four && ((uintptr_t)cb.layer[i].out % 16 == 0);
    if (four) {
        dim3 g((unsigned)((cb.n_rows + 1023) / 1024), (unsigned)n_tok, (unsigned)n_layers);
        hipLaunchKernelGGL(moe_combine4_kernel, g, dim3(256), 0, stream, cb);
    } else {
        dim3 g((unsigned)((cb.n_rows + 255) / 256), (unsigned)n_tok, (unsigned)n_layers);
        hipLaunchKernelGGL(moe_combine_kernel, g, dim3(256), 0, stream, cb);
    }
    return hipGetLastError() == hipSuccess ? 0 : -6;
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
                                                 int lane, int32_t *sums = nullptr)
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
        if (sums) sums[b] = s;        // validation output (null in the product path)
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

__global__ __launch_bounds__(kThreads) void moe_up_gate_generic_kernel(const UgParams p)
{
    extern __shared__ __align__(16) uint8_t xq[];      // nb blocks of 34 B
    const UgLayer &L = p.layer[blockIdx.z];
    generic_flag_invalid(L.ids, p.n_slots, p.n_expert, L.err);
    const int s = blockIdx.x;
    const int e = L.ids[s];
    quantize_row_to_blocks(L.x + (int64_t)(s / p.n_used) * p.nb * kQK, p.nb, xq);
    __syncthreads();
    const int j = blockIdx.y * kWaves + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (j >= p.n_ff) return;
    float *dst = L.h + (int64_t)s * p.n_ff + j;
    if (e < 0 || e >= p.n_expert) {
        if (lane == 0) *dst = __builtin_nanf("");
        return;
    }
    const int64_t row_bytes = (int64_t)p.nb * kBlockBytes;
    const uint8_t *We = L.w + (int64_t)e * 2 * p.n_ff * row_bytes;
    const uint8_t *xr = xq;
    int32_t *sg = p.emit.sums ? p.emit.sums + ((int64_t)s * 2 * p.n_ff + j) * p.nb : nullptr;
    const float g = generic_row_dot(We + (int64_t)j * row_bytes, xr, p.nb, lane, sg);
    const float u = generic_row_dot(We + (int64_t)(p.n_ff + j) * row_bytes, xr, p.nb, lane,
                                    sg ? sg + (int64_t)p.n_ff * p.nb : nullptr);
    if (lane == 0) *dst = g / (1.0f + expf(-g)) * u;
}

// grid (n_slots, ceil(n_rows / 4)); the slot's h row is quantized into LDS
// first (same rule and code as the activation quantizer).
__global__ __launch_bounds__(kThreads) void moe_down_generic_kernel(const DnParams p)
{
    extern __shared__ __align__(16) uint8_t hq[];      // nb blocks of 34 B
    const DnLayer &L = p.layer[blockIdx.z];
    generic_flag_invalid(L.ids, p.n_slots, p.n_expert, L.err);
    const int s = blockIdx.x;
    const int e = L.ids[s];
    if (e < 0 || e >= p.n_expert) return;              // the combine writes NaN
    const int tid = threadIdx.x;
    quantize_row_to_blocks(L.h + (int64_t)s * p.n_ff, p.nb, hq);
    __syncthreads();
    if (p.emit.hq && blockIdx.y == 0)          // validation: the bytes of q(h) used
        for (int i = tid; i < p.nb * kBlockBytes / 2; i += kThreads)
            ((uint16_t *)(p.emit.hq + (int64_t)s * p.nb * kBlockBytes))[i] = ((const uint16_t *)hq)[i];
    const int row = blockIdx.y * kWaves + (tid >> 6);
    const int lane = tid & 63;
    if (row >= p.n_rows) return;
    const int64_t row_bytes = (int64_t)p.nb * kBlockBytes;
    const uint8_t *wr = L.w + ((int64_t)e * p.n_rows + row) * row_bytes;
    const float y = generic_row_dot(wr, hq, p.nb, lane,
                                    p.emit.sums ? p.emit.sums + ((int64_t)s * p.n_rows + row) * p.nb
                                                : nullptr);
    if (lane == 0) L.yslot[(int64_t)s * p.n_rows + row] = y;
}

// Validation helpers: fill an int32 array; exclusive offsets [n_expert + 1]
// from per-expert counts (one workgroup, sequential scan by one thread).
__global__ void fill_i32_kernel(int32_t *p, int64_t n, int32_t v)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

__global__ void route_offsets_kernel(const int32_t *counts, int32_t *offsets, int n_expert)
{
    if (threadIdx.x != 0) return;
    int acc = 0;
    for (int e = 0; e < n_expert; ++e) {
        offsets[e] = acc;
        acc += counts[e];
    }
    offsets[n_expert] = acc;
}

int pick_mt(int64_t n_tok)
{
    if (n_tok <= 1) return 1;
    if (n_tok <= 2) return 2;
    return 4;
}

}  // namespace

int launch_fill_i32(int32_t *p, int64_t n, int32_t v, hipStream_t stream)
{
    if (n <= 0) return 0;
    hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p, n, v);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

int launch_route_offsets(const int32_t *counts, int32_t *offsets, int64_t n_expert,
                         hipStream_t stream)
{
    hipLaunchKernelGGL(route_offsets_kernel, dim3(1), dim3(64), 0, stream, counts, offsets,
                       (int)n_expert);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

int launch_moe_combine(const float *yslot, const int32_t *ids, const float *cw, float *out,
                       int64_t n_tok, int64_t n_rows, int64_t n_used, int64_t n_expert,
                       hipStream_t stream)
{
    if (n_tok == 0) return 0;
    if (n_tok > 65535) return -4;
    CbParams cb;
    memset(&cb, 0, sizeof(cb));
    cb.layer[0] = CbLayer{yslot, ids, cw, out};
    cb.n_rows = (int)n_rows;
    cb.n_used = (int)n_used;
    cb.n_expert = (int)n_expert;
    return launch_combine(cb, 1, n_tok, stream);
}

int launch_moe_combine_layers(const MoeCombineLayer *l, int n_layers, int64_t n_tok,
                              int64_t n_rows, int64_t n_used, int64_t n_expert, hipStream_t stream)
{
    if (n_tok == 0 || n_layers == 0) return 0;
    if (n_tok > 65535 || n_layers > kMoeMaxLayers) return -4;
    CbParams cb;
    memset(&cb, 0, sizeof(cb));
    for (int i = 0; i < n_layers; ++i) cb.layer[i] = CbLayer{l[i].yslot, l[i].ids, l[i].cw, l[i].out};
    cb.n_rows = (int)n_rows;
    cb.n_used = (int)n_used;
    cb.n_expert = (int)n_expert;
    return launch_combine(cb, n_layers, n_tok, stream);
}

size_t moe_ws_bytes(int64_t n_tok, int64_t n_embd, int64_t n_ff, int64_t n_expert,
                    int64_t n_used)
{
    if (moe_prefill_ok(n_tok, n_embd, n_ff, n_expert, n_used))
        return moe_prefill_ws_bytes(n_tok, n_embd, n_ff, n_expert, n_used);
    const size_t slots = (size_t)(n_tok * n_used);
    const size_t y = slots * (size_t)n_embd * 4;
    return 256 + ((y + 255) / 256) * 256;
}

template <int MT>
static int launch_ug_mt(const UgParams &p, int grid, hipStream_t stream, bool emit)
{
    const size_t lds = (size_t)kWaves * kStageBytes + (size_t)kWaves * 2 * MT * kWave * 4 +
                       (size_t)MT * p.nb * kBlockBytes + (size_t)MT * p.nb * 4 +
                       sizeof(PickShared) + MT * sizeof(int);
    if (lds > (size_t)max_lds_bytes()) return -4;
    if (emit)
        hipLaunchKernelGGL((moe_up_gate_kernel<MT, true>), dim3(grid), dim3(kThreads), lds, stream, p);
    else
        hipLaunchKernelGGL((moe_up_gate_kernel<MT, false>), dim3(grid), dim3(kThreads), lds, stream, p);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

// Tiles per workgroup: about 8 resident workgroups' worth of waves per CU
// share the tiles, at most 8 tiles per wave.  Smaller work units (more
// workgroups) were measured slower: each workgroup pays the ownership scan and
// the activation quantization before it streams.
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
    if (a.n_tok == 0 || a.n_layers == 0) return 0;
    if (moe_prefill_ok(a.n_tok, a.n_embd, a.n_ff, a.n_expert, a.n_used)) {
        for (int l = 0; l < a.n_layers; ++l) {
            const MoeUpGateArgs::Layer &L = a.layer[l];
            if (int rc = launch_moe_prefill_up_gate(L.w, L.x, L.ids, L.h, L.ws, a.n_tok, a.n_embd,
                                                    a.n_ff, a.n_expert, a.n_used, stream,
                                                    a.emit))
                return rc;
        }
        return 0;
    }
    const int64_t nb = a.n_embd / kQK;
    const bool fast = (nb % 8 == 0) && nb <= kStreamMaxNb;
    UgParams p;
    memset(&p, 0, sizeof(p));
    for (int l = 0; l < a.n_layers; ++l) {
        const MoeUpGateArgs::Layer &A = a.layer[l];
        p.layer[l] = UgLayer{A.w, A.x, A.ids, A.h, (int32_t *)A.ws};
    }
    p.n_layers = a.n_layers;
    p.n_slots = (int)(a.n_tok * a.n_used);
    p.n_used = (int)a.n_used;
    p.n_expert = (int)a.n_expert;
    p.nb = (int)nb;
    p.n_ff = (int)a.n_ff;
    const bool emit = a.emit != nullptr;
    if (emit) {
        p.emit = MoeEmitPtrs{a.emit->sums, nullptr, a.emit->counts, a.emit->pairs};
        // the generic kernels serve every slot on its own: no grouping to report
        if (!fast && a.emit->counts) return -4;
        if (a.emit->counts) {
            if (int rc = launch_fill_i32(a.emit->counts, a.n_expert, 0, stream)) return rc;
        }
    }
    p.R = fast ? (int)(64 / (nb / 4)) : 1;
    p.tiles_per_expert = (p.n_ff + p.R - 1) / p.R;
    const int64_t active = a.n_layers * (a.n_expert < p.n_slots ? a.n_expert : p.n_slots);
    p.tiles_per_wg = tiles_per_wg_for(active, p.tiles_per_expert);
    p.wgs_per_expert = (p.tiles_per_expert + p.tiles_per_wg - 1) / p.tiles_per_wg;
    p.wgs_per_layer = p.n_slots * p.wgs_per_expert;
    const int64_t grid = (int64_t)a.n_layers * p.wgs_per_layer;
    if (!fast) {
        const size_t lds = (size_t)nb * kBlockBytes;
        if (lds > (size_t)max_lds_bytes()) return -4;
        dim3 g((unsigned)p.n_slots, (unsigned)((p.n_ff + kWaves - 1) / kWaves), (unsigned)a.n_layers);
        hipLaunchKernelGGL(moe_up_gate_generic_kernel, g, dim3(kThreads), lds, stream, p);
        return hipGetLastError() == hipSuccess ? 0 : -6;
    }
    if (grid > 0x7fffffff) return -4;
    int rc;
    switch (pick_mt(a.n_tok)) {
        case 1: rc = launch_ug_mt<1>(p, (int)grid, stream, emit); break;
        case 2: rc = launch_ug_mt<2>(p, (int)grid, stream, emit); break;
        default: rc = launch_ug_mt<4>(p, (int)grid, stream, emit); break;
    }
    if (rc || !emit || !a.emit->counts) return rc;
    return launch_route_offsets(a.emit->counts, a.emit->offsets, a.n_expert, stream);
}

template <int MT>
static int launch_dn_mt(const DnParams &p, int grid, hipStream_t stream, bool emit)
{
    const size_t lds = (size_t)kWaves * kStageBytes + (size_t)kWaves * MT * kWave * 4 +
                       (size_t)MT * p.nb * kBlockBytes + (size_t)MT * p.nb * 4 +
                       sizeof(PickShared);
    if (lds > (size_t)max_lds_bytes()) return -4;
    if (emit)
        hipLaunchKernelGGL((moe_down_kernel<MT, true>), dim3(grid), dim3(kThreads), lds, stream, p);
    else
        hipLaunchKernelGGL((moe_down_kernel<MT, false>), dim3(grid), dim3(kThreads), lds, stream, p);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

int launch_moe_down(const MoeDownArgs &a, hipStream_t stream)
{
    if (a.n_tok == 0 || a.n_layers == 0) return 0;
    if (moe_prefill_ok(a.n_tok, a.n_embd, a.n_ff, a.n_expert, a.n_used)) {
        for (int l = 0; l < a.n_layers; ++l) {
            const MoeDownArgs::Layer &L = a.layer[l];
            if (int rc = launch_moe_prefill_down(L.w, L.h, L.ids, L.cw, L.out, L.ws, a.n_tok,
                                                 a.n_embd, a.n_ff, a.n_expert, a.n_used, stream,
                                                 a.emit))
                return rc;
        }
        return 0;
    }
    const int64_t nb = a.n_ff / kQK;
    const bool fast = (nb % 8 == 0) && nb <= kStreamMaxNb;
    const int64_t n_slots = a.n_tok * a.n_used;
    const bool emit = a.emit != nullptr;
    const MoeEmitPtrs ep = emit ? MoeEmitPtrs{a.emit->sums, (uint8_t *)a.emit->hq, nullptr, nullptr}
                                : MoeEmitPtrs{nullptr, nullptr, nullptr, nullptr};
    // The row-major kernel (combine fused, one launch) wins for a single layer,
    // where the call is latency-bound; over many layers the expert-major
    // kernel streams better (measured on 30 one-token layers: 198 us per step
    // against 298 us with the row-major kernel), so grouped calls use it.
    if (fast && n_slots <= kRowsMaxSlots && a.n_layers == 1) {
        DrParams r;
        memset(&r, 0, sizeof(r));
        for (int l = 0; l < a.n_layers; ++l) {
            const MoeDownArgs::Layer &A = a.layer[l];
            r.layer[l] = DrLayer{A.w, A.h, A.ids, A.cw, A.out, (int32_t *)A.ws};
        }
        r.n_layers = a.n_layers;
        r.emit = ep;
        r.n_used = (int)a.n_used; r.n_slots = (int)n_slots; r.n_expert = (int)a.n_expert;
        r.nb = (int)nb; r.n_ff = (int)a.n_ff; r.n_rows = (int)a.n_embd;
        r.R = (int)(64 / (nb / 4));
        r.wgs_per_layer = (int)((a.n_embd + r.R - 1) / r.R);
        const size_t lds = (size_t)kRowWaves * kStageBytes + (size_t)kRowsMaxSlots * nb * kBlockBytes +
                           (size_t)kRowsMaxSlots * nb * 4;
        if (lds > (size_t)max_lds_bytes()) return -4;
        const int64_t grid = (int64_t)a.n_layers * r.wgs_per_layer;
        if (grid > 0x7fffffff) return -4;
        if (emit)
            hipLaunchKernelGGL(moe_down_rows_kernel<true>, dim3((unsigned)grid), dim3(kRowThreads), lds,
                               stream, r);
        else
            hipLaunchKernelGGL(moe_down_rows_kernel<false>, dim3((unsigned)grid), dim3(kRowThreads), lds,
                               stream, r);
        return hipGetLastError() == hipSuccess ? 0 : -6;
    }
    DnParams p;
    memset(&p, 0, sizeof(p));
    CbParams cb;
    memset(&cb, 0, sizeof(cb));
    for (int l = 0; l < a.n_layers; ++l) {
        const MoeDownArgs::Layer &A = a.layer[l];
        float *yslot = (float *)((uint8_t *)A.ws + 256);
        p.layer[l] = DnLayer{A.w, A.h, A.ids, yslot, (int32_t *)A.ws};
        cb.layer[l] = CbLayer{yslot, A.ids, A.cw, A.out};
    }
    p.n_layers = a.n_layers;
    p.emit = ep;
    p.n_slots = (int)(a.n_tok * a.n_used);
    p.n_used = (int)a.n_used;
    p.n_expert = (int)a.n_expert;
    p.nb = (int)nb;
    p.n_ff = (int)a.n_ff;
    p.n_rows = (int)a.n_embd;
    p.R = fast ? (int)(64 / (nb / 4)) : 1;
    p.tiles_per_expert = (p.n_rows + p.R - 1) / p.R;
    const int64_t active = a.n_layers * (a.n_expert < p.n_slots ? a.n_expert : p.n_slots);
    p.tiles_per_wg = tiles_per_wg_for(active, p.tiles_per_expert);
    p.wgs_per_expert = (p.tiles_per_expert + p.tiles_per_wg - 1) / p.tiles_per_wg;
    p.wgs_per_layer = p.n_slots * p.wgs_per_expert;
    const int64_t grid = (int64_t)a.n_layers * p.wgs_per_layer;
    int rc;
    if (fast && grid > 0x7fffffff) return -4;
    if (!fast) {
        const size_t lds = (size_t)nb * kBlockBytes;
        if (lds > (size_t)max_lds_bytes()) return -4;
        dim3 g((unsigned)p.n_slots, (unsigned)((p.n_rows + kWaves - 1) / kWaves), (unsigned)a.n_layers);
        hipLaunchKernelGGL(moe_down_generic_kernel, g, dim3(kThreads), lds, stream, p);
        rc = hipGetLastError() == hipSuccess ? 0 : -6;
    } else switch (pick_mt(a.n_tok)) {
        case 1: rc = launch_dn_mt<1>(p, (int)grid, stream, emit); break;
        case 2: rc = launch_dn_mt<2>(p, (int)grid, stream, emit); break;
        default: rc = launch_dn_mt<4>(p, (int)grid, stream, emit); break;
    }
    if (rc) return rc;
    cb.n_rows = (int)a.n_embd;
    cb.n_used = (int)a.n_used;
    cb.n_expert = (int)a.n_expert;
    return launch_combine(cb, a.n_layers, a.n_tok, stream);
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
