// moe_r8.hip -- the decode expert FFN over expert weights in the R8 layout.
//
// What is computed is the expert FFN of moe.hip (Gemma-4-on-Xeon page,
// "GPUなしで13年前のXeon上でGemma 4 26Bを毎秒5トークンで実行する": the section on
// the broken op paths and the three-part fix, runtime graph fallback):
//   h[t][u][j] = silu(W_ug[e][j] . q(x_t)) * (W_ug[e][n_ff+j] . q(x_t)),  e = ids[t][u]
//   out[t]     = sum over u ascending of cw[t][u] * (W_d[e] . q(h[t][u]))
// with the weights repacked once into the row-interleaved R8 layout (r8.hip;
// the startup repack of the same page, section on the fallback's cost and the
// repacking bug): the combined up_gate tensor as n_expert*2*n_ff rows, the
// down tensor as n_expert*n_embd rows (every expert starts on a group).
//
// One token: two launches per call (several layers of one shape per launch):
//  1. up_gate: workgroup = (slot, 32 columns of h), 8 waves, one 8-row group
//     each: waves 0..3 the gate rows, waves 4..7 the up rows of the same
//     columns.  The token row is quantized into LDS by the workgroup (bytes of
//     q8_0_quantize_rows); the up sums meet the gate sums in LDS, silu(g)*u is
//     written to h, and the 32 h values (one Q8_0 block of the h row) are
//     quantized by the same rule into the workspace for the down launch.
//  2. down + combine: workgroup = (token, 32 output rows), one wave per active
//     slot of the token streaming that slot's expert rows (4 consecutive groups
//     as one stream of slices) against the slot's quantized h row; the n_used
//     results are combined in LDS in ascending u.
// At one token the slots name distinct experts and each streams its own.
// Several tokens: three launches (the expert-major kernels below, then the
// combine of the native path), each active expert's rows streamed once per
// call for all of its slots.
//
// Ids outside [0, n_expert): the up_gate workgroup of slot 0 / columns 0 sets
// the error word of the workspace (0 or 1, every call); such a slot's h row is
// NaN, and every output row of its token is NaN.
#include <string.h>

#include <mutex>
#include <type_traits>

#include "q8_device.h"
#include "q8_internal.h"
#include "q8_moe.h"

namespace q8 {

namespace {

constexpr int kGB = 8 * kBlockBytes;      // bytes per block column of an 8-row group
constexpr int kMrSlices = 8;              // 1 KB slices of a group in flight per wave
#ifndef Q8_MR_UG_SLICES
#define Q8_MR_UG_SLICES 8
#endif
#ifndef Q8_MR_UG_ONE_LAYER_SLICES
#define Q8_MR_UG_ONE_LAYER_SLICES 16   // up_gate launches of a single layer
#endif

// One 8-row group of nb blocks against an activation row in LDS (codes
// realigned to 32 bytes per block, binary16 scale bits); slice i, lane l:
// row (l>>1)&7, block 4i + (l>>4), half l&1.  Returns the lane's partial sum
// (blocks of its residue, ascending); the caller adds lanes l, l^16, l^32.
// EMIT (validation): every exact block sum is also written to srow[b], the
// sums row of this lane's weight row (lanes that hold a whole sum).
template <int POL, bool EMIT = false, int SL = kMrSlices>
struct GroupStream {
    __amdgpu_buffer_rsrc_t rs;
    int code0, scale0, nb;
    int32_t *srow = nullptr;
    u32x4 c[SL];
    uint32_t sb[SL];

    __device__ __forceinline__ void init(const uint8_t *group, int nb_, int lane, bool live)
    {
        nb = nb_;
        rs = __builtin_amdgcn_make_buffer_rsrc((void *)wave_uniform(group), 0,
                                               wave_uniform(live ? kGB * nb : 0), kBufferWord3);
        code0 = 16 * nb + 16 * lane;
        scale0 = 2 * (lane >> 1);
    }
    __device__ __forceinline__ void issue(int i0)
    {
#pragma unroll
        for (int u = 0; u < SL; ++u)
            c[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, code0 + 1024 * (i0 + u), 0, POL);
#pragma unroll
        for (int u = 0; u < SL; ++u)
            sb[u] = __builtin_amdgcn_raw_buffer_load_b16(rs, scale0 + 64 * (i0 + u), 0, POL);
    }
    // every slice is computed (a branch would make the compiler wait for each
    // load in turn): slices past the group read zero codes, scales masked
    __device__ __forceinline__ void compute(int i0, int lane, const uint8_t *xc,
                                            const uint16_t *xd16, float &acc)
    {
        const int half = lane & 1, bs = lane >> 4;
#pragma unroll
        for (int u = 0; u < SL; ++u) {
            const int b = 4 * (i0 + u) + bs;
            const bool live = b < nb;
            const int bb = live ? b : nb - 1;
            const u32x4 xv = *(const u32x4 *)(xc + 32 * bb + 16 * half);
            int s = sdot4(c[u].x, xv.x, 0);
            s = sdot4(c[u].y, xv.y, s);
            s = sdot4(c[u].z, xv.z, s);
            s = sdot4(c[u].w, xv.w, s);
            s += __builtin_amdgcn_mov_dpp(s, 0xB1, 0xF, 0xF, false);   // the other half
            if (EMIT && half == 0 && live) srow[b] = s;
            const float dw = live ? half_bits_to_float(sb[u]) : 0.0f;
            acc = fmaf(dw * half_bits_to_float(xd16[bb]), (float)s, acc);
        }
    }
    // the whole group after the first issue(0)
    __device__ __forceinline__ float run(int lane, const uint8_t *xc, const uint16_t *xd16)
    {
        const int slices = (nb + 3) >> 2;
        float acc = 0.0f;
        for (int i0 = 0;;) {
            compute(i0, lane, xc, xd16, acc);
            i0 += SL;
            if (i0 >= slices) break;
            issue(i0);
        }
        acc += __shfl_xor(acc, 16);
        acc += __shfl_xor(acc, 32);
        return acc;            // lanes with (lane & 0x31) == 0: row (lane >> 1) & 7
    }
};

// kDnG consecutive 8-row groups of one expert (contiguous in memory) as one
// stream of slices: flattened slice j = q*S + i is slice i of group q (S
// slices per group), so short groups still keep 8 slices in flight; each
// group accumulates its own blocks in ascending order.
constexpr int kDnG = 4;

// EMIT (validation): block sums to sbase[(8q + r) * nb + b] for group q, row r.
template <int POL, bool EMIT = false, int G = kDnG>
struct MultiStream {
    __amdgpu_buffer_rsrc_t rs;
    int nb, S, total, gb;
    int32_t *sbase = nullptr;
    u32x4 c[kMrSlices];
    uint32_t sb[kMrSlices];

    __device__ __forceinline__ void init(const uint8_t *base, int nb_)
    {
        nb = nb_;
        gb = kGB * nb;
        S = (nb + 3) >> 2;
        total = G * S;
        rs = __builtin_amdgcn_make_buffer_rsrc((void *)wave_uniform(base), 0,
                                               wave_uniform(G * gb), kBufferWord3);
    }
    __device__ __forceinline__ void issue(int j0, int lane)
    {
#pragma unroll
        for (int u = 0; u < kMrSlices; ++u) {
            const int j = j0 + u;                  // uniform
            const int q = j / S, i = j - q * S;
            const int off = j < total ? q * gb + 16 * nb + 1024 * i + 16 * lane : 0x7ffffff0;
            c[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, POL);
        }
#pragma unroll
        for (int u = 0; u < kMrSlices; ++u) {
            const int j = j0 + u;
            const int q = j / S, i = j - q * S;
            const int off = j < total ? q * gb + 64 * i + 2 * (lane >> 1) : 0x7ffffff0;
            sb[u] = __builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, POL);
        }
    }
    __device__ __forceinline__ void compute(int j0, int lane, const uint8_t *xc,
                                            const uint16_t *xd16, float (&acc)[G])
    {
        const int half = lane & 1, bs = lane >> 4;
#pragma unroll
        for (int u = 0; u < kMrSlices; ++u) {
            const int j = j0 + u;
            const int q = j / S, i = j - q * S;
            const int b = 4 * i + bs;
            const bool live = j < total && b < nb;
            const int bb = b < nb ? b : nb - 1;
            const u32x4 xv = *(const u32x4 *)(xc + 32 * bb + 16 * half);
            int s = sdot4(c[u].x, xv.x, 0);
            s = sdot4(c[u].y, xv.y, s);
            s = sdot4(c[u].z, xv.z, s);
            s = sdot4(c[u].w, xv.w, s);
            s += __builtin_amdgcn_mov_dpp(s, 0xB1, 0xF, 0xF, false);   // the other half
            if (EMIT && half == 0 && live) sbase[(8 * q + ((lane >> 1) & 7)) * nb + b] = s;
            const float dw = live ? half_bits_to_float(sb[u]) : 0.0f;
            const float p = dw * half_bits_to_float(xd16[bb]);
#pragma unroll
            for (int g = 0; g < G; ++g)
                if (q == g) acc[g] = fmaf(p, (float)s, acc[g]);
        }
    }
    __device__ __forceinline__ void run(int lane, const uint8_t *xc, const uint16_t *xd16,
                                        float (&acc)[G])
    {
#pragma unroll
        for (int g = 0; g < G; ++g) acc[g] = 0.0f;
        for (int j0 = 0;;) {
            compute(j0, lane, xc, xd16, acc);
            j0 += kMrSlices;
            if (j0 >= total) break;
            issue(j0, lane);
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            acc[g] += __shfl_xor(acc[g], 16);
            acc[g] += __shfl_xor(acc[g], 32);
        }
    }
};

// ---------------------------------------------------------------------------
// up_gate

constexpr int kUgWaves = 8;
constexpr int kUgThreads = kUgWaves * kWave;
constexpr int kUgQBlocks = kUgThreads / 8;     // activation blocks quantized per pass

struct MrUgArgs {
    struct Layer {
        const uint8_t *w;      // R8 up_gate
        const float *x;        // [n_tok][n_embd]
        const int32_t *ids;
        float *h;              // [n_tok][n_used][n_ff]
        uint8_t *ws;           // error word, then q(h) rows [slot][n_ff/32] blocks
    } layer[kMoeMaxLayers];
    int n_used, n_slots, n_embd, n_ff, n_expert;
    int wg_per_layer;
    int32_t *sums;             // validation: [slot][2*n_ff][n_embd/32] (layer 0 only)
    int32_t *counts, *pairs;   // validation, several tokens: the expert-major grouping
    int ug_cols;               // several tokens: 8-column groups per wave
};

template <int POL, bool EMIT, int SL = Q8_MR_UG_SLICES>
__global__ __launch_bounds__(kUgThreads) void moe_r8_up_gate_kernel(const MrUgArgs a)
{
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int li = wave_uniform((int)blockIdx.x / a.wg_per_layer);
    const int rel = (int)blockIdx.x - li * a.wg_per_layer;
    const int cols = a.n_ff / 32;
    const int slot = rel / cols;
    const int p = rel - slot * cols;
    const auto &L = a.layer[li];
    const int nb = a.n_embd / 32;
    const int e = wave_uniform(L.ids[slot]);
    const bool valid = e >= 0 && e < a.n_expert;

    if (slot == 0 && p == 0 && tid < kWave) {
        int bad = 0;
        for (int s = lane; s < a.n_slots; s += kWave) {
            const int v = L.ids[s];
            bad |= (v < 0 || v >= a.n_expert);
        }
        bad = __any(bad);
        if (lane == 0) *(int32_t *)L.ws = bad;
    }
    float *hrow = L.h + (int64_t)slot * a.n_ff + 32 * p;
    if (!valid) {
        if (tid < 32) hrow[tid] = __builtin_nanf("");
        return;
    }

    // gate groups 4p..4p+3 (waves 0..3), up groups n_ff/8 + 4p.. (waves 4..7)
    const int grp = wave < 4 ? 4 * p + wave : a.n_ff / 8 + 4 * p + (wave - 4);
    const uint8_t *gbase = L.w + ((int64_t)e * (2 * a.n_ff / 8) + grp) * kGB * nb;

    extern __shared__ __align__(16) uint8_t mr_lds[];
    uint8_t *xc = mr_lds;
    uint16_t *xd16 = (uint16_t *)(mr_lds + 32 * nb);
    float *upv = (float *)(mr_lds + (34 * nb + 15) / 16 * 16);   // 16-byte aligned
    float *hv = upv + 32;

    // the token row: loads first, then the weights, then the quantization
    const float *xf = L.x + (int64_t)(slot / a.n_used) * a.n_embd;
    const int q8 = tid & 7;
    const int passes = (nb + kUgQBlocks - 1) / kUgQBlocks;
    auto load_pass = [&](int ps) {
        const int b = min((tid >> 3) + kUgQBlocks * ps, nb - 1);
        return *(const float4 *)(xf + 32 * b + 4 * q8);
    };
    auto quantize_pass = [&](int ps, float4 v) {
        const int b = (tid >> 3) + kUgQBlocks * ps;
        uint32_t codes, dbits;
        quantize_block8(v.x, v.y, v.z, v.w, codes, dbits);
        if (b < nb) {
            *(uint32_t *)(xc + 32 * b + 4 * q8) = codes;
            if (q8 == 0) xd16[b] = (uint16_t)dbits;
        }
    };
    GroupStream<POL, EMIT, SL> gs;
    gs.init(gbase, nb, lane, true);
    if (EMIT) gs.srow = a.sums + ((int64_t)slot * 2 * a.n_ff + 8 * grp + ((lane >> 1) & 7)) * nb;
    if (passes <= 2) {
        const float4 v0 = load_pass(0);
        const float4 v1 = load_pass(passes > 1 ? 1 : 0);
        __builtin_amdgcn_sched_barrier(0);
        gs.issue(0);
        __builtin_amdgcn_sched_barrier(0);
        quantize_pass(0, v0);
        if (passes > 1) quantize_pass(1, v1);
    } else {
        for (int ps = 0; ps < passes; ++ps) quantize_pass(ps, load_pass(ps));
        gs.issue(0);
    }
    __syncthreads();

    const float acc = gs.run(lane, xc, xd16);
    const bool holder = (lane & 0x31) == 0;
    const int r = (lane >> 1) & 7;
    if (wave >= 4 && holder) upv[8 * (wave - 4) + r] = acc;
    __syncthreads();
    if (wave < 4 && holder) {
        const float g = acc;
        const float hval = g / (1.0f + expf(-g)) * upv[8 * wave + r];
        hrow[8 * wave + r] = hval;
        hv[8 * wave + r] = hval;
    }
    __syncthreads();
    // the 32 h values of this workgroup are block p of the slot's h row
    if (wave == 0) {
        const int l8 = lane & 7;
        const float4 v = *(const float4 *)(hv + 4 * l8);
        uint32_t codes, dbits;
        quantize_block8(v.x, v.y, v.z, v.w, codes, dbits);
        if (lane < 8) {
            uint16_t *blk = (uint16_t *)(L.ws + 256 + ((int64_t)slot * cols + p) * kBlockBytes);
            if (lane == 0) blk[0] = (uint16_t)dbits;
            blk[1 + 2 * lane] = (uint16_t)(codes & 0xffffu);
            blk[2 + 2 * lane] = (uint16_t)(codes >> 16);
        }
    }
}

// ---------------------------------------------------------------------------
// down + combine

struct MrDnArgs {
    struct Layer {
        const uint8_t *w;      // R8 down
        const int32_t *ids;
        const float *cw;
        float *out;            // [n_tok][n_embd]
        const uint8_t *ws;     // q(h) rows at +256
    } layer[kMoeMaxLayers];
    int n_used, n_embd, n_ff, n_expert;
    int wg_per_layer;
    int32_t *sums;             // validation: [slot][n_embd][n_ff/32] (layer 0 only)
};

// G: 8-row groups of the output per workgroup (4 normally; 1 when a launch
// would otherwise have too few workgroups to keep the memory system busy).
template <int POL, bool EMIT, int G>
__global__ __launch_bounds__(1024) void moe_r8_down_kernel(const MrDnArgs a)
{
    const int tid = threadIdx.x;
    const int wave = tid >> 6;                 // = the slot u of the token
    const int lane = tid & 63;
    const int li = wave_uniform((int)blockIdx.x / a.wg_per_layer);
    const int rel = (int)blockIdx.x - li * a.wg_per_layer;
    const int quads = a.n_embd / (8 * G);      // bands of 8*G output rows
    const int t = rel / quads;
    const int g = rel - t * quads;
    const auto &L = a.layer[li];
    const int nb = a.n_ff / 32;
    const int U = a.n_used;

    // a token with any out-of-range id gets NaN outputs
    int bad = 0;
    for (int u = 0; u < U; ++u) {
        const int v = L.ids[t * U + u];
        bad |= (v < 0 || v >= a.n_expert);
    }
    float *orow = L.out + (int64_t)t * a.n_embd + 8 * G * g;
    if (bad) {
        if (tid < 8 * G) orow[tid] = __builtin_nanf("");
        return;
    }
    const int e = wave_uniform(L.ids[t * U + wave]);
    const uint8_t *gbase = L.w + ((int64_t)e * (a.n_embd / 8) + G * g) * kGB * nb;

    // this wave's q(h) row in its own LDS region: loads first, then the
    // weights, then the LDS writes (waves do not share these regions)
    extern __shared__ __align__(16) uint8_t mr_lds[];
    const int region = (34 * nb + 15) / 16 * 16;   // 16-byte aligned per wave
    uint8_t *xc = mr_lds + wave * region;
    uint16_t *xd16 = (uint16_t *)(xc + 32 * nb);
    float *ybuf = (float *)(mr_lds + 16 * region);
    const uint8_t *hq = L.ws + 256 + ((int64_t)t * U + wave) * nb * kBlockBytes;
    constexpr int kHLoads = 16;                // 2-byte code pairs per lane (nb <= 64)
    uint32_t hv[kHLoads];
#pragma unroll
    for (int i = 0; i < kHLoads; ++i) {
        const int e2 = min(lane + kWave * i, 16 * nb - 1);
        hv[i] = *(const uint16_t *)(hq + (e2 >> 4) * kBlockBytes + 2 + 2 * (e2 & 15));
    }
    const uint32_t hs = *(const uint16_t *)(hq + min(lane, nb - 1) * kBlockBytes);
    MultiStream<POL, EMIT, G> ms;
    ms.init(gbase, nb);
    if (EMIT) ms.sbase = a.sums + ((int64_t)(t * U + wave) * a.n_embd + 8 * G * g) * nb;
    __builtin_amdgcn_sched_barrier(0);
    ms.issue(0, lane);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kHLoads; ++i) {
        const int e2 = lane + kWave * i;
        if (e2 < 16 * nb) ((uint16_t *)xc)[e2] = (uint16_t)hv[i];
    }
    if (lane < nb) xd16[lane] = (uint16_t)hs;
    wave_lds_sync();

    float acc[G];
    ms.run(lane, xc, xd16, acc);
    if ((lane & 0x31) == 0) {
#pragma unroll
        for (int q = 0; q < G; ++q) ybuf[8 * G * wave + 8 * q + ((lane >> 1) & 7)] = acc[q];
    }
    __syncthreads();
    if (tid < 8 * G) {
        float o = 0.0f;
        for (int u = 0; u < U; ++u) o = fmaf(L.cw[t * U + u], ybuf[8 * G * u + tid], o);
        orow[tid] = o;
    }
}

// ---------------------------------------------------------------------------
// one token, one layer per launch (a model's layers one after another): the
// up_gate product, q(h) and the down product in one launch
//
// Workgroup (slot u, h block p), as in moe_r8_up_gate_kernel up to the Q8_0
// block of its 32 h values.  It then multiplies that block with block p of
// every row of the slot's expert down matrix -- the block term (d_w * d_h) * s
// of each row, s the exact int32 block sum -- and writes the n_embd terms to
// terms[u][p][.] in the workspace (agent-scope stores: visible to every XCD
// once complete).  The down rows' block p is prefetched with the up_gate
// slices, before the token row is quantized, so the launch streams both
// matrices from its start.  Then every workgroup takes a ticket (agent-scope
// atomic add, after its stores have completed); the last R workgroups to
// finish each sum bands of 32 output rows once every ticket is out:
//   y[u][row] = terms[u][p][row] summed over p ascending,
//   out[row]  = fused multiply-adds of cw[u] * y[u][row], u ascending,
// and the last of them returns the two counters to zero for the next call.
// A workgroup waits only after its own work, for workgroups that are running
// or not yet started (all others are done), so the wait ends; it is bounded
// anyway (kFzMaxPolls polls, then bit 1 of the error word).
// Per block the arithmetic is that of the down kernel; the sum over the
// blocks of a row is taken in another order, so out matches the two-launch
// form within rounding, not bit for bit (h is the same bits).
// Measured on the Gemma-4-26B-A4B expert shape, 30 layers one after another:
// 558-566 us per step against 437-457 us for two launches per layer; ending
// every workgroup after its terms (timing-only copies) gave 402-417 us, so
// the summation's chain of round trips (store completion, ticket, wait,
// agent-scope reads) costs about 5 us per layer, more than the launch saved.

#ifndef Q8_FZ_SLICES
#define Q8_FZ_SLICES 8            // up_gate slices in flight per wave
#endif
constexpr int kFzMaxPolls = 1 << 16;
constexpr int kFzBatches = 8;     // down loads in flight per wave: 4 groups x 256 bytes each

struct MrFzArgs {
    const uint8_t *w_ug, *w_dn;    // R8 up_gate and down tensors
    const float *x;                // [n_embd]
    const int32_t *ids;            // [n_used]
    const float *cw;               // [n_used]
    float *h;                      // [n_used][n_ff]
    float *out;                    // [n_embd]
    uint8_t *ws;                   // error word, tickets, bands done; terms at +256
    int n_used, n_embd, n_ff, n_expert;
    int reducers;
};

__device__ __forceinline__ void st_agent_f32(float *p, float v)
{
    __hip_atomic_store((int32_t *)p, __builtin_bit_cast(int32_t, v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float ld_agent_f32(const float *p)
{
    return __builtin_bit_cast(float, __hip_atomic_load((const int32_t *)p, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT));
}

template <int POL>
__global__ __launch_bounds__(kUgThreads) void moe_r8_fused_kernel(const MrFzArgs a)
{
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int cols = a.n_ff / 32;                  // h blocks per slot
    const int slot = (int)blockIdx.x / cols;
    const int p = (int)blockIdx.x - slot * cols;
    const int total = a.n_used * cols;
    const int nb = a.n_embd / 32;                  // blocks of the token row
    const int e = wave_uniform(a.ids[slot]);
    const bool valid = e >= 0 && e < a.n_expert;
    int32_t *err = (int32_t *)a.ws;
    int32_t *tickets = err + 1;
    int32_t *bands_done = err + 2;
    float *terms = (float *)(a.ws + 256);
    float *trow = terms + (int64_t)(slot * cols + p) * a.n_embd;

    if (blockIdx.x == 0 && tid < kWave) {
        int bad = 0;
        for (int s = lane; s < a.n_used; s += kWave) {
            const int v = a.ids[s];
            bad |= (v < 0 || v >= a.n_expert);
        }
        bad = __any(bad);
        if (lane == 0) __hip_atomic_store(err, bad, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    extern __shared__ __align__(16) uint8_t mr_lds[];
    uint8_t *xc = mr_lds;
    uint16_t *xd16 = (uint16_t *)(mr_lds + 32 * nb);
    float *upv = (float *)(mr_lds + (34 * nb + 15) / 16 * 16);
    float *hv = upv + 32;
    uint32_t *hq = (uint32_t *)(hv + 32);          // the q(h) block: 8 code dwords, then the scale
    float *ybuf = (float *)(hq + 12);              // reducer: [n_used][32]
    float *hrow = a.h + (int64_t)slot * a.n_ff + 32 * p;

    if (valid) {
        // gate groups 4p..4p+3 (waves 0..3), up groups n_ff/8 + 4p.. (waves 4..7)
        const int grp = wave < 4 ? 4 * p + wave : a.n_ff / 8 + 4 * p + (wave - 4);
        const uint8_t *gbase = a.w_ug + ((int64_t)e * (2 * a.n_ff / 8) + grp) * kGB * nb;
        // down rows of the expert: n_embd/8 groups of cols blocks (n_embd % 256
        // == 0); wave w takes groups [gw0, gw0 + gpw), 4 per load, batch jj
        // (lane: group gw0 + 4jj + (lane >> 4), row (lane >> 1) & 7, half
        // lane & 1 of block p); a batch past the wave's groups reloads its
        // last one and is not used
        const int G = a.n_embd / 8;
        const int gpw = G / kUgWaves;
        const int gw0 = wave * gpw;
        const int dgb = kGB * cols;
        const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(a.w_dn + (int64_t)e * G * dgb), 0, G * dgb, kBufferWord3);
        const int nbat = gpw >> 2;
        u32x4 dc[kFzBatches];
        uint32_t ds[kFzBatches];
        auto d_issue = [&](int j0) {
#pragma unroll
            for (int j = 0; j < kFzBatches; ++j) {
                const int jj = min(j0 + j, nbat - 1);
                const int g = gw0 + 4 * jj + (lane >> 4);
                dc[j] = __builtin_amdgcn_raw_buffer_load_b128(
                    rd, g * dgb + 16 * cols + 256 * p + 16 * (lane & 15), 0, POL);
                ds[j] = __builtin_amdgcn_raw_buffer_load_b16(rd, g * dgb + 16 * p + 2 * ((lane >> 1) & 7),
                                                             0, POL);
            }
        };

        const float *xf = a.x;
        const int q8 = tid & 7;
        const int passes = (nb + kUgQBlocks - 1) / kUgQBlocks;
        auto load_pass = [&](int ps) {
            const int b = min((tid >> 3) + kUgQBlocks * ps, nb - 1);
            return *(const float4 *)(xf + 32 * b + 4 * q8);
        };
        auto quantize_pass = [&](int ps, float4 v) {
            const int b = (tid >> 3) + kUgQBlocks * ps;
            uint32_t codes, dbits;
            quantize_block8(v.x, v.y, v.z, v.w, codes, dbits);
            if (b < nb) {
                *(uint32_t *)(xc + 32 * b + 4 * q8) = codes;
                if (q8 == 0) xd16[b] = (uint16_t)dbits;
            }
        };
        GroupStream<POL, false, Q8_FZ_SLICES> gs;
        gs.init(gbase, nb, lane, true);
        if (passes <= 2) {
            const float4 v0 = load_pass(0);
            const float4 v1 = load_pass(passes > 1 ? 1 : 0);
            __builtin_amdgcn_sched_barrier(0);
            gs.issue(0);
            d_issue(0);
            __builtin_amdgcn_sched_barrier(0);
            quantize_pass(0, v0);
            if (passes > 1) quantize_pass(1, v1);
        } else {
            for (int ps = 0; ps < passes; ++ps) quantize_pass(ps, load_pass(ps));
            gs.issue(0);
            d_issue(0);
        }
        __syncthreads();

        const float acc = gs.run(lane, xc, xd16);
        const bool holder = (lane & 0x31) == 0;
        const int r = (lane >> 1) & 7;
        if (wave >= 4 && holder) upv[8 * (wave - 4) + r] = acc;
        __syncthreads();
        if (wave < 4 && holder) {
            const float g = acc;
            const float hval = g / (1.0f + expf(-g)) * upv[8 * wave + r];
            hrow[8 * wave + r] = hval;
            hv[8 * wave + r] = hval;
        }
        __syncthreads();
        if (wave == 0) {
            const int l8 = lane & 7;
            const float4 v = *(const float4 *)(hv + 4 * l8);
            uint32_t codes, dbits;
            quantize_block8(v.x, v.y, v.z, v.w, codes, dbits);
            if (lane < 8) hq[l8] = codes;
            if (lane == 0) hq[8] = dbits;
        }
        __syncthreads();

        // the down terms of block p: one 8-row group per 16 lanes and batch
        const int half = lane & 1;
        const u32x4 hx = *(const u32x4 *)(hq + 4 * half);
        const float dh = half_bits_to_float(hq[8]);
        for (int j0 = 0;;) {
#pragma unroll
            for (int j = 0; j < kFzBatches; ++j) {
                int sum = sdot4(dc[j].x, hx.x, 0);
                sum = sdot4(dc[j].y, hx.y, sum);
                sum = sdot4(dc[j].z, hx.z, sum);
                sum = sdot4(dc[j].w, hx.w, sum);
                sum += __builtin_amdgcn_mov_dpp(sum, 0xB1, 0xF, 0xF, false);   // the other half
                const int row = 8 * (gw0 + 4 * (j0 + j) + (lane >> 4)) + ((lane >> 1) & 7);
                if (half == 0 && j0 + j < nbat)
                    st_agent_f32(trow + row, fmaf(half_bits_to_float(ds[j]) * dh, (float)sum, 0.0f));
            }
            j0 += kFzBatches;
            if (j0 >= nbat) break;
            d_issue(j0);
        }
    } else {
        if (tid < 32) hrow[tid] = __builtin_nanf("");
        for (int i = tid; i < a.n_embd; i += kUgThreads) st_agent_f32(trow + i, __builtin_nanf(""));
    }

    // this workgroup's terms are complete at agent scope: take a ticket
    __builtin_amdgcn_s_waitcnt(0);
    __shared__ int s_ticket;
    __syncthreads();
    if (tid == 0)
        s_ticket = __hip_atomic_fetch_add(tickets, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int R = a.reducers;
    const int ri = s_ticket - (total - R);
    if (ri < 0) return;
    if (tid == 0) {
        int polls = 0;
        while (__hip_atomic_load(tickets, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < total) {
            if (++polls > kFzMaxPolls) {
                __hip_atomic_fetch_or(err, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
    }
    __syncthreads();
    for (int band = ri; band < a.n_embd / 32; band += R) {
        if (tid < 32 * a.n_used) {
            const int u = tid >> 5, rr = tid & 31;
            const float *src = terms + (int64_t)u * cols * a.n_embd + 32 * band + rr;
            float y = 0.0f;
#pragma unroll 8
            for (int q = 0; q < cols; ++q) y += ld_agent_f32(src + (int64_t)q * a.n_embd);
            ybuf[32 * u + rr] = y;
        }
        __syncthreads();
        if (tid < 32) {
            float o = 0.0f;
            for (int u = 0; u < a.n_used; ++u) o = fmaf(a.cw[u], ybuf[32 * u + tid], o);
            a.out[32 * band + tid] = o;
        }
        __syncthreads();
    }
    if (tid == 0) {
        const int d = __hip_atomic_fetch_add(bands_done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (d == R - 1) {
            __hip_atomic_store(tickets, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(bands_done, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// ---------------------------------------------------------------------------
// several tokens: each active expert's rows streamed once per call
//
// With more than one token, slots repeat experts (at 16 tokens, 8 of 128
// experts each, about a third of the slots).  The workgroups keep a
// (slot, part) layout, but the workgroup of slot s works only when s is the
// first slot naming its expert e (one ballot pass of wave 0 over the ids): it
// then serves every slot routed to e, ascending, kGtMax slots against each
// pass over its part of the rows; the other workgroups exit.  Each wave
// streams several 8-row groups as one rolling stream (slice u of the next
// batch is issued as soon as slice u of the current one is consumed, so about
// 8 KB stay in flight per wave), and needs no other wave after the rows are
// staged: up_gate pairs a gate group with the up group of the same 8 columns
// in one wave, and the down kernel quantizes h itself.  Per slot the
// arithmetic and its order are those of the one-token kernels above, so h,
// q(h) and the outputs are the same bits.  The down kernel writes one fp32
// row per slot to the workspace and the combine kernel of the native path
// (ascending u) forms out.

#ifndef Q8_GT_ROUNDS
#define Q8_GT_ROUNDS 8            // rounds of the resident waves the work per wave aims at
#endif
// up_gate slices in flight per wave: 8 (150 VGPRs, 3 waves per SIMD) against
// 16 (247 VGPRs, 2 waves per SIMD) at 16 tokens: 2.42 against 2.74 ms per
// 30-layer step layer after layer, 1.89 against 1.92 ms with all 30 layers
// in one call (6: 2.41 / 1.91 ms, 4: 2.46 / 1.90 ms)
#ifndef Q8_GT_SLICES
#define Q8_GT_SLICES 8
#endif
#ifndef Q8_GT_UG_OCC
#define Q8_GT_UG_OCC 2
#endif
#ifndef Q8_GT_DN_OCC
#define Q8_GT_DN_OCC 4
#endif
constexpr int kGtMax = 4;          // slots per pass over an expert's rows
constexpr int kGtIdRegs = 4;       // ids held in registers per lane of wave 0
#ifndef Q8_GT_DN_SLICES
#define Q8_GT_DN_SLICES 6
#endif
constexpr int kGtSlices = Q8_GT_SLICES;      // up_gate: 1 KB slices in flight per wave
constexpr int kGtDnSlices = Q8_GT_DN_SLICES; // down
#ifndef Q8_GT_UG_WAVES
#define Q8_GT_UG_WAVES 4
#endif
#ifndef Q8_GT_DN_WAVES
#define Q8_GT_DN_WAVES 4
#endif
constexpr int kGtUgWaves = Q8_GT_UG_WAVES;        // waves of an up_gate workgroup
constexpr int kGtDnWaves = Q8_GT_DN_WAVES;        // waves of a down workgroup
constexpr int kGtOwnPre = 2;                      // blocks of the own row per 8 lanes, prefetched

struct GtPick {
    int count;                     // slots served (0: not the owner)
    int less;                      // in-range slots with an id below e
};

// Wave 0 only: the ids in registers (loaded before anything else).
struct GtIds {
    int v[kGtIdRegs];
};

__device__ __forceinline__ void gt_load_ids(const int32_t *ids, int n_slots, GtIds &g)
{
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int c = 0; c < kGtIdRegs; ++c) g.v[c] = ids[min(c * kWave + lane, n_slots - 1)];
}

// Wave 0 only.  list[] gets the slots naming e in ascending order.
__device__ __forceinline__ void gt_pick(const int32_t *ids, const GtIds &g, int n_slots,
                                        int n_expert, int s, int e, int *list, GtPick &pk)
{
    const int lane = threadIdx.x & (kWave - 1);
    int cnt = 0, less = 0;
    bool first = true;
    auto step = [&](int i, int id) {
        const bool in = i < n_slots;
        const bool hit = in && id == e;
        const uint64_t m = __ballot(hit);
        first &= __ballot(hit && i < s) == 0;
        less += __popcll(__ballot(in && id >= 0 && id < e));
        if (hit) list[cnt + __popcll(m & __lanemask_lt())] = i;
        cnt += __popcll(m);
    };
#pragma unroll
    for (int c = 0; c < kGtIdRegs; ++c)
        if (c * kWave < n_slots) step(c * kWave + lane, g.v[c]);
    for (int base = kGtIdRegs * kWave; base < n_slots; base += kWave) {
        const int i = base + lane;
        step(i, ids[min(i, n_slots - 1)]);
    }
    if (lane == 0) {
        pk.count = first ? cnt : 0;
        pk.less = less;
    }
}

__host__ __device__ inline int gt_row_stride(int nb)
{
    return (34 * nb + 15) / 16 * 16;
}

// kGtMax activation rows, then the slot list
size_t gt_lds(int64_t n_slots, int64_t nb)
{
    return (size_t)kGtMax * gt_row_stride((int)nb) + (size_t)n_slots * 4;
}

// Quantize one 32-value block (4 values in each of 8 lanes) into LDS row xc
// (codes realigned to 32 bytes per block, binary16 scale bits at +32*nb).
__device__ __forceinline__ void gt_put(uint8_t *xc, int nb, int b, float4 v)
{
    const int q8 = threadIdx.x & 7;
    uint32_t codes, dbits;
    quantize_block8(v.x, v.y, v.z, v.w, codes, dbits);
    if (b < nb) {
        *(uint32_t *)(xc + 32 * b + 4 * q8) = codes;
        if (q8 == 0) ((uint16_t *)(xc + 32 * nb))[b] = (uint16_t)dbits;
    }
}

// The first kGtOwnPre*QB blocks of a row (QB = threads/8), 4 values per lane,
// loaded into registers ahead of the ownership scan.
template <int QB>
__device__ __forceinline__ void gt_prefetch(const float *row, int nb, float4 (&v)[kGtOwnPre])
{
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < kGtOwnPre; ++i)
        v[i] = *(const float4 *)(row + 32 * min((tid >> 3) + QB * i, nb - 1) + 4 * (tid & 7));
}

// Rows m = 0..ct-1 of a pass (fp32 row m at row_of(m)) into LDS, QB blocks
// per pass of the workgroup; row 0 may already be in registers (have_own:
// gt_prefetch of it, nb <= kGtOwnPre*QB).
template <int QB, class RowOf>
__device__ __forceinline__ void gt_stage(uint8_t *xr, int rstride, int nb, int ct, bool have_own,
                                         const float4 (&vown)[kGtOwnPre], RowOf row_of)
{
    const int tid = threadIdx.x, q8 = tid & 7;
    if (have_own) {
#pragma unroll
        for (int i = 0; i < kGtOwnPre; ++i) gt_put(xr, nb, (tid >> 3) + QB * i, vown[i]);
    }
    for (int bi = (tid >> 3) + (have_own ? nb : 0); bi < ct * nb; bi += QB) {
        const int m = bi / nb;
        const int b = bi - m * nb;
        gt_put(xr + m * rstride, nb, b, *(const float4 *)(row_of(m) + 32 * b + 4 * q8));
    }
}

// A wave's stream over ng 8-row groups of one buffer resource (group g at
// byte offset goff_of(g)) against CT activation rows in LDS (row m at xr +
// m*rstride, as gt_put leaves them).  A group is B batches of 8 slices of
// GroupStream's layout (slices past its last are issued out of range: zeros,
// no memory traffic, and masked).  Slice u of the next batch -- of this group
// or the next -- is issued right after slice u of the current batch has been
// consumed.  The first batch is issued by the caller: issue_batch(goff_of(0)).
template <int POL, bool EMIT, int SL>
struct GatherStream {
    __amdgpu_buffer_rsrc_t rs;
    int nb, S, B, size, code0, scale0;
    u32x4 c[SL];
    uint32_t sb[SL];

    __device__ __forceinline__ void init(const uint8_t *base, int nb_, int bytes, int lane)
    {
        nb = nb_;
        S = (nb + 3) >> 2;
        B = (S + SL - 1) / SL;
        size = bytes;
        rs = __builtin_amdgcn_make_buffer_rsrc((void *)wave_uniform(base), 0, wave_uniform(bytes),
                                               kBufferWord3);
        code0 = 16 * nb + 16 * lane;
        scale0 = 2 * (lane >> 1);
    }
    // slice i of the group at goff (goff < 0: none) into slot u, scale first
    __device__ __forceinline__ void issue_slice(int goff, int i, int u)
    {
        const bool in = goff >= 0 && i < S;
        sb[u] = __builtin_amdgcn_raw_buffer_load_b16(rs, in ? goff + scale0 + 64 * i : size, 0, POL);
        c[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, in ? goff + code0 + 1024 * i : size, 0, POL);
    }
    __device__ __forceinline__ void issue_batch(int goff)
    {
#pragma unroll
        for (int u = 0; u < SL; ++u) issue_slice(goff, u, u);
    }
    // epi(g, acc): the group's CT row sums, lanes with (lane & 0x31) == 0
    // holding row (lane >> 1) & 7; srow_of(g, m): the EMIT sums row
    template <int CT, class GoffOf, class SrowOf, class Epi>
    __device__ __forceinline__ void run(int ng, int lane, const uint8_t *xr, int rstride,
                                        GoffOf goff_of, SrowOf srow_of, Epi epi)
    {
        const int half = lane & 1, bs = lane >> 4;
        for (int g = 0; g < ng; ++g) {
            int32_t *srows[CT];
            float acc[CT];
#pragma unroll
            for (int m = 0; m < CT; ++m) {
                srows[m] = EMIT ? srow_of(g, m) : nullptr;
                acc[m] = 0.0f;
            }
            const int goff_next = g + 1 < ng ? goff_of(g + 1) : -1;
            const int goff_cur = goff_of(g);
            for (int kb = 0; kb < B; ++kb) {
                const bool last = kb + 1 == B;
                const int noff = last ? goff_next : goff_cur;
                const int ni0 = last ? 0 : SL * (kb + 1);
#pragma unroll
                for (int u = 0; u < SL; ++u) {
                    const int b = 4 * (SL * kb + u) + bs;
                    const bool live = b < nb;
                    const int bb = live ? b : nb - 1;
                    const float dw = live ? half_bits_to_float(sb[u]) : 0.0f;
                    const u32x4 cw = c[u];
#pragma unroll
                    for (int m = 0; m < CT; ++m) {
                        const uint8_t *xc = xr + m * rstride;
                        const u32x4 xv = *(const u32x4 *)(xc + 32 * bb + 16 * half);
                        int s = sdot4(cw.x, xv.x, 0);
                        s = sdot4(cw.y, xv.y, s);
                        s = sdot4(cw.z, xv.z, s);
                        s = sdot4(cw.w, xv.w, s);
                        s += __builtin_amdgcn_mov_dpp(s, 0xB1, 0xF, 0xF, false);   // the other half
                        if (EMIT && half == 0 && live) srows[m][b] = s;
                        const float dx = half_bits_to_float(((const uint16_t *)(xc + 32 * nb))[bb]);
                        acc[m] = fmaf(dw * dx, (float)s, acc[m]);
                        // pin the sum into its slice (else the compiler sinks the
                        // float work of every slice below the next issues)
                        asm volatile("" : "+v"(acc[m]));
                    }
                    issue_slice(noff, ni0 + u, u);
                }
            }
#pragma unroll
            for (int m = 0; m < CT; ++m) {
                acc[m] += __shfl_xor(acc[m], 16);
                acc[m] += __shfl_xor(acc[m], 32);
            }
            epi(g, acc);
        }
    }
};

// Dispatch a pass of ct (1..kGtMax) rows to the instance for that count.
template <class F>
__device__ __forceinline__ void gt_dispatch(int ct, F f)
{
    switch (ct) {
        case 1: f(std::integral_constant<int, 1>()); break;
        case 2: f(std::integral_constant<int, 2>()); break;
        case 3: f(std::integral_constant<int, 3>()); break;
        default: f(std::integral_constant<int, 4>()); break;
    }
}

// up_gate: workgroup = (slot, part of W*a.ug_cols 8-column groups of h, W the
// waves); wave w takes column groups cg = W*(a.ug_cols*part + j) + w (j < a.ug_cols),
// streaming for each the gate group cg, then the up group n_ff/8 + cg, and
// writes h of those 8 columns itself.
template <int POL, bool EMIT>
__global__ __launch_bounds__(kGtUgWaves * kWave, Q8_GT_UG_OCC) void moe_r8_up_gate_gather_kernel(const MrUgArgs a)
{
    constexpr int W = kGtUgWaves, T = W * kWave, QB = T / 8;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int li = wave_uniform((int)blockIdx.x / a.wg_per_layer);
    const int rel = (int)blockIdx.x - li * a.wg_per_layer;
    const int cgs = a.n_ff / 8;                              // 8-column groups
    const int parts = (cgs + W * a.ug_cols - 1) / (W * a.ug_cols);
    const int slot = rel / parts;
    const int part = rel - slot * parts;
    const auto &L = a.layer[li];
    const int nb = a.n_embd / 32;

    // small loads first: the ids of the ownership scan and this slot's token
    // row (the first row served when the slot owns its expert)
    GtIds gi;
    if (wave == 0) gt_load_ids(L.ids, a.n_slots, gi);
    float4 vown[kGtOwnPre];
    gt_prefetch<QB>(L.x + (int64_t)(slot / a.n_used) * a.n_embd, nb, vown);
    const int e = wave_uniform(L.ids[slot]);
    const bool valid = e >= 0 && e < a.n_expert;

    if (slot == 0 && part == 0 && wave == 0) {
        int bad = 0;
        for (int s = lane; s < a.n_slots; s += kWave) {
            const int v = L.ids[s];
            bad |= (v < 0 || v >= a.n_expert);
        }
        bad = __any(bad);
        if (lane == 0) *(int32_t *)L.ws = bad;
    }
    const int col0 = 8 * W * a.ug_cols * part;
    const int ncol = min(8 * W * a.ug_cols, a.n_ff - col0);
    if (!valid) {
        for (int i = tid; i < ncol; i += T)
            L.h[(int64_t)slot * a.n_ff + col0 + i] = __builtin_nanf("");
        return;
    }

    extern __shared__ __align__(16) uint8_t mr_lds[];
    const int rstride = gt_row_stride(nb);
    uint8_t *xr = mr_lds;                                     // kGtMax token rows
    int *list = (int *)(mr_lds + kGtMax * rstride);           // [n_slots]
    __shared__ GtPick pk;
    if (wave == 0) gt_pick(L.ids, gi, a.n_slots, a.n_expert, slot, e, list, pk);
    __syncthreads();
    const int cnt = pk.count;
    if (cnt == 0) return;
    if (EMIT && a.counts && part == 0) {
        if (tid == 0) a.counts[e] = cnt;
        for (int i = tid; i < cnt; i += T) a.pairs[pk.less + i] = list[i];
    }

    // this wave's column groups: a prefix j < ncg of cg = cg0 + W*j
    const int cg0 = W * a.ug_cols * part + wave;
    const int ncg = cg0 < cgs ? min(a.ug_cols, (cgs - 1 - cg0) / W + 1) : 0;
    const int gb = kGB * nb;
    // stream g: column group j = g/2, gate (g even) or up (g odd); offsets
    // from the expert's first group
    auto goff_of = [&](int g) { return ((g & 1) * cgs + cg0 + W * (g >> 1)) * gb; };
    GatherStream<POL, EMIT, kGtSlices> gs;
    gs.init(L.w + (int64_t)e * 2 * cgs * gb, nb, 2 * cgs * gb, lane);
    const int r = (lane >> 1) & 7;

    for (int c0 = 0; c0 < cnt; c0 += kGtMax) {
        const int ct = min(kGtMax, cnt - c0);
        gs.issue_batch(ncg > 0 ? goff_of(0) : -1);
        gt_stage<QB>(xr, rstride, nb, ct, c0 == 0 && nb <= kGtOwnPre * QB, vown, [&](int m) {
            return L.x + (int64_t)(list[c0 + m] / a.n_used) * a.n_embd;
        });
        __syncthreads();
        if (ncg > 0) {
            gt_dispatch(ct, [&](auto ctc) {
                constexpr int CT = decltype(ctc)::value;
                float accg[CT];
                auto srow_of = [&](int g, int m) {
                    const int row = 8 * ((g & 1) * cgs + cg0 + W * (g >> 1)) + r;
                    return a.sums + ((int64_t)list[c0 + m] * 2 * a.n_ff + row) * nb;
                };
                gs.template run<CT>(2 * ncg, lane, xr, rstride, goff_of, srow_of,
                                    [&](int g, float (&acc)[CT]) {
                    if (!(g & 1)) {
#pragma unroll
                        for (int m = 0; m < CT; ++m) accg[m] = acc[m];
                    } else if ((lane & 0x31) == 0) {
                        const int col = 8 * (cg0 + W * (g >> 1)) + r;
#pragma unroll
                        for (int m = 0; m < CT; ++m) {
                            const float gv = accg[m];
                            L.h[(int64_t)list[c0 + m] * a.n_ff + col] = gv / (1.0f + expf(-gv)) * acc[m];
                        }
                    }
                });
            });
        }
        if (c0 + kGtMax < cnt) __syncthreads();   // the LDS rows are reused by the next pass
    }
}

// Down for several tokens: workgroup = (slot, band of W*a.dn_groups*8 output
// rows), wave w streaming a.dn_groups consecutive 8-row groups; the owner of the
// slot's expert quantizes the h rows of every slot routed to it (the rule of
// q8_0_quantize_rows) and writes their fp32 rows y[s][band] to the workspace.

struct MrGdArgs {
    struct Layer {
        const uint8_t *w;      // R8 down
        const int32_t *ids;
        const float *h;        // [n_slots][n_ff]
        float *yslot;          // [n_slots][n_embd]
    } layer[kMoeMaxLayers];
    int n_slots, n_embd, n_ff, n_expert;
    int dn_groups;             // 8-row groups per wave
    int bands;                 // ceil(n_embd / (8 * waves * dn_groups))
    int wg_per_layer;          // n_slots * bands
    int32_t *sums;             // validation: [slot][n_embd][n_ff/32] (layer 0 only)
    uint8_t *hq;               // validation: the q(h) rows used [slot][n_ff/32] (layer 0 only)
};

template <int POL, bool EMIT>
__global__ __launch_bounds__(kGtDnWaves * kWave, Q8_GT_DN_OCC) void moe_r8_down_gather_kernel(const MrGdArgs a)
{
    constexpr int W = kGtDnWaves, T = W * kWave, QB = T / 8;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int li = wave_uniform((int)blockIdx.x / a.wg_per_layer);
    const int rel = (int)blockIdx.x - li * a.wg_per_layer;
    const int slot = rel / a.bands;
    const int band = rel - slot * a.bands;
    const auto &L = a.layer[li];
    const int nb = a.n_ff / 32;

    // small loads first: the ids and this slot's own h row
    GtIds gi;
    if (wave == 0) gt_load_ids(L.ids, a.n_slots, gi);
    float4 vown[kGtOwnPre];
    gt_prefetch<QB>(L.h + (int64_t)slot * a.n_ff, nb, vown);
    const int e = wave_uniform(L.ids[slot]);
    if (e < 0 || e >= a.n_expert) return;          // the combine writes NaN for its token

    extern __shared__ __align__(16) uint8_t mr_lds[];
    const int rstride = gt_row_stride(nb);
    uint8_t *xr = mr_lds;                            // kGtMax q(h) rows
    int *list = (int *)(mr_lds + kGtMax * rstride);  // [n_slots]
    __shared__ GtPick pk;
    if (wave == 0) gt_pick(L.ids, gi, a.n_slots, a.n_expert, slot, e, list, pk);
    __syncthreads();
    const int cnt = pk.count;
    if (cnt == 0) return;

    const int groups = a.n_embd / 8;
    const int g0 = (band * W + wave) * a.dn_groups;   // first group of the wave
    const int ng = max(0, min(a.dn_groups, groups - g0));
    const int gb = kGB * nb;
    auto goff_of = [&](int g) { return g * gb; };
    GatherStream<POL, EMIT, kGtDnSlices> gs;
    gs.init(L.w + ((int64_t)e * groups + (ng > 0 ? g0 : 0)) * gb, nb, ng * gb, lane);
    const int r = (lane >> 1) & 7;

    for (int c0 = 0; c0 < cnt; c0 += kGtMax) {
        const int ct = min(kGtMax, cnt - c0);
        gs.issue_batch(ng > 0 ? 0 : -1);
        gt_stage<QB>(xr, rstride, nb, ct, c0 == 0 && nb <= kGtOwnPre * QB, vown,
                 [&](int m) { return L.h + (int64_t)list[c0 + m] * a.n_ff; });
        __syncthreads();
        if (EMIT && a.hq && band == 0) {
            // the q(h) bytes this pass used, as Q8_0 blocks
            for (int i = tid; i < ct * nb * 17; i += T) {
                const int m = i / (nb * 17);
                const int k = i - m * nb * 17;
                const int b = k / 17, w = k - b * 17;
                const uint8_t *xc = xr + m * rstride;
                const uint16_t v = w == 0 ? ((const uint16_t *)(xc + 32 * nb))[b]
                                          : ((const uint16_t *)xc)[16 * b + w - 1];
                ((uint16_t *)(a.hq + (int64_t)list[c0 + m] * nb * kBlockBytes))[k] = v;
            }
        }
        if (ng > 0) {
            gt_dispatch(ct, [&](auto ctc) {
                constexpr int CT = decltype(ctc)::value;
                auto srow_of = [&](int g, int m) {
                    return a.sums + ((int64_t)list[c0 + m] * a.n_embd + 8 * (g0 + g) + r) * nb;
                };
                gs.template run<CT>(ng, lane, xr, rstride, goff_of, srow_of,
                                    [&](int g, float (&acc)[CT]) {
                    if ((lane & 0x31) == 0) {
#pragma unroll
                        for (int m = 0; m < CT; ++m)
                            L.yslot[(int64_t)list[c0 + m] * a.n_embd + 8 * (g0 + g) + r] = acc[m];
                    }
                });
            });
        }
        if (c0 + kGtMax < cnt) __syncthreads();   // the LDS rows are reused by the next pass
    }
}

}  // namespace

namespace {

bool r8_decode_ok(int64_t n_tok, int64_t n_embd, int64_t n_ff, int64_t n_expert, int64_t n_used)
{
    return n_ff % 32 == 0 && n_embd % 32 == 0 && n_ff / 32 <= 64 && n_embd / 32 <= kR8MaxNb &&
           n_used >= 1 && n_used <= kMoeMaxUsed && n_tok * n_used <= kMoeMaxSlots &&
           n_expert <= kMoeMaxExperts;
}

// Decode workspace: the error word, then at one token the q(h) rows
// [slot][n_ff/32] blocks at +256, with several tokens the fp32 slot rows
// [slot][n_embd] of the combine at +256.
struct R8DecodeWs {
    size_t yslot, total;
};

// LDS of the fused kernel: the token row, the up and h values, the q(h)
// block, the reducer's slot rows
size_t fused_lds(int64_t n_embd, int64_t n_used)
{
    return (size_t)(34 * (n_embd / 32) + 15) / 16 * 16 + 64 * 4 + 12 * 4 + (size_t)n_used * 32 * 4;
}

R8DecodeWs r8_decode_ws(int64_t n_tok, int64_t n_embd, int64_t n_ff, int64_t n_used)
{
    const size_t slots = (size_t)(n_tok * n_used);
    R8DecodeWs w;
    w.yslot = 256;
    w.total = 256 + (n_tok > 1 ? slots * (size_t)n_embd * 4
                               : (slots * (size_t)(n_ff / 32) * kBlockBytes + 255) / 256 * 256);
    return w;
}

}  // namespace

// more than kMoeDecodeMaxTok tokens go to the grouped matrix-core path where
// its shape conditions hold (as for native rows)
bool moe_r8_prefill_path(int64_t n_tok, int64_t n_embd, int64_t n_ff, int64_t n_expert,
                         int64_t n_used)
{
    return n_tok > kMoeDecodeMaxTok && moe_prefill_ok(n_tok, n_embd, n_ff, n_expert, n_used);
}

bool moe_r8_ok(int64_t n_tok, int64_t n_embd, int64_t n_ff, int64_t n_expert, int64_t n_used)
{
    return moe_r8_prefill_path(n_tok, n_embd, n_ff, n_expert, n_used) ||
           r8_decode_ok(n_tok, n_embd, n_ff, n_expert, n_used);
}

size_t moe_r8_ws_bytes(int64_t n_tok, int64_t n_embd, int64_t n_ff, int64_t n_expert,
                       int64_t n_used)
{
    if (moe_r8_prefill_path(n_tok, n_embd, n_ff, n_expert, n_used))
        return moe_prefill_ws_bytes(n_tok, n_embd, n_ff, n_expert, n_used);
    return r8_decode_ws(n_tok, n_embd, n_ff, n_used).total;
}

// The no-alloc entry point's workspace: one array per device for the life of
// the process.  In host code `moe_r8_scratch_array` names a host-side stand-in,
// not device memory: only the address hipGetSymbolAddress returns (one per
// device, the device current) is passed to kernels.
static __device__ __align__(256) uint8_t moe_r8_scratch_array[kMoeR8ScratchBytes];

constexpr int kScratchMaxDevices = 64;
static uint8_t *g_scratch[kScratchMaxDevices];
static std::mutex g_scratch_mu;

int moe_r8_scratch(uint8_t **base)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchMaxDevices) return -6;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(moe_r8_scratch_array)) != hipSuccess || !p) return -6;
        g_scratch[dev] = (uint8_t *)p;
    }
    *base = g_scratch[dev];
    return 0;
}

int moe_r8_ffn_check(int64_t n_tok, int64_t n_embd, int64_t n_ff, int64_t n_expert,
                     int64_t n_used)
{
    if (n_tok == 0) return 0;
    if (moe_r8_prefill_path(n_tok, n_embd, n_ff, n_expert, n_used))
        return moe_prefill_check(n_tok, n_embd, n_ff, n_expert, n_used);
    const int64_t n_slots = n_tok * n_used;
    const size_t ug_lds = n_tok > 1 ? gt_lds(n_slots, n_embd / 32)
                                    : (size_t)(34 * (n_embd / 32) + 15) / 16 * 16 + 64 * 4;
    const size_t dn_lds = n_tok > 1 ? gt_lds(n_slots, n_ff / 32)
                                    : (size_t)16 * ((34 * (n_ff / 32) + 15) / 16 * 16) +
                                          16 * 8 * kDnG * 4;
    if (ug_lds > (size_t)max_lds_bytes() || dn_lds > (size_t)max_lds_bytes()) return -4;
    const int64_t ug_wgs = kMoeMaxLayers * n_slots * (n_ff / 32);
    const int64_t dn_wgs = kMoeMaxLayers * (n_tok > 1 ? n_slots * ((n_embd / 8 + kGtDnWaves - 1) / kGtDnWaves)
                                                      : n_tok * (n_embd / 8));
    return (ug_wgs > 0x7fffffffLL || dn_wgs > 0x7fffffffLL) ? -4 : 0;
}

namespace {

#ifndef Q8_GT_NT
#define Q8_GT_NT 1
#endif
// cache policy of the expert-major kernels' weight loads: every active
// expert's rows are read once per call
constexpr int kGtPol = Q8_GT_NT ? kCacheNT : 0;

int launch_r8_gather(const MoeR8Layer *l, int n_layers, int64_t n_tok, int64_t n_embd,
                     int64_t n_ff, int64_t n_expert, int64_t n_used, hipStream_t stream,
                     const MoeEmit *emit_ug, const MoeEmit *emit_dn)
{
    const bool route = emit_ug && emit_ug->counts;
    int32_t *ug_sums = emit_ug ? emit_ug->sums : nullptr;
    int32_t *dn_sums = emit_dn ? emit_dn->sums : nullptr;
    const int64_t n_slots = n_tok * n_used;
    const size_t ug_lds = gt_lds(n_slots, n_embd / 32);
    const size_t dn_lds = gt_lds(n_slots, n_ff / 32);
    if (ug_lds > (size_t)max_lds_bytes() || dn_lds > (size_t)max_lds_bytes()) return -4;
    const R8DecodeWs W = r8_decode_ws(n_tok, n_embd, n_ff, n_used);
    // Work per wave: as much as keeps about Q8_GT_ROUNDS rounds of the
    // resident waves busy (8 per CU here) -- few layers per call (a model's
    // layer after layer) want short streams spread over the whole chip, many
    // layers long streams that pay the ownership scan and the row staging
    // once.  The active experts are bounded by min(n_expert, slots) per layer.
    // One layer of 16 tokens per call, 30 calls: 8 rounds 2.75 ms, 4 rounds
    // 2.78 ms, 2 rounds 2.82 ms, 1 round 3.18 ms, 16 rounds 2.94 ms (30 layers
    // per call reach the longest streams at any of these).
    const int64_t act = (int64_t)n_layers * (n_expert < n_slots ? n_expert : n_slots);
    const int64_t target = (int64_t)Q8_GT_ROUNDS * 256 * 8;
    int ug_cols = 4, dn_groups = 8;
    while (ug_cols > 1 && act * (n_ff / 8) / ug_cols < target) ug_cols /= 2;
    while (dn_groups > 1 && act * (n_embd / 8) / dn_groups < target) dn_groups /= 2;
    if (route)
        if (int rc = launch_fill_i32(emit_ug->counts, n_expert, 0, stream)) return rc;
    for (int l0 = 0; l0 < n_layers; l0 += kMoeMaxLayers) {
        const int nl = n_layers - l0 < kMoeMaxLayers ? n_layers - l0 : kMoeMaxLayers;
        MrUgArgs ug;
        memset(&ug, 0, sizeof(ug));
        MrGdArgs gd;
        memset(&gd, 0, sizeof(gd));
        MoeCombineLayer cb[kMoeMaxLayers];
        for (int i = 0; i < nl; ++i) {
            const MoeR8Layer &s = l[l0 + i];
            float *yslot = (float *)((uint8_t *)s.ws + W.yslot);
            ug.layer[i] = {(const uint8_t *)s.w_up_gate, s.x, s.ids, s.h, (uint8_t *)s.ws};
            gd.layer[i] = {(const uint8_t *)s.w_down, s.ids, s.h, yslot};
            cb[i] = {yslot, s.ids, s.cw, s.out};
        }
        ug.n_used = (int)n_used;
        ug.n_slots = (int)n_slots;
        ug.n_embd = (int)n_embd;
        ug.n_ff = (int)n_ff;
        ug.n_expert = (int)n_expert;
        ug.ug_cols = ug_cols;
        ug.wg_per_layer =
            (int)(n_slots * ((n_ff / 8 + kGtUgWaves * ug_cols - 1) / (kGtUgWaves * ug_cols)));
        ug.sums = ug_sums;
        ug.counts = route ? emit_ug->counts : nullptr;
        ug.pairs = route ? emit_ug->pairs : nullptr;
        const dim3 ug_grid((unsigned)(nl * ug.wg_per_layer));
        if (ug_sums || route)
            hipLaunchKernelGGL((moe_r8_up_gate_gather_kernel<kGtPol, true>), ug_grid,
                               dim3(kGtUgWaves * kWave), ug_lds, stream, ug);
        else
            hipLaunchKernelGGL((moe_r8_up_gate_gather_kernel<kGtPol, false>), ug_grid,
                               dim3(kGtUgWaves * kWave), ug_lds, stream, ug);
        if (hipGetLastError() != hipSuccess) return -6;
        gd.n_slots = (int)n_slots;
        gd.n_embd = (int)n_embd;
        gd.n_ff = (int)n_ff;
        gd.n_expert = (int)n_expert;
        gd.dn_groups = dn_groups;
        gd.bands = (int)((n_embd / 8 + kGtDnWaves * dn_groups - 1) / (kGtDnWaves * dn_groups));
        gd.wg_per_layer = (int)(n_slots * gd.bands);
        gd.sums = dn_sums;
        gd.hq = emit_dn ? (uint8_t *)emit_dn->hq : nullptr;
        const dim3 dn_grid((unsigned)(nl * gd.wg_per_layer));
        if (dn_sums || gd.hq)
            hipLaunchKernelGGL((moe_r8_down_gather_kernel<kGtPol, true>), dn_grid,
                               dim3(kGtDnWaves * kWave), dn_lds, stream, gd);
        else
            hipLaunchKernelGGL((moe_r8_down_gather_kernel<kGtPol, false>), dn_grid,
                               dim3(kGtDnWaves * kWave), dn_lds, stream, gd);
        if (hipGetLastError() != hipSuccess) return -6;
        if (int rc = launch_moe_combine_layers(cb, nl, n_tok, n_embd, n_used, n_expert, stream))
            return rc;
    }
    return route ? launch_route_offsets(emit_ug->counts, emit_ug->offsets, n_expert, stream) : 0;
}

}  // namespace

size_t moe_r8_fused_ws_bytes(int64_t n_embd, int64_t n_ff, int64_t n_used)
{
    return 256 + (size_t)n_used * (size_t)(n_ff / 32) * (size_t)n_embd * 4;
}

int moe_r8_fused_check(int64_t n_embd, int64_t n_ff, int64_t n_expert, int64_t n_used)
{
    if (!r8_decode_ok(1, n_embd, n_ff, n_expert, n_used) || n_embd % 256 != 0) return -4;
    const size_t lds = fused_lds(n_embd, n_used);
    if (lds > (size_t)max_lds_bytes()) return -4;
    // terms offsets are 32-bit element counts; the down rows' buffer range too
    if ((int64_t)n_used * (n_ff / 32) * n_embd > 0x7fffffffLL ||
        (int64_t)n_embd * (n_ff / 32) * kBlockBytes > 0x7f000000LL)
        return -4;
    return 0;
}

int launch_moe_r8_fused(const MoeR8Layer &l, int64_t n_embd, int64_t n_ff, int64_t n_expert,
                        int64_t n_used, hipStream_t stream)
{
    if (int rc = moe_r8_fused_check(n_embd, n_ff, n_expert, n_used)) return rc;
    MrFzArgs a;
    a.w_ug = (const uint8_t *)l.w_up_gate;
    a.w_dn = (const uint8_t *)l.w_down;
    a.x = l.x;
    a.ids = l.ids;
    a.cw = l.cw;
    a.h = l.h;
    a.out = l.out;
    a.ws = (uint8_t *)l.ws;
    a.n_used = (int)n_used;
    a.n_embd = (int)n_embd;
    a.n_ff = (int)n_ff;
    a.n_expert = (int)n_expert;
    const int total = (int)(n_used * (n_ff / 32));
    const int bands = (int)(n_embd / 32);
    a.reducers = total < bands ? total : bands;
    hipLaunchKernelGGL((moe_r8_fused_kernel<kCacheNT>), dim3((unsigned)total), dim3(kUgThreads),
                       fused_lds(n_embd, n_used), stream, a);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

int launch_moe_r8_ffn(const MoeR8Layer *l, int n_layers, int64_t n_tok, int64_t n_embd,
                      int64_t n_ff, int64_t n_expert, int64_t n_used, hipStream_t stream,
                      const MoeEmit *emit_ug, const MoeEmit *emit_dn)
{
    if (n_tok == 0) return 0;
    if (moe_r8_prefill_path(n_tok, n_embd, n_ff, n_expert, n_used)) {
        for (int i = 0; i < n_layers; ++i) {
            const MoeR8Layer &s = l[i];
            if (int rc = launch_moe_r8_prefill((const uint8_t *)s.w_up_gate, (const uint8_t *)s.w_down,
                                               s.x, s.ids, s.cw, s.h, s.out, s.ws, n_tok, n_embd,
                                               n_ff, n_expert, n_used, stream, emit_ug, emit_dn))
                return rc;
        }
        return 0;
    }
    if (n_tok > 1)
        return launch_r8_gather(l, n_layers, n_tok, n_embd, n_ff, n_expert, n_used, stream, emit_ug,
                                emit_dn);
    // one token: every slot is served on its own, no grouping to report
    if (emit_ug && emit_ug->counts) return -4;
    int32_t *ug_sums = emit_ug ? emit_ug->sums : nullptr;
    int32_t *dn_sums = emit_dn ? emit_dn->sums : nullptr;
    for (int l0 = 0; l0 < n_layers; l0 += kMoeMaxLayers) {
        const int nl = n_layers - l0 < kMoeMaxLayers ? n_layers - l0 : kMoeMaxLayers;
        MrUgArgs ug;
        memset(&ug, 0, sizeof(ug));
        MrDnArgs dn;
        memset(&dn, 0, sizeof(dn));
        for (int i = 0; i < nl; ++i) {
            const MoeR8Layer &s = l[l0 + i];
            ug.layer[i] = {(const uint8_t *)s.w_up_gate, s.x, s.ids, s.h, (uint8_t *)s.ws};
            dn.layer[i] = {(const uint8_t *)s.w_down, s.ids, s.cw, s.out, (const uint8_t *)s.ws};
        }
        ug.n_used = (int)n_used;
        ug.n_slots = (int)(n_tok * n_used);
        ug.n_embd = (int)n_embd;
        ug.n_ff = (int)n_ff;
        ug.n_expert = (int)n_expert;
        ug.wg_per_layer = (int)(n_tok * n_used * (n_ff / 32));
        ug.sums = ug_sums;
        const int64_t nb = n_embd / 32;
        const size_t ug_lds = (size_t)(34 * nb + 15) / 16 * 16 + 64 * 4;
        if (ug_lds > (size_t)max_lds_bytes()) return -4;   // also checked by moe_r8_ffn_check
        // cache policy of the weight loads: at one token every slot names a
        // different expert and nothing is read twice (non-temporal loads);
        // with several tokens slots repeat experts, and the default policy
        // lets the repeats find the rows in L2 or the Infinity Cache
        // (measured, 30 layers: 1 token 182.8 against 205.6 us, 16 tokens
        // 2449 against 2694 us)
        const bool reuse = n_tok > 1;
        const dim3 ug_grid((unsigned)(nl * ug.wg_per_layer));
        if (ug_sums)
            hipLaunchKernelGGL((moe_r8_up_gate_kernel<0, true>), ug_grid, dim3(kUgThreads), ug_lds,
                               stream, ug);
        else if (reuse)
            hipLaunchKernelGGL((moe_r8_up_gate_kernel<0, false>), ug_grid, dim3(kUgThreads), ug_lds,
                               stream, ug);
        else if (nl == 1)
            // one layer per launch (layers run one after another): a group's
            // 64 blocks all in flight at once, 16 slices per wave (30 layers
            // one per call: 434 against 443 us; all 30 in one call keep 8:
            // 185 against 207 us)
            hipLaunchKernelGGL((moe_r8_up_gate_kernel<kCacheNT, false, Q8_MR_UG_ONE_LAYER_SLICES>), ug_grid,
                               dim3(kUgThreads), ug_lds, stream, ug);
        else
            hipLaunchKernelGGL((moe_r8_up_gate_kernel<kCacheNT, false>), ug_grid, dim3(kUgThreads),
                               ug_lds, stream, ug);
        if (hipGetLastError() != hipSuccess) return -6;
        if (emit_dn && emit_dn->hq &&
            hipMemcpyAsync(emit_dn->hq, (const uint8_t *)l[0].ws + 256,
                           (size_t)(n_tok * n_used) * (n_ff / 32) * kBlockBytes,
                           hipMemcpyDeviceToDevice, stream) != hipSuccess)
            return -6;
        dn.n_used = (int)n_used;
        dn.n_embd = (int)n_embd;
        dn.n_ff = (int)n_ff;
        dn.n_expert = (int)n_expert;
        // one group per workgroup where a launch of 4-group workgroups would be
        // small (one token of one layer: 64 workgroups for 256 CUs; 13.4 MB
        // then stream with 4x the workgroups, each wave's group in flight at once)
        const int dn_g = (int64_t)nl * n_tok * (n_embd / (8 * kDnG)) < 512 ? 1 : kDnG;
        dn.wg_per_layer = (int)(n_tok * (n_embd / (8 * dn_g)));
        dn.sums = dn_sums;
        const size_t dn_lds = (size_t)16 * ((34 * (n_ff / 32) + 15) / 16 * 16) + 16 * 8 * kDnG * 4;
        const dim3 dn_grid((unsigned)(nl * dn.wg_per_layer)), dn_block((unsigned)(64 * n_used));
        if (dn_g == 1) {
            if (dn_sums)
                hipLaunchKernelGGL((moe_r8_down_kernel<0, true, 1>), dn_grid, dn_block, dn_lds, stream,
                                   dn);
            else if (reuse)
                hipLaunchKernelGGL((moe_r8_down_kernel<0, false, 1>), dn_grid, dn_block, dn_lds,
                                   stream, dn);
            else
                hipLaunchKernelGGL((moe_r8_down_kernel<kCacheNT, false, 1>), dn_grid, dn_block, dn_lds,
                                   stream, dn);
        } else if (dn_sums) {
            hipLaunchKernelGGL((moe_r8_down_kernel<0, true, kDnG>), dn_grid, dn_block, dn_lds, stream,
                               dn);
        } else if (reuse) {
            hipLaunchKernelGGL((moe_r8_down_kernel<0, false, kDnG>), dn_grid, dn_block, dn_lds, stream,
                               dn);
        } else {
            hipLaunchKernelGGL((moe_r8_down_kernel<kCacheNT, false, kDnG>), dn_grid, dn_block, dn_lds,
                               stream, dn);
        }
        if (hipGetLastError() != hipSuccess) return -6;
    }
    return 0;
}

}  // namespace q8
