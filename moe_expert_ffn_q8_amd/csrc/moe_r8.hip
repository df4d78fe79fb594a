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
// Two launches per call (several layers of one shape per launch):
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
// Each slot streams its expert's rows itself: at one token the 8 slots name
// distinct experts; with several tokens repeated experts are read once per
// slot (the expert-major kernels of moe.hip read them once per call).
//
// Ids outside [0, n_expert): the up_gate workgroup of slot 0 / columns 0 sets
// the error word of the workspace (0 or 1, every call); such a slot's h row is
// NaN, and every output row of its token is NaN.
#include <string.h>

#include "q8_device.h"
#include "q8_internal.h"
#include "q8_moe.h"

namespace q8 {

namespace {

constexpr int kGB = 8 * kBlockBytes;      // bytes per block column of an 8-row group
constexpr int kMrSlices = 8;              // 1 KB slices of a group in flight per wave

// One 8-row group of nb blocks against an activation row in LDS (codes
// realigned to 32 bytes per block, binary16 scale bits); slice i, lane l:
// row (l>>1)&7, block 4i + (l>>4), half l&1.  Returns the lane's partial sum
// (blocks of its residue, ascending); the caller adds lanes l, l^16, l^32.
template <int POL>
struct GroupStream {
    __amdgpu_buffer_rsrc_t rs;
    int code0, scale0, nb;
    u32x4 c[kMrSlices];
    uint32_t sb[kMrSlices];

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
        for (int u = 0; u < kMrSlices; ++u)
            c[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, code0 + 1024 * (i0 + u), 0, POL);
#pragma unroll
        for (int u = 0; u < kMrSlices; ++u)
            sb[u] = __builtin_amdgcn_raw_buffer_load_b16(rs, scale0 + 64 * (i0 + u), 0, POL);
    }
    // every slice is computed (a branch would make the compiler wait for each
    // load in turn): slices past the group read zero codes, scales masked
    __device__ __forceinline__ void compute(int i0, int lane, const uint8_t *xc,
                                            const uint16_t *xd16, float &acc)
    {
        const int half = lane & 1, bs = lane >> 4;
#pragma unroll
        for (int u = 0; u < kMrSlices; ++u) {
            const int b = 4 * (i0 + u) + bs;
            const bool live = b < nb;
            const int bb = live ? b : nb - 1;
            const u32x4 xv = *(const u32x4 *)(xc + 32 * bb + 16 * half);
            int s = sdot4(c[u].x, xv.x, 0);
            s = sdot4(c[u].y, xv.y, s);
            s = sdot4(c[u].z, xv.z, s);
            s = sdot4(c[u].w, xv.w, s);
            s += __builtin_amdgcn_mov_dpp(s, 0xB1, 0xF, 0xF, false);   // the other half
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
            i0 += kMrSlices;
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

template <int POL>
struct MultiStream {
    __amdgpu_buffer_rsrc_t rs;
    int nb, S, total, gb;
    u32x4 c[kMrSlices];
    uint32_t sb[kMrSlices];

    __device__ __forceinline__ void init(const uint8_t *base, int nb_)
    {
        nb = nb_;
        gb = kGB * nb;
        S = (nb + 3) >> 2;
        total = kDnG * S;
        rs = __builtin_amdgcn_make_buffer_rsrc((void *)wave_uniform(base), 0,
                                               wave_uniform(kDnG * gb), kBufferWord3);
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
                                            const uint16_t *xd16, float (&acc)[kDnG])
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
            const float dw = live ? half_bits_to_float(sb[u]) : 0.0f;
            const float p = dw * half_bits_to_float(xd16[bb]);
#pragma unroll
            for (int g = 0; g < kDnG; ++g)
                if (q == g) acc[g] = fmaf(p, (float)s, acc[g]);
        }
    }
    __device__ __forceinline__ void run(int lane, const uint8_t *xc, const uint16_t *xd16,
                                        float (&acc)[kDnG])
    {
#pragma unroll
        for (int g = 0; g < kDnG; ++g) acc[g] = 0.0f;
        for (int j0 = 0;;) {
            compute(j0, lane, xc, xd16, acc);
            j0 += kMrSlices;
            if (j0 >= total) break;
            issue(j0, lane);
        }
#pragma unroll
        for (int g = 0; g < kDnG; ++g) {
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
};

template <int POL>
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
    GroupStream<POL> gs;
    gs.init(gbase, nb, lane, true);
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
};

template <int POL>
__global__ __launch_bounds__(1024) void moe_r8_down_kernel(const MrDnArgs a)
{
    const int tid = threadIdx.x;
    const int wave = tid >> 6;                 // = the slot u of the token
    const int lane = tid & 63;
    const int li = wave_uniform((int)blockIdx.x / a.wg_per_layer);
    const int rel = (int)blockIdx.x - li * a.wg_per_layer;
    const int quads = a.n_embd / (8 * kDnG);      // 32-row bands of the output
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
    float *orow = L.out + (int64_t)t * a.n_embd + 8 * kDnG * g;
    if (bad) {
        if (tid < 8 * kDnG) orow[tid] = __builtin_nanf("");
        return;
    }
    const int e = wave_uniform(L.ids[t * U + wave]);
    const uint8_t *gbase = L.w + ((int64_t)e * (a.n_embd / 8) + kDnG * g) * kGB * nb;

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
    MultiStream<POL> ms;
    ms.init(gbase, nb);
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

    float acc[kDnG];
    ms.run(lane, xc, xd16, acc);
    if ((lane & 0x31) == 0) {
#pragma unroll
        for (int q = 0; q < kDnG; ++q) ybuf[8 * kDnG * wave + 8 * q + ((lane >> 1) & 7)] = acc[q];
    }
    __syncthreads();
    if (tid < 8 * kDnG) {
        float o = 0.0f;
        for (int u = 0; u < U; ++u) o = fmaf(L.cw[t * U + u], ybuf[8 * kDnG * u + tid], o);
        orow[tid] = o;
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
    const size_t hq = (size_t)(n_tok * n_used) * (size_t)(n_ff / 32) * kBlockBytes;
    return 256 + (hq + 255) / 256 * 256;
}

int launch_moe_r8_ffn(const MoeR8Layer *l, int n_layers, int64_t n_tok, int64_t n_embd,
                      int64_t n_ff, int64_t n_expert, int64_t n_used, hipStream_t stream)
{
    if (n_tok == 0) return 0;
    if (moe_r8_prefill_path(n_tok, n_embd, n_ff, n_expert, n_used)) {
        for (int i = 0; i < n_layers; ++i) {
            const MoeR8Layer &s = l[i];
            if (int rc = launch_moe_r8_prefill((const uint8_t *)s.w_up_gate, (const uint8_t *)s.w_down,
                                               s.x, s.ids, s.cw, s.h, s.out, s.ws, n_tok, n_embd,
                                               n_ff, n_expert, n_used, stream))
                return rc;
        }
        return 0;
    }
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
        const int64_t nb = n_embd / 32;
        const size_t ug_lds = (size_t)(34 * nb + 15) / 16 * 16 + 64 * 4;
        if (ug_lds > (size_t)max_lds_bytes()) return -4;
        // cache policy of the weight loads: at one token every slot names a
        // different expert and nothing is read twice (non-temporal loads);
        // with several tokens slots repeat experts, and the default policy
        // lets the repeats find the rows in L2 or the Infinity Cache
        // (measured, 30 layers: 1 token 182.8 against 205.6 us, 16 tokens
        // 2449 against 2694 us)
        const bool reuse = n_tok > 1;
        if (reuse)
            hipLaunchKernelGGL(moe_r8_up_gate_kernel<0>, dim3((unsigned)(nl * ug.wg_per_layer)),
                               dim3(kUgThreads), ug_lds, stream, ug);
        else
            hipLaunchKernelGGL(moe_r8_up_gate_kernel<kCacheNT>,
                               dim3((unsigned)(nl * ug.wg_per_layer)), dim3(kUgThreads), ug_lds,
                               stream, ug);
        if (hipGetLastError() != hipSuccess) return -6;
        dn.n_used = (int)n_used;
        dn.n_embd = (int)n_embd;
        dn.n_ff = (int)n_ff;
        dn.n_expert = (int)n_expert;
        dn.wg_per_layer = (int)(n_tok * (n_embd / (8 * kDnG)));
        const size_t dn_lds = (size_t)16 * ((34 * (n_ff / 32) + 15) / 16 * 16) + 16 * 8 * kDnG * 4;
        if (reuse)
            hipLaunchKernelGGL(moe_r8_down_kernel<0>, dim3((unsigned)(nl * dn.wg_per_layer)),
                               dim3((unsigned)(64 * n_used)), dn_lds, stream, dn);
        else
            hipLaunchKernelGGL(moe_r8_down_kernel<kCacheNT>, dim3((unsigned)(nl * dn.wg_per_layer)),
                               dim3((unsigned)(64 * n_used)), dn_lds, stream, dn);
        if (hipGetLastError() != hipSuccess) return -6;
    }
    return 0;
}

}  // namespace q8
