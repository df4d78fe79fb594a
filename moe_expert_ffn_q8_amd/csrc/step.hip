// step.hip -- a batch-1 (or 2) decode step in one launch: the activation
// quantization and every Q8_0 product of the step, each activation row
// quantized once.
//
// The activations of a Q8_0 product are quantized by the same rule as the
// weights before the integer block dot (quantize_row_q8_0 feeding
// ggml_vec_dot_q8_0_q8_0 on the Gemma-4-on-Xeon page, "GPUなしで13年前のXeon上
// でGemma 4 26Bを毎秒5トークンで実行する", sections on the three-part fix and on
// narrowing down the cause); the narray-llm README's Llama 2 110M int8 table
// measures exactly that per-matvec re-quantization, and its kernels-per-token
// table counts the launches.  Here the quantization and the products share one
// launch.
//
// Grid (single-wave workgroups):
//  * workgroups [0, n_quant) quantize: part p of batch entry b of job j takes
//    8 blocks of that entry's m fp32 rows, writes their Q8_0 bytes into the
//    workspace image (the bytes of q8_0_quantize_rows), and counts itself in
//    the entry's part counter.  The last part of an entry resets that counter
//    and sets the flag of every tile of the entry.
//  * workgroups [n_quant, n_quant + tiles) are the tiles of the decode engine
//    (one tile of R whole weight rows each, numbered as in the flat engine):
//    a tile takes its flag (atomic exchange with 0), issues its weight loads,
//    retakes the flag until it was set (normally it already is), reads its
//    quad of the quantized rows and computes exactly as the decode engine
//    does.
// Every flag and counter is zero again when the launch ends, so the next call
// on the same workspace starts from the same state.  Tiles have flags of their
// own (not one counter per entry) because same-address atomics are served one
// at a time: with one ready counter per entry that every tile decremented, the
// Llama-110M-shaped step took 176 us instead of 31 us.
//
// Visibility across the eight XCDs (each has its own L2): the image is written
// and read only with agent-scope accesses (stores and loads with the scope bit
// that makes each access coherent for the whole device), the counters only
// with agent-scope atomics.  A quantizer publishes after its image stores have
// completed (wait on the store counter), and a tile issues its image loads
// only after its poll has returned a positive count, so the loads are
// performed after the stores.  No cache-wide write-back or invalidate is
// needed: measured, one agent-scope acquire fence per tile (an L2 invalidate)
// cost ~110 us on the Llama-110M-shaped step, and a release fence per
// quantizer (an L2 write-back) tens of us.
//
// Progress: the quantizers have the lowest workgroup ids and wait on nothing;
// tiles wait only on quantizers.  The wait is bounded anyway: after kMaxPolls
// polls a tile sets the workspace's error word and continues (that call's
// outputs are then invalid; the counters still return to zero).
#include <string.h>

#include "q8_device.h"
#include "q8_internal.h"

namespace q8 {

namespace {

// Blocks per quantizer workgroup: one pass of 8.  Measured on the
// Llama-110M-shaped step: 8 -> 23.0 us, 16 -> 23.5, 32 -> 23.9, 64 -> 23.9
// (longer parts make the first tiles wait longer).
constexpr int kPartBlocks = 8;
constexpr int kPasses = kPartBlocks / 8;   // passes of 8 blocks
constexpr int kMaxPolls = 1 << 16;     // bound of a tile's wait (normally 0 or a few polls)
// The part counters of different entries sit in separate 256-byte lines.
constexpr int kCtrStride = 64;         // int32 per entry
#ifndef Q8_STEP_FLAG_STRIDE
#define Q8_STEP_FLAG_STRIDE 1
#endif
constexpr int kFlagStride = Q8_STEP_FLAG_STRIDE;   // int32 per tile flag
#ifndef Q8_STEP_SLEEP
#define Q8_STEP_SLEEP 8
#endif

struct StepJob {
    const uint8_t *w;
    const uint8_t *x;        // fp32 rows
    float *y;
    int64_t w_bstride;       // bytes
    int64_t x_bstride;       // bytes
    int64_t y_bstride;       // floats
    int64_t img0;            // byte offset of the job's quantized rows in the image area
    int32_t x_rstride;       // bytes
    int32_t y_rstride;       // floats
    int32_t n, nb, m, batch;
    int32_t R;               // rows per tile
    int32_t tpb;             // tiles per batch entry
    int32_t tile0;           // first tile of this job
    int32_t q0;              // first quantizer workgroup of this job
    int32_t ppe;             // quantizer parts per batch entry
    int32_t e0;              // counter index of the job's first batch entry
};

struct StepArgs {
    StepJob job[kStreamMaxJobs];
    int32_t n_jobs;
    int32_t n_quant;
    int32_t *err;            // error word
    int32_t *parts;          // entry e: part counter at parts[e * kCtrStride]
    int32_t *flag;           // tile t: 1 once its entry's rows are in the image
    uint8_t *img;            // quantized activation rows
};

static_assert(sizeof(StepArgs) <= 4000, "kernel arguments must stay below 4 KB");

// Agent-scope accesses (coherent across the XCDs' L2 caches by themselves).
__device__ __forceinline__ int ld_agent(const int32_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Read a tile flag and clear it in one agent-scope access (one lane only).
__device__ __forceinline__ int take_flag(int32_t *p)
{
    return __hip_atomic_exchange(p, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void st_agent(uint16_t *p, uint16_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Cache-policy bits of a buffer load: sc1 = agent scope (the load is coherent
// across the XCDs, as the compiler's agent-scope atomic loads are).
constexpr int kAgentScope = 16;

// Issue the agent-scope loads of one quantized row (nb blocks, nb*17/8 16-byte
// chunks, 16-byte aligned) into registers: chunk i of lane l is load u with
// i = 64u + l; chunks past the row read as zero without memory traffic.
__device__ __forceinline__ void row_issue(const uint8_t *row, int nb, int lane,
                                          u32x4 (&v)[kTileLoads])
{
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void *)wave_uniform(row), 0, wave_uniform(nb) * kBlockBytes, kBufferWord3);
#pragma unroll
    for (int u = 0; u < kTileLoads; ++u)
        v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, 16 * (u * kWave + lane), 0, kAgentScope);
}

// Stage a quantized row through LDS and take this lane's quad c of it as a
// masked image + scales (the layout of load_x_quad).
__device__ __forceinline__ void row_to_quad(uint8_t *stage, const u32x4 (&v)[kTileLoads], int nb,
                                            int lane, int c, uint32_t (&q)[kQuadDwords], float4 &d)
{
    const int chunks = nb * 17 / 8;
#pragma unroll
    for (int u = 0; u < kTileLoads; ++u) {
        const int i = u * kWave + lane;
        if (i < chunks) ((u32x4 *)stage)[i] = v[u];
    }
    wave_lds_sync();
    lds_quad(stage + kQuadBytes * c, q);
    wave_lds_sync();
    d.x = half_bits_to_float(q[0]);
    d.y = half_bits_to_float(q[8] >> 16);
    d.z = half_bits_to_float(q[17]);
    d.w = half_bits_to_float(q[25] >> 16);
    q[0] &= 0xffff0000u;
    q[8] &= 0x0000ffffu;
    q[17] &= 0xffff0000u;
    q[25] &= 0x0000ffffu;
}

// One quantizer part: blocks [8p, 8p + 8) of the entry's m x nb blocks
// (row-major), 8 lanes per block, 8 blocks per pass.  nb % 8 == 0, so the 8
// blocks of a pass lie in one row and the entry's block count is a multiple of
// 8 (a pass is all in or all out).  The loads of all passes are issued before
// any of them is used.
__device__ void quantize_part(const StepArgs &a, int q)
{
    const int lane = threadIdx.x;
    int j = 0;
    for (int i = 1; i < a.n_jobs; ++i)
        if (a.job[i].q0 <= q) j = i;
    const StepJob &J = a.job[j];
    const int qi = q - J.q0;
    const int bi = qi / J.ppe;
    const int part = qi - bi * J.ppe;
    const int nb = J.nb;
    const int items = J.m * nb;
    const uint8_t *X = J.x + (int64_t)bi * J.x_bstride;
    uint8_t *img = a.img + J.img0 + (int64_t)bi * items * kBlockBytes;
    const int li = lane & 7;

    const int it0 = part * kPartBlocks;
    const int it_end = min(it0 + kPartBlocks, items);
    float4 v[kPasses];
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        const int it = min(it0 + 8 * p, it_end - 8);       // a missing pass reloads the last
        const int r = it / nb;
        v[p] = *(const float4 *)(X + (int64_t)r * J.x_rstride + (it - r * nb) * 128 + lane * 16);
    }
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        uint32_t codes, dbits;
        quantize_block8(v[p].x, v[p].y, v[p].z, v[p].w, codes, dbits);
        if (it0 + 8 * p < it_end) {
            const int it = it0 + 8 * p + (lane >> 3);
            uint16_t *o = (uint16_t *)(img + (int64_t)it * kBlockBytes);
            if (li == 0) st_agent(o, (uint16_t)dbits);
            st_agent(o + 1 + 2 * li, (uint16_t)(codes & 0xffffu));
            st_agent(o + 2 + 2 * li, (uint16_t)(codes >> 16));
        }
    }
    // publish once every image store of this part is complete at agent scope;
    // the last part of the entry (the only one when ppe == 1) raises the flags
    // of the entry's tiles
    __builtin_amdgcn_s_waitcnt(0);
    bool last = true;
    if (J.ppe > 1) {
        int done = 0;
        if (lane == 0)
            done = __hip_atomic_fetch_add(a.parts + (int64_t)(J.e0 + bi) * kCtrStride, 1,
                                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = wave_uniform(done) == J.ppe - 1;
        if (last && lane == 0)
            __hip_atomic_store(a.parts + (int64_t)(J.e0 + bi) * kCtrStride, 0, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    if (last) {
        int32_t *f = a.flag + (J.tile0 + (int64_t)bi * J.tpb) * kFlagStride;
        for (int i = lane; i < J.tpb; i += kWave)
            __hip_atomic_store(f + (int64_t)i * kFlagStride, 1, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <int MT>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(MT == 1 ? 4 : 1)))
void step_kernel(const StepArgs a)
{
    __shared__ __align__(16) uint8_t stage[kStageBytes];
    __shared__ float red[MT * kWave];
    const int lane = threadIdx.x;
    if ((int)blockIdx.x < a.n_quant) {
        quantize_part(a, blockIdx.x);
        return;
    }
    const int t = (int)blockIdx.x - a.n_quant;
    int jj = 0;
    for (int i = 1; i < a.n_jobs; ++i)
        if (a.job[i].tile0 <= t) jj = i;
    const StepJob &J = a.job[jj];
    const int loc = t - J.tile0;
    const int bi = loc / J.tpb;
    const int row0 = (loc - bi * J.tpb) * J.R;
    const int rows = min(J.R, J.n - row0);
    const int nb = J.nb;
    const int Q = nb >> 2;
    const int live = rows * Q;
    const int c = lane % Q;
    const int M = J.m;

    // The tile takes its flag with an atomic exchange (read and clear in one
    // access, so no separate clearing store has to complete before the wave
    // ends), issued before the weight loads so that its value arrives without
    // waiting for them; normally the rows are already there.
    int32_t *flag = a.flag + (int64_t)t * kFlagStride;
    int f0 = 0;
    if (lane == 0) f0 = take_flag(flag);
    u32x4 g[kTileLoads];
    tile_issue(J.w + (int64_t)bi * J.w_bstride + (int64_t)row0 * nb * kBlockBytes,
               rows * nb * 17 / 8, lane, g);
    if (wave_uniform(f0) == 0) {
        int polls = 0;
        for (;;) {
            int f = 0;
            if (lane == 0) f = take_flag(flag);
            if (wave_uniform(f) != 0) break;
            if (++polls > kMaxPolls) {
                if (lane == 0)
                    __hip_atomic_store(a.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(Q8_STEP_SLEEP);
        }
    }
    const uint8_t *X = a.img + J.img0 + (int64_t)bi * M * nb * kBlockBytes;
    uint32_t xr[MT][kQuadDwords];
    float4 xd[MT];
    {
        u32x4 xv[kTileLoads];
        row_issue(X, nb, lane, xv);
        row_to_quad(stage, xv, nb, lane, c, xr[0], xd[0]);
    }
    if (MT > 1 && M > 1) {
        u32x4 xv[kTileLoads];
        row_issue(X + (int64_t)nb * kBlockBytes, nb, lane, xv);
        row_to_quad(stage, xv, nb, lane, c, xr[MT - 1], xd[MT - 1]);
    }
    uint32_t wq[kQuadDwords];
    tile_to_quad(stage, g, lane, live, wq);
    float dw0, dw1, dw2, dw3;
    quad_scales(wq, dw0, dw1, dw2, dw3);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        if (m < M) {
            int sb[4];
            const float acc = quad_dot(wq, xr[m], dw0, dw1, dw2, dw3, xd[m], sb);
            red[m * kWave + lane] = (lane < live) ? acc : 0.0f;
        }
    }
    wave_lds_sync();
    float *Y = J.y + (int64_t)bi * J.y_bstride;
    for (int i = lane; i < rows * M; i += kWave) {
        const int m = i / rows;
        const int r = i - m * rows;
        const float *pr = red + m * kWave + r * Q;
        float acc = pr[0];
        for (int cc = 1; cc < Q; ++cc) acc += pr[cc];
        Y[(int64_t)m * J.y_rstride + row0 + r] = acc;
    }
}

size_t align256(size_t v)
{
    return (v + 255) & ~(size_t)255;
}

}  // namespace

// Workspace: [0, 256) error word; then each job's quantized rows (batch x m x
// nb blocks, 256-byte aligned per job); then 256 bytes of part counter per
// batch entry; then one int32 flag per tile.
static int64_t tiles_of(const StreamDesc &d)
{
    const int64_t R = 64 / (d.nb / 4);
    return d.batch * ((d.n + R - 1) / R);
}

size_t step_ws_bytes(const StreamDesc *d, int n)
{
    size_t entries = 0, img = 0, tiles = 0;
    for (int i = 0; i < n; ++i) {
        entries += (size_t)d[i].batch;
        img += align256((size_t)(d[i].batch * d[i].m * d[i].nb) * kBlockBytes);
        tiles += (size_t)tiles_of(d[i]);
    }
    return 256 + img + entries * kCtrStride * 4 + align256(tiles * kFlagStride * 4);
}

bool step_ok(const StreamDesc &d)
{
    return d.x_f32 && d.m <= 2 && stream_fast_ok(d);
}

int launch_step(const StreamDesc *d, int n, void *ws, hipStream_t stream)
{
    StepArgs a;
    memset(&a, 0, sizeof(a));
    int64_t entries = 0, quant = 0, tiles = 0, img = 0;
    int mmax = 0, nj = 0;
    for (int i = 0; i < n; ++i) {
        if (d[i].n == 0 || d[i].m == 0 || d[i].batch == 0) continue;
        StepJob &J = a.job[nj++];
        const int64_t Q = d[i].nb / 4;
        const int64_t R = 64 / Q;
        const int64_t tpb = (d[i].n + R - 1) / R;
        const int64_t ppe = (d[i].m * d[i].nb + kPartBlocks - 1) / kPartBlocks;
        J.w = d[i].w; J.x = d[i].x; J.y = d[i].y;
        J.w_bstride = d[i].w_bstride; J.x_bstride = d[i].x_bstride; J.y_bstride = d[i].y_bstride;
        J.x_rstride = (int32_t)d[i].x_rstride; J.y_rstride = (int32_t)d[i].y_rstride;
        J.n = (int32_t)d[i].n; J.nb = (int32_t)d[i].nb; J.m = (int32_t)d[i].m;
        J.batch = (int32_t)d[i].batch;
        J.R = (int32_t)R;
        J.tpb = (int32_t)tpb;
        J.tile0 = (int32_t)tiles;
        J.q0 = (int32_t)quant;
        J.ppe = (int32_t)ppe;
        J.e0 = (int32_t)entries;
        J.img0 = img;
        tiles += d[i].batch * tpb;
        quant += d[i].batch * ppe;
        entries += d[i].batch;
        img += (int64_t)align256((size_t)(d[i].batch * d[i].m * d[i].nb) * kBlockBytes);
        if (d[i].m > mmax) mmax = (int)d[i].m;
    }
    if (nj == 0) return 0;
    const int64_t grid = quant + tiles;
    if (grid > 0x7fffffff || entries > 0x3fffffff) return -4;
    uint8_t *base = (uint8_t *)ws;
    a.n_jobs = nj;
    a.n_quant = (int32_t)quant;
    a.err = (int32_t *)base;
    a.img = base + 256;
    a.parts = (int32_t *)(base + 256 + img);
    a.flag = a.parts + entries * kCtrStride;
    if (mmax == 1)
        hipLaunchKernelGGL(step_kernel<1>, dim3((unsigned)grid), dim3(kWave), 0, stream, a);
    else
        hipLaunchKernelGGL(step_kernel<2>, dim3((unsigned)grid), dim3(kWave), 0, stream, a);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // namespace q8
