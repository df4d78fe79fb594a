// moe_gemm.hip -- the expert FFN for many tokens per call (prompt evaluation)
// on the gfx950 int8 matrix cores.
//
// Same computation as the decode kernels of moe.hip (Gemma-4-on-Xeon page,
// "GPUなしで13年前のXeon上でGemma 4 26Bを毎秒5トークンで実行する": the section on
// the broken op paths and the three-part fix, runtime graph fallback): mul_mat_id
// over the combined up_gate tensor with the gate half first, silu(gate) * up, the
// down projection of the quantized h rows, and the combine over a token's
// active experts.  That page reports prompt evaluation separately from decode;
// with many tokens each expert sees tens of token rows, so the products become
// small GEMMs and run on the matrix cores.
//
// One call:
//  1. routing (one workgroup per expert): slot counts per expert, exclusive offsets, the
//     slots grouped by expert, and a tile table -- expert e's c_e slots make
//     ceil(c_e / 32) tiles of at most 32 slots.  Slots with an out-of-range id
//     are left out; they set the error word and (up_gate call) get NaN h rows.
//  2. the token rows (up_gate) or h rows (down) quantized into the workspace
//     (codes and scales of q8_0_quantize_rows) in a layout made for the matrix
//     core: per row and block 32 code bytes, then the scales as fp32 in an
//     array of their own.  The codes of even blocks are stored rotated by two
//     bytes (code j at byte (j - 2) mod 32); the weight operand below uses the
//     same order, and a block's integer sum does not depend on the order of
//     its 32 products.
//  3. grouped GEMM: workgroup = (tile, block of output columns), 8 waves, one
//     32 x 32 tile of v_mfma_i32_32x32x32_i8 per wave (K = 32 = one block, so
//     each instruction gives exact int32 block sums, rescaled per block into
//     fp32 accumulators).  A = the tile's quantized rows, copied into LDS once
//     per 32 blocks (64 over R8 weights) by LDS-DMA loads, laid out so that
//     every operand read is one conflict-free 16-byte read.  B = the wave's
//     own 32 weight rows, no barrier inside the K loop:
//       native rows (moe_gemm_kernel): a 34-byte block holds its codes 2
//       bytes past a dword boundary in every other block, so each wave stages
//       the dword-aligned 16-byte pieces of the rotated order plus the dwords
//       holding the scales (and, for the second half of an even block, codes
//       0 and 1) through two per-wave LDS stages of 4 blocks, with coalesced
//       DMA at a row pitch of 11 slots;
//       R8 rows (moe_r8_gemm_kernel): the wave's rows are 4 whole groups, so
//       a block's operand is 4 runs of 256 contiguous bytes loaded straight
//       into registers, 8 blocks in flight, codes in their own order.
//     up_gate: waves 0..3 hold gate tiles, waves 4..7 the up tiles of the same
//     128 columns; the up tiles go through LDS and the epilogue writes
//     silu(g) * u element by element.  down: per-slot rows [slot][n_embd]
//     into the workspace.
//  4. down only: the decode path's combine kernel (ascending u per token).
// Every output element is a sum over its own row and column only, so the
// order of slots inside an expert's tiles does not change any result.
#include <string.h>

#include "q8_device.h"
#include "q8_internal.h"
#include "q8_moe.h"

namespace q8 {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kPWaves = 8;
constexpr int kPThreads = kPWaves * kWave;    // 512
constexpr int kPBM = 32;                      // slots per tile
constexpr int kPChunk = 32;                   // blocks of the A tile staged in LDS at a time
constexpr int kPDepth = 8;                    // blocks of the two weight stages of a wave
constexpr int kPSlots = 11;                   // 16-byte LDS slots per weight row and stage
constexpr int kPStageLoads = (32 * kPSlots + kWave - 1) / kWave;     // 6 DMA loads per stage
constexpr int kPWaveStage = kPStageLoads * kWave * 16;    // 6 KB: every DMA lane writes inside
constexpr int kPAlign = 4;                    // K in blocks must be a multiple of this
constexpr int kQaTileBlocks = 32;             // blocks per quantizer pass (256 threads)
constexpr int kRouteThreads = 1024;

struct TileEntry {
    int expert, row0, rows, pad;
};

struct RouteArgs {
    const int32_t *ids;
    int32_t *hdr;           // [0] error word, [1] tile count
    int32_t *offsets;       // [n_expert + 1]
    int32_t *pairs;         // [n_slots]
    TileEntry *tiles;       // [max_tiles]
    float *h_nan;           // up_gate call: h rows of out-of-range slots get NaN (else null)
    int n_slots, n_expert, n_ff;
};

constexpr int kRouteWaves = kRouteThreads / kWave;      // 16
constexpr int kRouteBatch = 4;                          // slot ids in flight per thread
constexpr int kRouteSuper = kRouteBatch * kRouteThreads;   // slots per pass of a workgroup

// The routing of one expert, e = the workgroup's index (a launch has one
// workgroup per expert).  Every workgroup reads all the ids and builds the
// whole per-expert histogram in LDS (the same counts in every workgroup),
// takes the exclusive prefixes of the counts and of the tile counts over the
// experts below e, and writes expert e's offset, its slots in ascending slot
// order and its tiles of at most kPBM slots; workgroup 0 also writes the
// totals, the error word and the NaN h rows of out-of-range slots.  Slot s of
// a pass starting at s0 is held by thread s - s0 - kRouteThreads k in its
// k-th register, so ascending slot order is (k, wave, lane) order.
__device__ __forceinline__ void route_tiles(const RouteArgs &a, int e)
{
    __shared__ int cnt[kMoeMaxExperts];
    __shared__ int wpre[kRouteBatch * kRouteWaves];      // hits per (k, wave), then their prefix
    __shared__ int red[4][kRouteWaves];
    __shared__ int bad;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    static_assert(kRouteThreads >= kMoeMaxExperts, "one thread per expert");
    static_assert(kRouteBatch * kRouteWaves <= kWave, "one lane per (k, wave) in the prefix");
    cnt[tid] = 0;
    if (tid == 0) bad = 0;
    __syncthreads();
    int ev[kRouteBatch];
    auto load = [&](int s0) {
#pragma unroll
        for (int k = 0; k < kRouteBatch; ++k) {
            const int s = s0 + k * kRouteThreads + tid;
            ev[k] = s < a.n_slots ? a.ids[s] : 0;
        }
    };
    for (int s0 = 0; s0 < a.n_slots; s0 += kRouteSuper) {
        load(s0);
#pragma unroll
        for (int k = 0; k < kRouteBatch; ++k) {
            const int s = s0 + k * kRouteThreads + tid;
            if (s >= a.n_slots) continue;
            if (ev[k] >= 0 && ev[k] < a.n_expert) {
                atomicAdd(&cnt[ev[k]], 1);
            } else {
                bad = 1;
                if (e == 0 && a.h_nan)
                    for (int j = 0; j < a.n_ff; ++j) a.h_nan[(int64_t)s * a.n_ff + j] = __builtin_nanf("");
            }
        }
    }
    __syncthreads();
    // exclusive prefixes below e and totals of the counts and tile counts
    const int c = tid < a.n_expert ? cnt[tid] : 0;
    const int t = (c + kPBM - 1) / kPBM;
    int v[4] = {tid < e ? c : 0, tid < e ? t : 0, c, t};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) v[q] += __shfl_xor(v[q], d);
        if (lane == 0) red[q][wave] = v[q];
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        v[q] = 0;
        for (int w = 0; w < kRouteWaves; ++w) v[q] += red[q][w];
    }
    const int off = v[0], toff = v[1];
    const int ce = cnt[e];
    if (tid == 0) a.offsets[e] = off;
    for (int i = tid; i * kPBM < ce; i += kRouteThreads)
        a.tiles[toff + i] = TileEntry{e, off + i * kPBM, min(kPBM, ce - i * kPBM), 0};
    if (e == 0 && tid == 0) {
        a.offsets[a.n_expert] = v[2];
        a.hdr[0] = bad;
        a.hdr[1] = v[3];
    }
    // expert e's slots in ascending order: per pass, the hits of every
    // (k, wave) are counted by ballots, one lane per (k, wave) of wave 0 takes
    // the exclusive prefix in slot order, and a hit's position is that prefix
    // plus its rank among the hits below it in its wave
    int run = 0;                             // hits of the passes before
    for (int s0 = 0; s0 < a.n_slots; s0 += kRouteSuper) {
        if (s0 > 0 || a.n_slots > kRouteSuper) load(s0);   // else the ids are still held
        uint64_t m[kRouteBatch];
#pragma unroll
        for (int k = 0; k < kRouteBatch; ++k) {
            const int s = s0 + k * kRouteThreads + tid;
            m[k] = __ballot(s < a.n_slots && ev[k] == e);
            if (lane == 0) wpre[k * kRouteWaves + wave] = __popcll(m[k]);
        }
        __syncthreads();
        if (wave == 0) {
            const int x = lane < kRouteBatch * kRouteWaves ? wpre[lane] : 0;
            int incl = x;
#pragma unroll
            for (int d = 1; d < kWave; d <<= 1) {
                const int y = __shfl_up(incl, d);
                if (lane >= d) incl += y;
            }
            if (lane < kRouteBatch * kRouteWaves) wpre[lane] = incl - x;
            red[0][0] = __shfl(incl, kWave - 1);
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kRouteBatch; ++k) {
            if ((m[k] >> lane) & 1)
                a.pairs[off + run + wpre[k * kRouteWaves + wave] + __popcll(m[k] & __lanemask_lt())] =
                    s0 + k * kRouteThreads + tid;
        }
        run += red[0][0];
        __syncthreads();                     // wpre and red reused by the next pass
    }
}

__global__ __launch_bounds__(kRouteThreads) void moe_route_tiles_kernel(const RouteArgs a)
{
    route_tiles(a, blockIdx.x);
}

// fp32 rows -> the tile layout of the A operand: codes [row][nb][32] (even
// blocks rotated by two bytes when the weights are native rows; in code order
// for R8 weights), scales [row][nb] as fp32.  Eight lanes own a block, four
// values each, with the rule and the bytes of q8_0_quantize_rows; workgroup
// wg of n_wg takes every n_wg-th pass of blockDim.x/8 blocks.
__device__ __forceinline__ void qa_quantize_tiles(const float *__restrict__ x, int64_t row_stride,
                                                  uint8_t *__restrict__ codes,
                                                  float *__restrict__ scales, int64_t nb,
                                                  int64_t total_blocks, int rotate, int64_t wg,
                                                  int64_t n_wg)
{
    const int tid = threadIdx.x;
    const int li = tid & 7;
    const int64_t per = blockDim.x / 8;
    for (int64_t blk0 = wg * per; blk0 < total_blocks; blk0 += n_wg * per) {
        const int64_t g = blk0 + (tid >> 3);
        const bool live = g < total_blocks;
        int64_t b = 0;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (live) {
            const int64_t r = g / nb;
            b = g - r * nb;
            v = *(const float4 *)(x + r * row_stride + b * kQK + 4 * li);
        }
        uint32_t c, dbits;
        quantize_block8(v.x, v.y, v.z, v.w, c, dbits);
        // codes 4li+2 .. 4li+5: the upper half of this lane's word and the
        // lower half of the next lane's (lane 7 wraps to codes 0 and 1)
        const uint32_t nxt = (uint32_t)__shfl((int)c, (tid & ~7) | ((tid + 1) & 7));
        const uint32_t out = (b & 1) || !rotate ? c : __builtin_amdgcn_alignbyte(nxt, c, 2);
        if (live) {
            ((uint32_t *)codes)[g * 8 + li] = out;
            if (li == 0) scales[g] = half_bits_to_float(dbits);
        }
    }
}

__global__ __launch_bounds__(256) void qa_quantize_kernel(const float *__restrict__ x,
                                                          int64_t row_stride,
                                                          uint8_t *__restrict__ codes,
                                                          float *__restrict__ scales, int64_t nb,
                                                          int64_t total_blocks, int rotate)
{
    qa_quantize_tiles(x, row_stride, codes, scales, nb, total_blocks, rotate, blockIdx.x, gridDim.x);
}

// The two independent first steps of a prefill call in one launch: the first
// n_expert workgroups route the slots (one expert each), the others quantize
// the token rows.
__global__ __launch_bounds__(kRouteThreads) void route_quantize_kernel(
    const RouteArgs r, const float *__restrict__ x, int64_t row_stride, uint8_t *__restrict__ codes,
    float *__restrict__ scales, int64_t nb, int64_t total_blocks, int rotate)
{
    if ((int)blockIdx.x < r.n_expert)
        route_tiles(r, blockIdx.x);
    else
        qa_quantize_tiles(x, row_stride, codes, scales, nb, total_blocks, rotate,
                          blockIdx.x - r.n_expert, gridDim.x - r.n_expert);
}

int launch_qa_quantize(const float *x, int64_t row_stride, uint8_t *codes, float *scales,
                       int64_t n_rows, int64_t nb, bool rotate, hipStream_t stream)
{
    const int64_t total = n_rows * nb;
    if (total == 0) return 0;
    const int64_t tiles = (total + kQaTileBlocks - 1) / kQaTileBlocks;
    const int64_t max_grid = 256 * 64;
    const unsigned grid = (unsigned)(tiles < max_grid ? tiles : max_grid);
    hipLaunchKernelGGL(qa_quantize_kernel, dim3(grid), dim3(256), 0, stream, x, row_stride, codes,
                       scales, nb, total, rotate ? 1 : 0);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

struct PgArgs {
    const uint8_t *a_codes;  // A rows, tile layout: token rows (up_gate) or slot rows (down)
    const float *a_scales;
    int a_rows;              // rows of the A arrays
    const uint8_t *w;        // weights [n_expert][w_rows][nb] native blocks
    int64_t expert_bytes;    // w_rows * nb * 34
    const int32_t *hdr;      // [1] = tile count
    const int32_t *pairs;
    const TileEntry *tiles;
    float *out;              // up_gate: h [slot][n_out]; down: yslot [slot][n_out]
    int n_out;               // n_ff (up_gate) or n_embd (down)
    int nb;                  // blocks per A / weight row (K / 32)
    int n_used;              // up_gate: A row of slot s is token s / n_used
    int tiles_n;             // column blocks
    int32_t *sums;           // validation (EMIT kernels): [slot][w_rows][nb] block sums
    uint8_t *hq_codes;       // R8 up_gate: q(h) in the A layout of the down product, or null
    float *hq_scales;
};

// Output columns per workgroup: up_gate pairs waves w and w + 4 (gate and up
// rows of the same 32 columns), down gives every wave its own 32 columns.
template <bool UG>
constexpr int pg_cols()
{
    return UG ? 32 * kPWaves / 2 : 32 * kPWaves;
}

// The work item (column block nt, tile mt) of this workgroup; false when it has
// none.  The grid is sized for the largest tile count; the T * tiles_n items of
// the tiles that exist (T, the routing's tile count, is known on the device
// only) are cut into 8 equal contiguous ranges, one per XCD (workgroups reach
// the XCDs round robin in launch order), so every XCD gets the same share, the
// workgroups with items are the first launched on each XCD, and consecutive
// items -- the tiles of one expert for one column block, which read the same
// weight rows -- run on one XCD and share its L2.
__device__ __forceinline__ bool pg_work(const PgArgs &a, int &nt, int &mt)
{
    const int T = a.hdr[1];
    const int n = T * a.tiles_n;
    const int per = (n + 7) >> 3;
    const int j = (int)(blockIdx.x >> 3);
    if (j >= per) return false;
    const int w = (int)(blockIdx.x & 7) * per + j;
    if (w >= n) return false;
    nt = w / T;
    mt = w - nt * T;
    return true;
}

// EMIT (validation builds of the same kernel): every exact int32 block sum is
// also written to a.sums.
template <bool UG, bool EMIT>
__global__ __launch_bounds__(kPThreads) void moe_gemm_kernel(const PgArgs a)
{
    // A tile: codes [b][half][row][16 bytes] (1 KB per block), scales [b][row]
    __shared__ __align__(16) uint8_t la[kPChunk * 1024];
    __shared__ __align__(16) float ldx[kPChunk * kPBM];
    // weights: two stages of 4 blocks per wave, as separate LDS objects so
    // that a read of one stage waits only for the copies into that stage
    __shared__ __align__(16) uint8_t bst0[kPWaves * kPWaveStage];
    __shared__ __align__(16) uint8_t bst1[kPWaves * kPWaveStage];
    __shared__ int a_row[kPBM];
    __shared__ int a_slot[kPBM];

    const int tid = threadIdx.x;
    const int wave = wave_uniform(tid >> 6);
    const int lane = tid & 63;
    const int h = lane >> 5;
    const int li = lane & 31;

    int nt, mt;
    if (!pg_work(a, nt, mt)) return;
    const TileEntry te = a.tiles[mt];
    const int nb = a.nb;
    const int steps = nb / 4;

    if (tid < kPBM) {
        const bool live = tid < te.rows;
        const int s = live ? a.pairs[te.row0 + tid] : -1;
        a_slot[tid] = s;
        a_row[tid] = live ? (UG ? s / a.n_used : s) : -1;
    }

    // this wave's 32 weight rows; rows past the output read as zero
    const int cbase = pg_cols<UG>() * nt + 32 * (UG ? (wave & 3) : wave);
    const int col = cbase + li;
    const bool wave_live = cbase < a.n_out;
    const int64_t row_bytes = (int64_t)nb * kBlockBytes;
    const int past = (int)a.expert_bytes;            // any offset here reads zero
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.w + (int64_t)te.expert * a.expert_bytes), 0, past, kBufferWord3);

    // A stage of 4 blocks (136 bytes of a row) in 11 slots of 16 bytes per row:
    // slots 0-3 bytes 4..68 (halves of blocks 0 and 1 in the rotated order),
    // 4-7 bytes 72..136 (blocks 2 and 3), 8 bytes 0..16 (block 0's scale and
    // codes 0,1), 9 bytes 64..80 (the same for block 2), 10 unused.  The row
    // pitch of 11 slots keeps 16-byte reads of 8 consecutive rows on distinct
    // banks.  DMA load u, lane l fills slot 64u + l of the wave's 32 x 11.
    int boff[kPStageLoads];
#pragma unroll
    for (int u = 0; u < kPStageLoads; ++u) {
        const int f = kWave * u + lane;
        const int r = f / kPSlots, q = f - r * kPSlots;
        const int wr = UG && wave >= 4 ? a.n_out + cbase + r : cbase + r;
        const int in_row = q < 4 ? 4 + 16 * q : q < 8 ? 72 + 16 * (q - 4) : q == 8 ? 0 : 64;
        boff[u] = (r < 32 && q < 10 && wave_live) ? (int)(wr * row_bytes) + in_row : -1;
    }
    auto issue_b = [&](int st, uint8_t *stage) {
        uint8_t *wbase = stage + wave * kPWaveStage;
        __builtin_amdgcn_s_waitcnt(0xc07f);    // lgkmcnt(0): this wave's reads of the stage are done
#pragma unroll
        for (int u = 0; u < kPStageLoads; ++u) {
            const int off = boff[u] >= 0 && st < steps ? boff[u] + st * 4 * kBlockBytes : past;
            auto *dst = (__attribute__((address_space(3))) void *)(wbase + 1024 * u);
            // default cache policy: a 136-byte stage is not line-aligned, so
            // consecutive stages of a row share a cache line (non-temporal
            // loads fetched 1.29x the weight bytes from HBM)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, dst, 16, off, 0, 0, 0);
        }
    };
    issue_b(0, bst0);
    issue_b(1, bst1);

    float acc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;

    const __amdgpu_buffer_rsrc_t rac = __builtin_amdgcn_make_buffer_rsrc(
        (void *)a.a_codes, 0, a.a_rows * nb * 32, kBufferWord3);
    const __amdgpu_buffer_rsrc_t ras = __builtin_amdgcn_make_buffer_rsrc(
        (void *)a.a_scales, 0, a.a_rows * nb * 4, kBufferWord3);
    const int a_past = a.a_rows * nb * 32;

    // The 4 blocks of a stage: every LDS operand is read first (the weight
    // halves from slot 11 li + 2j + h, the scale dwords, the token codes and
    // scales), then the 4 products are formed and rescaled in block order.
    // validation: the slot row of every result register, and this lane's
    // weight row within the expert (gate rows, then up rows, for up_gate)
    const int64_t w_rows = UG ? 2 * (int64_t)a.n_out : a.n_out;
    const int64_t wrow = (UG && wave >= 4 ? a.n_out : 0) + col;
    auto emit = [&](const v16i &sr, int b) {
        if (!EMIT || !wave_live || b >= nb) return;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = 8 * (r >> 2) + 4 * h + (r & 3);
            if (row < te.rows) a.sums[((int64_t)a_slot[row] * w_rows + wrow) * nb + b] = sr[r];
        }
    };

    auto compute = [&](const uint8_t *stage, int bi0, int bglob0) {
        const uint8_t *wb = stage + wave * kPWaveStage;
        u32x4 c[4], av[4];
        uint32_t d[4];
        float dx[4][16];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            c[j] = *(const u32x4 *)(wb + 16 * (kPSlots * li + 2 * j + h));
            // even j: the dword at the block's start (scale, codes 0 and 1);
            // odd j: the last dword of the previous block's second half
            const int dw_at = (j & 1) == 0 ? 4 * (kPSlots * li + 8 + j / 2) + j / 2
                                           : 4 * (kPSlots * li + 2 * j - 1) + 3;
            d[j] = ((const uint32_t *)wb)[dw_at];
            av[j] = *(const u32x4 *)(la + 1024 * (bi0 + j) + 16 * lane);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 v = *(const float4 *)&ldx[kPBM * (bi0 + j) + 8 * q + 4 * h];
                dx[j][4 * q + 0] = v.x; dx[j][4 * q + 1] = v.y;
                dx[j][4 * q + 2] = v.z; dx[j][4 * q + 3] = v.w;
            }
        }
        v16i sres[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            u32x4 cj = c[j];
            if ((j & 1) == 0 && h) cj.w = (cj.w & 0xffffu) | (d[j] & 0xffff0000u);
            sres[j] = (v16i){0};
            sres[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                (v4i){(int)av[j].x, (int)av[j].y, (int)av[j].z, (int)av[j].w},
                (v4i){(int)cj.x, (int)cj.y, (int)cj.z, (int)cj.w}, sres[j], 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t sbits = (j & 1) == 0 ? (d[j] & 0xffffu) : (d[j] >> 16);
            const float dw = half_bits_to_float(sbits);
            emit(sres[j], bglob0 + j);
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = fmaf(dx[j][r] * dw, (float)sres[j][r], acc[r]);
        }
    };

    for (int kb0 = 0; kb0 < nb; kb0 += kPChunk) {
        // blocks of this chunk, padded to whole stage pairs (the padding reads zero)
        const int kc = min(kPChunk, (nb - kb0 + kPDepth - 1) / kPDepth * kPDepth);
        __syncthreads();                 // a_row written; the previous chunk fully read
        const int ar = a_row[li];
        // codes: one DMA instruction per block (64 lanes x 16 bytes = 1 KB)
        for (int bi = wave; bi < kc; bi += kPWaves) {
            const int b = kb0 + bi;
            const int off = ar >= 0 && b < nb ? (ar * nb + b) * 32 + 16 * h : a_past;
            auto *dst = (__attribute__((address_space(3))) void *)(la + 1024 * bi);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rac, dst, 16, off, 0, 0, 0);
        }
        // scales: one dword DMA instruction per two blocks
        for (int q = wave; 2 * q < kc; q += kPWaves) {
            const int b = kb0 + 2 * q + h;
            const int off = ar >= 0 && b < nb ? (ar * nb + b) * 4 : a_past;
            auto *dst = (__attribute__((address_space(3))) void *)(ldx + 64 * q);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ras, dst, 4, off, 0, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(0x3f70);    // vmcnt(0): every copy of this wave landed
        __syncthreads();

        // two stages per iteration: wait for the older stage (the newer one's
        // 6 copies stay in flight), compute its 4 blocks, refill it 2 stages on
        for (int bi0 = 0; bi0 < kc; bi0 += kPDepth) {
            const int st = (kb0 + bi0) / 4;
            __builtin_amdgcn_s_waitcnt(0x3f70 | kPStageLoads);
            compute(bst0, bi0, kb0 + bi0);
            issue_b(st + 2, bst0);
            __builtin_amdgcn_s_waitcnt(0x3f70 | kPStageLoads);
            compute(bst1, bi0 + 4, kb0 + bi0 + 4);
            issue_b(st + 3, bst1);
        }
    }

    // slot row 8(r/4) + 4h + r%4 of the tile; column `col`
    if (UG) {
        float *xch = (float *)la;
        __syncthreads();                       // every wave is done with the A tile
        if (wave >= 4) {
#pragma unroll
            for (int r = 0; r < 16; ++r) xch[((wave - 4) * 16 + r) * kWave + lane] = acc[r];
        }
        __syncthreads();
        if (wave >= 4 || !wave_live) return;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = 8 * (r >> 2) + 4 * h + (r & 3);
            if (row >= te.rows) continue;
            const float g = acc[r];
            const float u = xch[(wave * 16 + r) * kWave + lane];
            a.out[(int64_t)a_slot[row] * a.n_out + col] = g / (1.0f + expf(-g)) * u;
        }
    } else {
        if (!wave_live) return;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = 8 * (r >> 2) + 4 * h + (r & 3);
            if (row < te.rows) a.out[(int64_t)a_slot[row] * a.n_out + col] = acc[r];
        }
    }
}

// The same grouped product over expert weights in the R8 layout (r8.hip: 8
// rows per group, scales first, 16-byte code chunks): a wave's 32 weight rows
// are 4 whole groups, so for one block its 64 lanes load 4 runs of 256
// contiguous bytes -- the MFMA operand itself, in code order -- straight into
// registers, 8 blocks in flight, and the 16 scale bytes of each group.  The
// token tile is staged in LDS once per 64 blocks (codes in code order).
#ifndef Q8_PG_R8_CHUNK
#define Q8_PG_R8_CHUNK 64
#endif
constexpr int kR8Chunk = Q8_PG_R8_CHUNK;
#ifndef Q8_PG_R8_DEPTH
#define Q8_PG_R8_DEPTH 8
#endif
constexpr int kR8Depth = Q8_PG_R8_DEPTH;       // weight blocks in flight per wave
// s_waitcnt operand for vmcnt(2 * kR8Depth) with the other counters left
// alone (vmcnt bits 3:0 and 15:14, expcnt 6:4 = 7, lgkmcnt 11:8 = 15)
constexpr int kVmcntDepth = ((2 * kR8Depth) & 15) | (((2 * kR8Depth) >> 4) << 14) | 0x70 | 0xf00;
static_assert(2 * kR8Depth < 64, "vmcnt holds at most 63");
// Build options of the kernel below, kept for measurement (512-token layer,
// R8 rows, per layer, 186 us with the defaults): Q8_PG_OUTER=1 forms the 16
// scale products of a block as an fp32 matrix-core outer product (2 VALU
// operations left per product instead of 3): 185 us; Q8_PG_R8_DEPTH (weight
// blocks in flight per wave) 4: 184 us (16: 235 us and more with the earlier
// work order); Q8_PG_R8_CHUNK=32 with Q8_PG_R8_OCC=6 and depth 4 (three
// workgroups per CU): 187 us; down workgroups of 4 waves
// (Q8_PG_R8_DN_WAVES=4, chunk 32, four workgroups per CU): 191 us; 16-wave
// down workgroups (512 columns, one per CU): 188 us, no change.  A second
// form of the K loop for tiles of at most 8 slots (the second tile of most
// experts with more than 32 slots), rescaling only the accumulators of its
// rows: 189 against 185 us (116 VGPRs, twice the code).  Per
// workgroup timestamps (s_memrealtime) put a workgroup's life at about 10 us
// waiting for its first blocks, 21 us in the K loop and 8 us in the epilogue
// (4 of them waiting for the last wave); the HBM reads (483 MB of the 428 MB
// of up_gate weights: the second tile of an expert mostly hits L2) run near
// what 64-lane loads of four 256-byte runs reach in a plain read (5.4 TB/s
// against 6.1 TB/s for 1 KB runs).
#ifndef Q8_PG_OUTER
#define Q8_PG_OUTER 0           // scale products on the fp32 matrix core (1) or the VALU (0)
#endif
typedef float v16f __attribute__((ext_vector_type(16)));

#ifndef Q8_PG_R8_OCC
#define Q8_PG_R8_OCC 2
#endif
// the down product's workgroups: waves (32 output columns each) and A-tile
// chunk in blocks
#ifndef Q8_PG_R8_DN_WAVES
#define Q8_PG_R8_DN_WAVES 8
#endif
#ifndef Q8_PG_R8_DN_CHUNK
#define Q8_PG_R8_DN_CHUNK 64
#endif
#ifndef Q8_PG_R8_DN_OCC
#define Q8_PG_R8_DN_OCC 2
#endif
constexpr int kR8DnWaves = Q8_PG_R8_DN_WAVES;
constexpr int kR8DnChunk = Q8_PG_R8_DN_CHUNK;
static_assert(kR8DnChunk % kR8Depth == 0, "whole prefetch batches per chunk");

// NW waves of 32 output columns (up_gate: 8, waves w and w + 4 the gate and
// up rows of the same columns), the A tile staged CH blocks at a time
template <bool UG, int NW>
constexpr int pg_r8_cols()
{
    return UG ? 32 * NW / 2 : 32 * NW;
}

template <bool UG, bool EMIT, int NW, int CH, int OCC>
__global__ __launch_bounds__(NW * kWave, OCC) void moe_r8_gemm_kernel(const PgArgs a)
{
    static_assert(!UG || NW == 8, "up_gate pairs waves w and w + 4");
    static_assert(!UG || CH * 1024 >= 2 * 16384, "the up_gate epilogue's up sums and h tile fit the A tile");
    static_assert(CH % kR8Depth == 0, "whole prefetch batches per chunk");
    // token scales first, then the token codes: every scale read of the K loop
    // then has an address below 64 KB, which the LDS read's immediate offset
    // field can hold (no vector address arithmetic per block)
    __shared__ __align__(16) uint8_t smem[CH * kPBM * 4 + CH * 1024];
    float *const ldx = (float *)smem;
    uint8_t *const la = smem + CH * kPBM * 4;
    __shared__ int a_row[kPBM];
    __shared__ int a_slot[kPBM];

    const int tid = threadIdx.x;
    const int wave = wave_uniform(tid >> 6);
    const int lane = tid & 63;
    const int h = lane >> 5;
    const int li = lane & 31;

    int nt, mt;
    if (!pg_work(a, nt, mt)) return;
    const TileEntry te = a.tiles[mt];
    const int nb = a.nb;

    if (tid < kPBM) {
        const bool live = tid < te.rows;
        const int s = live ? a.pairs[te.row0 + tid] : -1;
        a_slot[tid] = s;
        a_row[tid] = live ? (UG ? s / a.n_used : s) : -1;
    }

    // this wave's 32 weight rows = groups wrow0/8 .. wrow0/8 + 3 of the expert;
    // lane l takes row l%32 (group (l%32)/8, row l%8 of it), half l/32
    const int cbase = pg_r8_cols<UG, NW>() * nt + 32 * (UG ? (wave & 3) : wave);
    const int col = cbase + li;
    const bool wave_live = cbase < a.n_out;
    const int wrow0 = UG && wave >= 4 ? a.n_out + cbase : cbase;
    const int gbytes = 8 * kBlockBytes * nb;
    const int past = (int)a.expert_bytes;            // any offset here reads zero
    const int goff = wave_live ? (wrow0 / 8 + (li >> 3)) * gbytes : past;
    const int r = li & 7;
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.w + (int64_t)te.expert * a.expert_bytes), 0, past, kBufferWord3);

    u32x4 wc[kR8Depth];
    uint32_t ws32[kR8Depth];         // the aligned dword holding the row's binary16 scale
    // default cache policy: the second tile of an expert (more than 32
    // slots) runs beside the first on the same XCD and finds its rows in L2.
    // The lane's part of an offset is fixed; block b adds the same 256 b
    // (codes) and 16 b (scales) in every lane, passed as the scalar offset,
    // so a block's loads cost no vector arithmetic.  The prefetches past the
    // last block (never consumed) read the last block again.  The scale comes
    // as the dword holding it (rows r and r ^ 1; a whole 32-bit register, so
    // the compiler needs no zero-extension of it before the first use).
    const int vcode = goff + 16 * nb + 32 * r + 16 * h;
    const int vscale = goff + 2 * (r & 6);
    const int sshift = 16 * (r & 1);
    auto issue = [&](int b, int i) {
        const int bc = min(b, nb - 1);
        ws32[i] = __builtin_amdgcn_raw_buffer_load_b32(rw, vscale, 16 * bc, 0);
        wc[i] = __builtin_amdgcn_raw_buffer_load_b128(rw, vcode, 256 * bc, 0);
    };

    float acc[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[q] = 0.0f;

    const __amdgpu_buffer_rsrc_t rac = __builtin_amdgcn_make_buffer_rsrc(
        (void *)a.a_codes, 0, a.a_rows * nb * 32, kBufferWord3);
    const __amdgpu_buffer_rsrc_t ras = __builtin_amdgcn_make_buffer_rsrc(
        (void *)a.a_scales, 0, a.a_rows * nb * 4, kBufferWord3);
    const int a_past = a.a_rows * nb * 32;
    auto chunk_blocks = [&](int kb0) {
        return min(CH, (nb - kb0 + kR8Depth - 1) / kR8Depth * kR8Depth);
    };
    // the tile's codes and scales of blocks kb0 .. kb0 + kc - 1 into LDS
    // (zeros past the row or for missing slots), this wave's share
    auto stage = [&](int ar, int kb0, int kc) {
        for (int bi = wave; bi < kc; bi += NW) {
            const int b = kb0 + bi;
            const int off = ar >= 0 && b < nb ? (ar * nb + b) * 32 + 16 * h : a_past;
            auto *dst = (__attribute__((address_space(3))) void *)(la + 1024 * bi);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rac, dst, 16, off, 0, 0, 0);
        }
        for (int q = wave; 2 * q < kc; q += NW) {
            const int b = kb0 + 2 * q + h;
            const int off = ar >= 0 && b < nb ? (ar * nb + b) * 4 : a_past;
            auto *dst = (__attribute__((address_space(3))) void *)(ldx + 64 * q);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ras, dst, 4, off, 0, 0, 0);
        }
    };

    // The first chunk's copies go out before the weight prefetch: loads
    // complete in issue order, so the wave waits for its copies only (at
    // most the 2 * kR8Depth weight loads issued after them still in flight)
    // and starts on block 0 while the later blocks are still arriving.
    // The empty asm statements keep the compiler from reordering the loads.
    __syncthreads();                     // a_row written
    const int ar = a_row[li];
    stage(ar, 0, chunk_blocks(0));
    asm volatile("" ::: "memory");
    // block by block, scale before codes: the order the K loop issues them
    // in, so its waits count the same loads from the first block on
#pragma unroll
    for (int i = 0; i < kR8Depth; ++i) {
        issue(i, i);
        asm volatile("" ::: "memory");
    }

    for (int kb0 = 0; kb0 < nb; kb0 += CH) {
        const int kc = chunk_blocks(kb0);
        if (kb0 == 0) {
            __builtin_amdgcn_s_waitcnt(kVmcntDepth);
        } else {
            __syncthreads();             // the previous chunk fully read
            stage(ar, kb0, kc);
            __builtin_amdgcn_s_waitcnt(0x3f70);    // vmcnt(0): this wave's copies landed
        }
        __syncthreads();

        for (int bi0 = 0; bi0 < kc; bi0 += kR8Depth) {
#pragma unroll
            for (int i = 0; i < kR8Depth; ++i) {
                const int bi = bi0 + i;
                const u32x4 av = *(const u32x4 *)(la + 1024 * bi + 16 * lane);
                const u32x4 c = wc[i];
                v16i sres = {0};
                sres = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                    (v4i){(int)av.x, (int)av.y, (int)av.z, (int)av.w},
                    (v4i){(int)c.x, (int)c.y, (int)c.z, (int)c.w}, sres, 0, 0, 0);
                if (EMIT && wave_live && kb0 + bi < nb) {
                    const int64_t w_rows = UG ? 2 * (int64_t)a.n_out : a.n_out;
                    const int64_t wr = (UG && wave >= 4 ? a.n_out : 0) + col;
#pragma unroll
                    for (int q = 0; q < 16; ++q) {
                        const int row = 8 * (q >> 2) + 4 * h + (q & 3);
                        if (row < te.rows)
                            a.sums[((int64_t)a_slot[row] * w_rows + wr) * nb + kb0 + bi] = sres[q];
                    }
                }
                // the pin keeps the shift here: hoisted to the top of the
                // unrolled loop it would wait for every block in flight
                uint32_t sw = ws32[i];
                asm volatile("" : "+v"(sw));
                const float dw = half_bits_to_float(sw >> sshift);
                if (Q8_PG_OUTER) {
                    // P(r, c) = dx_r * dw_c as an outer product on the fp32 matrix
                    // core (k = 2, the second k row zero): the same 32x32
                    // register layout as the int32 tile, each product rounded once
                    const float adx = h == 0 ? ldx[kPBM * bi + li] : 0.0f;
                    v16f pz = {0.f};
                    const v16f P = __builtin_amdgcn_mfma_f32_32x32x2f32(adx, dw, pz, 0, 0, 0);
#pragma unroll
                    for (int q = 0; q < 16; ++q) {
                        acc[q] = fmaf(P[q], (float)sres[q], acc[q]);
                        // one block's sums at a time: left to itself the compiler
                        // sinks every block's float work below the loop and holds
                        // 32 matrix-core results per block
                        asm volatile("" : "+v"(acc[q]));
                    }
                } else {
                    float dx[16];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float4 v = *(const float4 *)&ldx[kPBM * bi + 8 * q + 4 * h];
                        dx[4 * q + 0] = v.x; dx[4 * q + 1] = v.y; dx[4 * q + 2] = v.z; dx[4 * q + 3] = v.w;
                    }
#pragma unroll
                    for (int q = 0; q < 16; ++q) acc[q] = fmaf(dx[q] * dw, (float)sres[q], acc[q]);
                }
                issue(kb0 + bi + kR8Depth, i);
            }
        }
    }

    if (UG) {
        float *xch = (float *)la;                        // up sums [4 waves][16][64]
        float *ht = (float *)(la + 4 * 16 * kWave * 4);  // h tile [kPBM][128]
        __syncthreads();                       // every wave is done with the A tile
        if (wave >= 4) {
#pragma unroll
            for (int q = 0; q < 16; ++q) xch[((wave - 4) * 16 + q) * kWave + lane] = acc[q];
        }
        __syncthreads();
        if (wave < 4 && wave_live) {
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int row = 8 * (q >> 2) + 4 * h + (q & 3);
                if (row >= te.rows) continue;
                const float g = acc[q];
                const float u = xch[(wave * 16 + q) * kWave + lane];
                const float hv = g / (1.0f + expf(-g)) * u;
                a.out[(int64_t)a_slot[row] * a.n_out + col] = hv;
                ht[row * 128 + 32 * wave + li] = hv;
            }
        }
        if (!a.hq_codes) return;
        __syncthreads();
        // q(h) of the tile (its rows x 4 blocks of 32 columns) with the rule and
        // the bytes of q8_0_quantize_rows, in the down product's A layout
        const int c0 = pg_r8_cols<UG, NW>() * nt;
        const int nbf = a.n_out / 32;
        for (int k = tid >> 3; k < kPBM * 4; k += NW * kWave / 8) {
            const int row = k >> 2, cb = k & 3;
            const bool live = row < te.rows && c0 + 32 * cb < a.n_out;
            const float4 v = live ? *(const float4 *)&ht[row * 128 + 32 * cb + 4 * (tid & 7)]
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
            uint32_t codes, dbits;
            quantize_block8(v.x, v.y, v.z, v.w, codes, dbits);
            if (live) {
                const int64_t blk = (int64_t)a_slot[row] * nbf + c0 / 32 + cb;
                ((uint32_t *)a.hq_codes)[blk * 8 + (tid & 7)] = codes;
                if ((tid & 7) == 0) a.hq_scales[blk] = half_bits_to_float(dbits);
            }
        }
    } else {
        if (!wave_live) return;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int row = 8 * (q >> 2) + 4 * h + (q & 3);
            if (row < te.rows) a.out[(int64_t)a_slot[row] * a.n_out + col] = acc[q];
        }
    }
}

size_t align256(size_t v)
{
    return (v + 255) & ~(size_t)255;
}

// Workspace layout of the prefill path (the up_gate call's token rows and the
// down call's slot rows share the data region).
struct PrefillWs {
    size_t offsets, pairs, tiles, data, xq_scales, hq_data, hq_scales, yslot, total;
    int64_t max_tiles;
};

PrefillWs prefill_layout(int64_t n_tok, int64_t n_embd, int64_t n_ff, int64_t n_expert,
                         int64_t n_used)
{
    PrefillWs L;
    const int64_t slots = n_tok * n_used;
    const int64_t nbe = n_embd / kQK, nbf = n_ff / kQK;
    L.max_tiles = slots / kPBM + n_expert + 1;
    L.offsets = 256;
    L.pairs = L.offsets + align256((size_t)(n_expert + 1) * 4);
    L.tiles = L.pairs + align256((size_t)slots * 4);
    L.data = L.tiles + align256((size_t)L.max_tiles * sizeof(TileEntry));
    L.xq_scales = L.data + align256((size_t)n_tok * nbe * 32);
    // the down product's A rows after the token rows: the R8 up_gate kernel
    // writes them while other workgroups still read the token rows
    L.hq_data = L.xq_scales + align256((size_t)n_tok * nbe * 4);
    L.hq_scales = L.hq_data + align256((size_t)slots * nbf * 32);
    L.yslot = L.hq_scales + align256((size_t)slots * nbf * 4);
    L.total = L.yslot + align256((size_t)slots * n_embd * 4);
    return L;
}

int launch_route(const int32_t *ids, uint8_t *ws, const PrefillWs &L, float *h_nan, int64_t n_slots,
                 int64_t n_expert, int64_t n_ff, hipStream_t stream)
{
    RouteArgs r;
    r.ids = ids;
    r.hdr = (int32_t *)ws;
    r.offsets = (int32_t *)(ws + L.offsets);
    r.pairs = (int32_t *)(ws + L.pairs);
    r.tiles = (TileEntry *)(ws + L.tiles);
    r.h_nan = h_nan;
    r.n_slots = (int)n_slots;
    r.n_expert = (int)n_expert;
    r.n_ff = (int)n_ff;
    hipLaunchKernelGGL(moe_route_tiles_kernel, dim3((unsigned)n_expert), dim3(kRouteThreads), 0, stream, r);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

// launch_route and launch_qa_quantize of the token rows in one launch
int launch_route_quantize(const int32_t *ids, uint8_t *ws, const PrefillWs &L, float *h_nan,
                          int64_t n_slots, int64_t n_expert, int64_t n_ff, const float *x,
                          int64_t row_stride, uint8_t *codes, float *scales, int64_t n_rows,
                          int64_t nb, bool rotate, hipStream_t stream)
{
    RouteArgs r;
    r.ids = ids;
    r.hdr = (int32_t *)ws;
    r.offsets = (int32_t *)(ws + L.offsets);
    r.pairs = (int32_t *)(ws + L.pairs);
    r.tiles = (TileEntry *)(ws + L.tiles);
    r.h_nan = h_nan;
    r.n_slots = (int)n_slots;
    r.n_expert = (int)n_expert;
    r.n_ff = (int)n_ff;
    const int64_t total = n_rows * nb;
    const int64_t per = kRouteThreads / 8;
    int64_t qwg = (total + per - 1) / per;
    if (qwg > 256 * 16) qwg = 256 * 16;
    hipLaunchKernelGGL(route_quantize_kernel, dim3((unsigned)(n_expert + qwg)), dim3(kRouteThreads), 0,
                       stream, r, x, row_stride, codes, scales, nb, total, rotate ? 1 : 0);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

template <bool UG, bool R8>
int launch_grouped(const uint8_t *a_codes, const float *a_scales, int64_t a_rows, const uint8_t *w,
                   int64_t w_rows, int64_t nb, uint8_t *ws, const PrefillWs &L, float *out,
                   int64_t n_out, int64_t n_used, hipStream_t stream, int32_t *sums = nullptr,
                   uint8_t *hq_codes = nullptr, float *hq_scales = nullptr)
{
    PgArgs p;
    p.sums = sums;
    p.hq_codes = hq_codes;
    p.hq_scales = hq_scales;
    p.a_codes = a_codes;
    p.a_scales = a_scales;
    p.a_rows = (int)a_rows;
    p.w = w;
    p.expert_bytes = w_rows * nb * kBlockBytes;
    p.hdr = (const int32_t *)ws;
    p.pairs = (const int32_t *)(ws + L.pairs);
    p.tiles = (const TileEntry *)(ws + L.tiles);
    p.out = out;
    p.n_out = (int)n_out;
    p.nb = (int)nb;
    p.n_used = (int)n_used;
    constexpr int NW = UG ? kPWaves : kR8DnWaves;
    constexpr int CH = UG ? kR8Chunk : kR8DnChunk;
    constexpr int OCC = UG ? Q8_PG_R8_OCC : Q8_PG_R8_DN_OCC;
    const int cols = R8 ? pg_r8_cols<UG, NW>() : pg_cols<UG>();
    p.tiles_n = (int)((n_out + cols - 1) / cols);
    int64_t grid = L.max_tiles * p.tiles_n;
    grid = (grid + 7) & ~(int64_t)7;
    if (grid > 0x7fffffff) return -4;
    if (R8 && sums)
        hipLaunchKernelGGL((moe_r8_gemm_kernel<UG, true, NW, CH, OCC>), dim3((unsigned)grid),
                           dim3(NW * kWave), 0, stream, p);
    else if (R8)
        hipLaunchKernelGGL((moe_r8_gemm_kernel<UG, false, NW, CH, OCC>), dim3((unsigned)grid),
                           dim3(NW * kWave), 0, stream, p);
    else if (sums)
        hipLaunchKernelGGL((moe_gemm_kernel<UG, true>), dim3((unsigned)grid), dim3(kPThreads), 0,
                           stream, p);
    else
        hipLaunchKernelGGL((moe_gemm_kernel<UG, false>), dim3((unsigned)grid), dim3(kPThreads), 0,
                           stream, p);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

// Validation: the routing tables of the workspace as counts [n_expert],
// offsets [n_expert + 1] and pairs [offsets[n_expert]] (one workgroup).
__global__ void route_export_kernel(const int32_t *ws_offsets, const int32_t *ws_pairs,
                                    int32_t *counts, int32_t *offsets, int32_t *pairs, int n_expert)
{
    const int total = ws_offsets[n_expert];
    for (int e = threadIdx.x; e <= n_expert; e += blockDim.x) {
        offsets[e] = ws_offsets[e];
        if (e < n_expert) counts[e] = ws_offsets[e + 1] - ws_offsets[e];
    }
    for (int i = threadIdx.x; i < total; i += blockDim.x) pairs[i] = ws_pairs[i];
}

// Validation: the Q8_0 bytes of rows in the A-operand layout (fp32 scales;
// codes of even blocks stored rotated, code j at byte (j - 2) mod 32, when
// `rotate`), one thread per block.
__global__ void qa_export_kernel(const uint8_t *codes, const float *scales, int64_t total_blocks,
                                 int64_t nb, int rotate, uint8_t *out)
{
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= total_blocks) return;
    const bool rot = rotate && ((g % nb) & 1) == 0;
    const uint8_t *src = codes + g * 32;
    uint8_t *dst = out + g * kBlockBytes;
    const uint16_t d = __builtin_bit_cast(uint16_t, (_Float16)scales[g]);
    dst[0] = (uint8_t)(d & 0xff);
    dst[1] = (uint8_t)(d >> 8);
    for (int j = 0; j < 32; ++j) dst[2 + j] = src[rot ? (j + 30) & 31 : j];
}

int launch_qa_export(const uint8_t *codes, const float *scales, int64_t n_rows, int64_t nb,
                     bool rotate, void *out, hipStream_t stream)
{
    const int64_t total = n_rows * nb;
    if (total == 0) return 0;
    hipLaunchKernelGGL(qa_export_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                       codes, scales, total, nb, rotate ? 1 : 0, (uint8_t *)out);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

int launch_route_export(const uint8_t *ws, const PrefillWs &L, const MoeEmit &e, int64_t n_expert,
                        hipStream_t stream)
{
    hipLaunchKernelGGL(route_export_kernel, dim3(1), dim3(1024), 0, stream,
                       (const int32_t *)(ws + L.offsets), (const int32_t *)(ws + L.pairs), e.counts,
                       e.offsets, e.pairs, (int)n_expert);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // namespace

bool moe_prefill_ok(int64_t n_tok, int64_t n_embd, int64_t n_ff, int64_t n_expert, int64_t n_used)
{
    if (n_tok <= kMoeDecodeMaxTok) return false;
    const int64_t nbe = n_embd / kQK, nbf = n_ff / kQK;
    if (nbe % kPAlign != 0 || nbf % kPAlign != 0) return false;
    if (n_tok > kMoePrefillMaxTok || n_tok * n_used > kMoePrefillMaxSlots) return false;
    // buffer-resource ranges and offsets are 32-bit
    const int64_t ug_expert = 2 * n_ff * nbe * kBlockBytes, dn_expert = n_embd * nbf * kBlockBytes;
    const int64_t xq = n_tok * nbe * kBlockBytes, hq = n_tok * n_used * nbf * kBlockBytes;
    const int64_t lim = 0x7f000000LL;   // leaves room for a row past the end
    if (nbe * kBlockBytes > (1 << 20) || nbf * kBlockBytes > (1 << 20)) return false;
    return ug_expert < lim && dn_expert < lim && xq < lim && hq < lim && n_expert <= kMoeMaxExperts;
}

int moe_prefill_check(int64_t n_tok, int64_t n_embd, int64_t n_ff, int64_t n_expert,
                      int64_t n_used)
{
    // the launch-shape limit of the two grouped products (checked again at
    // each launch; here before the call enqueues anything)
    const PrefillWs L = prefill_layout(n_tok, n_embd, n_ff, n_expert, n_used);
    const int64_t ug = L.max_tiles * ((n_ff + pg_cols<true>() - 1) / pg_cols<true>());
    constexpr int dn_cols = pg_r8_cols<false, kR8DnWaves>() < pg_cols<false>()
                                ? pg_r8_cols<false, kR8DnWaves>() : pg_cols<false>();
    const int64_t dn = L.max_tiles * ((n_embd + dn_cols - 1) / dn_cols);
    return (ug + 7 > 0x7fffffffLL || dn + 7 > 0x7fffffffLL) ? -4 : 0;
}

size_t moe_prefill_ws_bytes(int64_t n_tok, int64_t n_embd, int64_t n_ff, int64_t n_expert,
                            int64_t n_used)
{
    return prefill_layout(n_tok, n_embd, n_ff, n_expert, n_used).total;
}

int launch_moe_prefill_up_gate(const uint8_t *w, const float *x, const int32_t *ids, float *h,
                               void *ws_, int64_t n_tok, int64_t n_embd, int64_t n_ff,
                               int64_t n_expert, int64_t n_used, hipStream_t stream,
                               const MoeEmit *emit)
{
    uint8_t *ws = (uint8_t *)ws_;
    const PrefillWs L = prefill_layout(n_tok, n_embd, n_ff, n_expert, n_used);
    const int64_t nb = n_embd / kQK;
    uint8_t *xq = ws + L.data;
    float *xs = (float *)(ws + L.xq_scales);
    if (int rc = launch_route_quantize(ids, ws, L, h, n_tok * n_used, n_expert, n_ff, x, n_embd, xq,
                                       xs, n_tok, nb, true, stream))
        return rc;
    if (emit && emit->counts)
        if (int rc = launch_route_export(ws, L, *emit, n_expert, stream)) return rc;
    return launch_grouped<true, false>(xq, xs, n_tok, w, 2 * n_ff, nb, ws, L, h, n_ff, n_used, stream,
                                       emit ? emit->sums : nullptr);
}

int launch_moe_prefill_down(const uint8_t *w, const float *h, const int32_t *ids, const float *cw,
                            float *out, void *ws_, int64_t n_tok, int64_t n_embd, int64_t n_ff,
                            int64_t n_expert, int64_t n_used, hipStream_t stream,
                            const MoeEmit *emit)
{
    uint8_t *ws = (uint8_t *)ws_;
    const PrefillWs L = prefill_layout(n_tok, n_embd, n_ff, n_expert, n_used);
    const int64_t nb = n_ff / kQK;
    const int64_t slots = n_tok * n_used;
    if (int rc = launch_route(ids, ws, L, nullptr, slots, n_expert, n_ff, stream)) return rc;
    uint8_t *hq = ws + L.hq_data;
    float *hs = (float *)(ws + L.hq_scales);
    if (int rc = launch_qa_quantize(h, n_ff, hq, hs, slots, nb, true, stream)) return rc;
    if (emit && emit->hq)
        if (int rc = launch_qa_export(hq, hs, slots, nb, true, emit->hq, stream)) return rc;
    float *yslot = (float *)(ws + L.yslot);
    if (int rc = launch_grouped<false, false>(hq, hs, slots, w, n_embd, nb, ws, L, yslot, n_embd, n_used,
                                              stream, emit ? emit->sums : nullptr))
        return rc;
    return launch_moe_combine(yslot, ids, cw, out, n_tok, n_embd, n_used, n_expert, stream);
}

int launch_moe_r8_prefill(const uint8_t *w_ug, const uint8_t *w_dn, const float *x,
                          const int32_t *ids, const float *cw, float *h, float *out, void *ws_,
                          int64_t n_tok, int64_t n_embd, int64_t n_ff, int64_t n_expert,
                          int64_t n_used, hipStream_t stream, const MoeEmit *emit_ug,
                          const MoeEmit *emit_dn)
{
    uint8_t *ws = (uint8_t *)ws_;
    const PrefillWs L = prefill_layout(n_tok, n_embd, n_ff, n_expert, n_used);
    const int64_t nbe = n_embd / kQK, nbf = n_ff / kQK;
    const int64_t slots = n_tok * n_used;
    // one routing for both products (the tables stay in the workspace),
    // launched with the quantization of the token rows
    uint8_t *q = ws + L.data;
    if (int rc = launch_route_quantize(ids, ws, L, h, slots, n_expert, n_ff, x, n_embd, q,
                                       (float *)(ws + L.xq_scales), n_tok, nbe, false, stream))
        return rc;
    if (emit_ug && emit_ug->counts)
        if (int rc = launch_route_export(ws, L, *emit_ug, n_expert, stream)) return rc;
    // the up_gate kernel also writes q(h) in the down product's A layout
    uint8_t *hq = ws + L.hq_data;
    float *hs = (float *)(ws + L.hq_scales);
    if (int rc = launch_grouped<true, true>(q, (const float *)(ws + L.xq_scales), n_tok, w_ug,
                                            2 * n_ff, nbe, ws, L, h, n_ff, n_used, stream,
                                            emit_ug ? emit_ug->sums : nullptr, hq, hs))
        return rc;
    if (emit_dn && emit_dn->hq)
        if (int rc = launch_qa_export(hq, hs, slots, nbf, false, emit_dn->hq, stream)) return rc;
    float *yslot = (float *)(ws + L.yslot);
    if (int rc = launch_grouped<false, true>(hq, hs, slots, w_dn,
                                             n_embd, nbf, ws, L, yslot, n_embd, n_used, stream,
                                             emit_dn ? emit_dn->sums : nullptr))
        return rc;
    return launch_moe_combine(yslot, ids, cw, out, n_tok, n_embd, n_used, n_expert, stream);
}

}  // namespace q8
