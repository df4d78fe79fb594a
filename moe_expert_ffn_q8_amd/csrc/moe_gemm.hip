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
//  1. routing (one workgroup): slot counts per expert, exclusive offsets, the
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

__global__ __launch_bounds__(kRouteThreads) void moe_route_tiles_kernel(const RouteArgs a)
{
    __shared__ int cnt[kMoeMaxExperts];
    __shared__ int scan_c[kMoeMaxExperts];
    __shared__ int scan_t[kMoeMaxExperts];
    __shared__ int bad;
    const int tid = threadIdx.x;
    for (int e = tid; e < kMoeMaxExperts; e += kRouteThreads) cnt[e] = 0;
    if (tid == 0) bad = 0;
    __syncthreads();
    for (int s = tid; s < a.n_slots; s += kRouteThreads) {
        const int e = a.ids[s];
        if (e < 0 || e >= a.n_expert) {
            atomicOr(&bad, 1);
            if (a.h_nan)
                for (int j = 0; j < a.n_ff; ++j) a.h_nan[(int64_t)s * a.n_ff + j] = __builtin_nanf("");
        } else {
            atomicAdd(&cnt[e], 1);
        }
    }
    __syncthreads();
    // inclusive scans of the counts and of the tile counts (Hillis-Steele)
    const int c = cnt[tid];
    int vc = c, vt = (c + kPBM - 1) / kPBM;
    scan_c[tid] = vc;
    scan_t[tid] = vt;
    __syncthreads();
    for (int d = 1; d < kMoeMaxExperts; d <<= 1) {
        const int ac = tid >= d ? scan_c[tid - d] : 0;
        const int at = tid >= d ? scan_t[tid - d] : 0;
        __syncthreads();
        vc += ac;
        vt += at;
        scan_c[tid] = vc;
        scan_t[tid] = vt;
        __syncthreads();
    }
    const int off = vc - c;                        // exclusive
    const int toff = vt - (c + kPBM - 1) / kPBM;
    if (tid < a.n_expert) {
        a.offsets[tid] = off;
        for (int i = 0; i * kPBM < c; ++i)
            a.tiles[toff + i] = TileEntry{tid, off + i * kPBM, min(kPBM, c - i * kPBM), 0};
    }
    if (tid == kRouteThreads - 1) {
        a.offsets[a.n_expert] = scan_c[a.n_expert - 1];
        a.hdr[0] = bad;
        a.hdr[1] = scan_t[a.n_expert - 1];
    }
    __syncthreads();
    // scatter the slots (the fill counters reuse cnt)
    for (int e = tid; e < kMoeMaxExperts; e += kRouteThreads) cnt[e] = 0;
    __syncthreads();
    for (int s = tid; s < a.n_slots; s += kRouteThreads) {
        const int e = a.ids[s];
        if (e >= 0 && e < a.n_expert) {
            const int p = atomicAdd(&cnt[e], 1);
            a.pairs[(e > 0 ? scan_c[e - 1] : 0) + p] = s;
        }
    }
}

// fp32 rows -> the tile layout of the A operand: codes [row][nb][32] (even
// blocks rotated by two bytes when the weights are native rows; in code order
// for R8 weights), scales [row][nb] as fp32.  Eight lanes own a block, four
// values each, with the rule and the bytes of q8_0_quantize_rows.
__global__ __launch_bounds__(256) void qa_quantize_kernel(const float *__restrict__ x,
                                                          int64_t row_stride,
                                                          uint8_t *__restrict__ codes,
                                                          float *__restrict__ scales, int64_t nb,
                                                          int64_t total_blocks, int rotate)
{
    const int tid = threadIdx.x;
    const int li = tid & 7;
    for (int64_t blk0 = (int64_t)blockIdx.x * kQaTileBlocks; blk0 < total_blocks;
         blk0 += (int64_t)gridDim.x * kQaTileBlocks) {
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
    int max_tiles, tiles_n;
};

// Output columns per workgroup: up_gate pairs waves w and w + 4 (gate and up
// rows of the same 32 columns), down gives every wave its own 32 columns.
template <bool UG>
constexpr int pg_cols()
{
    return UG ? 32 * kPWaves / 2 : 32 * kPWaves;
}

template <bool UG>
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

    // work = (column block, tile) with tiles fastest; consecutive work items
    // (the tiles of one expert for one column block) share an XCD
    const int nwg = (int)gridDim.x;
    const int work = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
    const int nt = work / a.max_tiles;
    const int mt = work - nt * a.max_tiles;
    if (nt >= a.tiles_n || mt >= a.hdr[1]) return;
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
    auto compute = [&](const uint8_t *stage, int bi0) {
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
            compute(bst0, bi0);
            issue_b(st + 2, bst0);
            __builtin_amdgcn_s_waitcnt(0x3f70 | kPStageLoads);
            compute(bst1, bi0 + 4);
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
constexpr int kR8Chunk = 64;

template <bool UG>
__global__ __launch_bounds__(kPThreads, 2) void moe_r8_gemm_kernel(const PgArgs a)
{
    __shared__ __align__(16) uint8_t la[kR8Chunk * 1024];
    __shared__ __align__(16) float ldx[kR8Chunk * kPBM];
    __shared__ int a_row[kPBM];
    __shared__ int a_slot[kPBM];

    const int tid = threadIdx.x;
    const int wave = wave_uniform(tid >> 6);
    const int lane = tid & 63;
    const int h = lane >> 5;
    const int li = lane & 31;

    const int nwg = (int)gridDim.x;
    const int work = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
    const int nt = work / a.max_tiles;
    const int mt = work - nt * a.max_tiles;
    if (nt >= a.tiles_n || mt >= a.hdr[1]) return;
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
    const int cbase = pg_cols<UG>() * nt + 32 * (UG ? (wave & 3) : wave);
    const int col = cbase + li;
    const bool wave_live = cbase < a.n_out;
    const int wrow0 = UG && wave >= 4 ? a.n_out + cbase : cbase;
    const int gbytes = 8 * kBlockBytes * nb;
    const int past = (int)a.expert_bytes;            // any offset here reads zero
    const int goff = wave_live ? (wrow0 / 8 + (li >> 3)) * gbytes : past;
    const int r = li & 7;
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.w + (int64_t)te.expert * a.expert_bytes), 0, past, kBufferWord3);

    u32x4 wc[kPDepth];
    uint32_t ws16[kPDepth];
    // default cache policy: the second tile of an expert (more than 32
    // slots) runs beside the first on the same XCD and finds its rows in L2
    auto issue = [&](int b, int i) {
        const bool in = b < nb;
        wc[i] = __builtin_amdgcn_raw_buffer_load_b128(
            rw, in ? goff + 16 * nb + 32 * (8 * b + r) + 16 * h : past, 0, 0);
        ws16[i] = __builtin_amdgcn_raw_buffer_load_b16(rw, in ? goff + 2 * (8 * b + r) : past, 0, 0);
    };
#pragma unroll
    for (int i = 0; i < kPDepth; ++i) issue(i, i);

    float acc[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[q] = 0.0f;

    const __amdgpu_buffer_rsrc_t rac = __builtin_amdgcn_make_buffer_rsrc(
        (void *)a.a_codes, 0, a.a_rows * nb * 32, kBufferWord3);
    const __amdgpu_buffer_rsrc_t ras = __builtin_amdgcn_make_buffer_rsrc(
        (void *)a.a_scales, 0, a.a_rows * nb * 4, kBufferWord3);
    const int a_past = a.a_rows * nb * 32;

    for (int kb0 = 0; kb0 < nb; kb0 += kR8Chunk) {
        const int kc = min(kR8Chunk, (nb - kb0 + kPDepth - 1) / kPDepth * kPDepth);
        __syncthreads();                 // a_row written; the previous chunk fully read
        const int ar = a_row[li];
        for (int bi = wave; bi < kc; bi += kPWaves) {
            const int b = kb0 + bi;
            const int off = ar >= 0 && b < nb ? (ar * nb + b) * 32 + 16 * h : a_past;
            auto *dst = (__attribute__((address_space(3))) void *)(la + 1024 * bi);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rac, dst, 16, off, 0, 0, 0);
        }
        for (int q = wave; 2 * q < kc; q += kPWaves) {
            const int b = kb0 + 2 * q + h;
            const int off = ar >= 0 && b < nb ? (ar * nb + b) * 4 : a_past;
            auto *dst = (__attribute__((address_space(3))) void *)(ldx + 64 * q);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ras, dst, 4, off, 0, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(0x3f70);    // vmcnt(0): this wave's copies landed
        __syncthreads();

        for (int bi0 = 0; bi0 < kc; bi0 += kPDepth) {
#pragma unroll
            for (int i = 0; i < kPDepth; ++i) {
                const int bi = bi0 + i;
                const u32x4 av = *(const u32x4 *)(la + 1024 * bi + 16 * lane);
                const u32x4 c = wc[i];
                v16i sres = {0};
                sres = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                    (v4i){(int)av.x, (int)av.y, (int)av.z, (int)av.w},
                    (v4i){(int)c.x, (int)c.y, (int)c.z, (int)c.w}, sres, 0, 0, 0);
                const float dw = half_bits_to_float(ws16[i]);
                float dx[16];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 v = *(const float4 *)&ldx[kPBM * bi + 8 * q + 4 * h];
                    dx[4 * q + 0] = v.x; dx[4 * q + 1] = v.y; dx[4 * q + 2] = v.z; dx[4 * q + 3] = v.w;
                }
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[q] = fmaf(dx[q] * dw, (float)sres[q], acc[q]);
                issue(kb0 + bi + kPDepth, i);
            }
        }
    }

    if (UG) {
        float *xch = (float *)la;
        __syncthreads();                       // every wave is done with the A tile
        if (wave >= 4) {
#pragma unroll
            for (int q = 0; q < 16; ++q) xch[((wave - 4) * 16 + q) * kWave + lane] = acc[q];
        }
        __syncthreads();
        if (wave >= 4 || !wave_live) return;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int row = 8 * (q >> 2) + 4 * h + (q & 3);
            if (row >= te.rows) continue;
            const float g = acc[q];
            const float u = xch[(wave * 16 + q) * kWave + lane];
            a.out[(int64_t)a_slot[row] * a.n_out + col] = g / (1.0f + expf(-g)) * u;
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
    size_t offsets, pairs, tiles, data, xq_scales, hq_scales, yslot, total;
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
    const size_t up_end = L.xq_scales + align256((size_t)n_tok * nbe * 4);
    L.hq_scales = L.data + align256((size_t)slots * nbf * 32);
    L.yslot = L.hq_scales + align256((size_t)slots * nbf * 4);
    const size_t down_end = L.yslot + align256((size_t)slots * n_embd * 4);
    L.total = down_end > up_end ? down_end : up_end;
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
    hipLaunchKernelGGL(moe_route_tiles_kernel, dim3(1), dim3(kRouteThreads), 0, stream, r);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

template <bool UG, bool R8>
int launch_grouped(const uint8_t *a_codes, const float *a_scales, int64_t a_rows, const uint8_t *w,
                   int64_t w_rows, int64_t nb, uint8_t *ws, const PrefillWs &L, float *out,
                   int64_t n_out, int64_t n_used, hipStream_t stream)
{
    PgArgs p;
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
    p.max_tiles = (int)L.max_tiles;
    p.tiles_n = (int)((n_out + pg_cols<UG>() - 1) / pg_cols<UG>());
    int64_t grid = L.max_tiles * p.tiles_n;
    grid = (grid + 7) & ~(int64_t)7;
    if (grid > 0x7fffffff) return -4;
    if (R8)
        hipLaunchKernelGGL(moe_r8_gemm_kernel<UG>, dim3((unsigned)grid), dim3(kPThreads), 0, stream, p);
    else
        hipLaunchKernelGGL(moe_gemm_kernel<UG>, dim3((unsigned)grid), dim3(kPThreads), 0, stream, p);
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

size_t moe_prefill_ws_bytes(int64_t n_tok, int64_t n_embd, int64_t n_ff, int64_t n_expert,
                            int64_t n_used)
{
    return prefill_layout(n_tok, n_embd, n_ff, n_expert, n_used).total;
}

int launch_moe_prefill_up_gate(const uint8_t *w, const float *x, const int32_t *ids, float *h,
                               void *ws_, int64_t n_tok, int64_t n_embd, int64_t n_ff,
                               int64_t n_expert, int64_t n_used, hipStream_t stream)
{
    uint8_t *ws = (uint8_t *)ws_;
    const PrefillWs L = prefill_layout(n_tok, n_embd, n_ff, n_expert, n_used);
    const int64_t nb = n_embd / kQK;
    if (int rc = launch_route(ids, ws, L, h, n_tok * n_used, n_expert, n_ff, stream)) return rc;
    uint8_t *xq = ws + L.data;
    float *xs = (float *)(ws + L.xq_scales);
    if (int rc = launch_qa_quantize(x, n_embd, xq, xs, n_tok, nb, true, stream)) return rc;
    return launch_grouped<true, false>(xq, xs, n_tok, w, 2 * n_ff, nb, ws, L, h, n_ff, n_used, stream);
}

int launch_moe_prefill_down(const uint8_t *w, const float *h, const int32_t *ids, const float *cw,
                            float *out, void *ws_, int64_t n_tok, int64_t n_embd, int64_t n_ff,
                            int64_t n_expert, int64_t n_used, hipStream_t stream)
{
    uint8_t *ws = (uint8_t *)ws_;
    const PrefillWs L = prefill_layout(n_tok, n_embd, n_ff, n_expert, n_used);
    const int64_t nb = n_ff / kQK;
    const int64_t slots = n_tok * n_used;
    if (int rc = launch_route(ids, ws, L, nullptr, slots, n_expert, n_ff, stream)) return rc;
    uint8_t *hq = ws + L.data;
    float *hs = (float *)(ws + L.hq_scales);
    if (int rc = launch_qa_quantize(h, n_ff, hq, hs, slots, nb, true, stream)) return rc;
    float *yslot = (float *)(ws + L.yslot);
    if (int rc = launch_grouped<false, false>(hq, hs, slots, w, n_embd, nb, ws, L, yslot, n_embd, n_used,
                                       stream))
        return rc;
    return launch_moe_combine(yslot, ids, cw, out, n_tok, n_embd, n_used, n_expert, stream);
}

int launch_moe_r8_prefill(const uint8_t *w_ug, const uint8_t *w_dn, const float *x,
                          const int32_t *ids, const float *cw, float *h, float *out, void *ws_,
                          int64_t n_tok, int64_t n_embd, int64_t n_ff, int64_t n_expert,
                          int64_t n_used, hipStream_t stream)
{
    uint8_t *ws = (uint8_t *)ws_;
    const PrefillWs L = prefill_layout(n_tok, n_embd, n_ff, n_expert, n_used);
    const int64_t nbe = n_embd / kQK, nbf = n_ff / kQK;
    const int64_t slots = n_tok * n_used;
    // one routing for both products (the tables stay in the workspace)
    if (int rc = launch_route(ids, ws, L, h, slots, n_expert, n_ff, stream)) return rc;
    uint8_t *q = ws + L.data;
    if (int rc = launch_qa_quantize(x, n_embd, q, (float *)(ws + L.xq_scales), n_tok, nbe, false,
                                    stream))
        return rc;
    if (int rc = launch_grouped<true, true>(q, (const float *)(ws + L.xq_scales), n_tok, w_ug,
                                            2 * n_ff, nbe, ws, L, h, n_ff, n_used, stream))
        return rc;
    if (int rc = launch_qa_quantize(h, n_ff, q, (float *)(ws + L.hq_scales), slots, nbf, false,
                                    stream))
        return rc;
    float *yslot = (float *)(ws + L.yslot);
    if (int rc = launch_grouped<false, true>(q, (const float *)(ws + L.hq_scales), slots, w_dn,
                                             n_embd, nbf, ws, L, yslot, n_embd, n_used, stream))
        return rc;
    return launch_moe_combine(yslot, ids, cw, out, n_tok, n_embd, n_used, n_expert, stream);
}

}  // namespace q8
