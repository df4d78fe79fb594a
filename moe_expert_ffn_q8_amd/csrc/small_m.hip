// small_m.hip -- decode products for a small batch of token rows (3 <= m <= 16)
// on the gfx950 int8 matrix cores, streaming every weight byte from HBM once.
//
// The block arithmetic is ggml_vec_dot_q8_0_q8_0's (Gemma-4-on-Xeon page,
// "GPUなしで13年前のXeon上でGemma 4 26Bを毎秒5トークンで実行する", section on
// narrowing down the cause): an exact int32 sum of the 32 code products of a
// block, then (d_w * d_x) * s in fp32, summed over the blocks of a row.
//
// With m tokens every weight quad would need m separate 4x int8 dot-product
// chains on the VALU; here one v_mfma_i32_16x16x32_i8 gives the exact int32
// block sums of up to 16 tokens x 16 weight rows for one block (K = 32 is
// exactly one block), so the VALU only rescales: per lane and block four
// converts, four scale products and four fused multiply-adds.
//
// Work decomposition:
//  * A row group is 16 consecutive weight rows; a wave owns whole row groups
//    and walks K in tiles of 8 blocks (16 rows x 272 B = 4352 B).  Tiles are
//    fetched with coalesced 16-byte non-temporal buffer loads into registers,
//    kDepth tiles ahead, then written to the wave's LDS slot and read back as
//    MFMA operands.  A row's 272-byte piece is 17 16-byte chunks, so the LDS
//    row pitch is 68 dwords and the 16 rows of a read fall on distinct banks.
//  * The workgroup (4 waves) works on one matrix of one batch entry: it first
//    copies the m activation rows into LDS in MFMA operand order (the "A
//    image") plus their fp32 block scales.  A = tokens (lane l: token l%16),
//    B = weight rows (lane l: row l%16); both operands carry the 32 codes of
//    a block in the same byte order, so the integer sum covers each code
//    product once.  Result register r of lane l is token 4*(l/16) + r, weight
//    row l%16.
//  * Byte order inside a block: a block whose codes start on a dword boundary
//    (odd block index: 34*b + 2 is then a multiple of 4) is taken as it is; a
//    block whose scale starts on a dword boundary (even index) has its first
//    and last code pairs in the dwords shared with the scales, so its first
//    virtual dword is [q0 q1 q30 q31] (one v_perm) and the other seven are
//    the aligned dwords in between.  The activation image uses the same order.
//  * Each output element is accumulated by one lane over the blocks in order,
//    so a launch shape always gives the same bits.
#include <string.h>

#include "q8_device.h"
#include "q8_internal.h"

namespace q8 {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kSmWaves = 4;
constexpr int kSmThreads = kSmWaves * kWave;
constexpr int kGroupRows = 16;
constexpr int kTileBlocks = 8;
constexpr int kPieceBytes = kTileBlocks * kBlockBytes;          // 272: one row's share of a tile
constexpr int kPieceChunks = kPieceBytes / 16;                  // 17
constexpr int kTileChunks = kGroupRows * kPieceChunks;          // 272
constexpr int kLoadsPerTile = (kTileChunks + kWave - 1) / kWave;   // 5
constexpr int kStageSlot = kLoadsPerTile * kWave * 16;          // 5120: a wave's LDS slot
#ifndef Q8_SMALLM_DEPTH
#define Q8_SMALLM_DEPTH 2
#endif
constexpr int kDepth = Q8_SMALLM_DEPTH;    // tiles in flight per wave
constexpr int kZeroPad = 16;
#ifndef Q8_SMALLM_WG_PER_CU
#define Q8_SMALLM_WG_PER_CU 8
#endif
constexpr int kWgPerCu = Q8_SMALLM_WG_PER_CU;
// Cache policy of this engine's weight loads.  A row's 272-byte pieces do not
// start on 128-byte lines, so consecutive tiles of a row share a line; with
// the default policy the second read usually hits L2 (non-temporal loads
// measured 1.25x the weight bytes in HBM reads and a lower rate).
#ifndef Q8_SMALLM_CACHE_POLICY
#define Q8_SMALLM_CACHE_POLICY 0
#endif
constexpr int kSmCache = Q8_SMALLM_CACHE_POLICY;

struct SmJob {
    const uint8_t *w;
    const uint8_t *x;
    float *y;
    int32_t *sums;
    int64_t w_bstride;   // bytes
    int64_t x_bstride;   // bytes
    int64_t y_bstride;   // floats
    int32_t x_rstride;   // bytes
    int32_t y_rstride;   // floats
    int32_t n, nb, m, batch;
    int32_t groups;      // row groups per matrix: ceil(n / 16)
    int32_t gpw;         // row groups per workgroup
    int32_t wpb;         // workgroups per batch entry
    int32_t wg0;         // first workgroup of this job
    int32_t x_al4;       // activation rows start on 4-byte boundaries
    int32_t x_f32;       // fp32 activation rows, quantized into the image here
};

struct SmArgs {
    SmJob job[kStreamMaxJobs];
    int32_t n_jobs;
};

static_assert(sizeof(SmArgs) <= 4000, "kernel arguments must stay below 4 KB");

__device__ __forceinline__ _Float16 half_lo(uint32_t v)
{
    return __builtin_bit_cast(_Float16, (uint16_t)(v & 0xffffu));
}

__device__ __forceinline__ _Float16 half_hi(uint32_t v)
{
    return __builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}

// Write the m activation rows of one matrix as the A image: for block b,
// lane group g (virtual dwords 2g, 2g+1) and token t, 8 bytes at
// ((b*4 + g)*MT + t)*8; then the fp32 block scales at [b][t].  Tokens m..MT-1
// are zero, and so are kZeroPad bytes after the scales (lanes past MT read
// their operands there instead of branching).  One thread per (block, token),
// items first_item.. (the earlier ones may have been written by a_q8_store);
// with 4-byte aligned rows every dword is one load.
template <int MT>
__device__ void build_a_image(const uint8_t *X, int x_rstride, bool al4, int m, int nb,
                              uint8_t *img, float *xsc, int tid, int first_item)
{
    for (int i = first_item + tid; i < nb * MT; i += kSmThreads) {
        const int b = i / MT;
        const int t = i - b * MT;
        uint32_t v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        uint32_t dbits = 0;
        if (t < m) {
            const uint8_t *blk = X + (int64_t)t * x_rstride + b * kBlockBytes;
            if (al4 && (b & 1) == 0) {
                // scale | q0 q1, seven code dwords, q30 q31 | next scale
                const uint32_t *p = (const uint32_t *)blk;
                const uint32_t d0 = p[0], d8 = p[8];
                dbits = d0 & 0xffffu;
                v[0] = (d0 >> 16) | (d8 << 16);
#pragma unroll
                for (int k = 1; k < 8; ++k) v[k] = p[k];
            } else if (al4) {
                // scale, then eight aligned code dwords
                const uint32_t *p = (const uint32_t *)(blk + 2);
                dbits = load_u16(blk);
#pragma unroll
                for (int k = 0; k < 8; ++k) v[k] = p[k];
            } else {
                // halfword h_i = bytes 2i, 2i+1 of the block (h0 = scale)
                dbits = load_u16(blk);
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    int lo, hi;
                    if ((b & 1) == 0) {
                        lo = k == 0 ? 1 : 2 * k;
                        hi = k == 0 ? 16 : 2 * k + 1;
                    } else {
                        lo = 2 * k + 1;
                        hi = 2 * k + 2;
                    }
                    v[k] = load_u16(blk + 2 * lo) | (load_u16(blk + 2 * hi) << 16);
                }
            }
        }
#pragma unroll
        for (int g = 0; g < 4; ++g)
            *(u32x2 *)(img + ((b * 4 + g) * MT + t) * 8) = (u32x2){v[2 * g], v[2 * g + 1]};
        xsc[i] = t < m ? half_bits_to_float(dbits) : 0.0f;
    }
    if (tid < kZeroPad / 4) xsc[nb * MT + tid] = 0.0f;
}

// The same image from fp32 activation rows, quantized here with the
// activation rule (8 lanes per (block, token), as the quantizer does; the
// codes are those of q8_0_quantize_rows).  A lane holds codes 4*li .. 4*li+3
// of its block; the virtual dword li of an even block is made from the high
// half of lane li-1 and the low half of lane li (lane 0: its low half and the
// high half of lane 7).  Loads go in batches of kFB per thread; the first
// batch is issued by the caller before the weights (first_batch).
constexpr int kFB = 8;

template <int MT>
__device__ __forceinline__ void a_f32_load(const uint8_t *X, int x_rstride, int m, int nb, int pass0,
                                           int tid, float4 (&v)[kFB])
{
    const int items = nb * MT;
#pragma unroll
    for (int i = 0; i < kFB; ++i) {
        int it = min((tid >> 3) + (pass0 + i) * (kSmThreads / 8), items - 1);
        int b = it / MT;
        int t = it - b * MT;
        if (t >= m) t = m - 1;                    // clamped: always a real load
        v[i] = *(const float4 *)(X + (int64_t)t * x_rstride + b * 128 + (tid & 7) * 16);
    }
}

template <int MT>
__device__ __forceinline__ void a_f32_store(int m, int nb, int pass0, int tid, const float4 (&v)[kFB],
                                            uint8_t *img, float *xsc)
{
    const int items = nb * MT;
    const int li = tid & 7;
    const int lane = tid & 63;
#pragma unroll
    for (int i = 0; i < kFB; ++i) {
        const int it = (tid >> 3) + (pass0 + i) * (kSmThreads / 8);
        if (it < items) {
            const int b = it / MT;
            const int t = it - b * MT;
            uint32_t codes, dbits;
            quantize_block8(v[i].x, v[i].y, v[i].z, v[i].w, codes, dbits);
            const uint32_t prev = (uint32_t)__shfl((int)codes, (lane & ~7) | ((li + 7) & 7));
            uint32_t vd = codes;
            if ((b & 1) == 0)
                vd = li == 0 ? (codes & 0xffffu) | (prev & 0xffff0000u) : (prev >> 16) | (codes << 16);
            if (t >= m) vd = 0;
            *(uint32_t *)(img + ((b * 4 + (li >> 1)) * MT + t) * 8 + (li & 1) * 4) = vd;
            if (li == 0) xsc[b * MT + t] = t < m ? half_bits_to_float(dbits) : 0.0f;
        }
    }
}

// Early form of the Q8_0 image copy for 4-byte aligned rows: the 9 dwords of
// up to kQP items (block, token) per thread are loaded before the weights
// (a_q8_load), and written once the weights are in flight (a_q8_store); the
// loads are unconditional (clamped item and token), so later waits are exact.
// The 9 dwords start at the block for an even block (scale | q0 q1, ..., q30
// q31 | next scale) and 2 bytes before it for an odd block (previous q30 q31 |
// scale, then the 8 aligned code dwords); neither reaches past the row.
constexpr int kQP = 2;

template <int MT>
__device__ __forceinline__ void a_q8_load(const uint8_t *X, int x_rstride, int m, int nb, int tid,
                                          uint32_t (&d)[kQP][9])
{
    const int items = nb * MT;
#pragma unroll
    for (int j = 0; j < kQP; ++j) {
        const int it = min(tid + j * kSmThreads, items - 1);
        const int b = it / MT;
        const int t = min(it - b * MT, m - 1);
        const uint32_t *p = (const uint32_t *)(X + (int64_t)t * x_rstride + b * kBlockBytes -
                                               ((b & 1) ? 2 : 0));
#pragma unroll
        for (int i = 0; i < 9; ++i) d[j][i] = p[i];
    }
}

template <int MT>
__device__ __forceinline__ void a_q8_store(int m, int nb, int tid, const uint32_t (&d)[kQP][9],
                                           uint8_t *img, float *xsc)
{
    const int items = nb * MT;
#pragma unroll
    for (int j = 0; j < kQP; ++j) {
        const int it = tid + j * kSmThreads;
        if (it < items) {
            const int b = it / MT;
            const int t = it - b * MT;
            uint32_t v[8];
            uint32_t dbits;
            if ((b & 1) == 0) {
                dbits = d[j][0] & 0xffffu;
                v[0] = (d[j][0] >> 16) | (d[j][8] << 16);
#pragma unroll
                for (int k = 1; k < 8; ++k) v[k] = d[j][k];
            } else {
                dbits = d[j][0] >> 16;
#pragma unroll
                for (int k = 0; k < 8; ++k) v[k] = d[j][k + 1];
            }
            const bool live = t < m;
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *(u32x2 *)(img + ((b * 4 + g) * MT + t) * 8) =
                    live ? (u32x2){v[2 * g], v[2 * g + 1]} : (u32x2){0u, 0u};
            xsc[it] = live ? half_bits_to_float(dbits) : 0.0f;
        }
    }
}

template <int MT, bool SUMS>
__global__ __launch_bounds__(kSmThreads) void stream_mfma_kernel(const SmArgs a)
{
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x;
    const int wave = wave_uniform(tid >> 6);
    const int lane = tid & 63;
    const int j16 = lane & 15;     // B column (weight row of the group) / A row (token)
    const int grp = lane >> 4;     // k-group of the operands, token quad of the result

    int jj = 0;
    for (int i = 1; i < a.n_jobs; ++i)
        if (a.job[i].wg0 <= (int)blockIdx.x) jj = i;
    const SmJob &J = a.job[jj];

    const int wg = (int)blockIdx.x - J.wg0;
    const int bi = wg / J.wpb;
    const int g0 = (wg - bi * J.wpb) * J.gpw;
    const int g1 = min(g0 + J.gpw, J.groups);
    const int nb = J.nb;
    const int kc = nb / kTileBlocks;             // tiles per row group
    const int n = J.n;
    const int m = J.m;
    const int64_t row_bytes = (int64_t)nb * kBlockBytes;

    const uint8_t *W = J.w + (int64_t)bi * J.w_bstride;
    const uint8_t *X = J.x + (int64_t)bi * J.x_bstride;
    float *Y = J.y + (int64_t)bi * J.y_bstride;

    uint8_t *stage = smem + wave * kStageSlot;
    uint8_t *img = smem + kSmWaves * kStageSlot;
    float *xsc = (float *)(img + nb * 32 * MT);

    // This wave's row groups: g0 + wave, g0 + wave + 4, ...; its tile count is
    // padded to a multiple of kDepth with empty tiles (no loads, no stores),
    // so every pass of the loop below issues and stages the same loads.
    const int my_groups = g1 - g0 > wave ? (g1 - g0 - wave + kSmWaves - 1) / kSmWaves : 0;
    const int ntiles = my_groups * kc;
    const int ntiles_pad = (ntiles + kDepth - 1) / kDepth * kDepth;

    // Chunk c of a tile (c = 64u + lane) is chunk c % 17 of row c / 17.
    uint32_t off[kLoadsPerTile];
#pragma unroll
    for (int u = 0; u < kLoadsPerTile; ++u) {
        const int c = u * kWave + lane;
        const int r = c / kPieceChunks;
        off[u] = c < kTileChunks ? (uint32_t)(r * row_bytes + 16 * (c - r * kPieceChunks))
                                 : 0x7ffffff0u;
    }

    u32x4 g[kDepth][kLoadsPerTile];
    int it = 0, ig = 0, ic = 0;     // issue pointer: tile, its group index and chunk
    auto issue = [&](u32x4 (&dst)[kLoadsPerTile]) {
        const bool live = it < ntiles;
        const int row0 = (g0 + wave + kSmWaves * ig) * kGroupRows;
        const int rows = min(kGroupRows, n - row0);
        const uint8_t *base = live ? W + (int64_t)row0 * row_bytes + ic * kPieceBytes : W;
        const int nrec = live ? (int)((rows - 1) * row_bytes) + kPieceBytes : 0;
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            (void *)wave_uniform(base), 0, wave_uniform(nrec), kBufferWord3);
#pragma unroll
        for (int u = 0; u < kLoadsPerTile; ++u)
            dst[u] = __builtin_amdgcn_raw_buffer_load_b128(r, off[u], 0, kSmCache);
        ++it;
        if (++ic == kc) {
            ic = 0;
            ++ig;
        }
    };

    if (J.x_f32) {
        // fp32 activations: the first batch of row loads goes out before the
        // weights, so waiting for it does not wait for the weights
        const int passes = (nb * MT * 8 + kSmThreads - 1) / kSmThreads;
        float4 v[kFB];
        a_f32_load<MT>(X, J.x_rstride, m, nb, 0, tid, v);
#pragma unroll
        for (int s = 0; s < kDepth; ++s) issue(g[s]);
        a_f32_store<MT>(m, nb, 0, tid, v, img, xsc);
        for (int p0 = kFB; p0 < passes; p0 += kFB) {
            a_f32_load<MT>(X, J.x_rstride, m, nb, p0, tid, v);
            a_f32_store<MT>(m, nb, p0, tid, v, img, xsc);
        }
        if (tid < kZeroPad / 4) xsc[nb * MT + tid] = 0.0f;
    } else if (J.x_al4) {
        // the first kQP items per thread are loaded before the weights
        uint32_t d[kQP][9];
        a_q8_load<MT>(X, J.x_rstride, m, nb, tid, d);
#pragma unroll
        for (int s = 0; s < kDepth; ++s) issue(g[s]);
        a_q8_store<MT>(m, nb, tid, d, img, xsc);
        if (nb * MT > kQP * kSmThreads)
            build_a_image<MT>(X, J.x_rstride, true, m, nb, img, xsc, tid, kQP * kSmThreads);
        else if (tid < kZeroPad / 4)
            xsc[nb * MT + tid] = 0.0f;
    } else {
#pragma unroll
        for (int s = 0; s < kDepth; ++s) issue(g[s]);
        build_a_image<MT>(X, J.x_rstride, false, m, nb, img, xsc, tid, 0);
    }
    __syncthreads();

    const uint32_t sel = grp == 0 ? 0x05040302u : 0x03020100u;
    // Operand addresses.  Lanes past MT (tokens that do not exist) read a live
    // token's operands instead of zeros: a row of A only reaches the same row
    // of the result, and those rows are never stored, so every lane can use
    // the same per-block stride (folded into the LDS offsets).
    const uint8_t *a_base = img + (grp * MT + (j16 % MT)) * 8;
    const uint8_t *d_base = (const uint8_t *)xsc + (grp % (MT / 4)) * 16;
    const uint8_t *w_row = stage + j16 * kPieceBytes;

    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    int ct = 0, cg = 0, cc = 0;    // compute pointer: tile, group index, chunk

    for (int t = 0; t < ntiles_pad; t += kDepth) {
#pragma unroll
        for (int s = 0; s < kDepth; ++s) {
            // stage tile t+s, refill its registers with tile t+s+kDepth
#pragma unroll
            for (int u = 0; u < kLoadsPerTile; ++u) ((u32x4 *)stage)[u * kWave + lane] = g[s][u];
            wave_lds_sync();
            issue(g[s]);

            // this tile's activation operands: blocks cc*8 .. cc*8+7
            const uint8_t *a_t = a_base + cc * (kTileBlocks * 32 * MT);
            const uint8_t *d_t = d_base + cc * (kTileBlocks * 4 * MT);
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const uint8_t *wr = w_row + q * kQuadBytes;
                const uint32_t *w32 = (const uint32_t *)wr;
                const int b0 = cc * kTileBlocks + 4 * q;
                // operands of the quad's four blocks
                const u32x2 p0 = *(const u32x2 *)(wr + 8 * grp);
                const u32x2 p3 = *(const u32x2 *)(wr + 104 + 8 * grp);
                const uint32_t d0 = w32[0], d8 = w32[8], d17 = w32[17], d25 = w32[25];
                const uint32_t p1x = w32[9 + 2 * grp], p1y = w32[10 + 2 * grp];
                const uint32_t p2x = w32[17 + 2 * grp], p2y = w32[18 + 2 * grp];
                uint64_t av[4];
                float4 dx[4];
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) {
                    av[bb] = *(const uint64_t *)(a_t + (4 * q + bb) * (32 * MT));
                    dx[bb] = *(const float4 *)(d_t + (4 * q + bb) * (4 * MT));
                }
                uint64_t wv[4];
                wv[0] = (uint64_t)__builtin_amdgcn_perm(d8, p0.x, sel) | ((uint64_t)p0.y << 32);
                wv[1] = (uint64_t)p1x | ((uint64_t)p1y << 32);
                wv[2] = (uint64_t)__builtin_amdgcn_perm(d25, p2x, sel) | ((uint64_t)p2y << 32);
                wv[3] = (uint64_t)p3.x | ((uint64_t)p3.y << 32);
                // Weight scales stay binary16: each scale product d_w * d_x is
                // one mixed-precision FMA with a zero addend (the same fp32
                // rounding as converting d_w first and multiplying).
                _Float16 dw[4];
                dw[0] = half_lo(d0);
                dw[1] = half_hi(d8);
                dw[2] = half_lo(d17);
                dw[3] = half_hi(d25);
                v4i S[4];
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) {
                    const v4i zero = {0, 0, 0, 0};
                    S[bb] = __builtin_amdgcn_mfma_i32_16x16x32_i8((long)av[bb], (long)wv[bb], zero,
                                                                  0, 0, 0);
                }
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) {
                    const float w = (float)dw[bb];
                    acc[0] = fmaf(fmaf(w, dx[bb].x, 0.0f), (float)S[bb][0], acc[0]);
                    acc[1] = fmaf(fmaf(w, dx[bb].y, 0.0f), (float)S[bb][1], acc[1]);
                    acc[2] = fmaf(fmaf(w, dx[bb].z, 0.0f), (float)S[bb][2], acc[2]);
                    acc[3] = fmaf(fmaf(w, dx[bb].w, 0.0f), (float)S[bb][3], acc[3]);
                    if (SUMS && ct < ntiles) {
                        const int row = (g0 + wave + kSmWaves * cg) * kGroupRows + j16;
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int tok = 4 * grp + r;
                            if (tok < m && row < n)
                                J.sums[((int64_t)tok * n + row) * nb + b0 + bb] = S[bb][r];
                        }
                    }
                }
            }
            wave_lds_sync();

            if (ct < ntiles && ++cc == kc) {
                const int row = (g0 + wave + kSmWaves * cg) * kGroupRows + j16;
                if (row < n) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int tok = 4 * grp + r;
                        if (tok < m) Y[(int64_t)tok * J.y_rstride + row] = acc[r];
                    }
                }
                acc[0] = acc[1] = acc[2] = acc[3] = 0.f;
                cc = 0;
                ++cg;
            }
            ++ct;
        }
    }
}

struct SmDev {
    int cus = 0;
};
SmDev g_sm;

template <int MT, bool SUMS>
int launch_mt(const SmArgs &a, int grid, size_t lds, hipStream_t stream)
{
    if (lds > 65536) {
        static bool attr_set = false;
        if (!attr_set) {
            if (hipFuncSetAttribute((const void *)stream_mfma_kernel<MT, SUMS>,
                                    hipFuncAttributeMaxDynamicSharedMemorySize,
                                    max_lds_bytes()) != hipSuccess)
                return -6;
            attr_set = true;
        }
    }
    hipLaunchKernelGGL((stream_mfma_kernel<MT, SUMS>), dim3(grid), dim3(kSmThreads), lds, stream, a);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // namespace

size_t small_m_lds_bytes(int64_t m, int64_t nb)
{
    const int mt = m <= 4 ? 4 : (m <= 8 ? 8 : 16);
    return (size_t)kSmWaves * kStageSlot + (size_t)nb * (32 + 4) * mt + kZeroPad;
}

bool small_m_ok(const StreamDesc *d, int n)
{
    int64_t mmax = 1, nbmax = 8;
    for (int i = 0; i < n; ++i) {
        if (d[i].m > mmax) mmax = d[i].m;
        if (d[i].nb > nbmax) nbmax = d[i].nb;
    }
    return mmax >= 3 && small_m_lds_bytes(mmax, nbmax) <= (size_t)max_lds_bytes();
}

int launch_small_m(const StreamDesc *d, int n, hipStream_t stream)
{
    if (g_sm.cus == 0) {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            v <= 0)
            v = 256;
        g_sm.cus = v;
    }
    SmArgs a;
    memset(&a, 0, sizeof(a));
    int64_t mmax = 1, nbmax = 8, total_bytes = 0;
    bool sums = false;
    for (int i = 0; i < n; ++i) {
        if (d[i].m > mmax) mmax = d[i].m;
        if (d[i].nb > nbmax) nbmax = d[i].nb;
        if (d[i].sums) sums = true;
        total_bytes += d[i].batch * d[i].n * d[i].nb * kBlockBytes;
    }
    // Workgroup size in bytes: the whole product spread over about
    // kWgPerCu workgroups per CU, each at least 4 row groups (one per wave).
    int64_t target = total_bytes / ((int64_t)g_sm.cus * kWgPerCu);
    if (target < 1) target = 1;
    int64_t wg_total = 0;
    for (int i = 0; i < n; ++i) {
        SmJob &J = a.job[i];
        const int64_t groups = (d[i].n + kGroupRows - 1) / kGroupRows;
        const int64_t group_bytes = (int64_t)kGroupRows * d[i].nb * kBlockBytes;
        int64_t gpw = (target + group_bytes - 1) / group_bytes;
        gpw = (gpw + kSmWaves - 1) / kSmWaves * kSmWaves;
        if (gpw < kSmWaves) gpw = kSmWaves;
        if (gpw > groups) gpw = groups;
        const int64_t wpb = (groups + gpw - 1) / gpw;
        J.w = d[i].w; J.x = d[i].x; J.y = d[i].y; J.sums = d[i].sums;
        J.w_bstride = d[i].w_bstride; J.x_bstride = d[i].x_bstride; J.y_bstride = d[i].y_bstride;
        J.x_rstride = (int32_t)d[i].x_rstride; J.y_rstride = (int32_t)d[i].y_rstride;
        J.n = (int32_t)d[i].n; J.nb = (int32_t)d[i].nb; J.m = (int32_t)d[i].m;
        J.batch = (int32_t)d[i].batch;
        J.groups = (int32_t)groups;
        J.gpw = (int32_t)gpw;
        J.wpb = (int32_t)wpb;
        J.wg0 = (int32_t)wg_total;
        J.x_al4 = (((uintptr_t)d[i].x) % 4 == 0 && d[i].x_rstride % 4 == 0 &&
                   d[i].x_bstride % 4 == 0) ? 1 : 0;
        J.x_f32 = d[i].x_f32;
        wg_total += d[i].batch * wpb;
    }
    if (wg_total > 0x7fffffff) return -4;
    a.n_jobs = n;
    const size_t lds = small_m_lds_bytes(mmax, nbmax);
    if (lds > (size_t)max_lds_bytes()) return -4;
    const int grid = (int)wg_total;
    if (mmax <= 4) return sums ? launch_mt<4, true>(a, grid, lds, stream)
                               : launch_mt<4, false>(a, grid, lds, stream);
    if (mmax <= 8) return sums ? launch_mt<8, true>(a, grid, lds, stream)
                               : launch_mt<8, false>(a, grid, lds, stream);
    return sums ? launch_mt<16, true>(a, grid, lds, stream) : launch_mt<16, false>(a, grid, lds, stream);
}

}  // namespace q8
