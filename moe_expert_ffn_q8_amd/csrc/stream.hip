// stream.hip -- the decode engine: Q8_0 x Q8_0 products with few token rows
// (m <= 16), streaming every weight byte from HBM exactly once.
//
// The block arithmetic is the dot product behind ggml_vec_dot_q8_0_q8_0 on
// the Gemma-4-on-Xeon page ("GPUなしで13年前のXeon上でGemma 4 26Bを毎秒5トーク
// ンで実行する", section on narrowing down the cause): an exact int32 sum of 32
// code products per block, then (d_w * d_x) * s in fp32.
//
// Work decomposition (gfx950, wave64):
//  * A weight row of nb blocks is nb/4 "quads" of 4 blocks (136 B).  A tile is
//    R = floor(64 / (nb/4)) whole rows, so each lane of a wave owns one quad
//    (lanes past R*(nb/4) idle).  With nb % 8 == 0 a tile starts on a 16-byte
//    boundary and is rows*nb*17/8 16-byte chunks long.
//  * A wave loads its tile with fully coalesced 16-byte non-temporal loads
//    (1 KB per instruction, up to 9 per lane), writes the chunks to its own
//    8.5 KB LDS slot in the same order, then every lane reads back its quad
//    with 17 8-byte LDS reads (lane stride 136 B: conflict-free).  The next
//    tile's loads are issued before the current tile is computed.
//  * Activations: the workgroup copies the m token rows of its matrix into
//    LDS once, as a "masked image" (the same 34-byte block layout with the
//    scale bytes zeroed) plus an fp32 scale array.  A lane's quad column is
//    the same for every tile, so with m == 1 the lane keeps its 34 image dwords
//    and 4 scales in registers for the whole kernel.
//  * Per quad and token: 34 v_dot4 (one per weight dword, no byte shuffling),
//    giving the four exact block sums; then 4 fp32 scale products.
//  * The nb/4 lanes of a row are combined in a fixed order through LDS, so a
//    launch shape always gives the same bits.
//
// Rows with nb % 8 != 0, nb > 256 or a weight matrix not on a 16-byte boundary
// go to a plain generic kernel (one wave per row, 2-byte loads).
#include <string.h>

#include "q8_device.h"
#include "q8_internal.h"

namespace q8 {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;

struct StreamJob {
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
    int32_t wg0;             // first workgroup of this job
    int32_t tiles_per_wg;
    int32_t rows_per_tile;   // R
    int32_t tiles_per_batch; // ceil(n / R)
    int32_t wg_per_batch;    // ceil(tiles_per_batch / tiles_per_wg)
};

struct StreamArgs {
    StreamJob job[kStreamMaxJobs];
    int32_t n_jobs;
    int32_t nb_max;
};

static_assert(sizeof(StreamArgs) <= 4000, "kernel arguments must stay below 4 KB");

template <int MT, bool SUMS>
__global__ __launch_bounds__(kThreads) void stream_kernel(const StreamArgs args)
{
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;

    int j = 0;
    for (int i = 1; i < args.n_jobs; ++i)
        if (args.job[i].wg0 <= (int)blockIdx.x) j = i;
    const StreamJob &J = args.job[j];

    const int wg = (int)blockIdx.x - J.wg0;
    const int bi = wg / J.wg_per_batch;
    const int wb = wg - bi * J.wg_per_batch;
    const int t0 = wb * J.tiles_per_wg;
    const int t1 = min(t0 + J.tiles_per_wg, J.tiles_per_batch);
    const int nb = J.nb;
    const int Q = nb >> 2;             // quads per row
    const int R = J.rows_per_tile;
    const int M = J.m;
    const int n = J.n;
    const int64_t row_bytes = (int64_t)nb * kBlockBytes;

    const uint8_t *W = J.w + (int64_t)bi * J.w_bstride;
    const uint8_t *X = J.x + (int64_t)bi * J.x_bstride;
    float *Y = J.y + (int64_t)bi * J.y_bstride;

    uint8_t *stage = smem + wave * kStageBytes;
    float *red = (float *)(smem + kWaves * kStageBytes) + wave * MT * kWave;
    uint8_t *ximg = smem + kWaves * kStageBytes + kWaves * MT * kWave * 4;
    const int img_row = nb * kBlockBytes;
    float *xsc = (float *)(ximg + MT * args.nb_max * kBlockBytes);

    u32x4 g[kTileLoads];
    auto issue = [&](int tt) {
        const int row0 = tt * R;
        const int rows = min(R, n - row0);
        tile_issue(W + (int64_t)row0 * row_bytes, rows * nb * 17 / 8, lane, g);
    };

    // The first tile's weight loads do not depend on the activations: issue
    // them before the activation round trip so the two latencies overlap.
    int t = t0 + wave;
    if (t < t1) issue(t);

    // ---- activations -> masked image + fp32 scales (whole workgroup) ----
    const int halves = M * nb * 17;
    for (int i = tid; i < halves; i += kThreads) {
        const int r = i / (nb * 17);
        const int rem = i - r * nb * 17;
        const int b = rem / 17;
        const int h = rem - b * 17;
        const uint32_t v = load_u16(X + (int64_t)r * J.x_rstride + b * kBlockBytes + 2 * h);
        uint16_t *img16 = (uint16_t *)(ximg + r * img_row);
        if (h == 0) {
            xsc[r * nb + b] = half_bits_to_float(v);
            img16[b * 17] = 0;
        } else {
            img16[b * 17 + h] = (uint16_t)v;
        }
    }
    __syncthreads();

    const int c = lane % Q;            // this lane's quad column (same for every tile)
    uint32_t xr[kQuadDwords];
    float xd0 = 0.f, xd1 = 0.f, xd2 = 0.f, xd3 = 0.f;
    if (MT == 1) {
        lds_quad(ximg + kQuadBytes * c, xr);
        const float4 s = *(const float4 *)(xsc + 4 * c);
        xd0 = s.x; xd1 = s.y; xd2 = s.z; xd3 = s.w;
    }

    for (; t < t1; t += kWaves) {
        const int row0 = t * R;
        const int rows = min(R, n - row0);
        const int live = rows * Q;
        uint32_t wq[kQuadDwords];
        tile_to_quad(stage, g, lane, live, wq);
        if (t + kWaves < t1) issue(t + kWaves);

        float dw0, dw1, dw2, dw3;
        quad_scales(wq, dw0, dw1, dw2, dw3);
        const int row = row0 + lane / Q;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            if (m < M) {
                uint32_t xt[kQuadDwords];
                const uint32_t *xq = xr;
                float4 dx = make_float4(xd0, xd1, xd2, xd3);
                if (MT != 1) {
                    lds_quad(ximg + m * img_row + kQuadBytes * c, xt);
                    xq = xt;
                    dx = *(const float4 *)(xsc + m * nb + 4 * c);
                }
                int s[4];
                const float acc = quad_dot(wq, xq, dw0, dw1, dw2, dw3, dx, s);
                red[m * kWave + lane] = (lane < live) ? acc : 0.0f;
                if (SUMS && lane < live) {
                    int32_t *o = J.sums + ((int64_t)m * n + row) * nb + 4 * c;
                    o[0] = s[0]; o[1] = s[1]; o[2] = s[2]; o[3] = s[3];
                }
            }
        }
        wave_lds_sync();
        for (int i = lane; i < rows * M; i += kWave) {
            const int m = i / rows;
            const int r = i - m * rows;
            const float *p = red + m * kWave + r * Q;
            float acc = p[0];
            for (int cc = 1; cc < Q; ++cc) acc += p[cc];
            Y[(int64_t)m * J.y_rstride + row0 + r] = acc;
        }
        wave_lds_sync();
    }
}

// ---------------------------------------------------------------------------
// Flat engine for m <= 2 (decode at batch 1 and 2).
//
// Every tile of every job and batch entry is numbered in one flat space; each
// workgroup is a single wave that takes a contiguous slice of that space (the
// launcher gives every wave one tile: the hardware dispatcher then balances the
// grid; with longer slices the wave keeps the next tile's loads in flight while
// it computes the current one).  A lane's
// activation quad (4 blocks) is loaded straight from global memory into
// registers, with the scale halfwords masked out, whenever the wave moves to
// a new (job, batch entry); there is no workgroup-wide staging and no barrier.

struct FlatJob {
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
    int32_t R;           // rows per tile
    int32_t tpb;         // tiles per batch entry
    int32_t tile0;       // first flat tile of this job
    int32_t x_al8;       // activation rows start on 8-byte boundaries
};

struct FlatArgs {
    FlatJob job[kStreamMaxJobs];
    int32_t n_jobs;
    int32_t total_tiles;
    int32_t tiles_per_wave;
    int32_t nb_max;      // XF: LDS image row length (blocks)
};

static_assert(sizeof(FlatArgs) <= 4000, "kernel arguments must stay below 4 KB");

// fp32 activations (XF): the wave quantizes the M rows of a (job, batch entry)
// into its LDS image, 8 lanes per block with the activation rule (the bytes
// are those of q8_0_quantize_rows), then every lane takes its quad.  The first
// kXPre passes of loads can be issued early (before the weights) into
// registers; longer rows load the rest pass by pass.
constexpr int kXPre = 3;

template <int P>
__device__ __forceinline__ void xf_prefetch(const uint8_t *X, int rstride, int M, int nb, int lane,
                                            float4 (&v)[P])
{
    const int items = M * nb;
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const int it = min((lane >> 3) + 8 * i, items - 1);     // clamped: always a real load
        const int row = it / nb;
        const int b = it - row * nb;
        v[i] = *(const float4 *)(X + (int64_t)row * rstride + b * 128 + (lane & 7) * 16);
    }
}

template <int P>
__device__ __forceinline__ void xf_quantize(const uint8_t *X, int rstride, int M, int nb, int lane,
                                            const float4 (&v)[P], uint8_t *img, float *sc)
{
    const int items = M * nb;
    const int img_row = nb * kBlockBytes;
    wave_lds_sync();
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const int it = (lane >> 3) + 8 * i;
        if (it < items) {
            const int row = it / nb;
            const int b = it - row * nb;
            quantize8_to_image(v[i], img + row * img_row, sc + row * nb, b, lane & 7);
        }
    }
    for (int it0 = 8 * P; it0 < items; it0 += 8) {
        const int it = it0 + (lane >> 3);
        if (it < items) {
            const int row = it / nb;
            const int b = it - row * nb;
            const float4 x = *(const float4 *)(X + (int64_t)row * rstride + b * 128 + (lane & 7) * 16);
            quantize8_to_image(x, img + row * img_row, sc + row * nb, b, lane & 7);
        }
    }
    wave_lds_sync();
}

template <int MT, bool SUMS, bool XF>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(MT == 1 ? 4 : 1)))
void stream_flat_kernel(const FlatArgs a)
{
    __shared__ __align__(16) uint8_t stage[kStageBytes];
    __shared__ float red[MT * kWave];
    extern __shared__ __align__(16) uint8_t xf_lds[];   // XF: MT image rows, then scales
    uint8_t *xf_img = xf_lds;
    float *xf_sc = (float *)(xf_lds + ((MT * a.nb_max * kBlockBytes + 15) & ~15));
    const int lane = threadIdx.x;
    const int t_begin = blockIdx.x * a.tiles_per_wave;
    const int t_end = min(t_begin + a.tiles_per_wave, a.total_tiles);
    if (t_begin >= t_end) return;

    int jj = 0;
    for (int i = 1; i < a.n_jobs; ++i)
        if (a.job[i].tile0 <= t_begin) jj = i;
    int loc = t_begin - a.job[jj].tile0;

    u32x4 g[kTileLoads];
    auto issue = [&](int j, int l) {
        const FlatJob &J = a.job[j];
        const int bi = l / J.tpb;
        const int row0 = (l - bi * J.tpb) * J.R;
        const int rows = min(J.R, J.n - row0);
        const uint8_t *base = J.w + (int64_t)bi * J.w_bstride +
                              (int64_t)row0 * J.nb * kBlockBytes;
        tile_issue(base, rows * J.nb * 17 / 8, lane, g);
    };

    int jx = -1, bx = -1;
    uint32_t xr[MT][kQuadDwords];
    float4 xd[MT];
    // XF: lanes take their quads from the wave's freshly quantized image
    auto xf_take = [&](const FlatJob &J, int c) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            if (m < J.m) {
                lds_quad(xf_img + m * J.nb * kBlockBytes + kQuadBytes * c, xr[m]);
                xd[m] = *(const float4 *)(xf_sc + m * J.nb + 4 * c);
            }
        }
    };
    if (XF) {
        // the first job's fp32 rows are loaded before the weights, so the
        // wait for them does not cover the tile loads
        const FlatJob &J = a.job[jj];
        const int bi = loc / J.tpb;
        const uint8_t *X = J.x + (int64_t)bi * J.x_bstride;
        float4 xv[kXPre];
        xf_prefetch<kXPre>(X, J.x_rstride, J.m, J.nb, lane, xv);
        issue(jj, loc);
        xf_quantize<kXPre>(X, J.x_rstride, J.m, J.nb, lane, xv, xf_img, xf_sc);
        xf_take(J, lane % (J.nb >> 2));
        jx = jj;
        bx = bi;
    } else {
        issue(jj, loc);
        // the first tile's activations, in flight together with its weights
        const FlatJob &J = a.job[jj];
        const int bi = loc / J.tpb;
        const int c = lane % (J.nb >> 2);
        const uint8_t *X = J.x + (int64_t)bi * J.x_bstride + kQuadBytes * c;
#pragma unroll
        for (int m = 0; m < MT; ++m)
            if (m < J.m) load_x_quad(X + (int64_t)m * J.x_rstride, J.x_al8 != 0, xr[m], xd[m]);
        jx = jj;
        bx = bi;
    }
    for (int t = t_begin; t < t_end; ++t) {
        const FlatJob &J = a.job[jj];
        const int bi = loc / J.tpb;
        const int row0 = (loc - bi * J.tpb) * J.R;
        const int rows = min(J.R, J.n - row0);
        const int Q = J.nb >> 2;
        const int live = rows * Q;
        const int c = lane % Q;
        const int M = J.m;

        int jn = jj, ln = loc + 1;
        if (ln == J.batch * J.tpb) {
            jn = jj + 1;
            ln = 0;
        }
        // A new (job, batch entry): its activations first, while this tile's
        // weights are still in flight and before the next tile is issued, so
        // the wait covers only loads needed now (and the tile's quad is not
        // live yet, which keeps the register peak low).
        if (jj != jx || bi != bx) {
            if (XF) {
                const uint8_t *X = J.x + (int64_t)bi * J.x_bstride;
                float4 xv[kXPre];
                xf_prefetch<kXPre>(X, J.x_rstride, M, J.nb, lane, xv);
                xf_quantize<kXPre>(X, J.x_rstride, M, J.nb, lane, xv, xf_img, xf_sc);
                xf_take(J, c);
            } else {
                const uint8_t *X = J.x + (int64_t)bi * J.x_bstride + kQuadBytes * c;
#pragma unroll
                for (int m = 0; m < MT; ++m)
                    if (m < M) load_x_quad(X + (int64_t)m * J.x_rstride, J.x_al8 != 0, xr[m], xd[m]);
            }
            jx = jj;
            bx = bi;
        }

        uint32_t wq[kQuadDwords];
        tile_to_quad(stage, g, lane, live, wq);
        if (t + 1 < t_end) issue(jn, ln);

        float dw0, dw1, dw2, dw3;
        quad_scales(wq, dw0, dw1, dw2, dw3);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            if (m < M) {
                int sb[4];
                const float acc = quad_dot(wq, xr[m], dw0, dw1, dw2, dw3, xd[m], sb);
                red[m * kWave + lane] = (lane < live) ? acc : 0.0f;
                if (SUMS && lane < live) {
                    int32_t *o = J.sums + ((int64_t)m * J.n + row0 + lane / Q) * J.nb + 4 * c;
                    o[0] = sb[0]; o[1] = sb[1]; o[2] = sb[2]; o[3] = sb[3];
                }
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
        wave_lds_sync();
        jj = jn;
        loc = ln;
    }
}

// Paired tiles (m == 1): a single-wave workgroup issues the loads of two
// consecutive tiles at once (two register sets, 17 KB in flight per wave,
// 117 VGPRs: still 4 waves per SIMD), then computes the first and the second;
// the activation quad is reloaded only when the second tile belongs to another
// (job, batch entry).  Measured against one tile per workgroup: the
// Llama-110M-shaped step's engine launch 20.5 -> 19.8 us, the 262144 x 2048
// matvec 86.5 -> 85.7 us.  Q8_FLAT_PAIR=0 builds the one-tile form only.
#ifndef Q8_FLAT_PAIR
#define Q8_FLAT_PAIR 1
#endif

// Four independent waves (eight consecutive tiles) per workgroup: the
// 262144 x 2048 matvec 85.1 -> 83.4 us (a plain streaming read of the same
// 571 MB takes 83.0 us), the Llama-110M-shaped step unchanged (19.7 us).
#ifndef Q8_PAIR_WAVES
#define Q8_PAIR_WAVES 4
#endif
constexpr int kPairWaves = Q8_PAIR_WAVES;   // independent waves per workgroup

__global__ __launch_bounds__(kWave * kPairWaves) __attribute__((amdgpu_waves_per_eu(3)))
void stream_pair_kernel(const FlatArgs a)
{
    __shared__ __align__(16) uint8_t stage_all[kPairWaves][kStageBytes];
    __shared__ float red_all[kPairWaves][kWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = kPairWaves == 1 ? 0 : wave_uniform((int)threadIdx.x >> 6);
    uint8_t *stage = stage_all[wave];
    float *red = red_all[wave];
    const int t0 = 2 * ((int)blockIdx.x * kPairWaves + wave);
    if (t0 >= a.total_tiles) return;

    struct Tile {
        int j, bi, row0, rows;
    };
    auto locate = [&](int t) {
        int jj = 0;
        for (int i = 1; i < a.n_jobs; ++i)
            if (a.job[i].tile0 <= t) jj = i;
        const FlatJob &J = a.job[jj];
        const int loc = t - J.tile0;
        Tile T;
        T.j = jj;
        T.bi = loc / J.tpb;
        T.row0 = (loc - T.bi * J.tpb) * J.R;
        T.rows = min(J.R, J.n - T.row0);
        return T;
    };
    const bool two = t0 + 1 < a.total_tiles;
    const Tile A = locate(t0);
    const Tile B = locate(two ? t0 + 1 : t0);
    auto issue = [&](const Tile &T, bool real, u32x4 (&g)[kTileLoads]) {
        const FlatJob &J = a.job[T.j];
        const uint8_t *base = J.w + (int64_t)T.bi * J.w_bstride + (int64_t)T.row0 * J.nb * kBlockBytes;
        tile_issue(base, real ? T.rows * J.nb * 17 / 8 : 0, lane, g);
    };
    u32x4 ga[kTileLoads], gb[kTileLoads];
    issue(A, true, ga);
    issue(B, two, gb);

    uint32_t xr[kQuadDwords];
    float4 xd;
    auto load_x = [&](const Tile &T) {
        const FlatJob &J = a.job[T.j];
        const int c = lane % (J.nb >> 2);
        load_x_quad(J.x + (int64_t)T.bi * J.x_bstride + kQuadBytes * c, J.x_al8 != 0, xr, xd);
    };
    auto compute = [&](const Tile &T, const u32x4 (&g)[kTileLoads]) {
        const FlatJob &J = a.job[T.j];
        const int Q = J.nb >> 2;
        const int live = T.rows * Q;
        uint32_t wq[kQuadDwords];
        tile_to_quad(stage, g, lane, live, wq);
        float dw0, dw1, dw2, dw3;
        quad_scales(wq, dw0, dw1, dw2, dw3);
        int sb[4];
        const float acc = quad_dot(wq, xr, dw0, dw1, dw2, dw3, xd, sb);
        red[lane] = (lane < live) ? acc : 0.0f;
        wave_lds_sync();
        float *Y = J.y + (int64_t)T.bi * J.y_bstride;
        for (int r = lane; r < T.rows; r += kWave) {
            const float *pr = red + r * Q;
            float s = pr[0];
            for (int cc = 1; cc < Q; ++cc) s += pr[cc];
            Y[T.row0 + r] = s;
        }
        wave_lds_sync();
    };
    load_x(A);
    compute(A, ga);
    if (two) {
        if (B.j != A.j || B.bi != A.bi) load_x(B);
        compute(B, gb);
    }
}

// Generic path: one wave per (matrix, row); lanes stride over blocks with
// 2-byte loads; fixed-order xor-tree reduction.
__global__ __launch_bounds__(kWave) void stream_generic_kernel(StreamDesc d)
{
    const int lane = threadIdx.x;
    const int64_t row = blockIdx.x;
    const int64_t bi = blockIdx.y;
    const uint8_t *Wr = d.w + bi * d.w_bstride + row * d.nb * kBlockBytes;
    for (int64_t m = 0; m < d.m; ++m) {
        const uint8_t *Xr = d.x + bi * d.x_bstride + m * d.x_rstride;
        float acc = 0.0f;
        for (int64_t b = lane; b < d.nb; b += kWave) {
            const uint8_t *wb = Wr + b * kBlockBytes;
            const uint8_t *xb = Xr + b * kBlockBytes;
            int s = 0;
            for (int h = 1; h < 17; ++h) {
                const uint32_t wv = load_u16(wb + 2 * h);
                const uint32_t xv = load_u16(xb + 2 * h);
                s += (int)(int8_t)(wv & 0xff) * (int)(int8_t)(xv & 0xff);
                s += (int)(int8_t)(wv >> 8) * (int)(int8_t)(xv >> 8);
            }
            if (d.sums) d.sums[(m * d.n + row) * d.nb + b] = s;
            acc = fmaf(half_bits_to_float(load_u16(wb)) * half_bits_to_float(load_u16(xb)),
                       (float)s, acc);
        }
        for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
        if (lane == 0) d.y[bi * d.y_bstride + m * d.y_rstride + row] = acc;
    }
}

bool stream_fast_ok(const StreamDesc &d)
{
    if (d.nb % 8 != 0 || d.nb > kStreamMaxNb) return false;
    if (d.x_f32 && (((uintptr_t)d.x) % 16 != 0 || d.x_rstride % 16 != 0 || d.x_bstride % 16 != 0))
        return false;
    if (((uintptr_t)d.w) % 16 != 0 || d.w_bstride % 16 != 0) return false;
    if (d.m > kStreamMaxM) return false;
    if (d.n > (int64_t)1 << 30 || d.batch > (int64_t)1 << 20) return false;
    if (d.x_rstride > ((int64_t)1 << 31) - 1 || d.y_rstride > ((int64_t)1 << 31) - 1) return false;
    return true;
}

static int g_max_lds = 0;

int max_lds_bytes()
{
    if (g_max_lds == 0) {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
            v <= 0)
            v = 65536;
        g_max_lds = v;
    }
    return g_max_lds;
}

template <int MT, bool SUMS>
static int launch_fast_mt(const StreamArgs &a, int grid, size_t lds, hipStream_t stream)
{
    hipLaunchKernelGGL((stream_kernel<MT, SUMS>), dim3(grid), dim3(kThreads), lds, stream, a);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

static int cu_count()
{
    static int cus = 0;
    if (cus == 0) {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            v <= 0)
            v = 256;
        cus = v;
    }
    return cus;
}

template <int MT, bool SUMS, bool XF>
static int launch_flat_mt(const StreamDesc *d, int n, hipStream_t stream)
{
    int64_t nb_max = 8;
    for (int i = 0; i < n; ++i)
        if (d[i].nb > nb_max) nb_max = d[i].nb;
    const size_t lds = XF ? (size_t)((MT * nb_max * kBlockBytes + 15) & ~15) + (size_t)MT * nb_max * 4 : 0;
    if (lds + kStageBytes + MT * kWave * 4 > (size_t)max_lds_bytes()) return -4;
    FlatArgs a;
    memset(&a, 0, sizeof(a));
    a.nb_max = (int32_t)nb_max;
    int64_t total = 0;
    for (int i = 0; i < n; ++i) {
        FlatJob &J = a.job[i];
        const int64_t Q = d[i].nb / 4;
        const int64_t R = 64 / Q;
        const int64_t tpb = (d[i].n + R - 1) / R;
        J.w = d[i].w; J.x = d[i].x; J.y = d[i].y; J.sums = d[i].sums;
        J.w_bstride = d[i].w_bstride; J.x_bstride = d[i].x_bstride; J.y_bstride = d[i].y_bstride;
        J.x_rstride = (int32_t)d[i].x_rstride; J.y_rstride = (int32_t)d[i].y_rstride;
        J.n = (int32_t)d[i].n; J.nb = (int32_t)d[i].nb; J.m = (int32_t)d[i].m;
        J.batch = (int32_t)d[i].batch;
        J.R = (int32_t)R;
        J.tpb = (int32_t)tpb;
        J.tile0 = (int32_t)total;
        J.x_al8 = (((uintptr_t)d[i].x) % 8 == 0 && d[i].x_rstride % 8 == 0 &&
                   d[i].x_bstride % 8 == 0) ? 1 : 0;
        total += d[i].batch * tpb;
    }
    if (total > 0x7fffffff) return -4;
    // One tile per workgroup: the hardware dispatcher hands a freed wave slot
    // the next tile.  Measured against resident grids with contiguous tile
    // ranges per wave (2..8 tiles, the next tile's loads in flight): the
    // Llama-110M-shaped step's engine launch 21.3 -> 20.5 us, the 262144 x
    // 2048 matvec 93.5 -> 86.5 us.  The kernel still takes any tiles_per_wave.
    // With fp32 activations every wave quantizes the rows it reads, so there
    // the waves take longer slices (a resident grid of 16 waves per CU).
    int64_t tpw = 1;
    if (XF) {
        const int64_t waves = (int64_t)cu_count() * 16;
        tpw = (total + waves - 1) / waves;
        if (tpw < 1) tpw = 1;
    }
    a.n_jobs = n;
    a.total_tiles = (int32_t)total;
    a.tiles_per_wave = (int32_t)tpw;
    // pairs only where there are tiles enough to fill every wave slot twice
    // over (a 768 x 768 matvec, 77 tiles, takes 3.3 us paired against 2.7 us)
    if (Q8_FLAT_PAIR && MT == 1 && !SUMS && !XF && total >= 8192) {
        const int64_t pairs = (total + 1) / 2;
        hipLaunchKernelGGL(stream_pair_kernel, dim3((unsigned)((pairs + kPairWaves - 1) / kPairWaves)),
                           dim3(kWave * kPairWaves), 0, stream, a);
        return hipGetLastError() == hipSuccess ? 0 : -6;
    }
    const int64_t grid = (total + tpw - 1) / tpw;
    hipLaunchKernelGGL((stream_flat_kernel<MT, SUMS, XF>), dim3((unsigned)grid), dim3(kWave), lds, stream,
                       a);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

static int launch_flat(const StreamDesc *d, int n, hipStream_t stream)
{
    int mmax = 1;
    bool sums = false;
    for (int i = 0; i < n; ++i) {
        if (d[i].m > mmax) mmax = (int)d[i].m;
        if (d[i].sums) sums = true;
    }
    if (d[0].x_f32)
        return mmax == 1 ? launch_flat_mt<1, false, true>(d, n, stream)
                         : launch_flat_mt<2, false, true>(d, n, stream);
    if (sums) return mmax == 1 ? launch_flat_mt<1, true, false>(d, n, stream)
                               : launch_flat_mt<2, true, false>(d, n, stream);
    return mmax == 1 ? launch_flat_mt<1, false, false>(d, n, stream)
                     : launch_flat_mt<2, false, false>(d, n, stream);
}

static int launch_fast(const StreamDesc *d, int n, hipStream_t stream)
{
    StreamArgs a;
    memset(&a, 0, sizeof(a));
    int64_t total_tiles = 0;
    int mmax = 1, nbmax = 8;
    bool sums = false;
    for (int i = 0; i < n; ++i) {
        const int64_t Q = d[i].nb / 4;
        const int64_t R = 64 / Q;
        total_tiles += d[i].batch * ((d[i].n + R - 1) / R);
        if (d[i].m > mmax) mmax = (int)d[i].m;
        if (d[i].nb > nbmax) nbmax = (int)d[i].nb;
        if (d[i].sums) sums = true;
    }
    // Tiles per wave: enough waves to fill 256 CUs several times over, and
    // more tiles per wave (so each wave prefetches) once there are plenty.
    int64_t per_wave = total_tiles / (256 * 8 * kWaves);
    if (per_wave < 1) per_wave = 1;
    if (per_wave > 16) per_wave = 16;
    int64_t wg_total = 0;
    for (int i = 0; i < n; ++i) {
        StreamJob &J = a.job[i];
        const int64_t Q = d[i].nb / 4;
        const int64_t R = 64 / Q;
        const int64_t tpb = (d[i].n + R - 1) / R;
        int64_t tpw = per_wave * kWaves;
        if (total_tiles < 256 * kWaves) tpw = 1;           // small problems: spread wide
        else if (total_tiles < 256 * 8 * kWaves) tpw = 2;
        if (tpw > tpb) tpw = tpb;
        const int64_t wpb = (tpb + tpw - 1) / tpw;
        J.w = d[i].w; J.x = d[i].x; J.y = d[i].y; J.sums = d[i].sums;
        J.w_bstride = d[i].w_bstride; J.x_bstride = d[i].x_bstride; J.y_bstride = d[i].y_bstride;
        J.x_rstride = (int32_t)d[i].x_rstride; J.y_rstride = (int32_t)d[i].y_rstride;
        J.n = (int32_t)d[i].n; J.nb = (int32_t)d[i].nb; J.m = (int32_t)d[i].m;
        J.batch = (int32_t)d[i].batch;
        J.wg0 = (int32_t)wg_total;
        J.tiles_per_wg = (int32_t)tpw;
        J.rows_per_tile = (int32_t)R;
        J.tiles_per_batch = (int32_t)tpb;
        J.wg_per_batch = (int32_t)wpb;
        wg_total += d[i].batch * wpb;
    }
    if (wg_total > ((int64_t)1 << 31) - 1) return -4;
    a.n_jobs = n;
    a.nb_max = nbmax;
    int mt = 1;
    while (mt < mmax) mt <<= 1;
    const size_t lds = (size_t)kWaves * kStageBytes + (size_t)kWaves * mt * kWave * 4 +
                       (size_t)mt * nbmax * kBlockBytes + (size_t)mt * nbmax * 4;
    if (lds > (size_t)max_lds_bytes()) return -4;
    const int grid = (int)wg_total;
    if (sums) {
        switch (mt) {
            case 1: return launch_fast_mt<1, true>(a, grid, lds, stream);
            case 2: return launch_fast_mt<2, true>(a, grid, lds, stream);
            case 4: return launch_fast_mt<4, true>(a, grid, lds, stream);
            case 8: return launch_fast_mt<8, true>(a, grid, lds, stream);
            default: return launch_fast_mt<16, true>(a, grid, lds, stream);
        }
    }
    switch (mt) {
        case 1: return launch_fast_mt<1, false>(a, grid, lds, stream);
        case 2: return launch_fast_mt<2, false>(a, grid, lds, stream);
        case 4: return launch_fast_mt<4, false>(a, grid, lds, stream);
        case 8: return launch_fast_mt<8, false>(a, grid, lds, stream);
        default: return launch_fast_mt<16, false>(a, grid, lds, stream);
    }
}

int launch_stream(const StreamDesc *d, int n, hipStream_t stream)
{
    // Every limit is checked before anything is enqueued: the generic
    // descriptors' grid limits first, then the fast launch (whose own checks
    // precede its launch), and only then the generic launches, so a rejected
    // call has enqueued nothing.
    StreamDesc fast[kStreamMaxJobs];
    int generic[kStreamMaxJobs];
    int nf = 0, ng = 0;
    for (int i = 0; i < n; ++i) {
        if (d[i].n == 0 || d[i].m == 0 || d[i].batch == 0) continue;
        if (stream_fast_ok(d[i])) {
            fast[nf++] = d[i];
        } else if (d[i].x_f32) {
            return -4;                 // checked by the caller: fast shapes only
        } else {
            if (d[i].n > 0x7fffffff || d[i].batch > 65535) return -4;
            generic[ng++] = i;
        }
    }
    if (nf > 0) {
        int mmax = 1;
        for (int i = 0; i < nf; ++i)
            if (fast[i].m > mmax) mmax = (int)fast[i].m;
        int rc;
        if (mmax <= 2) rc = launch_flat(fast, nf, stream);
        else if (small_m_ok(fast, nf)) rc = launch_small_m(fast, nf, stream);
        else if (fast[0].x_f32) rc = -4;      // fp32 activations: matrix-core engine only
        else rc = launch_fast(fast, nf, stream);
        if (rc) return rc;
    }
    for (int g = 0; g < ng; ++g) {
        const StreamDesc &s = d[generic[g]];
        hipLaunchKernelGGL(stream_generic_kernel, dim3((unsigned)s.n, (unsigned)s.batch),
                           dim3(kWave), 0, stream, s);
        if (hipGetLastError() != hipSuccess) return -6;
    }
    return 0;
}

}  // namespace q8
