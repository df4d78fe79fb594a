// ffn.hip -- the dense FFN up_gate with SwiGLU in one pass (decode, m <= 2):
//   h[t][j] = silu(W[j] . x_t) * (W[n_ff + j] . x_t),   j < n_ff
// for a combined weight W [2*n_ff][n_embd] whose gate rows come first.
//
// The op is FUSED_UP_GATE, named beside MOE_FUSED_UP_GATE on the
// Gemma-4-on-Xeon page ("GPUなしで13年前のXeon上でGemma 4 26Bを毎秒5トークンで
// 実行する", section on the broken op paths); its split form is the one the
// runtime graph fallback of the three-part fix builds for the MoE case (two row
// views of the combined tensor, two products, silu(gate) * up).  Here the
// dense layer is the one-expert case of that computation.
//
// Work decomposition: the decode engine's tiles (R = floor(64 / (nb/4)) whole
// rows, one 4-block quad per lane, coalesced 16-byte loads staged through the
// wave's LDS slot), taken in pairs: a single-wave workgroup loads the gate
// rows [j0, j0 + R) and the up rows [n_ff + j0, n_ff + j0 + R) together (two
// register sets in flight), reduces both in the engine's fixed order and
// applies silu(g) * u in the epilogue, so g and u never leave the chip.  The
// gate and up sums are bitwise those of the decode engine for the same rows.
#include <string.h>

#include "q8_device.h"
#include "q8_internal.h"

namespace q8 {

namespace {

struct FfnJob {
    const uint8_t *w;        // [batch][2 n][nb] blocks
    const uint8_t *x;        // Q8_0 activation rows
    float *h;
    int64_t w_bstride;       // bytes
    int64_t x_bstride;       // bytes
    int64_t h_bstride;       // floats
    int32_t x_rstride;       // bytes
    int32_t h_rstride;       // floats
    int32_t n, nb, m, batch; // n = n_ff (rows per half)
    int32_t R;               // rows per tile
    int32_t tpb;             // tiles per batch entry
    int32_t tile0;           // first tile of this job
    int32_t x_al8;           // activation rows start on 8-byte boundaries
};

struct FfnArgs {
    FfnJob job[kStreamMaxJobs];
    int32_t n_jobs;
};

static_assert(sizeof(FfnArgs) <= 4000, "kernel arguments must stay below 4 KB");

template <int MT>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(MT == 1 ? 4 : 1)))
void dense_up_gate_kernel(const FfnArgs a)
{
    __shared__ __align__(16) uint8_t stage[kStageBytes];
    __shared__ float redg[MT * kWave];
    __shared__ float redu[MT * kWave];
    const int lane = threadIdx.x;
    const int t = blockIdx.x;
    int jj = 0;
    for (int i = 1; i < a.n_jobs; ++i)
        if (a.job[i].tile0 <= t) jj = i;
    const FfnJob &J = a.job[jj];
    const int loc = t - J.tile0;
    const int bi = loc / J.tpb;
    const int j0 = (loc - bi * J.tpb) * J.R;
    const int rows = min(J.R, J.n - j0);
    const int nb = J.nb;
    const int Q = nb >> 2;
    const int live = rows * Q;
    const int c = lane % Q;
    const int M = J.m;
    const int64_t row_bytes = (int64_t)nb * kBlockBytes;
    const int chunks = rows * nb * 17 / 8;

    const uint8_t *W = J.w + (int64_t)bi * J.w_bstride;
    u32x4 gg[kTileLoads], gu[kTileLoads];
    tile_issue(W + (int64_t)j0 * row_bytes, chunks, lane, gg);
    tile_issue(W + (int64_t)(J.n + j0) * row_bytes, chunks, lane, gu);

    uint32_t xr[MT][kQuadDwords];
    float4 xd[MT];
    const uint8_t *X = J.x + (int64_t)bi * J.x_bstride + kQuadBytes * c;
#pragma unroll
    for (int m = 0; m < MT; ++m)
        if (m < M) load_x_quad(X + (int64_t)m * J.x_rstride, J.x_al8 != 0, xr[m], xd[m]);

#pragma unroll
    for (int half = 0; half < 2; ++half) {
        uint32_t wq[kQuadDwords];
        tile_to_quad(stage, half == 0 ? gg : gu, lane, live, wq);
        float dw0, dw1, dw2, dw3;
        quad_scales(wq, dw0, dw1, dw2, dw3);
        float *red = half == 0 ? redg : redu;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            if (m < M) {
                int sb[4];
                const float acc = quad_dot(wq, xr[m], dw0, dw1, dw2, dw3, xd[m], sb);
                red[m * kWave + lane] = (lane < live) ? acc : 0.0f;
            }
        }
    }
    wave_lds_sync();
    float *H = J.h + (int64_t)bi * J.h_bstride;
    for (int i = lane; i < rows * M; i += kWave) {
        const int m = i / rows;
        const int r = i - m * rows;
        const float *pg = redg + m * kWave + r * Q;
        const float *pu = redu + m * kWave + r * Q;
        float gs = pg[0], us = pu[0];
        for (int cc = 1; cc < Q; ++cc) {
            gs += pg[cc];
            us += pu[cc];
        }
        H[(int64_t)m * J.h_rstride + j0 + r] = gs / (1.0f + expf(-gs)) * us;
    }
}

}  // namespace

// d[i].n = n_ff (rows per half of the combined weight), d[i].y = h; every
// descriptor on the fast path (checked by the caller), m <= 2.
int launch_dense_up_gate(const StreamDesc *d, int n, hipStream_t stream)
{
    FfnArgs a;
    memset(&a, 0, sizeof(a));
    int64_t total = 0;
    int mmax = 1, nj = 0;
    for (int i = 0; i < n; ++i) {
        if (d[i].n == 0 || d[i].m == 0 || d[i].batch == 0) continue;
        FfnJob &J = a.job[nj++];
        const int64_t Q = d[i].nb / 4;
        const int64_t R = 64 / Q;
        const int64_t tpb = (d[i].n + R - 1) / R;
        J.w = d[i].w; J.x = d[i].x; J.h = d[i].y;
        J.w_bstride = d[i].w_bstride; J.x_bstride = d[i].x_bstride; J.h_bstride = d[i].y_bstride;
        J.x_rstride = (int32_t)d[i].x_rstride; J.h_rstride = (int32_t)d[i].y_rstride;
        J.n = (int32_t)d[i].n; J.nb = (int32_t)d[i].nb; J.m = (int32_t)d[i].m;
        J.batch = (int32_t)d[i].batch;
        J.R = (int32_t)R;
        J.tpb = (int32_t)tpb;
        J.tile0 = (int32_t)total;
        J.x_al8 = (((uintptr_t)d[i].x) % 8 == 0 && d[i].x_rstride % 8 == 0 &&
                   d[i].x_bstride % 8 == 0) ? 1 : 0;
        total += d[i].batch * tpb;
        if (d[i].m > mmax) mmax = (int)d[i].m;
    }
    if (nj == 0) return 0;
    if (total > 0x7fffffff) return -4;
    a.n_jobs = nj;
    if (mmax == 1)
        hipLaunchKernelGGL(dense_up_gate_kernel<1>, dim3((unsigned)total), dim3(kWave), 0, stream, a);
    else
        hipLaunchKernelGGL(dense_up_gate_kernel<2>, dim3((unsigned)total), dim3(kWave), 0, stream, a);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // namespace q8
