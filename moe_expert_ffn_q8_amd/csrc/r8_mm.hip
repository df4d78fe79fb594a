// r8_mm.hip -- small-batch decode products (2..16 token rows) over weights in
// the row-interleaved R8 layout, on the gfx950 int8 matrix cores.
//
// Layout (see r8.hip; the Q8_0_R8 startup repack of the Gemma-4-on-Xeon page,
// "GPUなしで13年前のXeon上でGemma 4 26Bを毎秒5トークンで実行する", section on
// the fallback's cost and the repacking bug, read for 64-wide waves): group g
// of 8 rows is 272*nb bytes, scales first (index 8*b + r), then the 32 codes
// of row r at block b at 16*nb + 32*(8*b + r).
//
// Arithmetic (the block dot of ggml_vec_dot_q8_0_q8_0, same page, section on
// narrowing down the cause): exact int32 block sums, then (d_w*d_x)*s in fp32,
// blocks in ascending order per (token, row).
//
// One v_mfma_i32_32x32x32_i8 per block gives the exact int32 block sums of 32
// weight rows x 32 token rows (K = 32 = one block).  Its weight operand is
// lane l: row l%32, codes 16*(l/32)..+15 -- for the 32 rows of 4 consecutive
// groups at block b that is one 16-byte load per lane from four 256-byte runs,
// so the operand arrives straight from HBM in MFMA order, with no LDS pass and
// no byte shuffling.  The token operand (lane l: token l%32, same codes) comes
// from the activation rows staged once per workgroup in LDS (codes realigned to
// 32 bytes per block, fp32 scales), zeros past m.  Result register r of lane
// l holds token 8*(r/4) + 4*(l/32) + r%4 and weight row l%32: the lane rescales
// its 4 (m <= 8) or 8 (m <= 16) live values by d_w*d_x and accumulates them.
// Rows of 64 blocks or more are split over 2 or 4 waves of the workgroup
// (partial sums added in a fixed order through LDS); the blocks stream through
// two register buffers of 2 blocks each (68 VGPRs; 3, 4, 6 or 8 blocks per
// buffer measured slower).
//
// Measured on the GPT-2-shaped batch-8 step (49 products, 136 MB): 26.8 us per
// launch, level with the native-layout matrix-core engine (27.1 us).  What
// cost time on the way: activation loads made conditional (the compiler then
// waited for each in turn: 35 us), staging before the weight issue (31 us);
// more waves per unit and 8 or 16 waves per workgroup did not help.  The
// batch-1 engine's weight stream (one group per wave, contiguous 1 KB slices)
// with 4 v_dot4 and a DPP swap per slice and token instead of the matrix core
// (8 tokens, 71 VGPRs) took 40 us: per 1 KB slice the VALU work grows with m.
#include <string.h>

#include "q8_device.h"
#include "q8_internal.h"

namespace q8 {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kMmGroupBlockBytes = 8 * kBlockBytes;     // 272 per block column of a group
#ifndef Q8_R8MM_WAVES
#define Q8_R8MM_WAVES 4
#endif
constexpr int kMmWaves = Q8_R8MM_WAVES;
constexpr int kMmThreads = kMmWaves * kWave;
constexpr int kMmGroups = 4;                            // 32 weight rows per wave
#ifndef Q8_R8MM_SLICES
#define Q8_R8MM_SLICES 2
#endif
constexpr int kMmSlices = Q8_R8MM_SLICES;              // blocks per register buffer (two)

struct MmJob {
    const uint8_t *w;
    const uint8_t *x;      // Q8_0 rows of matrix 0
    float *y;
    int64_t w_bstride;     // bytes
    int64_t x_rstride;     // bytes between token rows
    int64_t x_bstride;     // bytes between matrices
    int64_t y_rstride;     // floats
    int64_t y_bstride;     // floats
    int32_t *sums;         // validation: int32 [batch][m][n][nb] block sums (SUMS kernels)
    int64_t n;
    int nb, m;
    int gpm;               // groups per matrix
    int upm;               // units (4 groups, 32 rows) per matrix
    int ks;                // waves sharing a unit, each over a slice of the blocks
    int nbp;               // blocks per slice
    int wgpm;              // workgroups per matrix
    int wg0;
};

struct MmArgs {
    MmJob job[kStreamMaxJobs];
    int n_jobs;
};

// SUMS (validation builds of the same kernel): every exact int32 block sum is
// also written out.
template <int MT, bool SUMS>
__global__ __launch_bounds__(kMmThreads) void r8_mm_kernel(const MmArgs a)
{
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int tid = threadIdx.x;
    int j = 0;
    while (j + 1 < a.n_jobs && (int)blockIdx.x >= a.job[j + 1].wg0) ++j;
    const MmJob &jb = a.job[j];
    const int rel = (int)blockIdx.x - jb.wg0;
    const int mb = rel / jb.wgpm;
    const int ks = jb.ks;
    const int unit = (rel - mb * jb.wgpm) * (kMmWaves / ks) + wave / ks;
    const int kp = wave % ks;                 // this wave's slice of the blocks
    const bool active = unit < jb.upm;
    const int nb = jb.nb;
    const int m = jb.m;
    const int bbeg = kp * jb.nbp;
    const int bend = min(nb, bbeg + jb.nbp);
    const int g0 = unit * kMmGroups;
    const int ng = active ? min(kMmGroups, jb.gpm - g0) : 0;
    const int gb = kMmGroupBlockBytes * nb;

    // the wave's groups (32 rows) through one bounded resource: groups past the
    // matrix read as zero, blocks past the slice are sent past the resource
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)wave_uniform(jb.w + mb * jb.w_bstride + (int64_t)g0 * gb), 0,
        wave_uniform(ng * gb), kBufferWord3);
    const int nl = lane & 31;          // weight row within the wave's 32
    const int hi = lane >> 5;          // code half
    const int q = nl >> 3, r = nl & 7;
    const int code0 = q * gb + 16 * nb + 32 * r + 16 * hi;    // + 256 per block
    const int scale0 = q * gb + 2 * r;                        // + 16 per block

    // two register buffers of kMmSlices blocks each: the next blocks stream in
    // while the current ones are computed
    v4i c0[kMmSlices], c1[kMmSlices];
    uint32_t s0[kMmSlices], s1[kMmSlices];
    auto issue = [&](v4i (&c)[kMmSlices], uint32_t (&sb)[kMmSlices], int b0) {
#pragma unroll
        for (int u = 0; u < kMmSlices; ++u) {
            // a block past the slice could land in the next group: send it past
            // the resource instead, so it reads zero
            const int b = b0 + u;
            const int off = b < bend ? code0 + 256 * b : 0x7ffffff0;
            c[u] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kCacheNT));
        }
#pragma unroll
        for (int u = 0; u < kMmSlices; ++u) {
            const int b = b0 + u;
            sb[u] = __builtin_amdgcn_raw_buffer_load_b16(rs, b < bend ? scale0 + 16 * b : 0x7ffffff0,
                                                         0, kCacheNT);
        }
    };

    // activation rows in LDS: codes [nb][MT][32 B], scales [nb][MT] fp32; one
    // thread per (block, token) loads the 34 bytes as 17 halves at once.  The
    // first round of these loads goes out before the weights, so its LDS writes
    // wait only for the rows (loads complete in issue order).
    extern __shared__ __align__(16) uint8_t mm_lds[];
    float *xd = (float *)(mm_lds + 32 * MT * nb);
    const uint8_t *x = jb.x + mb * jb.x_bstride;
    const int nblk = MT * nb;
    // the loads are unconditional (clamped to a valid block; a conditional
    // load would make the compiler wait for each one in turn), the values of
    // tokens past m are replaced by zeros afterwards
    auto load_blk = [&](int bt, uint32_t (&v)[17]) {
        const int bc = min(bt, nblk - 1);
        const int t = min(bc % MT, m - 1), b = bc / MT;
        const uint16_t *src = (const uint16_t *)(x + t * jb.x_rstride + b * kBlockBytes);
#pragma unroll
        for (int i = 0; i < 17; ++i) v[i] = (uint32_t)src[i];
    };
    auto store_blk = [&](int bt, const uint32_t (&v)[17]) {
        if (bt >= nblk) return;
        const uint32_t keep = bt % MT < m ? 0xffffffffu : 0u;
        u32x4 *dst = (u32x4 *)(mm_lds + 32 * bt);
        dst[0] = (u32x4){v[1] | (v[2] << 16), v[3] | (v[4] << 16), v[5] | (v[6] << 16),
                         v[7] | (v[8] << 16)} & keep;
        dst[1] = (u32x4){v[9] | (v[10] << 16), v[11] | (v[12] << 16), v[13] | (v[14] << 16),
                         v[15] | (v[16] << 16)} & keep;
        xd[bt] = half_bits_to_float(v[0] & keep);
    };
    {
        uint32_t v[17];
        load_blk(tid, v);
        // keep the rows' loads, then the weights, then the LDS writes in this order
        __builtin_amdgcn_sched_barrier(0);
        issue(c0, s0, bbeg);
        issue(c1, s1, bbeg + kMmSlices);
        __builtin_amdgcn_sched_barrier(0);
        store_blk(tid, v);
        for (int bt = tid + kMmThreads; bt < nblk; bt += kMmThreads) {
            load_blk(bt, v);
            store_blk(bt, v);
        }
    }
    __syncthreads();

    constexpr int kLive = MT / 2;           // result registers that hold tokens < MT
    float acc[kLive];
#pragma unroll
    for (int v = 0; v < kLive; ++v) acc[v] = 0.0f;
    const int ta = lane & 31;               // token of this lane's operand
    auto compute = [&](const v4i (&c)[kMmSlices], const uint32_t (&sb)[kMmSlices], int b0) {
#pragma unroll
        for (int u = 0; u < kMmSlices; ++u) {
            const int b = min(b0 + u, nb - 1);
            const v4i A = ta < MT ? *(const v4i *)(mm_lds + 32 * (MT * b + ta) + 16 * hi)
                                  : (v4i){0, 0, 0, 0};
            v16i s = {0};
            s = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, c[u], s, 0, 0, 0);
            if (SUMS && b0 + u < bend) {
                const int64_t row = (int64_t)g0 * 8 + nl;
#pragma unroll
                for (int v = 0; v < kLive; ++v) {
                    const int t = 8 * (v >> 2) + 4 * hi + (v & 3);
                    if (t < m && row < jb.n)
                        jb.sums[(((int64_t)mb * m + t) * jb.n + row) * nb + b] = s[v];
                }
            }
            const float dw = b0 + u < bend ? half_bits_to_float(sb[u]) : 0.0f;
            const float *dxb = xd + MT * b;
#pragma unroll
            for (int v = 0; v < kLive; ++v) {
                const int t = 8 * (v >> 2) + 4 * hi + (v & 3);
                acc[v] = fmaf(dw * dxb[t], (float)s[v], acc[v]);
            }
        }
    };
    if (active) {
        for (int b0 = bbeg;;) {
            compute(c0, s0, b0);
            if (b0 + kMmSlices >= bend) break;
            if (b0 + 2 * kMmSlices < bend) issue(c0, s0, b0 + 2 * kMmSlices);
            compute(c1, s1, b0 + kMmSlices);
            b0 += 2 * kMmSlices;
            if (b0 >= bend) break;
            if (b0 + kMmSlices < bend) issue(c1, s1, b0 + kMmSlices);
        }
    }
    // the ks slices of a unit are added in slice order by its first wave
    float *red = (float *)(mm_lds + 36 * MT * nb);
    if (ks > 1) {
#pragma unroll
        for (int v = 0; v < kLive; ++v) red[(wave * kLive + v) * kWave + lane] = acc[v];
        __syncthreads();
        if (kp != 0) return;
#pragma unroll
        for (int v = 0; v < kLive; ++v) {
            float sum = red[(wave * kLive + v) * kWave + lane];
            for (int p = 1; p < ks; ++p) sum += red[((wave + p) * kLive + v) * kWave + lane];
            acc[v] = sum;
        }
    }
    if (!active) return;
    const int64_t row = (int64_t)g0 * 8 + nl;
    if (row < jb.n) {
        float *y = jb.y + mb * jb.y_bstride + row;
#pragma unroll
        for (int v = 0; v < kLive; ++v) {
            const int t = 8 * (v >> 2) + 4 * hi + (v & 3);
            if (t < m) y[t * jb.y_rstride] = acc[v];
        }
    }
}

size_t mm_lds_bytes(int mt, int64_t nb) { return (size_t)36 * mt * nb + (size_t)kMmWaves * kWave * (mt / 2) * 4; }

template <int MT, bool SUMS>
int launch_mt(const MmArgs &a, unsigned grid, size_t lds, hipStream_t stream)
{
    if (lds > 65536) {
        static bool attr_set = false;
        if (!attr_set) {
            if (hipFuncSetAttribute((const void *)r8_mm_kernel<MT, SUMS>,
                                    hipFuncAttributeMaxDynamicSharedMemorySize,
                                    max_lds_bytes()) != hipSuccess)
                return -6;
            attr_set = true;
        }
    }
    hipLaunchKernelGGL((r8_mm_kernel<MT, SUMS>), dim3(grid), dim3(kMmThreads), lds, stream, a);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // namespace

// Waves per unit: long rows are split over 2 or 4 waves of the workgroup so
// that no wave walks more than about 24 blocks in sequence.
#ifndef Q8_R8MM_SPLIT
#define Q8_R8MM_SPLIT 32
#endif
static int mm_split(int64_t nb) { return nb >= 2 * Q8_R8MM_SPLIT ? 4 : nb >= Q8_R8MM_SPLIT ? 2 : 1; }

bool r8_mm_ok(int64_t n, int64_t nb, int64_t m, int64_t batch)
{
    if (m < 1 || m > 16) return false;
    const int mt = m <= 8 ? 8 : 16;
    if (mm_lds_bytes(mt, nb) > (size_t)max_lds_bytes()) return false;
    if ((int64_t)kMmGroupBlockBytes * nb * kMmGroups > 0x7fffffffLL) return false;
    const int64_t gpm = (n + 7) / 8;
    const int64_t upm = (gpm + kMmGroups - 1) / kMmGroups;
    const int64_t upw = kMmWaves / mm_split(nb);
    return (upm + upw - 1) / upw * batch < 0x7fffffffLL;
}

int launch_r8_mm(const R8MmDesc *d, int n_desc, hipStream_t stream)
{
    MmArgs a;
    memset(&a, 0, sizeof(a));
    int64_t wg = 0;
    int64_t nb_max = 1;
    int m_max = 1;
    int nj = 0;
    bool sums = false;
    for (int i = 0; i < n_desc; ++i) {
        if (d[i].n == 0 || d[i].m == 0 || d[i].batch == 0) continue;
        MmJob &j = a.job[nj++];
        j.w = d[i].w; j.x = d[i].x; j.y = d[i].y;
        j.w_bstride = d[i].w_bstride; j.x_rstride = d[i].x_rstride; j.x_bstride = d[i].x_bstride;
        j.y_rstride = d[i].y_rstride; j.y_bstride = d[i].y_bstride;
        j.sums = d[i].sums;
        if (d[i].sums) sums = true;
        j.n = d[i].n;
        j.nb = (int)d[i].nb;
        j.m = (int)d[i].m;
        j.gpm = (int)((d[i].n + 7) / 8);
        j.upm = (j.gpm + kMmGroups - 1) / kMmGroups;
        j.ks = mm_split(d[i].nb);
        j.nbp = (j.nb + j.ks - 1) / j.ks;
        const int upw = kMmWaves / j.ks;
        j.wgpm = (j.upm + upw - 1) / upw;
        j.wg0 = (int)wg;
        wg += (int64_t)j.wgpm * d[i].batch;
        if (wg > 0x7fffffffLL) return -4;
        nb_max = d[i].nb > nb_max ? d[i].nb : nb_max;
        m_max = j.m > m_max ? j.m : m_max;
    }
    if (nj == 0) return 0;
    a.n_jobs = nj;
    if (sums)
        return m_max <= 8 ? launch_mt<8, true>(a, (unsigned)wg, mm_lds_bytes(8, nb_max), stream)
                          : launch_mt<16, true>(a, (unsigned)wg, mm_lds_bytes(16, nb_max), stream);
    if (m_max <= 8) return launch_mt<8, false>(a, (unsigned)wg, mm_lds_bytes(8, nb_max), stream);
    return launch_mt<16, false>(a, (unsigned)wg, mm_lds_bytes(16, nb_max), stream);
}

}  // namespace q8
