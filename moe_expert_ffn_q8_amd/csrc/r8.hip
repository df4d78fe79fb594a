// r8.hip -- the row-interleaved weight layout (R8) and its decode product.
//
// The Gemma-4-on-Xeon page ("GPUなしで13年前のXeon上でGemma 4 26Bを毎秒5トークン
// で実行する", section on the fallback's cost and the repacking bug) describes an
// option that reorders the quantized weights once, at startup, into an
// interleaved form named Q8_0_R8, made for one CPU instruction set.  It prints
// no layout.  This file's layout keeps the idea -- 8 rows interleaved, built
// once at load time -- and lays the bytes out for 64-wide wavefronts:
//
//   group g = rows 8g .. 8g+7 (the last group padded with zero rows),
//   272*nb bytes at g*272*nb:
//     [0, 16*nb)         binary16 scales, index 8*b + r   (block b, row r)
//     [16*nb, 272*nb)    codes, 32 bytes at 16*nb + 32*(8*b + r)
//
// Same bytes as the native rows, moved: the scales leave the code stream, and
// every 16-byte chunk holds codes of one row and one block.  A wave then reads
// a group as contiguous 1 KB slices: slice i, lane l covers row (l>>1)&7,
// block 4i + (l>>4), half l&1 of that block's codes, and its scale sits at
// 64*i + 2*(l>>1) -- no masked activation image and no per-row tails (a group
// is always 8 whole rows).
//
// Arithmetic per (row, block): the exact int32 sum of the 32 code products
// (two lanes of 16 codes each, joined by a lane swap), then (d_w*d_x)*s in
// fp32; a lane accumulates its blocks in ascending order, the four lanes of a
// row are then added in a fixed tree.
#include <string.h>

#include "q8_device.h"
#include "q8_internal.h"

namespace q8 {

namespace {

constexpr int kR8Rows = 8;
constexpr int kR8GroupBlockBytes = kR8Rows * kBlockBytes;   // 272 per block column
#ifndef Q8_R8_WAVES
#define Q8_R8_WAVES 4
#endif
constexpr int kR8Waves = Q8_R8_WAVES;                       // one group per wave
constexpr int kR8Threads = kR8Waves * kWave;
constexpr int kR8QBlocks = kR8Threads / 8;                  // blocks quantized per pass
#ifndef Q8_R8_SLICES
#define Q8_R8_SLICES 8
#endif
constexpr int kR8Slices = Q8_R8_SLICES;   // 1 KB slices of a group in flight per wave
constexpr int kR8QuickNb = 64;                              // rows staged from registers
constexpr int kR8QuickLoads = 16 * kR8QuickNb / kR8Threads;  // 2-byte loads per thread

// One descriptor of a launch: `batch` matrices of n rows of nb blocks in the
// R8 layout, each with its own activation row and output vector.  Workgroups
// are numbered across descriptors: a matrix takes wgpm consecutive workgroups
// of 4 groups each.
struct R8Job {
    const uint8_t *w;
    const uint8_t *x;      // Q8_0 row of matrix 0
    float *y;
    int64_t w_bstride;     // bytes between matrices
    int64_t x_bstride;     // bytes between activation rows
    int64_t y_bstride;     // floats between output vectors
    int32_t *sums;         // validation: int32 [batch][n][nb] block sums (SUMS kernels only)
    int64_t n;
    int nb;
    int gpm;               // groups per matrix
    int wgpm;              // workgroups per matrix
    int wg0;               // first workgroup of the descriptor
};

struct R8Args {
    R8Job job[kStreamMaxJobs];
    int n_jobs;
};

// One thread per (group, row, block), block fastest: reads one native block
// (2-byte aligned) and writes its scale and its two 16-byte code chunks.
__global__ __launch_bounds__(256) void r8_repack_kernel(const uint8_t *__restrict__ w,
                                                        uint8_t *__restrict__ out, int64_t n,
                                                        int64_t nb, int64_t units)
{
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= units) return;
    const int64_t b = t % nb;
    const int64_t gr = t / nb;
    const int r = (int)(gr & (kR8Rows - 1));
    const int64_t g = gr / kR8Rows;
    const int64_t row = g * kR8Rows + r;
    uint32_t sc = 0;
    uint32_t c[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (row < n) {
        const uint16_t *src = (const uint16_t *)(w + (row * nb + b) * kBlockBytes);
        sc = src[0];
#pragma unroll
        for (int i = 0; i < 8; ++i) c[i] = (uint32_t)src[1 + 2 * i] | ((uint32_t)src[2 + 2 * i] << 16);
    }
    uint8_t *gp = out + g * kR8GroupBlockBytes * nb;
    *(uint16_t *)(gp + 2 * (b * kR8Rows + r)) = (uint16_t)sc;
    u32x4 *dst = (u32x4 *)(gp + 16 * nb + 32 * (b * kR8Rows + r));
    dst[0] = (u32x4){c[0], c[1], c[2], c[3]};
    dst[1] = (u32x4){c[4], c[5], c[6], c[7]};
}

// XF: the activation rows are fp32 and every workgroup quantizes its row
// into LDS itself (the bytes of q8_0_quantize_rows), so a decode step needs no
// separate quantization launch.  SUMS (validation builds of the same kernel):
// every exact int32 block sum is also written out.
#ifndef Q8_R8_OCC
#define Q8_R8_OCC 1
#endif
template <bool XF, bool SUMS>
__global__ __launch_bounds__(kR8Threads, Q8_R8_OCC) void r8_matvec_kernel(const R8Args a)
{
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    int j = 0;
    while (j + 1 < a.n_jobs && (int)blockIdx.x >= a.job[j + 1].wg0) ++j;
    const R8Job &jb = a.job[j];
    const int rel = (int)blockIdx.x - jb.wg0;
    const int mb = rel / jb.wgpm;
    const int g = (rel - mb * jb.wgpm) * kR8Waves + wave;
    const bool active = g < jb.gpm;          // the last workgroup of a matrix may hold idle waves
    const int nb = jb.nb;

    // buffer resource bounded to the group: slices past its end read as zero
    const int gbytes = kR8GroupBlockBytes * nb;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)wave_uniform(jb.w + mb * jb.w_bstride + (int64_t)g * gbytes), 0,
        wave_uniform(active ? gbytes : 0), kBufferWord3);
    const int half = lane & 1;
    const int bs = lane >> 4;
    const int code0 = 16 * nb + 16 * lane;     // + 1024 per slice
    const int scale0 = 2 * (lane >> 1);        // + 64 per slice
    const int slices = (nb + 3) >> 2;

    u32x4 c[kR8Slices];
    uint32_t sb[kR8Slices];
    auto issue = [&](int i0) {
#pragma unroll
        for (int u = 0; u < kR8Slices; ++u)
            c[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, code0 + 1024 * (i0 + u), 0, kCacheNT);
#pragma unroll
        for (int u = 0; u < kR8Slices; ++u)
            sb[u] = __builtin_amdgcn_raw_buffer_load_b16(rs, scale0 + 64 * (i0 + u), 0, kCacheNT);
    };
    // The activation row goes to LDS: codes realigned to 32 bytes per block,
    // then the binary16 scale bits.  Up to 64 blocks (k <= 2048) every thread
    // loads its share into registers first and the group's first slices are
    // issued behind those loads, so that the LDS writes wait for the row only
    // (loads complete in issue order) while the weights are in flight.
    extern __shared__ __align__(16) uint8_t r8_lds[];
    uint8_t *xc = r8_lds;
    uint16_t *xc16 = (uint16_t *)xc;
    uint16_t *xd16 = (uint16_t *)(r8_lds + 32 * nb);
    const uint8_t *x = jb.x + mb * jb.x_bstride;
    const int tid = threadIdx.x;
    if (XF) {
        // 8 lanes per 32-value block, 4 values each; kR8QBlocks blocks per pass
        const float *xf = (const float *)x;
        const int li = tid & 7;
        const int passes = (nb + kR8QBlocks - 1) / kR8QBlocks;
        auto quantize_pass = [&](int p, float4 v) {
            const int b = (tid >> 3) + kR8QBlocks * p;
            uint32_t codes, dbits;
            quantize_block8(v.x, v.y, v.z, v.w, codes, dbits);
            if (b < nb) {
                *(uint32_t *)(xc + 32 * b + 4 * li) = codes;
                if (li == 0) xd16[b] = (uint16_t)dbits;
            }
        };
        auto load_pass = [&](int p) {
            const int b = min((tid >> 3) + kR8QBlocks * p, nb - 1);
            return *(const float4 *)(xf + 32 * b + 4 * li);
        };
        if (passes <= 2) {
            const float4 v0 = load_pass(0);
            const float4 v1 = load_pass(passes > 1 ? 1 : 0);
            __builtin_amdgcn_sched_barrier(0);
            issue(0);
            __builtin_amdgcn_sched_barrier(0);
            quantize_pass(0, v0);
            if (passes > 1) quantize_pass(1, v1);
        } else {
            for (int p = 0; p < passes; ++p) quantize_pass(p, load_pass(p));
            issue(0);
        }
    } else if (nb <= kR8QuickNb) {
        uint32_t xv[kR8QuickLoads];
#pragma unroll
        for (int u = 0; u < kR8QuickLoads; ++u) {
            const int e = min(tid + kR8Threads * u, 16 * nb - 1);
            xv[u] = load_u16(x + (e >> 4) * kBlockBytes + 2 + 2 * (e & 15));
        }
        const uint32_t xs = load_u16(x + min(tid, nb - 1) * kBlockBytes);
        // keep the row's loads, then the weights, then the LDS writes in this order
        __builtin_amdgcn_sched_barrier(0);
        issue(0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kR8QuickLoads; ++u) {
            const int e = tid + kR8Threads * u;
            if (e < 16 * nb) xc16[e] = (uint16_t)xv[u];
        }
        if (tid < nb) xd16[tid] = (uint16_t)xs;
    } else {
        for (int e = tid; e < 16 * nb; e += kR8Threads)
            xc16[e] = *(const uint16_t *)(x + (e >> 4) * kBlockBytes + 2 + 2 * (e & 15));
        for (int b = tid; b < nb; b += kR8Threads)
            xd16[b] = *(const uint16_t *)(x + b * kBlockBytes);
        issue(0);
    }
    __syncthreads();
    if (!active) return;

    float acc = 0.0f;
    for (int i0 = 0;;) {
        // every slice of the pass is computed (a branch here would make the
        // compiler wait for each load in turn): slices past the group read as
        // zero codes and their scales are masked, so they add exact zeros
#pragma unroll
        for (int u = 0; u < kR8Slices; ++u) {
            const int b = 4 * (i0 + u) + bs;
            const bool live = b < nb;
            const int bb = live ? b : nb - 1;
            const u32x4 xv = *(const u32x4 *)(xc + 32 * bb + 16 * half);
            int s = sdot4(c[u].x, xv.x, 0);
            s = sdot4(c[u].y, xv.y, s);
            s = sdot4(c[u].z, xv.z, s);
            s = sdot4(c[u].w, xv.w, s);
            // the other half of the block from the neighbouring lane (quad_perm 1,0,3,2)
            s += __builtin_amdgcn_mov_dpp(s, 0xB1, 0xF, 0xF, false);
            if (SUMS && half == 0 && live) {
                const int64_t row = (int64_t)g * kR8Rows + ((lane >> 1) & 7);
                if (row < jb.n) jb.sums[((int64_t)mb * jb.n + row) * nb + b] = s;
            }
            const float dw = live ? half_bits_to_float(sb[u]) : 0.0f;
            acc = fmaf(dw * half_bits_to_float(xd16[bb]), (float)s, acc);
        }
        i0 += kR8Slices;
        if (i0 >= slices) break;
        issue(i0);
    }
    // the four lanes of a row (block residues 0..3), fixed order
    acc += __shfl_xor(acc, 16);
    acc += __shfl_xor(acc, 32);
    if ((lane & 0x31) == 0) {
        const int64_t row = (int64_t)g * kR8Rows + ((lane >> 1) & 7);
        if (row < jb.n) jb.y[mb * jb.y_bstride + row] = acc;
    }
}

}  // namespace

int64_t r8_bytes(int64_t n, int64_t nb)
{
    return (n + kR8Rows - 1) / kR8Rows * kR8GroupBlockBytes * nb;
}

int launch_r8_repack(const uint8_t *w, uint8_t *out, int64_t n, int64_t nb, hipStream_t stream)
{
    const int64_t units = (n + kR8Rows - 1) / kR8Rows * kR8Rows * nb;
    const int64_t grid = (units + 255) / 256;
    if (grid > 0x7fffffff) return -4;
    hipLaunchKernelGGL(r8_repack_kernel, dim3((unsigned)grid), dim3(256), 0, stream, w, out, n,
                       nb, units);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

bool r8_matvec_ok(int64_t n, int64_t nb, int64_t batch)
{
    // group offsets inside the buffer resource are 32-bit; the activation row
    // is staged in LDS (34 bytes per block); workgroup numbers are 32-bit
    const int64_t gpm = (n + kR8Rows - 1) / kR8Rows;
    return nb <= kR8MaxNb && (gpm + kR8Waves - 1) / kR8Waves * batch < 0x7fffffffLL;
}

int launch_r8_matvec(const R8Desc *d, int n_desc, bool x_f32, hipStream_t stream)
{
    R8Args a;
    memset(&a, 0, sizeof(a));
    int64_t wg = 0;
    int nb_max = 1;
    int nj = 0;
    bool sums = false;
    // Descriptors with the longest rows (most blocks per group) get the first
    // workgroups, the rest keep their order: workgroups start in launch order,
    // so the long groups no longer start last and set the tail of the launch
    // (Llama-110M-shaped step, the k = 2048 products moved to the front:
    // 19.55-19.60 against 19.90 us).  Outputs do not depend on the order.
    int order[kStreamMaxJobs];
    int live = 0;
    for (int i = 0; i < n_desc; ++i) {
        if (d[i].n == 0 || d[i].batch == 0) continue;
        int p = live++;
        for (; p > 0 && d[order[p - 1]].nb < d[i].nb; --p) order[p] = order[p - 1];
        order[p] = i;
    }
    for (int oi = 0; oi < live; ++oi) {
        const int i = order[oi];
        R8Job &j = a.job[nj++];
        j.w = d[i].w; j.x = d[i].x; j.y = d[i].y;
        j.w_bstride = d[i].w_bstride; j.x_bstride = d[i].x_bstride; j.y_bstride = d[i].y_bstride;
        j.sums = d[i].sums;
        if (d[i].sums) sums = true;
        j.n = d[i].n;
        j.nb = (int)d[i].nb;
        j.gpm = (int)((d[i].n + kR8Rows - 1) / kR8Rows);
        j.wgpm = (j.gpm + kR8Waves - 1) / kR8Waves;
        j.wg0 = (int)wg;
        wg += (int64_t)j.wgpm * d[i].batch;
        if (wg > 0x7fffffffLL) return -4;
        nb_max = j.nb > nb_max ? j.nb : nb_max;
    }
    if (nj == 0) return 0;
    a.n_jobs = nj;
    const size_t lds = (size_t)34 * nb_max;
    if (sums) {
        if (x_f32)
            hipLaunchKernelGGL((r8_matvec_kernel<true, true>), dim3((unsigned)wg), dim3(kR8Threads),
                               lds, stream, a);
        else
            hipLaunchKernelGGL((r8_matvec_kernel<false, true>), dim3((unsigned)wg), dim3(kR8Threads),
                               lds, stream, a);
    } else if (x_f32) {
        hipLaunchKernelGGL((r8_matvec_kernel<true, false>), dim3((unsigned)wg), dim3(kR8Threads),
                           lds, stream, a);
    } else {
        hipLaunchKernelGGL((r8_matvec_kernel<false, false>), dim3((unsigned)wg), dim3(kR8Threads),
                           lds, stream, a);
    }
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // namespace q8
