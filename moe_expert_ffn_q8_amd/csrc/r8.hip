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
#include "q8_device.h"
#include "q8_internal.h"

namespace q8 {

namespace {

constexpr int kR8Rows = 8;
constexpr int kR8GroupBlockBytes = kR8Rows * kBlockBytes;   // 272 per block column
constexpr int kR8Threads = 256;
constexpr int kR8Waves = kR8Threads / kWave;                // one group per wave
#ifndef Q8_R8_SLICES
#define Q8_R8_SLICES 8
#endif
constexpr int kR8Slices = Q8_R8_SLICES;   // 1 KB slices of a group in flight per wave

struct R8Args {
    const uint8_t *w;    // R8 layout
    const uint8_t *x;    // one Q8_0 row [nb] blocks
    float *y;            // [n]
    int64_t n;
    int nb;
    int64_t groups;
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

__global__ __launch_bounds__(kR8Threads) void r8_matvec_kernel(const R8Args a)
{
    // the activation row, codes realigned to 32 bytes per block, scales as fp32
    extern __shared__ __align__(16) uint8_t r8_lds[];
    const int nb = a.nb;
    uint8_t *xc = r8_lds;
    float *xd = (float *)(r8_lds + 32 * nb);
    {
        uint16_t *xc16 = (uint16_t *)xc;
        for (int e = threadIdx.x; e < 16 * nb; e += kR8Threads) {
            const int b = e >> 4, p = e & 15;
            xc16[16 * b + p] = *(const uint16_t *)(a.x + b * kBlockBytes + 2 + 2 * p);
        }
        for (int b = threadIdx.x; b < nb; b += kR8Threads)
            xd[b] = half_bits_to_float(load_u16(a.x + b * kBlockBytes));
    }
    __syncthreads();

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int64_t g = (int64_t)blockIdx.x * kR8Waves + wave;
    if (g >= a.groups) return;

    // buffer resource bounded to the group: slices past its end read as zero
    const int gbytes = kR8GroupBlockBytes * nb;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)wave_uniform(a.w + g * gbytes), 0, gbytes, kBufferWord3);
    const int half = lane & 1;
    const int bs = lane >> 4;
    const int code0 = 16 * nb + 16 * lane;     // + 1024 per slice
    const int scale0 = 2 * (lane >> 1);        // + 64 per slice
    const int slices = (nb + 3) >> 2;

    float acc = 0.0f;
    for (int i0 = 0; i0 < slices; i0 += kR8Slices) {
        u32x4 c[kR8Slices];
        uint32_t sb[kR8Slices];
#pragma unroll
        for (int u = 0; u < kR8Slices; ++u)
            c[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, code0 + 1024 * (i0 + u), 0, kCacheNT);
#pragma unroll
        for (int u = 0; u < kR8Slices; ++u)
            sb[u] = __builtin_amdgcn_raw_buffer_load_b16(rs, scale0 + 64 * (i0 + u), 0, kCacheNT);
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
            const float dw = live ? half_bits_to_float(sb[u]) : 0.0f;
            acc = fmaf(dw * xd[bb], (float)s, acc);
        }
    }
    // the four lanes of a row (block residues 0..3), fixed order
    acc += __shfl_xor(acc, 16);
    acc += __shfl_xor(acc, 32);
    if ((lane & 0x31) == 0) {
        const int64_t row = g * kR8Rows + ((lane >> 1) & 7);
        if (row < a.n) a.y[row] = acc;
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

bool r8_matvec_ok(int64_t n, int64_t nb)
{
    // group offsets inside the buffer resource are 32-bit; the activation row
    // is staged in LDS (36 bytes per block)
    return nb <= kR8MaxNb && (int64_t)kR8GroupBlockBytes * nb < 0x7fffffffLL &&
           (n + kR8Rows - 1) / kR8Rows / kR8Waves < 0x7fffffffLL;
}

int launch_r8_matvec(const uint8_t *w_r8, const uint8_t *x, float *y, int64_t n, int64_t nb,
                     hipStream_t stream)
{
    R8Args a;
    a.w = w_r8; a.x = x; a.y = y; a.n = n; a.nb = (int)nb;
    a.groups = (n + kR8Rows - 1) / kR8Rows;
    const int64_t grid = (a.groups + kR8Waves - 1) / kR8Waves;
    const size_t lds = (size_t)36 * nb;
    hipLaunchKernelGGL(r8_matvec_kernel, dim3((unsigned)grid), dim3(kR8Threads), lds, stream, a);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // namespace q8
