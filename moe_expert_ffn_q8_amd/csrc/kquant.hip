// kquant.hip -- Q8_1 activations and the decode product over 4/5-bit K-quant
// weights (Q4_K, Q5_K) on gfx950.
//
// The Gemma-4-on-Xeon page ("GPUなしで13年前のXeon上でGemma 4 26Bを毎秒5トークン
// で実行する", three-part fix, compile-fix part) names a Q8_1 activation
// quantizer beside the Q8_0 one, and the other pages serve Q4_K_M / Q5_K_M
// model files (the Nemotron review's closing section; the ARM page's server
// commands).  No page prints a layout; the layouts read here:
//
//   Q8_1 block, 36 bytes: binary16 d, binary16 s, 32 int8 codes; d and codes
//     by the Q8_0 rule, s = binary16(d32 * sum of codes) with d32 = amax/127.
//   Super-block of 256 values = 8 sub-blocks of 32:
//     Q4_K, 144 bytes: binary16 d, binary16 dmin, 12 bytes of packed 6-bit
//       sub-block scales sc[8] and mins m[8], 128 bytes of 4-bit codes;
//     Q5_K, 176 bytes: the same header, 32 bytes of high bits, 128 bytes of
//       low 4-bit codes.
//   Value l of sub-block j = d*sc[j]*q - dmin*m[j].
//
// Product per sub-block j against Q8_1 block (dx, codes qx): the exact int32
// sums S = sum q*qx (v_dot4: the 4- or 5-bit codes are small non-negative
// bytes) and Q = sum qx, then (d*sc*dx)*S - (dmin*m*dx)*Q in fp32; the stored
// s is not used, so no binary16 rounding of the code sum enters the result.
//
// Work decomposition: a wave-tile is R = 64/S whole rows of S super-blocks
// (S = k/256), one super-block per lane.  Q4_K: the lane loads its super-block
// itself (9 16-byte buffer loads, a 144-byte stride across the wave, every
// byte of the tile used).  Q5_K: the tile arrives with 1 KB coalesced loads,
// goes to the wave's LDS slot in load order and is read back one super-block
// per lane.  Measured on 262144 x 2048: Q4_K 46.1 us direct against 50.0 us
// through LDS, Q5_K 57.8 us through LDS against 60.7 us direct.  The activation row is staged once per workgroup,
// one thread per block (codes realigned to 32 bytes per block, fp32 scales,
// code sums).  The S partial sums of a row are added in a fixed order.
#include <string.h>

#include "q8_device.h"
#include "q8_internal.h"

namespace q8 {

namespace {

constexpr int kQ81Bytes = 36;
// Q4_K tiles are loaded by their lanes directly, Q5_K tiles go through an LDS
// slot per wave (the faster form of each, measured)
template <int T> constexpr bool kq_direct() { return T == 4; }
constexpr int kKqThreads = 256;
constexpr int kKqWaves = kKqThreads / kWave;

template <int T> struct KqFmt;
template <> struct KqFmt<4> { static constexpr int kBytes = 144, kQs = 16; };
template <> struct KqFmt<5> { static constexpr int kBytes = 176, kQs = 48; };

// 8 lanes per block (4 values each): Q8_1 block bytes of one 32-value block.
__global__ __launch_bounds__(256) void q8_1_quantize_kernel(const float *__restrict__ x,
                                                            int64_t row_stride,
                                                            uint8_t *__restrict__ y, int64_t nb,
                                                            int64_t total_blocks)
{
    const int tid = threadIdx.x;
    const int li = tid & 7;
    for (int64_t g = ((int64_t)blockIdx.x * 256 + tid) >> 3; g < total_blocks;
         g += ((int64_t)gridDim.x * 256) >> 3) {
        const int64_t r = g / nb;
        const int64_t b = g - r * nb;
        const float4 v = *(const float4 *)(x + r * row_stride + b * kQK + 4 * li);
        uint32_t codes, dbits;
        quantize_block8(v.x, v.y, v.z, v.w, codes, dbits);
        float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
        a = fmaxf(a, __shfl_xor(a, 1));
        a = fmaxf(a, __shfl_xor(a, 2));
        a = fmaxf(a, __shfl_xor(a, 4));
        const float d32 = a / 127.0f;
        int sum = sdot4(codes, 0x01010101u, 0);
        sum += __shfl_xor(sum, 1);
        sum += __shfl_xor(sum, 2);
        sum += __shfl_xor(sum, 4);
        // the product rounds to fp32 first, then to binary16: the empty asm
        // keeps the fp32 value in a register, so the compiler cannot fuse the
        // multiply and the conversion into one rounding (v_fma_mix), which
        // differs where the fp32 product sits on a binary16 rounding boundary
        float sprod = d32 * (float)sum;
        asm volatile("" : "+v"(sprod));
        const uint32_t sbits = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)sprod);
        uint32_t *out = (uint32_t *)(y + g * kQ81Bytes);
        if (li == 0) out[0] = (dbits & 0xffffu) | (sbits << 16);
        out[1 + li] = codes;
    }
}

struct KqJob {
    const uint8_t *w;      // super-blocks of matrix 0
    const uint8_t *x;      // Q8_1 row of matrix 0 (4-byte aligned)
    float *y;
    int64_t w_bstride;     // bytes between matrices
    int64_t x_bstride;     // bytes between activation rows
    int64_t y_bstride;     // floats between output vectors
    int64_t n;
    int S;                 // super-blocks per row
    int R;                 // rows per wave-tile
    int tiles;             // wave-tiles per matrix
    int wgpm;              // workgroups per matrix
    int wg0;
};

struct KqArgs {
    KqJob job[kStreamMaxJobs];
    int n_jobs;
};

template <int T>
__global__ __launch_bounds__(kKqThreads) void kq_matvec_kernel(const KqArgs a)
{
    constexpr int BB = KqFmt<T>::kBytes;
    constexpr int kSlot = kWave * BB;                 // one wave's tile, bytes
    constexpr int kChunks = kSlot / 16;               // 576 or 704
    constexpr int kLoads = (kChunks + kWave - 1) / kWave;
    constexpr int kDw = BB / 4;                       // dwords per super-block

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int tid = threadIdx.x;
    int j = 0;
    while (j + 1 < a.n_jobs && (int)blockIdx.x >= a.job[j + 1].wg0) ++j;
    const KqJob &jb = a.job[j];
    const int rel = (int)blockIdx.x - jb.wg0;
    const int mb = rel / jb.wgpm;
    const int t = (rel - mb * jb.wgpm) * kKqWaves + wave;
    const bool active = t < jb.tiles;
    const int S = jb.S;
    const int nb = 8 * S;
    const int64_t row0 = (int64_t)t * jb.R;
    const int rows = active ? (int)min((int64_t)jb.R, jb.n - row0) : 0;

    // the tile's loads first (bounded to the tile: chunks past it read zero)
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)wave_uniform(jb.w + mb * jb.w_bstride + row0 * S * BB), 0,
        wave_uniform(rows * S * BB), kBufferWord3);
    const int lr = lane / S;            // this lane's super-block: row lane / S, column lane % S
    const int s0 = lane - lr * S;
    const bool live = lr < rows;
    uint32_t q[kDw];
    u32x4 g[kLoads];
    if constexpr (kq_direct<T>()) {
        // each lane loads its own super-block (16-byte pieces 144 bytes apart
        // across the wave; lanes past the tile read zeros)
#pragma unroll
        for (int v = 0; v < kDw / 4; ++v) {
            const u32x4 c = __builtin_amdgcn_raw_buffer_load_b128(rs, BB * lane + 16 * v, 0, 0);
            q[4 * v] = c.x; q[4 * v + 1] = c.y; q[4 * v + 2] = c.z; q[4 * v + 3] = c.w;
        }
    } else {
#pragma unroll
        for (int u = 0; u < kLoads; ++u)
            g[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * (u * kWave + lane), 0, kCacheNT);
    }

    // LDS: [4 wave slots] | activation codes (32 B per block) | dx | code sums | row partials
    extern __shared__ __align__(16) uint8_t kq_lds[];
    uint8_t *slot = kq_lds + wave * kSlot;
    uint32_t *xc = (uint32_t *)(kq_lds + (kq_direct<T>() ? 0 : kKqWaves * kSlot));
    float *xd = (float *)(xc + 8 * nb);
    int *xq = (int *)(xd + nb);
    float *red = (float *)(xq + nb) + wave * kWave;

    // one thread per activation block (nb <= 256): codes, scale and code sum
    const uint32_t *x32 = (const uint32_t *)(jb.x + mb * jb.x_bstride);
    if (tid < nb) {
        uint32_t v[9];
#pragma unroll
        for (int p = 0; p < 9; ++p) v[p] = x32[9 * tid + p];
        int qs = 0;
#pragma unroll
        for (int p = 0; p < 8; ++p) qs = sdot4(v[1 + p], 0x01010101u, qs);
        u32x4 *dst = (u32x4 *)(xc + 8 * tid);
        dst[0] = (u32x4){v[1], v[2], v[3], v[4]};
        dst[1] = (u32x4){v[5], v[6], v[7], v[8]};
        xd[tid] = half_bits_to_float(v[0]);
        xq[tid] = qs;
    }
    if constexpr (!kq_direct<T>()) {
#pragma unroll
        for (int u = 0; u < kLoads; ++u) {
            const int i = u * kWave + lane;
            if (i < kChunks) ((u32x4 *)slot)[i] = g[u];
        }
    }
    __syncthreads();
    if (!active) return;

    if constexpr (!kq_direct<T>()) {
        const u32x4 *src = (const u32x4 *)(slot + BB * (live ? lane : 0));
#pragma unroll
        for (int v = 0; v < kDw / 4; ++v) {
            const u32x4 c = src[v];
            q[4 * v] = c.x; q[4 * v + 1] = c.y; q[4 * v + 2] = c.z; q[4 * v + 3] = c.w;
        }
    }
    const float d = half_bits_to_float(q[0]);
    const float dmin = half_bits_to_float(q[0] >> 16);
    // the 12 scale bytes are dwords 1..3
    uint32_t sc8[8], m8[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
        if (jj < 4) {
            sc8[jj] = (q[1] >> (8 * jj)) & 63u;
            m8[jj] = (q[2] >> (8 * jj)) & 63u;
        } else {
            const uint32_t bj = (q[3] >> (8 * (jj - 4))) & 0xffu;   // byte j+4
            const uint32_t lo = (q[1] >> (8 * (jj - 4))) & 0xffu;   // byte j-4
            const uint32_t hi = (q[2] >> (8 * (jj - 4))) & 0xffu;   // byte j
            sc8[jj] = (bj & 15u) | ((lo >> 6) << 4);
            m8[jj] = (bj >> 4) | ((hi >> 6) << 4);
        }
    }
    float acc = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int jj = 2 * c + h;
            const int xb = 8 * s0 + jj;
            const u32x4 *xv4 = (const u32x4 *)(xc + 8 * xb);
            const u32x4 xa = xv4[0], xbv = xv4[1];
            const uint32_t xw[8] = {xa.x, xa.y, xa.z, xa.w, xbv.x, xbv.y, xbv.z, xbv.w};
            int s = 0;
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                const uint32_t w = q[KqFmt<T>::kQs / 4 + 8 * c + p];
                uint32_t nib = h ? (w >> 4) & 0x0f0f0f0fu : w & 0x0f0f0f0fu;
                if (T == 5) nib |= ((q[4 + p] >> jj) & 0x01010101u) << 4;
                s = sdot4(nib, xw[p], s);
            }
            const float dx = xd[xb];
            acc = fmaf((d * (float)sc8[jj]) * dx, (float)s, acc);
            acc = fmaf(-((dmin * (float)m8[jj]) * dx), (float)xq[xb], acc);
        }
    }
    // the S partials of a row, in column order
    red[lane] = live ? acc : 0.0f;
    wave_lds_sync();
    if (lane < rows) {
        float y = 0.0f;
        for (int s = 0; s < S; ++s) y += red[lane * S + s];
        jb.y[mb * jb.y_bstride + row0 + lane] = y;
    }
}

}  // namespace

int launch_q8_1_quantize_rows(const float *x, int64_t row_stride, void *y, int64_t n_rows,
                              int64_t k, hipStream_t stream)
{
    const int64_t nb = k / kQK;
    const int64_t total = n_rows * nb;
    if (total == 0) return 0;
    const int64_t wgs = (total * 8 + 255) / 256;
    const unsigned grid = (unsigned)(wgs < 256 * 64 ? wgs : 256 * 64);
    hipLaunchKernelGGL(q8_1_quantize_kernel, dim3(grid), dim3(256), 0, stream, x, row_stride,
                       (uint8_t *)y, nb, total);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

static_assert(8 * kKqMaxS <= kKqThreads, "one thread per activation block");

bool kq_matvec_ok(int type, int64_t n, int64_t k, int64_t batch)
{
    if (type != 4 && type != 5) return false;
    const int64_t S = k / 256;
    if (k % 256 != 0 || S < 1 || S > kKqMaxS) return false;
    const int64_t R = kWave / S;
    const int64_t tiles = (n + R - 1) / R;
    return (tiles + kKqWaves - 1) / kKqWaves * batch < 0x7fffffffLL;
}

static size_t kq_lds_bytes(int type, int S)
{
    const int bb = type == 4 ? KqFmt<4>::kBytes : KqFmt<5>::kBytes;
    const int nb = 8 * S;
    const bool direct = type == 4 ? kq_direct<4>() : kq_direct<5>();
    return (size_t)(direct ? 0 : kKqWaves * kWave * bb) + (size_t)nb * 32 + (size_t)nb * 8 +
           kKqThreads * 4;
}

int launch_kq_matvec(int type, const KqDesc *d, int n_desc, hipStream_t stream)
{
    KqArgs a;
    memset(&a, 0, sizeof(a));
    int64_t wg = 0;
    int S_max = 1;
    int nj = 0;
    for (int i = 0; i < n_desc; ++i) {
        if (d[i].n == 0 || d[i].batch == 0) continue;
        KqJob &j = a.job[nj++];
        j.w = d[i].w; j.x = d[i].x; j.y = d[i].y;
        j.w_bstride = d[i].w_bstride; j.x_bstride = d[i].x_bstride; j.y_bstride = d[i].y_bstride;
        j.n = d[i].n;
        j.S = (int)(d[i].k / 256);
        j.R = kWave / j.S;
        j.tiles = (int)((d[i].n + j.R - 1) / j.R);
        j.wgpm = (j.tiles + kKqWaves - 1) / kKqWaves;
        j.wg0 = (int)wg;
        wg += (int64_t)j.wgpm * d[i].batch;
        if (wg > 0x7fffffffLL) return -4;
        S_max = j.S > S_max ? j.S : S_max;
    }
    if (nj == 0) return 0;
    a.n_jobs = nj;
    const size_t lds = kq_lds_bytes(type, S_max);
    if (type == 4)
        hipLaunchKernelGGL(kq_matvec_kernel<4>, dim3((unsigned)wg), dim3(kKqThreads), lds, stream, a);
    else
        hipLaunchKernelGGL(kq_matvec_kernel<5>, dim3((unsigned)wg), dim3(kKqThreads), lds, stream, a);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // namespace q8
