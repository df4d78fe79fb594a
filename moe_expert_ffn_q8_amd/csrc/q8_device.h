// q8_device.h -- device-side helpers shared by the gfx950 kernels of libq8moe.
//
// Q8_0 block: 34 bytes = binary16 scale (little-endian) + 32 int8 codes.
// Rows of blocks are back to back, so 8 blocks (272 B) span exactly 17
// 16-byte chunks and 4 blocks (136 B) span 17 8-byte words: a "quad" of 4
// blocks starting on an 8-byte boundary has a fixed internal layout:
//
//   dword  0      : scale(b0) | q0 q1 of b0
//   dwords 1..7   : codes of b0
//   dword  8      : q30 q31 of b0 | scale(b1)
//   dwords 9..16  : codes of b1 (aligned)
//   dword  17     : scale(b2) | q0 q1 of b2
//   dwords 18..24 : codes of b2
//   dword  25     : q30 q31 of b2 | scale(b3)
//   dwords 26..33 : codes of b3 (aligned)
//
// The activation side is kept in the same byte layout with the scale bytes
// set to zero ("masked image"), so a 4x int8 dot product of weight dword w with
// image dword w gives exactly the code products that dword holds: block b0 is
// the sum over dwords 0..8, b1 over 9..16, b2 over 17..25, b3 over 26..33.  No
// byte realignment is needed, and the integer block sums are exact.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q8 {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kQK = 32;
constexpr int kBlockBytes = 34;
constexpr int kQuadBytes = 136;       // 4 blocks
constexpr int kQuadDwords = 34;
constexpr int kWave = 64;

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16)
{
    _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)(bits16 & 0xffffu));
    return (float)h;
}

__device__ __forceinline__ int sdot4(uint32_t a, uint32_t b, int c)
{
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// Exact int32 block sums of one quad (weights w[34] against masked image x[34]).
__device__ __forceinline__ void quad_block_sums(const uint32_t *w, const uint32_t *x,
                                                int &s0, int &s1, int &s2, int &s3)
{
    int a = 0, b = 0, c = 0, d = 0;
#pragma unroll
    for (int i = 0; i <= 8; ++i) a = sdot4(w[i], x[i], a);
#pragma unroll
    for (int i = 9; i <= 16; ++i) b = sdot4(w[i], x[i], b);
#pragma unroll
    for (int i = 17; i <= 25; ++i) c = sdot4(w[i], x[i], c);
#pragma unroll
    for (int i = 26; i <= 33; ++i) d = sdot4(w[i], x[i], d);
    s0 = a; s1 = b; s2 = c; s3 = d;
}

// Scales of the four blocks of a quad, as fp32.
__device__ __forceinline__ void quad_scales(const uint32_t *w, float &d0, float &d1,
                                            float &d2, float &d3)
{
    d0 = half_bits_to_float(w[0]);
    d1 = half_bits_to_float(w[8] >> 16);
    d2 = half_bits_to_float(w[17]);
    d3 = half_bits_to_float(w[25] >> 16);
}

// Wave-scope ordering of LDS traffic between lanes of one wave: the compiler
// may not move LDS accesses across it, and the hardware has completed the
// wave's earlier LDS operations.
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Streaming (non-temporal) 16-byte global load.
__device__ __forceinline__ u32x4 load_nt16(const void *p)
{
    return __builtin_nontemporal_load((const u32x4 *)p);
}

// Plain 2-byte load of a possibly 2-byte-aligned location.
__device__ __forceinline__ uint32_t load_u16(const uint8_t *p)
{
    return (uint32_t)(*(const uint16_t *)p);
}

// ---------------------------------------------------------------------------
// Tile engine pieces shared by the decode and expert kernels.
//
// A wave-tile is `rows` whole weight rows of nb blocks (nb % 8 == 0), i.e.
// rows*nb/4 quads, at most 64.  It is rows*nb*17/8 16-byte chunks long and
// starts on a 16-byte boundary.

constexpr int kStageBytes = kWave * kQuadBytes;            // 8704: one wave's LDS slot
constexpr int kStageChunks = kStageBytes / 16;             // 544
constexpr int kTileLoads = (kStageChunks + kWave - 1) / kWave;   // 9 per lane

// Buffer resource word 3 for gfx9-family raw buffers (32-bit data format,
// no swizzle): loads past num_records return zero instead of faulting.
constexpr int kBufferWord3 = 0x00020000;
// Cache policy of the weight stream (aux bits of the buffer load): 2 = nt,
// non-temporal streaming.  A build option so the policy can be measured.
#ifndef Q8_WEIGHT_CACHE_POLICY
#define Q8_WEIGHT_CACHE_POLICY 2
#endif
constexpr int kCacheNT = Q8_WEIGHT_CACHE_POLICY;

// Values that are the same in every lane of a wave but that the compiler
// cannot prove so (they derive from threadIdx.x / 64, from LDS or from a
// ballot): read from the first lane into scalar registers, so that a buffer
// resource built from them needs no per-lane waterfall loop around each load.
__device__ __forceinline__ int wave_uniform(int v)
{
    return __builtin_amdgcn_readfirstlane(v);
}

__device__ __forceinline__ const uint8_t *wave_uniform(const uint8_t *p)
{
    const uint64_t v = (uint64_t)p;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
    return (const uint8_t *)(((uint64_t)hi << 32) | lo);
}

// Issue the coalesced 16-byte loads of one wave-tile into registers, through a
// raw buffer resource bounded to the tile: chunk i of lane l is load u with
// i = 64u + l, and chunks past the tile read as zero without a predicate (so
// no per-load masks or 64-bit addresses stay live in registers).
__device__ __forceinline__ void tile_issue(const uint8_t *base, int chunks, int lane,
                                           u32x4 (&g)[kTileLoads])
{
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void *)wave_uniform(base), 0, wave_uniform(chunks) * 16, kBufferWord3);
#pragma unroll
    for (int u = 0; u < kTileLoads; ++u)
        g[u] = __builtin_amdgcn_raw_buffer_load_b128(r, 16 * (u * kWave + lane), 0, kCacheNT);
}

// Write the loaded chunks to the wave's LDS slot in load order, then read back
// this lane's quad (lane stride 136 B).  Lanes >= live get zeros.
__device__ __forceinline__ void tile_to_quad(uint8_t *stage, const u32x4 (&g)[kTileLoads],
                                             int lane, int live, uint32_t (&wq)[kQuadDwords])
{
#pragma unroll
    for (int u = 0; u < kTileLoads; ++u) {
        const int i = u * kWave + lane;
        if (i < kStageChunks) ((u32x4 *)stage)[i] = g[u];
    }
    wave_lds_sync();
    const u32x2 *src = (const u32x2 *)(stage + kQuadBytes * lane);
#pragma unroll
    for (int v = 0; v < 17; ++v) {
        u32x2 p = (lane < live) ? src[v] : (u32x2){0u, 0u};
        wq[2 * v] = p.x;
        wq[2 * v + 1] = p.y;
    }
    wave_lds_sync();
}

// Load a 34-dword masked-image quad from LDS.
__device__ __forceinline__ void lds_quad(const uint8_t *p, uint32_t (&q)[kQuadDwords])
{
    const u32x2 *src = (const u32x2 *)p;
#pragma unroll
    for (int v = 0; v < 17; ++v) {
        u32x2 t = src[v];
        q[2 * v] = t.x;
        q[2 * v + 1] = t.y;
    }
}

// Load one activation quad (136 B) into registers as a masked image + scales.
__device__ __forceinline__ void load_x_quad(const uint8_t *p, bool al8, uint32_t (&q)[kQuadDwords],
                                            float4 &d)
{
    if (al8) {
        const u32x2 *src = (const u32x2 *)p;
#pragma unroll
        for (int v = 0; v < 17; ++v) {
            const u32x2 t = src[v];
            q[2 * v] = t.x;
            q[2 * v + 1] = t.y;
        }
    } else {
        const uint16_t *src = (const uint16_t *)p;
#pragma unroll
        for (int v = 0; v < kQuadDwords; ++v)
            q[v] = (uint32_t)src[2 * v] | ((uint32_t)src[2 * v + 1] << 16);
    }
    d.x = half_bits_to_float(q[0]);
    d.y = half_bits_to_float(q[8] >> 16);
    d.z = half_bits_to_float(q[17]);
    d.w = half_bits_to_float(q[25] >> 16);
    q[0] &= 0xffff0000u;
    q[8] &= 0x0000ffffu;
    q[17] &= 0xffff0000u;
    q[25] &= 0x0000ffffu;
}

// fp32 contribution of one quad: sum_b (d_w,b * d_x,b) * s_b, in block order.
__device__ __forceinline__ float quad_dot(const uint32_t (&wq)[kQuadDwords],
                                          const uint32_t *xq, float dw0, float dw1, float dw2,
                                          float dw3, float4 dx, int (&s)[4])
{
    quad_block_sums(wq, xq, s[0], s[1], s[2], s[3]);
    float acc = (dw0 * dx.x) * (float)s[0];
    acc = fmaf(dw1 * dx.y, (float)s[1], acc);
    acc = fmaf(dw2 * dx.z, (float)s[2], acc);
    acc = fmaf(dw3 * dx.w, (float)s[3], acc);
    return acc;
}

// Quantize one 32-value block held by 8 consecutive lanes (4 values each,
// lane & 7 = position): d = amax/127 (fp32 division), codes roundf(v/d)
// (half away from zero, saturating at +-127), d rounded to binary16 (RNE).
// Returns the 4 codes of this lane packed in a dword and the scale bits.
__device__ __forceinline__ void quantize_block8(float v0, float v1, float v2, float v3,
                                                uint32_t &codes, uint32_t &dbits)
{
    float a = fmaxf(fmaxf(fabsf(v0), fabsf(v1)), fmaxf(fabsf(v2), fabsf(v3)));
    a = fmaxf(a, __shfl_xor(a, 1));
    a = fmaxf(a, __shfl_xor(a, 2));
    a = fmaxf(a, __shfl_xor(a, 4));
    const float d = a / 127.0f;
    dbits = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)d);
    uint32_t packed = 0;
    if (d != 0.0f) {
        const float r[4] = {v0, v1, v2, v3};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float q = roundf(r[i] / d);
            q = fminf(fmaxf(q, -127.0f), 127.0f);
            packed |= ((uint32_t)(int)q & 0xffu) << (8 * i);
        }
    }
    codes = packed;
}

// Quantize the block held by 8 lanes (4 values each, lane & 7 = position) into
// a masked-image row (scale bytes zero; codes at the block's byte offsets) and
// its fp32 scale: the image bytes are those of q8_0_quantize_rows with the
// scale bytes cleared.
__device__ __forceinline__ void quantize8_to_image(float4 v, uint8_t *img_row, float *sc_row,
                                                   int b, int li)
{
    uint32_t codes, dbits;
    quantize_block8(v.x, v.y, v.z, v.w, codes, dbits);
    uint16_t *img16 = (uint16_t *)img_row;
    if (li == 0) {
        img16[b * 17] = 0;
        sc_row[b] = half_bits_to_float(dbits);
    }
    img16[b * 17 + 1 + 2 * li] = (uint16_t)(codes & 0xffffu);
    img16[b * 17 + 2 + 2 * li] = (uint16_t)(codes >> 16);
}

}  // namespace q8
