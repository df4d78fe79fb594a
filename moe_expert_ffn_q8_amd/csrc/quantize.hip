// quantize.hip -- fp32 rows -> Q8_0 blocks on gfx950.
//
// Rule (per 32 values): d = max|x| / 127 with an IEEE fp32 division, each code
// round(x / d) (fp32 division, ties away from zero, saturating at +-127), d
// stored as round-to-nearest-even binary16; an all-zero block gives d = +0.
// The role is that of quantize_row_q8_0 on the Gemma-4-on-Xeon page
// ("GPUなしで13年前のXeon上でGemma 4 26Bを毎秒5トークンで実行する", three-part
// fix, compile-fix part), applied to every row.
//
// Layout of the work: eight lanes own one block (4 values each, one 16-byte
// load per lane, so a wave reads 1 KB of contiguous fp32).  The block's amax
// is combined across the eight lanes with xor shuffles.  The 34-byte blocks
// of a 32-block tile are assembled in LDS and written back as 16-byte stores
// (1088 B per tile = 68 x 16 B), so the 2-byte-aligned block layout never
// costs a narrow global store on the main path.
//
// Numerics: no fast-math anywhere in this library: `/` is the correctly
// rounded fp32 division, roundf rounds half away from zero, and the fp16
// conversion is v_cvt_f16_f32 (round to nearest even, subnormals kept).
#include "q8_device.h"
#include "q8_internal.h"

namespace q8 {

constexpr int kQTileBlocks = 32;   // 256 threads / 8 lanes per block

__global__ __launch_bounds__(256) void quantize_rows_kernel(const float *__restrict__ x,
                                                            int64_t row_stride,
                                                            uint8_t *__restrict__ y,
                                                            int64_t nb, int64_t total_blocks)
{
    __shared__ __align__(16) uint16_t tile[kQTileBlocks * 17];   // 1088 bytes
    const int tid = threadIdx.x;
    const int gi = tid >> 3;        // block within the tile
    const int li = tid & 7;         // lane within the block

    for (int64_t blk0 = (int64_t)blockIdx.x * kQTileBlocks; blk0 < total_blocks;
         blk0 += (int64_t)gridDim.x * kQTileBlocks) {
        const int64_t g = blk0 + gi;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (g < total_blocks) {
            const int64_t r = g / nb;
            const int64_t b = g - r * nb;
            v = *(const float4 *)(x + r * row_stride + b * kQK + 4 * li);
        }
        uint32_t codes, dbits;
        quantize_block8(v.x, v.y, v.z, v.w, codes, dbits);
        if (li == 0) tile[17 * gi] = (uint16_t)dbits;
        tile[17 * gi + 1 + 2 * li] = (uint16_t)(codes & 0xffffu);
        tile[17 * gi + 2 + 2 * li] = (uint16_t)(codes >> 16);
        __syncthreads();

        const int64_t left = total_blocks - blk0;
        const int nblk = left < kQTileBlocks ? (int)left : kQTileBlocks;
        uint8_t *out = y + blk0 * kBlockBytes;
        if (nblk == kQTileBlocks && (((uintptr_t)out) & 15u) == 0) {
            if (tid < kQTileBlocks * kBlockBytes / 16)
                ((u32x4 *)out)[tid] = ((const u32x4 *)tile)[tid];
        } else {
            for (int i = tid; i < nblk * 17; i += 256) ((uint16_t *)out)[i] = tile[i];
        }
        __syncthreads();
    }
}

int launch_quantize_rows(const float *x, int64_t row_stride, void *y, int64_t n_rows,
                         int64_t k, hipStream_t stream)
{
    const int64_t nb = k / kQK;
    const int64_t total = n_rows * nb;
    if (total == 0) return 0;
    int64_t tiles = (total + kQTileBlocks - 1) / kQTileBlocks;
    const int64_t max_grid = 256 * 64;
    const unsigned grid = (unsigned)(tiles < max_grid ? tiles : max_grid);
    hipLaunchKernelGGL(quantize_rows_kernel, dim3(grid), dim3(256), 0, stream, x, row_stride,
                       (uint8_t *)y, nb, total);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace q8
