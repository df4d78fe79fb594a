// gemm.hip -- the prefill product Y[m][n] = X[m][k] . W[n][k]^T for many token
// rows, on the gfx950 int8 matrix cores.
//
// The arithmetic is the same as the decode engine's (the block dot product of
// ggml_vec_dot_q8_0_q8_0, on the Gemma-4-on-Xeon page, "GPUなしで13年前のXeon
// 上でGemma 4 26Bを毎秒5トークンで実行する", section on narrowing down the
// cause): an exact int32 sum per 32-block, then (d_x * d_w) * s in fp32.  Prompt
// evaluation is the compute-bound side of the same path (that page reports it
// separately from decode).
//
// v_mfma_i32_32x32x32_i8 has K = 32, exactly one Q8_0 block: one instruction
// gives the exact int32 block sums of a 32x32 (token x weight-row) tile, and
// blocks never mix inside an integer sum, so every block's tile is rescaled by
// its own scales into fp32 accumulators, and that rescale, not the int8
// matrix core, bounds this kernel.  By default (Q8_GEMM_OUTER=2) the scale
// products of a tile come from a second matrix instruction (an outer product
// of the scales' binary16 bits), leaving a convert and a fused multiply-add
// per element and block on the VALU, and the int8 sums are carried one block
// ahead so that no rescale waits for them (see compute_pipelined); with the
// products on the VALU (Q8_GEMM_OUTER=0) it is 3 operations per element and
// block.  The staged rows are 144 bytes apart (16-byte DMA
// granularity), so the 4-byte reads that codes 2 bytes past a dword boundary
// need would put 32 rows on 8 bank offsets (4-way conflicts): each step, every
// thread first realigns one staged row in place (codes of block b to bytes
// 32b..32b+31, its scale to an fp32 array), and the fragments are then single
// 16-byte reads, conflict-free for 8 rows 144 bytes apart (Q8_GEMM_REALIGN;
// 130 against 143 us).  (Measured before the pipelined form: build option
// Q8_GEMM_OUTER=1 forms the rank-1 scale products of a block as an outer
// product on the fp32 matrix core instead, same register layout, leaving 2
// VALU operations: 150.5 against 141.3 us with each tile's sums pinned in
// place (Q8_GEMM_PIN, else 198 us at 1 wave per SIMD), so it is off.  The same
// outer product from a K = 16 binary16 product (v_mfma_f32_32x32x16_f16, the
// scales' own bits) measured 138.6 to 142.8 us against 133.4 us.  A variant
// with the codes themselves on the binary16 matrix cores -- a Q8_0 code is
// exact in binary16 and a block's sums are exact in the fp32 accumulator of
// v_mfma_f32_32x32x16_f16, so two such instructions give S with no
// conversion, a third gives the scale products, and one fused multiply-add
// per element and block is left (40% fewer VALU instructions, 3x the matrix
// instructions, each thread converting its staged row to binary16 in 2-block
// steps) -- measured 142-144 us against 131-132 us: at 2 waves per SIMD
// (202 VGPRs, 76 KB of LDS) neither pipe fills (VALU 38%, matrix cores 27% of
// the active cycles), the waves wait on LDS reads and result latencies.)
//
// Work decomposition:
//  * Workgroup = 4 waves, output tile 128 tokens x 128 weight rows; wave
//    (wm, wn) computes the 64 x 64 quadrant (wm, wn) as 2 x 2 MFMA tiles.
//  * K is walked in steps of 4 blocks (136 bytes per row).  A step of both
//    operands (2 x 128 rows)
//    goes straight from HBM to LDS with coalesced 16-byte buffer loads in LDS
//    DMA mode (rows past m or n read as zero), double-buffered so the next
//    step streams in while the current one is computed; the block scales are
//    unpacked once per step (binary16 bits for the default form, fp32 for
//    the VALU form) while each thread realigns its staged row.
//  * Operand layout of the MFMA: lane l supplies row l%32 of its tile and the
//    16 codes of k-group l/32 (A = tokens, B = weight rows, same byte order, so
//    the integer sum covers the block's 32 codes once); result register r of
//    lane l holds token 8*(r/4) + 4*(l/32) + r%4, weight row l%32.
//  * Workgroups that share a weight tile are placed on the same XCD (its L2).
#include <string.h>

#include "q8_device.h"
#include "q8_internal.h"

namespace q8 {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));

constexpr int kGThreads = 256;
constexpr int kBM = 128;                 // tokens per workgroup tile
constexpr int kBN = 128;                 // weight rows per workgroup tile
#ifndef Q8_GEMM_STEP_BLOCKS
#define Q8_GEMM_STEP_BLOCKS 4
#endif
constexpr int kStepBlocks = Q8_GEMM_STEP_BLOCKS;           // blocks per K step (4 or 8)
constexpr int kStepRowBytes = kStepBlocks * kBlockBytes;    // 136 or 272 bytes of a row
constexpr int kStepChunks = (kStepRowBytes + 15) / 16;      // 9 or 17 16-byte chunks
constexpr int kRowStride = 16 * kStepChunks;                // staged row: 144 or 272 B
constexpr int kStageRows = kBM + kBN;                       // 256
constexpr int kStageLoads = kStageRows * kStepChunks / kGThreads;   // 9 or 17 per thread
#ifndef Q8_GEMM_REALIGN
#define Q8_GEMM_REALIGN 1
#endif
static_assert(!Q8_GEMM_REALIGN || (kStepBlocks <= 4 && kStageRows == kGThreads),
              "realigning: one staged row of up to 4 blocks per thread");
#ifndef Q8_GEMM_PIN
#define Q8_GEMM_PIN 1
#endif
#ifndef Q8_GEMM_PIN_VALU
#define Q8_GEMM_PIN_VALU 0
#endif
#ifndef Q8_GEMM_OUTER
// scale products on the VALU (0), on the fp32 matrix core (1), or on the
// binary16 matrix core with the tiles software-pipelined (2)
#define Q8_GEMM_OUTER 2
#endif
static_assert(kStepBlocks == 2 || kStepBlocks == 4 || kStepBlocks == 8, "K step of 2, 4 or 8 blocks");
// the token/weight row boundary falls on a wave boundary of the load pattern
static_assert((kBM * kStepChunks) % 64 == 0, "uniform buffer resource per load");

static_assert(kStageRows * kStepChunks % kGThreads == 0, "whole loads per thread");

struct GemmArgs {
    const uint8_t *w;      // [n][nb] blocks
    const uint8_t *x;      // [m][nb] blocks
    float *y;              // [m][ldy]
    int32_t *sums;         // validation (SUMS kernel): int32 [m][n][nb] block sums
    int m, n, nb, ldy;
    int tiles_n, tiles_m;
};

// 16 code bytes of a block fragment from the staged LDS rows: `off` is 2-byte
// aligned; the compiler resolves the alignment per unrolled block.
__device__ __forceinline__ v4i lds_codes16(const uint8_t *row, int off)
{
    const uint32_t *p = (const uint32_t *)(row + (off & ~3));
    if ((off & 3) == 0) return (v4i){(int)p[0], (int)p[1], (int)p[2], (int)p[3]};
    const uint32_t d0 = p[0], d1 = p[1], d2 = p[2], d3 = p[3], d4 = p[4];
    return (v4i){(int)__builtin_amdgcn_alignbyte(d1, d0, 2), (int)__builtin_amdgcn_alignbyte(d2, d1, 2),
                 (int)__builtin_amdgcn_alignbyte(d3, d2, 2), (int)__builtin_amdgcn_alignbyte(d4, d3, 2)};
}

// SUMS (validation build of the same kernel): every exact int32 block sum is
// also written out.
#ifndef Q8_GEMM_OCC
#define Q8_GEMM_OCC 1
#endif
template <bool SUMS>
__global__ __launch_bounds__(kGThreads, Q8_GEMM_OCC) void gemm_q8_kernel(const GemmArgs a)
{
    // Two K-step buffers as separate LDS objects: the compiler then orders an
    // LDS read only after the DMA loads into the buffer it reads (with one
    // stage-indexed array every read waited for the next step's loads too).
    __shared__ __align__(16) uint8_t stage0[kStageRows * kRowStride];
    __shared__ __align__(16) uint8_t stage1[kStageRows * kRowStride];
    __shared__ __align__(16) float sc[kStepBlocks][kStageRows];              // 8192 B
    __shared__ __align__(16) uint16_t sc16[kStepBlocks][kStageRows];         // binary16 bits
    constexpr bool kPipe = Q8_GEMM_OUTER == 2;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int h = lane >> 5;           // k-group of this lane
    const int li = lane & 31;

    // Tile order: the tiles_m token tiles of one weight tile are consecutive
    // in `work`, and work is spread so that they share an XCD (workgroups are
    // dealt to the 8 XCDs round robin by blockIdx.x).
    const int nwg = a.tiles_n * a.tiles_m;
    int work = blockIdx.x;
    if ((nwg & 7) == 0) work = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
    const int tn = work / a.tiles_m;
    const int tm = work - tn * a.tiles_m;
    const int m0 = tm * kBM, n0 = tn * kBN;

    const int64_t row_bytes = (int64_t)a.nb * kBlockBytes;
    const int steps = a.nb / kStepBlocks;

    // Buffer resources over the operand rows of this tile: rows past m or n
    // fall outside num_records and read as zero.
    const int xr_rows = min(kBM, a.m - m0), wr_rows = min(kBN, a.n - n0);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.x + (int64_t)m0 * row_bytes), 0, (int)(xr_rows * row_bytes), kBufferWord3);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.w + (int64_t)n0 * row_bytes), 0, (int)(wr_rows * row_bytes), kBufferWord3);

    // Chunk f = 64*wave + lane + 256*u of a step (row f/C, 16-byte chunk f%C
    // with C = kStepChunks; rows 0..127 tokens, 128..255 weight rows) lands at
    // LDS byte 16*f of the step buffer, because a staged row is 16*C bytes.
    // That is the LDS DMA pattern (64 lanes -> 1 KB contiguous per
    // instruction), and a (u, wave) pair never straddles the token/weight
    // boundary, so its buffer resource is uniform.  With 4-block steps a row's
    // 136 bytes are fetched as 9 chunks (8 bytes past the step, read but not
    // used; past the operand they read as zero).
    auto issue = [&](int st, uint8_t *sbuf, bool real) {
#pragma unroll
        for (int u = 0; u < kStageLoads; ++u) {
            const int f = 64 * wave + lane + kGThreads * u;
            const int r = f / kStepChunks;
            const int c = f - r * kStepChunks;
            // a step past the end loads zeros (offset past both ranges), so
            // issues are unconditional and every wait count is exact
            const int off = real ? (int)((r & (kBM - 1)) * row_bytes) + st * kStepRowBytes + 16 * c
                                 : 0x7ffffff0;
            auto *dst = (__attribute__((address_space(3))) void *)(&sbuf[16 * (64 * wave + kGThreads * u)]);
            if (kGThreads * u + 64 * wave < kBM * kStepChunks)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, dst, 16, off, 0, 0, 0);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, dst, 16, off, 0, 0, kCacheNT);
        }
    };

    float acc[2][2][16];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // Q8_GEMM_OUTER == 2: per tile and block two matrix instructions -- the
    // exact int32 sums S of the block (int8, K = 32) and the scale products
    // P = d_x * d_w as an outer product on the binary16 matrix core (each
    // scale's own bits at k = 0, zeros elsewhere; a product of two binary16
    // values is exact in fp32, so P has the bits of the VALU product) -- and
    // 16 converts and 16 fused multiply-adds, acc = fma(P, float(S), acc), the
    // same operation on the same values as the VALU form, with one VALU
    // operation per element and block fewer.  The blocks of a step are a
    // runtime loop whose sums S are carried into the next iteration: an
    // iteration rescales block b tile by tile (P formed just before its
    // rescale) and, right after each tile, issues that tile's int8 product
    // for block b + 1 into the registers the rescale has just read, so no
    // rescale waits for its sums and nothing is hoisted across iterations
    // (256 VGPRs, two waves per SIMD).  Measured on 512 x 4096 x 14336:
    // 125.5 against 131.5 us for the VALU form; carrying P as well (299
    // VGPRs, one wave per SIMD): 151 us; the VALU form pipelined the same way:
    // no change (129 us).
    // kmask: all ones on the lanes of k-group 0, opaque to the compiler (a
    // select there would become a branch around each scale read).
    int kmask = h == 0 ? 0xffff : 0;
    asm volatile("" : "+v"(kmask));
    auto compute_pipelined = [&](int st, const uint8_t *sb) {
        v4i A[2], B[2];
        int sa_n[2], sb_n[2], sa_c[2], sb_c[2];     // scale bits of blocks b + 1 and b
        auto load = [&](int b) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int r = 64 * wm + 32 * i + li;
                A[i] = *(const v4i *)(sb + r * kRowStride + 32 * b + 16 * h);
                sa_n[i] = (int)sc16[b][r] & kmask;
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int r = kBM + 64 * wn + 32 * j + li;
                B[j] = *(const v4i *)(sb + r * kRowStride + 32 * b + 16 * h);
                sb_n[j] = (int)sc16[b][r] & kmask;
            }
        };
        auto advance = [&]() {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                sa_c[i] = sa_n[i];
                sb_c[i] = sb_n[i];
            }
        };
        v16i S[2][2];
        auto issue = [&](int i, int j) {
            const v16i zi = {0};
            S[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[i], B[j], zi, 0, 0, 0);
        };
        auto rescale = [&](int b, int i, int j) {
            if (SUMS) {
                const int n = n0 + 64 * wn + 32 * j + li;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = m0 + 64 * wm + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                    if (m < a.m && n < a.n)
                        a.sums[((int64_t)m * a.n + n) * a.nb + st * kStepBlocks + b] = S[i][j][r];
                }
            }
            const v16f zf = {0.f};
            const v16f P = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                __builtin_bit_cast(h8, (v4i){sa_c[i], 0, 0, 0}),
                __builtin_bit_cast(h8, (v4i){sb_c[j], 0, 0, 0}), zf, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = fmaf(P[r], (float)S[i][j][r], acc[i][j][r]);
        };
        load(0);
        advance();
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) issue(i, j);
#pragma unroll 1
        for (int b = 0; b + 1 < kStepBlocks; ++b) {
            load(b + 1);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    rescale(b, i, j);
                    issue(i, j);
                }
            advance();
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) rescale(kStepBlocks - 1, i, j);
    };

    // Step st: wait for this wave's loads of st, barrier (every wave's
    // landed; every wave is done with st-1, whose buffer the next issue
    // fills), issue st+1, unpack the scales, barrier, compute.  Raw barriers
    // with explicit waits: the workgroup fence of __syncthreads would also
    // wait for the loads of st+1.
    auto body = [&](int st, uint8_t *sb, uint8_t *next) {
        __builtin_amdgcn_s_waitcnt(0x3f70);    // vmcnt(0): this wave's loads of st landed
        __builtin_amdgcn_s_barrier();
        issue(st + 1, next, st + 1 < steps);
        if (Q8_GEMM_REALIGN) {
            // thread t realigns staged row t in place: the codes of block b to
            // bytes 32b .. 32b+31 (4-byte aligned, 16-byte reads from then on),
            // its scale to sc[b][t]; the 16-byte reads of 8 consecutive rows
            // (144 bytes apart) fall on distinct banks
            uint8_t *rowp = sb + tid * kRowStride;
            uint32_t d[4 * kStepChunks];
#pragma unroll
            for (int c = 0; c < kStepChunks; ++c) {
                const u32x4 v = *(const u32x4 *)(rowp + 16 * c);
                d[4 * c] = v.x; d[4 * c + 1] = v.y; d[4 * c + 2] = v.z; d[4 * c + 3] = v.w;
            }
            uint32_t cw[kStepBlocks][8];
#pragma unroll
            for (int b = 0; b < kStepBlocks; ++b) {
                // block b at byte 34b: 34b = 4*(17b/2) (+2 when b is odd)
                const int D = (17 * b) >> 1;
                if (kPipe) {
                    sc16[b][tid] = (uint16_t)((b & 1) == 0 ? d[D] & 0xffffu : d[D] >> 16);
                    if ((b & 1) == 0) {
#pragma unroll
                        for (int j = 0; j < 8; ++j) cw[b][j] = __builtin_amdgcn_alignbyte(d[D + j + 1], d[D + j], 2);
                    } else {
#pragma unroll
                        for (int j = 0; j < 8; ++j) cw[b][j] = d[D + 1 + j];
                    }
                } else if ((b & 1) == 0) {
                    sc[b][tid] = half_bits_to_float(d[D] & 0xffffu);
#pragma unroll
                    for (int j = 0; j < 8; ++j) cw[b][j] = __builtin_amdgcn_alignbyte(d[D + j + 1], d[D + j], 2);
                } else {
                    sc[b][tid] = half_bits_to_float(d[D] >> 16);
#pragma unroll
                    for (int j = 0; j < 8; ++j) cw[b][j] = d[D + 1 + j];
                }
            }
#pragma unroll
            for (int b = 0; b < kStepBlocks; ++b) {
                *(u32x4 *)(rowp + 32 * b) = (u32x4){cw[b][0], cw[b][1], cw[b][2], cw[b][3]};
                *(u32x4 *)(rowp + 32 * b + 16) = (u32x4){cw[b][4], cw[b][5], cw[b][6], cw[b][7]};
            }
        } else {
#pragma unroll
            for (int i = 0; i < kStepBlocks * kStageRows / kGThreads; ++i) {
                const int e = tid + kGThreads * i;
                const int r = e & (kStageRows - 1);
                const int b = e >> 8;
                sc[b][r] = half_bits_to_float(*(const uint16_t *)(sb + r * kRowStride + b * kBlockBytes));
            }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);    // lgkmcnt(0): the scales are written
        __builtin_amdgcn_s_barrier();

        if (kPipe) {
            compute_pipelined(st, sb);
            return;
        }
        // two blocks per unrolled iteration: the full unroll of a step keeps
        // too many operands live (256 VGPRs and spills against 176)
#pragma unroll 2
        for (int b = 0; b < kStepBlocks; ++b) {
            const int off = b * kBlockBytes + 2 + 16 * h;
            v4i A[2], B[2];
            if (Q8_GEMM_REALIGN) {
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    A[i] = *(const v4i *)(sb + (64 * wm + 32 * i + li) * kRowStride + 32 * b + 16 * h);
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    B[j] = *(const v4i *)(sb + (kBM + 64 * wn + 32 * j + li) * kRowStride + 32 * b + 16 * h);
            } else {
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    A[i] = lds_codes16(sb + (64 * wm + 32 * i + li) * kRowStride, off);
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    B[j] = lds_codes16(sb + (kBM + 64 * wn + 32 * j + li) * kRowStride, off);
            }
            // Scale products of the block as outer products on the fp32 matrix
            // core: P(i,j) = dx_i (x) dw_j with k = 2 and the second k row zero,
            // so P lands in the same 32x32 register layout as the int32 tile
            // (exact: a product of two binary16 values fits fp32).
            float adx[2], bdw[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) adx[i] = h == 0 ? sc[b][64 * wm + 32 * i + li] : 0.0f;
#pragma unroll
            for (int j = 0; j < 2; ++j) bdw[j] = sc[b][kBM + 64 * wn + 32 * j + li];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                float dx[16];
                if (!Q8_GEMM_OUTER) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float4 v = *(const float4 *)&sc[b][64 * wm + 32 * i + 8 * q + 4 * h];
                        dx[4 * q + 0] = v.x; dx[4 * q + 1] = v.y; dx[4 * q + 2] = v.z; dx[4 * q + 3] = v.w;
                    }
                }
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    v16i s = {0};
                    s = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[i], B[j], s, 0, 0, 0);
                    if (SUMS) {
                        const int n = n0 + 64 * wn + 32 * j + li;
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int m = m0 + 64 * wm + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                            if (m < a.m && n < a.n)
                                a.sums[((int64_t)m * a.n + n) * a.nb + st * kStepBlocks + b] = s[r];
                        }
                    }
                    if (Q8_GEMM_OUTER) {
                        v16f pz = {0.f};
                        const v16f P = __builtin_amdgcn_mfma_f32_32x32x2f32(adx[i], bdw[j], pz, 0, 0, 0);
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            acc[i][j][r] = fmaf(P[r], (float)s[r], acc[i][j][r]);
                            // one tile's sums at a time (else every tile's two
                            // matrix-core results stay live across the block)
                            if (Q8_GEMM_PIN) asm volatile("" : "+v"(acc[i][j][r]));
                        }
                    } else {
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            acc[i][j][r] = fmaf(dx[r] * bdw[j], (float)s[r], acc[i][j][r]);
                            if (Q8_GEMM_PIN_VALU) asm volatile("" : "+v"(acc[i][j][r]));
                        }
                    }
                }
            }
        }
    };

    issue(0, stage0, true);
    for (int st = 0; st < steps; st += 2) {
        body(st, stage0, stage1);
        if (st + 1 < steps) body(st + 1, stage1, stage0);
    }

    // store: token m0 + 64wm + 32i + 8(r/4) + 4h + r%4, weight row n0 + 64wn + 32j + li
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = n0 + 64 * wn + 32 * j + li;
            if (n >= a.n) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + 64 * wm + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                if (m < a.m) a.y[(int64_t)m * a.ldy + n] = acc[i][j][r];
            }
        }
}

}  // namespace

bool gemm_ok(int64_t n, int64_t nb, int64_t m)
{
    if (nb % 8 != 0) return false;
    // buffer-resource ranges are 32-bit: a tile's rows must fit
    const int64_t row_bytes = nb * kBlockBytes;
    if (row_bytes * kBM > 0x7fffffffLL) return false;
    if (n > 0x7fffffffLL || m > 0x7fffffffLL) return false;
    return true;
}

int launch_gemm(const uint8_t *w, const uint8_t *x, float *y, int64_t n, int64_t nb, int64_t m,
                int64_t ldy, hipStream_t stream, int32_t *sums)
{
    GemmArgs a;
    a.w = w; a.x = x; a.y = y; a.sums = sums;
    a.m = (int)m; a.n = (int)n; a.nb = (int)nb; a.ldy = (int)ldy;
    a.tiles_n = (int)((n + kBN - 1) / kBN);
    a.tiles_m = (int)((m + kBM - 1) / kBM);
    const int64_t grid = (int64_t)a.tiles_n * a.tiles_m;
    if (grid > 0x7fffffff) return -4;
    if (sums)
        hipLaunchKernelGGL(gemm_q8_kernel<true>, dim3((unsigned)grid), dim3(kGThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(gemm_q8_kernel<false>, dim3((unsigned)grid), dim3(kGThreads), 0, stream, a);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // namespace q8
