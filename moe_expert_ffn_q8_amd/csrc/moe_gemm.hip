// moe_gemm.hip -- the expert FFN for many tokens per call (prompt evaluation)
// on the gfx950 int8 matrix cores.
//
// Same computation as the decode kernels of moe.hip (Gemma-4-on-Xeon page,
// "GPUなしで13年前のXeon上でGemma 4 26Bを毎秒5トークンで実行する": the section on
// the broken op paths and the three-part fix, runtime graph fallback): mul_mat_id
// over the combined up_gate tensor with the gate half first, silu(gate) * up, the
// down projection of the quantized h rows, and the combine over a token's
// active experts.  That page reports prompt evaluation separately from decode;
// with many tokens each expert sees tens of token rows, so the products become
// small GEMMs and run on the matrix cores.
//
// One call:
//  1. routing (one workgroup): slot counts per expert, exclusive offsets, the
//     slots grouped by expert, and a tile table -- expert e's c_e slots make
//     ceil(c_e / 32) tiles of at most 32 slots.  Slots with an out-of-range id
//     are left out; they set the error word and (up_gate call) get NaN h rows.
//  2. the token rows (up_gate) or h rows (down) quantized into the workspace by
//     the quantizer kernel (bytes of q8_0_quantize_rows).
//  3. grouped GEMM: workgroup = (tile, block of 128 output columns).  A = the
//     tile's quantized rows, gathered straight from the workspace into LDS by
//     per-lane offsets of the LDS-DMA buffer loads; B = the expert's weight
//     rows; one v_mfma_i32_32x32x32_i8 per 32-block (K = 32 = one block) gives
//     exact int32 block sums, rescaled per block into fp32 accumulators as in
//     the prefill GEMM.  up_gate: wave w holds the 32 x 32 gate tile of columns
//     [n0 + 32w, n0 + 32w + 32) and the up tile of the same columns in the same
//     register layout, so the epilogue writes silu(g) * u element by element.
//     down: per-slot rows [slot][n_embd] into the workspace.
//  4. down only: the decode path's combine kernel (ascending u per token).
// Every output element is a sum over its own row and column only, so the
// order of slots inside an expert's tiles does not change any result.
#include <string.h>

#include "q8_device.h"
#include "q8_internal.h"
#include "q8_moe.h"

namespace q8 {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kPWaves = 8;
constexpr int kPThreads = kPWaves * kWave;    // 512
constexpr int kPBM = 32;                      // slots per tile
constexpr int kPBRows = kPWaves * 32;         // staged weight rows: one 32-row MFMA tile per wave
constexpr int kPStep = 4;                     // blocks per K step
constexpr int kPStepBytes = kPStep * kBlockBytes;    // 136 bytes of a row
constexpr int kPChunks = 9;                   // 16-byte chunks fetched per staged row
constexpr int kPRowStride = 16 * kPChunks;    // 144
constexpr int kPAChunks = 512;                // 32 rows x 9 = 288, padded to one load per thread
constexpr int kRouteThreads = 1024;

struct TileEntry {
    int expert, row0, rows, pad;
};

struct RouteArgs {
    const int32_t *ids;
    int32_t *hdr;           // [0] error word, [1] tile count
    int32_t *offsets;       // [n_expert + 1]
    int32_t *pairs;         // [n_slots]
    TileEntry *tiles;       // [max_tiles]
    float *h_nan;           // up_gate call: h rows of out-of-range slots get NaN (else null)
    int n_slots, n_expert, n_ff;
};

__global__ __launch_bounds__(kRouteThreads) void moe_route_tiles_kernel(const RouteArgs a)
{
    __shared__ int cnt[kMoeMaxExperts];
    __shared__ int scan_c[kMoeMaxExperts];
    __shared__ int scan_t[kMoeMaxExperts];
    __shared__ int bad;
    const int tid = threadIdx.x;
    for (int e = tid; e < kMoeMaxExperts; e += kRouteThreads) cnt[e] = 0;
    if (tid == 0) bad = 0;
    __syncthreads();
    for (int s = tid; s < a.n_slots; s += kRouteThreads) {
        const int e = a.ids[s];
        if (e < 0 || e >= a.n_expert) {
            atomicOr(&bad, 1);
            if (a.h_nan)
                for (int j = 0; j < a.n_ff; ++j) a.h_nan[(int64_t)s * a.n_ff + j] = __builtin_nanf("");
        } else {
            atomicAdd(&cnt[e], 1);
        }
    }
    __syncthreads();
    // inclusive scans of the counts and of the tile counts (Hillis-Steele)
    const int c = cnt[tid];
    int vc = c, vt = (c + kPBM - 1) / kPBM;
    scan_c[tid] = vc;
    scan_t[tid] = vt;
    __syncthreads();
    for (int d = 1; d < kMoeMaxExperts; d <<= 1) {
        const int ac = tid >= d ? scan_c[tid - d] : 0;
        const int at = tid >= d ? scan_t[tid - d] : 0;
        __syncthreads();
        vc += ac;
        vt += at;
        scan_c[tid] = vc;
        scan_t[tid] = vt;
        __syncthreads();
    }
    const int off = vc - c;                        // exclusive
    const int toff = vt - (c + kPBM - 1) / kPBM;
    if (tid < a.n_expert) {
        a.offsets[tid] = off;
        for (int i = 0; i * kPBM < c; ++i)
            a.tiles[toff + i] = TileEntry{tid, off + i * kPBM, min(kPBM, c - i * kPBM), 0};
    }
    if (tid == kRouteThreads - 1) {
        a.offsets[a.n_expert] = scan_c[a.n_expert - 1];
        a.hdr[0] = bad;
        a.hdr[1] = scan_t[a.n_expert - 1];
    }
    __syncthreads();
    // scatter the slots (the fill counters reuse cnt)
    for (int e = tid; e < kMoeMaxExperts; e += kRouteThreads) cnt[e] = 0;
    __syncthreads();
    for (int s = tid; s < a.n_slots; s += kRouteThreads) {
        const int e = a.ids[s];
        if (e >= 0 && e < a.n_expert) {
            const int p = atomicAdd(&cnt[e], 1);
            a.pairs[(e > 0 ? scan_c[e - 1] : 0) + p] = s;
        }
    }
}

struct PgArgs {
    const uint8_t *a;       // quantized A rows: token rows (up_gate) or slot rows (down)
    int64_t a_bytes;        // size of the A array (rows past it read as zero)
    const uint8_t *w;       // weights [n_expert][w_rows][nb] blocks
    int64_t expert_bytes;   // w_rows * nb * 34
    int w_rows;             // weight rows per expert (2 n_ff or n_embd)
    const int32_t *hdr;     // [1] = tile count
    const int32_t *pairs;
    const TileEntry *tiles;
    float *out;             // up_gate: h [slot][n_out]; down: yslot [slot][n_out]
    int n_out;              // n_ff (up_gate) or n_embd (down)
    int nb;                 // blocks per A / weight row (K / 32)
    int n_used;             // up_gate: A row of slot s is token s / n_used
    int max_tiles, tiles_n;
};

// 16 code bytes of a block fragment from a staged LDS row (`off` 2-byte aligned).
__device__ __forceinline__ v4i lds_codes16(const uint8_t *row, int off)
{
    const uint32_t *p = (const uint32_t *)(row + (off & ~3));
    if ((off & 3) == 0) return (v4i){(int)p[0], (int)p[1], (int)p[2], (int)p[3]};
    const uint32_t d0 = p[0], d1 = p[1], d2 = p[2], d3 = p[3], d4 = p[4];
    return (v4i){(int)__builtin_amdgcn_alignbyte(d1, d0, 2), (int)__builtin_amdgcn_alignbyte(d2, d1, 2),
                 (int)__builtin_amdgcn_alignbyte(d3, d2, 2), (int)__builtin_amdgcn_alignbyte(d4, d3, 2)};
}

// Output columns per workgroup: up_gate pairs waves w and w + 4 (gate and up
// rows of the same 32 columns), down gives every wave its own 32 columns.
template <bool UG>
constexpr int pg_cols()
{
    return UG ? kPBRows / 2 : kPBRows;
}

template <bool UG>
__global__ __launch_bounds__(kPThreads) void moe_gemm_kernel(const PgArgs a)
{
    constexpr int kBChunks = kPBRows * kPChunks;          // 2304
    constexpr int kBLoads = (kBChunks + kPThreads - 1) / kPThreads;    // 5 per thread
    constexpr int kALoads = kPAChunks / kPThreads;        // 1 per thread
    constexpr int kLoads = kALoads + kBLoads;             // per thread and step (all threads alike)
    constexpr int kBPad = kBLoads * kPThreads;            // B chunks incl. padding
    constexpr int kRows = kPBM + kPBRows;
    constexpr int kStage = 16 * (kPAChunks + kBPad);
    constexpr int kCols = pg_cols<UG>();
    static_assert(kPAChunks % kPThreads == 0, "whole A loads per thread");
    static_assert(kStage >= 4 * kWave * 16 * 4, "the epilogue exchange fits a stage buffer");
    // three K-step buffers as separate LDS objects: the compiler then orders
    // an LDS read only after the DMA loads into the buffer it reads (one array
    // indexed by stage would make every read wait for every DMA in flight)
    __shared__ __align__(16) uint8_t stage0[kStage];
    __shared__ __align__(16) uint8_t stage1[kStage];
    __shared__ __align__(16) uint8_t stage2[kStage];
    __shared__ __align__(16) float sc[kPStep][kRows];
    __shared__ int a_off[kPBM];
    __shared__ int a_slot[kPBM];

    const int tid = threadIdx.x;
    const int wave = wave_uniform(tid >> 6);
    const int lane = tid & 63;
    const int h = lane >> 5;
    const int li = lane & 31;

    // work = (column block, tile) with tiles fastest; consecutive work items
    // (the tiles of one expert for one column block) share an XCD
    const int nwg = (int)gridDim.x;
    const int work = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
    const int nt = work / a.max_tiles;
    const int mt = work - nt * a.max_tiles;
    if (nt >= a.tiles_n || mt >= a.hdr[1]) return;
    const TileEntry te = a.tiles[mt];
    const int n0 = nt * kCols;
    const int64_t row_bytes = (int64_t)a.nb * kBlockBytes;

    if (tid < kPBM) {
        const bool live = tid < te.rows;
        const int s = live ? a.pairs[te.row0 + tid] : -1;
        a_slot[tid] = s;
        a_off[tid] = live ? (int)((UG ? s / a.n_used : s) * row_bytes) : (int)a.a_bytes;
    }
    __syncthreads();

    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void *)a.a, 0, (int)a.a_bytes, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.w + (int64_t)te.expert * a.expert_bytes), 0, (int)a.expert_bytes, kBufferWord3);
    const int steps = a.nb / kPStep;

    // chunk f of a step lands at LDS byte 16 f of the stage buffer (row f / 9,
    // 16-byte chunk f % 9 of the row's 136 bytes; A rows first, padded to 512
    // chunks, then the weight rows).  Every thread issues kLoads loads per
    // step (padding chunks read past the buffers' ends: zeros, no traffic), so
    // one wait count covers "this step landed, the next ones in flight".
    auto issue = [&](int st, uint8_t *base, bool real) {
#pragma unroll
        for (int u = 0; u < kALoads; ++u) {
            const int f = 64 * wave + lane + kPThreads * u;
            const int r = f / kPChunks;
            const int c = f - r * kPChunks;
            const int off = (r < kPBM && real ? a_off[r] + st * kPStepBytes : (int)a.a_bytes) + 16 * c;
            auto *dst = (__attribute__((address_space(3))) void *)(base + 16 * (64 * wave + kPThreads * u));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, dst, 16, off, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kBLoads; ++u) {
            const int f = 64 * wave + lane + kPThreads * u;
            const int i = f / kPChunks;
            const int c = f - i * kPChunks;
            // rows past the expert's (clamped to its end) and padding read as zero
            const int wrow = f >= kBChunks ? a.w_rows :
                             min(UG ? (i < kCols ? n0 + i : a.n_out + n0 + i - kCols) : n0 + i, a.w_rows);
            const int off = real ? (int)(wrow * row_bytes) + st * kPStepBytes + 16 * c
                                 : (int)a.expert_bytes + 16 * c;
            auto *dst = (__attribute__((address_space(3))) void *)(
                base + 16 * (kPAChunks + 64 * wave + kPThreads * u));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, dst, 16, off, 0, 0, kCacheNT);
        }
    };

    float acc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;

    // Step st: wait for this wave's loads of st (the loads of st+1 stay in
    // flight), barrier (every wave's landed, and every wave is done with
    // st-1), issue st+2 into the buffer of st-1, unpack the scales, barrier,
    // compute.  Raw barriers with explicit waits: a workgroup fence would
    // also wait for the loads still in flight.  Issues are unconditional (a
    // step past the end loads zeros without traffic), so one wait count
    // always holds and the compiler's own tracking of which buffer each load
    // fills stays exact.
    auto body = [&](int st, const uint8_t *cur, uint8_t *next2) {
        __builtin_amdgcn_s_waitcnt(0x3f70 | (kLoads & 15) | ((kLoads >> 4) << 14));
        __builtin_amdgcn_s_barrier();
        issue(st + 2, next2, st + 2 < steps);
        const uint8_t *sa = cur;
        const uint8_t *sw = cur + 16 * kPAChunks;
        for (int e = tid; e < kPStep * kRows; e += kPThreads) {
            const int b = e / kRows;
            const int r = e - b * kRows;
            const int ro = r < kPBM ? r * kPRowStride : 16 * kPAChunks + (r - kPBM) * kPRowStride;
            sc[b][r] = half_bits_to_float(*(const uint16_t *)(cur + ro + b * kBlockBytes));
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);    // lgkmcnt(0): the scales are written
        __builtin_amdgcn_s_barrier();
        const int wr = 32 * wave + li;
#pragma unroll
        for (int b = 0; b < kPStep; ++b) {
            const int off = b * kBlockBytes + 2 + 16 * h;
            const v4i A = lds_codes16(sa + li * kPRowStride, off);
            const v4i B = lds_codes16(sw + wr * kPRowStride, off);
            const float dw = sc[b][kPBM + wr];
            float dx[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 v = *(const float4 *)&sc[b][8 * q + 4 * h];
                dx[4 * q + 0] = v.x; dx[4 * q + 1] = v.y; dx[4 * q + 2] = v.z; dx[4 * q + 3] = v.w;
            }
            v16i s = {0};
            s = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, B, s, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = fmaf(dx[r] * dw, (float)s[r], acc[r]);
        }
    };

    issue(0, stage0, true);
    issue(1, stage1, 1 < steps);
    for (int st = 0; st < steps; st += 3) {
        body(st, stage0, stage2);
        if (st + 1 < steps) body(st + 1, stage1, stage0);
        if (st + 2 < steps) body(st + 2, stage2, stage1);
    }

    // slot row 8(r/4) + 4h + r%4 of the tile; column n0 + 32 (wave % 4) + li
    // (up_gate: waves 4..7 hand their up tiles to waves 0..3 through LDS, in
    // the same register layout)
    const int col = n0 + 32 * (UG ? (wave & 3) : wave) + li;
    if (UG) {
        float *xch = (float *)stage0;
        __syncthreads();                       // every wave is done with the stage buffers
        if (wave >= 4) {
#pragma unroll
            for (int r = 0; r < 16; ++r) xch[((wave - 4) * 16 + r) * kWave + lane] = acc[r];
        }
        __syncthreads();
        if (wave >= 4 || col >= a.n_out) return;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = 8 * (r >> 2) + 4 * h + (r & 3);
            if (row >= te.rows) continue;
            const float g = acc[r];
            const float u = xch[(wave * 16 + r) * kWave + lane];
            a.out[(int64_t)a_slot[row] * a.n_out + col] = g / (1.0f + expf(-g)) * u;
        }
    } else {
        if (col >= a.n_out) return;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = 8 * (r >> 2) + 4 * h + (r & 3);
            if (row < te.rows) a.out[(int64_t)a_slot[row] * a.n_out + col] = acc[r];
        }
    }
}

size_t align256(size_t v)
{
    return (v + 255) & ~(size_t)255;
}

// Workspace layout of the prefill path.
struct PrefillWs {
    size_t offsets, pairs, tiles, data, hq, yslot, total;
    int64_t max_tiles;
};

PrefillWs prefill_layout(int64_t n_tok, int64_t n_embd, int64_t n_ff, int64_t n_expert,
                         int64_t n_used)
{
    PrefillWs L;
    const int64_t slots = n_tok * n_used;
    L.max_tiles = slots / kPBM + n_expert + 1;
    L.offsets = 256;
    L.pairs = L.offsets + align256((size_t)(n_expert + 1) * 4);
    L.tiles = L.pairs + align256((size_t)slots * 4);
    L.data = L.tiles + align256((size_t)L.max_tiles * sizeof(TileEntry));
    const size_t xq = align256((size_t)n_tok * (n_embd / kQK) * kBlockBytes);
    L.hq = L.data;
    L.yslot = L.hq + align256((size_t)slots * (n_ff / kQK) * kBlockBytes);
    const size_t down = L.yslot + align256((size_t)slots * n_embd * 4);
    L.total = down > L.data + xq ? down : L.data + xq;
    return L;
}

int launch_route(const int32_t *ids, uint8_t *ws, const PrefillWs &L, float *h_nan, int64_t n_slots,
                 int64_t n_expert, int64_t n_ff, hipStream_t stream)
{
    RouteArgs r;
    r.ids = ids;
    r.hdr = (int32_t *)ws;
    r.offsets = (int32_t *)(ws + L.offsets);
    r.pairs = (int32_t *)(ws + L.pairs);
    r.tiles = (TileEntry *)(ws + L.tiles);
    r.h_nan = h_nan;
    r.n_slots = (int)n_slots;
    r.n_expert = (int)n_expert;
    r.n_ff = (int)n_ff;
    hipLaunchKernelGGL(moe_route_tiles_kernel, dim3(1), dim3(kRouteThreads), 0, stream, r);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

template <bool UG>
int launch_grouped(const uint8_t *A, int64_t a_bytes, const uint8_t *w, int64_t w_rows, int64_t nb,
                   uint8_t *ws, const PrefillWs &L, float *out, int64_t n_out, int64_t n_used,
                   hipStream_t stream)
{
    PgArgs p;
    p.a = A;
    p.a_bytes = a_bytes;
    p.w = w;
    p.expert_bytes = w_rows * nb * kBlockBytes;
    p.w_rows = (int)w_rows;
    p.hdr = (const int32_t *)ws;
    p.pairs = (const int32_t *)(ws + L.pairs);
    p.tiles = (const TileEntry *)(ws + L.tiles);
    p.out = out;
    p.n_out = (int)n_out;
    p.nb = (int)nb;
    p.n_used = (int)n_used;
    p.max_tiles = (int)L.max_tiles;
    p.tiles_n = (int)((n_out + pg_cols<UG>() - 1) / pg_cols<UG>());
    int64_t grid = L.max_tiles * p.tiles_n;
    grid = (grid + 7) & ~(int64_t)7;
    if (grid > 0x7fffffff) return -4;
    hipLaunchKernelGGL(moe_gemm_kernel<UG>, dim3((unsigned)grid), dim3(kPThreads), 0, stream, p);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // namespace

bool moe_prefill_ok(int64_t n_tok, int64_t n_embd, int64_t n_ff, int64_t n_expert, int64_t n_used)
{
    if (n_tok <= kMoeDecodeMaxTok) return false;
    const int64_t nbe = n_embd / kQK, nbf = n_ff / kQK;
    if (nbe % kPStep != 0 || nbf % kPStep != 0) return false;
    if (n_tok > kMoePrefillMaxTok || n_tok * n_used > kMoePrefillMaxSlots) return false;
    // buffer-resource ranges and LDS-DMA offsets are 32-bit
    const int64_t ug_expert = 2 * n_ff * nbe * kBlockBytes, dn_expert = n_embd * nbf * kBlockBytes;
    const int64_t xq = n_tok * nbe * kBlockBytes, hq = n_tok * n_used * nbf * kBlockBytes;
    const int64_t lim = 0x7f000000LL;   // leaves room for a row past the end
    if (nbe * kBlockBytes > (1 << 20) || nbf * kBlockBytes > (1 << 20)) return false;
    return ug_expert < lim && dn_expert < lim && xq < lim && hq < lim && n_expert <= kMoeMaxExperts;
}

size_t moe_prefill_ws_bytes(int64_t n_tok, int64_t n_embd, int64_t n_ff, int64_t n_expert,
                            int64_t n_used)
{
    return prefill_layout(n_tok, n_embd, n_ff, n_expert, n_used).total;
}

int launch_moe_prefill_up_gate(const uint8_t *w, const float *x, const int32_t *ids, float *h,
                               void *ws_, int64_t n_tok, int64_t n_embd, int64_t n_ff,
                               int64_t n_expert, int64_t n_used, hipStream_t stream)
{
    uint8_t *ws = (uint8_t *)ws_;
    const PrefillWs L = prefill_layout(n_tok, n_embd, n_ff, n_expert, n_used);
    const int64_t nb = n_embd / kQK;
    if (int rc = launch_route(ids, ws, L, h, n_tok * n_used, n_expert, n_ff, stream)) return rc;
    uint8_t *xq = ws + L.data;
    if (int rc = launch_quantize_rows(x, n_embd, xq, n_tok, n_embd, stream)) return rc < 0 ? -6 : rc;
    return launch_grouped<true>(xq, n_tok * nb * kBlockBytes, w, 2 * n_ff, nb, ws, L, h, n_ff, n_used,
                                stream);
}

int launch_moe_prefill_down(const uint8_t *w, const float *h, const int32_t *ids, const float *cw,
                            float *out, void *ws_, int64_t n_tok, int64_t n_embd, int64_t n_ff,
                            int64_t n_expert, int64_t n_used, hipStream_t stream)
{
    uint8_t *ws = (uint8_t *)ws_;
    const PrefillWs L = prefill_layout(n_tok, n_embd, n_ff, n_expert, n_used);
    const int64_t nb = n_ff / kQK;
    const int64_t slots = n_tok * n_used;
    if (int rc = launch_route(ids, ws, L, nullptr, slots, n_expert, n_ff, stream)) return rc;
    uint8_t *hq = ws + L.hq;
    if (int rc = launch_quantize_rows(h, n_ff, hq, slots, n_ff, stream)) return rc < 0 ? -6 : rc;
    float *yslot = (float *)(ws + L.yslot);
    if (int rc = launch_grouped<false>(hq, slots * nb * kBlockBytes, w, n_embd, nb, ws, L, yslot,
                                       n_embd, n_used, stream))
        return rc;
    return launch_moe_combine(yslot, ids, cw, out, n_tok, n_embd, n_used, n_expert, stream);
}

}  // namespace q8
