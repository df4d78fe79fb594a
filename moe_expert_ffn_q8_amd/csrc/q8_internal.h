// q8_internal.h -- host-side declarations shared by the translation units of
// libq8moe (launchers called by the C ABI layer in abi.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q8 {

// One matrix product of the streaming (decode) engine, already validated.
struct StreamDesc {
    const uint8_t *w;      // [batch][n][nb] blocks (16-byte aligned per matrix)
    const uint8_t *x;      // activations, rows of nb blocks
    float *y;
    int32_t *sums;         // optional int32 [m][n][nb] (validation; batch must be 1)
    int64_t n, nb, m, batch;
    int64_t w_bstride;     // bytes
    int64_t x_rstride;     // bytes
    int64_t x_bstride;     // bytes
    int64_t y_rstride;     // floats
    int64_t y_bstride;     // floats
    int x_f32;             // x is fp32 rows (quantized inside) instead of Q8_0 blocks
};

// Limits of the streaming engine (checked by the ABI layer).
constexpr int kStreamMaxJobs = 32;
constexpr int kStreamMaxM = 16;
constexpr int kStreamMaxNb = 256;   // k <= 8192 on the fast path

// True when the fast streaming kernel handles this descriptor (else the
// generic kernel is used).
bool stream_fast_ok(const StreamDesc &d);

// Enqueue descriptors; returns 0 or a negative q8_status.
int launch_stream(const StreamDesc *d, int n, hipStream_t stream);

// Matrix-core engine for 3 <= m <= 16 (all descriptors on the fast path).
bool small_m_ok(const StreamDesc *d, int n);
size_t small_m_lds_bytes(int64_t m, int64_t nb);
int launch_small_m(const StreamDesc *d, int n, hipStream_t stream);

// One-launch decode step from fp32 activations (m <= 2, fast shapes): the
// rows are quantized once into the workspace by the first workgroups of the
// launch, the product tiles wait for their entry's rows.
bool step_ok(const StreamDesc &d);
size_t step_ws_bytes(const StreamDesc *d, int n);
int launch_step(const StreamDesc *d, int n, void *ws, hipStream_t stream);

// Dense FFN up_gate + SwiGLU (m <= 2, fast shapes): d[i].n = n_ff, d[i].y = h.
int launch_dense_up_gate(const StreamDesc *d, int n, hipStream_t stream);

int launch_quantize_rows(const float *x, int64_t row_stride, void *y, int64_t n_rows,
                         int64_t k, hipStream_t stream);

// Prefill product on the int8 matrix cores (m token rows, any m >= 1).
bool gemm_ok(int64_t n, int64_t nb, int64_t m);
// sums: validation, int32 [m][n][nb] block sums (null in the product path).
int launch_gemm(const uint8_t *w, const uint8_t *x, float *y, int64_t n, int64_t nb, int64_t m,
                int64_t ldy, hipStream_t stream, int32_t *sums = nullptr);

// Row-interleaved weight layout (R8): 8-row groups of 272*nb bytes, the
// group's scales first, ordered by (block, row), then its codes, ordered by
// (block, row, position); the last group padded with zero rows.
constexpr int64_t kR8MaxNb = 1024;   // k <= 32768 (the activation row is staged in LDS, 36 B per block)
int64_t r8_bytes(int64_t n, int64_t nb);
int launch_r8_repack(const uint8_t *w, uint8_t *out, int64_t n, int64_t nb, hipStream_t stream);
// Matrix-vector products over R8 weights, several descriptors per launch
// (already validated): `batch` matrices each, strides in bytes (w, x) and
// floats (y); x_f32: the activation rows are fp32 (16-byte aligned), quantized
// inside the launch.
struct R8Desc {
    const uint8_t *w;
    const uint8_t *x;
    float *y;
    int64_t n, nb, batch;
    int64_t w_bstride, x_bstride, y_bstride;
    int32_t *sums;         // validation: int32 [batch][n][nb] block sums, else null
};
bool r8_matvec_ok(int64_t n, int64_t nb, int64_t batch);
int launch_r8_matvec(const R8Desc *d, int n_desc, bool x_f32, hipStream_t stream);

// Small-batch products (1 <= m <= 16 token rows, Q8_0 activations) over R8
// weights on the int8 matrix cores; strides in bytes (w, x) and floats (y).
struct R8MmDesc {
    const uint8_t *w;
    const uint8_t *x;
    float *y;
    int64_t n, nb, m, batch;
    int64_t w_bstride, x_rstride, x_bstride, y_rstride, y_bstride;
    int32_t *sums;         // validation: int32 [batch][m][n][nb] block sums, else null
};
bool r8_mm_ok(int64_t n, int64_t nb, int64_t m, int64_t batch);
int launch_r8_mm(const R8MmDesc *d, int n_desc, hipStream_t stream);

// Q8_1 activations (36-byte blocks: binary16 d and s, 32 codes) and the
// decode product over K-quant weights (type 4 = Q4_K, 144-byte super-blocks
// of 256 values; type 5 = Q5_K, 176 bytes) against one Q8_1 row per matrix.
constexpr int64_t kKqMaxS = 32;      // super-blocks per row: k <= 8192
struct KqDesc {
    const uint8_t *w;
    const uint8_t *x;
    float *y;
    int64_t n, k, batch;
    int64_t w_bstride, x_bstride, y_bstride;   // bytes, bytes, floats
};
int launch_q8_1_quantize_rows(const float *x, int64_t row_stride, void *y, int64_t n_rows,
                              int64_t k, hipStream_t stream);
bool kq_matvec_ok(int type, int64_t n, int64_t k, int64_t batch);
int launch_kq_matvec(int type, const KqDesc *d, int n_desc, hipStream_t stream);

// Streaming-read probe (measurement): reads `bytes` from p, writes one word
// per workgroup (at most 4096) to sink.
int launch_read_probe(const void *p, int64_t bytes, uint32_t *sink, int64_t sink_words,
                      hipStream_t stream);

// Largest dynamic LDS a workgroup may use on the current device.
int max_lds_bytes();

}  // namespace q8
