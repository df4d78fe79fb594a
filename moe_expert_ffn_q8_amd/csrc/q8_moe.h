// q8_moe.h -- host-side declarations of the expert-FFN launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace q8 {

constexpr int kMoeMaxUsed = 16;      // active experts per token
constexpr int kMoeMaxSlots = 1024;   // n_tok * n_used per call (decode sizes)
constexpr int kMoeMaxExperts = 1024;
constexpr int kMoeMaxLayers = 32;    // independent layers of one shape per launch
constexpr int kMoeDecodeMaxTok = 16;        // more tokens per call: the prefill path
constexpr int kMoePrefillMaxTok = 8192;
constexpr int kMoePrefillMaxSlots = 65536;

// Validation outputs of the expert FFN (single-layer calls only; every
// pointer may be null): block sums int32 [slot][weight row][block], the Q8_0
// bytes of the h rows the down products used [slot][n_ff/32], and the
// expert-major slot grouping of the up_gate kernels (counts [n_expert],
// offsets [n_expert + 1], pairs [slots]).
struct MoeEmit {
    int32_t *sums;
    void *hq;
    int32_t *counts, *offsets, *pairs;
};

// One launch covers n_layers independent layers of the same shape; every
// layer has its own weights, inputs, outputs and workspace.
struct MoeUpGateArgs {
    struct Layer {
        const uint8_t *w;   // [n_expert][2*n_ff][n_embd/32] blocks
        const float *x;     // fp32 [n_tok][n_embd], quantized inside
        const int32_t *ids; // [n_tok][n_used]
        float *h;           // [n_tok][n_used][n_ff]
        void *ws;
    } layer[kMoeMaxLayers];
    int n_layers;
    int64_t n_tok, n_embd, n_ff, n_expert, n_used;
    const MoeEmit *emit = nullptr;     // validation (n_layers == 1)
};

struct MoeDownArgs {
    struct Layer {
        const uint8_t *w;   // [n_expert][n_embd][n_ff/32] blocks
        const float *h;     // [n_tok][n_used][n_ff]
        const int32_t *ids; // [n_tok][n_used]
        const float *cw;    // [n_tok][n_used]
        float *out;         // [n_tok][n_embd]
        void *ws;
    } layer[kMoeMaxLayers];
    int n_layers;
    int64_t n_tok, n_embd, n_ff, n_expert, n_used;
    const MoeEmit *emit = nullptr;     // validation (n_layers == 1)
};

// Validation helpers: fill n int32 with v; offsets[0..n_expert] = exclusive
// prefix of counts.
int launch_fill_i32(int32_t *p, int64_t n, int32_t v, hipStream_t stream);
int launch_route_offsets(const int32_t *counts, int32_t *offsets, int64_t n_expert,
                         hipStream_t stream);

// Workspace (decode path): [0, 256) error word; [256, ...) per-slot down
// outputs fp32 [n_tok*n_used][n_embd].  The prefill path's layout is larger
// (routing tables, quantized rows); moe_ws_bytes covers the path a shape takes.
size_t moe_ws_bytes(int64_t n_tok, int64_t n_embd, int64_t n_ff, int64_t n_expert,
                    int64_t n_used);

int launch_moe_up_gate(const MoeUpGateArgs &a, hipStream_t stream);
int launch_moe_down(const MoeDownArgs &a, hipStream_t stream);
int launch_moe_route(const int32_t *ids, int32_t *counts, int32_t *offsets, int32_t *pairs,
                     int64_t n_tok, int64_t n_expert, int64_t n_used, void *ws,
                     hipStream_t stream);

// out[t] = sum over u ascending of cw[t][u] * yslot[t*n_used+u] (NaN for a
// token with an out-of-range id); one launch.
int launch_moe_combine(const float *yslot, const int32_t *ids, const float *cw, float *out,
                       int64_t n_tok, int64_t n_rows, int64_t n_used, int64_t n_expert,
                       hipStream_t stream);

// The same over several layers of one shape in one launch.
struct MoeCombineLayer {
    const float *yslot;
    const int32_t *ids;
    const float *cw;
    float *out;
};
int launch_moe_combine_layers(const MoeCombineLayer *l, int n_layers, int64_t n_tok,
                              int64_t n_rows, int64_t n_used, int64_t n_expert, hipStream_t stream);

// Prefill path (n_tok > kMoeDecodeMaxTok, K = n_embd and n_ff in multiples of
// 4 blocks): routing + quantization + grouped int8 GEMM per call.
bool moe_prefill_ok(int64_t n_tok, int64_t n_embd, int64_t n_ff, int64_t n_expert, int64_t n_used);
size_t moe_prefill_ws_bytes(int64_t n_tok, int64_t n_embd, int64_t n_ff, int64_t n_expert,
                            int64_t n_used);
// The launch-shape limits of the prefill path's launches: 0 or -4 (unsupported).
int moe_prefill_check(int64_t n_tok, int64_t n_embd, int64_t n_ff, int64_t n_expert,
                      int64_t n_used);
int launch_moe_prefill_up_gate(const uint8_t *w, const float *x, const int32_t *ids, float *h,
                               void *ws, int64_t n_tok, int64_t n_embd, int64_t n_ff,
                               int64_t n_expert, int64_t n_used, hipStream_t stream,
                               const MoeEmit *emit = nullptr);
int launch_moe_prefill_down(const uint8_t *w, const float *h, const int32_t *ids, const float *cw,
                            float *out, void *ws, int64_t n_tok, int64_t n_embd, int64_t n_ff,
                            int64_t n_expert, int64_t n_used, hipStream_t stream,
                            const MoeEmit *emit = nullptr);

// Decode expert FFN over R8 weights (up_gate + SwiGLU, down + combine in two
// launches per call): the combined up_gate tensor repacked as n_expert*2*n_ff
// rows, the down tensor as n_expert*n_embd rows.  Workspace: [0, 256) error
// word, then the quantized h rows [n_tok*n_used][n_ff/32] blocks.
struct MoeR8Layer {
    const void *w_up_gate;
    const void *w_down;
    const float *x;
    const int32_t *ids;
    const float *cw;
    float *h;
    float *out;
    void *ws;
};
bool moe_r8_ok(int64_t n_tok, int64_t n_embd, int64_t n_ff, int64_t n_expert, int64_t n_used);
size_t moe_r8_ws_bytes(int64_t n_tok, int64_t n_embd, int64_t n_ff, int64_t n_expert,
                       int64_t n_used);
bool moe_r8_prefill_path(int64_t n_tok, int64_t n_embd, int64_t n_ff, int64_t n_expert,
                         int64_t n_used);
// More than kMoeDecodeMaxTok tokens over R8 weights (moe_prefill_ok shapes):
// routing, quantization, the two grouped products and the combine of one layer.
// emit_ug / emit_dn: validation outputs of the up_gate and down products.
int launch_moe_r8_prefill(const uint8_t *w_ug, const uint8_t *w_dn, const float *x,
                          const int32_t *ids, const float *cw, float *h, float *out, void *ws,
                          int64_t n_tok, int64_t n_embd, int64_t n_ff, int64_t n_expert,
                          int64_t n_used, hipStream_t stream, const MoeEmit *emit_ug = nullptr,
                          const MoeEmit *emit_dn = nullptr);
// The library's own workspace for callers that cannot allocate
// (moe_r8_ffn_batched_noalloc): a file-scope device array of
// kMoeR8ScratchBytes per device.  moe_r8_scratch sets *base to the current
// device's copy (looked up once per device); 0, or -6 if the lookup fails.
constexpr size_t kMoeR8ScratchBytes = (size_t)48 << 20;
int moe_r8_scratch(uint8_t **base);

// The launch-shape limits of launch_moe_r8_ffn for this shape: 0 or -4.
int moe_r8_ffn_check(int64_t n_tok, int64_t n_embd, int64_t n_ff, int64_t n_expert,
                     int64_t n_used);
// One token, one layer, one launch (moe_r8_ffn_fused): workspace bytes,
// the shape limits (0 or -4), the launch.
size_t moe_r8_fused_ws_bytes(int64_t n_embd, int64_t n_ff, int64_t n_used);
int moe_r8_fused_check(int64_t n_embd, int64_t n_ff, int64_t n_expert, int64_t n_used);
int launch_moe_r8_fused(const MoeR8Layer &l, int64_t n_embd, int64_t n_ff, int64_t n_expert,
                        int64_t n_used, hipStream_t stream);
int launch_moe_r8_ffn(const MoeR8Layer *l, int n_layers, int64_t n_tok, int64_t n_embd,
                      int64_t n_ff, int64_t n_expert, int64_t n_used, hipStream_t stream,
                      const MoeEmit *emit_ug = nullptr, const MoeEmit *emit_dn = nullptr);

}  // namespace q8
