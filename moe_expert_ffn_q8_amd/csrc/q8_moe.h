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
};

// Workspace: [0, 256) error word; [256, ...) per-slot down outputs fp32
// [n_tok*n_used][n_embd].
size_t moe_ws_bytes(int64_t n_tok, int64_t n_embd, int64_t n_ff, int64_t n_expert,
                    int64_t n_used);

int launch_moe_up_gate(const MoeUpGateArgs &a, hipStream_t stream);
int launch_moe_down(const MoeDownArgs &a, hipStream_t stream);
int launch_moe_route(const int32_t *ids, int32_t *counts, int32_t *offsets, int32_t *pairs,
                     int64_t n_tok, int64_t n_expert, int64_t n_used, void *ws,
                     hipStream_t stream);

}  // namespace q8
