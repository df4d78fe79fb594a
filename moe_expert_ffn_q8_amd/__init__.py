"""moe_expert_ffn_q8_amd: Q8_0 decode matvec and MoE expert FFN for MI355X (gfx950).

The product is libq8moe.so (hand-written HIP kernels behind a C ABI, declared
in include/q8moe.h); this package is its thin Python binding.  Importing it
fails if the library has not been built: there is no CPU fallback.
"""
from ._lib import (BLOCK_BYTES, EXPORTS, LIB_PATH, QK, MoeDownDesc, MoeUpGateDesc, Q8Error,
                   Q8MatmulDesc, Q8MatmulF32Desc, Q8UpGateDesc, make_desc, make_f32_desc,
                   make_up_gate_desc, q8_0_up_gate_swiglu_batched, moe_down_combine, moe_down_combine_batched,
                   moe_error_word, moe_route, q8v_moe_up_gate, q8v_moe_hq, q8v_moe_r8_ffn, moe_up_gate_swiglu, moe_up_gate_swiglu_batched,
                   moe_workspace, moe_workspace_bytes, q8_0_matmul, q8_0_matmul_batched,
                   q8_0_matmul_blocksums, q8v_matvec_r8_batched_blocksums, q8v_matvec_r8_f32_batched_blocksums, q8v_matmul_r8_batched_blocksums, q8_0_matmul_f32_batched, q8_0_matmul_f32_step,
                   q8_0_matmul_f32_step_workspace, q8_0_matmul_f32_step_ws_bytes, q8_0_matvec,
                   q8_0_matvec_r8, q8_0_matvec_r8_batched, make_r8_desc, Q8R8Desc,
                   q8_0_matvec_r8_f32_batched, make_r8_f32_desc, Q8R8F32Desc,
                   q8_1_quantize_rows, kq_matvec, kq_matvec_batched, make_kq_desc, KqMatvecDesc,
                   q8_0_matmul_r8_batched, make_r8_mm_desc, Q8R8MmDesc,
                   moe_r8_workspace, moe_r8_ffn_batched, moe_r8_ffn_batched_noalloc, moe_r8_fused_workspace, moe_r8_ffn_fused, MoeR8FfnDesc, q8_0_quantize_rows, q8_0_r8_bytes, q8_0_repack_r8, q8_empty, q8_read_probe, raw, status_str, version)

__all__ = ["BLOCK_BYTES", "EXPORTS", "LIB_PATH", "QK", "MoeDownDesc", "MoeUpGateDesc", "Q8Error",
           "Q8MatmulDesc", "Q8MatmulF32Desc", "Q8UpGateDesc", "make_desc", "make_f32_desc",
           "make_up_gate_desc", "q8_0_up_gate_swiglu_batched", "moe_down_combine", "moe_down_combine_batched",
           "moe_error_word", "moe_route", "q8v_moe_up_gate", "q8v_moe_hq", "q8v_moe_r8_ffn", "moe_up_gate_swiglu", "moe_up_gate_swiglu_batched",
           "moe_workspace", "moe_workspace_bytes", "q8_0_matmul", "q8_0_matmul_batched",
           "q8_0_matmul_blocksums", "q8v_matvec_r8_batched_blocksums", "q8v_matvec_r8_f32_batched_blocksums", "q8v_matmul_r8_batched_blocksums", "q8_0_matmul_f32_batched", "q8_0_matmul_f32_step",
           "q8_0_matmul_f32_step_workspace", "q8_0_matmul_f32_step_ws_bytes", "q8_0_matvec",
           "q8_0_matvec_r8", "q8_0_matvec_r8_batched", "make_r8_desc", "Q8R8Desc",
           "q8_0_matvec_r8_f32_batched", "make_r8_f32_desc", "Q8R8F32Desc",
           "q8_1_quantize_rows", "kq_matvec", "kq_matvec_batched", "make_kq_desc", "KqMatvecDesc",
           "q8_0_matmul_r8_batched", "make_r8_mm_desc", "Q8R8MmDesc",
           "moe_r8_workspace", "moe_r8_ffn_batched", "moe_r8_ffn_batched_noalloc", "moe_r8_fused_workspace", "moe_r8_ffn_fused", "MoeR8FfnDesc", "q8_0_quantize_rows", "q8_0_r8_bytes", "q8_0_repack_r8", "q8_empty", "q8_read_probe", "raw",
           "status_str", "version"]
