"""ffn-mi355x: the forward hot path of a Llama-style dense SwiGLU FFN block
(fused residual RMSNorm, per-tensor e4m3 quantisation, fused gate+up with
SwiGLU, down projection) and its FP8 single-token decode, as hand-written HIP
kernels for MI355X (gfx950) behind the C ABI of ``include/ffn.h``.

The binding functions (``ffn_rmsnorm_fwd``, ``ffn_quant_absmax``,
``ffn_quant_rows``, ``ffn_gateup``, ``ffn_gateup_swiglu_quant``, ``ffn_swiglu``,
``ffn_down``,
``ffn_decode_gemv``, its arms ``ffn_decode_gemv_arm``, its bf16-weight form
``ffn_decode_gemv_bf16``, and ``bind_decode_gemv``, its checked-once form) live in
``binding``; accessing any of them here loads
``libffn.so`` and raises if it has not been built.  ``workloads`` (seeded
synthetic inputs) and ``build`` import without the library.
"""

_BINDING_NAMES = {
    "ffn_rmsnorm_fwd", "ffn_quant_absmax", "ffn_quant_rows", "ffn_gateup", "ffn_gateup_swiglu_quant",
    "ffn_swiglu", "ffn_down", "ffn_rmsnorm_fwd_acc", "ffn_quant_absmax_clear", "ffn_gateup_acc",
    "ffn_decode_gemv", "ffn_decode_gemv_arm", "ffn_decode_gemv_bf16", "bind_decode_gemv",
    "bind_decode_gemv_arm", "bind_decode_gemv_bf16", "ffn_decode_pack_weight", "ffn_decode_packed_workspace_bytes",
    "ffn_decode_gemv_packed", "bind_decode_gemv_packed", "ffn_decode_noalloc_scratch_bytes",
    "ffn_decode_gemv_packed_noalloc",
    "ffn_matmul_tn", "ffn_matmul_tn_swiglu_bwd", "ffn_transpose", "ffn_quant_transpose", "ffn_swiglu_bwd", "ffn_rmsnorm_bwd",
    "ffn_rmsnorm_bwd_scratch_bytes", "ffn_matmul_tn_swiglu_bwd_acc", "ffn_quant_transpose_clear", "ffn_swiglu_bwd_acc",
    "ffn_rmsnorm_bwd_acc", "ffn_tile_bytes", "ffn_tile_pack", "ffn_quant_absmax_clear_tiled", "ffn_gateup_acc_tiled",
    "ffn_gateup_swiglu_quant_tiled", "ffn_down_tiled", "ffn_rmsnorm_fwd_tiled", "ffn_gateup_tiled_bf16",
    "ffn_down_tiled_bf16", "ffn_transpose_tiled", "ffn_quant_transpose_tiled", "FFN_TN_TILED",
    "FFN_DECODE_SPLIT_SILU", "FFN_DECODE_SILU_INPUT", "FFN_DECODE_PER_PROJECTION", "FFNError", "FFN_BF16", "FFN_E4M3", "FFN_E5M2", "FFN_TN_ACCUMULATE", "FFN_TN_TILE_GRID", "FFN_OK", "FFN_ERR_INVALID",
    "FFN_ERR_UNSUPPORTED", "FFN_ERR_HIP", "version", "last_error", "LIB_PATH",
}


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
