"""MI355X (gfx950) hot path of quantization-based self-speculative decoding.

One packed INT4 weight buffer serves a W4A4 drafter and a W4A16 verifier; a
verify step accepts or rewrites the drafted tokens.  Every step runs in the
hand-written HIP kernels of ``libqspec.so`` (C ABI in ``include/qspec.h``);
this package only marshals torch tensors (device memory and streams) into
those calls.  There is no CPU fallback: if the library is missing the calls
raise.  ``e2e.Decoder`` runs greedy self-speculative decoding of a whole
decoder on these calls (decoder kernels in ``include/qspec_harness.h``).
"""

from .binding import (  # noqa: F401
    QSpecError,
    lib,
    lib_path,
    pack_w4,
    padded_rows,
    quant_act,
    quant_act_rot,
    rotate_w,
    rotate_x,
    gemm_w4a4,
    gemm_w4a4_bf16,
    gemm_w4a8,
    quant_act8,
    gemm_w4a16,
    gemm_w4a16_swiglu,
    gemm_w4a4_swiglu,
    gemm_w4a8_swiglu,
    gemm_family,
    pair_rows,
    verify,
    verify_noalloc,
    workspace_bytes,
    OP_GEMM_W4A4,
    OP_GEMM_W4A16,
    OP_GEMM_W4A8,
    GEMM_AUTO,
    GEMM_GEMV,
    GEMM_SKINNY,
    GEMM_TILED,
    GEMM_STREAM,
    VERIFY_GREEDY,
    VERIFY_SAMPLE,
    embed,
    add_rmsnorm,
    rope_kv,
    attention,
    rope_attention,
    silu_mul,
    silu_mul_pairs,
    add_rmsnorm_quant,
    add_rmsnorm_quant8,
    argmax,
    spec_prepare,
    spec_commit,
)
