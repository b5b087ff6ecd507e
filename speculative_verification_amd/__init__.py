"""MI355X-native ISD (Introspective Strided Decoding) verify-and-propose step.

The computation lives in libisd (HIP kernels for gfx950 behind the C ABI of
include/isd.h); this package only marshals torch tensors into those calls.
"""

from .isd import (  # noqa: F401
    DTYPE_BF16,
    DTYPE_F32,
    MODE_GREEDY,
    MODE_SAMPLE,
    SAMPLER_CDF,
    SAMPLER_GUMBEL,
    IsdError,
    Shape,
    Decoder,
    StepCall,
    alpha,
    check_device_error,
    decode_commit,
    decode_masks,
    gemm_workspace,
    lib,
    lm_head,
    lm_head_pack,
    lm_head_packed,
    lm_head_stats,
    lora_gemm,
    lora_pack,
    make_shape,
    propose,
    propose_masked,
    read_probe,
    set_trunc_tuning,
    set_tuning,
    step,
    step_fused,
    step_masked,
    step_noalloc,
    verify_step,
    workspace,
    workspace_bytes,
)
