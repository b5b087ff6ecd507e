"""MI355X-native ISD (Introspective Strided Decoding) verify-and-propose step.

The computation lives in libisd (HIP kernels for gfx950 behind the C ABI of
include/isd.h); this package only marshals torch tensors into those calls.
"""

from .isd import (  # noqa: F401
    DTYPE_BF16,
    DTYPE_F32,
    MODE_GREEDY,
    MODE_SAMPLE,
    IsdError,
    Shape,
    StepCall,
    alpha,
    check_device_error,
    lib,
    lm_head,
    make_shape,
    propose,
    set_tuning,
    step,
    verify_step,
    workspace,
    workspace_bytes,
)
