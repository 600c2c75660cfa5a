"""CPU oracle for the GPT-2 training step (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  The HIP product path
never calls it and shares no code with it.
"""

from .gpt2_oracle import (  # noqa: F401
    OracleConfig,
    param_shapes,
    linear_forward,
    linear_backward,
    layernorm_forward,
    layernorm_backward,
    gelu_tanh,
    gelu_tanh_backward,
    relu2,
    relu2_backward,
    rms_norm_forward,
    rms_norm_backward,
    rope_angles,
    rope_forward,
    rope_backward,
    RMS_EPS,
    ROPE_BASE,
    causal_attention_forward,
    causal_attention_backward,
    softmax_cross_entropy,
    encoder_forward,
    encoder_backward,
    adamw_update,
    gpt2_forward,
    gpt2_backward,
    gpt2_step,
    accumulate_grads,
    global_grad_norm,
    clip_factor,
    gpt2_step_accumulated,
)
from .init_rng import splitmix64_stream, gpt2_init_params  # noqa: F401
from .fp8 import (  # noqa: F401
    E4M3,
    E5M2,
    fp8_decode,
    fp8_encode,
    fp8_linear_backward,
    fp8_linear_forward,
    fp8_matmul_nt,
    fp8_scales,
    quantize,
    round_to_fp8,
)
