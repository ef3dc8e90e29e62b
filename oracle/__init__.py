"""CPU oracle for the Llama-3 decoder block (TEST INFRASTRUCTURE ONLY).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg import
this package.  The product path (dense_decoder_only_amd) never does, and the
two share no code: only the seeded input generators in `workloads` serve both.
"""
from .block import (  # noqa: F401
    block_forward,
    block_param_counts,
    expected_weight_shapes,
    rmsnorm,
    rope_inv_freq,
    rope_angles,
    rope_cos_sin,
    apply_rope,
    attention,
    silu,
    swiglu,
    to64,
)
from .model import embed, model_forward, model_param_counts  # noqa: F401,E402
