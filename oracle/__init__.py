"""Plain fp64 CPU oracle of the large-chunk TTT layer (ZipMap / LaCT).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only the test suite, the package smoke check and the
CPU-baseline leg of the benchmark use it.  It shares no code with the HIP
library (no kernels, headers, tables or helpers) and imports nothing from it.

Every function states the passage of the source pages it follows; see
``ttt_oracle`` for the arithmetic.
"""
from .ttt_oracle import (  # noqa: F401
    sigmoid,
    silu,
    silu_grad,
    swiglu,
    linear_fw,
    vjp_swiglu,
    vjp_linear,
    chunk_gradient,
    gradient_step,
    renorm_rows,
    newton_schulz,
    MUON_NS_COEFFS,
    NS_STEPS,
    update_head,
    apply_head,
    update,
    apply,
    update_apply,
    stream,
    chunked,
    virtual_loss,
    update_rows_sampled,
    rmsnorm,
    output_gate,
    project,
    layer,
    RMS_EPS,
)
