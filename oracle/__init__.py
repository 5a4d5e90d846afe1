"""Float64 CPU oracle for causal RoPE attention (forward and backward).

TEST INFRASTRUCTURE, not part of the product: only the test suite, the package
smoke check and the CPU baseline leg of the benchmark may import it. It shares
no code with the HIP path. Every function is pinned by tests that do not call
the oracle's own formulas again (invariants, closed forms, centred finite
differences, brute force and a library routine); see the test suite.
"""

from .attention import (  # noqa: F401
    DEFAULT_BASE,
    attention_backward,
    attention_decode,
    attention_forward,
    attention_probabilities,
    rope,
    rope_frequencies,
)
from .layers import (  # noqa: F401
    DEFAULT_EPS,
    rmsnorm_backward,
    rmsnorm_forward,
    swiglu_backward,
    swiglu_forward,
)
