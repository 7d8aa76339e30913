"""CPU oracle for sink attention (float64, NumPy).

TEST INFRASTRUCTURE ONLY: imported by the test suite, by the package smoke
check and by the benchmark's CPU-baseline leg, never by the product path.
It shares no code with the HIP kernels or their C-ABI; the only code both
sides use is the seeded input generator in ``synthetic``.

Pins (all in tests/test_oracle_pins.py, CPU only):
  forward, backward  -> torch SDPA (CPU, float64) with the sink emulated as an
                        extra key column, incl. GQA, window and its autograd;
                        central finite differences; closed forms (S -> -inf,
                        S -> +inf, q = 0, length 1, window 1); invariants
                        (varlen packing, GQA == repeated MHA, window >= L).
  forward_rows, backward_rows, backward_keys
                     -> equal to the corresponding entries of forward/backward.
No function here is "parity unpinned".
"""
from .sink_attention import (  # noqa: F401
    backward,
    backward_keys,
    backward_rows,
    forward,
    forward_rows,
    kv_head_of,
    visible_key_range,
)
