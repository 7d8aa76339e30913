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
  forward_rows, backward_rows, backward_keys, backward_keys_blocked
                     -> equal to the corresponding entries of forward/backward,
                        and (backward_keys_blocked) to the SDPA reference's
                        dK, dV and dS directly.
  gather_paged, forward_paged
                     -> a paged cache holding whole sequences with q_len ==
                        kv_len equals forward; new tokens at the end of a
                        cached context equal the last rows of forward over the
                        whole sequence; page order does not matter; a length-1
                        context gives the one-key closed form.
  token_logps, token_logps_grad (oracle/token_logps.py)
                     -> torch log_softmax + gather in float64 and its autograd;
                        constant rows give -ln V; a per-row shift changes
                        nothing; the gradient rows sum to zero; finite
                        differences.
No function here is "parity unpinned".
"""
from .sink_attention import (  # noqa: F401
    backward,
    backward_keys,
    backward_keys_blocked,
    backward_rows,
    forward,
    forward_paged,
    forward_rows,
    gather_paged,
    kv_head_of,
    visible_key_range,
)
from .token_logps import token_logps, token_logps_grad  # noqa: F401
