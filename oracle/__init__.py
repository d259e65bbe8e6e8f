"""fp64 CPU oracle for Kimi Delta Attention (KDA) -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product path (the HIP library and its Python binding) never
imports, links or calls it, and the two share no code.

Two implementations of the same definition:
  * `kda_oracle.c` (fp64, OpenMP), wrapped here by `gate`, `forward`,
    `decode_step`;
  * a NumPy twin (`gate_np`, `forward_np`, `decode_step_np`) for small cases;
  * `backward_np`: the reverse mode of the same token loop (gradients of
    <o, do> + <S_T, dS_T> with respect to q, k, v, g, beta and S_0), pinned by
    central finite differences of `forward_np`.

The definition they follow ("Kimi K3 internal structure analysis", section
"Sequence mixing: 3 KDA layers per global MLA layer"; recurrence as written in
the C file's header):
    g = -5 * sigmoid(exp(A) * z),  alpha = exp(g)
    S' = Diag(alpha_t) S_{t-1}                 (retention before the write)
    u_t = beta_t (v_t - S'^T k_t),  S_t = S' + k_t u_t^T   (delta rule)
    o_t = S_t^T q_t

Pins: every function here is checked by the `-m "not gpu"` tests against closed
forms, brute-force unrolled products and invariants; see tests/test_oracle_*.py.
"""
from .core import (  # noqa: F401
    GMIN,
    RhoAccumulator,
    TILE,
    backward_np,
    build_oracle,
    decode_step,
    decode_step_np,
    forward,
    forward_np,
    gate,
    gate_backward_np,
    gate_np,
    max_threads,
    rho,
    tile_log_decay_sums,
)
