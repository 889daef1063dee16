"""CPU oracle for the gated delta rule and the mLSTM cell — TEST INFRASTRUCTURE.

Plain, slow, float64 numpy code that states what the GPU library must compute.
Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
it; the library itself never does, and the two share no code.

Sources (cited by page title and section/equation):

* "Muir: Linear Attention with Sensitivity-Allocated Gating and Matched-Filter
  Readout" — §2.1 eq.(1) (the GDN-2 state update and readout), §2.2 (effective
  write, GLA form, chunkwise form), §4.2 stage (i) and eq.(10) (the chunk
  matrix T = I + L_strict and the chunkwise readout and state update, used to
  measure how ill-conditioned the tests' chunk systems are).
* the same page, §4.2 "Custom Backward Pass": gradients of a scalar loss
  through eq.(1) (float64 reverse-mode differentiation of the step, pinned by
  finite differences and closed forms).
* the same page, §2.1 (gate parameterisation) and §4.1 eq.(8)-(9): the Muir
  gate prologue (gates from logits, readout with the gain-modulated query).
* "Exponential gates and matrix memory: xLSTM and RWKV-7" — §13.3 and the
  solution to Exercise 13.5: RWKV-7's generalized delta rule (free removal
  direction, decoupled write key), pinned by the page's eviction demo.
* the same page — §13.2 (spectrum of
  the diagonal-plus-rank-one transition, Prop. 13.1 and Exercise 13.4), §13.3
  (reduction to Gated DeltaNet), §13.4 and Exercise 13.6 (mLSTM cell, log-domain
  stabilizer).

Orientation: the state is ``S[d_k, d_v]`` acted on from the left and read as
``o = q S`` (row vectors), as in the Muir page. The xLSTM page writes the
transpose (``S[d_v, d_k]`` read as ``S q``); the two are transposes of each
other.

Pinning status: every function here is checked by ``tests/test_oracle_*.py``
against closed forms, special cases and exact rational brute force. The pages
print no worked numeric GDN-2 example, so absolute GDN-2 outputs on random
inputs are pinned only through those checks. The mLSTM overflow-cliff figures
printed on the xLSTM page (peak 5.9e303, 50% NaN, peak 2.5) depend on companion
inputs the page does not print: parity unpinned for those three values; the
checks use the qualitative behaviour instead.
"""
from .gdn2 import (  # noqa: F401
    gdn2_recurrent, gdn2_step, gdn2_transition, gdn2_materialized,
    gdn2_effective_write, gdn2_decode, delta_rule_textbook, gated_deltanet,
    gla_closed_form, linear_attention_closed_form, bruteforce_exact,
    gdn2_chunk_system, gdn2_chunkwise, chunk_condition_numbers,
)
from .gdn2_grad import gdn2_grad  # noqa: F401
from .rwkv7 import rwkv7_recurrent, rwkv7_decode, rwkv7_materialized  # noqa: F401
from .muir import (  # noqa: F401
    muir_gates, muir_recurrent, muir_decode,
)
from .mlstm import (  # noqa: F401
    mlstm_stabilized, mlstm_naive, mlstm_with_stabilizer, stabilizer_closed_form,
    log_sigmoid,
)
from .spectrum import (  # noqa: F401
    generalized_transition, scalar_diagonal_spectrum, secular_residual,
    symmetrized_transition,
)
