"""CPU oracle for the stabilized parallel mLSTM forward pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The GPU library never routes through it, and it shares no code with
the HIP path: its only inputs are plain NumPy arrays.

Every function follows "xLSTM: Extended Long Short-Term Memory", Appendix A.3
("Parallel mLSTM Forward Pass", Eqs. 71-78, and the stabilized forward summary
at the start of "Parallel mLSTM Backward Pass", Eqs. 79-86, with the log forget
gate matrix of Eq. 101), in float64 unless a caller asks for float32 (an
error-floor instrument, never the reference).

Parity status of each function (what pins it, in ``tests/test_oracle_pins.py``):

* ``forward_stabilized``   pinned: equals the recurrent form (``forward_recurrent``)
  and the unstabilized form (``forward_unstabilized``), exact rational worked
  examples, causal linear attention and geometric-decay special cases, the
  T = 1 closed form, and the input-gate shift identity.
* ``forward_rows``         pinned: row-by-row equal to ``forward_stabilized``
  and to the exact rational examples.
* ``forward_recurrent``    pinned: exact rational examples (independent of the
  parallel forms), and the normalizer identity n_i = exp(-m_i) max(|n_i.q_i|, 1).
* ``forward_unstabilized`` pinned: exact rational examples.
* ``gate_matrices``        pinned: F_ii = 1, zero above the diagonal, explicit
  products, log F = -inf / 0 / partial sums (Eqs. 71, 72, 101).
* ``recurrent_step_stabilized`` / ``forward_recurrent_stabilized``  pinned:
  h equals the unstabilized recurrent form, m and the normalizer equal the
  parallel form's m and n, and exp(m_T) times the final states equals their
  definition as gate-weighted sums of v k^T and k (brute force on tiny
  inputs), also where exp(i~) overflows the unstabilized form.
* ``backward_stabilized``  pinned: central finite differences of
  ``forward_stabilized`` for every input (q, k, v, i~, f~), on inputs with
  rows on both sides of the normalizer floor, and the derivative identity
  d/dx log sigma(x) = sigma(-x) (Eq. 104).
* every function above takes ``forget="sigmoid"`` (default) or ``"exp"``:
  the exponential forget gate is pinned the same way (all forms agree, the
  closed form of F, finite differences of the backward).
* ``output_gate``          pinned: sigma(0) = 1/2 and sigma(-x) = 1 - sigma(x)
  closed forms (Eq. 78).
"""

from .mlstm import (  # noqa: F401
    log_sigmoid,
    forget_gate,
    log_forget,
    FORGET_ACTIVATIONS,
    gate_matrices,
    log_gate_matrix,
    forward_stabilized,
    forward_rows,
    forward_recurrent,
    recurrent_step_stabilized,
    forward_recurrent_stabilized,
    forward_unstabilized,
    output_gate,
    backward_stabilized,
)
