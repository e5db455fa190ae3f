"""CPU oracle of the MoE FFN layer forward -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import or run anything in this package.  The product path (the HIP
library and its binding) never imports it and shares no code with it.

Contents:

* ``codec``  -- bf16 and OCP e4m3fn encode/decode and the fp8 block rule;
* ``layer``  -- the layer in fp64, one function per step (router product,
  gating, top-k, permutation, SwiGLU experts, shared expert, combine);
* ``dense``  -- brute-force dense evaluation (every expert on every token,
  masked by the top-k gate weights), used to pin ``layer`` on tiny inputs.

Pins (``tests/test_oracle_*.py``): the codecs against their closed-form
definitions, brute-force nearest-value search and torch's casts; gating
against closed forms and special cases; the permutation against
``np.argsort(kind="stable")`` and round-trip invariants; the whole layer
against ``dense`` and against textbook reductions (one expert, k = 1 ->
plain SwiGLU MLP) and symmetries (token permutation, expert relabelling,
scaling of w2).  Absolute layer outputs at the large shapes are parity
unpinned beyond these: the pages print no worked example.
"""
from .layer import LayerSpec, forward  # noqa: F401
