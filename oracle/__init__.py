"""FP64 CPU oracle for the per-token NVFP4 W4A4 MoE expert path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this package: only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
constant generator with the HIP library; it depends on numpy alone.

Everything is computed in float64 with one explicit round-to-nearest-even per
quantiser Q(.), following the pages:

* miniTE Technical Report, section 5.1 (the block-scale equation): block scale
  d = Q_E4M3(amax(b) / (6 s)), reconstruction x_hat = s d Q_E2M1(x / (s d)).
* rainbus review of the miniTE paper, "method steps" step 4: per-token outer
  scale g = max|X| / (6 * 448), weights "similarly" per row.
* miniTE AI summary, "Methodology in Plain English": outer factors applied in
  FP32 after the block-scaled product, BF16 cast only at the end, Hadamard and
  stochastic rounding off, straight-through BF16 backward on saved operands.

Modules
-------
``nvfp4``  the E2M1 / E4M3 / BF16 codecs and the row quantiser.
``moe``    routing, quantize+permute, the grouped expert forward and the
           straight-through backward (NVFP4; and the forward of the MXFP4
           recipe).
``mxfp4``  the MXFP4 recipe's E8M0 codec and row quantiser (E2M1 elements,
           one power-of-two scale per 32).
``linear`` the dense per-token NVFP4 linear layer.

Parity status: every function here is pinned by tests under ``tests/``
(``-m "not gpu"``) against closed forms, exact rational brute force, worked
examples under ``tests/golden/`` and float64 autograd.  SwiGLU, FC2 and the
unpermute have no printed values on the pages; they are pinned only through
closed forms and the autograd check of their derivatives (see the docstrings
in ``moe``).
"""

from . import nvfp4, mxfp4, moe  # noqa: F401
