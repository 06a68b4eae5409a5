"""The per-expert composition of the oracle that the full-size GPU tests use
(tests/oracle_by_expert.py) against the oracle's whole-layer forward and
backward, on the CPU: every token's y and dX, every expert's dW1 and dW2 and
every row's pre-cast FC1 value and FC2-input codes must agree (bit for bit
after the bf16 roundings; the FP64 sums over a token's k slots run in another
order, which can move a value by an FP64 ulp, never a bf16 one here)."""
import numpy as np
import pytest

from oracle import moe, nvfp4 as q
from precision_rl_amd import synth

import oracle_by_expert as obe

pytestmark = pytest.mark.cpu


@pytest.mark.parametrize("routing,n_empty", [("uniform", 0), ("zipf", 2)])
def test_per_expert_layer_equals_the_whole_layer(routing, n_empty):
    T, H, E, k, I = 96, 256, 7, 3, 128
    d = synth.make_inputs(T, H, E, k, I, routing=routing, backward=True, seed=41, n_empty=n_empty)
    x = q.bf16_bits_to_f64(d["x"])
    w1 = q.bf16_bits_to_f64(d["w1"])
    w2 = q.bf16_bits_to_f64(d["w2"])
    ref = moe.forward(x, d["topk_idx"], d["topk_w"], moe.quantize_weights(w1), moe.quantize_weights(w2), E)
    xq = ref["xq"]
    rb = moe.backward(q.bf16_bits_to_f64(d["dy"]), x, w1, w2, ref["h"], ref["a"], d["topk_w"], xq["offsets"],
                      xq["row_map"], xq["src_row"])
    got = obe.layer(d, E, backward=True, want_rows=True, n_workers=2)
    assert np.array_equal(got["y"], ref["y"])
    assert np.array_equal(got["dX"], rb["dX"])
    assert np.array_equal(got["dW1"], rb["dW1"])
    assert np.array_equal(got["dW2"], rb["dW2"])
    off = xq["offsets"]
    for e in range(E):
        r0, r1 = off[e], off[e + 1]
        assert np.array_equal(got["h64"][e], ref["h64"][r0:r1])
        assert np.array_equal(got["a_codes"][e], ref["a_codes"][r0:r1])
        assert np.array_equal(got["a"][e], ref["a"][r0:r1])
    if n_empty:
        empty = np.diff(off) == 0
        assert empty.any() and not got["dW1"][empty].any()
