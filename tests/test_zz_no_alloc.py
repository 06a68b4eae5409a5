"""The allocation-free quantize+permute entry point against the one with a
workspace, through the C ABI: bit-identical codes, block scales, outer
scales, expert offsets, row map and source rows, on two calls in a row (the
second with a smaller input, so the library's scratch holds the first call's
counts when it starts), then once more at the first size; and a call whose
routing scratch would exceed the library's is refused before any launch."""
import numpy as np
import pytest

from precision_rl_amd import synth
from gpu_util import bf16_dev, print_case

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _b():
    from precision_rl_amd import binding
    return binding


def _same(a, b, rows):
    assert torch.equal(a["offsets"], b["offsets"])
    assert torch.equal(a["row_map"], b["row_map"])
    assert torch.equal(a["src_row"][:rows], b["src_row"][:rows])
    assert torch.equal(a["codes"][:rows], b["codes"][:rows])
    assert torch.equal(a["scales"][:rows], b["scales"][:rows])
    assert torch.equal(a["outer"][:rows].view(torch.int32), b["outer"][:rows].view(torch.int32))


@pytest.mark.parametrize("A", [1, 16])
def test_noalloc_quantize_permute_matches_the_workspace_call(A):
    b = _b()
    cases = [(16384, 2048, 128, 8, 1101), (3000, 512, 24, 4, 1102), (16384, 2048, 128, 8, 1103)]
    for T, H, E, k, seed in cases:
        d = synth.make_inputs(T, H, E, k, 0, routing="zipf" if seed == 1102 else "uniform", x_dist="t3",
                              seed=seed, n_empty=3)
        print_case("noalloc_quantize_permute", T=T, H=H, E=E, k=k, A=A, seed=seed)
        x = bf16_dev(d["x"], torch)
        idx = torch.from_numpy(d["topk_idx"]).cuda()
        ref = b.w4a4_quantize_permute(x, idx, E, A)
        got = b.w4a4_quantize_permute_noalloc(x, idx, E, A)
        torch.cuda.synchronize()
        rows = int(ref["offsets"][-1].item())
        _same(got, ref, rows)


def test_noalloc_identity_routing_and_empty_batch():
    b = _b()
    w = bf16_dev(synth.normal_bf16(np.random.default_rng(5), (4 * 256, 512), synth.W_STD), torch)
    print_case("noalloc_identity", T=w.shape[0], K=w.shape[1])
    ref = b.w4a4_quantize_permute(w, None, 1)
    got = b.w4a4_quantize_permute_noalloc(w, None, 1)
    torch.cuda.synchronize()
    _same(got, ref, w.shape[0])
    x = torch.zeros((0, 256), dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros((0, 2), dtype=torch.int32, device="cuda")
    got = b.w4a4_quantize_permute_noalloc(x, idx, 8, 1)
    torch.cuda.synchronize()
    assert not got["offsets"].any()


def test_noalloc_refuses_calls_beyond_its_scratch():
    b = _b()
    T, E, k = 524032 + 256, 128, 8   # one routing chunk more than the scratch holds
    x = torch.zeros((T, 16), dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros((T, k), dtype=torch.int32, device="cuda")
    print_case("noalloc_refused", T=T, E=E, k=k)
    with pytest.raises(b.W4A4Error, match="scratch"):
        b.w4a4_quantize_permute_noalloc(x, idx, E, 1)
