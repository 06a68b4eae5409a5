"""Helpers for the GPU parity tests: host<->device conversion and metrics."""
import numpy as np

from oracle import nvfp4 as q


def rel_l2(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def bf16_dev(bits, torch):
    """uint16 bf16 bit patterns (numpy) -> torch.bfloat16 CUDA tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def bf16_host(t):
    """torch bf16 tensor -> float64 numpy (exact)."""
    import torch
    return q.bf16_bits_to_f64(t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16))


def u8(t):
    return t.detach().cpu().numpy()


def f32_bits(t):
    return t.detach().cpu().numpy().view(np.uint32)


def print_case(name, **kw):
    """Names the case on stdout before a GPU step (flushed)."""
    print(f"[case] {name} " + " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)
