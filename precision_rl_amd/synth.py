"""Seeded synthetic inputs for the W4A4 MoE expert path.

This module draws inputs only: it holds none of the method's arithmetic
(no quantiser, no GEMM, no epilogue).  The tests, the benchmark and the smoke
check use it, and both the HIP path and the FP64 oracle receive the same
arrays from it.  It needs numpy alone.

Workloads (shapes of a Qwen3-30B-A3B MoE layer: H = 2048, I = 768, E = 128,
top-8, as on the pages' learner benchmarks):

  tiny      T=64,    H=256,  E=8,   k=2, I=128   uniform router, forward
  qp        T=16384, H=2048, E=128, k=8          Student-t(3) activations
  fwd       T=8192,  H=2048, E=128, k=8, I=768   uniform router, forward
  skew      T=32768, H=2048, E=128, k=8, I=768   Zipf(1.2) router, 10 empty
  learner   T=16384, H=2048, E=128, k=8, I=768   forward + backward

Recipe: ``numpy.random.Generator(PCG64(SeedSequence(1000 + index)))`` spawned
into independent streams (router, x, W1, W2, dY, popularity).  Normal and
Student-t draws are float32 and rounded to bf16 with round-to-nearest-even;
router weights are float32.  The uniform router takes the softmax of N(0,1)
logits over all experts, keeps the top-k (ties to the lower expert id) and
renormalises over the k.  The skewed router gives 118 experts Zipf weights
r^-1.2 by a seeded rank permutation, gives 10 seeded experts weight 0, picks
k distinct experts per token by Gumbel-top-k on the log-weights and weights
them by a softmax of N(0,1) logits over the chosen k.
"""

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    T: int
    H: int
    E: int
    k: int
    I: int          # 0 for the quantize+permute-only workload
    routing: str    # "uniform" | "zipf"
    x_dist: str     # "normal" | "t3"
    backward: bool


WORKLOADS = {
    "tiny": Workload("tiny", 0, 64, 256, 8, 2, 128, "uniform", "normal", False),
    "qp": Workload("qp", 1, 16384, 2048, 128, 8, 0, "uniform", "t3", False),
    "fwd": Workload("fwd", 2, 8192, 2048, 128, 8, 768, "uniform", "normal", False),
    "skew": Workload("skew", 3, 32768, 2048, 128, 8, 768, "zipf", "normal", False),
    "learner": Workload("learner", 4, 16384, 2048, 128, 8, 768, "uniform", "normal", True),
}

ZIPF_S = 1.2
ZIPF_EMPTY = 10
W_STD = 0.02


def f32_to_bf16_bits(v):
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> 16) & np.uint32(1))
    return (rounded >> 16).astype(np.uint16)


def _streams(seed):
    ss = np.random.SeedSequence(seed)
    names = ("router", "x", "w1", "w2", "dy", "popularity")
    return {n: np.random.Generator(np.random.PCG64(s)) for n, s in zip(names, ss.spawn(len(names)))}


def _softmax(z, axis=-1):
    z = z - z.max(axis=axis, keepdims=True)
    ez = np.exp(z)
    return ez / ez.sum(axis=axis, keepdims=True)


def uniform_router(rng, T, E, k):
    logits = rng.standard_normal((T, E))
    prob = _softmax(logits)
    idx = np.argsort(-prob, axis=1, kind="stable")[:, :k]
    w = np.take_along_axis(prob, idx, axis=1)
    w = w / w.sum(axis=1, keepdims=True)
    return idx.astype(np.int32), w.astype(np.float32)


def zipf_router(rng_router, rng_pop, T, E, k, s=ZIPF_S, n_empty=ZIPF_EMPTY):
    perm = rng_pop.permutation(E)
    weight = np.zeros(E)
    live = perm[n_empty:]
    weight[live] = np.arange(1, live.size + 1, dtype=np.float64) ** -s
    logw = np.where(weight > 0, np.log(np.where(weight > 0, weight, 1.0)), -np.inf)
    idx = np.empty((T, k), dtype=np.int32)
    chunk = 4096
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        keys = logw[None, :] + rng_router.gumbel(size=(t1 - t0, E))
        idx[t0:t1] = np.argsort(-keys, axis=1, kind="stable")[:, :k]
    w = _softmax(rng_router.standard_normal((T, k))).astype(np.float32)
    return idx, w, perm[:n_empty].copy()


def normal_bf16(rng, shape, std=1.0):
    v = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    return f32_to_bf16_bits(v)


def t3_bf16(rng, shape):
    return f32_to_bf16_bits(rng.standard_t(3.0, size=shape).astype(np.float32))


def make_inputs(T, H, E, k, I=0, routing="uniform", x_dist="normal", backward=False,
                seed=1000, weights=True, n_empty=ZIPF_EMPTY):
    """Draw one workload's inputs.  Returns a dict of numpy arrays.

    x, w1, w2, dy are bf16 bit patterns (uint16); topk_idx int32 [T, k];
    topk_w float32 [T, k]; w1 [E, 2I, H]; w2 [E, H, I].
    """
    rs = _streams(seed)
    out = {}
    if routing == "uniform":
        out["topk_idx"], out["topk_w"] = uniform_router(rs["router"], T, E, k)
    elif routing == "zipf":
        if E - n_empty < k:
            raise ValueError("the skewed router needs at least k experts with tokens")
        out["topk_idx"], out["topk_w"], out["empty_experts"] = zipf_router(
            rs["router"], rs["popularity"], T, E, k, n_empty=n_empty)
    else:
        raise ValueError(routing)
    out["x"] = t3_bf16(rs["x"], (T, H)) if x_dist == "t3" else normal_bf16(rs["x"], (T, H))
    if I and weights:
        out["w1"] = normal_bf16(rs["w1"], (E, 2 * I, H), W_STD)
        out["w2"] = normal_bf16(rs["w2"], (E, H, I), W_STD)
    if backward:
        out["dy"] = normal_bf16(rs["dy"], (T, H))
    return out


def workload_inputs(name, weights=True):
    w = WORKLOADS[name]
    return make_inputs(w.T, w.H, w.E, w.k, w.I, w.routing, w.x_dist, w.backward,
                       seed=1000 + w.index, weights=weights)
