"""The FP64 oracle over a whole layer, one expert at a time (test helper).

A dispatched row's forward outputs (h, a, its FC2-input encoding, o) and its
backward rows (dO, dH, dXp) depend only on that row and its expert's weights,
and an expert's dW only on the rows routed to it.  So the oracle of a full
layer is the oracle of E sub-problems -- expert e with its tokens in
ascending order, k = 1, router weight of the slot that chose e -- whose row
results go back to the full layer's rows, plus the two sums over a token's
k slots (y and dX), accumulated in FP64 and rounded to bf16 once, as the
oracle's unpermute and gather-sum do.  The sub-problems run in a pool of
freshly started worker processes (numpy only; nothing here touches the
GPU), so peak memory stays at a few experts' sub-problems plus the [T, H]
accumulators.
"""
import concurrent.futures as cf
import multiprocessing as mp
import os

import numpy as np

from oracle import moe, nvfp4 as q


def _bf16_bits(v):
    """float64 values that are bf16 -> their bit patterns (exact)."""
    return q.f64_to_bf16_bits(v)


def _worker_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover
        pass


def _expert(task):
    """One expert's sub-problem.  Row results return as bf16 bit patterns
    (every one of them is a bf16 value), pre-cast FC1 values as float64."""
    e, xb, pe, w1b, w2b, dyb, want_rows = task
    x = q.bf16_bits_to_f64(xb)
    w1 = q.bf16_bits_to_f64(w1b)
    w2 = q.bf16_bits_to_f64(w2b)
    sub_idx = np.zeros((x.shape[0], 1), np.int32)
    f = moe.forward(x, sub_idx, pe, moe.quantize_weights(w1), moe.quantize_weights(w2), 1)
    res = {"e": e, "o": _bf16_bits(f["o"])}
    if want_rows:
        res.update(h64=f["h64"], a_codes=f["a_codes"].astype(np.uint8), a=_bf16_bits(f["a"]))
    if dyb is not None:
        xq = f["xq"]
        rb = moe.backward(q.bf16_bits_to_f64(dyb), x, w1, w2, f["h"], f["a"], pe, xq["offsets"],
                          xq["row_map"], xq["src_row"])
        res.update(dXp=_bf16_bits(rb["dXp"]), dW1=_bf16_bits(rb["dW1"][0]), dW2=_bf16_bits(rb["dW2"][0]))
    return res


def workers():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def layer(d, E, backward=False, want_rows=False, n_workers=None):
    """Oracle results of the layer in `d` (synth.make_inputs arrays).

    Returns dict(y [T, H], and with `backward` dX [T, H], dW1 [E, 2I, H],
    dW2 [E, H, I] (float64); with `want_rows`, per expert (lists indexed by
    expert, rows in the expert's order) the pre-cast FC1 values h64, the
    FC2-input codes a_codes and the bf16 a."""
    idx = np.asarray(d["topk_idx"])
    T, k = idx.shape
    H = d["x"].shape[1]
    I = d["w1"].shape[1] // 2
    p = np.asarray(d["topk_w"])
    tasks, toks = [], {}
    for e in range(E):
        tok, slot = np.nonzero(idx == e)            # ascending tokens: the route's stable order
        toks[e] = tok
        if tok.size:
            tasks.append((e, d["x"][tok], p[tok, slot][:, None].copy(), d["w1"][e:e + 1], d["w2"][e:e + 1],
                          d["dy"][tok] if backward else None, want_rows))
    # largest experts first, so that the pool's tail is short
    tasks.sort(key=lambda t: -t[1].shape[0])
    y_acc = np.zeros((T, H))
    out = {}
    if backward:
        dx_acc = np.zeros((T, H))
        out["dW1"] = np.zeros((E, 2 * I, H))
        out["dW2"] = np.zeros((E, H, I))
    if want_rows:
        out["h64"] = [np.zeros((0, 2 * I))] * E
        out["a_codes"] = [np.zeros((0, I), np.uint8)] * E
        out["a"] = [np.zeros((0, I))] * E
    ctx = mp.get_context("spawn")
    with cf.ProcessPoolExecutor(max_workers=n_workers or workers(), mp_context=ctx,
                                initializer=_worker_init) as ex:
        for r in ex.map(_expert, tasks):
            e = r["e"]
            tok = toks[e]
            pe = p[tok, np.nonzero(idx[tok] == e)[1]].astype(np.float64)[:, None]
            y_acc[tok] += pe * q.bf16_bits_to_f64(r["o"])
            if want_rows:
                out["h64"][e] = r["h64"]
                out["a_codes"][e] = r["a_codes"]
                out["a"][e] = q.bf16_bits_to_f64(r["a"])
            if backward:
                dx_acc[tok] += q.bf16_bits_to_f64(r["dXp"])
                out["dW1"][e] = q.bf16_bits_to_f64(r["dW1"])
                out["dW2"][e] = q.bf16_bits_to_f64(r["dW2"])
    out["y"] = q.round_bf16(y_acc)
    if backward:
        out["dX"] = q.round_bf16(dx_acc)
    return out
