"""Dense per-token NVFP4 linear layer: forward and straight-through BF16 backward (oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

The pages' module layer has ordinary linear layers beside the MoE grouped
ones, behind the same quantisation interface (miniTE Technical Report,
section 4.1; layer table of section 4.2).  With the nvfp4_per_token recipe
(section 4.3) the activation outer scale is per token and the weight outer
scale per output row; the outer factors apply in the FP32 epilogue after the
block-scaled product and the output is cast to BF16 once (section 5.1).  The
backward is the BF16 layer bypass on the saved original operands (section
4.3).  Everything here is float64; BF16 roundings sit where the GPU path
stores BF16 tensors.
"""

import numpy as np

from . import nvfp4 as q


def forward(x, w):
    """y = x W^T for x [T, K] and W [N, K] (float64 holding bf16 values).

    Both operands are quantised per row (quantize_rows); then
        pre[t, n] = g_x[t] g_w[n] sum_k (d c)_x[t, k] (d c)_w[n, k]
    and y = bf16(pre).  Returns dict(xq, wq, pre, y); xq / wq are
    (codes, scales, outer) as quantize_rows returns them.
    """
    xq = q.quantize_rows(np.asarray(x, dtype=np.float64))
    wq = q.quantize_rows(np.asarray(w, dtype=np.float64))
    acc = q.block_values(xq[0], xq[1]) @ q.block_values(wq[0], wq[1]).T
    pre = acc * xq[2].astype(np.float64)[:, None] * wq[2].astype(np.float64)[None, :]
    return dict(xq=xq, wq=wq, pre=pre, y=q.round_bf16(pre))


def backward(dy, x, w, rnd=True):
    """Straight-through backward of ``forward`` (the quantisers as identity):
    dX = dY W [T, K], dW = dY^T X [N, K]; each rounded to bf16 when ``rnd``
    (READING: as the MoE path, BF16 outputs from FP32 accumulation)."""
    R = q.round_bf16 if rnd else (lambda v: v)
    dy = np.asarray(dy, dtype=np.float64)
    return dict(dX=R(dy @ np.asarray(w, dtype=np.float64)),
                dW=R(dy.T @ np.asarray(x, dtype=np.float64)))
