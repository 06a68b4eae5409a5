"""Routing, quantize+permute, grouped expert forward and STE backward (oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Notation: T tokens, H hidden, E experts, k experts per token, I SwiGLU width,
A row alignment of each expert group.  Expert e's FC1 weight W1[e] is [2I, H]
(rows 0..I-1 are the gate half, rows I..2I-1 the up half); its FC2 weight
W2[e] is [H, I].  All arithmetic is float64; the BF16 roundings sit exactly
where the GPU path stores BF16 tensors.

The pages (rainbus review, "prerequisites: MoE and grouped GEMM"; AI summary,
"Methodology in Plain English"; miniTE Technical Report, section 5.1) fix:
per-token activation outer scales, per-row weight outer scales, expert FFN
FC1 -> SwiGLU -> FC2 over ragged, possibly empty expert groups with
device-side offsets, FP32 epilogue rescaling by g_x * g_w after the block-scaled
product, BF16 only at the end, and a straight-through BF16 backward on the
saved high-precision operands.  Points they leave open are marked READING.
"""

import numpy as np

from . import mxfp4 as mx
from . import nvfp4 as q


# ---------------------------------------------------------------------------
# Routing.
# ---------------------------------------------------------------------------
def rows_capacity(T, k, E, row_align):
    """Upper bound on the padded dispatched-row count: T*k + E*(A-1)."""
    return T * k + E * (row_align - 1)


def route(topk_idx, E, row_align=1):
    """Expert-contiguous row assignment.

    READING (the rainbus review's method step 6 only says "sort" and
    "padding carries statistics"; padding strategy is an implementation
    freedom): rows of expert e are its tokens in ascending token order,
    starting at off[e]; each group is padded to a multiple of ``row_align``;
    pad rows have src_row = -1.

    Returns (offsets int32 [E+1], row_map int32 [T, k], src_row int32 [off[E]]).
    """
    topk_idx = np.asarray(topk_idx, dtype=np.int64)
    T, k = topk_idx.shape
    counts = np.zeros(E, dtype=np.int64)
    for e in topk_idx.reshape(-1):
        counts[e] += 1
    padded = (counts + row_align - 1) // row_align * row_align
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(padded)
    row_map = np.empty((T, k), dtype=np.int64)
    src_row = np.full(offsets[E], -1, dtype=np.int64)
    fill = offsets[:E].copy()
    for t in range(T):                       # ascending token order = stable
        for j in range(k):
            e = topk_idx[t, j]
            row_map[t, j] = fill[e]
            src_row[fill[e]] = t
            fill[e] += 1
    return offsets.astype(np.int32), row_map.astype(np.int32), src_row.astype(np.int32)


def route_fast(topk_idx, E, row_align=1):
    """Same result as ``route`` via vectorised numpy (for large T)."""
    topk_idx = np.asarray(topk_idx, dtype=np.int64)
    T, k = topk_idx.shape
    flat = topk_idx.reshape(-1)
    counts = np.bincount(flat, minlength=E)
    padded = (counts + row_align - 1) // row_align * row_align
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(padded)
    order = np.argsort(flat, kind="stable")          # entries grouped by expert, t ascending
    starts = np.zeros(E + 1, dtype=np.int64)
    starts[1:] = np.cumsum(counts)
    e_sorted = flat[order]
    rank = np.arange(flat.size) - starts[e_sorted]
    rows = offsets[e_sorted] + rank
    row_map = np.empty(flat.size, dtype=np.int64)
    row_map[order] = rows
    src_row = np.full(offsets[E], -1, dtype=np.int64)
    src_row[rows] = order // k
    return offsets.astype(np.int32), row_map.reshape(T, k).astype(np.int32), src_row.astype(np.int32)


# ---------------------------------------------------------------------------
# Quantize + permute (per-token amax, encode, scatter).
# ---------------------------------------------------------------------------
def quantize_permute(x, topk_idx, E, row_align=1, routed=None, group_rows=1):
    """Per-token NVFP4 of x, written to every destination row of the token.

    The amax is per token (per dispatched row; the k copies of a token are
    identical because the scale domain is the row), as in the rainbus
    review's method step 4.  Pad rows get codes 0, scales 0 and g = 0.
    With ``group_rows`` > 1 the outer scale is shared by groups of that many
    consecutive tokens (group_rows = T: the per-tensor variant);
    see nvfp4.quantize_rows_grouped.

    Returns dict(codes [rows, K] unpacked, packed [rows, K/2], scales
    [rows, K/16], outer [rows], offsets, row_map, src_row).
    """
    x = np.asarray(x, dtype=np.float64)
    if routed is None:
        routed = route_fast(topk_idx, E, row_align)
    offsets, row_map, src_row = routed
    rows = int(offsets[-1])
    T, K = x.shape
    tc, ts, tg = q.quantize_rows_grouped(x, group_rows)   # token rows; copies share them
    codes = np.zeros((rows, K), dtype=np.uint8)
    scales = np.zeros((rows, K // q.BLOCK), dtype=np.uint8)
    outer = np.zeros(rows, dtype=np.float32)
    live = src_row >= 0
    codes[live] = tc[src_row[live]]
    scales[live] = ts[src_row[live]]
    outer[live] = tg[src_row[live]]
    return dict(codes=codes, packed=q.pack_codes(codes), scales=scales, outer=outer,
                offsets=offsets, row_map=row_map, src_row=src_row)


def quantize_weights(w, per_expert=False):
    """Offline weight quantisation: per-row NVFP4 of stacked expert weights [E, N, K] (per output row n).

    READING of "per row of the flattened expert weights" (Technical Report,
    section 4.3 table): one outer scale per output feature n, over the
    reduction axis K.  ``per_expert``: one outer scale per expert weight
    tensor instead (the table's miniTE CUTLASS column), stored once per row.
    """
    w = np.asarray(w, dtype=np.float64)
    E, N, K = w.shape
    c, s, g = q.quantize_rows_grouped(w.reshape(E * N, K), N if per_expert else 1)
    return dict(codes=c.reshape(E, N, K), packed=q.pack_codes(c).reshape(E, N, K // 2),
                scales=s.reshape(E, N, K // q.BLOCK), outer=g.reshape(E, N))


# ---------------------------------------------------------------------------
# Forward: FC1, SwiGLU, requantise, FC2, unpermute.
# ---------------------------------------------------------------------------
def expert_of_rows(offsets):
    """Expert id of every padded row."""
    offsets = np.asarray(offsets, dtype=np.int64)
    return np.repeat(np.arange(offsets.size - 1), np.diff(offsets))


def grouped_gemm_nvfp4(a_codes, a_scales, a_outer, offsets, w_codes, w_scales, w_outer):
    """Block-scaled grouped product with the FP32-epilogue outer factors.

    For row r of expert e and output n:
        out[r, n] = g_a[r] * g_w[e, n] * sum_k (d c)_a[r, k] (d c)_w[e, n, k]
    (rainbus review, "core method": U_e = MMA(X_e, W_e^T), then g_x g_w
    broadcast in the epilogue; the outer factors do not depend on k).
    Returns float64 [rows, N]: the pre-cast value the GPU's FP32 epilogue
    approximates.
    """
    offsets = np.asarray(offsets, dtype=np.int64)
    rows = int(offsets[-1])
    E, N, _ = w_codes.shape
    out = np.zeros((rows, N))
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 == r0:
            continue
        av = q.block_values(a_codes[r0:r1], a_scales[r0:r1])
        wv = q.block_values(w_codes[e], w_scales[e])
        acc = av @ wv.T
        out[r0:r1] = acc * a_outer[r0:r1].astype(np.float64)[:, None] \
            * w_outer[e].astype(np.float64)[None, :]
    return out


def swiglu(h, I):
    """a = silu(gate) * up with gate = h[:, :I], up = h[:, I:] (float64).

    READING: the pages name SwiGLU between FC1 and FC2 (rainbus review,
    "prerequisites: MoE") but not the half order; the first I features are
    the gate.
    """
    gate, up = h[:, :I], h[:, I:]
    return gate / (1.0 + np.exp(-gate)) * up


def forward(x, topk_idx, topk_w, w1q, w2q, E, row_align=1, act_group_rows=1):
    """Whole forward: quantize+permute, FC1, SwiGLU, requantize, FC2, unpermute.

    Cast points (READING of "casts to BF16 only at the end", AI summary):
    h = bf16(FC1); a = bf16(SwiGLU(h)); o = bf16(FC2); y = bf16(sum_j p o).
    Router coefficients (READING; their position is an explicit
    implementation freedom on the pages): applied in the unpermute, to the
    bf16 o, summed over j in ascending order, one final bf16 rounding.
    ``act_group_rows``: outer-scale domain of the input activations (1 per
    token; T per tensor); the FC2 input stays per dispatched row.
    """
    x = np.asarray(x, dtype=np.float64)
    T, H = x.shape
    I = w1q["codes"].shape[1] // 2
    xq = quantize_permute(x, topk_idx, E, row_align, group_rows=act_group_rows)
    h64 = grouped_gemm_nvfp4(xq["codes"], xq["scales"], xq["outer"], xq["offsets"],
                             w1q["codes"], w1q["scales"], w1q["outer"])
    h = q.round_bf16(h64)
    a = q.round_bf16(swiglu(h, I))
    ac, as_, ag = q.quantize_rows(a)
    live = xq["src_row"] >= 0
    o64 = grouped_gemm_nvfp4(ac, as_, ag, xq["offsets"],
                             w2q["codes"], w2q["scales"], w2q["outer"])
    o = q.round_bf16(o64)
    y = q.round_bf16(unpermute_sum(o, xq["row_map"], topk_w))
    return dict(xq=xq, h64=h64, h=h, a=a, a_codes=ac, a_scales=as_, a_outer=ag,
                o64=o64, o=o, y=y, live=live)


def unpermute_sum(o, row_map, topk_w):
    """y[t] = sum_j p[t, j] * o[row_map[t, j]] (float64, before the bf16 cast)."""
    T, k = row_map.shape
    p = np.asarray(topk_w, dtype=np.float64)
    y = np.zeros((T, o.shape[1]))
    for j in range(k):
        y += p[:, j:j + 1] * o[row_map[:, j]]
    return y


# ---------------------------------------------------------------------------
# Straight-through BF16 backward.
# ---------------------------------------------------------------------------
def backward(dy, x, w1, w2, h, a, topk_w, offsets, row_map, src_row, rnd=True):
    """Straight-through backward on the saved BF16 operands.

    The quantisers are treated as identity (AI summary, "Methodology in
    Plain English": a straight-through estimator on saved original BF16
    activations and weights; Technical Report, section 4.3: the "layer
    bypass" skips backward quantisation).  Saved operands: x, W1, W2 (bf16
    originals), h (bf16 FC1 output), a (bf16 SwiGLU output).

      dO gather:  dO[r]   = p[t,j] dY[t]                 r = row_map[t, j]
      FC2 dgrad:  dA      = dO_e W2[e]                   [n_e, I]
      FC2 wgrad:  dW2[e]  = dO_e^T a_e                   [H, I]
      SwiGLU bwd: dgate   = dA * up * s (1 + gate (1 - s)),  dup = dA * gate * s,
          s = sigmoid(gate)
      FC1 dgrad:  dXp     = dH_e W1[e]                   [n_e, H]
      FC1 wgrad:  dW1[e]  = dH_e^T x[src_row]            [2I, H]
      dX gather:  dX[t]   = sum_j dXp[row_map[t, j]]

    With ``rnd`` every stored tensor (dO, dA, dH, dXp, dX, dW) is rounded to
    bf16 as the GPU stores it; without it the function is the exact float64
    derivative (used to pin it against autograd).
    READINGS: dW and dX are bf16 tensors with FP32 accumulation on the GPU;
    the router-weight gradient is not produced; dW of an empty expert is 0.
    """
    R = q.round_bf16 if rnd else (lambda v: v)
    x = np.asarray(x, dtype=np.float64)
    T, H = x.shape
    E, I2, _ = w1.shape
    I = I2 // 2
    offsets = np.asarray(offsets, dtype=np.int64)
    rows = int(offsets[-1])
    k = row_map.shape[1]
    p = np.asarray(topk_w, dtype=np.float64)

    dO = np.zeros((rows, H))
    for j in range(k):
        dO[row_map[:, j]] = R(p[:, j:j + 1] * dy)

    dA = np.zeros((rows, I))
    dW2 = np.zeros((E, H, I))
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        dA[r0:r1] = R(dO[r0:r1] @ w2[e])
        dW2[e] = R(dO[r0:r1].T @ a[r0:r1])

    gate, up = h[:, :I], h[:, I:]
    s = 1.0 / (1.0 + np.exp(-gate))
    dH = np.concatenate([R(dA * up * s * (1.0 + gate * (1.0 - s))),
                         R(dA * gate * s)], axis=1)

    xs = np.zeros((rows, H))
    live = src_row >= 0
    xs[live] = x[src_row[live]]
    dXp = np.zeros((rows, H))
    dW1 = np.zeros((E, I2, H))
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        dXp[r0:r1] = R(dH[r0:r1] @ w1[e])
        dW1[e] = R(dH[r0:r1].T @ xs[r0:r1])

    dX = np.zeros((T, H))
    for j in range(k):
        dX += dXp[row_map[:, j]]
    dX = R(dX)
    return dict(dO=dO, dA=dA, dH=dH, dXp=dXp, dX=dX, dW1=dW1, dW2=dW2)


# ---------------------------------------------------------------------------
# MXFP4 recipe (E2M1 + E8M0 per 32; see mxfp4): the same forward with the
# NVFP4 quantiser replaced and no outer scales.
# ---------------------------------------------------------------------------
def quantize_permute_mx(x, topk_idx, E, row_align=1, routed=None):
    """MXFP4 of every token row, written to each of its k destination rows.

    Same routing and scatter as ``quantize_permute``; a row's scales depend
    on that row alone.  Pad rows get codes 0 and scale bytes 0.
    Returns dict(codes [rows, K], packed [rows, K/2], scales [rows, K/32],
    offsets, row_map, src_row).
    """
    x = np.asarray(x, dtype=np.float64)
    if routed is None:
        routed = route_fast(topk_idx, E, row_align)
    offsets, row_map, src_row = routed
    rows = int(offsets[-1])
    T, K = x.shape
    tc, ts = mx.quantize_rows_mx(x)
    codes = np.zeros((rows, K), dtype=np.uint8)
    scales = np.zeros((rows, K // mx.MX_BLOCK), dtype=np.uint8)
    live = src_row >= 0
    codes[live] = tc[src_row[live]]
    scales[live] = ts[src_row[live]]
    return dict(codes=codes, packed=q.pack_codes(codes), scales=scales,
                offsets=offsets, row_map=row_map, src_row=src_row)


def quantize_weights_mx(w):
    """Offline MXFP4 of stacked expert weights [E, N, K], blocks along K."""
    w = np.asarray(w, dtype=np.float64)
    E, N, K = w.shape
    c, s = mx.quantize_rows_mx(w.reshape(E * N, K))
    return dict(codes=c.reshape(E, N, K), packed=q.pack_codes(c).reshape(E, N, K // 2),
                scales=s.reshape(E, N, K // mx.MX_BLOCK))


def grouped_gemm_mx(a_codes, a_scales, offsets, w_codes, w_scales):
    """out[r, n] = sum_k (c 2^X)_a[r, k] (c 2^X)_w[e, n, k] for row r of expert e.

    Every term is exact in float64; returns the float64 value the GPU's FP32
    accumulation approximates.
    """
    offsets = np.asarray(offsets, dtype=np.int64)
    rows = int(offsets[-1])
    E, N, _ = w_codes.shape
    out = np.zeros((rows, N))
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 == r0:
            continue
        out[r0:r1] = mx.block_values_mx(a_codes[r0:r1], a_scales[r0:r1]) @ \
            mx.block_values_mx(w_codes[e], w_scales[e]).T
    return out


def forward_mx(x, topk_idx, topk_w, w1q, w2q, E, row_align=1):
    """Whole forward in the MXFP4 recipe: quantize+permute, FC1, SwiGLU,
    requantise, FC2, unpermute, with the cast points and router-coefficient
    position of ``forward``."""
    x = np.asarray(x, dtype=np.float64)
    I = w1q["codes"].shape[1] // 2
    xq = quantize_permute_mx(x, topk_idx, E, row_align)
    h64 = grouped_gemm_mx(xq["codes"], xq["scales"], xq["offsets"], w1q["codes"], w1q["scales"])
    h = q.round_bf16(h64)
    a = q.round_bf16(swiglu(h, I))
    ac, as_ = mx.quantize_rows_mx(a)
    o64 = grouped_gemm_mx(ac, as_, xq["offsets"], w2q["codes"], w2q["scales"])
    o = q.round_bf16(o64)
    y = q.round_bf16(unpermute_sum(o, xq["row_map"], topk_w))
    return dict(xq=xq, h64=h64, h=h, a=a, a_codes=ac, a_scales=as_, o64=o64, o=o, y=y,
                live=xq["src_row"] >= 0)


def backward_mx8(dy, x, w1, w2, h, a, topk_w, offsets, row_map, src_row):
    """Straight-through backward with every GEMM operand in MXFP8.

    The pages compare their BF16 backward with an MXFP8 one (AI summary,
    key findings; Technical Report, section 4.3: backward precision is
    configured apart from the forward).  READING of the MXFP8 backward: each
    GEMM operand is quantised to MXFP8 (E4M3 elements, one E8M0 scale per 32,
    mxfp4.quantize_rows_mx8) along that GEMM's reduction axis, from the same
    bf16 tensors the BF16 backward uses, and the bf16 cast points are the
    BF16 backward's:

      FC2 dgrad  dA     = bf16(Q_H(dO_e) Q_H(W2[e]))        blocks along H
      FC2 wgrad  dW2[e] = bf16(Q_r(dO_e)^T Q_r(a_e))        blocks along the expert's rows
      SwiGLU bwd on the bf16 dA and h (as ``backward``)
      FC1 dgrad  dXp    = bf16(Q_2I(dH_e) Q_2I(W1[e]))      blocks along 2I
      FC1 wgrad  dW1[e] = bf16(Q_r(dH_e)^T Q_r(xp_e))
      dX gather  as ``backward``

    Blocks along the rows never straddle two experts: every expert group's
    first row must be a multiple of 32 (row_align a multiple of 32), and the
    zero pad rows fill the last block.
    """
    R = q.round_bf16
    offsets = np.asarray(offsets, dtype=np.int64)
    if np.any(offsets % mx.MX_BLOCK):
        raise ValueError("expert groups must start at multiples of 32 rows")
    x = np.asarray(x, dtype=np.float64)
    T, H = x.shape
    E, I2, _ = w1.shape
    I = I2 // 2
    rows = int(offsets[-1])
    k = row_map.shape[1]
    p = np.asarray(topk_w, dtype=np.float64)

    dO = np.zeros((rows, H))
    for j in range(k):
        dO[row_map[:, j]] = R(p[:, j:j + 1] * dy)
    qdO_h = mx.mx8_along_rows(dO)
    dA = np.zeros((rows, I))
    dW2 = np.zeros((E, H, I))
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        dA[r0:r1] = R(qdO_h[r0:r1] @ mx.mx8_along_columns(w2[e]))
        if r1 > r0:
            dW2[e] = R(mx.mx8_along_columns(dO[r0:r1]).T @ mx.mx8_along_columns(a[r0:r1]))

    gate, up = h[:, :I], h[:, I:]
    s = 1.0 / (1.0 + np.exp(-gate))
    dH = np.concatenate([R(dA * up * s * (1.0 + gate * (1.0 - s))),
                         R(dA * gate * s)], axis=1)

    xs = np.zeros((rows, H))
    live = src_row >= 0
    xs[live] = x[src_row[live]]
    qdH = mx.mx8_along_rows(dH)
    dXp = np.zeros((rows, H))
    dW1 = np.zeros((E, I2, H))
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        dXp[r0:r1] = R(qdH[r0:r1] @ mx.mx8_along_columns(w1[e]))
        if r1 > r0:
            dW1[e] = R(mx.mx8_along_columns(dH[r0:r1]).T @ mx.mx8_along_columns(xs[r0:r1]))

    dX = np.zeros((T, H))
    for j in range(k):
        dX += dXp[row_map[:, j]]
    dX = R(dX)
    return dict(dO=dO, dA=dA, dH=dH, dXp=dXp, dX=dX, dW1=dW1, dW2=dW2)
