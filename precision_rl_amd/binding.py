"""ctypes binding of libw4a4moe (include/w4a4_moe.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  PyTorch provides device memory and the current stream.  Loading
fails loudly when the library has not been built.
"""
import ctypes
import json
import os

import torch

from . import build as _build

_lib = None

c_i64, c_int, c_sz, c_vp = ctypes.c_int64, ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p

_SIGS = {
    "w4a4_rows_capacity": (c_i64, [c_i64, c_int, c_int, c_int]),
    "w4a4_workspace_size": (c_sz, [c_int, c_i64, c_int, c_int, c_int, c_int, c_int]),
    "w4a4_quantize_permute": (c_int, [c_vp, c_i64, c_int, c_vp, c_int, c_int, c_int,
                                      c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "w4a4_grouped_expert_fwd": (c_int, [c_i64, c_int, c_int, c_int, c_int, c_int,
                                        c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                        c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                        c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                        c_vp, c_sz, c_vp]),
    "w4a4_expert_bwd": (c_int, [c_i64, c_int, c_int, c_int, c_int, c_int,
                                c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "w4a4_quantize_permute_domain": (c_int, [c_vp, c_i64, c_int, c_vp, c_int, c_int, c_int, c_i64,
                                             c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "w4a4_linear_fwd": (c_int, [c_i64, c_int, c_int, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                c_vp, c_vp]),
    "w4a4_linear_bwd": (c_int, [c_i64, c_int, c_int, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                c_vp, c_sz, c_vp]),
    "w4a4_mx_quantize_permute": (c_int, [c_vp, c_i64, c_int, c_vp, c_int, c_int, c_int,
                                         c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "w4a4_mx_grouped_expert_fwd": (c_int, [c_i64, c_int, c_int, c_int, c_int, c_int,
                                           c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                           c_vp, c_vp, c_vp, c_vp,
                                           c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                           c_vp, c_sz, c_vp]),
    "w4a4_mx8_expert_bwd": (c_int, [c_i64, c_int, c_int, c_int, c_int, c_int,
                                    c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                    c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "w4a4_mx8_quantize": (c_int, [c_vp, c_i64, c_int, c_vp, c_vp, c_vp, c_vp, c_i64, c_vp]),
    "w4a4_check_routing": (c_int, [c_vp, c_i64, c_int, c_int, c_vp, c_vp]),
    "w4a4_quantize_permute_noalloc": (c_int, [c_vp, c_i64, c_int, c_vp, c_int, c_int, c_int,
                                              c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "w4a4_status_string": (ctypes.c_char_p, [c_int]),
    "w4a4_last_error": (ctypes.c_char_p, []),
    "w4a4_profiler_enable": (c_int, [c_int]),
    "w4a4_profiler_report": (c_int, [ctypes.c_char_p, c_sz]),
}

WS_QUANTIZE_PERMUTE, WS_FORWARD, WS_BACKWARD, WS_LINEAR_BACKWARD = 0, 1, 2, 3
WS_QUANTIZE_PERMUTE_DOMAIN = 4
WS_MX8_BACKWARD = 5


class W4A4Error(RuntimeError):
    pass


def lib_path():
    return _build.LIB


def load():
    """Load the built library (no build here: build with ``precision_rl_amd.build``)."""
    global _lib
    if _lib is None:
        path = lib_path()
        if not os.path.exists(path):
            raise W4A4Error(f"HIP library not built: {path} is missing "
                            "(run `python -m precision_rl_amd.build`)")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(status):
    if status != 0:
        lib = load()
        raise W4A4Error(f"{lib.w4a4_status_string(status).decode()} ({status}): "
                        f"{lib.w4a4_last_error().decode()}")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def rows_capacity(T, k, E, row_align=1):
    return int(load().w4a4_rows_capacity(T, k, E, row_align))


def workspace_size(kind, T, H, I, E, k, row_align=1):
    return int(load().w4a4_workspace_size(kind, T, H, I, E, k, row_align))


def _workspace(nbytes, device, ws=None):
    if ws is not None and ws.numel() >= nbytes:
        return ws
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


# ----------------------------------------------------------------- wrappers
def w4a4_quantize_permute(x, topk_idx, E, row_align=1, out=None, workspace=None):
    """Route + per-token amax + NVFP4 encode + scatter.  x: [T, K] bf16 cuda; topk_idx: [T, k] int32 or None
    (identity routing, one encoded row per input row).  Returns a dict of
    tensors: codes [cap, K/2] u8, scales [cap, K/16] u8, outer [cap] f32,
    offsets [E+1], row_map [T, k], src_row [cap] (int32)."""
    lib = load()
    T, K = x.shape
    dev = x.device
    if topk_idx is None:
        k, E, row_align = 1, 1, 1
    else:
        k = topk_idx.shape[1]
    cap = rows_capacity(T, k, E, row_align)
    if out is None:
        out = dict(
            codes=torch.empty(cap, K // 2, dtype=torch.uint8, device=dev),
            scales=torch.empty(cap, K // 16, dtype=torch.uint8, device=dev),
            outer=torch.empty(cap, dtype=torch.float32, device=dev),
            offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
            row_map=torch.empty(T, k, dtype=torch.int32, device=dev),
            src_row=torch.empty(cap, dtype=torch.int32, device=dev))
    need = workspace_size(WS_QUANTIZE_PERMUTE, T, K, 0, E, k, row_align)
    ws = _workspace(need, dev, workspace)
    _check(lib.w4a4_quantize_permute(
        _p(x), T, K, _p(topk_idx), k, E, row_align,
        _p(out["codes"]), _p(out["scales"]), _p(out["outer"]), _p(out["offsets"]),
        _p(out["row_map"]), _p(out["src_row"]), _p(ws), ws.numel(), _stream()))
    return out


def w4a4_quantize_permute_domain(x, topk_idx, E, row_align=1, group_rows=1, out=None, workspace=None):
    """w4a4_quantize_permute with one outer scale per group of `group_rows` consecutive
    input rows (T: per tensor).  Same outputs."""
    lib = load()
    T, K = x.shape
    dev = x.device
    if topk_idx is None:
        k, E, row_align = 1, 1, 1
    else:
        k = topk_idx.shape[1]
    cap = rows_capacity(T, k, E, row_align)
    if out is None:
        out = dict(
            codes=torch.empty(cap, K // 2, dtype=torch.uint8, device=dev),
            scales=torch.empty(cap, K // 16, dtype=torch.uint8, device=dev),
            outer=torch.empty(cap, dtype=torch.float32, device=dev),
            offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
            row_map=torch.empty(T, k, dtype=torch.int32, device=dev),
            src_row=torch.empty(cap, dtype=torch.int32, device=dev))
    need = workspace_size(WS_QUANTIZE_PERMUTE_DOMAIN, T, K, 0, E, k, row_align)
    ws = _workspace(need, dev, workspace)
    _check(lib.w4a4_quantize_permute_domain(
        _p(x), T, K, _p(topk_idx), k, E, row_align, group_rows,
        _p(out["codes"]), _p(out["scales"]), _p(out["outer"]), _p(out["offsets"]),
        _p(out["row_map"]), _p(out["src_row"]), _p(ws), ws.numel(), _stream()))
    return out


def w4a4_quantize_permute_noalloc(x, topk_idx, E, row_align=1, out=None):
    """w4a4_quantize_permute without a workspace (the library's per-GPU scratch holds
    the routing counts).  `out`: preallocated outputs as w4a4_quantize_permute returns
    them (allocated here when None)."""
    lib = load()
    T, K = x.shape
    dev = x.device
    if topk_idx is None:
        k, E, row_align = 1, 1, 1
    else:
        k = topk_idx.shape[1]
    cap = rows_capacity(T, k, E, row_align)
    if out is None:
        out = dict(
            codes=torch.empty(cap, K // 2, dtype=torch.uint8, device=dev),
            scales=torch.empty(cap, K // 16, dtype=torch.uint8, device=dev),
            outer=torch.empty(cap, dtype=torch.float32, device=dev),
            offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
            row_map=torch.empty(T, k, dtype=torch.int32, device=dev),
            src_row=torch.empty(cap, dtype=torch.int32, device=dev))
    _check(lib.w4a4_quantize_permute_noalloc(
        _p(x), T, K, _p(topk_idx), k, E, row_align,
        _p(out["codes"]), _p(out["scales"]), _p(out["outer"]), _p(out["offsets"]),
        _p(out["row_map"]), _p(out["src_row"]), _stream()))
    return out


def w4a4_check_routing(topk_idx, E, out=None):
    """Routing validity of topk_idx [T, k] int32 cuda.  Returns an int32 [2] device
    tensor: (number of invalid entries, smallest flat index of one or INT32_MAX)."""
    lib = load()
    T, k = topk_idx.shape
    if out is None:
        out = torch.empty(2, dtype=torch.int32, device=topk_idx.device)
    _check(lib.w4a4_check_routing(_p(topk_idx), T, k, E, _p(out), _stream()))
    return out


def quantize_weights(w, per_expert=False):
    """NVFP4 of stacked expert weights w [E, N, K] bf16 (offline, identity routing): one
    outer scale per row, or per expert weight tensor with `per_expert`.
    Returns dict(codes [E, N, K/2], scales [E, N, K/16], outer [E, N])."""
    E, N, K = w.shape
    if per_expert:
        q = w4a4_quantize_permute_domain(w.reshape(E * N, K), None, 1, group_rows=N)
    else:
        q = w4a4_quantize_permute(w.reshape(E * N, K), None, 1)
    return dict(codes=q["codes"].view(E, N, K // 2), scales=q["scales"].view(E, N, K // 16),
                outer=q["outer"].view(E, N))


def w4a4_grouped_expert_fwd(xq, topk_w, w1q, w2q, T, H, I, E, k, row_align=1,
                            save=False, debug=False, y=None, workspace=None, saved=None):
    """Grouped expert forward: FC1 -> SwiGLU -> requantise -> FC2 -> unpermute.  xq: result of ``w4a4_quantize_permute``; w1q / w2q: results
    of ``quantize_weights``.  Returns dict(y, and h/a when ``save``, and the
    FC1 pre-cast values plus the FC2-input encoding when ``debug``)."""
    lib = load()
    dev = xq["codes"].device
    cap = rows_capacity(T, k, E, row_align)
    res = {}
    res["y"] = y if y is not None else torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    if save:
        if saved is None:
            saved = dict(h=torch.empty(cap, 2 * I, dtype=torch.bfloat16, device=dev),
                         a=torch.empty(cap, I, dtype=torch.bfloat16, device=dev))
        res.update(saved)
    if debug:
        res["fc1_f32"] = torch.empty(cap, 2 * I, dtype=torch.float32, device=dev)
        res["a_codes"] = torch.empty(cap, I // 2, dtype=torch.uint8, device=dev)
        res["a_scales"] = torch.empty(cap, I // 16, dtype=torch.uint8, device=dev)
        res["a_outer"] = torch.empty(cap, dtype=torch.float32, device=dev)
    need = workspace_size(WS_FORWARD, T, H, I, E, k, row_align)
    ws = _workspace(need, dev, workspace)
    _check(lib.w4a4_grouped_expert_fwd(
        T, H, I, E, k, row_align,
        _p(xq["codes"]), _p(xq["scales"]), _p(xq["outer"]),
        _p(xq["offsets"]), _p(xq["row_map"]), _p(xq["src_row"]), _p(topk_w),
        _p(w1q["codes"]), _p(w1q["scales"]), _p(w1q["outer"]),
        _p(w2q["codes"]), _p(w2q["scales"]), _p(w2q["outer"]),
        _p(res["y"]), _p(res.get("h")), _p(res.get("a")), _p(res.get("fc1_f32")),
        _p(res.get("a_codes")), _p(res.get("a_scales")), _p(res.get("a_outer")),
        _p(ws), ws.numel(), _stream()))
    return res


def w4a4_expert_bwd(dy, x, w1, w2, h, a, topk_w, xq, T, H, I, E, k, row_align=1,
                    out=None, workspace=None):
    """Straight-through BF16 backward.  Returns dict(dx [T, H], dw1 [E, 2I, H], dw2 [E, H, I]) bf16."""
    lib = load()
    dev = dy.device
    if out is None:
        out = dict(dx=torch.empty(T, H, dtype=torch.bfloat16, device=dev),
                   dw1=torch.empty(E, 2 * I, H, dtype=torch.bfloat16, device=dev),
                   dw2=torch.empty(E, H, I, dtype=torch.bfloat16, device=dev))
    need = workspace_size(WS_BACKWARD, T, H, I, E, k, row_align)
    ws = _workspace(need, dev, workspace)
    _check(lib.w4a4_expert_bwd(
        T, H, I, E, k, row_align, _p(dy), _p(x), _p(w1), _p(w2), _p(h), _p(a), _p(topk_w),
        _p(xq["offsets"]), _p(xq["row_map"]), _p(xq["src_row"]),
        _p(out["dx"]), _p(out["dw1"]), _p(out["dw2"]), _p(ws), ws.numel(), _stream()))
    return out


def w4a4_mx8_expert_bwd(dy, x, w1, w2, h, a, topk_w, xq, T, H, I, E, k, row_align=128,
                        out=None, workspace=None):
    """Straight-through backward with MXFP8 GEMM operands (row_align 128).
    Returns dict(dx [T, H], dw1 [E, 2I, H], dw2 [E, H, I]) bf16."""
    lib = load()
    dev = dy.device
    if out is None:
        out = dict(dx=torch.empty(T, H, dtype=torch.bfloat16, device=dev),
                   dw1=torch.empty(E, 2 * I, H, dtype=torch.bfloat16, device=dev),
                   dw2=torch.empty(E, H, I, dtype=torch.bfloat16, device=dev))
    need = workspace_size(WS_MX8_BACKWARD, T, H, I, E, k, row_align)
    ws = _workspace(need, dev, workspace)
    _check(lib.w4a4_mx8_expert_bwd(
        T, H, I, E, k, row_align, _p(dy), _p(x), _p(w1), _p(w2), _p(h), _p(a), _p(topk_w),
        _p(xq["offsets"]), _p(xq["row_map"]), _p(xq["src_row"]),
        _p(out["dx"]), _p(out["dw1"]), _p(out["dw2"]), _p(ws), ws.numel(), _stream()))
    return out


def w4a4_mx8_quantize(x):
    """MXFP8 (E4M3 + E8M0 per 32) of x [R, C] bf16 along rows and along columns.
    Returns dict(q_rows [R, C], s_rows [R, C/32], q_cols [C, R], s_cols [C, R/32]) uint8."""
    lib = load()
    R, C = x.shape
    dev = x.device
    pitch = (R + 127) // 128 * 128
    out = dict(q_rows=torch.empty(R, C, dtype=torch.uint8, device=dev),
               s_rows=torch.empty(R, C // 32, dtype=torch.uint8, device=dev),
               q_cols=torch.empty(C, pitch, dtype=torch.uint8, device=dev),
               s_cols=torch.empty(C, pitch // 32, dtype=torch.uint8, device=dev))
    _check(lib.w4a4_mx8_quantize(_p(x), R, C, _p(out["q_rows"]), _p(out["s_rows"]), _p(out["q_cols"]),
                                 _p(out["s_cols"]), pitch, _stream()))
    out["q_cols"] = out["q_cols"][:, :R]
    out["s_cols"] = out["s_cols"][:, :R // 32]
    return out


def w4a4_linear_fwd(xq, wq, T, K, N, y=None):
    """Dense per-token NVFP4 linear layer y = x W^T.  xq: w4a4_quantize_permute(x, None, 1)
    of x [T, K]; wq: the same of W [N, K].  Returns y [T, N] bf16."""
    lib = load()
    dev = wq["codes"].device
    if y is None:
        y = torch.empty(T, N, dtype=torch.bfloat16, device=dev)
    _check(lib.w4a4_linear_fwd(T, K, N, _p(xq["codes"]), _p(xq["scales"]), _p(xq["outer"]),
                               _p(xq["offsets"]), _p(wq["codes"]), _p(wq["scales"]),
                               _p(wq["outer"]), _p(y), _stream()))
    return y


def w4a4_linear_bwd(dy, x, w, xq, T, K, N, out=None, workspace=None):
    """Straight-through BF16 backward of w4a4_linear_fwd.  Returns dict(dx [T, K], dw [N, K]) bf16."""
    lib = load()
    dev = w.device
    if out is None:
        out = dict(dx=torch.empty(T, K, dtype=torch.bfloat16, device=dev),
                   dw=torch.empty(N, K, dtype=torch.bfloat16, device=dev))
    ws = _workspace(workspace_size(WS_LINEAR_BACKWARD, 0, K, N, 1, 1), dev, workspace)
    _check(lib.w4a4_linear_bwd(T, K, N, _p(dy), _p(x), _p(w), _p(xq["offsets"]),
                               _p(out["dx"]), _p(out["dw"]), _p(ws), ws.numel(), _stream()))
    return out


# ------------------------------------------------------------ MXFP4 recipe
def w4a4_mx_quantize_permute(x, topk_idx, E, row_align=1, out=None, workspace=None):
    """Route + MXFP4 encode (E2M1, one E8M0 scale per 32) + scatter.  x: [T, K] bf16 cuda,
    K % 32 == 0; topk_idx: [T, k] int32 or None (identity routing).  Returns a dict:
    codes [cap, K/2] u8, scales [cap, K/32] u8, offsets [E+1], row_map [T, k], src_row [cap]."""
    lib = load()
    T, K = x.shape
    dev = x.device
    if topk_idx is None:
        k, E, row_align = 1, 1, 1
    else:
        k = topk_idx.shape[1]
    cap = rows_capacity(T, k, E, row_align)
    if out is None:
        out = dict(
            codes=torch.empty(cap, K // 2, dtype=torch.uint8, device=dev),
            scales=torch.empty(cap, K // 32, dtype=torch.uint8, device=dev),
            offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
            row_map=torch.empty(T, k, dtype=torch.int32, device=dev),
            src_row=torch.empty(cap, dtype=torch.int32, device=dev))
    need = workspace_size(WS_QUANTIZE_PERMUTE, T, K, 0, E, k, row_align)
    ws = _workspace(need, dev, workspace)
    _check(lib.w4a4_mx_quantize_permute(
        _p(x), T, K, _p(topk_idx), k, E, row_align, _p(out["codes"]), _p(out["scales"]),
        _p(out["offsets"]), _p(out["row_map"]), _p(out["src_row"]), _p(ws), ws.numel(), _stream()))
    return out


def quantize_weights_mx(w):
    """MXFP4 of stacked expert weights w [E, N, K] bf16 along K (offline, identity routing).
    Returns dict(codes [E, N, K/2], scales [E, N, K/32])."""
    E, N, K = w.shape
    q = w4a4_mx_quantize_permute(w.reshape(E * N, K), None, 1)
    return dict(codes=q["codes"].view(E, N, K // 2), scales=q["scales"].view(E, N, K // 32))


def w4a4_mx_grouped_expert_fwd(xq, topk_w, w1q, w2q, T, H, I, E, k, row_align=1,
                               save=False, debug=False, y=None, workspace=None, saved=None):
    """MXFP4 grouped expert forward: FC1 -> SwiGLU -> requantise -> FC2 -> unpermute on the
    scaled FP4 MFMA.  xq: result of ``w4a4_mx_quantize_permute``; w1q / w2q: of
    ``quantize_weights_mx``.  Returns dict(y, h/a when ``save``, fc1_f32 and the FC2-input
    encoding a_codes / a_scales when ``debug``)."""
    lib = load()
    dev = xq["codes"].device
    cap = rows_capacity(T, k, E, row_align)
    res = {}
    res["y"] = y if y is not None else torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    if save:
        if saved is None:
            saved = dict(h=torch.empty(cap, 2 * I, dtype=torch.bfloat16, device=dev),
                         a=torch.empty(cap, I, dtype=torch.bfloat16, device=dev))
        res.update(saved)
    if debug:
        res["fc1_f32"] = torch.empty(cap, 2 * I, dtype=torch.float32, device=dev)
        res["a_codes"] = torch.empty(cap, I // 2, dtype=torch.uint8, device=dev)
        res["a_scales"] = torch.empty(cap, I // 32, dtype=torch.uint8, device=dev)
    need = workspace_size(WS_FORWARD, T, H, I, E, k, row_align)
    ws = _workspace(need, dev, workspace)
    _check(lib.w4a4_mx_grouped_expert_fwd(
        T, H, I, E, k, row_align, _p(xq["codes"]), _p(xq["scales"]),
        _p(xq["offsets"]), _p(xq["row_map"]), _p(xq["src_row"]), _p(topk_w),
        _p(w1q["codes"]), _p(w1q["scales"]), _p(w2q["codes"]), _p(w2q["scales"]),
        _p(res["y"]), _p(res.get("h")), _p(res.get("a")), _p(res.get("fc1_f32")),
        _p(res.get("a_codes")), _p(res.get("a_scales")), _p(ws), ws.numel(), _stream()))
    return res


def w4a4_profiler_enable(on=True):
    load().w4a4_profiler_enable(1 if on else 0)


def w4a4_profiler_report():
    lib = load()
    n = lib.w4a4_profiler_report(None, 0)
    if n < 0:
        raise W4A4Error("profiler report failed")
    buf = ctypes.create_string_buffer(n + 1)
    lib.w4a4_profiler_report(buf, n + 1)
    return json.loads(buf.value.decode())
