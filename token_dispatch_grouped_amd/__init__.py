"""MI355X (gfx950) MoE expert-layer forward on one rank's share: Python binding.

Thin ctypes marshalling over libmoe.so (include/moe.h). Every step of the path
runs in the library's HIP kernels; PyTorch only provides device memory and the
current stream. There is no fallback: if the library is missing, importing the
binding works only for introspection (`lib_path`, `declared_symbols`) and every
compute call raises.
"""
from __future__ import annotations

import ctypes
import os
import re
from dataclasses import dataclass

_PKG = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_PKG)
lib_path = os.path.join(_PKG, "libmoe.so")
header_path = os.path.join(_ROOT, "include", "moe.h")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EHIP = 0, 1, 2, 3
MOE_F32, MOE_BF16 = 0, 1


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class moe_shape(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int64),
        ("d", ctypes.c_int32),
        ("d_ff", ctypes.c_int32),
        ("E", ctypes.c_int32),
        ("k", ctypes.c_int32),
        ("e_begin", ctypes.c_int32),
        ("e_end", ctypes.c_int32),
    ]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(lib_path):
            raise ImportError(
                f"{lib_path} is missing: build it with token_dispatch_grouped_amd.build.build() "
                "(there is no fallback path)")
        lib = ctypes.CDLL(lib_path)
        P, S, I32, I64, SZ = ctypes.c_void_p, ctypes.POINTER(moe_shape), ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        sigs = {
            "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
            "moe_expert_range": (ctypes.c_int, [I32, I32, I32, ctypes.POINTER(I32), ctypes.POINTER(I32)]),
            "moe_route_topk": (ctypes.c_int, [S, P, P, P, P]),
            "moe_dispatch_workspace_bytes": (SZ, [S]),
            "moe_dispatch": (ctypes.c_int, [S, ctypes.c_int, P, P, P, P, P, P, P, P, P]),
            "moe_dispatch_indices": (ctypes.c_int, [S, P, P, P, P, P, P, P]),
            "moe_grouped_gemm_gather": (ctypes.c_int, [S, ctypes.c_int, P, P, P, P, P, P, P, P, P]),
            "moe_grouped_gemm_workspace_bytes": (SZ, [S, ctypes.c_int]),
            "moe_grouped_gemm": (ctypes.c_int, [S, ctypes.c_int, P, P, P, P, P, P, P, P]),
            "moe_combine": (ctypes.c_int, [S, ctypes.c_int, P, P, P, P, P]),
            "moe_combine_backward": (ctypes.c_int, [S, ctypes.c_int, P, P, P, P, P, P, P]),
            "moe_grouped_gemm_backward_workspace_bytes": (SZ, [S, ctypes.c_int]),
            "moe_grouped_gemm_backward": (ctypes.c_int, [S, ctypes.c_int, P, P, P, P, P, P, P, P, P, P, P, P]),
            "moe_dispatch_backward": (ctypes.c_int, [S, ctypes.c_int, P, P, P, P]),
            "moe_route_topk_backward": (ctypes.c_int, [S, P, P, P, P, P]),
            "moe_grouped_gemm_gather_save": (ctypes.c_int, [S, ctypes.c_int, P, P, P, P, P, P, P, P, P, P]),
            "moe_grouped_gemm_backward_saved": (ctypes.c_int,
                                                [S, ctypes.c_int, P, P, P, P, P, P, P, P, P, P, P, P, P]),
        }
        for name, (res, args) in sigs.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def lib():
    """The loaded ctypes library (raises ImportError when it is not built)."""
    return _load()


def declared_symbols() -> list[str]:
    """Function names declared in include/moe.h."""
    with open(header_path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


def status_string(status: int) -> str:
    try:
        return _load().moe_status_string(int(status)).decode()
    except ImportError:
        return f"status {status}"


def _check(status: int, where: str) -> None:
    if status != MOE_OK:
        raise MoeError(status, where)


# ----------------------------------------------------------------------------- torch helpers

def _torch():
    import torch
    return torch


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float32:
        return MOE_F32
    raise TypeError(f"unsupported dtype {t.dtype}; expected bfloat16 or float32")


def _dev(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("every tensor must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("every tensor must be contiguous (row-major)")


def shape(T, d, d_ff, E, k, e_begin, e_end) -> moe_shape:
    return moe_shape(int(T), int(d), int(d_ff), int(E), int(k), int(e_begin), int(e_end))


def expert_range(E: int, ep: int, rank: int) -> tuple[int, int]:
    lo, hi = ctypes.c_int32(), ctypes.c_int32()
    _check(_load().moe_expert_range(E, ep, rank, ctypes.byref(lo), ctypes.byref(hi)), "moe_expert_range")
    return lo.value, hi.value


# ----------------------------------------------------------------------------- the four steps

def route_topk(logits, k: int, topk_idx=None, topk_w=None, stream=None):
    """logits [T, E] fp32 -> (topk_idx [T, k] int32, topk_w [T, k] fp32)."""
    torch = _torch()
    _dev(logits)
    if logits.dtype != torch.float32 or logits.dim() != 2:
        raise TypeError("logits must be a [T, E] float32 tensor")
    T, E = logits.shape
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _dev(topk_idx, topk_w)
    s = shape(T, 8, 8, E, k, 0, E)
    _check(_load().moe_route_topk(ctypes.byref(s), _ptr(logits), _ptr(topk_idx), _ptr(topk_w), _stream(stream)),
           "moe_route_topk")
    return topk_idx, topk_w


@dataclass
class Dispatch:
    counts: object
    offsets: object
    perm: object
    pair_pos: object
    x_perm: object
    workspace: object


def dispatch_alloc(x, k: int, E: int, e_begin: int, e_end: int, gather: bool = True) -> Dispatch:
    """Allocate every dispatch output (sized on the host, no device read); without
    `gather` there is no x_perm (the fused path reads rows straight from x)."""
    torch = _torch()
    T, d = x.shape
    n_max = T * min(k, e_end - e_begin)
    s = shape(T, d, 8, E, k, e_begin, e_end)
    ws_bytes = _load().moe_dispatch_workspace_bytes(ctypes.byref(s))
    dev = x.device
    return Dispatch(
        counts=torch.empty(E, dtype=torch.int32, device=dev),
        offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
        perm=torch.empty(T * k, dtype=torch.int32, device=dev),
        pair_pos=torch.empty(T * k, dtype=torch.int32, device=dev),
        x_perm=torch.empty((n_max, d), dtype=x.dtype, device=dev) if gather else None,
        workspace=torch.empty(max(1, ws_bytes), dtype=torch.uint8, device=dev),
    )


def dispatch(x, topk_idx, E: int, e_begin: int, e_end: int, out: Dispatch | None = None, stream=None,
             gather: bool = True) -> Dispatch:
    """Histogram, offsets, stable permutation and (with `gather`) the local-row
    gather into x_perm; without it, moe_dispatch_indices (no x_perm)."""
    _dev(x, topk_idx)
    T, d = x.shape
    k = topk_idx.shape[1] if topk_idx.dim() == 2 else 1
    if out is None:
        out = dispatch_alloc(x, k, E, e_begin, e_end, gather=gather)
    s = shape(T, d, 8, E, k, e_begin, e_end)
    if gather:
        if out.x_perm is None:
            raise ValueError("this Dispatch has no x_perm; allocate it with gather=True")
        _check(_load().moe_dispatch(ctypes.byref(s), _dtype_code(x), _ptr(x), _ptr(topk_idx), _ptr(out.counts),
                                    _ptr(out.offsets), _ptr(out.perm), _ptr(out.pair_pos), _ptr(out.x_perm),
                                    _ptr(out.workspace), _stream(stream)), "moe_dispatch")
    else:
        _check(_load().moe_dispatch_indices(ctypes.byref(s), _ptr(topk_idx), _ptr(out.counts), _ptr(out.offsets),
                                            _ptr(out.perm), _ptr(out.pair_pos), _ptr(out.workspace),
                                            _stream(stream)), "moe_dispatch_indices")
    return out


def grouped_gemm(x_perm, offsets, w_gate_up, w_down, T: int, k: int, E: int, e_begin: int, e_end: int,
                 h=None, y=None, stream=None):
    """Local experts' SwiGLU FFN: returns (h [N_max, d_ff], y [N_max, d])."""
    torch = _torch()
    _dev(x_perm, offsets, w_gate_up, w_down)
    n_max, d = x_perm.shape
    e_loc, d_ff, _ = w_down.shape
    if w_gate_up.shape != (e_loc, d, 2 * d_ff) or w_down.shape != (e_loc, d_ff, d):
        raise ValueError("w_gate_up must be [E_loc, d, 2*d_ff] and w_down [E_loc, d_ff, d]")
    if e_loc != e_end - e_begin:
        raise ValueError("expert weights must hold exactly the local experts")
    if h is None:
        h = torch.empty((n_max, d_ff), dtype=x_perm.dtype, device=x_perm.device)
    if y is None:
        y = torch.empty((n_max, d), dtype=x_perm.dtype, device=x_perm.device)
    _dev(h, y)
    s = shape(T, d, d_ff, E, k, e_begin, e_end)
    dt = _dtype_code(x_perm)
    ws_bytes = _load().moe_grouped_gemm_workspace_bytes(ctypes.byref(s), dt)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=x_perm.device) if ws_bytes else None
    _check(_load().moe_grouped_gemm(ctypes.byref(s), dt, _ptr(x_perm), _ptr(offsets), _ptr(w_gate_up),
                                    _ptr(w_down), _ptr(h), _ptr(y), _ptr(ws), _stream(stream)),
           "moe_grouped_gemm")
    return h, y


def grouped_gemm_gather(x, perm, offsets, w_gate_up, w_down, k: int, E: int, e_begin: int, e_end: int,
                        h=None, y=None, stream=None, gu=None):
    """grouped_gemm reading each local row straight from x through perm (no
    x_perm): returns (h [N_max, d_ff], y [N_max, d]), bit-identical to
    dispatch + grouped_gemm. With gu (a [N_max, 2*d_ff] tensor) the gate/up
    pre-activations are kept there as well (moe_grouped_gemm_gather_save)."""
    torch = _torch()
    _dev(x, perm, offsets, w_gate_up, w_down)
    T, d = x.shape
    e_loc, d_ff, _ = w_down.shape
    if w_gate_up.shape != (e_loc, d, 2 * d_ff) or w_down.shape != (e_loc, d_ff, d):
        raise ValueError("w_gate_up must be [E_loc, d, 2*d_ff] and w_down [E_loc, d_ff, d]")
    if e_loc != e_end - e_begin:
        raise ValueError("expert weights must hold exactly the local experts")
    n_max = T * min(k, e_loc)
    if h is None:
        h = torch.empty((n_max, d_ff), dtype=x.dtype, device=x.device)
    if y is None:
        y = torch.empty((n_max, d), dtype=x.dtype, device=x.device)
    _dev(h, y)
    s = shape(T, d, d_ff, E, k, e_begin, e_end)
    dt = _dtype_code(x)
    ws_bytes = _load().moe_grouped_gemm_workspace_bytes(ctypes.byref(s), dt)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device) if ws_bytes else None
    if gu is None:
        _check(_load().moe_grouped_gemm_gather(ctypes.byref(s), dt, _ptr(x), _ptr(perm), _ptr(offsets),
                                               _ptr(w_gate_up), _ptr(w_down), _ptr(h), _ptr(y), _ptr(ws),
                                               _stream(stream)), "moe_grouped_gemm_gather")
    else:
        _dev(gu)
        if tuple(gu.shape) != (n_max, 2 * d_ff) or gu.dtype != x.dtype:
            raise ValueError("gu must be [N_max, 2*d_ff] in the activations' dtype")
        _check(_load().moe_grouped_gemm_gather_save(ctypes.byref(s), dt, _ptr(x), _ptr(perm), _ptr(offsets),
                                                    _ptr(w_gate_up), _ptr(w_down), _ptr(h), _ptr(y), _ptr(gu),
                                                    _ptr(ws), _stream(stream)), "moe_grouped_gemm_gather_save")
    return h, y


def combine(y, pair_pos, topk_w, T: int, k: int, E: int, e_begin: int, e_end: int, out=None, stream=None):
    """out[t] = sum_j topk_w[t, j] * y[pair_pos[t*k + j]] over local pairs; [T, d]."""
    torch = _torch()
    _dev(y, pair_pos, topk_w)
    d = y.shape[1]
    if out is None:
        out = torch.empty((T, d), dtype=y.dtype, device=y.device)
    _dev(out)
    s = shape(T, d, 8, E, k, e_begin, e_end)
    _check(_load().moe_combine(ctypes.byref(s), _dtype_code(y), _ptr(y), _ptr(pair_pos), _ptr(topk_w),
                               _ptr(out), _stream(stream)), "moe_combine")
    return out


def layer(x, logits, w_gate_up, w_down, k: int, e_begin: int, e_end: int, stream=None, fused: bool = False,
          save: bool = False) -> dict:
    """The whole forward of one rank: route -> dispatch -> grouped GEMM -> combine.
    With `fused`, the dispatch writes indices only and the GEMM gathers the rows.
    With `save` (fused path), the gate/up pre-activations are kept in the result
    as "gu", for layer_backward to use instead of recomputing them."""
    torch = _torch()
    T = x.shape[0]
    E = logits.shape[1]
    if save and not fused:
        raise ValueError("save needs the fused path")
    idx, w = route_topk(logits, k, stream=stream)
    disp = dispatch(x, idx, E, e_begin, e_end, stream=stream, gather=not fused)
    gu = None
    if fused:
        if save:
            e_loc, d_ff = w_down.shape[0], w_down.shape[1]
            gu = torch.empty((T * min(k, e_loc), 2 * d_ff), dtype=x.dtype, device=x.device)
        h, y = grouped_gemm_gather(x, disp.perm, disp.offsets, w_gate_up, w_down, k, E, e_begin, e_end,
                                   stream=stream, gu=gu)
    else:
        h, y = grouped_gemm(disp.x_perm, disp.offsets, w_gate_up, w_down, T, k, E, e_begin, e_end, stream=stream)
    out = combine(y, disp.pair_pos, w, T, k, E, e_begin, e_end, stream=stream)
    return dict(idx=idx, w=w, counts=disp.counts, offsets=disp.offsets, perm=disp.perm,
                pair_pos=disp.pair_pos, x_perm=disp.x_perm, h=h, y=y, out=out, gu=gu)


# ----------------------------------------------------------------------------- backward

def combine_backward(d_out, y, pair_pos, topk_w, T: int, k: int, E: int, e_begin: int, e_end: int,
                     d_y=None, d_topk_w=None, stream=None):
    """(d_y [N_max, d], d_topk_w [T, k] fp32): the gradient of combine."""
    torch = _torch()
    _dev(d_out, y, pair_pos, topk_w)
    d = d_out.shape[1]
    if d_y is None:
        d_y = torch.empty_like(y)
    if d_topk_w is None:
        d_topk_w = torch.empty((T, k), dtype=torch.float32, device=d_out.device)
    s = shape(T, d, 8, E, k, e_begin, e_end)
    _check(_load().moe_combine_backward(ctypes.byref(s), _dtype_code(d_out), _ptr(d_out), _ptr(y), _ptr(pair_pos),
                                        _ptr(topk_w), _ptr(d_y), _ptr(d_topk_w), _stream(stream)),
           "moe_combine_backward")
    return d_y, d_topk_w


def grouped_gemm_backward_workspace_bytes(T: int, d: int, d_ff: int, E: int, k: int, e_begin: int, e_end: int) -> int:
    s = shape(T, d, d_ff, E, k, e_begin, e_end)
    return int(_load().moe_grouped_gemm_backward_workspace_bytes(ctypes.byref(s), MOE_BF16))


def grouped_gemm_backward(x, perm, offsets, w_gate_up, w_down, h, d_y, k: int, E: int, e_begin: int, e_end: int,
                          d_x_perm=None, d_w_gate_up=None, d_w_down=None, workspace=None, stream=None, gu=None):
    """(d_x_perm, d_w_gate_up, d_w_down): the gradient of the grouped expert FFN.
    With gu (the pre-activations the saving forward kept) they are not
    recomputed (moe_grouped_gemm_backward_saved)."""
    torch = _torch()
    _dev(x, perm, offsets, w_gate_up, w_down, h, d_y)
    T, d = x.shape
    e_loc, d_ff, _ = w_down.shape
    s = shape(T, d, d_ff, E, k, e_begin, e_end)
    dt = _dtype_code(x)
    if d_x_perm is None:
        d_x_perm = torch.empty_like(d_y)
    if d_w_gate_up is None:
        d_w_gate_up = torch.empty_like(w_gate_up)
    if d_w_down is None:
        d_w_down = torch.empty_like(w_down)
    ws = workspace
    if ws is None:
        ws_bytes = _load().moe_grouped_gemm_backward_workspace_bytes(ctypes.byref(s), dt)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device) if ws_bytes else None
    if gu is None:
        _check(_load().moe_grouped_gemm_backward(ctypes.byref(s), dt, _ptr(x), _ptr(perm), _ptr(offsets),
                                                 _ptr(w_gate_up), _ptr(w_down), _ptr(h), _ptr(d_y), _ptr(d_x_perm),
                                                 _ptr(d_w_gate_up), _ptr(d_w_down), _ptr(ws), _stream(stream)),
               "moe_grouped_gemm_backward")
    else:
        _dev(gu)
        if tuple(gu.shape) != (h.shape[0], 2 * d_ff) or gu.dtype != h.dtype:
            raise ValueError("gu must be [N_max, 2*d_ff] in the activations' dtype")
        _check(_load().moe_grouped_gemm_backward_saved(ctypes.byref(s), dt, _ptr(x), _ptr(perm), _ptr(offsets),
                                                       _ptr(w_gate_up), _ptr(w_down), _ptr(h), _ptr(gu), _ptr(d_y),
                                                       _ptr(d_x_perm), _ptr(d_w_gate_up), _ptr(d_w_down), _ptr(ws),
                                                       _stream(stream)), "moe_grouped_gemm_backward_saved")
    return d_x_perm, d_w_gate_up, d_w_down


def dispatch_backward(d_x_perm, pair_pos, T: int, k: int, E: int, e_begin: int, e_end: int, d_x=None, stream=None):
    """d_x [T, d]: the gradient of the row gather."""
    torch = _torch()
    _dev(d_x_perm, pair_pos)
    d = d_x_perm.shape[1]
    if d_x is None:
        d_x = torch.empty((T, d), dtype=d_x_perm.dtype, device=d_x_perm.device)
    s = shape(T, d, 8, E, k, e_begin, e_end)
    _check(_load().moe_dispatch_backward(ctypes.byref(s), _dtype_code(d_x_perm), _ptr(d_x_perm), _ptr(pair_pos),
                                         _ptr(d_x), _stream(stream)), "moe_dispatch_backward")
    return d_x


def route_topk_backward(topk_idx, topk_w, d_topk_w, E: int, d_logits=None, stream=None):
    """d_logits [T, E] fp32: the gradient of route_topk's weights w.r.t. the logits."""
    torch = _torch()
    _dev(topk_idx, topk_w, d_topk_w)
    T, k = topk_idx.shape
    if d_logits is None:
        d_logits = torch.empty((T, E), dtype=torch.float32, device=topk_idx.device)
    s = shape(T, 8, 8, E, k, 0, E)
    _check(_load().moe_route_topk_backward(ctypes.byref(s), _ptr(topk_idx), _ptr(topk_w), _ptr(d_topk_w),
                                           _ptr(d_logits), _stream(stream)), "moe_route_topk_backward")
    return d_logits


def layer_backward(x, w_gate_up, w_down, fwd: dict, d_out, k: int, e_begin: int, e_end: int, stream=None) -> dict:
    """The whole backward of one rank, given the forward's dict (from layer()):
    combine -> experts -> row gather -> router softmax. The gate/up
    pre-activations come from the forward's "gu" when it kept them."""
    T = x.shape[0]
    E = fwd["counts"].shape[0]
    d_y, d_w = combine_backward(d_out, fwd["y"], fwd["pair_pos"], fwd["w"], T, k, E, e_begin, e_end, stream=stream)
    d_x_perm, d_wgu, d_wdn = grouped_gemm_backward(x, fwd["perm"], fwd["offsets"], w_gate_up, w_down, fwd["h"], d_y,
                                                   k, E, e_begin, e_end, stream=stream, gu=fwd.get("gu"))
    d_x = dispatch_backward(d_x_perm, fwd["pair_pos"], T, k, E, e_begin, e_end, stream=stream)
    d_logits = route_topk_backward(fwd["idx"], fwd["w"], d_w, E, stream=stream)
    return dict(d_y=d_y, d_w=d_w, d_x_perm=d_x_perm, d_w_gate_up=d_wgu, d_w_down=d_wdn, d_x=d_x, d_logits=d_logits)
