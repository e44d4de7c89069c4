"""MI355X (gfx950) MoE expert-layer forward on one rank's share: Python binding.

Thin ctypes marshalling over libmoe.so (include/moe.h). Every step of the path
runs in the library's HIP kernels; PyTorch only provides device memory and the
current stream. There is no fallback: if the library is missing, importing the
binding works only for introspection (`lib_path`, `declared_symbols`) and every
compute call raises.

Every wrapper checks the dtype and shape of each tensor it is given (inputs and
caller-provided outputs alike) against the sizes of the call before anything
reaches the library: a wrong dtype raises TypeError, a wrong shape ValueError.

Debug mode (`set_debug(True)`, or MOE_DEBUG=1 in the environment at import)
loads libmoe_debug.so instead, whose dispatch also counts the expert ids outside
[0, E) on the device; `dispatch` then waits for its stream and raises ValueError
when there are any. That wait makes the dispatch synchronous, so debug mode is
for finding bad input, not for graph capture or timing.
"""
from __future__ import annotations

import ctypes
import os
import re
from dataclasses import dataclass

_PKG = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_PKG)
lib_path = os.path.join(_PKG, "libmoe.so")
debug_lib_path = os.path.join(_PKG, "libmoe_debug.so")
header_path = os.path.join(_ROOT, "include", "moe.h")
_SIZE_MAX = ctypes.c_size_t(-1).value

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


_libs: dict = {}
_debug = os.environ.get("MOE_DEBUG", "") not in ("", "0")


def set_debug(enabled: bool) -> None:
    """Use libmoe_debug.so (True) or libmoe.so (False) for the calls that follow."""
    global _debug
    _debug = bool(enabled)


def debug_enabled() -> bool:
    return _debug


def _load():
    path = debug_lib_path if _debug else lib_path
    if path not in _libs:
        if not os.path.exists(path):
            raise ImportError(
                f"{path} is missing: build it with token_dispatch_grouped_amd.build.build() "
                "(there is no fallback path)")
        lib = ctypes.CDLL(path)
        P, S, I32, I64, SZ = ctypes.c_void_p, ctypes.POINTER(moe_shape), ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        sigs = {
            "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
            "moe_expert_range": (ctypes.c_int, [I32, I32, I32, ctypes.POINTER(I32), ctypes.POINTER(I32)]),
            "moe_route_topk": (ctypes.c_int, [S, P, P, P, P]),
            "moe_dispatch_workspace_bytes": (SZ, [S]),
            "moe_dispatch_debug_word_offset": (SZ, []),
            "moe_dispatch": (ctypes.c_int, [S, ctypes.c_int, P, P, P, P, P, P, P, P, P]),
            "moe_dispatch_indices": (ctypes.c_int, [S, P, P, P, P, P, P, P]),
            "moe_dispatch_indices_noalloc": (ctypes.c_int, [S, P, P, P, P, P, P]),
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
        _libs[path] = lib
    return _libs[path]


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


def _want(t, name: str, dtype=None, shape=None, min_rows=None):
    """Check one tensor argument: its dtype (TypeError) and its shape (ValueError).
    `shape` is the exact shape; with `min_rows`, shape[0] may be any count of at
    least min_rows (a buffer sized for more rows than this call's N_max)."""
    if t is None:
        raise ValueError(f"{name} is required")
    if dtype is not None:
        allowed = dtype if isinstance(dtype, tuple) else (dtype,)
        if t.dtype not in allowed:
            want = " or ".join(str(a) for a in allowed)
            raise TypeError(f"{name} must be {want}, got {t.dtype}")
    if shape is not None:
        got = tuple(t.shape)
        if min_rows is not None:
            ok = len(got) == len(shape) and got[1:] == tuple(shape[1:]) and got[0] >= min_rows
            if not ok:
                raise ValueError(f"{name} must have shape [>= {min_rows}, {', '.join(map(str, shape[1:]))}], "
                                 f"got {list(got)}")
        elif got != tuple(shape):
            raise ValueError(f"{name} must have shape {list(shape)}, got {list(got)}")


def _act_dtypes():
    torch = _torch()
    return (torch.bfloat16, torch.float32)


def _n_max(T: int, k: int, e_begin: int, e_end: int) -> int:
    return T * min(k, e_end - e_begin)


def _expert_weights(w_gate_up, w_down, dtype, d: int, e_begin: int, e_end: int) -> int:
    """Checks the local experts' weights against the activations; returns d_ff."""
    _want(w_down, "w_down", dtype)
    if w_down.dim() != 3:
        raise ValueError(f"w_down must be [E_loc, d_ff, d], got {list(w_down.shape)}")
    e_loc, d_ff = int(w_down.shape[0]), int(w_down.shape[1])
    if e_loc != e_end - e_begin:
        raise ValueError(f"expert weights must hold exactly the {e_end - e_begin} local experts, got {e_loc}")
    _want(w_down, "w_down", dtype, (e_loc, d_ff, d))
    _want(w_gate_up, "w_gate_up", dtype, (e_loc, d, 2 * d_ff))
    return d_ff


def _range(E: int, k: int, e_begin: int, e_end: int) -> None:
    if not 1 <= k <= E:
        raise ValueError(f"need 1 <= k <= E, got k={k}, E={E}")
    if not 0 <= e_begin < e_end <= E:
        raise ValueError(f"local experts [{e_begin}, {e_end}) must be a non-empty range inside [0, {E})")


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
    _want(logits, "logits", torch.float32)
    if logits.dim() != 2:
        raise ValueError(f"logits must be [T, E], got {list(logits.shape)}")
    T, E = (int(v) for v in logits.shape)
    if not 1 <= k <= E:
        raise ValueError(f"need 1 <= k <= E, got k={k}, E={E}")
    if topk_idx is not None:
        _want(topk_idx, "topk_idx", torch.int32, (T, k))
    if topk_w is not None:
        _want(topk_w, "topk_w", torch.float32, (T, k))
    _dev(logits, topk_idx, topk_w)
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
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


def dispatch_workspace_bytes(T: int, k: int, E: int) -> int:
    s = shape(T, 8, 8, E, k, 0, E)
    return int(_load().moe_dispatch_workspace_bytes(ctypes.byref(s)))


def dispatch_alloc(x, k: int, E: int, e_begin: int, e_end: int, gather: bool = True) -> Dispatch:
    """Allocate every dispatch output (sized on the host, no device read); without
    `gather` there is no x_perm (the fused path reads rows straight from x)."""
    torch = _torch()
    T, d = x.shape
    n_max = _n_max(T, k, e_begin, e_end)
    ws_bytes = dispatch_workspace_bytes(T, k, E)
    dev = x.device
    return Dispatch(
        counts=torch.empty(E, dtype=torch.int32, device=dev),
        offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
        perm=torch.empty(T * k, dtype=torch.int32, device=dev),
        pair_pos=torch.empty(T * k, dtype=torch.int32, device=dev),
        x_perm=torch.empty((n_max, d), dtype=x.dtype, device=dev) if gather else None,
        workspace=torch.empty(max(1, ws_bytes), dtype=torch.uint8, device=dev),
    )


def _check_dispatch(out: Dispatch, x, T: int, k: int, E: int, n_max: int, gather: bool) -> None:
    torch = _torch()
    _want(out.counts, "counts", torch.int32, (E,))
    _want(out.offsets, "offsets", torch.int32, (E + 1,))
    _want(out.perm, "perm", torch.int32, (T * k,))
    _want(out.pair_pos, "pair_pos", torch.int32, (T * k,))
    if gather:
        if out.x_perm is None:
            raise ValueError("this Dispatch has no x_perm; allocate it with gather=True")
        _want(out.x_perm, "x_perm", x.dtype, (n_max, x.shape[1]), min_rows=n_max)
    _want(out.workspace, "workspace", torch.uint8)
    need = dispatch_workspace_bytes(T, k, E)
    if out.workspace.numel() < need:
        raise ValueError(f"workspace must hold at least {need} bytes, got {out.workspace.numel()}")


def _debug_word(out: Dispatch, E: int, stream) -> None:
    """Debug mode: wait for the dispatch, then refuse ids outside [0, E)."""
    torch = _torch()
    off = int(_load().moe_dispatch_debug_word_offset())
    if off == _SIZE_MAX:
        return
    (stream if stream is not None else torch.cuda.current_stream()).synchronize()
    bad = int(out.workspace[off:off + 4].view(torch.int32).item())
    if bad:
        raise ValueError(f"moe_dispatch: topk_idx holds {bad} expert id(s) outside [0, {E})")


def dispatch(x, topk_idx, E: int, e_begin: int, e_end: int, out: Dispatch | None = None, stream=None,
             gather: bool = True) -> Dispatch:
    """Histogram, offsets, stable permutation and (with `gather`) the local-row
    gather into x_perm; without it, moe_dispatch_indices (no x_perm)."""
    torch = _torch()
    _want(x, "x", _act_dtypes())
    if x.dim() != 2:
        raise ValueError(f"x must be [T, d], got {list(x.shape)}")
    T, d = (int(v) for v in x.shape)
    _want(topk_idx, "topk_idx", torch.int32)
    if topk_idx.dim() != 2 or topk_idx.shape[0] != T:
        raise ValueError(f"topk_idx must be [T={T}, k], got {list(topk_idx.shape)}")
    k = int(topk_idx.shape[1])
    _range(E, k, e_begin, e_end)
    n_max = _n_max(T, k, e_begin, e_end)
    if out is not None:
        _check_dispatch(out, x, T, k, E, n_max, gather)
    _dev(x, topk_idx)
    if out is None:
        out = dispatch_alloc(x, k, E, e_begin, e_end, gather=gather)
    _dev(out.counts, out.offsets, out.perm, out.pair_pos, out.x_perm if gather else None, out.workspace)
    s = shape(T, d, 8, E, k, e_begin, e_end)
    if gather:
        _check(_load().moe_dispatch(ctypes.byref(s), _dtype_code(x), _ptr(x), _ptr(topk_idx), _ptr(out.counts),
                                    _ptr(out.offsets), _ptr(out.perm), _ptr(out.pair_pos), _ptr(out.x_perm),
                                    _ptr(out.workspace), _stream(stream)), "moe_dispatch")
    else:
        _check(_load().moe_dispatch_indices(ctypes.byref(s), _ptr(topk_idx), _ptr(out.counts), _ptr(out.offsets),
                                            _ptr(out.perm), _ptr(out.pair_pos), _ptr(out.workspace),
                                            _stream(stream)), "moe_dispatch_indices")
    if _debug:
        _debug_word(out, E, stream)
    return out


def dispatch_indices_noalloc(topk_idx, E: int, e_begin: int, e_end: int, counts, offsets, perm, pair_pos,
                             stream=None) -> None:
    """moe_dispatch_indices_noalloc: the dispatch's indices into caller-provided
    buffers, with the library's per-GPU array as workspace (nothing allocated;
    calls that overlap on one GPU race)."""
    torch = _torch()
    _want(topk_idx, "topk_idx", torch.int32)
    if topk_idx.dim() != 2:
        raise ValueError(f"topk_idx must be [T, k], got {list(topk_idx.shape)}")
    T, k = (int(v) for v in topk_idx.shape)
    _range(E, k, e_begin, e_end)
    _want(counts, "counts", torch.int32, (E,))
    _want(offsets, "offsets", torch.int32, (E + 1,))
    _want(perm, "perm", torch.int32, (T * k,))
    _want(pair_pos, "pair_pos", torch.int32, (T * k,))
    _dev(topk_idx, counts, offsets, perm, pair_pos)
    s = shape(T, 8, 8, E, k, e_begin, e_end)
    _check(_load().moe_dispatch_indices_noalloc(ctypes.byref(s), _ptr(topk_idx), _ptr(counts), _ptr(offsets),
                                                _ptr(perm), _ptr(pair_pos), _stream(stream)),
           "moe_dispatch_indices_noalloc")


def _gemm_outputs(h, y, n_max: int, d: int, d_ff: int, dtype, device):
    torch = _torch()
    if h is None:
        h = torch.empty((n_max, d_ff), dtype=dtype, device=device)
    else:
        _want(h, "h", dtype, (n_max, d_ff), min_rows=n_max)
    if y is None:
        y = torch.empty((n_max, d), dtype=dtype, device=device)
    else:
        _want(y, "y", dtype, (n_max, d), min_rows=n_max)
    return h, y


def grouped_gemm(x_perm, offsets, w_gate_up, w_down, T: int, k: int, E: int, e_begin: int, e_end: int,
                 h=None, y=None, stream=None):
    """Local experts' SwiGLU FFN: returns (h [N_max, d_ff], y [N_max, d])."""
    torch = _torch()
    _range(E, k, e_begin, e_end)
    n_max = _n_max(T, k, e_begin, e_end)
    _want(x_perm, "x_perm", _act_dtypes())
    if x_perm.dim() != 2:
        raise ValueError(f"x_perm must be [N_max, d], got {list(x_perm.shape)}")
    d = int(x_perm.shape[1])
    _want(x_perm, "x_perm", x_perm.dtype, (n_max, d), min_rows=n_max)
    _want(offsets, "offsets", torch.int32, (E + 1,))
    d_ff = _expert_weights(w_gate_up, w_down, x_perm.dtype, d, e_begin, e_end)
    h, y = _gemm_outputs(h, y, n_max, d, d_ff, x_perm.dtype, x_perm.device)
    _dev(x_perm, offsets, w_gate_up, w_down, h, y)
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
    _range(E, k, e_begin, e_end)
    _want(x, "x", _act_dtypes())
    if x.dim() != 2:
        raise ValueError(f"x must be [T, d], got {list(x.shape)}")
    T, d = (int(v) for v in x.shape)
    n_max = _n_max(T, k, e_begin, e_end)
    _want(perm, "perm", torch.int32, (T * k,))
    _want(offsets, "offsets", torch.int32, (E + 1,))
    d_ff = _expert_weights(w_gate_up, w_down, x.dtype, d, e_begin, e_end)
    h, y = _gemm_outputs(h, y, n_max, d, d_ff, x.dtype, x.device)
    if gu is not None:
        _want(gu, "gu", x.dtype, (n_max, 2 * d_ff), min_rows=n_max)
    _dev(x, perm, offsets, w_gate_up, w_down, h, y, gu)
    s = shape(T, d, d_ff, E, k, e_begin, e_end)
    dt = _dtype_code(x)
    ws_bytes = _load().moe_grouped_gemm_workspace_bytes(ctypes.byref(s), dt)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device) if ws_bytes else None
    if gu is None:
        _check(_load().moe_grouped_gemm_gather(ctypes.byref(s), dt, _ptr(x), _ptr(perm), _ptr(offsets),
                                               _ptr(w_gate_up), _ptr(w_down), _ptr(h), _ptr(y), _ptr(ws),
                                               _stream(stream)), "moe_grouped_gemm_gather")
    else:
        _check(_load().moe_grouped_gemm_gather_save(ctypes.byref(s), dt, _ptr(x), _ptr(perm), _ptr(offsets),
                                                    _ptr(w_gate_up), _ptr(w_down), _ptr(h), _ptr(y), _ptr(gu),
                                                    _ptr(ws), _stream(stream)), "moe_grouped_gemm_gather_save")
    return h, y


def combine(y, pair_pos, topk_w, T: int, k: int, E: int, e_begin: int, e_end: int, out=None, stream=None):
    """out[t] = sum_j topk_w[t, j] * y[pair_pos[t*k + j]] over local pairs; [T, d]."""
    torch = _torch()
    _range(E, k, e_begin, e_end)
    n_max = _n_max(T, k, e_begin, e_end)
    _want(y, "y", _act_dtypes())
    if y.dim() != 2:
        raise ValueError(f"y must be [N_max, d], got {list(y.shape)}")
    d = int(y.shape[1])
    _want(y, "y", y.dtype, (n_max, d), min_rows=n_max)
    _want(pair_pos, "pair_pos", torch.int32, (T * k,))
    _want(topk_w, "topk_w", torch.float32, (T, k))
    if out is not None:
        _want(out, "out", y.dtype, (T, d))
    _dev(y, pair_pos, topk_w, out)
    if out is None:
        out = torch.empty((T, d), dtype=y.dtype, device=y.device)
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
    if logits.dim() != 2 or logits.shape[0] != T:
        raise ValueError(f"logits must be [T={T}, E], got {list(logits.shape)}")
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
    _range(E, k, e_begin, e_end)
    n_max = _n_max(T, k, e_begin, e_end)
    _want(d_out, "d_out", _act_dtypes())
    if d_out.dim() != 2:
        raise ValueError(f"d_out must be [T, d], got {list(d_out.shape)}")
    d = int(d_out.shape[1])
    _want(d_out, "d_out", d_out.dtype, (T, d))
    _want(y, "y", d_out.dtype, (n_max, d), min_rows=n_max)
    _want(pair_pos, "pair_pos", torch.int32, (T * k,))
    _want(topk_w, "topk_w", torch.float32, (T, k))
    if d_y is not None:
        _want(d_y, "d_y", d_out.dtype, (n_max, d), min_rows=n_max)
    if d_topk_w is not None:
        _want(d_topk_w, "d_topk_w", torch.float32, (T, k))
    _dev(d_out, y, pair_pos, topk_w, d_y, d_topk_w)
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
    _range(E, k, e_begin, e_end)
    _want(x, "x", _act_dtypes())
    if x.dim() != 2:
        raise ValueError(f"x must be [T, d], got {list(x.shape)}")
    T, d = (int(v) for v in x.shape)
    n_max = _n_max(T, k, e_begin, e_end)
    dt_ = x.dtype
    _want(perm, "perm", torch.int32, (T * k,))
    _want(offsets, "offsets", torch.int32, (E + 1,))
    d_ff = _expert_weights(w_gate_up, w_down, dt_, d, e_begin, e_end)
    _want(h, "h", dt_, (n_max, d_ff), min_rows=n_max)
    _want(d_y, "d_y", dt_, (n_max, d), min_rows=n_max)
    if d_x_perm is not None:
        _want(d_x_perm, "d_x_perm", dt_, (n_max, d), min_rows=n_max)
    if d_w_gate_up is not None:
        _want(d_w_gate_up, "d_w_gate_up", dt_, tuple(w_gate_up.shape))
    if d_w_down is not None:
        _want(d_w_down, "d_w_down", dt_, tuple(w_down.shape))
    if gu is not None:
        _want(gu, "gu", dt_, (n_max, 2 * d_ff), min_rows=n_max)
    s = shape(T, d, d_ff, E, k, e_begin, e_end)
    dt = _dtype_code(x)
    ws_bytes = int(_load().moe_grouped_gemm_backward_workspace_bytes(ctypes.byref(s), dt))
    if workspace is not None:
        _want(workspace, "workspace", torch.uint8)
        if workspace.numel() < ws_bytes:
            raise ValueError(f"workspace must hold at least {ws_bytes} bytes, got {workspace.numel()}")
    _dev(x, perm, offsets, w_gate_up, w_down, h, d_y, d_x_perm, d_w_gate_up, d_w_down, gu, workspace)
    if d_x_perm is None:
        d_x_perm = torch.empty((n_max, d), dtype=dt_, device=x.device)
    if d_w_gate_up is None:
        d_w_gate_up = torch.empty_like(w_gate_up)
    if d_w_down is None:
        d_w_down = torch.empty_like(w_down)
    ws = workspace
    if ws is None:
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device) if ws_bytes else None
    if gu is None:
        _check(_load().moe_grouped_gemm_backward(ctypes.byref(s), dt, _ptr(x), _ptr(perm), _ptr(offsets),
                                                 _ptr(w_gate_up), _ptr(w_down), _ptr(h), _ptr(d_y), _ptr(d_x_perm),
                                                 _ptr(d_w_gate_up), _ptr(d_w_down), _ptr(ws), _stream(stream)),
               "moe_grouped_gemm_backward")
    else:
        _check(_load().moe_grouped_gemm_backward_saved(ctypes.byref(s), dt, _ptr(x), _ptr(perm), _ptr(offsets),
                                                       _ptr(w_gate_up), _ptr(w_down), _ptr(h), _ptr(gu), _ptr(d_y),
                                                       _ptr(d_x_perm), _ptr(d_w_gate_up), _ptr(d_w_down), _ptr(ws),
                                                       _stream(stream)), "moe_grouped_gemm_backward_saved")
    return d_x_perm, d_w_gate_up, d_w_down


def dispatch_backward(d_x_perm, pair_pos, T: int, k: int, E: int, e_begin: int, e_end: int, d_x=None, stream=None):
    """d_x [T, d]: the gradient of the row gather."""
    torch = _torch()
    _range(E, k, e_begin, e_end)
    n_max = _n_max(T, k, e_begin, e_end)
    _want(d_x_perm, "d_x_perm", _act_dtypes())
    if d_x_perm.dim() != 2:
        raise ValueError(f"d_x_perm must be [N_max, d], got {list(d_x_perm.shape)}")
    d = int(d_x_perm.shape[1])
    _want(d_x_perm, "d_x_perm", d_x_perm.dtype, (n_max, d), min_rows=n_max)
    _want(pair_pos, "pair_pos", torch.int32, (T * k,))
    if d_x is not None:
        _want(d_x, "d_x", d_x_perm.dtype, (T, d))
    _dev(d_x_perm, pair_pos, d_x)
    if d_x is None:
        d_x = torch.empty((T, d), dtype=d_x_perm.dtype, device=d_x_perm.device)
    s = shape(T, d, 8, E, k, e_begin, e_end)
    _check(_load().moe_dispatch_backward(ctypes.byref(s), _dtype_code(d_x_perm), _ptr(d_x_perm), _ptr(pair_pos),
                                         _ptr(d_x), _stream(stream)), "moe_dispatch_backward")
    return d_x


def route_topk_backward(topk_idx, topk_w, d_topk_w, E: int, d_logits=None, stream=None):
    """d_logits [T, E] fp32: the gradient of route_topk's weights w.r.t. the logits."""
    torch = _torch()
    _want(topk_idx, "topk_idx", torch.int32)
    if topk_idx.dim() != 2:
        raise ValueError(f"topk_idx must be [T, k], got {list(topk_idx.shape)}")
    T, k = (int(v) for v in topk_idx.shape)
    if not 1 <= k <= E:
        raise ValueError(f"need 1 <= k <= E, got k={k}, E={E}")
    _want(topk_w, "topk_w", torch.float32, (T, k))
    _want(d_topk_w, "d_topk_w", torch.float32, (T, k))
    if d_logits is not None:
        _want(d_logits, "d_logits", torch.float32, (T, E))
    _dev(topk_idx, topk_w, d_topk_w, d_logits)
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
