"""Plain, slow, fp64 CPU oracle of the gradient of one rank's MoE expert-layer
forward.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline may import this module; the GPU path never routes through it.

The pages ask for the backward pass only as the training use of the layer
("Paralelismo de especialistas": gradients flow back to every rank that holds a
token, and the partial outputs of the masking variant are summed across ranks,
so their gradients are too). They print no formula for it, so each function here
is the exact derivative, by the chain rule, of the forward step of the same name
in oracle/moe.py, taken in the reverse order of the forward:

    forward                                  backward
    w = softmax(top-k logits)        <-      d_logits from d_w
    out[t] = sum_j w[t,j] y[p(t,j)]  <-      d_y, d_w from d_out
    y = h @ W_dn                     <-      d_h = d_y @ W_dn^T, d_W_dn = h^T @ d_y
    h = silu(g) * u                  <-      d_g = d_h * u * silu'(g), d_u = d_h * silu(g)
    [g | u] = x_perm @ W_gu          <-      d_x_perm = [d_g | d_u] @ W_gu^T,
                                             d_W_gu = x_perm^T @ [d_g | d_u]
    x_perm = x[token of each pair]   <-      d_x[t] = sum over t's local pairs of d_x_perm

The top-k selection is piecewise constant in the logits, so it contributes no
gradient; only the softmax over the selected logits does.

Pins: tests/test_oracle_backward.py checks every function against central finite
differences of the forward oracle (fp64, inputs chosen so that no selection
changes inside the difference step), plus closed forms and sum identities.
"""
from __future__ import annotations

import numpy as np

from .moe import combine, dispatch, route_topk, silu


def silu_grad(z: np.ndarray) -> np.ndarray:
    """d/dz [z * sigmoid(z)] = sigmoid(z) * (1 + z * (1 - sigmoid(z)))."""
    z = np.asarray(z, dtype=np.float64)
    s = np.empty_like(z)
    pos = z >= 0
    s[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    s[~pos] = ez / (1.0 + ez)
    return s * (1.0 + z * (1.0 - s))


def route_topk_backward(logits: np.ndarray, k: int, d_w: np.ndarray) -> np.ndarray:
    """Gradient w.r.t. the logits [T, E], given d_w = dL/dw [T, k] for the combine
    weights of route_topk. With w = softmax(s) over the selected logits s:
    ds_j = w_j * (d_w_j - sum_i w_i d_w_i); non-selected experts get 0."""
    logits = np.asarray(logits)
    idx, w = route_topk(logits, k)
    d_w = np.asarray(d_w, dtype=np.float64)
    d_sel = w * (d_w - np.sum(w * d_w, axis=1, keepdims=True))
    d_logits = np.zeros(logits.shape, dtype=np.float64)
    np.put_along_axis(d_logits, idx, d_sel, axis=1)
    return d_logits


def combine_backward(d_out: np.ndarray, y: np.ndarray, pair_pos: np.ndarray, w: np.ndarray,
                     T: int, k: int) -> tuple[np.ndarray, np.ndarray]:
    """Gradient of combine: out[t] = sum_j w[t, j] * y[pair_pos[t*k + j]] over local pairs.

    Returns d_y [N_loc, d] (d_y[r] = w[t, j] * d_out[t] for the pair at row r) and
    d_w [T, k] (d_w[t, j] = <d_out[t], y[r]> for a local pair, 0 otherwise)."""
    d_out = np.asarray(d_out, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    d_y = np.zeros_like(y)
    d_w = np.zeros((T, k), dtype=np.float64)
    for t in range(T):
        for j in range(k):
            r = pair_pos[t * k + j]
            if r >= 0:
                d_y[r] = w[t, j] * d_out[t]
                d_w[t, j] = float(np.dot(d_out[t], y[r]))
    return d_y, d_w


def swiglu_backward(g: np.ndarray, u: np.ndarray, d_h: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Gradient of h = silu(g) * u: returns (d_g, d_u)."""
    g = np.asarray(g, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    d_h = np.asarray(d_h, dtype=np.float64)
    return d_h * u * silu_grad(g), d_h * silu(g)


def expert_ffn_backward(rows: np.ndarray, w_gate_up: np.ndarray, w_down: np.ndarray,
                        d_y: np.ndarray) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradient of expert_ffn (y = (silu(g) * u) @ W_dn, [g | u] = rows @ W_gu).

    Returns d_rows [n, d], d_w_gate_up [d, 2 d_ff], d_w_down [d_ff, d]."""
    rows = np.asarray(rows, dtype=np.float64)
    w_gate_up = np.asarray(w_gate_up, dtype=np.float64)
    w_down = np.asarray(w_down, dtype=np.float64)
    d_y = np.asarray(d_y, dtype=np.float64)
    d_ff = w_gate_up.shape[1] // 2
    gu = rows @ w_gate_up
    g, u = gu[:, :d_ff], gu[:, d_ff:]
    h = silu(g) * u
    d_h = d_y @ w_down.T
    d_w_down = h.T @ d_y
    d_g, d_u = swiglu_backward(g, u, d_h)
    d_gu = np.concatenate([d_g, d_u], axis=1)
    return d_gu @ w_gate_up.T, rows.T @ d_gu, d_w_down


def dispatch_backward(d_x_perm: np.ndarray, pair_pos: np.ndarray, T: int, k: int) -> np.ndarray:
    """Gradient of the row gather x_perm[r] = x[token of r]: d_x[t] is the sum of
    d_x_perm over t's local pairs (slot order); zero for tokens without one."""
    d_x_perm = np.asarray(d_x_perm, dtype=np.float64)
    d = d_x_perm.shape[1] if d_x_perm.ndim == 2 else 0
    d_x = np.zeros((T, d), dtype=np.float64)
    for t in range(T):
        for j in range(k):
            r = pair_pos[t * k + j]
            if r >= 0:
                d_x[t] += d_x_perm[r]
    return d_x


def moe_layer_backward(x, logits, k: int, e_lo: int, e_hi: int, w_gate_up, w_down, d_out) -> dict:
    """Gradient of oracle.moe_layer's output, contracted with d_out, w.r.t. x,
    the logits and the local expert weights (the rank's partial gradients; the
    full gradient is their sum over ranks, as for the partial outputs)."""
    x = np.asarray(x, dtype=np.float64)
    T, d = x.shape
    E = logits.shape[1]
    idx, w = route_topk(logits, k)
    counts, offsets, perm, pair_pos, x_perm = dispatch(idx, E, e_lo, e_hi, x)
    base = offsets[e_lo]
    n_loc = x_perm.shape[0]
    e_loc = e_hi - e_lo
    d_ff = np.asarray(w_gate_up[0]).shape[1] // 2 if e_loc else 0
    y = np.zeros((n_loc, d), dtype=np.float64)
    h = np.zeros((n_loc, d_ff), dtype=np.float64)
    for e in range(e_lo, e_hi):
        r0, r1 = offsets[e] - base, offsets[e + 1] - base
        if r1 > r0:
            wgu = np.asarray(w_gate_up[e - e_lo], dtype=np.float64)
            gu = x_perm[r0:r1] @ wgu
            h[r0:r1] = silu(gu[:, :d_ff]) * gu[:, d_ff:]
            y[r0:r1] = h[r0:r1] @ np.asarray(w_down[e - e_lo], dtype=np.float64)
    out = combine(y, pair_pos, w, T, k, d)
    d_y, d_w = combine_backward(d_out, y, pair_pos, w, T, k)
    d_x_perm = np.zeros_like(x_perm)
    d_wgu = np.zeros((e_loc, d, 2 * d_ff), dtype=np.float64)
    d_wdn = np.zeros((e_loc, d_ff, d), dtype=np.float64)
    for e in range(e_lo, e_hi):
        r0, r1 = offsets[e] - base, offsets[e + 1] - base
        if r1 > r0:
            d_x_perm[r0:r1], d_wgu[e - e_lo], d_wdn[e - e_lo] = expert_ffn_backward(
                x_perm[r0:r1], w_gate_up[e - e_lo], w_down[e - e_lo], d_y[r0:r1])
    d_x = dispatch_backward(d_x_perm, pair_pos, T, k)
    d_logits = route_topk_backward(logits, k, d_w)
    return dict(idx=idx, w=w, offsets=offsets, perm=perm, pair_pos=pair_pos, x_perm=x_perm, h=h, y=y, out=out,
                d_y=d_y, d_w=d_w, d_x_perm=d_x_perm, d_x=d_x, d_logits=d_logits, d_w_gate_up=d_wgu,
                d_w_down=d_wdn)
