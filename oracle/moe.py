"""Plain, slow, fp64 CPU oracle of one rank's MoE expert-layer forward.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline may import this module; the GPU path never routes through it.

It follows the pages' statement of the problem step by step, with no blocking,
fusion or reordering beyond what each step's definition states. Sources:
  [EP]  "Paralelismo de especialistas" (transformers v5.23.0 docs, pt), with its
        translations "Uzman paralelliği" (tr) and "专家并行" (zh) of transformers main;
  [TP]  "Paralelismo de tensor para inferência" (transformers main docs, pt);
  [UP]  "Ultra-Scale Playbook, часть 3" (ru), section "Экспертный параллелизм".

Readings where the pages are silent (each is also listed with its reason in the
design notes of the repository):
  * combine weights = softmax over the k selected logits;
  * top-k ties go to the lower expert id; -0.0 and +0.0 are equal logits;
  * the k slots of a token are ordered by descending logit, then ascending id;
  * pairs inside an expert's segment keep flat-pair order p = t*k + j;
  * counts cover all E experts; the local segment is a slice of them;
  * SwiGLU = silu(gate) * up with gate = the first d_ff columns of gate_up;
  * the routing weight is applied after the down projection, in the combine;
  * tokens with no local pair get an all-zero output row.

Every array is a numpy array; floating inputs are the exact values the device
sees (bf16 inputs widened without rounding), arithmetic is fp64 and there is no
intermediate rounding.

Pins: see tests/test_oracle.py. The final layer output values have no numeric
worked example on the pages; they are pinned by the closed forms, the
brute-force dense evaluation, the rank-sum identity and the identity-expert
round trip built there.
"""
from __future__ import annotations

import numpy as np


def expert_range(E: int, ep: int, rank: int) -> tuple[int, int]:
    """Local experts [lo, hi) of `rank` under expert parallelism of size `ep`.

    [EP] "Como os tamanhos se combinam" and its rank/expert diagram: ep_size cuts
    the expert list into ep_size contiguous blocks, each rank computes
    num_experts / ep_size of them, and ep_size consecutive ranks hold a full set
    (so the block repeats every ep ranks). ep must divide E ("Sobrescrevendo os
    planos" launch note; [TP] EpRouterParallel row).
    """
    if ep < 1 or E % ep != 0:
        raise ValueError(f"ep={ep} must divide E={E}")
    if rank < 0:
        raise ValueError("rank must be >= 0")
    per = E // ep
    r = rank % ep
    return r * per, (r + 1) * per


def route_topk(logits: np.ndarray, k: int) -> tuple[np.ndarray, np.ndarray]:
    """Router top-k and combine weights.

    [EP] intro: each token activates only a few experts; "Adicionando uma
    implementação": the implementation receives top_k_index and top_k_weights.
    For each token t the experts are ordered by the key (-logit[t, e], e) and the
    first k are taken; weights are the softmax of the k selected logits.

    Returns idx int64 [T, k] (global expert ids) and w float64 [T, k].
    """
    logits = np.asarray(logits)
    T, E = logits.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    vals = logits.astype(np.float64)
    vals = vals + 0.0  # -0.0 + 0.0 == +0.0: signed zeros compare as one value
    ids = np.broadcast_to(np.arange(E), (T, E))
    # np.lexsort sorts by the last key first: primary -logit, secondary id
    order = np.lexsort((ids, -vals), axis=-1)
    idx = order[:, :k].astype(np.int64)
    sel = np.take_along_axis(vals, idx, axis=1)
    ex = np.exp(sel - sel[:, :1])
    w = ex / ex.sum(axis=1, keepdims=True)
    return idx, w


def dispatch(idx: np.ndarray, E: int, e_lo: int, e_hi: int, x: np.ndarray):
    """Token dispatch on one rank: histogram, offsets, permutation, row gather.

    [EP] "Despacho de tokens": every (token, expert) pair goes to the rank that
    owns the expert, which runs its local experts on what it receives; no rank
    computes experts for tokens it does not own. Ownership is contiguous ("Como
    os tamanhos se combinam"), so a rank's pairs are one contiguous segment of
    the expert-sorted pair list. [TP] EpRouterParallel: only local experts run,
    addressed by local ids.

    Returns
      counts   int64 [E]      pairs per expert, all experts (sums to T*k)
      offsets  int64 [E+1]    exclusive prefix sum of counts
      perm     int64 [T*k]    sorted slot -> flat pair p = t*k + j (stable in p)
      pair_pos int64 [T*k]    flat pair -> local row, or -1 for a non-local pair
      x_perm   float  [N_loc, d] row r = x[token of the pair at local row r]
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    flat = idx.reshape(-1)
    counts = np.bincount(flat, minlength=E).astype(np.int64)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    perm = np.argsort(flat, kind="stable").astype(np.int64)
    seg0, seg1 = offsets[e_lo], offsets[e_hi]
    pair_pos = np.full(T * k, -1, dtype=np.int64)
    pair_pos[perm[seg0:seg1]] = np.arange(seg1 - seg0)
    x_perm = np.asarray(x)[perm[seg0:seg1] // k]
    return counts, offsets, perm, pair_pos, x_perm


def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z / (1 + exp(-z)), written to stay finite for large |z|."""
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = z[pos] / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = z[~pos] * ez / (1.0 + ez)
    return out


def swiglu_hidden(rows: np.ndarray, w_gate_up: np.ndarray) -> np.ndarray:
    """H = silu(gate) * up for one expert's rows, gate/up from the packed weight.

    [TP] "Estratégias empacotadas": gate_up = x @ gate_up_proj, then
    chunk(2, dim=-1) gives gate (first half of the columns) and up (second half).
    """
    w_gate_up = np.asarray(w_gate_up, dtype=np.float64)
    d_ff = w_gate_up.shape[1] // 2
    g = np.asarray(rows, dtype=np.float64) @ w_gate_up
    return silu(g[:, :d_ff]) * g[:, d_ff:]


def expert_ffn(rows: np.ndarray, w_gate_up: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """One expert's SwiGLU FFN on its rows.

    [TP] "Estratégias empacotadas": gate_up_proj has shape [hidden, 2*expert_dim]
    per expert; gate_up = x @ gate_up_proj, then chunk(2, dim=-1) gives gate
    (first half) and up (second half). The activation is SwiGLU,
    silu(gate) * up; the down projection [d_ff, d] follows ([EP] plan entry
    "mlp.experts.down_proj" with rule "grouped_gemm").
    """
    return swiglu_hidden(rows, w_gate_up) @ np.asarray(w_down, dtype=np.float64)


def grouped_experts(x_perm: np.ndarray, offsets: np.ndarray, e_lo: int, e_hi: int,
                    w_gate_up, w_down, return_hidden: bool = False):
    """experts_forward of [EP] "Adicionando uma implementação": run each local
    expert on its contiguous segment of x_perm. w_gate_up / w_down are indexed
    by local expert (sharded along the expert dimension, [EP] GroupedGemmParallel)
    and may be arrays or callables e -> matrix. Experts with no rows are skipped.

    Each segment is expert_ffn taken in its two steps, H = swiglu_hidden(rows)
    then Y = H @ W_dn. Returns Y [N_loc, d], or (H [N_loc, d_ff], Y) with
    return_hidden.
    """
    x_perm = np.asarray(x_perm, dtype=np.float64)
    d = x_perm.shape[1] if x_perm.ndim == 2 else 0
    base = offsets[e_lo]
    y = np.zeros((x_perm.shape[0], d), dtype=np.float64)
    h = None
    for e in range(e_lo, e_hi):
        r0, r1 = offsets[e] - base, offsets[e + 1] - base
        if r1 == r0:
            continue
        wgu = w_gate_up(e - e_lo) if callable(w_gate_up) else w_gate_up[e - e_lo]
        wdn = w_down(e - e_lo) if callable(w_down) else w_down[e - e_lo]
        h_e = swiglu_hidden(x_perm[r0:r1], wgu)
        if return_hidden:
            if h is None:
                h = np.zeros((x_perm.shape[0], h_e.shape[1]), dtype=np.float64)
            h[r0:r1] = h_e
        y[r0:r1] = h_e @ np.asarray(wdn, dtype=np.float64)
    if return_hidden:
        return (h if h is not None else np.zeros((x_perm.shape[0], 0))), y
    return y


def combine(y: np.ndarray, pair_pos: np.ndarray, w: np.ndarray, T: int, k: int, d: int) -> np.ndarray:
    """Weighted combine back to token order.

    [EP] "Despacho de tokens": results come back and are combined with the
    routing weights; "Adicionando uma implementação": the output is the weighted
    expert output for each token this rank holds. Only local pairs contribute
    (the partial sum that the masking variant adds up across ranks); a token with
    no local pair gets a zero row. Sum in slot order j = 0..k-1.
    """
    out = np.zeros((T, d), dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    for t in range(T):
        for j in range(k):
            r = pair_pos[t * k + j]
            if r >= 0:
                out[t] += w[t, j] * y[r]
    return out


def moe_layer(x, logits, k: int, e_lo: int, e_hi: int, w_gate_up, w_down):
    """The whole forward of one rank: route -> dispatch -> experts -> combine.

    Returns a dict with every intermediate the GPU path exposes (H included).
    """
    x = np.asarray(x, dtype=np.float64)
    T, d = x.shape
    E = logits.shape[1]
    idx, w = route_topk(logits, k)
    counts, offsets, perm, pair_pos, x_perm = dispatch(idx, E, e_lo, e_hi, x)
    h, y = grouped_experts(x_perm, offsets, e_lo, e_hi, w_gate_up, w_down, return_hidden=True)
    out = combine(y, pair_pos, w, T, k, d)
    return dict(idx=idx, w=w, counts=counts, offsets=offsets, perm=perm,
                pair_pos=pair_pos, x_perm=x_perm, h=h, y=y, out=out)


def brute_force_dense(x, idx, w, e_lo: int, e_hi: int, w_gate_up, w_down) -> np.ndarray:
    """Every local expert on every token, masked by the routing (no dispatch).

    The form in which experts see all tokens ([EP] intro note on Llama 4), used
    only as an independent check of the dispatched result:
    out[t] = sum over slots j with e_lo <= idx[t, j] < e_hi of w[t, j] * FFN_e(x_t).
    """
    x = np.asarray(x, dtype=np.float64)
    T, d = x.shape
    out = np.zeros((T, d), dtype=np.float64)
    for e in range(e_lo, e_hi):
        wgu = w_gate_up(e - e_lo) if callable(w_gate_up) else w_gate_up[e - e_lo]
        wdn = w_down(e - e_lo) if callable(w_down) else w_down[e - e_lo]
        y_all = expert_ffn(x, wgu, wdn)
        for t in range(T):
            for j in range(idx.shape[1]):
                if idx[t, j] == e:
                    out[t] += w[t, j] * y_all[t]
    return out


def token_outputs(tokens, x_rows, idx_rows, w_rows, e_lo: int, e_hi: int, w_gate_up, w_down):
    """The layer output of a few sampled tokens, computed one by one.

    For full-size workloads where the whole oracle is too slow: for each sampled
    token t (with its hidden row, its k routed ids and weights), sum the weighted
    FFN outputs of its local experts. Experts are visited in ascending id so each
    expert's weights are materialised once. Returns [len(tokens), d] fp64.
    """
    x_rows = np.asarray(x_rows, dtype=np.float64)
    n, d = x_rows.shape
    out = np.zeros((n, d), dtype=np.float64)
    k = idx_rows.shape[1]
    for e in range(e_lo, e_hi):
        hits = [(i, j) for i in range(n) for j in range(k) if idx_rows[i, j] == e]
        if not hits:
            continue
        wgu = w_gate_up(e - e_lo) if callable(w_gate_up) else w_gate_up[e - e_lo]
        wdn = w_down(e - e_lo) if callable(w_down) else w_down[e - e_lo]
        rows = np.stack([x_rows[i] for i, _ in hits])
        ys = expert_ffn(rows, wgu, wdn)
        for (i, j), yv in zip(hits, ys):
            out[i] += float(w_rows[i, j]) * yv
    return out
