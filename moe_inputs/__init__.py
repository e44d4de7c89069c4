"""Seeded synthetic inputs for the MoE expert-layer forward (one rank's share).

This module is shared by the tests, the benchmark and the oracle checks. It holds
the workload shapes and the random draws only: no step of the layer's arithmetic
(routing, dispatch, expert FFN, combine) lives here.

Recipe (every draw is reproducible from the workload's seed alone):
  * numpy ``Generator(PCG64)`` fed by ``SeedSequence(seed, spawn_key=...)`` with
    one key per tensor: (0,) router logits, (1,) per-expert router bias,
    (2, blk) hidden states by token block, (3, e, blk) gate/up weights of local
    expert e by row block, (4, e, blk) down weights. Keys are fixed, so any
    expert or block can be drawn alone, in any order, on any thread.
  * router logits ~ N(0, 1) in fp32, plus a per-expert bias ~ N(0, bias_std)
    where the workload asks for load skew;
  * hidden states X ~ N(0, 1); gate/up weights ~ N(0, 1/sqrt(d)); down weights
    ~ N(0, 1/sqrt(d_ff)) (standard deviations);
  * fp32 draws are rounded to bf16 with round-to-nearest-even for bf16 workloads.
Only the rank's local experts [e_begin, e_end) are drawn, since the expert
weights are sharded along the expert dimension (each rank loads only its own).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

_ROW_BLOCK = 512  # rows drawn per generator stream (unit of parallel generation)


@dataclass(frozen=True)
class Workload:
    name: str
    T: int          # tokens held by this rank
    d: int          # hidden size
    d_ff: int       # expert FFN width
    E: int          # global experts
    k: int          # experts per token
    e_begin: int    # first local expert (global id)
    e_end: int      # one past the last local expert
    dtype: str      # "f32" or "bf16" for activations, weights and outputs
    seed: int
    bias_std: float = 0.0  # per-expert router bias (load skew); 0 = none

    @property
    def E_loc(self) -> int:
        return self.e_end - self.e_begin

    @property
    def n_max(self) -> int:
        """Upper bound on local (token, expert) pairs: T * min(k, E_loc)."""
        return self.T * min(self.k, self.E_loc)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads of the headline study, by what they are.
WORKLOADS = {
    # tiny layer, fp32 throughout, all 8 experts local
    "tiny_fp32": Workload("tiny_fp32", 64, 128, 256, 8, 2, 0, 8, "f32", 1001),
    # 8 experts all local, dense-ish: T=4096, d=4096, d_ff=14336, top-2
    "dense8": Workload("dense8", 4096, 4096, 14336, 8, 2, 0, 8, "bf16", 1002),
    # one rank's share at ep=8 of a 128-expert layer (local ids 0-15), top-4
    "ep8_share128": Workload("ep8_share128", 8192, 2880, 2880, 128, 4, 0, 16, "bf16", 1003),
    # fine-grained 256 experts with skewed router bias, rank share ids 0-31, top-8.
    # The bias makes the local pair count swing with the seed: over seeds
    # 1004-1067 it runs from 1413 to 31729 (median 14684). The seed is the first
    # from 1004 up whose count lies within 10 % of that median, a typical batch:
    # 15882 local pairs, 18 of 32 local experts active, the largest with 3757 rows.
    "skew256": Workload("skew256", 16384, 7168, 2048, 256, 8, 0, 32, "bf16", 1008, 1.5),
    # decode-shaped, weight-streaming bound: 128 experts all local, top-4
    "decode32": Workload("decode32", 32, 2880, 2880, 128, 4, 0, 128, "bf16", 1005),
    "decode256": Workload("decode256", 256, 2880, 2880, 128, 4, 0, 128, "bf16", 1006),
}


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round-to-nearest-even); returns uint16 bit patterns.

    Inputs are finite by construction (normal draws), so no NaN handling is needed.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to fp32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_rows(seed: int, key: tuple, rows: int, cols: int, std: float) -> np.ndarray:
    """fp32 N(0, std) draws of shape [rows, cols], in row blocks with keys key+(blk,)."""
    out = np.empty((rows, cols), dtype=np.float32)

    def fill(blk: int) -> None:
        r0 = blk * _ROW_BLOCK
        r1 = min(rows, r0 + _ROW_BLOCK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key + (blk,))))
        g.standard_normal((r1 - r0, cols), dtype=np.float32, out=out[r0:r1])
        if std != 1.0:
            out[r0:r1] *= np.float32(std)

    nblk = (rows + _ROW_BLOCK - 1) // _ROW_BLOCK
    if nblk <= 1:
        for b in range(nblk):
            fill(b)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nblk)))
    return out


def _as_dtype(a32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(a32) if dtype == "bf16" else a32


def router_logits(w: Workload) -> np.ndarray:
    """fp32 [T, E] router logits: N(0,1), plus a per-expert N(0, bias_std) bias if set."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(w.seed, spawn_key=(0,))))
    logits = g.standard_normal((w.T, w.E), dtype=np.float32)
    if w.bias_std > 0:
        gb = np.random.Generator(np.random.PCG64(np.random.SeedSequence(w.seed, spawn_key=(1,))))
        bias = gb.standard_normal(w.E, dtype=np.float32) * np.float32(w.bias_std)
        logits = logits + bias[None, :]
    return np.ascontiguousarray(logits, dtype=np.float32)


def hidden_states(w: Workload) -> np.ndarray:
    """[T, d] hidden states ~ N(0,1): fp32, or bf16 bit patterns (uint16)."""
    return _as_dtype(_normal_rows(w.seed, (2,), w.T, w.d, 1.0), w.dtype)


def gate_up_weight(w: Workload, e_local: int) -> np.ndarray:
    """[d, 2*d_ff] packed gate/up weight of local expert e_local ~ N(0, 1/sqrt(d))."""
    a = _normal_rows(w.seed, (3, e_local), w.d, 2 * w.d_ff, 1.0 / np.sqrt(w.d))
    return _as_dtype(a, w.dtype)


def down_weight(w: Workload, e_local: int) -> np.ndarray:
    """[d_ff, d] down weight of local expert e_local ~ N(0, 1/sqrt(d_ff))."""
    a = _normal_rows(w.seed, (4, e_local), w.d_ff, w.d, 1.0 / np.sqrt(w.d_ff))
    return _as_dtype(a, w.dtype)


def expert_weights(w: Workload):
    """All local experts: (w_gate_up [E_loc, d, 2*d_ff], w_down [E_loc, d_ff, d])."""
    gu = np.stack([gate_up_weight(w, e) for e in range(w.E_loc)])
    dn = np.stack([down_weight(w, e) for e in range(w.E_loc)])
    return gu, dn


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """The exact values a device sees, as fp64 (bf16 bit patterns are widened)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)
