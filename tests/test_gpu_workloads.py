"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times.

Top-k ids, counts, offsets, the permutation and pair positions are checked in
full against the oracle; gathered rows, expert outputs and layer outputs on
samples the oracle computes one by one (rows of x_perm, rows of Y through their
expert's FFN, tokens through oracle.token_outputs, including tokens with no
local pair). The fused path (moe_dispatch_indices + moe_grouped_gemm_gather)
must reproduce the staged path's Y and output bit for bit.
"""
import numpy as np
import pytest

import moe_inputs as mi
import oracle
from tests import _gpu as g

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import token_dispatch_grouped_amd as moe  # noqa: E402

FULL = ["tiny_fp32", "dense8", "ep8_share128", "skew256", "decode32", "decode256"]


@pytest.mark.parametrize("name", FULL)
def test_full_workload_sampled(name):
    w = mi.WORKLOADS[name]
    print(f"workload {w}", flush=True)
    rng = np.random.default_rng(w.seed)
    logits = mi.router_logits(w)
    x = mi.hidden_states(w)
    wgu, wdn = mi.expert_weights(w)
    print("  inputs drawn", flush=True)
    dx, dl = g.to_dev(x, w.dtype), g.to_dev(logits, "f32")
    dgu, ddn = g.to_dev(wgu, w.dtype), g.to_dev(wdn, w.dtype)
    res = moe.layer(dx, dl, dgu, ddn, w.k, w.e_begin, w.e_end)
    torch.cuda.synchronize()
    print("  device layer done", flush=True)
    if w.dtype == "bf16":
        # the fused path (row gather in the GEMM loads) gives the same bits
        fused = moe.layer(dx, dl, dgu, ddn, w.k, w.e_begin, w.e_end, fused=True)
        torch.cuda.synchronize()
        n = int(res["offsets"][w.e_end].item() - res["offsets"][w.e_begin].item())
        assert torch.equal(fused["y"][:n], res["y"][:n])
        assert torch.equal(fused["out"], res["out"])
        del fused
        print("  fused path bit-identical", flush=True)
    del dgu, ddn

    # routing and dispatch in full
    idx, wts = oracle.route_topk(logits, w.k)
    np.testing.assert_array_equal(res["idx"].cpu().numpy(), idx)
    np.testing.assert_allclose(res["w"].cpu().numpy(), wts, rtol=0, atol=g.W_ATOL)
    flat = idx.reshape(-1)
    counts = np.bincount(flat, minlength=w.E)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    perm = np.argsort(flat, kind="stable")
    np.testing.assert_array_equal(res["counts"].cpu().numpy(), counts)
    np.testing.assert_array_equal(res["offsets"].cpu().numpy(), offsets)
    np.testing.assert_array_equal(res["perm"].cpu().numpy(), perm)
    seg0, seg1 = offsets[w.e_begin], offsets[w.e_end]
    n_loc = int(seg1 - seg0)
    pair_pos = np.full(w.T * w.k, -1)
    pair_pos[perm[seg0:seg1]] = np.arange(n_loc)
    np.testing.assert_array_equal(res["pair_pos"].cpu().numpy(), pair_pos)
    print(f"  indices exact, N_loc = {n_loc}", flush=True)
    if n_loc == 0:
        return

    # sampled rows of x_perm (bit copies) and of Y (through the row's expert)
    rows = np.unique(np.concatenate([rng.choice(n_loc, size=min(n_loc, 48), replace=False), [0, n_loc - 1]]))
    tok = perm[seg0 + rows] // w.k
    xp = g.to_f64(res["x_perm"][torch.from_numpy(rows).cuda()])
    x64 = mi.to_f64(x[tok], w.dtype)
    np.testing.assert_array_equal(xp, x64)
    expert_of_row = np.searchsorted(offsets[w.e_begin:w.e_end + 1] - seg0, rows, side="right") - 1
    y_gpu = g.to_f64(res["y"][torch.from_numpy(rows).cuda()])
    y_ref = np.zeros_like(y_gpu)
    for el in np.unique(expert_of_row):
        sel = expert_of_row == el
        y_ref[sel] = oracle.expert_ffn(x64[sel], mi.to_f64(wgu[el], w.dtype), mi.to_f64(wdn[el], w.dtype))
    tol = g.TOL[w.dtype]
    err_y = g.rel_err(y_gpu, y_ref)
    print(f"  sampled Y rows: max|err|/max|ref| = {err_y:.3e}", flush=True)
    assert err_y <= tol

    # sampled tokens of the output, with and without local pairs
    local = ((idx >= w.e_begin) & (idx < w.e_end)).any(axis=1)
    with_local = np.flatnonzero(local)
    without = np.flatnonzero(~local)
    pick = list(rng.choice(with_local, size=min(24, with_local.size), replace=False))
    pick += list(without[:4]) + [0, w.T - 1]
    pick = np.unique(np.array(pick, dtype=np.int64))
    out_gpu = g.to_f64(res["out"][torch.from_numpy(pick).cuda()])
    out_ref = oracle.token_outputs(pick, mi.to_f64(x[pick], w.dtype), idx[pick], wts[pick], w.e_begin, w.e_end,
                                   lambda e: mi.to_f64(wgu[e], w.dtype), lambda e: mi.to_f64(wdn[e], w.dtype))
    err = g.rel_err(out_gpu, out_ref)
    print(f"  sampled tokens: max|err|/max|ref| = {err:.3e}", flush=True)
    assert err <= tol
    for t_i, t in enumerate(pick):
        if not local[t]:
            assert np.all(out_gpu[t_i] == 0.0)
