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


TRAIN = ["dense8", "ep8_share128"]


@pytest.mark.parametrize("name", TRAIN)
def test_full_workload_training_pair_sampled(name):
    """The training pair as `bench.py --train` runs it (forward keeping [G | U],
    backward reading it) at the full workload size. One local expert, the one
    with the most rows, is checked in full against the oracle's
    expert_ffn_backward: its d_w_gate_up, d_w_down and the d_x_perm rows. d_x and
    d_logits are checked on sampled tokens whose local pairs all fall in the two
    largest experts, and on tokens with no local pair, which must get zeros."""
    w = mi.WORKLOADS[name]
    print(f"workload {w}", flush=True)
    rng = np.random.default_rng(w.seed + 7)
    logits = mi.router_logits(w)
    x = mi.hidden_states(w)
    wgu, wdn = mi.expert_weights(w)
    d_out = mi.f32_to_bf16_bits(np.random.default_rng(w.seed + 500).standard_normal((w.T, w.d)).astype(np.float32))
    print("  inputs drawn", flush=True)
    dx, dl = g.to_dev(x, "bf16"), g.to_dev(logits, "f32")
    dgu, ddn = g.to_dev(wgu, "bf16"), g.to_dev(wdn, "bf16")
    fwd = moe.layer(dx, dl, dgu, ddn, w.k, w.e_begin, w.e_end, fused=True, save=True)
    bwd = moe.layer_backward(dx, dgu, ddn, fwd, g.to_dev(d_out, "bf16"), w.k, w.e_begin, w.e_end)
    torch.cuda.synchronize()
    print("  device training step done", flush=True)
    del dgu, ddn

    idx, wts = oracle.route_topk(logits, w.k)
    np.testing.assert_array_equal(fwd["idx"].cpu().numpy(), idx)
    flat = idx.reshape(-1)
    counts = np.bincount(flat, minlength=w.E)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    perm = np.argsort(flat, kind="stable")
    np.testing.assert_array_equal(fwd["perm"].cpu().numpy(), perm)
    seg0 = offsets[w.e_begin]
    tol = g.TOL["bf16"]

    # the largest local expert in full
    local_counts = counts[w.e_begin:w.e_end]
    order = np.argsort(-local_counts, kind="stable")
    el, el2 = int(order[0]), int(order[1])
    e = w.e_begin + el
    r0, r1 = offsets[e] - seg0, offsets[e + 1] - seg0
    pairs = perm[offsets[e]:offsets[e + 1]]
    tok, slot = pairs // w.k, pairs % w.k
    x_rows = mi.to_f64(x[tok], "bf16")
    d_y_rows = wts[tok, slot][:, None] * mi.to_f64(d_out[tok], "bf16")
    wgu64 = {el: mi.to_f64(wgu[el], "bf16"), el2: mi.to_f64(wgu[el2], "bf16")}
    wdn64 = {el: mi.to_f64(wdn[el], "bf16"), el2: mi.to_f64(wdn[el2], "bf16")}
    d_rows_ref, d_wgu_ref, d_wdn_ref = oracle.expert_ffn_backward(x_rows, wgu64[el], wdn64[el], d_y_rows)
    errs = {
        "d_w_gate_up": g.rel_err(g.to_f64(bwd["d_w_gate_up"][el]), d_wgu_ref),
        "d_w_down": g.rel_err(g.to_f64(bwd["d_w_down"][el]), d_wdn_ref),
        "d_x_perm": g.rel_err(g.to_f64(bwd["d_x_perm"][r0:r1]), d_rows_ref),
    }
    print(f"  expert {e} ({r1 - r0} rows): " + ", ".join(f"{k_}={v:.2e}" for k_, v in errs.items()), flush=True)
    for key, err in errs.items():
        assert err <= tol, (key, err)
    del d_wgu_ref, d_wdn_ref, d_rows_ref

    # sampled tokens: every local pair in expert e or e2, and tokens with none
    loc = (idx >= w.e_begin) & (idx < w.e_end)
    in_two = np.isin(idx - w.e_begin, [el, el2]) & loc
    ok = loc.any(axis=1) & ((in_two | ~loc).all(axis=1))
    cand = np.flatnonzero(ok)
    pick = np.sort(rng.choice(cand, size=min(8, cand.size), replace=False))
    none = np.flatnonzero(~loc.any(axis=1))[:4]
    d_x_gpu = g.to_f64(bwd["d_x"][torch.from_numpy(pick).cuda()])
    d_l_gpu = bwd["d_logits"][torch.from_numpy(pick).cuda()].cpu().numpy().astype(np.float64)
    d_x_ref = np.zeros_like(d_x_gpu)
    d_w_ref = np.zeros((pick.size, w.k))
    for i, t in enumerate(pick):
        xt = mi.to_f64(x[t:t + 1], "bf16")
        dot = mi.to_f64(d_out[t:t + 1], "bf16")
        for j in range(w.k):
            if not loc[t, j]:
                continue
            ex = int(idx[t, j]) - w.e_begin
            d_ff = wgu64[ex].shape[1] // 2
            gu = xt @ wgu64[ex]
            y = (oracle.silu(gu[:, :d_ff]) * gu[:, d_ff:]) @ wdn64[ex]
            d_w_ref[i, j] = float(np.dot(dot[0], y[0]))
            d_g, d_u = oracle.swiglu_backward(gu[:, :d_ff], gu[:, d_ff:], (wts[t, j] * dot) @ wdn64[ex].T)
            d_x_ref[i] += (np.concatenate([d_g, d_u], axis=1) @ wgu64[ex].T)[0]
    d_l_ref = oracle.route_topk_backward(logits[pick], w.k, d_w_ref)
    err_x, err_l = g.rel_err(d_x_gpu, d_x_ref), g.rel_err(d_l_gpu, d_l_ref)
    print(f"  sampled tokens: d_x {err_x:.2e}, d_logits {err_l:.2e}", flush=True)
    assert err_x <= tol and err_l <= tol
    if none.size:
        nt = torch.from_numpy(none).cuda()
        assert torch.count_nonzero(bwd["d_x"][nt]).item() == 0
        assert torch.count_nonzero(bwd["d_logits"][nt]).item() == 0
