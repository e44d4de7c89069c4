"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times, element by element against the oracle.

Every workload runs the whole layer on the device and oracle.moe_layer on the
host on the same seeded inputs (the expert weights handed to the oracle one
expert at a time, so host memory stays bounded). Compared:
  * top-k ids, counts, offsets, perm, pair_pos and the gathered rows: bit for
    bit, against oracle.route_topk / oracle.dispatch;
  * routing weights within 1e-6 absolute;
  * every row of H and Y and every token of the output within
    max|err|/max|ref| <= 2e-2 (bf16) or 1e-5 (fp32), over the whole tensor and
    row by row; tokens with no local pair must be exactly zero.
The fused path (moe_dispatch_indices + moe_grouped_gemm_gather, the one the
benchmark times) must reproduce the staged path's H, Y and output bit for bit.

The training pair (`bench.py --train`) is checked the same way against
oracle.moe_layer_backward: d_x and d_logits of every token, d_w_gate_up and
d_w_down of every local expert.
"""
import time

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


class _Experts:
    """Local expert weights widened to fp64 one expert at a time, on access."""

    def __init__(self, a, dtype):
        self.a, self.dtype = a, dtype

    def __getitem__(self, e):
        return mi.to_f64(self.a[e], self.dtype)

    def __call__(self, e):
        return self[e]

    def __len__(self):
        return self.a.shape[0]


def _log(t0, msg):
    print(f"  [{time.perf_counter() - t0:6.1f} s] {msg}", flush=True)


def _compare_rows(name, got, ref, tol, t0, by_row=True):
    """max|err|/max|ref| over the whole tensor and (by_row) row by row, where an
    all-zero reference row counts its largest |value|."""
    err = g.rel_err(got, ref)
    row_err = g.row_rel_err(got, ref) if by_row else float("nan")
    _log(t0, f"{name}: {ref.shape[0]} rows, max|err|/max|ref| = {err:.3e}, worst row {row_err:.3e}")
    assert err <= tol, (name, err)
    if by_row:
        assert row_err <= tol, (name, row_err)


def _indices_exact(res, ref, w):
    np.testing.assert_array_equal(res["idx"].cpu().numpy(), ref["idx"])
    np.testing.assert_allclose(res["w"].cpu().numpy(), ref["w"], rtol=0, atol=g.W_ATOL)
    for key in ("counts", "offsets", "perm", "pair_pos"):
        np.testing.assert_array_equal(res[key].cpu().numpy(), ref[key], err_msg=key)


@pytest.mark.parametrize("name", FULL)
def test_full_workload_matches_oracle(name):
    w = mi.WORKLOADS[name]
    t0 = time.perf_counter()
    print(f"workload {w}", flush=True)
    logits = mi.router_logits(w)
    x = mi.hidden_states(w)
    wgu, wdn = mi.expert_weights(w)
    _log(t0, "inputs drawn")
    dx, dl = g.to_dev(x, w.dtype), g.to_dev(logits, "f32")
    dgu, ddn = g.to_dev(wgu, w.dtype), g.to_dev(wdn, w.dtype)
    res = moe.layer(dx, dl, dgu, ddn, w.k, w.e_begin, w.e_end)
    torch.cuda.synchronize()
    _log(t0, "device layer done (staged)")
    if w.dtype == "bf16":
        fused = moe.layer(dx, dl, dgu, ddn, w.k, w.e_begin, w.e_end, fused=True)
        torch.cuda.synchronize()
        n = int(res["offsets"][w.e_end].item() - res["offsets"][w.e_begin].item())
        for key in ("idx", "counts", "offsets", "perm", "pair_pos"):
            assert torch.equal(fused[key], res[key]), key
        assert torch.equal(fused["h"][:n].view(torch.int16), res["h"][:n].view(torch.int16))
        assert torch.equal(fused["y"][:n].view(torch.int16), res["y"][:n].view(torch.int16))
        assert torch.equal(fused["out"].view(torch.int16), res["out"].view(torch.int16))
        del fused
        _log(t0, "fused path bit-identical to the staged path")
    del dgu, ddn, dx, dl

    ref = oracle.moe_layer(mi.to_f64(x, w.dtype), logits, w.k, w.e_begin, w.e_end,
                           _Experts(wgu, w.dtype), _Experts(wdn, w.dtype))
    _log(t0, "oracle done")
    _indices_exact(res, ref, w)
    n_loc = ref["x_perm"].shape[0]
    np.testing.assert_array_equal(g.to_f64(res["x_perm"][:n_loc]), ref["x_perm"])
    _log(t0, f"indices and gathered rows exact, N_loc = {n_loc}")
    tol = g.TOL[w.dtype]
    if n_loc:
        _compare_rows("H", g.to_f64(res["h"][:n_loc]), ref["h"], tol, t0)
        _compare_rows("Y", g.to_f64(res["y"][:n_loc]), ref["y"], tol, t0)
    out = g.to_f64(res["out"])
    _compare_rows("out", out, ref["out"], tol, t0)
    no_local = (ref["pair_pos"].reshape(w.T, w.k) < 0).all(axis=1)
    assert np.all(out[no_local] == 0.0)
    _log(t0, f"{int(no_local.sum())} tokens without a local pair are zero rows")


TRAIN = ["dense8", "ep8_share128"]


@pytest.mark.parametrize("name", TRAIN)
def test_full_workload_training_pair_matches_oracle(name):
    """The training pair as `bench.py --train` runs it (forward keeping [G | U],
    backward reading it) at the full workload size, against the oracle's
    gradient of every input: d_x and d_logits of every token, d_w_gate_up and
    d_w_down of every local expert (zero for an expert without rows)."""
    w = mi.WORKLOADS[name]
    t0 = time.perf_counter()
    print(f"workload {w}", flush=True)
    logits = mi.router_logits(w)
    x = mi.hidden_states(w)
    wgu, wdn = mi.expert_weights(w)
    d_out = mi.f32_to_bf16_bits(np.random.default_rng(w.seed + 500).standard_normal((w.T, w.d)).astype(np.float32))
    _log(t0, "inputs drawn")
    dx, dl = g.to_dev(x, "bf16"), g.to_dev(logits, "f32")
    dgu, ddn = g.to_dev(wgu, "bf16"), g.to_dev(wdn, "bf16")
    fwd = moe.layer(dx, dl, dgu, ddn, w.k, w.e_begin, w.e_end, fused=True, save=True)
    bwd = moe.layer_backward(dx, dgu, ddn, fwd, g.to_dev(d_out, "bf16"), w.k, w.e_begin, w.e_end)
    torch.cuda.synchronize()
    _log(t0, "device training step done")
    del dgu, ddn, dx, dl

    ref = oracle.moe_layer_backward(mi.to_f64(x, "bf16"), logits, w.k, w.e_begin, w.e_end,
                                    _Experts(wgu, "bf16"), _Experts(wdn, "bf16"), mi.to_f64(d_out, "bf16"))
    _log(t0, "oracle backward done")
    np.testing.assert_array_equal(fwd["idx"].cpu().numpy(), ref["idx"])
    np.testing.assert_array_equal(fwd["perm"].cpu().numpy(), ref["perm"])
    np.testing.assert_array_equal(fwd["pair_pos"].cpu().numpy(), ref["pair_pos"])
    tol = g.TOL["bf16"]
    _compare_rows("out", g.to_f64(fwd["out"]), ref["out"], tol, t0)
    np.testing.assert_allclose(bwd["d_w"].cpu().numpy(), ref["d_w"], rtol=0,
                               atol=tol * max(np.abs(ref["d_w"]).max(), 1e-30))
    _compare_rows("d_x", g.to_f64(bwd["d_x"]), ref["d_x"], tol, t0)
    # a token's d_logits row is proportional to its few routing-weight gradients, each a dot product that
    # may nearly cancel, so only the whole tensor is held to the bound
    _compare_rows("d_logits", bwd["d_logits"].cpu().numpy().astype(np.float64), ref["d_logits"], tol, t0,
                  by_row=False)
    # weight gradients expert by expert (an expert without rows must be exactly zero)
    worst = {"d_w_gate_up": 0.0, "d_w_down": 0.0}
    for el in range(w.E_loc):
        for key in worst:
            got = g.to_f64(bwd[key][el])
            want = ref[key][el]
            if not np.any(want):
                assert not np.any(got), (key, el)
                continue
            err = g.rel_err(got, want)
            worst[key] = max(worst[key], err)
            assert err <= tol, (key, el, err)
    _log(t0, "weight gradients of all experts: " + ", ".join(f"{k_} worst {v:.3e}" for k_, v in worst.items()))
