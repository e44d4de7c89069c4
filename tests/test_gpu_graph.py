"""The whole layer captured in one HIP graph (the decode use the pages give for
a path with no host synchronisation: "Paralelismo de especialistas", the
masking variant that keeps shapes static).

Every step of the layer takes its sizes from the host-side shape and its row
counts from device memory, allocates nothing and never synchronises, so the
four calls capture as they are. Each replay runs on new inputs copied into the
captured buffers, with eager work and synchronisations between replays. It must
equal the eager layer on the same inputs bit for bit, and the oracle on those
inputs (ids exactly, floating results within max|err|/max|ref| <= 2e-2).
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


def _buffers(w, dev):
    T, k = w.T, w.k
    n_max = T * min(k, w.E_loc)
    x = torch.empty((T, w.d), dtype=torch.bfloat16, device=dev)
    logits = torch.empty((T, w.E), dtype=torch.float32, device=dev)
    return dict(
        x=x, logits=logits,
        idx=torch.empty((T, k), dtype=torch.int32, device=dev),
        w=torch.empty((T, k), dtype=torch.float32, device=dev),
        h=torch.empty((n_max, w.d_ff), dtype=torch.bfloat16, device=dev),
        y=torch.empty((n_max, w.d), dtype=torch.bfloat16, device=dev),
        out=torch.empty((T, w.d), dtype=torch.bfloat16, device=dev),
    )


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "staged"])
def test_layer_graph_replays_match_eager(fused):
    w = mi.Workload("graph_decode", 48, 256, 192, 64, 4, 0, 64, "bf16", 31)
    dev = torch.device("cuda:0")
    wgu, wdn = mi.expert_weights(w)
    dgu, ddn = g.to_dev(wgu, "bf16"), g.to_dev(wdn, "bf16")
    b = _buffers(w, dev)
    disp = moe.dispatch_alloc(b["x"], w.k, w.E, w.e_begin, w.e_end, gather=not fused)

    def step():
        moe.route_topk(b["logits"], w.k, b["idx"], b["w"])
        moe.dispatch(b["x"], b["idx"], w.E, w.e_begin, w.e_end, out=disp, gather=not fused)
        if fused:
            moe.grouped_gemm_gather(b["x"], disp.perm, disp.offsets, dgu, ddn, w.k, w.E, w.e_begin, w.e_end,
                                    h=b["h"], y=b["y"])
        else:
            moe.grouped_gemm(disp.x_perm, disp.offsets, dgu, ddn, w.T, w.k, w.E, w.e_begin, w.e_end,
                             h=b["h"], y=b["y"])
        moe.combine(b["y"], disp.pair_pos, b["w"], w.T, w.k, w.E, w.e_begin, w.e_end, out=b["out"])

    def load_inputs(seed):
        rng = np.random.default_rng(seed)
        x = mi.f32_to_bf16_bits(rng.standard_normal((w.T, w.d)).astype(np.float32))
        lg = rng.standard_normal((w.T, w.E)).astype(np.float32)
        b["x"].copy_(g.to_dev(x, "bf16"))
        b["logits"].copy_(g.to_dev(lg, "f32"))
        return x, lg

    load_inputs(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for seed in (1, 2, 3, 4):
        x, lg = load_inputs(seed)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = b["out"].clone()
        got_idx = b["idx"].clone()
        # the eager layer on the same inputs, in separate buffers
        eager = moe.layer(g.to_dev(x, "bf16"), g.to_dev(lg, "f32"), dgu, ddn, w.k, w.e_begin, w.e_end,
                          fused=fused)
        torch.cuda.synchronize()
        assert torch.equal(got_idx, eager["idx"]), seed
        assert torch.equal(got, eager["out"]), seed
        assert torch.count_nonzero(got).item() > 0
        # and the oracle on the replay's inputs
        ref = oracle.moe_layer(mi.to_f64(x, "bf16"), lg, w.k, w.e_begin, w.e_end, mi.to_f64(wgu, "bf16"),
                               mi.to_f64(wdn, "bf16"))
        np.testing.assert_array_equal(got_idx.cpu().numpy(), ref["idx"])
        err = g.rel_err(g.to_f64(got), ref["out"])
        print(f"  replay {seed}: out max|err|/max|ref| = {err:.3e}", flush=True)
        assert err <= g.TOL["bf16"], (seed, err)


def test_training_step_graph_replays_match_eager():
    """Forward keeping the gate/up pre-activations, then the backward that reads
    them, captured as one graph: every replay on new inputs and a new output
    gradient equals the eager training step bit for bit."""
    w = mi.Workload("graph_train", 48, 256, 192, 64, 4, 0, 64, "bf16", 32)
    dev = torch.device("cuda:0")
    wgu, wdn = mi.expert_weights(w)
    dgu, ddn = g.to_dev(wgu, "bf16"), g.to_dev(wdn, "bf16")
    b = _buffers(w, dev)
    n_max = w.T * min(w.k, w.E_loc)
    disp = moe.dispatch_alloc(b["x"], w.k, w.E, w.e_begin, w.e_end, gather=False)
    gu = torch.empty((n_max, 2 * w.d_ff), dtype=torch.bfloat16, device=dev)
    d_out = torch.empty((w.T, w.d), dtype=torch.bfloat16, device=dev)
    d_y = torch.empty((n_max, w.d), dtype=torch.bfloat16, device=dev)
    d_w = torch.empty((w.T, w.k), dtype=torch.float32, device=dev)
    d_xp = torch.empty((n_max, w.d), dtype=torch.bfloat16, device=dev)
    d_wgu, d_wdn = torch.empty_like(dgu), torch.empty_like(ddn)
    d_x = torch.empty((w.T, w.d), dtype=torch.bfloat16, device=dev)
    d_logits = torch.empty((w.T, w.E), dtype=torch.float32, device=dev)
    ws_bytes = moe.grouped_gemm_backward_workspace_bytes(w.T, w.d, w.d_ff, w.E, w.k, w.e_begin, w.e_end)
    bws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

    def step():
        moe.route_topk(b["logits"], w.k, b["idx"], b["w"])
        moe.dispatch(b["x"], b["idx"], w.E, w.e_begin, w.e_end, out=disp, gather=False)
        moe.grouped_gemm_gather(b["x"], disp.perm, disp.offsets, dgu, ddn, w.k, w.E, w.e_begin, w.e_end,
                                h=b["h"], y=b["y"], gu=gu)
        moe.combine(b["y"], disp.pair_pos, b["w"], w.T, w.k, w.E, w.e_begin, w.e_end, out=b["out"])
        moe.combine_backward(d_out, b["y"], disp.pair_pos, b["w"], w.T, w.k, w.E, w.e_begin, w.e_end,
                             d_y=d_y, d_topk_w=d_w)
        moe.grouped_gemm_backward(b["x"], disp.perm, disp.offsets, dgu, ddn, b["h"], d_y, w.k, w.E, w.e_begin,
                                  w.e_end, d_x_perm=d_xp, d_w_gate_up=d_wgu, d_w_down=d_wdn, workspace=bws, gu=gu)
        moe.dispatch_backward(d_xp, disp.pair_pos, w.T, w.k, w.E, w.e_begin, w.e_end, d_x=d_x)
        moe.route_topk_backward(b["idx"], b["w"], d_w, w.E, d_logits=d_logits)

    def load_inputs(seed):
        rng = np.random.default_rng(seed)
        x = mi.f32_to_bf16_bits(rng.standard_normal((w.T, w.d)).astype(np.float32))
        lg = rng.standard_normal((w.T, w.E)).astype(np.float32)
        do = mi.f32_to_bf16_bits(rng.standard_normal((w.T, w.d)).astype(np.float32))
        b["x"].copy_(g.to_dev(x, "bf16"))
        b["logits"].copy_(g.to_dev(lg, "f32"))
        d_out.copy_(g.to_dev(do, "bf16"))
        return x, lg, do

    load_inputs(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for seed in (11, 12, 13):
        x, lg, do = load_inputs(seed)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = {"out": b["out"].clone(), "d_x": d_x.clone(), "d_logits": d_logits.clone(),
               "d_w_gate_up": d_wgu.clone(), "d_w_down": d_wdn.clone()}
        dx_e, dl_e = g.to_dev(x, "bf16"), g.to_dev(lg, "f32")
        fwd = moe.layer(dx_e, dl_e, dgu, ddn, w.k, w.e_begin, w.e_end, fused=True, save=True)
        bwd = moe.layer_backward(dx_e, dgu, ddn, fwd, g.to_dev(do, "bf16"), w.k, w.e_begin, w.e_end)
        torch.cuda.synchronize()
        want = {"out": fwd["out"], "d_x": bwd["d_x"], "d_logits": bwd["d_logits"],
                "d_w_gate_up": bwd["d_w_gate_up"], "d_w_down": bwd["d_w_down"]}
        for key, t in got.items():
            a, e = t, want[key]
            if a.dtype == torch.bfloat16:
                a, e = a.view(torch.int16), e.view(torch.int16)
            assert torch.equal(a, e), (seed, key)
        assert torch.count_nonzero(got["d_w_gate_up"]).item() > 0
        # and the oracle's forward and gradient on the replay's inputs
        ref = oracle.moe_layer_backward(mi.to_f64(x, "bf16"), lg, w.k, w.e_begin, w.e_end,
                                        list(mi.to_f64(wgu, "bf16")), list(mi.to_f64(wdn, "bf16")),
                                        mi.to_f64(do, "bf16"))
        errs = {key: g.rel_err(t.float().cpu().numpy().astype(np.float64), ref[key]) for key, t in got.items()}
        print(f"  replay {seed}: " + ", ".join(f"{k_} {v:.2e}" for k_, v in errs.items()), flush=True)
        for key, err in errs.items():
            assert err <= g.TOL["bf16"], (seed, key, err)
