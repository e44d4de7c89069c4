"""GPU parity of the backward path against the fp64 backward oracle.

moe.layer (fused forward) then moe.layer_backward on a seeded d_out; every
gradient is compared with oracle.moe_layer_backward on the same bf16 inputs:
max|err| / max|ref| within the bf16 tolerance (the GPU rounds y, h, the
recomputed gate/up pre-activations and the intermediate gradients to bf16; the
oracle rounds nothing).
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

TOL = g.TOL["bf16"]


def _d_out(w):
    rng = np.random.default_rng(w.seed + 500)
    return mi.f32_to_bf16_bits(rng.standard_normal((w.T, w.d)).astype(np.float32))


def _backward_case(w, logits=None):
    if logits is None:
        logits = mi.router_logits(w)
    x = mi.hidden_states(w)
    wgu, wdn = mi.expert_weights(w)
    d_out = _d_out(w)
    print(f"case {w}", flush=True)
    dx, dl = g.to_dev(x, "bf16"), g.to_dev(logits, "f32")
    dgu, ddn = g.to_dev(wgu, "bf16"), g.to_dev(wdn, "bf16")
    fwd = moe.layer(dx, dl, dgu, ddn, w.k, w.e_begin, w.e_end, fused=True)
    bwd = moe.layer_backward(dx, dgu, ddn, fwd, g.to_dev(d_out, "bf16"), w.k, w.e_begin, w.e_end)
    torch.cuda.synchronize()
    x64, wgu64, wdn64 = mi.to_f64(x, "bf16"), mi.to_f64(wgu, "bf16"), mi.to_f64(wdn, "bf16")
    ref = oracle.moe_layer_backward(x64, logits, w.k, w.e_begin, w.e_end, list(wgu64), list(wdn64),
                                    mi.to_f64(d_out, "bf16"))
    n_loc = ref["x_perm"].shape[0]
    errs = {}
    if n_loc:
        errs["d_y"] = g.rel_err(g.to_f64(bwd["d_y"][:n_loc]), ref["d_y"])
        errs["d_x_perm"] = g.rel_err(g.to_f64(bwd["d_x_perm"][:n_loc]), ref["d_x_perm"])
        errs["d_w"] = g.rel_err(bwd["d_w"].cpu().numpy().astype(np.float64), ref["d_w"])
        errs["d_logits"] = g.rel_err(bwd["d_logits"].cpu().numpy().astype(np.float64), ref["d_logits"])
        errs["d_x"] = g.rel_err(g.to_f64(bwd["d_x"]), ref["d_x"])
    for name in ("d_w_gate_up", "d_w_down"):
        got = g.to_f64(bwd[name])
        if np.any(ref[name]):
            errs[name] = g.rel_err(got, ref[name])
        else:
            assert np.all(got == 0), name
    print("  " + ", ".join(f"{k_}={v:.2e}" for k_, v in errs.items()), flush=True)
    for name, err in errs.items():
        assert err <= TOL, (name, err)
    # gradients of pairs that are not local are exactly zero
    pp = ref["pair_pos"].reshape(w.T, w.k)
    assert np.all(bwd["d_w"].cpu().numpy()[pp < 0] == 0)
    no_local = ~(pp >= 0).any(axis=1)
    assert np.all(g.to_f64(bwd["d_x"])[no_local] == 0)
    # experts without rows get zero weight gradients
    counts = np.diff(ref["offsets"])[w.e_begin:w.e_end]
    for el in np.flatnonzero(counts == 0):
        assert torch.count_nonzero(bwd["d_w_gate_up"][el]).item() == 0
        assert torch.count_nonzero(bwd["d_w_down"][el]).item() == 0
    return fwd, bwd, ref


CASES = [
    mi.Workload("bwd_small", 600, 256, 160, 8, 2, 0, 8, "bf16", 41),
    mi.Workload("bwd_share", 900, 192, 128, 32, 4, 8, 16, "bf16", 42),
    mi.Workload("bwd_skew", 1000, 320, 128, 64, 8, 0, 16, "bf16", 43, 1.5),   # skewed, empty experts
    mi.Workload("bwd_decode", 5, 256, 192, 128, 4, 0, 128, "bf16", 44),       # mostly empty experts
    mi.Workload("bwd_ragged_dims", 700, 288, 96, 8, 2, 0, 8, "bf16", 45),    # d, d_ff not multiples of 256
]


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_layer_backward_matches_oracle(w):
    _backward_case(w)


def _one_hot_logits(counts, E, seed):
    rng = np.random.default_rng(seed)
    T = int(sum(counts))
    owner = np.repeat(np.arange(E), counts)
    rng.shuffle(owner)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[np.arange(T), owner] += 50.0
    return logits


def test_backward_every_row_count():
    """Expert row counts at the edges of the row tiles (forward and NT) and of the
    32-row K stages of the weight gradients, including empty experts."""
    counts = [0, 1, 31, 32, 33, 63, 64, 65, 255, 256, 257, 300, 0, 513]
    E = len(counts)
    w = mi.Workload("bwd_rows", int(sum(counts)), 256, 160, E, 1, 0, E, "bf16", 46)
    _backward_case(w, _one_hot_logits(counts, E, 46))


def test_backward_zero_tokens_writes_zero_weight_gradients():
    w = mi.Workload("bwd_empty", 0, 64, 64, 8, 2, 0, 8, "bf16", 47)
    wgu, wdn = mi.expert_weights(w)
    dgu, ddn = g.to_dev(wgu, "bf16"), g.to_dev(wdn, "bf16")
    offsets = torch.zeros(w.E + 1, dtype=torch.int32, device="cuda")
    x = torch.empty((0, w.d), dtype=torch.bfloat16, device="cuda")
    perm = torch.empty(0, dtype=torch.int32, device="cuda")
    h = torch.empty((0, w.d_ff), dtype=torch.bfloat16, device="cuda")
    d_y = torch.empty((0, w.d), dtype=torch.bfloat16, device="cuda")
    d_wgu = torch.full_like(dgu, 3.0)
    d_wdn = torch.full_like(ddn, 3.0)
    moe.grouped_gemm_backward(x, perm, offsets, dgu, ddn, h, d_y, w.k, w.E, w.e_begin, w.e_end,
                              d_w_gate_up=d_wgu, d_w_down=d_wdn)
    torch.cuda.synchronize()
    assert torch.count_nonzero(d_wgu).item() == 0 and torch.count_nonzero(d_wdn).item() == 0


def test_backward_rejects_unsupported_shapes():
    x = torch.zeros((16, 72), dtype=torch.bfloat16, device="cuda")  # d not a multiple of 32
    perm = torch.zeros(32, dtype=torch.int32, device="cuda")
    offsets = torch.zeros(9, dtype=torch.int32, device="cuda")
    wgu = torch.zeros((8, 72, 128), dtype=torch.bfloat16, device="cuda")
    wdn = torch.zeros((8, 64, 72), dtype=torch.bfloat16, device="cuda")
    h = torch.zeros((32, 64), dtype=torch.bfloat16, device="cuda")
    d_y = torch.zeros((32, 72), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoeError) as e:
        moe.grouped_gemm_backward(x, perm, offsets, wgu, wdn, h, d_y, 2, 8, 0, 8)
    assert e.value.status == moe.MOE_EUNSUPPORTED


@pytest.mark.parametrize("w", [CASES[1], CASES[2]], ids=[CASES[1].name, CASES[2].name])
def test_backward_ignores_workspace_contents(w):
    """The workspace's rows past N_loc are never written; the gradients must not
    read them. Filled with NaN (0xFFFF) or with zeros before the call, both
    backward entry points give the same bits (the last expert's row count is not a
    multiple of 32 here, so the weight gradients' last K stage ends inside a block
    of the workspace's [dG | dU])."""
    logits = mi.router_logits(w)
    x = mi.hidden_states(w)
    wgu, wdn = mi.expert_weights(w)
    print(f"case {w}", flush=True)
    dx, dl = g.to_dev(x, "bf16"), g.to_dev(logits, "f32")
    dgu, ddn = g.to_dev(wgu, "bf16"), g.to_dev(wdn, "bf16")
    fwd = moe.layer(dx, dl, dgu, ddn, w.k, w.e_begin, w.e_end, fused=True, save=True)
    offs = fwd["offsets"].cpu().numpy()
    n_loc = int(offs[w.e_end] - offs[w.e_begin])
    n_max = w.T * min(w.k, w.E_loc)
    last = [int(c) for c in np.diff(offs)[w.e_begin:w.e_end] if c > 0][-1]
    assert n_loc < n_max and last % 32 != 0, (n_loc, n_max, last)
    rng = np.random.default_rng(w.seed + 900)
    d_y = g.to_dev(mi.f32_to_bf16_bits(rng.standard_normal((n_max, w.d)).astype(np.float32)), "bf16")
    ws_bytes = moe.grouped_gemm_backward_workspace_bytes(w.T, w.d, w.d_ff, w.E, w.k, w.e_begin, w.e_end)
    for gu in (None, fwd["gu"]):
        outs = []
        for fill in (0xFF, 0x00):
            ws = torch.full((ws_bytes,), fill, dtype=torch.uint8, device="cuda")
            outs.append(moe.grouped_gemm_backward(dx, fwd["perm"], fwd["offsets"], dgu, ddn, fwd["h"], d_y, w.k, w.E,
                                                  w.e_begin, w.e_end, workspace=ws, gu=gu))
        torch.cuda.synchronize()
        (dxp0, dgu0, ddn0), (dxp1, dgu1, ddn1) = outs
        assert torch.equal(dxp0[:n_loc].view(torch.int16), dxp1[:n_loc].view(torch.int16))
        assert torch.equal(dgu0.view(torch.int16), dgu1.view(torch.int16))
        assert torch.equal(ddn0.view(torch.int16), ddn1.view(torch.int16))
        assert not torch.isnan(dgu0.float()).any()


# ----------------------------------------------------------------------------- kept pre-activations

def _split_counts(counts):
    return counts + [0] * (64 - len(counts))


SAVED = [
    (CASES[0], None), (CASES[2], None), (CASES[3], None), (CASES[4], None),
    # one height class among 64 experts: every tile of both launches at half width
    (mi.Workload("saved_split_over128", 3581, 320, 160, 64, 1, 0, 64, "bf16", 48),
     [129, 255, 256, 257, 288, 289, 300, 350, 400, 513, 544]),
    (mi.Workload("saved_split_to32", 80, 320, 160, 64, 1, 0, 64, "bf16", 49), [1, 16, 31, 32]),
    (mi.Workload("saved_split_to128", 293, 320, 160, 64, 1, 0, 64, "bf16", 50), [65, 100, 128]),
    # gathered rows through their blocked copy (d_ff / 128 = 20 column tiles, N_max / E_loc = 150)
    (mi.Workload("saved_blocked_rows", 600, 128, 2560, 8, 2, 0, 8, "bf16", 51), None),
]


@pytest.mark.parametrize("w,counts", SAVED, ids=[w.name for w, _ in SAVED])
def test_saved_preactivations_match_recompute(w, counts):
    """moe_grouped_gemm_gather_save writes the same h, y (and so out) as the plain
    fused forward, and [G | U] matching the oracle's pre-activations; the backward
    that reads them (moe_grouped_gemm_backward_saved) gives every gradient bit for
    bit as the one that recomputes them."""
    logits = mi.router_logits(w) if counts is None else _one_hot_logits(_split_counts(counts), w.E, w.seed)
    if counts is not None:
        assert int(sum(counts)) == w.T
    x = mi.hidden_states(w)
    wgu, wdn = mi.expert_weights(w)
    d_out = g.to_dev(_d_out(w), "bf16")
    print(f"case {w}", flush=True)
    dx, dl = g.to_dev(x, "bf16"), g.to_dev(logits, "f32")
    dgu, ddn = g.to_dev(wgu, "bf16"), g.to_dev(wdn, "bf16")
    plain = moe.layer(dx, dl, dgu, ddn, w.k, w.e_begin, w.e_end, fused=True)
    kept = moe.layer(dx, dl, dgu, ddn, w.k, w.e_begin, w.e_end, fused=True, save=True)
    b_plain = moe.layer_backward(dx, dgu, ddn, plain, d_out, w.k, w.e_begin, w.e_end)
    b_kept = moe.layer_backward(dx, dgu, ddn, kept, d_out, w.k, w.e_begin, w.e_end)
    torch.cuda.synchronize()
    n_loc = int(plain["offsets"][w.e_end] - plain["offsets"][w.e_begin])
    for key in ("h", "y"):
        assert torch.equal(kept[key][:n_loc].view(torch.int16), plain[key][:n_loc].view(torch.int16)), key
    assert torch.equal(kept["out"].view(torch.int16), plain["out"].view(torch.int16))
    # [G | U] against the oracle's gate/up product of the same rows
    ref = oracle.moe_layer(mi.to_f64(x, "bf16"), logits, w.k, w.e_begin, w.e_end, mi.to_f64(wgu, "bf16"),
                           mi.to_f64(wdn, "bf16"))
    offs = ref["offsets"]
    base = offs[w.e_begin]
    gu_gpu = g.to_f64(kept["gu"][:n_loc])
    gu_ref = np.zeros_like(gu_gpu)
    wgu64 = mi.to_f64(wgu, "bf16")
    for e in range(w.e_begin, w.e_end):
        r0, r1 = offs[e] - base, offs[e + 1] - base
        if r1 > r0:
            gu_ref[r0:r1] = ref["x_perm"][r0:r1] @ wgu64[e - w.e_begin]
    if n_loc:
        assert g.rel_err(gu_gpu, gu_ref) <= TOL
    for key in ("d_y", "d_w", "d_x_perm", "d_w_gate_up", "d_w_down", "d_x", "d_logits"):
        a, b = b_kept[key], b_plain[key]
        if key in ("d_y", "d_x_perm"):  # rows [0, N_loc) are written, the rest left as they were
            a, b = a[:n_loc], b[:n_loc]
        if a.dtype == torch.bfloat16:
            a, b = a.view(torch.int16), b.view(torch.int16)
        assert torch.equal(a, b), key


def test_saved_entry_points_reject_a_missing_buffer():
    w = CASES[0]
    x = torch.zeros((w.T, w.d), dtype=torch.bfloat16, device="cuda")
    perm = torch.zeros(w.T * w.k, dtype=torch.int32, device="cuda")
    offsets = torch.zeros(w.E + 1, dtype=torch.int32, device="cuda")
    wgu = torch.zeros((w.E_loc, w.d, 2 * w.d_ff), dtype=torch.bfloat16, device="cuda")
    wdn = torch.zeros((w.E_loc, w.d_ff, w.d), dtype=torch.bfloat16, device="cuda")
    n_max = w.T * min(w.k, w.E_loc)
    h = torch.empty((n_max, w.d_ff), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((n_max, w.d), dtype=torch.bfloat16, device="cuda")
    s = moe.shape(w.T, w.d, w.d_ff, w.E, w.k, w.e_begin, w.e_end)
    import ctypes
    lib = moe.lib()
    st = lib.moe_grouped_gemm_gather_save(ctypes.byref(s), moe.MOE_BF16, x.data_ptr(), perm.data_ptr(),
                                          offsets.data_ptr(), wgu.data_ptr(), wdn.data_ptr(), h.data_ptr(),
                                          y.data_ptr(), None, None, None)
    assert st == moe.MOE_EINVAL
    st = lib.moe_grouped_gemm_backward_saved(ctypes.byref(s), moe.MOE_BF16, x.data_ptr(), perm.data_ptr(),
                                             offsets.data_ptr(), wgu.data_ptr(), wdn.data_ptr(), h.data_ptr(), None,
                                             y.data_ptr(), y.data_ptr(), wgu.data_ptr(), wdn.data_ptr(), None, None)
    assert st == moe.MOE_EINVAL
