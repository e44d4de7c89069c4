"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Indices (top-k ids, counts, offsets, permutation, pair positions) and gathered
rows are compared bit for bit; floating results within max|err|/max|ref| of
2e-2 (bf16) or 1e-5 (fp32), routing weights within 1e-6 absolute.
"""
import numpy as np
import pytest

import moe_inputs as mi
import oracle
from tests import _gpu as g

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - collected on CPU hosts too
    pytest.skip("no GPU", allow_module_level=True)

import token_dispatch_grouped_amd as moe  # noqa: E402


def _layer_case(w: mi.Workload, logits=None):
    """Run the layer on the device and the oracle on the host; compare everything."""
    if logits is None:
        logits = mi.router_logits(w)
    x = mi.hidden_states(w)
    wgu, wdn = mi.expert_weights(w)
    print(f"case {w}", flush=True)
    res = moe.layer(g.to_dev(x, w.dtype), g.to_dev(logits, "f32"), g.to_dev(wgu, w.dtype),
                    g.to_dev(wdn, w.dtype), w.k, w.e_begin, w.e_end)
    torch.cuda.synchronize()
    x64, wgu64, wdn64 = mi.to_f64(x, w.dtype), mi.to_f64(wgu, w.dtype), mi.to_f64(wdn, w.dtype)
    ref = oracle.moe_layer(x64, logits, w.k, w.e_begin, w.e_end, wgu64, wdn64)
    np.testing.assert_array_equal(res["idx"].cpu().numpy(), ref["idx"])
    np.testing.assert_allclose(res["w"].cpu().numpy(), ref["w"], rtol=0, atol=g.W_ATOL)
    np.testing.assert_array_equal(res["counts"].cpu().numpy(), ref["counts"])
    np.testing.assert_array_equal(res["offsets"].cpu().numpy(), ref["offsets"])
    np.testing.assert_array_equal(res["perm"].cpu().numpy(), ref["perm"])
    np.testing.assert_array_equal(res["pair_pos"].cpu().numpy(), ref["pair_pos"])
    n_loc = ref["x_perm"].shape[0]
    np.testing.assert_array_equal(g.to_f64(res["x_perm"][:n_loc]), ref["x_perm"])
    # H against the oracle's H on the same rows
    offs = ref["offsets"]
    base = offs[w.e_begin]
    h_gpu = g.to_f64(res["h"][:n_loc])
    h_ref = np.zeros_like(h_gpu)
    for e in range(w.e_begin, w.e_end):
        r0, r1 = offs[e] - base, offs[e + 1] - base
        if r1 > r0:
            h_ref[r0:r1] = oracle.swiglu_hidden(ref["x_perm"][r0:r1], wgu64[e - w.e_begin])
    tol = g.TOL[w.dtype]
    assert g.rel_err(h_gpu, h_ref) <= tol
    assert g.rel_err(g.to_f64(res["y"][:n_loc]), ref["y"]) <= tol
    err = g.rel_err(g.to_f64(res["out"]), ref["out"])
    print(f"  out max|err|/max|ref| = {err:.3e}", flush=True)
    assert err <= tol
    return res, ref


# ----------------------------------------------------------------------------- route top-k

@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (7, 2, 2), (33, 3, 2), (257, 8, 2), (129, 8, 8), (100, 100, 7),
                                   (300, 128, 4), (65, 256, 8), (10, 1024, 3), (3, 1024, 1024), (0, 16, 4),
                                   (77, 512, 16), (50, 64, 6), (90, 1000, 33), (40, 12, 5)])
def test_route_topk_matches_oracle(T, E, k):
    rng = np.random.default_rng(T * 1000 + E * 10 + k)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    idx, w = moe.route_topk(g.to_dev(logits, "f32"), k)
    ref_idx, ref_w = oracle.route_topk(logits, k)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
    np.testing.assert_allclose(w.cpu().numpy(), ref_w, rtol=0, atol=g.W_ATOL)


@pytest.mark.parametrize("E,k", [(8, 2), (128, 4), (256, 8), (40, 40), (512, 16), (1024, 9)])
def test_route_topk_ties_and_signed_zeros(E, k):
    rng = np.random.default_rng(E + k)
    T = 500
    logits = (rng.integers(-2, 3, size=(T, E)) * 0.5).astype(np.float32)  # many exact ties
    logits[rng.random((T, E)) < 0.2] = -0.0
    logits[rng.random((T, E)) < 0.1] = 0.0
    logits[0] = 0.0  # an all-equal row: ids 0..k-1
    idx, w = moe.route_topk(g.to_dev(logits, "f32"), k)
    ref_idx, ref_w = oracle.route_topk(logits, k)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
    np.testing.assert_allclose(w.cpu().numpy(), ref_w, rtol=0, atol=g.W_ATOL)
    np.testing.assert_array_equal(idx.cpu().numpy()[0], np.arange(k))


# ----------------------------------------------------------------------------- dispatch

@pytest.mark.parametrize("T,E,k,lo,hi", [(1, 8, 2, 0, 8), (1000, 8, 2, 0, 8), (1500, 32, 4, 8, 12),
                                         (3000, 256, 8, 0, 32), (2047, 1024, 4, 1000, 1024),
                                         (5, 128, 4, 0, 128), (1025, 16, 16, 3, 4),
                                         # either side of the single-workgroup path (at most 2048 pairs)
                                         (2047, 8, 1, 0, 8), (1024, 1024, 2, 512, 1024), (683, 128, 3, 16, 32),
                                         (1, 1024, 1024, 0, 1024), (256, 256, 8, 0, 32),
                                         # an ep8_share128-sized table (128 experts x 128 chunks) and one chunk more
                                         (8192, 128, 4, 0, 16), (8193, 128, 4, 112, 128)])
def test_dispatch_matches_oracle(T, E, k, lo, hi):
    rng = np.random.default_rng(T + E + k)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[:, lo] += 2.0  # one heavy local expert
    d = 72
    x = mi.f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    idx_np, _ = oracle.route_topk(logits, k)
    idx = torch.from_numpy(idx_np.astype(np.int32)).cuda()
    disp = moe.dispatch(g.to_dev(x, "bf16"), idx, E, lo, hi)
    torch.cuda.synchronize()
    counts, offsets, perm, pair_pos, x_perm = oracle.dispatch(idx_np, E, lo, hi, mi.to_f64(x, "bf16"))
    np.testing.assert_array_equal(disp.counts.cpu().numpy(), counts)
    np.testing.assert_array_equal(disp.offsets.cpu().numpy(), offsets)
    np.testing.assert_array_equal(disp.perm.cpu().numpy(), perm)
    np.testing.assert_array_equal(disp.pair_pos.cpu().numpy(), pair_pos)
    np.testing.assert_array_equal(g.to_f64(disp.x_perm[: x_perm.shape[0]]), x_perm)


def test_dispatch_zero_tokens_writes_zero_counts():
    E = 16
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty((0, 2), dtype=torch.int32, device="cuda")
    disp = moe.dispatch_alloc(x, 2, E, 0, 8)
    disp.counts.fill_(7)
    disp.offsets.fill_(7)
    moe.dispatch(x, idx, E, 0, 8, out=disp)
    torch.cuda.synchronize()
    assert disp.counts.cpu().tolist() == [0] * E
    assert disp.offsets.cpu().tolist() == [0] * (E + 1)


def test_dispatch_drops_out_of_range_ids():
    T, E, k, d = 300, 8, 2, 64
    rng = np.random.default_rng(5)
    idx_np = rng.integers(0, E, size=(T, k)).astype(np.int32)
    bad = rng.random((T, k)) < 0.1
    idx_np[bad] = np.where(rng.random(bad.sum()) < 0.5, -1, E + 3)
    x = mi.f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    disp = moe.dispatch(g.to_dev(x, "bf16"), torch.from_numpy(idx_np).cuda(), E, 0, E)
    torch.cuda.synchronize()
    good = idx_np.reshape(-1)[~bad.reshape(-1)]
    np.testing.assert_array_equal(disp.counts.cpu().numpy(), np.bincount(good, minlength=E))
    pp = disp.pair_pos.cpu().numpy()
    assert np.all(pp[bad.reshape(-1)] == -1)
    assert sorted(pp[~bad.reshape(-1)].tolist()) == list(range(good.size))


# ----------------------------------------------------------------------------- whole layer, small

SMALL = [
    mi.WORKLOADS["tiny_fp32"],  # the full tiny fp32 workload
    mi.Workload("dense8_small", 1200, 328, 200, 8, 2, 0, 8, "bf16", 11),          # K tails, ragged N, 2 row tiles
    mi.Workload("ep_share_small", 900, 256, 264, 32, 4, 8, 12, "bf16", 12),       # 4 of 32 experts local
    mi.Workload("skew_small", 1000, 320, 128, 64, 8, 0, 16, "bf16", 13, 1.5),    # skewed, empty experts
    mi.Workload("decode_small", 5, 256, 192, 128, 4, 0, 128, "bf16", 14),        # mostly empty experts
    mi.Workload("single_token", 1, 64, 64, 8, 2, 0, 8, "bf16", 15),
    mi.Workload("one_local_expert", 700, 128, 136, 8, 3, 5, 6, "bf16", 16),
    mi.Workload("fp32_ragged", 200, 72, 40, 6, 2, 1, 5, "f32", 17),
]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_layer_matches_oracle(w):
    _layer_case(w)


def test_layer_all_tokens_on_one_expert():
    w = mi.Workload("one_hot", 700, 192, 256, 16, 1, 0, 16, "bf16", 18)
    logits = mi.router_logits(w)
    logits[:, 9] += 100.0  # every token's top-1 is expert 9: 700 rows, 3 row tiles
    res, ref = _layer_case(w, logits)
    assert int(ref["counts"][9]) == 700


@pytest.mark.parametrize("w", [mi.Workload("max_experts", 512, 64, 64, 1024, 8, 0, 1024, "bf16", 35),
                               mi.Workload("k_equals_E", 200, 64, 96, 16, 16, 0, 16, "bf16", 36),
                               mi.Workload("k_equals_E_share", 150, 96, 64, 12, 12, 4, 8, "bf16", 37)],
                         ids=["max_experts", "k_equals_E", "k_equals_E_share"])
def test_layer_extreme_expert_counts(w):
    """The largest expert count the library takes (E = E_loc = 1024, so the tile
    map holds 1024 experts, most with a row or none) and the degenerate top-k
    with k = E, every token routed to every expert; the fused path too."""
    res, ref = _layer_case(w)
    logits = mi.router_logits(w)
    x = mi.hidden_states(w)
    wgu, wdn = mi.expert_weights(w)
    fused = moe.layer(g.to_dev(x, w.dtype), g.to_dev(logits, "f32"), g.to_dev(wgu, w.dtype),
                      g.to_dev(wdn, w.dtype), w.k, w.e_begin, w.e_end, fused=True)
    torch.cuda.synchronize()
    assert torch.equal(fused["out"].view(torch.int16), res["out"].view(torch.int16))
    if w.k == w.E:
        assert np.all(ref["counts"] == w.T)


def test_layer_zero_tokens():
    w = mi.Workload("empty", 0, 64, 64, 8, 2, 0, 8, "bf16", 19)
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    logits = torch.empty((0, 8), dtype=torch.float32, device="cuda")
    wgu = torch.zeros((8, 64, 128), dtype=torch.bfloat16, device="cuda")
    wdn = torch.zeros((8, 64, 64), dtype=torch.bfloat16, device="cuda")
    res = moe.layer(x, logits, wgu, wdn, w.k, 0, 8)
    torch.cuda.synchronize()
    assert res["out"].shape == (0, 64)
    assert res["counts"].cpu().tolist() == [0] * 8


def test_rank_sum_on_one_gpu():
    """Masked partial outputs of every rank's share: each equals the oracle's
    partial output of that rank, and they add up to the oracle's full layer."""
    base = mi.Workload("rank_sum", 512, 192, 128, 16, 4, 0, 16, "bf16", 20)
    logits_np, x_np = mi.router_logits(base), mi.hidden_states(base)
    logits = g.to_dev(logits_np, "f32")
    x = g.to_dev(x_np, "bf16")
    wgu_np, wdn_np = mi.expert_weights(base)
    wgu, wdn = g.to_dev(wgu_np, "bf16"), g.to_dev(wdn_np, "bf16")
    x64, wgu64, wdn64 = mi.to_f64(x_np, "bf16"), mi.to_f64(wgu_np, "bf16"), mi.to_f64(wdn_np, "bf16")
    full_ref = oracle.moe_layer(x64, logits_np, base.k, 0, 16, wgu64, wdn64)["out"]
    full = g.to_f64(moe.layer(x, logits, wgu, wdn, base.k, 0, 16)["out"])
    assert g.rel_err(full, full_ref) <= 2e-2
    for ep in (2, 4, 8):
        acc = np.zeros_like(full)
        for r in range(ep):
            lo, hi = moe.expert_range(16, ep, r)
            part = g.to_f64(moe.layer(x, logits, wgu[lo:hi].contiguous(), wdn[lo:hi].contiguous(), base.k, lo,
                                      hi)["out"])
            part_ref = oracle.moe_layer(x64, logits_np, base.k, lo, hi, wgu64[lo:hi], wdn64[lo:hi])["out"]
            assert g.rel_err(part, part_ref) <= 2e-2, (ep, r)
            acc += part
        err = g.rel_err(acc, full_ref)
        assert err <= 2e-2, (ep, err)


def test_identity_expert_round_trip():
    """dispatch then combine with y = x_perm (an identity expert) gives back x."""
    T, E, k, d = 777, 8, 3, 136
    rng = np.random.default_rng(21)
    x_np = mi.f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    x = g.to_dev(x_np, "bf16")
    idx, w = moe.route_topk(g.to_dev(rng.standard_normal((T, E)).astype(np.float32), "f32"), k)
    disp = moe.dispatch(x, idx, E, 0, E)
    out = moe.combine(disp.x_perm, disp.pair_pos, w, T, k, E, 0, E)
    torch.cuda.synchronize()
    # sum_j w_j = 1 in fp32: out equals x up to one bf16 rounding
    assert g.rel_err(g.to_f64(out), mi.to_f64(x_np, "bf16")) <= 2 ** -8


def test_layer_is_deterministic():
    w = mi.Workload("determinism", 1500, 256, 192, 32, 4, 0, 32, "bf16", 22)
    args = (g.to_dev(mi.hidden_states(w), "bf16"), g.to_dev(mi.router_logits(w), "f32"),
            *(g.to_dev(a, "bf16") for a in mi.expert_weights(w)))
    a = moe.layer(*args, w.k, w.e_begin, w.e_end)
    b = moe.layer(*args, w.k, w.e_begin, w.e_end)
    torch.cuda.synchronize()
    n_loc = int(a["offsets"][w.e_end] - a["offsets"][w.e_begin])
    for key in ("perm", "pair_pos", "out", "h", "y"):
        ta, tb = a[key], b[key]
        if key in ("h", "y"):
            ta, tb = ta[:n_loc], tb[:n_loc]
        if ta.dtype == torch.bfloat16:
            ta, tb = ta.view(torch.int16), tb.view(torch.int16)
        assert torch.equal(ta, tb), key


def _one_hot_logits(counts, E, seed):
    """Router logits that send exactly counts[e] tokens to expert e as their top-1."""
    rng = np.random.default_rng(seed)
    T = int(sum(counts))
    owner = np.repeat(np.arange(len(counts)), counts)
    rng.shuffle(owner)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[np.arange(T), owner] += 50.0
    return logits


def test_layer_every_tile_height():
    """Experts whose row counts hit every row-tile height (32/64/128/256, and 256 plus a
    merged tail of up to 32 rows) and the edges between them."""
    counts = [0, 1, 31, 32, 33, 64, 65, 128, 129, 255, 256, 257, 288, 289, 300, 513, 544]
    E = len(counts)
    w = mi.Workload("tile_heights", int(sum(counts)), 256, 160, E, 1, 0, E, "bf16", 23)
    res, ref = _layer_case(w, _one_hot_logits(counts, E, 23))
    top1 = ref["idx"][:, 0]
    assert [int((top1 == e).sum()) for e in range(E)] == counts


def _fused_matches_staged(w, logits, res, ref):
    x = mi.hidden_states(w)
    wgu, wdn = mi.expert_weights(w)
    fused = moe.layer(g.to_dev(x, w.dtype), g.to_dev(logits, "f32"), g.to_dev(wgu, w.dtype),
                      g.to_dev(wdn, w.dtype), w.k, w.e_begin, w.e_end, fused=True)
    torch.cuda.synchronize()
    n_loc = ref["x_perm"].shape[0]
    assert torch.equal(fused["h"][:n_loc], res["h"][:n_loc])
    assert torch.equal(fused["y"][:n_loc], res["y"][:n_loc])
    assert torch.equal(fused["out"], res["out"])


@pytest.mark.parametrize("counts", [
    [129, 255, 256, 257, 288, 289, 300, 350, 400, 513, 544],  # rows > 128: 256/288-row tiles, 64/128/256-row tails
    [65, 100, 128],  # 128-row tiles
    [33, 50, 64],  # 64-row tiles
    [1, 16, 31, 32],  # 32-row tiles
], ids=["over128", "to128", "to64", "to32"])
def test_layer_split_last_round_every_tile_height(counts):
    """Experts of one height class among 64 local experts, the rest empty: the
    grid (sized for the worst case) is more than twice the tile count, so both
    GEMMs run their only round as half-width tiles, and the second half of each
    last column block (d_ff = 160 and d = 320 leave it at most half full) has
    no columns."""
    counts = counts + [0] * (64 - len(counts))
    E = len(counts)
    w = mi.Workload("split_tile_heights", int(sum(counts)), 320, 160, E, 1, 0, E, "bf16", 31)
    logits = _one_hot_logits(counts, E, 31)
    res, ref = _layer_case(w, logits)
    top1 = ref["idx"][:, 0]
    assert [int((top1 == e).sum()) for e in range(E)] == counts
    _fused_matches_staged(w, logits, res, ref)


def test_layer_split_after_full_rounds():
    """64 experts of 77 to 121 rows (one height class) and nine gate/up column
    blocks: 576 tiles, two full rounds on 256 workgroups and a third of 64 tiles
    run as 128 half tiles."""
    w = mi.Workload("split_after_rounds", 3072, 256, 1152, 64, 2, 0, 64, "bf16", 32)
    res, ref = _layer_case(w)
    _fused_matches_staged(w, mi.router_logits(w), res, ref)


REGS = [mi.Workload("regs_skew", 1000, 328, 136, 64, 8, 0, 16, "bf16", 13, 1.5),      # skewed, empty experts
        mi.Workload("regs_decode", 5, 264, 200, 128, 4, 0, 128, "bf16", 14),         # mostly empty experts
        mi.Workload("regs_heights", 600, 264, 200, 8, 2, 0, 8, "bf16", 24),
        mi.Workload("regs_d_only", 700, 328, 192, 8, 2, 0, 8, "bf16", 33),            # d_ff a multiple of 32
        mi.Workload("regs_dff_only", 700, 256, 200, 8, 2, 0, 8, "bf16", 34)]          # d a multiple of 32


@pytest.mark.parametrize("w", REGS, ids=[w.name for w in REGS])
def test_layer_register_staged_kernel(w):
    """The register-staged GEMM, which takes every shape whose d or d_ff is a
    multiple of 8 but not of 32, on skewed, decode-shaped and multi-tile inputs."""
    assert w.d % 32 or w.d_ff % 32
    _layer_case(w)


# ----------------------------------------------------------------------------- fused path (row gather in the GEMM loads)

FUSED = [SMALL[3], SMALL[4], SMALL[5],
         mi.Workload("fused_ragged_experts", 1100, 256, 160, 24, 3, 4, 20, "bf16", 25),
         mi.Workload("fused_partial_range", 640, 192, 128, 16, 4, 6, 10, "bf16", 26),
         # d_ff / 128 = 20 column tiles and N_max / E_loc = 150: the gathered rows go
         # through their blocked copy (moe_grouped_gemm_workspace_bytes > 0)
         mi.Workload("fused_blocked_rows", 600, 128, 2560, 8, 2, 0, 8, "bf16", 28)]


@pytest.mark.parametrize("w", FUSED, ids=[w.name for w in FUSED])
def test_fused_layer_matches_oracle_and_staged_path(w):
    """moe_dispatch_indices + moe_grouped_gemm_gather: the oracle's result, and
    bit for bit the staged path's H, Y and output."""
    res, ref = _layer_case(w)
    logits = mi.router_logits(w)
    x = mi.hidden_states(w)
    wgu, wdn = mi.expert_weights(w)
    fused = moe.layer(g.to_dev(x, w.dtype), g.to_dev(logits, "f32"), g.to_dev(wgu, w.dtype),
                      g.to_dev(wdn, w.dtype), w.k, w.e_begin, w.e_end, fused=True)
    torch.cuda.synchronize()
    assert fused["x_perm"] is None
    n_loc = ref["x_perm"].shape[0]
    for key in ("idx", "counts", "offsets", "perm", "pair_pos"):
        assert torch.equal(fused[key], res[key]), key
    assert torch.equal(fused["h"][:n_loc], res["h"][:n_loc])
    assert torch.equal(fused["y"][:n_loc], res["y"][:n_loc])
    assert torch.equal(fused["out"], res["out"])


@pytest.mark.parametrize("d_ff", [160, 2560], ids=["rows_gathered", "rows_blocked"])
def test_fused_layer_every_tile_height(d_ff):
    counts = [0, 1, 31, 32, 33, 64, 65, 128, 129, 255, 256, 257, 288, 289, 300, 513, 544]
    E = len(counts)
    w = mi.Workload("fused_tile_heights", int(sum(counts)), 256, d_ff, E, 1, 0, E, "bf16", 27)
    s = moe.shape(w.T, w.d, w.d_ff, w.E, w.k, w.e_begin, w.e_end)
    assert (moe.lib().moe_grouped_gemm_workspace_bytes(moe.ctypes.byref(s), moe.MOE_BF16) > 0) == (d_ff == 2560)
    logits = _one_hot_logits(counts, E, 27)
    res, ref = _layer_case(w, logits)
    x = mi.hidden_states(w)
    wgu, wdn = mi.expert_weights(w)
    fused = moe.layer(g.to_dev(x, w.dtype), g.to_dev(logits, "f32"), g.to_dev(wgu, w.dtype),
                      g.to_dev(wdn, w.dtype), w.k, w.e_begin, w.e_end, fused=True)
    torch.cuda.synchronize()
    n_loc = ref["x_perm"].shape[0]
    assert torch.equal(fused["h"][:n_loc], res["h"][:n_loc])
    assert torch.equal(fused["out"], res["out"])


def test_fused_gemm_workspace_contents_do_not_matter():
    """The blocked-rows workspace also holds the per-XCD tile counts that pace the
    gate/up workgroups; the call clears them itself. With the workspace filled with
    0xFF bytes, and again on the counts the first call left, H and Y equal the
    staged path's (the oracle-checked layer) bit for bit. 2 row tiles x 20 column
    tiles x 8 experts = 320 tiles, more than one round, so the pacing waits."""
    import ctypes
    w = mi.Workload("fused_paced", 2048, 128, 2560, 8, 2, 0, 8, "bf16", 29)
    res, ref = _layer_case(w)
    s = moe.shape(w.T, w.d, w.d_ff, w.E, w.k, w.e_begin, w.e_end)
    ws_bytes = moe.lib().moe_grouped_gemm_workspace_bytes(ctypes.byref(s), moe.MOE_BF16)
    assert ws_bytes == w.n_max * w.d * 2 + 1024
    x = g.to_dev(mi.hidden_states(w), w.dtype)
    wgu, wdn = (g.to_dev(a, w.dtype) for a in mi.expert_weights(w))
    ws = torch.full((ws_bytes,), 0xFF, dtype=torch.uint8, device="cuda")
    n_loc = ref["x_perm"].shape[0]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    for call in range(2):
        h = torch.full((w.n_max, w.d_ff), float("nan"), dtype=torch.bfloat16, device="cuda")
        y = torch.full((w.n_max, w.d), float("nan"), dtype=torch.bfloat16, device="cuda")
        st = moe.lib().moe_grouped_gemm_gather(ctypes.byref(s), moe.MOE_BF16, p(x), p(res["perm"]),
                                               p(res["offsets"]), p(wgu), p(wdn), p(h), p(y), p(ws), stream)
        assert st == moe.MOE_OK
        torch.cuda.synchronize()
        assert torch.equal(h[:n_loc], res["h"][:n_loc]), call
        assert torch.equal(y[:n_loc], res["y"][:n_loc]), call


def test_fused_gemm_rejects_unsupported_shapes():
    w = SMALL[7]  # fp32
    x = torch.zeros((w.T, w.d), dtype=torch.float32, device="cuda")
    logits = torch.zeros((w.T, w.E), dtype=torch.float32, device="cuda")
    wgu = torch.zeros((w.E_loc, w.d, 2 * w.d_ff), dtype=torch.float32, device="cuda")
    wdn = torch.zeros((w.E_loc, w.d_ff, w.d), dtype=torch.float32, device="cuda")
    with pytest.raises(moe.MoeError) as e:
        moe.layer(x, logits, wgu, wdn, w.k, w.e_begin, w.e_end, fused=True)
    assert e.value.status == moe.MOE_EUNSUPPORTED


# ----------------------------------------------------------------------------- decode-shaped, skewed

DECODE_SHAPED = [
    # few rows per local expert on average, but skewed routing puts hundreds of rows
    # on a few experts (several row tiles each, next to many one-row experts)
    mi.Workload("decode_uneven", 200, 256, 192, 64, 8, 0, 64, "bf16", 28, 2.0),
    mi.Workload("decode_uneven_share", 300, 320, 160, 128, 4, 32, 96, "bf16", 29, 2.0),
]


@pytest.mark.parametrize("w", DECODE_SHAPED, ids=[w.name for w in DECODE_SHAPED])
def test_decode_shaped_skewed_layer_matches_oracle(w):
    res, ref = _layer_case(w)
    counts = np.diff(ref["offsets"])[w.e_begin:w.e_end]
    assert counts.max() > 64
    logits = mi.router_logits(w)
    x = mi.hidden_states(w)
    wgu, wdn = mi.expert_weights(w)
    fused = moe.layer(g.to_dev(x, w.dtype), g.to_dev(logits, "f32"), g.to_dev(wgu, w.dtype),
                      g.to_dev(wdn, w.dtype), w.k, w.e_begin, w.e_end, fused=True)
    torch.cuda.synchronize()
    assert torch.equal(fused["out"], res["out"])


@pytest.mark.parametrize("T,k,E,lo,hi", [(600000, 8, 256, 0, 32), (40000, 4, 256, 0, 32), (70000, 4, 128, 16, 32),
                                         (16384, 8, 256, 0, 32), (16385, 4, 512, 480, 512),
                                         (16385, 4, 513, 480, 513),
                                         (4096, 8, 256, 0, 32), (8192, 8, 1024, 1000, 1024), (257, 8, 16, 0, 8)],
                         ids=["four_launches_chunks_of_1024", "four_launches_chunks_of_256",
                              "four_launches_chunks_of_256_ragged", "two_launches_largest",
                              "two_launches_smallest_ragged_most_experts", "four_launches_past_the_two_launch_experts", "one_launch", "one_launch_largest",
                              "one_launch_smallest"])
def test_dispatch_every_path(T, k, E, lo, hi):
    """Every dispatch path gives the oracle's stable permutation: one launch per
    1024 pairs up to 65536 pairs (above the single-workgroup 2048), then two
    launches (chunk counts, then scan and scatter per 512 pairs) up to 131072
    pairs and 512 experts, then four launches with 256-pair chunks, switching
    to 1024-pair chunks once the (expert, chunk) tables would pass 4M entries."""
    rng = np.random.default_rng(T + k + E)
    idx_np = rng.integers(0, E, size=(T, k)).astype(np.int32)
    x = torch.empty((T, 8), dtype=torch.bfloat16, device="cuda")
    disp = moe.dispatch(x, torch.from_numpy(idx_np).cuda(), E, lo, hi, gather=False)
    torch.cuda.synchronize()
    counts, offsets, perm, pair_pos, _ = oracle.dispatch(idx_np, E, lo, hi, np.zeros((T, 0)))
    np.testing.assert_array_equal(disp.counts.cpu().numpy(), counts)
    np.testing.assert_array_equal(disp.offsets.cpu().numpy(), offsets)
    np.testing.assert_array_equal(disp.perm.cpu().numpy(), perm)
    np.testing.assert_array_equal(disp.pair_pos.cpu().numpy(), pair_pos)


@pytest.mark.parametrize("T,k,E,lo,hi", [(40000, 4, 256, 0, 32), (16384, 8, 256, 0, 32), (4096, 8, 256, 0, 32),
                                         (200, 8, 64, 0, 16)],
                         ids=["four_launches", "two_launches", "one_launch", "one_workgroup"])
def test_dispatch_every_path_on_skewed_ids(T, k, E, lo, hi):
    """Each path on ids where a few experts take most pairs (a token's ids are its k
    largest of N(0,1) + a per-expert bias of N(0,3)): long runs of one expert in a
    wave's ballot ranking and in the LDS counts. Bit-exact against the oracle."""
    rng = np.random.default_rng(T + 7 * k + E)
    logits = rng.standard_normal((T, E)) + rng.normal(0.0, 3.0, size=E)
    idx_np = np.argsort(-logits, axis=1, kind="stable")[:, :k].astype(np.int32)
    x = torch.empty((T, 8), dtype=torch.bfloat16, device="cuda")
    disp = moe.dispatch(x, torch.from_numpy(idx_np).cuda(), E, lo, hi, gather=False)
    torch.cuda.synchronize()
    counts, offsets, perm, pair_pos, _ = oracle.dispatch(idx_np, E, lo, hi, np.zeros((T, 0)))
    assert counts.max() >= T // 2  # the skew holds
    np.testing.assert_array_equal(disp.counts.cpu().numpy(), counts)
    np.testing.assert_array_equal(disp.offsets.cpu().numpy(), offsets)
    np.testing.assert_array_equal(disp.perm.cpu().numpy(), perm)
    np.testing.assert_array_equal(disp.pair_pos.cpu().numpy(), pair_pos)


def test_layers_on_two_streams_from_two_threads():
    """The library keeps no state between calls, so two host threads, each running
    a different layer on its own stream at the same time, get the results of the
    same layers run one after the other, bit for bit."""
    import threading

    cases = [mi.Workload("stream_a", 900, 256, 256, 32, 4, 8, 12, "bf16", 51),
             mi.Workload("stream_b", 1200, 320, 192, 8, 2, 0, 8, "bf16", 52)]
    args = []
    for w in cases:
        args.append((g.to_dev(mi.hidden_states(w), "bf16"), g.to_dev(mi.router_logits(w), "f32"),
                     *(g.to_dev(a, "bf16") for a in mi.expert_weights(w)), w.k, w.e_begin, w.e_end))
    alone = []
    for a in args:
        alone.append(moe.layer(*a, fused=True)["out"])
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    got = [[], []]
    errors = []

    def run(i):
        try:
            with torch.cuda.stream(streams[i]):
                for _ in range(3):
                    got[i].append(moe.layer(*args[i], stream=streams[i], fused=True)["out"])
        except Exception as e:  # pragma: no cover - reported below
            errors.append(e)

    threads = [threading.Thread(target=run, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(2):
        for out in got[i]:
            assert torch.equal(out.view(torch.int16), alone[i].view(torch.int16)), i


# ----------------------------------------------------------------------------- debug build

@pytest.mark.parametrize("T,E,k", [(300, 8, 2), (3000, 64, 4), (20000, 64, 4), (40000, 64, 4), (0, 16, 2)],
                         ids=["one_workgroup", "one_launch", "two_launches", "four_launches", "empty"])
def test_debug_build_refuses_out_of_range_ids(T, E, k):
    """libmoe_debug.so counts the ids outside [0, E) on the device and the binding
    refuses them; valid ids give the release build's results bit for bit."""
    rng = np.random.default_rng(T + E)
    d = 64
    x = g.to_dev(mi.f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32)), "bf16")
    good = rng.integers(0, E, size=(T, k)).astype(np.int32)
    release = moe.dispatch(x, torch.from_numpy(good).cuda(), E, 0, E // 2)
    torch.cuda.synchronize()
    moe.set_debug(True)
    try:
        dbg = moe.dispatch(x, torch.from_numpy(good).cuda(), E, 0, E // 2)
        torch.cuda.synchronize()
        for key in ("counts", "offsets", "perm", "pair_pos"):
            assert torch.equal(getattr(dbg, key), getattr(release, key)), key
        n = dbg.offsets[E // 2].item()
        assert torch.equal(dbg.x_perm[:n].view(torch.int16), release.x_perm[:n].view(torch.int16))
        if T == 0:
            return
        bad = good.copy()
        flat = bad.reshape(-1)
        where = rng.choice(flat.size, size=7, replace=False)
        flat[where[:4]] = -1 - where[:4].astype(np.int32)
        flat[where[4:]] = E + where[4:].astype(np.int32)
        with pytest.raises(ValueError, match=r"holds 7 expert id\(s\) outside"):
            moe.dispatch(x, torch.from_numpy(bad).cuda(), E, 0, E // 2)
        with pytest.raises(ValueError, match=r"holds 7 expert id\(s\) outside"):
            moe.dispatch(x, torch.from_numpy(bad).cuda(), E, 0, E // 2, gather=False)
        # the word is rewritten by every call: valid ids pass again on the same buffers
        moe.dispatch(x, torch.from_numpy(good).cuda(), E, 0, E // 2, out=dbg)
    finally:
        moe.set_debug(False)
