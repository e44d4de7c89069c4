"""Pins of the CPU oracle against what the pages and mathematics fix.

Each check_* function takes the oracle functions it exercises as arguments, so
the same checks run on the oracle (must pass) and on copies of it with a
planted mistake (must fail): a dropped term, a wrong sign or index, a swapped
operand or an unstable sort is caught by at least one pin.
"""
import json
import os

import numpy as np
import pytest
from scipy.special import expit, softmax

import oracle
from oracle import moe as om

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- fixtures

def _worked():
    with open(os.path.join(GOLDEN, "worked_tiny_layer.json")) as f:
        g = json.load(f)
    # every logit is exactly representable in fp32, so the closed forms hold exactly
    logits = np.array([[float(s) for s in row] for row in g["logits"]], dtype=np.float32)
    return g, logits


def _closed_w():
    a, b = expit(0.75), expit(1.5)
    return np.array([[a, 1.0 - a], [b, 1.0 - b], [0.5, 0.5]])


def _worked_weights(d=2):
    eye = np.eye(d)
    wgu = np.concatenate([eye, 2.0 * eye], axis=1)  # [I | 2I]: gate = x, up = 2x
    return np.stack([wgu, wgu]), np.stack([eye, eye])


# ----------------------------------------------------------------------------- checks

def check_worked_example(route_topk, dispatch, moe_layer):
    g, logits = _worked()
    idx, w = route_topk(logits, g["k"])
    np.testing.assert_array_equal(idx, g["idx"])
    np.testing.assert_allclose(w, _closed_w(), rtol=0, atol=1e-15)
    x = np.array(g["x"])
    counts, offsets, perm, pair_pos, x_perm = dispatch(idx, g["E"], g["e_lo"], g["e_hi"], x)
    np.testing.assert_array_equal(counts, g["counts"])
    np.testing.assert_array_equal(offsets, g["offsets"])
    np.testing.assert_array_equal(perm, g["perm"])
    np.testing.assert_array_equal(pair_pos, g["pair_pos"])
    np.testing.assert_array_equal(x_perm, x[g["x_perm_tokens"]])
    wgu, wdn = _worked_weights()
    res = moe_layer(x, logits, g["k"], g["e_lo"], g["e_hi"], wgu, wdn)
    ffn = lambda v: 2.0 * v * v * expit(v)  # closed form of silu(v) * 2v
    expect = np.zeros_like(x)
    expect[1] = expit(1.5) * ffn(x[1])
    expect[2] = 0.5 * ffn(x[2])
    np.testing.assert_allclose(res["out"], expect, rtol=1e-14, atol=1e-15)


def check_topk_properties(route_topk, T=200, E=16, k=5, seed=0):
    rng = np.random.default_rng(seed)
    # coarse values so many ties occur, plus signed zeros
    logits = (rng.integers(-3, 4, size=(T, E)) * 0.5).astype(np.float32)
    logits[rng.random((T, E)) < 0.1] = -0.0
    idx, w = route_topk(logits, k)
    assert idx.shape == (T, k) and w.shape == (T, k)
    for t in range(T):
        sel = list(idx[t])
        assert len(set(sel)) == k and all(0 <= e < E for e in sel)
        rest = [e for e in range(E) if e not in sel]
        v = logits[t].astype(np.float64)
        for a, b in zip(sel, sel[1:]):  # descending value, ties ascending id
            assert v[a] > v[b] or (v[a] == v[b] and a < b)
        for s in sel:
            for u in rest:  # every pick beats every non-pick; ties go to the lower id
                assert v[s] > v[u] or (v[s] == v[u] and s < u)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    assert np.all(np.diff(w, axis=1) <= 1e-15)


def check_topk_matches_renormalised_softmax(route_topk, T=64, E=32, k=6, seed=1):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    idx, w = route_topk(logits, k)
    p = softmax(logits.astype(np.float64), axis=1)
    sel = np.take_along_axis(p, idx, axis=1)
    np.testing.assert_allclose(w, sel / sel.sum(axis=1, keepdims=True), rtol=1e-13, atol=0)
    # sorted full order agrees with a plain python sort on the key (-value, id)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:k]
        assert list(idx[t]) == order


def check_topk_special_cases(route_topk):
    T, E = 5, 8
    for k in (1, 3, 8):
        idx, w = route_topk(np.zeros((T, E), np.float32), k)
        np.testing.assert_array_equal(idx, np.tile(np.arange(k), (T, 1)))
        np.testing.assert_allclose(w, 1.0 / k, rtol=0, atol=1e-15)
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    idx, w = route_topk(logits, 1)
    assert np.all(w == 1.0)
    np.testing.assert_array_equal(idx[:, 0], np.argmax(logits, axis=1))
    idx, w = route_topk(logits, E)  # k = E: the full softmax, in descending order
    full = softmax(logits.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, -np.sort(-full, axis=1), rtol=1e-13)


def check_dispatch_properties(route_topk, dispatch, T=97, E=12, k=3, e_lo=4, e_hi=8, d=5, seed=2):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[:, 5] += 1.0  # make one expert heavy
    logits[:, 9] -= 9.0  # and one (non-local) expert nearly always empty
    idx, _ = route_topk(logits, k)
    x = rng.standard_normal((T, d))
    counts, offsets, perm, pair_pos, x_perm = dispatch(idx, E, e_lo, e_hi, x)
    flat = idx.reshape(-1)
    # brute-force count and sort, pair by pair
    brute_counts = [sum(1 for p in range(T * k) if flat[p] == e) for e in range(E)]
    np.testing.assert_array_equal(counts, brute_counts)
    assert counts.sum() == T * k
    assert offsets[0] == 0 and offsets[-1] == T * k and np.all(np.diff(offsets) == counts)
    brute_perm = sorted(range(T * k), key=lambda p: (flat[p], p))
    np.testing.assert_array_equal(perm, brute_perm)
    assert sorted(perm.tolist()) == list(range(T * k))
    # local pairs only, numbered 0..N_loc-1 in segment order; the rest -1
    n_loc = sum(brute_counts[e_lo:e_hi])
    assert x_perm.shape == (n_loc, d)
    local = [p for p in brute_perm if e_lo <= flat[p] < e_hi]
    for r, p in enumerate(local):
        assert pair_pos[p] == r
        np.testing.assert_array_equal(x_perm[r], x[p // k])
    assert all(pair_pos[p] == -1 for p in range(T * k) if not e_lo <= flat[p] < e_hi)


def check_ffn_closed_form(expert_ffn):
    x = np.array([[-3.0, -0.5, 0.0, 0.7, 2.0, 9.0]])
    d = x.shape[1]
    eye = np.eye(d)
    y = expert_ffn(x, np.concatenate([eye, 2.0 * eye], axis=1), eye)
    np.testing.assert_allclose(y, 2.0 * x * x * expit(x), rtol=1e-14, atol=1e-300)
    # the down projection is a plain matrix product: a permutation matrix permutes
    pm = eye[::-1]
    y2 = expert_ffn(x, np.concatenate([eye, 2.0 * eye], axis=1), pm)
    np.testing.assert_allclose(y2, (2.0 * x * x * expit(x))[:, ::-1], rtol=1e-14, atol=1e-300)
    # an up projection of all-ones rows sums x: H = silu(x_i) * sum(x)
    d_ff = d
    wgu = np.concatenate([eye, np.ones((d, d_ff))], axis=1)
    y3 = expert_ffn(x, wgu, eye)
    np.testing.assert_allclose(y3, x * expit(x) * x.sum(), rtol=1e-14, atol=1e-300)


def check_silu(silu):
    z = np.linspace(-40, 40, 161)
    np.testing.assert_allclose(silu(z), z * expit(z), rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(silu(z) - silu(-z), z, rtol=1e-14, atol=1e-14)
    assert silu(np.array([0.0]))[0] == 0.0
    assert np.all(np.isfinite(silu(np.array([-1e4, 1e4]))))


def _small_layer(seed, T=40, E=8, k=3, d=6, d_ff=10, e_lo=0, e_hi=8):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    wgu = rng.standard_normal((e_hi - e_lo, d, 2 * d_ff)) / np.sqrt(d)
    wdn = rng.standard_normal((e_hi - e_lo, d_ff, d)) / np.sqrt(d_ff)
    return x, logits, wgu, wdn


def check_brute_force_dense(route_topk, moe_layer, brute_force_dense):
    for (e_lo, e_hi) in ((0, 8), (2, 6), (7, 8)):
        x, logits, wgu, wdn = _small_layer(4, e_lo=e_lo, e_hi=e_hi)
        idx, w = route_topk(logits, 3)
        res = moe_layer(x, logits, 3, e_lo, e_hi, wgu, wdn)
        ref = brute_force_dense(x, idx, w, e_lo, e_hi, wgu, wdn)
        np.testing.assert_allclose(res["out"], ref, rtol=0, atol=1e-12)


def check_rank_sum(expert_range, moe_layer):
    E = 8
    x, logits, wgu_all, wdn_all = _small_layer(5, E=E)
    full = moe_layer(x, logits, 3, 0, E, wgu_all, wdn_all)["out"]
    for ep in (2, 4, 8):
        acc = np.zeros_like(full)
        for r in range(ep):
            lo, hi = expert_range(E, ep, r)
            acc += moe_layer(x, logits, 3, lo, hi, wgu_all[lo:hi], wdn_all[lo:hi])["out"]
        np.testing.assert_allclose(acc, full, rtol=0, atol=1e-12)


def check_identity_round_trip(route_topk, dispatch, combine):
    rng = np.random.default_rng(6)
    T, E, k, d = 33, 8, 3, 7
    x = rng.standard_normal((T, d))
    idx, w = route_topk(rng.standard_normal((T, E)).astype(np.float32), k)
    counts, offsets, perm, pair_pos, x_perm = dispatch(idx, E, 0, E, x)
    out = combine(x_perm, pair_pos, w, T, k, d)  # identity expert: Y = rows received
    np.testing.assert_allclose(out, x, rtol=0, atol=1e-14)
    # a rank that owns experts [2, 6) only: out[t] = (weight mass of its local picks) * x[t]
    counts, offsets, perm, pair_pos, x_perm = dispatch(idx, E, 2, 6, x)
    out = combine(x_perm, pair_pos, w, T, k, d)
    mass = np.where((idx >= 2) & (idx < 6), w, 0.0).sum(axis=1)
    np.testing.assert_allclose(out, mass[:, None] * x, rtol=0, atol=1e-14)


def check_ownership(expert_range):
    with open(os.path.join(GOLDEN, "ep_ownership_8ranks.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    for row in rows:
        ep = int(row[0])
        for rank, spec in enumerate(row[1:]):
            lo, hi_incl = (int(v) for v in spec.split("-"))
            assert expert_range(8, ep, rank) == (lo, hi_incl + 1)


# ----------------------------------------------------------------------------- the oracle passes

def test_worked_example():
    check_worked_example(oracle.route_topk, oracle.dispatch, oracle.moe_layer)


def check_layer_hidden(moe_layer):
    """H and Y of the worked example: gate_up = [I | 2I] gives H = silu(x) * 2x =
    2 x^2 sigmoid(x) on the gathered rows (tokens 1 and 2), and a down
    projection that swaps the two columns gives Y = H with its columns swapped."""
    g, logits = _worked()
    x = np.array(g["x"])
    wgu, _ = _worked_weights()
    swap = np.array([[0.0, 1.0], [1.0, 0.0]])
    res = moe_layer(x, logits, g["k"], g["e_lo"], g["e_hi"], wgu, np.stack([swap, swap]))
    rows = x[g["x_perm_tokens"]]
    np.testing.assert_allclose(res["h"], 2.0 * rows * rows * expit(rows), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(res["y"], res["h"][:, ::-1], rtol=1e-14, atol=1e-15)


def test_layer_hidden_closed_form():
    check_layer_hidden(oracle.moe_layer)


def test_planted_hidden_mistakes_are_caught():
    def layer_gate_only(x, logits, k, e_lo, e_hi, wgu, wdn):
        res = om.moe_layer(x, logits, k, e_lo, e_hi, wgu, wdn)
        res["h"] = om.silu(res["x_perm"])  # silu(gate) without the up projection
        return res

    def layer_unprojected(x, logits, k, e_lo, e_hi, wgu, wdn):
        res = om.moe_layer(x, logits, k, e_lo, e_hi, wgu, wdn)
        res["y"] = res["h"]  # down projection dropped
        return res

    _fails(check_layer_hidden, layer_gate_only)
    _fails(check_layer_hidden, layer_unprojected)


def test_topk_properties():
    check_topk_properties(oracle.route_topk)


def test_topk_renormalised_softmax():
    check_topk_matches_renormalised_softmax(oracle.route_topk)


def test_topk_special_cases():
    check_topk_special_cases(oracle.route_topk)


def test_dispatch_properties():
    check_dispatch_properties(oracle.route_topk, oracle.dispatch)


def test_ffn_closed_form():
    check_ffn_closed_form(oracle.expert_ffn)


def test_silu():
    check_silu(oracle.silu)


def test_brute_force_dense():
    check_brute_force_dense(oracle.route_topk, oracle.moe_layer, oracle.brute_force_dense)


def test_rank_sum():
    check_rank_sum(oracle.expert_range, oracle.moe_layer)


def test_identity_round_trip():
    check_identity_round_trip(oracle.route_topk, oracle.dispatch, oracle.combine)


def test_ownership_diagram():
    check_ownership(oracle.expert_range)
    with pytest.raises(ValueError):
        oracle.expert_range(8, 3, 0)


def test_token_outputs_match_layer():
    x, logits, wgu, wdn = _small_layer(7, e_lo=2, e_hi=6)
    res = oracle.moe_layer(x, logits, 3, 2, 6, wgu, wdn)
    pick = [0, 5, 17, 39]
    got = oracle.token_outputs(pick, x[pick], res["idx"][pick], res["w"][pick], 2, 6, wgu, wdn)
    np.testing.assert_allclose(got, res["out"][pick], rtol=0, atol=1e-13)


def test_empty_and_single_token():
    rng = np.random.default_rng(8)
    E, k, d, d_ff = 8, 2, 4, 6
    wgu = rng.standard_normal((E, d, 2 * d_ff))
    wdn = rng.standard_normal((E, d_ff, d))
    res = oracle.moe_layer(np.zeros((0, d)), np.zeros((0, E), np.float32), k, 0, E, wgu, wdn)
    assert res["out"].shape == (0, d) and res["counts"].sum() == 0
    x = rng.standard_normal((1, d))
    logits = rng.standard_normal((1, E)).astype(np.float32)
    res = oracle.moe_layer(x, logits, k, 0, E, wgu, wdn)
    ref = oracle.brute_force_dense(x, res["idx"], res["w"], 0, E, wgu, wdn)
    np.testing.assert_allclose(res["out"], ref, atol=1e-12)


# ----------------------------------------------------------------------------- planted mistakes fail

def _route_high_id_ties(logits, k):  # tie-break to the higher id
    T, E = logits.shape
    v = logits.astype(np.float64) + 0.0
    order = np.lexsort((-np.broadcast_to(np.arange(E), (T, E)), -v), axis=-1)
    idx = order[:, :k]
    sel = np.take_along_axis(v, idx, axis=1)
    ex = np.exp(sel - sel[:, :1])
    return idx, ex / ex.sum(axis=1, keepdims=True)


def _route_signed_zero(logits, k):  # -0.0 ranked below +0.0
    T, E = logits.shape
    bits = np.signbit(logits).astype(np.float64)
    v = logits.astype(np.float64)
    order = np.lexsort((np.broadcast_to(np.arange(E), (T, E)), bits * (v == 0), -v), axis=-1)
    idx = order[:, :k]
    sel = np.take_along_axis(v, idx, axis=1)
    ex = np.exp(sel - sel[:, :1])
    return idx, ex / ex.sum(axis=1, keepdims=True)


def _route_no_renorm(logits, k):  # full-softmax weights, not renormalised over the k picks
    idx, _ = om.route_topk(logits, k)
    p = softmax(logits.astype(np.float64), axis=1)
    return idx, np.take_along_axis(p, idx, axis=1)


def _dispatch_unstable(idx, E, e_lo, e_hi, x):
    counts, offsets, perm, pair_pos, x_perm = om.dispatch(idx, E, e_lo, e_hi, x)
    perm = perm.copy()
    for e in range(E):  # reverse order inside each segment
        perm[offsets[e]:offsets[e + 1]] = perm[offsets[e]:offsets[e + 1]][::-1]
    k = idx.shape[1]
    seg0, seg1 = offsets[e_lo], offsets[e_hi]
    pair_pos = np.full(idx.size, -1)
    pair_pos[perm[seg0:seg1]] = np.arange(seg1 - seg0)
    return counts, offsets, perm, pair_pos, np.asarray(x)[perm[seg0:seg1] // k]


def _dispatch_global_pos(idx, E, e_lo, e_hi, x):  # forgets to subtract the segment base
    counts, offsets, perm, pair_pos, x_perm = om.dispatch(idx, E, e_lo, e_hi, x)
    pp = pair_pos.copy()
    pp[pp >= 0] += offsets[e_lo]
    return counts, offsets, perm, pp, x_perm


def _ffn_swapped(rows, wgu, wdn):  # gate and up halves swapped
    d_ff = wdn.shape[0]
    g = np.asarray(rows, float) @ wgu
    return (om.silu(g[:, d_ff:]) * g[:, :d_ff]) @ wdn


def _ffn_no_gate(rows, wgu, wdn):  # plain SiLU MLP, up half dropped
    d_ff = wdn.shape[0]
    g = np.asarray(rows, float) @ wgu
    return om.silu(g[:, :d_ff]) @ wdn


def _silu_sign(z):
    z = np.asarray(z, float)
    return z * expit(-z)


def _expert_range_off_by_one(E, ep, rank):
    per = E // ep
    return rank * per, (rank + 1) * per  # forgets that blocks repeat every ep ranks


def _combine_unweighted(y, pair_pos, w, T, k, d):
    return om.combine(y, pair_pos, np.ones_like(w), T, k, d)


def _layer_with(**swap):
    """The oracle's layer composition with one step replaced."""
    route = swap.get("route", om.route_topk)
    disp = swap.get("dispatch", om.dispatch)
    ffn = swap.get("ffn", om.expert_ffn)
    comb = swap.get("combine", om.combine)

    def layer(x, logits, k, e_lo, e_hi, wgu, wdn):
        x = np.asarray(x, float)
        T, d = x.shape
        idx, w = route(logits, k)
        counts, offsets, perm, pair_pos, x_perm = disp(idx, logits.shape[1], e_lo, e_hi, x)
        y = np.zeros((x_perm.shape[0], d))
        base = offsets[e_lo]
        for e in range(e_lo, e_hi):
            r0, r1 = offsets[e] - base, offsets[e + 1] - base
            if r1 > r0:
                y[r0:r1] = ffn(x_perm[r0:r1], wgu[e - e_lo], wdn[e - e_lo])
        return dict(idx=idx, w=w, out=comb(y, pair_pos, w, T, k, d))
    return layer


def _fails(fn, *args):
    # a planted mistake is caught when a pin fails or the mistake breaks indexing outright
    with pytest.raises((AssertionError, IndexError)):
        fn(*args)


def test_planted_topk_mistakes_are_caught():
    _fails(check_worked_example, _route_high_id_ties, om.dispatch, _layer_with(route=_route_high_id_ties))
    _fails(check_topk_properties, _route_high_id_ties)
    _fails(check_worked_example, _route_signed_zero, om.dispatch, om.moe_layer)
    _fails(check_topk_properties, _route_no_renorm)
    _fails(check_topk_matches_renormalised_softmax, _route_no_renorm)


def test_planted_dispatch_mistakes_are_caught():
    _fails(check_dispatch_properties, om.route_topk, _dispatch_unstable)
    _fails(check_worked_example, om.route_topk, _dispatch_unstable, om.moe_layer)
    _fails(check_dispatch_properties, om.route_topk, _dispatch_global_pos)
    _fails(check_identity_round_trip, om.route_topk, _dispatch_global_pos, om.combine)


def test_planted_ffn_mistakes_are_caught():
    _fails(check_ffn_closed_form, _ffn_swapped)
    _fails(check_ffn_closed_form, _ffn_no_gate)
    _fails(check_silu, _silu_sign)
    _fails(check_worked_example, om.route_topk, om.dispatch, _layer_with(ffn=_ffn_swapped))


def test_planted_layout_mistakes_are_caught():
    _fails(check_ownership, _expert_range_off_by_one)
    # an unweighted combine breaks the worked example's closed form
    _fails(check_worked_example, om.route_topk, om.dispatch, _layer_with(combine=_combine_unweighted))


def test_bf16_rounding_helper_matches_torch():
    torch = pytest.importorskip("torch")
    from moe_inputs import f32_to_bf16_bits, bf16_bits_to_f32
    rng = np.random.default_rng(9)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, 1e-40, 1.00390625, 1.01171875], np.float32)])
    ours = f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    back = bf16_bits_to_f32(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(ours.view(np.int16)).view(torch.bfloat16).float().numpy())
