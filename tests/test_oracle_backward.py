"""Pins of the backward oracle (CPU only).

The pages print no gradient formula, so the pins are fixed by the mathematics,
independently of the oracle's own formulas:
  * central finite differences of the forward oracle (fp64) for every input of
    the layer, on inputs where no top-k selection changes inside the step;
  * closed forms: silu'(0) = 1/2, silu' -> 1 and -> 0 at the tails; the softmax
    gradient sums to zero per token; k = 1 gives a zero logit gradient;
  * the rank-sum identity: the ranks' partial gradients add up to the gradient
    of the full layer (the outputs they come from add up the same way);
  * planted mistakes in copies of the backward are caught by the differences.
"""
import numpy as np
import pytest

import oracle
from oracle import moe_backward as mb

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _tiny(seed=0, T=6, d=5, d_ff=3, E=4, k=2):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    # logits far apart inside each row so that +-h never reorders the top-k
    logits = np.stack([rng.permutation(E) * 1.0 + 0.1 * rng.standard_normal(E) for _ in range(T)])
    wgu = rng.standard_normal((E, d, 2 * d_ff)) * 0.7
    wdn = rng.standard_normal((E, d_ff, d)) * 0.7
    d_out = rng.standard_normal((T, d))
    return x, logits, wgu, wdn, d_out


def _loss(x, logits, wgu, wdn, d_out, k, lo, hi):
    out = oracle.moe_layer(x, logits, k, lo, hi, list(wgu[lo:hi]), list(wdn[lo:hi]))["out"]
    return float(np.sum(out * d_out))


def _fd(f, a, h=1e-6):
    g = np.zeros_like(a)
    it = np.nditer(a, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = a[i]
        a[i] = old + h
        fp = f()
        a[i] = old - h
        fm = f()
        a[i] = old
        g[i] = (fp - fm) / (2 * h)
    return g


@pytest.mark.parametrize("lo,hi", [(0, 4), (1, 3), (2, 3)])
def test_layer_gradient_matches_finite_differences(lo, hi):
    x, logits, wgu, wdn, d_out = _tiny(seed=lo * 10 + hi)
    k = 2
    res = oracle.moe_layer_backward(x, logits, k, lo, hi, list(wgu[lo:hi]), list(wdn[lo:hi]), d_out)
    f = lambda: _loss(x, logits, wgu, wdn, d_out, k, lo, hi)  # noqa: E731
    np.testing.assert_allclose(res["d_x"], _fd(f, x), rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(res["d_logits"], _fd(f, logits), rtol=1e-6, atol=1e-7)
    fd_wgu = _fd(f, wgu)
    fd_wdn = _fd(f, wdn)
    np.testing.assert_allclose(res["d_w_gate_up"], fd_wgu[lo:hi], rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(res["d_w_down"], fd_wdn[lo:hi], rtol=1e-6, atol=1e-7)
    # weights of non-local experts do not touch this rank's output
    assert np.all(np.abs(np.delete(fd_wgu, range(lo, hi), axis=0)) < 1e-8)


def test_combine_gradient_matches_finite_differences():
    rng = np.random.default_rng(3)
    T, k, d, n = 5, 3, 4, 9
    y = rng.standard_normal((n, d))
    w = rng.random((T, k))
    pair_pos = np.array([0, 1, -1, 2, -1, 3, 4, 5, 6, -1, -1, -1, 7, 8, -1])
    d_out = rng.standard_normal((T, d))
    d_y, d_w = oracle.combine_backward(d_out, y, pair_pos, w, T, k)
    f = lambda: float(np.sum(oracle.combine(y, pair_pos, w, T, k, d) * d_out))  # noqa: E731
    np.testing.assert_allclose(d_y, _fd(f, y), rtol=1e-7, atol=1e-8)
    np.testing.assert_allclose(d_w, _fd(f, w), rtol=1e-7, atol=1e-8)
    assert np.all(d_w[pair_pos.reshape(T, k) < 0] == 0)


def test_silu_grad_closed_forms():
    assert mb.silu_grad(np.array([0.0]))[0] == 0.5
    z = np.array([-60.0, -30.0, 30.0, 60.0])
    g = mb.silu_grad(z)
    assert np.all(np.isfinite(g))
    assert abs(g[0]) < 1e-20 and abs(g[3] - 1.0) < 1e-12
    zz = np.linspace(-8, 8, 33)
    expected = mb.silu_grad(zz)
    f = lambda: float(np.sum(oracle.silu(zz)))  # noqa: E731
    np.testing.assert_allclose(expected, _fd(f, zz), rtol=1e-6, atol=1e-7)


def test_softmax_gradient_sums_to_zero_and_k1_is_zero():
    rng = np.random.default_rng(4)
    logits = rng.standard_normal((7, 6))
    d_w = rng.standard_normal((7, 3))
    dl = oracle.route_topk_backward(logits, 3, d_w)
    np.testing.assert_allclose(dl.sum(axis=1), 0.0, atol=1e-12)
    idx, _ = oracle.route_topk(logits, 3)
    mask = np.zeros_like(dl, dtype=bool)
    np.put_along_axis(mask, idx, True, axis=1)
    assert np.all(dl[~mask] == 0)
    assert np.all(oracle.route_topk_backward(logits, 1, rng.standard_normal((7, 1))) == 0)


def test_rank_sum_of_partial_gradients():
    x, logits, wgu, wdn, d_out = _tiny(seed=9, E=4)
    k = 2
    full = oracle.moe_layer_backward(x, logits, k, 0, 4, list(wgu), list(wdn), d_out)
    parts = [oracle.moe_layer_backward(x, logits, k, lo, lo + 2, list(wgu[lo:lo + 2]), list(wdn[lo:lo + 2]), d_out)
             for lo in (0, 2)]
    np.testing.assert_allclose(sum(p["d_x"] for p in parts), full["d_x"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(sum(p["d_logits"] for p in parts), full["d_logits"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(np.concatenate([p["d_w_gate_up"] for p in parts]), full["d_w_gate_up"], rtol=1e-12)


def test_empty_expert_and_no_local_token_give_zero_gradients():
    x, logits, wgu, wdn, d_out = _tiny(seed=5, E=4)
    logits[:, 3] = -100.0  # expert 3 never chosen
    res = oracle.moe_layer_backward(x, logits, 2, 3, 4, [wgu[3]], [wdn[3]], d_out)
    assert np.all(res["d_x"] == 0) and np.all(res["d_logits"] == 0)
    assert np.all(res["d_w_gate_up"] == 0) and np.all(res["d_w_down"] == 0)


@pytest.mark.parametrize("mistake", ["no_silu_prime", "up_without_silu", "dy_unweighted", "wdn_not_transposed"])
def test_planted_mistakes_fail_the_differences(mistake, monkeypatch):
    x, logits, wgu, wdn, d_out = _tiny(seed=7, d=4, d_ff=4)
    k, lo, hi = 2, 0, 4
    if mistake == "no_silu_prime":
        monkeypatch.setattr(mb, "silu_grad", lambda z: np.ones_like(np.asarray(z, dtype=np.float64)))
    elif mistake == "up_without_silu":
        monkeypatch.setattr(mb, "swiglu_backward", lambda g, u, dh: (dh * u * mb.silu_grad(g), dh * g))
    elif mistake == "dy_unweighted":
        orig = mb.combine_backward

        def bad(d_out_, y, pair_pos, w, T, k_):
            d_y, d_w = orig(d_out_, y, pair_pos, np.ones_like(w), T, k_)
            return d_y, orig(d_out_, y, pair_pos, w, T, k_)[1]
        monkeypatch.setattr(mb, "combine_backward", bad)
    elif mistake == "wdn_not_transposed":
        orig = mb.expert_ffn_backward

        def bad(rows, w_gate_up, w_down, d_y):
            a, b, c = orig(rows, w_gate_up, w_down, d_y)
            return a, b, c.T.reshape(c.shape)
        monkeypatch.setattr(mb, "expert_ffn_backward", bad)
    res = mb.moe_layer_backward(x, logits, k, lo, hi, list(wgu), list(wdn), d_out)
    f = lambda: _loss(x, logits, wgu, wdn, d_out, k, lo, hi)  # noqa: E731
    checks = [(res["d_x"], _fd(f, x)), (res["d_w_gate_up"], _fd(f, wgu)), (res["d_w_down"], _fd(f, wdn))]
    assert any(not np.allclose(a, b, rtol=1e-5, atol=1e-6) for a, b in checks)
