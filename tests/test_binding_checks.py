"""The Python binding refuses tensors of the wrong dtype or shape before any of
them reaches the library: a wrong dtype raises TypeError, a wrong shape (inputs
and caller-provided outputs alike) ValueError. These checks run ahead of the
device check, so CPU tensors exercise them without a GPU."""
import os

import pytest

import token_dispatch_grouped_amd as moe

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.skipif(not os.path.exists(moe.lib_path), reason="libmoe.so not built")

T, D, DFF, E, K, LO, HI = 16, 64, 32, 8, 2, 0, 8
NMAX = T * min(K, HI - LO)
bf16, f32, i32, i64 = torch.bfloat16, torch.float32, torch.int32, torch.int64


def t(shape, dtype):
    return torch.zeros(shape, dtype=dtype)


def test_route_topk_checks():
    with pytest.raises(TypeError):
        moe.route_topk(t((T, E), bf16), K)
    with pytest.raises(ValueError):
        moe.route_topk(t((T * E,), f32), K)
    with pytest.raises(ValueError):
        moe.route_topk(t((T, E), f32), E + 1)
    with pytest.raises(TypeError):  # what torch.topk returns
        moe.route_topk(t((T, E), f32), K, topk_idx=t((T, K), i64))
    with pytest.raises(TypeError):
        moe.route_topk(t((T, E), f32), K, topk_w=t((T, K), bf16))
    with pytest.raises(ValueError):
        moe.route_topk(t((T, E), f32), K, topk_idx=t((T - 1, K), i32))


def test_dispatch_checks():
    x = t((T, D), bf16)
    with pytest.raises(TypeError):
        moe.dispatch(x, t((T, K), i64), E, LO, HI)
    with pytest.raises(ValueError):
        moe.dispatch(x, t((T + 1, K), i32), E, LO, HI)
    with pytest.raises(ValueError):
        moe.dispatch(x, t((T * K,), i32), E, LO, HI)
    with pytest.raises(TypeError):
        moe.dispatch(t((T, D), torch.float16), t((T, K), i32), E, LO, HI)
    with pytest.raises(ValueError):
        moe.dispatch(x, t((T, K), i32), E, 4, 2)
    good = moe.Dispatch(counts=t((E,), i32), offsets=t((E + 1,), i32), perm=t((T * K,), i32),
                        pair_pos=t((T * K,), i32), x_perm=t((NMAX, D), bf16),
                        workspace=t((moe.dispatch_workspace_bytes(T, K, E),), torch.uint8))
    bad = [dict(counts=t((E,), i64)), dict(offsets=t((E,), i32)), dict(perm=t((T * K - 1,), i32)),
           dict(pair_pos=t((T * K,), f32)), dict(x_perm=t((NMAX - 1, D), bf16)), dict(x_perm=t((NMAX, D), f32)),
           dict(workspace=t((1,), torch.uint8))]
    for change in bad:
        fields = dict(good.__dict__)
        fields.update(change)
        exc = TypeError if any(v.dtype != getattr(good, k).dtype for k, v in change.items()) else ValueError
        with pytest.raises(exc):
            moe.dispatch(x, t((T, K), i32), E, LO, HI, out=moe.Dispatch(**fields))


def _weights(dtype=bf16, e_loc=HI - LO, d=D, d_ff=DFF):
    return t((e_loc, d, 2 * d_ff), dtype), t((e_loc, d_ff, d), dtype)


def test_grouped_gemm_checks():
    wgu, wdn = _weights()
    offs = t((E + 1,), i32)
    with pytest.raises(TypeError):  # fp32 activations with bf16 weights
        moe.grouped_gemm(t((NMAX, D), f32), offs, wgu, wdn, T, K, E, LO, HI)
    with pytest.raises(ValueError):
        moe.grouped_gemm(t((NMAX - 1, D), bf16), offs, wgu, wdn, T, K, E, LO, HI)
    with pytest.raises(ValueError):
        moe.grouped_gemm(t((NMAX, D), bf16), offs, *_weights(e_loc=HI - LO - 1), T, K, E, LO, HI)
    with pytest.raises(ValueError):
        moe.grouped_gemm(t((NMAX, D), bf16), offs, t((HI - LO, D, DFF), bf16), wdn, T, K, E, LO, HI)
    with pytest.raises(TypeError):
        moe.grouped_gemm(t((NMAX, D), bf16), t((E + 1,), i64), wgu, wdn, T, K, E, LO, HI)
    with pytest.raises(ValueError):
        moe.grouped_gemm(t((NMAX, D), bf16), offs, wgu, wdn, T, K, E, LO, HI, h=t((NMAX - 1, DFF), bf16))
    with pytest.raises(ValueError):
        moe.grouped_gemm(t((NMAX, D), bf16), offs, wgu, wdn, T, K, E, LO, HI, y=t((NMAX, D + 8), bf16))


def test_grouped_gemm_gather_checks():
    wgu, wdn = _weights()
    x, offs, perm = t((T, D), bf16), t((E + 1,), i32), t((T * K,), i32)
    with pytest.raises(ValueError):
        moe.grouped_gemm_gather(x, t((T * K - 1,), i32), offs, wgu, wdn, K, E, LO, HI)
    with pytest.raises(TypeError):
        moe.grouped_gemm_gather(x, perm, offs, *_weights(dtype=f32), K, E, LO, HI)
    with pytest.raises(ValueError):
        moe.grouped_gemm_gather(x, perm, offs, wgu, wdn, K, E, LO, HI, gu=t((NMAX, DFF), bf16))


def test_combine_checks():
    y, pp, w = t((NMAX, D), bf16), t((T * K,), i32), t((T, K), f32)
    with pytest.raises(TypeError):  # read as fp32, past the end of a bf16 buffer
        moe.combine(y, pp, t((T, K), bf16), T, K, E, LO, HI)
    with pytest.raises(ValueError):
        moe.combine(t((NMAX - 1, D), bf16), pp, w, T, K, E, LO, HI)
    with pytest.raises(ValueError):
        moe.combine(y, pp, w, T, K, E, LO, HI, out=t((T - 1, D), bf16))
    with pytest.raises(TypeError):
        moe.combine(y, pp, w, T, K, E, LO, HI, out=t((T, D), f32))
    with pytest.raises(TypeError):
        moe.combine(y, t((T * K,), i64), w, T, K, E, LO, HI)


def test_backward_checks():
    wgu, wdn = _weights()
    x, perm, offs = t((T, D), bf16), t((T * K,), i32), t((E + 1,), i32)
    h, d_y = t((NMAX, DFF), bf16), t((NMAX, D), bf16)
    with pytest.raises(ValueError):
        moe.combine_backward(t((T, D), bf16), t((NMAX - 2, D), bf16), perm, t((T, K), f32), T, K, E, LO, HI)
    with pytest.raises(TypeError):
        moe.combine_backward(t((T, D), bf16), t((NMAX, D), f32), perm, t((T, K), f32), T, K, E, LO, HI)
    with pytest.raises(ValueError):
        moe.grouped_gemm_backward(x, perm, offs, wgu, wdn, t((NMAX - 1, DFF), bf16), d_y, K, E, LO, HI)
    with pytest.raises(ValueError):
        moe.grouped_gemm_backward(x, perm, offs, wgu, wdn, h, d_y, K, E, LO, HI, d_w_down=t((1, DFF, D), bf16))
    with pytest.raises(ValueError):
        moe.grouped_gemm_backward(x, perm, offs, wgu, wdn, h, d_y, K, E, LO, HI,
                                  workspace=t((1,), torch.uint8))
    with pytest.raises(ValueError):
        moe.dispatch_backward(t((NMAX - 1, D), bf16), perm, T, K, E, LO, HI)
    with pytest.raises(TypeError):
        moe.route_topk_backward(t((T, K), i64), t((T, K), f32), t((T, K), f32), E)
    with pytest.raises(ValueError):
        moe.route_topk_backward(t((T, K), i32), t((T, K), f32), t((T, K + 1), f32), E)
