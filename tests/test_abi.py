"""The C ABI without a GPU: the library loads, exports every declared symbol, and
rejects invalid arguments on the host before any HIP call."""
import ctypes
import os

import pytest

import token_dispatch_grouped_amd as moe

pytestmark = pytest.mark.skipif(not os.path.exists(moe.lib_path), reason="libmoe.so not built")

NULL = ctypes.c_void_p(0)
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def test_exports_every_declared_symbol():
    declared = moe.declared_symbols()
    assert set(declared) >= {"moe_route_topk", "moe_dispatch", "moe_grouped_gemm", "moe_combine",
                             "moe_expert_range", "moe_status_string"}
    lib = moe.lib()
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings():
    for code in (0, 1, 2, 3):
        assert moe.status_string(code).startswith("MOE_")


def test_expert_range_matches_ownership_diagram():
    golden = os.path.join(os.path.dirname(__file__), "golden", "ep_ownership_8ranks.txt")
    with open(golden) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    for row in rows:
        ep = int(row[0])
        for rank, spec in enumerate(row[1:]):
            lo, hi = (int(v) for v in spec.split("-"))
            assert moe.expert_range(8, ep, rank) == (lo, hi + 1)
    with pytest.raises(moe.MoeError):
        moe.expert_range(8, 3, 0)
    with pytest.raises(moe.MoeError):
        moe.expert_range(8, 2, -1)


def _shape(**kw):
    base = dict(T=16, d=64, d_ff=64, E=8, k=2, e_begin=0, e_end=8)
    base.update(kw)
    return moe.shape(**base)


def _route(s, logits=FAKE, idx=FAKE, w=FAKE):
    return moe.lib().moe_route_topk(ctypes.byref(s), logits, idx, w, NULL)


def _dispatch(s, dt=moe.MOE_BF16, ptrs=None):
    p = ptrs or [FAKE] * 7
    return moe.lib().moe_dispatch(ctypes.byref(s), dt, p[0], p[1], p[2], p[3], p[4], p[5], p[6], FAKE, NULL)


def _gemm(s, dt=moe.MOE_BF16, ptrs=None):
    p = ptrs or [FAKE] * 6
    return moe.lib().moe_grouped_gemm(ctypes.byref(s), dt, p[0], p[1], p[2], p[3], p[4], p[5], NULL, NULL)


def _combine(s, dt=moe.MOE_BF16, ptrs=None):
    p = ptrs or [FAKE] * 4
    return moe.lib().moe_combine(ctypes.byref(s), dt, p[0], p[1], p[2], p[3], NULL)


@pytest.mark.parametrize("kw", [dict(k=0), dict(k=9), dict(E=0), dict(T=-1), dict(T=2**30, k=4)])
def test_route_rejects_bad_shapes(kw):
    assert _route(_shape(**kw)) == moe.MOE_EINVAL


def test_route_rejects_null_and_large_E():
    assert _route(_shape(), logits=NULL) == moe.MOE_EINVAL
    assert _route(_shape(), idx=NULL) == moe.MOE_EINVAL
    assert _route(_shape(E=2048, k=2)) == moe.MOE_EUNSUPPORTED
    assert moe.lib().moe_route_topk(None, FAKE, FAKE, FAKE, NULL) == moe.MOE_EINVAL


@pytest.mark.parametrize("kw", [dict(d=12), dict(d_ff=20), dict(d=0), dict(e_begin=4, e_end=4),
                                dict(e_begin=-1), dict(e_end=9), dict(k=0)])
def test_layer_steps_reject_bad_shapes(kw):
    s = _shape(**kw)
    assert _dispatch(s) == moe.MOE_EINVAL
    assert _gemm(s) == moe.MOE_EINVAL
    assert _combine(s) == moe.MOE_EINVAL


def test_layer_steps_reject_null_and_bad_dtype():
    s = _shape()
    for i in range(7):
        p = [FAKE] * 7
        p[i] = NULL
        assert _dispatch(s, ptrs=p) == moe.MOE_EINVAL, i
    for i in range(6):
        p = [FAKE] * 6
        p[i] = NULL
        assert _gemm(s, ptrs=p) == moe.MOE_EINVAL, i
    for i in range(4):
        p = [FAKE] * 4
        p[i] = NULL
        assert _combine(s, ptrs=p) == moe.MOE_EINVAL, i
    assert _dispatch(s, dt=7) == moe.MOE_EINVAL
    assert _gemm(s, dt=7) == moe.MOE_EINVAL
    assert _combine(s, dt=7) == moe.MOE_EINVAL


def test_workspace_sizes():
    lib = moe.lib()
    s = _shape(T=0)
    assert lib.moe_dispatch_workspace_bytes(ctypes.byref(s)) == 0
    s = _shape(T=16384, k=8, E=256)
    # per (expert, chunk of 256 pairs): the histogram and the chunk bases; plus E totals
    assert lib.moe_dispatch_workspace_bytes(ctypes.byref(s)) == (2 * 256 * 512 + 256) * 4
    # chunks of 1024 pairs once the tables would pass 4M entries
    s = _shape(T=2**20, k=8, E=1024)
    assert lib.moe_dispatch_workspace_bytes(ctypes.byref(s)) == (2 * 1024 * 8192 + 1024) * 4
    assert lib.moe_grouped_gemm_workspace_bytes(ctypes.byref(s), moe.MOE_BF16) == 0


def test_zero_tokens_is_a_no_op_on_the_host():
    s = _shape(T=0)
    # T = 0: nothing is enqueued for route, gemm and combine, so null tensors are fine
    assert _route(s, logits=NULL, idx=NULL, w=NULL) == moe.MOE_OK
    assert _gemm(s, ptrs=[NULL] * 6) == moe.MOE_OK
    assert _combine(s, ptrs=[NULL] * 4) == moe.MOE_OK


def _dispatch_indices(s, ptrs=None):
    p = ptrs or [FAKE] * 5
    return moe.lib().moe_dispatch_indices(ctypes.byref(s), p[0], p[1], p[2], p[3], p[4], FAKE, NULL)


def _gemm_gather(s, dt=moe.MOE_BF16, ptrs=None):
    p = ptrs or [FAKE] * 7
    return moe.lib().moe_grouped_gemm_gather(ctypes.byref(s), dt, p[0], p[1], p[2], p[3], p[4], p[5], p[6],
                                             NULL, NULL)


def test_fused_path_entry_points_validate_on_the_host():
    s = _shape()
    for i in range(5):
        p = [FAKE] * 5
        p[i] = NULL
        assert _dispatch_indices(s, ptrs=p) == moe.MOE_EINVAL, i
    for i in range(7):
        p = [FAKE] * 7
        p[i] = NULL
        assert _gemm_gather(s, ptrs=p) == moe.MOE_EINVAL, i
    assert _dispatch_indices(_shape(k=0)) == moe.MOE_EINVAL
    assert _gemm_gather(_shape(d=12)) == moe.MOE_EINVAL
    assert _gemm_gather(s, dt=7) == moe.MOE_EINVAL
    # the row gather lives only in the pipelined bf16 kernel
    assert _gemm_gather(s, dt=moe.MOE_F32) == moe.MOE_EUNSUPPORTED
    assert _gemm_gather(_shape(d=72)) == moe.MOE_EUNSUPPORTED
    assert _gemm_gather(_shape(d_ff=40)) == moe.MOE_EUNSUPPORTED
    # x is addressed with 32-bit offsets: T * d * 2 bytes must stay below 2^31
    assert _gemm_gather(_shape(T=2**20, d=1024, k=1)) == moe.MOE_EUNSUPPORTED
    # T = 0: nothing is enqueued
    assert _gemm_gather(_shape(T=0), ptrs=[NULL] * 7) == moe.MOE_OK


def test_backward_entry_points_validate_on_the_host():
    lib = moe.lib()
    s = _shape()
    # combine backward: 6 pointers
    for i in range(6):
        p = [FAKE] * 6
        p[i] = NULL
        assert lib.moe_combine_backward(ctypes.byref(s), moe.MOE_BF16, *p, NULL) == moe.MOE_EINVAL, i
    # grouped GEMM backward: 10 pointers before the workspace
    for i in range(10):
        p = [FAKE] * 10
        p[i] = NULL
        assert lib.moe_grouped_gemm_backward(ctypes.byref(s), moe.MOE_BF16, *p, FAKE, NULL) == moe.MOE_EINVAL, i
    assert lib.moe_grouped_gemm_backward(ctypes.byref(s), moe.MOE_BF16, *([FAKE] * 10), NULL, NULL) == moe.MOE_EINVAL
    assert lib.moe_grouped_gemm_backward(ctypes.byref(s), moe.MOE_F32, *([FAKE] * 11), NULL) == moe.MOE_EUNSUPPORTED
    s72 = _shape(d=72)
    assert lib.moe_grouped_gemm_backward(ctypes.byref(s72), moe.MOE_BF16, *([FAKE] * 11), NULL) == \
        moe.MOE_EUNSUPPORTED
    # dispatch and route backward
    for i in range(3):
        p = [FAKE] * 3
        p[i] = NULL
        assert lib.moe_dispatch_backward(ctypes.byref(s), moe.MOE_BF16, *p, NULL) == moe.MOE_EINVAL, i
    for i in range(4):
        p = [FAKE] * 4
        p[i] = NULL
        assert lib.moe_route_topk_backward(ctypes.byref(s), *p, NULL) == moe.MOE_EINVAL, i
    # workspace: x_perm [N_max, d], two [N_max, 2 d_ff] blocks and a blocked copy of d_y [N_max, d], each
    # 256-byte aligned; none for fp32
    s = _shape(T=16, d=64, d_ff=64, k=2)
    n_max = 32
    assert lib.moe_grouped_gemm_backward_workspace_bytes(ctypes.byref(s), moe.MOE_BF16) == \
        2 * n_max * 64 * 2 + 2 * n_max * 128 * 2
    assert lib.moe_grouped_gemm_backward_workspace_bytes(ctypes.byref(s), moe.MOE_F32) == 0


def test_grouped_gemm_workspace_is_the_blocked_rows_when_they_pay():
    """moe_grouped_gemm_workspace_bytes: N_max * d * 2 bytes (the gathered rows in
    32-column blocks) plus 1 KB of per-XCD tile counts for bf16 when d_ff / 128 >= 20
    and N_max / E_loc >= 128; 0 otherwise, and for fp32."""
    lib = moe.lib()
    cases = [  # (T, d, d_ff, E, k, e_begin, e_end), blocked?
        ((4096, 4096, 14336, 8, 2, 0, 8), True),        # dense8: 112 column tiles, 1024 rows per expert
        ((8192, 2880, 2880, 128, 4, 0, 16), True),      # ep8_share128: 22, 2048
        ((16384, 7168, 2048, 256, 8, 0, 32), False),    # skew256: 16 column tiles
        ((32, 2880, 2880, 128, 4, 0, 128), False),      # decode32: 1 row per expert
        ((600, 128, 2560, 8, 2, 0, 8), True),           # 20, 150
        ((600, 128, 2528, 8, 2, 0, 8), False),          # 19 column tiles
        ((500, 128, 2560, 8, 2, 0, 8), False),          # 125 rows per expert
    ]
    for (T, d, d_ff, E, k, lo, hi), blocked in cases:
        s = moe.shape(T, d, d_ff, E, k, lo, hi)
        n_max = T * min(k, hi - lo)
        want = n_max * d * 2 + 1024 if blocked else 0
        assert lib.moe_grouped_gemm_workspace_bytes(ctypes.byref(s), moe.MOE_BF16) == want, (T, d, d_ff)
        assert lib.moe_grouped_gemm_workspace_bytes(ctypes.byref(s), moe.MOE_F32) == 0


# ----------------------------------------------------------------------------- debug build

debug_built = pytest.mark.skipif(not os.path.exists(moe.debug_lib_path), reason="libmoe_debug.so not built")


@debug_built
def test_debug_library_exports_every_declared_symbol_and_has_the_error_word():
    release = moe.lib()
    assert release.moe_dispatch_debug_word_offset() == moe._SIZE_MAX
    moe.set_debug(True)
    try:
        lib = moe.lib()
        for name in moe.declared_symbols():
            assert hasattr(lib, name), name
        assert lib.moe_dispatch_debug_word_offset() == 0
        # the word needs workspace even when there are no pairs, and a call without it is refused
        assert moe.dispatch_workspace_bytes(0, 2, 8) >= 4
        s = _shape(T=0)
        assert lib.moe_dispatch_indices(ctypes.byref(s), NULL, FAKE, FAKE, NULL, NULL, NULL, NULL) == moe.MOE_EINVAL
        assert moe.dispatch_workspace_bytes(100, 2, 8) > 4
    finally:
        moe.set_debug(False)
    assert moe.dispatch_workspace_bytes(0, 2, 8) == 0


def test_noalloc_dispatch_refuses_shapes_past_its_array():
    lib = moe.lib()
    big = _shape(T=1 << 20, k=8, E=256, e_begin=0, e_end=32)  # 8M pairs: a 64 MiB workspace
    assert moe.lib().moe_dispatch_workspace_bytes(ctypes.byref(big)) > 8 << 20
    assert lib.moe_dispatch_indices_noalloc(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, FAKE, NULL) == \
        moe.MOE_EUNSUPPORTED
    s = _shape()
    assert lib.moe_dispatch_indices_noalloc(ctypes.byref(s), FAKE, NULL, FAKE, FAKE, FAKE, NULL) == moe.MOE_EINVAL
    assert lib.moe_dispatch_indices_noalloc(ctypes.byref(s), NULL, FAKE, FAKE, FAKE, FAKE, NULL) == moe.MOE_EINVAL
    assert lib.moe_dispatch_indices_noalloc(ctypes.byref(_shape(k=9)), FAKE, FAKE, FAKE, FAKE, FAKE, NULL) == \
        moe.MOE_EINVAL
