"""moe_dispatch_indices_noalloc, the dispatch for callers that cannot allocate:
called through the C ABI, it must give moe_dispatch_indices' outputs bit for
bit, on consecutive calls that share the library's per-GPU workspace array (the
second call smaller than the first, so stale contents of the larger one are
still there)."""
import ctypes

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import token_dispatch_grouped_amd as moe  # noqa: E402


def _outputs(T, k, E):
    dev = torch.device("cuda:0")
    fill = lambda n: torch.full((n,), -7, dtype=torch.int32, device=dev)  # noqa: E731
    return dict(counts=fill(E), offsets=fill(E + 1), perm=fill(T * k), pair_pos=fill(T * k))


def _run(name, T, k, E, lo, hi, idx, out, ws=None):
    s = moe.shape(T, 8, 8, E, k, lo, hi)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    lib = moe.lib()
    if name == "noalloc":
        st = lib.moe_dispatch_indices_noalloc(ctypes.byref(s), p(idx), p(out["counts"]), p(out["offsets"]),
                                              p(out["perm"]), p(out["pair_pos"]), stream)
    else:
        st = lib.moe_dispatch_indices(ctypes.byref(s), p(idx), p(out["counts"]), p(out["offsets"]), p(out["perm"]),
                                      p(out["pair_pos"]), p(ws), stream)
    assert st == moe.MOE_OK, (name, st)


@pytest.mark.parametrize("shapes", [
    [(16384, 8, 256, 0, 32), (700, 4, 128, 16, 32), (300, 2, 8, 0, 8)],  # two launches, one launch, one workgroup
], ids=["large_then_smaller"])
def test_noalloc_matches_dispatch_indices(shapes):
    for T, k, E, lo, hi in shapes:
        print(f"noalloc dispatch T={T} k={k} E={E} local [{lo}, {hi})", flush=True)
        rng = np.random.default_rng(T + E)
        logits = rng.standard_normal((T, E)) + rng.normal(0.0, 1.5, size=E)  # skewed expert loads
        idx_np = np.argsort(-logits, axis=1, kind="stable")[:, :k].astype(np.int32)
        idx = torch.from_numpy(idx_np).cuda()
        ws = torch.empty(max(1, moe.dispatch_workspace_bytes(T, k, E)), dtype=torch.uint8, device="cuda")
        assert moe.dispatch_workspace_bytes(T, k, E) <= 8 << 20
        want, got = _outputs(T, k, E), _outputs(T, k, E)
        _run("indices", T, k, E, lo, hi, idx, want, ws)
        _run("noalloc", T, k, E, lo, hi, idx, got)
        torch.cuda.synchronize()
        for key in want:
            assert torch.equal(got[key], want[key]), (T, key)
        assert int(want["offsets"][E].item()) == T * k
