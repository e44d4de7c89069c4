"""Helpers shared by the GPU tests: host <-> device copies and error measures."""
import numpy as np

import moe_inputs as mi


def torch():
    import torch as _t
    return _t


def dev():
    return torch().device("cuda:0")


def to_dev(a: np.ndarray, dtype: str):
    """numpy input (bf16 bit patterns as uint16, or fp32/int32) -> device tensor."""
    t = torch()
    if dtype == "bf16":
        return t.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev()).view(t.bfloat16)
    return t.from_numpy(np.ascontiguousarray(a)).to(dev())


def to_f64(tensor) -> np.ndarray:
    """Device tensor -> exact fp64 values on the host."""
    t = torch()
    if tensor.dtype == t.bfloat16:
        return mi.bf16_bits_to_f32(tensor.contiguous().view(t.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    return tensor.cpu().numpy().astype(np.float64)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / max |ref| (0 when both are empty or all zero)."""
    if ref.size == 0:
        return 0.0
    scale = np.abs(ref).max()
    err = np.abs(got - ref).max()
    if scale == 0:
        return float(err)
    return float(err / scale)


def row_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """The worst row of max |got - ref| / max |ref| taken row by row; a row whose
    reference is all zero counts its largest |got - ref| (0 when both are zero)."""
    if ref.size == 0:
        return 0.0
    scale = np.abs(ref).max(axis=1)
    err = np.abs(got - ref).max(axis=1)
    zero = scale == 0
    return float(np.where(zero, err, err / np.where(zero, 1.0, scale)).max())


# max |err| / max |ref| bound on floating outputs: bf16 activations and weights
# with fp32 accumulation, fp32 throughout for the fp32 path.
TOL = {"bf16": 2e-2, "f32": 1e-5}
# routing weights are computed in fp32 on the device and fp64 in the oracle
W_ATOL = 1e-6
