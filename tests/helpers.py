"""Shared test utilities: tolerance metrics and bitwise comparison."""
import numpy as np
import torch


def f64(t):
    """A torch tensor (any float dtype, any device) as a float64 numpy array."""
    return t.detach().to("cpu", torch.float64).numpy()


def row_rel_err(got, ref):
    """Per-row normwise relative error: max_j |got - ref| / max_j |ref| (rows = leading dims)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    g = got.reshape(-1, got.shape[-1])
    r = ref.reshape(-1, ref.shape[-1])
    num = np.max(np.abs(g - r), axis=1)
    den = np.max(np.abs(r), axis=1)
    den = np.where(den == 0, 1.0, den)
    return num / den


def bits(t):
    """Exact bit pattern of a bf16 / fp32 tensor as an integer numpy array."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy()
    if t.dtype in (torch.int32, torch.int64):
        return t.numpy()
    raise TypeError(t.dtype)


def assert_bitwise_equal(a, b, what=""):
    ba, bb = bits(a), bits(b)
    if not np.array_equal(ba, bb):
        n = int(np.sum(ba != bb))
        raise AssertionError(f"{what}: {n} of {ba.size} elements differ bitwise")


# gated tolerances: bf16 outputs and fp32 logits
TOL_BF16 = 2e-2
TOL_F32_LOGITS = 1e-3


def gpu_available():
    return torch.cuda.is_available()
