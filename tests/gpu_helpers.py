"""Shared helpers for the GPU tests: host<->device copies of numpy arrays and
the relative-error measure used for matvec parity.

Tolerance: per batch row, max_n |y_gpu - y_oracle| / max_n |y_oracle| <= 1e-3
(fp32 accumulation on the GPU against the fp64 oracle sum)."""
import numpy as np

RTOL = 1e-3


def torch():
    import torch as t
    return t


def dev(a: np.ndarray):
    t = torch()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return t.from_numpy(a.view(np.int16)).cuda().view(t.uint16)
    if a.dtype == np.uint32:   # 32-bit plane words travel as int32 (the binding allocates them so)
        return t.from_numpy(a.view(np.int32)).cuda()
    return t.from_numpy(a).cuda()


def host(x) -> np.ndarray:
    t = torch()
    if x.dtype == t.uint16:
        return x.view(t.int16).cpu().numpy().view(np.uint16)
    return x.cpu().numpy()


def bits_equal(a: np.ndarray, b: np.ndarray) -> bool:
    """Same shape and the same bytes (uint32 plane words against their int32 view)."""
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    return a.shape == b.shape and a.dtype.itemsize == b.dtype.itemsize and np.array_equal(a.view(np.uint8),
                                                                                         b.view(np.uint8))


def rel_err(y, ref):
    """Per batch row max |y - ref| / max |ref|; returns the worst row."""
    y = np.atleast_2d(np.asarray(y, np.float64))
    ref = np.atleast_2d(np.asarray(ref, np.float64))
    assert y.shape == ref.shape, (y.shape, ref.shape)
    worst = 0.0
    for b in range(ref.shape[0]):
        den = np.max(np.abs(ref[b]))
        num = np.max(np.abs(y[b] - ref[b]))
        worst = max(worst, num / den if den > 0 else num)
    return worst


def sample_rows(N, n=256, seed=0):
    """First, last and boundary rows plus a seeded random sample."""
    rng = np.random.default_rng(seed)
    fixed = [0, 1, N // 2, N - 2, N - 1]
    rnd = rng.choice(N, size=min(n, N), replace=False)
    return np.unique(np.concatenate([fixed, rnd]).clip(0, N - 1))
