"""Helpers shared by the GPU parity tests (no method arithmetic here)."""
import sys

import numpy as np
import torch

ATTN_MAX_ABS = 1e-2   # attention output vs the float64 oracle
ATTN_MEAN_ABS = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def np_(t):
    return t.detach().cpu().numpy()


def f64(t):
    """bf16 / any float tensor -> float64 numpy (exact for bf16)."""
    return t.detach().cpu().to(torch.float64).numpy()


def sel_of(idx_row, n):
    return np.asarray(idx_row[:n], dtype=np.int64)


def assert_attn_close(got, ref, what=""):
    """Max-abs per element and mean-abs over every element compared in one call."""
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    mx, mean = float(err.max()), float(err.mean())
    assert mx <= ATTN_MAX_ABS and mean <= ATTN_MEAN_ABS, f"{what}: max-abs {mx:.3g}, mean-abs {mean:.3g}"
    return mx, mean


class AttnErrors:
    """Collects (got, ref) pairs of one output tensor, then checks the
    tolerance over all of them: max-abs per element, mean-abs over the whole
    compared set (a row with few keys has |o| near 1, where bf16 output
    rounding alone is ~1e-3 on average)."""

    def __init__(self, what=""):
        self.what, self.n, self.sum, self.max = what, 0, 0.0, 0.0

    def add(self, got, ref):
        err = np.abs(np.asarray(got, dtype=np.float64) - ref)
        self.n += err.size
        self.sum += float(err.sum())
        self.max = max(self.max, float(err.max()))

    def check(self):
        mean = self.sum / max(1, self.n)
        assert self.max <= ATTN_MAX_ABS and mean <= ATTN_MEAN_ABS, \
            f"{self.what}: max-abs {self.max:.3g}, mean-abs {mean:.3g} over {self.n} values"
        return self.max, mean


def need_gpu():
    if not torch.cuda.is_available():
        import pytest
        pytest.skip("no GPU")
