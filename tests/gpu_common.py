"""Helpers shared by the GPU parity tests: device copies and tolerance checks."""
import math
import sys

import numpy as np
import pytest
import torch

TOL_OUT = {torch.float16: 2e-3, torch.bfloat16: 1e-2, torch.float32: 1e-2}
TOL_GRAD = 1e-2
TOL_FP8 = 5e-2
TOL_LSE_REL = 1e-4


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(t):
    return t.contiguous().cuda()


def assert_close_out(got, ref, tol, what):
    g = got.detach().float().cpu().double().numpy()
    err = np.abs(g - ref)
    bad = ~(err <= tol)
    assert not bad.any(), f"{what}: max abs err {np.nanmax(err):.3e} > {tol} at {np.argwhere(bad)[:5].tolist()}"
    return float(np.nanmax(err)) if err.size else 0.0


def assert_close_lse(got, ref, what):
    g = got.detach().cpu().double().numpy()
    inf_ref = np.isneginf(ref)
    assert np.array_equal(np.isneginf(g), inf_ref), f"{what}: -inf pattern differs"
    fin = ~inf_ref
    err = np.abs(g[fin] - ref[fin])
    lim = TOL_LSE_REL * np.maximum(1.0, np.abs(ref[fin]))
    assert np.all(err <= lim), f"{what}: LSE max err {err.max():.3e}"
    return float(err.max()) if err.size else 0.0
