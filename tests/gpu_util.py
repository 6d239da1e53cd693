"""Helpers shared by the GPU parity tests (comparison and tolerances)."""

import numpy as np
import torch

# Tolerances against the fp64 oracle on the same (bf16-rounded) inputs.
BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
BF16_LSE_MAX_ABS = 1e-3
F32_MAX_ABS = 1e-5
F32_LSE_MAX_ABS = 1e-5


def gpu_available():
    return torch.cuda.is_available()


def to_dev(*ts):
    return [t.to("cuda") for t in ts]


def f64(t):
    return t.detach().to("cpu").double().numpy()


def check_bf16(o_gpu, o_ref, what):
    err = np.abs(f64(o_gpu) - o_ref)
    assert np.isfinite(err).all(), f"{what}: non-finite output"
    mx, mean = err.max(), err.mean()
    assert mx <= BF16_MAX_ABS, f"{what}: max-abs {mx:.3e} > {BF16_MAX_ABS}"
    assert mean <= BF16_MEAN_ABS, f"{what}: mean-abs {mean:.3e} > {BF16_MEAN_ABS}"
    return mx, mean


def check_close(x_gpu, ref, tol, what):
    err = np.abs(f64(x_gpu) - ref)
    assert np.isfinite(err).all(), f"{what}: non-finite output"
    mx = err.max()
    assert mx <= tol, f"{what}: max-abs {mx:.3e} > {tol}"
    return mx
