"""Shared helpers for the GPU parity tests: tolerance checks against the fp64
oracle and seeded sampling of rows for workloads too large to check in full.

Tolerances (element-wise, against the fp64 oracle on the same input bits):
  bf16 inputs : O max |err| <= 2e-2 and mean |err| <= 2e-3; LSE max |err| <= 2.5e-3
  fp32 inputs : O max |err| <= 1e-5;                         LSE max |err| <= 1e-5

The O bounds are the ones the method is held to.  The LSE bound for bf16 is
derived from the arithmetic: the MFMA paths round every probability p to bf16
(relative error <= 2^-9) before it enters both P.V and the running sum l, so
l -- and hence exp(LSE) -- carries a relative error of at most 2^-9, i.e.
|dLSE| <= ln(1 + 2^-9) = 1.95e-3; the remaining 5.5e-4 covers the fp32 score
accumulation, the hardware exp2/log2 and the fp32 sum of up to 32K terms.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

TOL = {
    torch.bfloat16: dict(o_max=2e-2, o_mean=2e-3, lse_max=2.5e-3),
    torch.float32: dict(o_max=1e-5, o_mean=1e-5, lse_max=1e-5),
}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check_close(name, o_gpu, o_ref, lse_gpu, lse_ref, dtype):
    tol = TOL[dtype]
    og = o_gpu.detach().float().cpu().numpy().astype(np.float64) if isinstance(o_gpu, torch.Tensor) else o_gpu
    lg = lse_gpu.detach().cpu().numpy().astype(np.float64) if isinstance(lse_gpu, torch.Tensor) else lse_gpu
    assert np.isfinite(og).all(), "%s: non-finite output" % name
    err = np.abs(og - o_ref)
    lerr = np.abs(lg - lse_ref)
    log("  %s: O max %.3e mean %.3e | LSE max %.3e" % (name, err.max(), err.mean(), lerr.max()))
    assert err.max() <= tol["o_max"], (name, float(err.max()))
    assert err.mean() <= tol["o_mean"], (name, float(err.mean()))
    assert lerr.max() <= tol["lse_max"], (name, float(lerr.max()))
    return float(err.max()), float(err.mean()), float(lerr.max())
