"""Shared helpers for the GPU parity tests: tolerance checks against the fp64
oracle and seeded sampling of rows for workloads too large to check in full.

Tolerances (element-wise, against the fp64 oracle on the same input bits):
  bf16 inputs : O max |err| <= 2e-2 and mean |err| <= 2e-3; LSE max |err| <= 2.5e-3
  fp32 inputs : O max |err| <= 1e-5;                         LSE max |err| <= 1e-5

The O bounds are the ones the method is held to.  The LSE bound for bf16 is a
worst case of the fp32 arithmetic: the running sum l adds the fp32
probabilities (p itself is rounded to bf16 only as the P.V operand), so LSE
carries the rounding of the fp32 scores (d = 128 exact bf16 products summed in
fp32: at most 127 u sum|q_i k_i| scale, ~5e-5 for N(0,1) inputs at scale
1/sqrt(d)), of the sum of up to 33K positive terms (at most (n - 1) u = 2.0e-3
relative, u = 2^-24) and of the hardware exp2 / log2 (a few ulp) -- together
under 2.5e-3.

Regression margins (bf16 inputs; asserted beside the bounds above, which at
long context are of the order of the outputs themselves, so a tile-level
mistake could hide under them):
  per row, mean |err| <= 1e-2 rms(O_ref row) + 2e-5
  LSE max |err| <= 2.5e-4
The rounding model behind the first: O is rounded to bf16 once (mean error
2^-10 .. 2^-9 of |o|, about 1.1e-3 of the row's rms) and each p to bf16
before P.V (relative 2^-9 per key, about 1.1e-3 |v| / sqrt(N_eff) over the
N_eff keys a row effectively weighs, again about 1e-3 of the rms), so a
row's mean error is a few thousandths of its rms (C3: about 3.5e-3), and
1e-2 leaves a factor of ~3; one 32-key tile dropped from an 8192-key row
(rms ~0.018) moves its mean by ~5.6e-4, about 3e-2 of the rms, which the
margin catches.  The floor is 1e-3 of the smallest row rms of the workloads
(~0.009 at 33K keys).  The LSE margin is five times the score-rounding bound
above; with random inputs the fp32 sum contributes about sqrt(n) u ~ 1e-5.
The long-context cases (up to 262144 keys in one row) are past the length
for which the worst case (n - 1) u of the fp32 sum stays under the LSE bound
(it reaches 1.6e-2 there); the rounding errors of a sum of positive terms
that are not adversarially ordered grow like sqrt(n) u (~3e-5 at 262144),
and those cases are held to the same bounds and margins.
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


# regression margins for bf16 inputs (module docstring)
ROW_MEAN_RMS = 1e-2
ROW_FLOOR = 2e-5
LSE_MARGIN = 2.5e-4


def check_close(name, o_gpu, o_ref, lse_gpu, lse_ref, dtype):
    tol = TOL[dtype]
    og = o_gpu.detach().float().cpu().numpy().astype(np.float64) if isinstance(o_gpu, torch.Tensor) else o_gpu
    lg = lse_gpu.detach().cpu().numpy().astype(np.float64) if isinstance(lse_gpu, torch.Tensor) else lse_gpu
    o_ref = np.asarray(o_ref, dtype=np.float64)
    assert np.isfinite(og).all(), "%s: non-finite output" % name
    err = np.abs(og - o_ref)
    lerr = np.abs(lg - lse_ref)
    d = o_ref.shape[-1]
    row_err = err.reshape(-1, d).mean(axis=1)
    row_rms = np.sqrt((o_ref.reshape(-1, d) ** 2).mean(axis=1))
    ratio = row_err / (ROW_MEAN_RMS * row_rms + ROW_FLOOR)
    log("  %s: O max %.3e mean %.3e | LSE max %.3e | worst row mean/rms %.2e (margin used %.2f)"
        % (name, err.max(), err.mean(), lerr.max(), float((row_err / np.maximum(row_rms, 1e-30)).max()),
           float(ratio.max())))
    assert err.max() <= tol["o_max"], (name, float(err.max()))
    assert err.mean() <= tol["o_mean"], (name, float(err.mean()))
    assert lerr.max() <= tol["lse_max"], (name, float(lerr.max()))
    if dtype == torch.bfloat16:
        worst = int(ratio.argmax())
        assert ratio.max() <= 1.0, (name, "row", worst, float(row_err[worst]), float(row_rms[worst]))
        assert lerr.max() <= LSE_MARGIN, (name, float(lerr.max()))
    return float(err.max()), float(err.mean()), float(lerr.max())
