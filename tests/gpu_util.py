"""Shared helpers of the GPU tests: device copies, exact widening for the
oracle, and the parity bars.

Bars (the reading of the parity targets):
  * bf16 path: max |O_gpu - O_ref| <= 2e-2 over all elements, oracle fed the
    bf16-rounded inputs; plus a guard against trivially small outputs (at
    n = 8192 typical |O| is ~0.015): ||O_gpu - O_ref||_2 / ||O_ref||_2 <= 1e-2.
  * fp32 check path: max |O_gpu - O_ref| / max |O_ref| <= 1e-5.
"""
import sys

import numpy as np
import torch

BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 1e-2
F32_REL_MAX = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(t):
    return None if t is None else t.to("cuda")


def np64(t):
    """Exact widening: bf16 and fp32 values are representable in fp64."""
    return t.detach().to("cpu", torch.float32).double().numpy()


def check(out, ref, dtype, what=""):
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert out.shape == ref.shape, (out.shape, ref.shape)
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    err = np.abs(out - ref)
    if dtype == torch.bfloat16:
        max_abs = float(err.max()) if err.size else 0.0
        nref = float(np.linalg.norm(ref))
        rel_l2 = float(np.linalg.norm(out - ref)) / nref if nref > 0 else float(np.linalg.norm(out))
        say(f"  {what}: max_abs={max_abs:.3e} rel_l2={rel_l2:.3e}")
        assert max_abs <= BF16_MAX_ABS, f"{what}: max abs error {max_abs}"
        assert rel_l2 <= BF16_REL_L2, f"{what}: relative L2 error {rel_l2}"
    else:
        denom = float(np.abs(ref).max()) if ref.size else 0.0
        rel = float(err.max()) / denom if denom > 0 else float(err.max() if err.size else 0.0)
        say(f"  {what}: max_rel={rel:.3e}")
        assert rel <= F32_REL_MAX, f"{what}: relative max error {rel}"
