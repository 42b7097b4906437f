"""Helpers shared by the GPU parity tests: device copies, tolerances and the
normwise comparison of a HIP-path output against the oracle.

Tolerances (normwise relative error ||y - y_ref||_2 / ||y_ref||_2 over a
tensor, and per expert): 1e-3 for fp32 outputs, 1e-2 for bf16/fp16 outputs.
"""
import sys

import numpy as np
import torch

from oracle import oracle as orc
from moe_grouped_gemm_offset_amd import synth

TOL = {orc.F32: 1e-3, orc.BF16: 1e-2, orc.F16: 1e-2}
ORC_DT = {torch.float32: orc.F32, torch.bfloat16: orc.BF16, torch.float16: orc.F16,
          torch.float8_e4m3fn: orc.E4M3, torch.float8_e5m2: orc.E5M2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(x):
    return x.cuda() if isinstance(x, torch.Tensor) else x


def normwise(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((got - ref).ravel())
    if den == 0.0:
        return 0.0 if num == 0.0 else np.inf
    return num / den


def values(t):
    """float64 numpy values of a tensor (any float dtype)."""
    return t.detach().float().double().cpu().numpy() if t.dtype != torch.float64 else t.cpu().numpy()


def assert_close(got, ref, dtype, what):
    err = normwise(got, ref)
    say(f"  {what}: normwise rel err {err:.3e} (tol {TOL[dtype]:.0e})")
    assert err <= TOL[dtype], f"{what}: normwise error {err:.3e} > {TOL[dtype]:.0e}"
    return err
