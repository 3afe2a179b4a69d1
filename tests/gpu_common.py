"""Shared helpers for the GPU parity tests (test infrastructure)."""
import sys

import numpy as np

TOL = {"f32": 2.0 ** -19, "bf16": 2.0 ** -7, "f16": 2.0 ** -7}


def say(*args):
    """Name the case before each GPU step, flushed, so a failing run says where it was."""
    print("[gpu-case]", *args, flush=True)
    sys.stdout.flush()


def to_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def from_dev(t):
    import torch
    if t.dtype in (torch.bfloat16, torch.float16):
        t = t.float()
    return t.cpu().numpy()


def check_gemm(d, d_ref, s_ref, out, label=""):
    """max |D - D_ref| / S <= tolerance; where S == 0, D must be 0."""
    d = np.asarray(d, dtype=np.float64)
    err = np.abs(d - d_ref)
    zero = s_ref == 0
    assert np.all(d[zero] == 0), f"{label}: nonzero output where every product is zero"
    if np.any(~zero):
        ratio = err[~zero] / s_ref[~zero]
        worst = float(ratio.max())
    else:
        worst = 0.0
    lg = np.log2(worst) if worst > 0 else -np.inf
    say(f"{label}: max |D-Dref|/S = {worst:.3e} (2^{lg:.2f}), tolerance 2^{np.log2(TOL[out]):.0f}")
    assert worst <= TOL[out], f"{label}: {worst:.3e} > {TOL[out]:.3e}"
    return worst


def check_gemm_ex(d, d_ref, s_ref, alpha, beta, c, out, label=""):
    """The alpha/beta epilogue: |D - (alpha D_ref + beta C)| <= tol (|alpha| S + |beta C|),
    the reference composed in fp64 from the oracle's product; where the bound is
    0, D must be 0."""
    d = np.asarray(d, dtype=np.float64)
    cc = np.zeros_like(d) if c is None else np.asarray(c, dtype=np.float64)
    ref = alpha * d_ref + beta * cc
    bound = abs(alpha) * s_ref + np.abs(beta * cc)
    err = np.abs(d - ref)
    zero = bound == 0
    assert np.all(d[zero] == 0), f"{label}: nonzero output where the exact result is 0"
    worst = float((err[~zero] / bound[~zero]).max()) if np.any(~zero) else 0.0
    lg = np.log2(worst) if worst > 0 else -np.inf
    say(f"{label}: max |D-ref|/(|a|S+|bC|) = {worst:.3e} (2^{lg:.2f}), tolerance 2^{np.log2(TOL[out]):.0f}")
    assert worst <= TOL[out], f"{label}: {worst:.3e} > {TOL[out]:.3e}"
    return worst
