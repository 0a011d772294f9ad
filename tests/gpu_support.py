"""Helpers of the GPU parity tests: tolerances, rounding of oracle values to device
dtypes, and comparison reports.  Values only ever flow oracle -> device, never back
into the oracle."""
import numpy as np
import torch

from oracle import csa_oracle as O

# fp32 inputs: max-abs 1e-5; bf16 inputs: max|gpu - ref| / max|ref| <= 2e-2 (norm-relative);
# KL loss: relative 1e-3.  "f32_sum" is the fp32 bound of the one reduced case whose outputs
# are sums of thousands of fp32 products of magnitude ~1 (64 heads x 512-wide rows): there an
# fp32 sum of n terms of magnitude m carries a rounding error of a few ulp(m) each, so the
# absolute 1e-5 applies per unit of max|ref| (1e-5 * max(1, max|ref|)).
TOL_F32_ABS = 1e-5
TOL_BF16_REL = 2e-2
TOL_LOSS_REL = 1e-3


def torch_dtype(name):
    return {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.bfloat16}[name]


def dev(x, dtype, device="cuda"):
    """A float64 oracle array rounded once to a device tensor of `dtype`."""
    return torch.as_tensor(np.ascontiguousarray(x), dtype=torch.float64).to(dtype).to(device)


def back(t):
    """Device tensor -> exact float64 numpy (for the comparison only)."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def rounded(x, dtype):
    """What the device sees when given `x` rounded to `dtype`, as float64."""
    return torch.as_tensor(np.asarray(x, dtype=np.float64)).to(dtype).to(torch.float64).numpy()


def check(name, got, ref, dtype, report=None, abs_tol=None, rel_tol=None):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values in the GPU result"
    err = float(np.abs(got - ref).max()) if got.size else 0.0
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    line = f"{name}: max_abs_err={err:.3e} max_ref={scale:.3e}"
    if report is not None:
        report.append(line)
    print(line, flush=True)
    if dtype == "f32":
        tol = abs_tol if abs_tol is not None else TOL_F32_ABS
        assert err <= tol, line
    elif dtype == "f32_sum":
        tol = (abs_tol if abs_tol is not None else TOL_F32_ABS) * max(1.0, scale)
        assert err <= tol, line
    else:
        tol = rel_tol if rel_tol is not None else TOL_BF16_REL
        assert err <= tol * max(scale, 1e-30), line + f" rel={err / max(scale, 1e-30):.3e}"


def idx_sets_equal(got, ref):
    """Compare idx rows as sets (-1 padding ignored); returns number of differing rows."""
    bad = 0
    for g, r in zip(np.asarray(got), np.asarray(ref)):
        if set(g[g >= 0].tolist()) != set(r[r >= 0].tolist()):
            bad += 1
    return bad


def real_rows(cu):
    return np.arange(int(cu[-1]))
