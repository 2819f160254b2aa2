"""Helpers shared by the GPU parity tests: device copies of seeded inputs and the error metrics.

Tolerances: bf16 storage must meet max-abs <= 2e-2 AND relative L2 <= 5e-3 over the checked
elements; the fp32 checking mode must meet max-abs <= 1e-5 AND relative L2 <= 1e-5.  Relative L2
is ||got - ref||_2 / ||ref||_2 over the same elements.
"""
import sys

import numpy as np
import torch

from st_inputs import QKV

BF16_MAX_ABS, BF16_REL_L2 = 2e-2, 5e-3
F32_MAX_ABS, F32_REL_L2 = 1e-5, 1e-5


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(x: QKV, device="cuda"):
    if x.dtype == "f32":
        return tuple(torch.from_numpy(np.ascontiguousarray(a)).to(device) for a in (x.q, x.k, x.v))
    return tuple(torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(device)
                 for b in (x.q_bits, x.k_bits, x.v_bits))


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def errors(got: np.ndarray, ref: np.ndarray):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    diff = got - ref
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff) / nref) if nref > 0 else float(np.linalg.norm(diff))
    return max_abs, rel


def assert_close(got, ref, dtype: str, what: str = ""):
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    max_abs, rel = errors(got, ref)
    log(f"    {what}: max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    if dtype == "bf16":
        assert max_abs <= BF16_MAX_ABS and rel <= BF16_REL_L2, (what, max_abs, rel)
    else:
        assert max_abs <= F32_MAX_ABS and rel <= F32_REL_L2, (what, max_abs, rel)
    return max_abs, rel
