"""Helpers shared by the GPU tests: device transfer of seeded inputs and comparisons."""
import json
import os
import sys

import numpy as np
import pytest
import torch

LOGP_ATOL = 2e-3      # |delta logp|, |delta entropy| bound from the parity target
GRAD_RTOL = 1e-2      # normwise relative bound on gradients
# Regression guards beside the parity bounds. The fp32 accumulation of bf16 products gives
# logp/entropy/lse errors of a few 1e-6 at H=4096, and the bf16 rounding of G gives gradient
# errors of ~2e-3 normwise; a guard far below the bound but well above what is observed makes
# a large loss of accuracy fail even while it is still inside the bound.
LOGP_GUARD = 1e-4
GRAD_GUARD = 4e-3


def record(name, value):
    """Print an observed error and, when LLP_PARITY_LOG names a file, append it there as a
    JSON line (the record of what the parity runs observed)."""
    say(f"observed {name}: {value:.3e}")
    path = os.environ.get("LLP_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"check": name, "value": value}) + "\n")


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> device bf16 tensor (bit-exact)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def dev(x: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_bits_to_f64(u16: np.ndarray) -> np.ndarray:
    return (u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def assert_rows_close(gpu, ref, atol, name, rows=None):
    """Same -inf pattern, no NaN, finite entries within atol. Returns the max error."""
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    if rows is not None:
        g, r = g[rows], r[rows]
    assert not np.isnan(g).any(), f"{name}: NaN in GPU output"
    ninf_r, ninf_g = np.isneginf(r), np.isneginf(g)
    assert np.array_equal(ninf_r, ninf_g), f"{name}: -inf pattern differs at {np.nonzero(ninf_r != ninf_g)[0][:8]}"
    fin = ~ninf_r
    err = float(np.max(np.abs(g[fin] - r[fin]))) if fin.any() else 0.0
    assert err <= atol, f"{name}: max |gpu - oracle| = {err:.3g} > {atol}"
    return err


def normwise_rel(gpu, ref):
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(r)
    return float(np.linalg.norm(g - r) / den) if den > 0 else float(np.linalg.norm(g))


def bytes_equal(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))
