"""Shared helpers of the GPU tests: pools from workloads, tolerance checks."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from lora_bgmv_shrink_amd import workloads as wl

HAS_GPU = torch.cuda.is_available()
requires_gpu = pytest.mark.skipif(not HAS_GPU, reason="needs an MI355X")

# |gpu - oracle| <= tol * max(1, |oracle|): fp32 path and bf16 inputs with fp32
# accumulation.
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def binding():
    from lora_bgmv_shrink_amd import binding as b
    return b


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def pool_of(p: wl.Pool):
    b = binding()
    if p.layout == wl.UNIFORM:
        return b.lora_pool_create(b.LORA_LAYOUT_UNIFORM, p.A, p.B, p.n_adapters, p.d_in, p.d_out, p.r_max,
                                  p.scales)
    return b.lora_pool_create(b.LORA_LAYOUT_RAGGED, p.A, p.B, p.n_adapters, p.d_in, p.d_out, p.r_max,
                              p.scales, ranks=p.ranks, a_off=p.a_off, b_off=p.b_off)


def ids_dev(w: wl.Workload, device="cuda") -> torch.Tensor:
    return torch.as_tensor(w.ids, dtype=torch.int32, device=device)


def scaled_err(gpu, ref) -> np.ndarray:
    g = gpu.detach().float().cpu().double().numpy() if isinstance(gpu, torch.Tensor) else np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    return np.abs(g - r) / np.maximum(1.0, np.abs(r))


def assert_close(gpu, ref, tol: float, what: str):
    e = scaled_err(gpu, ref)
    g = gpu.detach().float().cpu().numpy() if isinstance(gpu, torch.Tensor) else np.asarray(gpu)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    m = float(e.max()) if e.size else 0.0
    say(f"  {what}: max scaled err {m:.3e} (tol {tol:.0e}) over {e.size} values")
    assert m <= tol, f"{what}: max scaled err {m:.3e} > {tol:.1e}"


def w_stored(W: torch.Tensor, layout: int) -> torch.Tensor:
    """W in the storage layout the call uses (IN_OUT as generated, OUT_IN transposed once)."""
    b = binding()
    return W if layout == b.LORA_W_IN_OUT else W.t().contiguous()
