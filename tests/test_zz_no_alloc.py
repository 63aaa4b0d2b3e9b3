"""lora_layer_apply_noalloc (static device scratch, no workspace argument)
against lora_layer_apply on the same inputs, through the C ABI.

Each case makes two calls in a row on the shared scratch, the second with a
smaller batch, so the second runs over what the first left in the array.
Both must match lora_layer_apply to |gpu - oracle|-style tolerance (and, as
they run the same kernels in the same order, bit for bit).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from _gpu import TOL, assert_close, binding, ids_dev, pool_of, requires_gpu, say, w_stored
from lora_bgmv_shrink_amd import workloads as wl

pytestmark = [pytest.mark.gpu, requires_gpu]

DEV = "cuda"

# (what, first batch, second batch): the second is smaller; the modes cover
# the decode launches (<= 64 rows), the BGMV split form (65..2048 rows of a
# bf16 pool) and SGMV (segments, shrink, GEMM), uniform and ragged pools.
CASES = {
    "decode_bf16": [
        dict(seed=1, n_rows=64, d_in=1024, d_out=768, n_adapters=40, ranks=16, dtype=torch.bfloat16),
        dict(seed=2, n_rows=17, d_in=1024, d_out=768, n_adapters=40, ranks=16, dtype=torch.bfloat16),
    ],
    "bgmv_split_bf16": [
        dict(seed=3, n_rows=300, d_in=512, d_out=1024, n_adapters=200, ranks=16, dtype=torch.bfloat16),
        dict(seed=4, n_rows=90, d_in=512, d_out=1024, n_adapters=200, ranks=16, dtype=torch.bfloat16),
    ],
    "sgmv_bf16_ragged": [
        dict(seed=5, d_in=1000, d_out=776, n_adapters=12, ranks=[1, 3, 4, 8, 12, 16, 24, 32, 40, 64, 8, 16],
             layout=wl.RAGGED, dtype=torch.bfloat16, run_lengths=[300, 7, 200, 1, 64, 65, 63]),
        dict(seed=6, d_in=1000, d_out=776, n_adapters=12, ranks=[1, 3, 4, 8, 12, 16, 24, 32, 40, 64, 8, 16],
             layout=wl.RAGGED, dtype=torch.bfloat16, run_lengths=[100, 3, 40]),
    ],
    "f32_uniform": [
        dict(seed=7, n_rows=333, d_in=320, d_out=288, n_adapters=12, ranks=16, dtype=torch.float32),
        dict(seed=8, n_rows=45, d_in=320, d_out=288, n_adapters=12, ranks=16, dtype=torch.float32),
    ],
}


def _one(b, kw, mode, layout):
    w = wl.small_batch(device=DEV, frac_base=0.1, **kw)
    p = w.projections[0]
    pool = pool_of(p.pool)
    ids = ids_dev(w)
    Ws = w_stored(p.W, layout)
    y_ref = b.lora_layer_apply(pool, p.x, Ws, ids, w_layout=layout, mode=mode)
    y_na = torch.full_like(y_ref, float("nan"))
    b.lora_layer_apply_noalloc(pool, p.x, Ws, ids, layout, y_na, mode=mode)
    torch.cuda.synchronize()
    return w, pool, y_ref, y_na


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("mode", ["auto", "bgmv", "sgmv"])
def test_noalloc_matches_workspace_entry(name, mode):
    b = binding()
    m = {"auto": b.LORA_MODE_AUTO, "bgmv": b.LORA_MODE_BGMV, "sgmv": b.LORA_MODE_SGMV}[mode]
    layout = b.LORA_W_OUT_IN
    for k, kw in enumerate(CASES[name]):
        say(f"noalloc {name} mode {mode} call {k}: rows {kw.get('n_rows', sum(kw.get('run_lengths', [])))}")
        w, pool, y_ref, y_na = _one(b, kw, m, layout)
        assert_close(y_na, y_ref.double().cpu().numpy(), TOL[w.dtype], f"noalloc vs workspace ({name}, call {k})")
        assert torch.equal(y_na, y_ref), f"{name} call {k}: not the same bits as lora_layer_apply"
        pool.destroy()


def test_noalloc_in_out_layout_and_empty():
    b = binding()
    say("noalloc: W stored [d_in, d_out], then an empty batch")
    kw = CASES["f32_uniform"][0]
    w, pool, y_ref, y_na = _one(b, kw, b.LORA_MODE_AUTO, b.LORA_W_IN_OUT)
    assert torch.equal(y_na, y_ref)
    p = w.projections[0]
    empty = torch.zeros(0, dtype=torch.int32, device=DEV)
    y0 = torch.zeros((0, p.d_out), dtype=p.x.dtype, device=DEV)
    b.lora_layer_apply_noalloc(pool, p.x, p.W, empty, b.LORA_W_IN_OUT, y0)
    pool.destroy()


def test_noalloc_rejects_more_than_the_scratch():
    b = binding()
    # BGMV split form over a wide projection: n_rows * d_out * 4 bytes of
    # fp32 base partials, past the static array's size
    n_rows, d_in, d_out, n_ad, r = 1024, 256, 28672, 600, 16
    need = None
    A = torch.zeros((n_ad, d_in, r), dtype=torch.bfloat16, device=DEV)
    B = torch.zeros((n_ad, r, d_out), dtype=torch.bfloat16, device=DEV)
    pool = b.lora_pool_create(b.LORA_LAYOUT_UNIFORM, A, B, n_ad, d_in, d_out, r, 2.0)
    need = b.lora_layer_workspace(pool, n_rows, b.LORA_MODE_BGMV)
    say(f"noalloc: {need} bytes needed against {b.LORA_NOALLOC_SCRATCH_BYTES}")
    assert need > b.LORA_NOALLOC_SCRATCH_BYTES
    x = torch.zeros((n_rows, d_in), dtype=torch.bfloat16, device=DEV)
    W = torch.zeros((d_out, d_in), dtype=torch.bfloat16, device=DEV)
    ids = torch.zeros(n_rows, dtype=torch.int32, device=DEV)
    y = torch.full((n_rows, d_out), 7.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(b.LoraError) as e:
        b.lora_layer_apply_noalloc(pool, x, W, ids, b.LORA_W_OUT_IN, y, mode=b.LORA_MODE_BGMV)
    assert e.value.status == b.LORA_E_SCRATCH
    torch.cuda.synchronize()
    assert bool((y == 7.0).all()), "a rejected call must not touch y"
    pool.destroy()
