"""lora_merge_adapter (W += sign * s_a * A_a B_a, in place) against the fp64
oracle, through the C ABI.

Floats within |gpu - oracle| <= tol * max(1, |oracle|) with tol 1e-4 (fp32
W) or 2e-2 (bf16 W, fp32 arithmetic, one rounding per element).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from _gpu import TOL, assert_close, binding, pool_of, requires_gpu, say, w_stored
from _marshal import f64, oracle_pool
from lora_bgmv_shrink_amd import workloads as wl

pytestmark = [pytest.mark.gpu, requires_gpu]

DEV = "cuda"
RAGGED_RANKS = [1, 3, 4, 8, 12, 16, 24, 32, 40, 64, 8, 16]

CASES = {
    "bf16_uniform_r16": dict(dtype=torch.bfloat16, layout=wl.UNIFORM, ranks=16, d_in=320, d_out=288, n_adapters=4),
    "bf16_ragged": dict(dtype=torch.bfloat16, layout=wl.RAGGED, ranks=RAGGED_RANKS, d_in=1000, d_out=776,
                        n_adapters=12),
    "bf16_uniform_r64_tails": dict(dtype=torch.bfloat16, layout=wl.UNIFORM, ranks=64, d_in=200, d_out=136,
                                   n_adapters=3),
    "f32_ragged": dict(dtype=torch.float32, layout=wl.RAGGED, ranks=RAGGED_RANKS, d_in=1000, d_out=772,
                       n_adapters=12),
}


def _case(name):
    kw = dict(CASES[name])
    scale = np.linspace(-1.5, 2.5, kw["n_adapters"]).astype(np.float32)
    return wl.small_batch(seed=7, n_rows=8, device=DEV, frac_base=0.0, scale=scale, **kw)


def _stored_to_in_out(Ws, lay, b):
    return Ws if lay == b.LORA_W_IN_OUT else Ws.t()


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("wl_layout", ["in_out", "out_in"])
def test_merge_matches_oracle(name, wl_layout):
    say(f"merge vs oracle: {name}, W {wl_layout}")
    b = binding()
    w = _case(name)
    p = w.projections[0]
    pool = pool_of(p.pool)
    op, _ = oracle_pool(p.pool)
    lay = b.LORA_W_IN_OUT if wl_layout == "in_out" else b.LORA_W_OUT_IN
    W0 = f64(p.W)
    for a, sign in ((0, 1.0), (p.pool.n_adapters - 1, -1.0), (p.pool.n_adapters // 2, 0.5)):
        Ws = w_stored(p.W, lay).clone()
        b.lora_merge_adapter(pool, Ws, a, w_layout=lay, sign=sign)
        torch.cuda.synchronize()
        ref = oracle.merge(W0, op, a, sign)
        assert_close(_stored_to_in_out(Ws, lay, b), ref, TOL[w.dtype], f"adapter {a} sign {sign}")


@pytest.mark.parametrize("name", ["bf16_ragged", "f32_ragged"])
def test_merge_then_unmerge(name):
    """Taking the adapter back out restores W to within one rounding per step."""
    say(f"merge then unmerge: {name}")
    b = binding()
    w = _case(name)
    p = w.projections[0]
    pool = pool_of(p.pool)
    for a in (2, 9):
        Ws = p.W.clone()
        b.lora_merge_adapter(pool, Ws, a, b.LORA_W_IN_OUT, sign=1.0)
        b.lora_merge_adapter(pool, Ws, a, b.LORA_W_IN_OUT, sign=-1.0)
        torch.cuda.synchronize()
        assert_close(Ws, f64(p.W), TOL[w.dtype], f"unmerged adapter {a}")


def test_merged_weight_serves_the_adapter():
    """A merged replica answers the adapter's requests with the base GEMM
    alone, matching the multi-LoRA layer on the unmerged weight.

    The merged bf16 weight carries one rounding per element (relative error
    at most 2^-9), which the product x W' sums over d_in terms; so beside the
    layer's tolerance the merged product may differ from x (W + s A B) by up
    to 2^-9 * (|x| |W'|) per output (taken as 2^-8 for margin), computed
    from the oracle's W'."""
    say("merged weight vs multi-LoRA layer")
    b = binding()
    w = wl.small_batch(seed=21, n_rows=150, device=DEV, dtype=torch.bfloat16, d_in=512, d_out=384,
                       n_adapters=5, layout=wl.RAGGED, ranks=[4, 16, 64, 8, 32], frac_base=0.0)
    p = w.projections[0]
    pool = pool_of(p.pool)
    for lay in (b.LORA_W_IN_OUT, b.LORA_W_OUT_IN):
        for a in range(5):
            ids = torch.full((w.n_rows,), a, dtype=torch.int32, device=DEV)
            Ws = w_stored(p.W, lay)
            y_lora = b.lora_layer_apply(pool, p.x, Ws, ids, w_layout=lay, y_dtype=torch.float32)
            Wm = b.lora_merge_adapter(pool, Ws.clone(), a, w_layout=lay)
            y_merged = b.lora_base_gemm_expand(pool, p.x, Wm, ids, None, w_layout=lay, y_dtype=torch.float32)
            torch.cuda.synchronize()
            Wref = oracle.merge(f64(p.W), oracle_pool(p.pool)[0], a)
            ref = f64(p.x) @ Wref
            assert_close(y_lora, ref, TOL[torch.bfloat16], f"multi-LoRA layer, adapter {a}, layout {lay}")
            bound = TOL[torch.bfloat16] * np.maximum(1.0, np.abs(ref)) + 2.0 ** -8 * (np.abs(f64(p.x)) @ np.abs(Wref))
            err = np.abs(y_merged.double().cpu().numpy() - ref)
            say(f"  merged base GEMM, adapter {a}, layout {lay}: max err / bound {float((err / bound).max()):.3f}")
            assert np.all(err <= bound), f"merged base GEMM, adapter {a}, layout {lay}"


def test_merge_q_proj_full_size():
    """8B q_proj (4096 x 4096), rank-16 pool of 250: every element checked."""
    say("merge at full size: 4096 x 4096, r16")
    b = binding()
    w = wl.decode_q_proj(device=DEV)
    p = w.projections[0]
    pool = pool_of(p.pool)
    op, _ = oracle_pool(p.pool, used=[17])
    for lay in (b.LORA_W_OUT_IN, b.LORA_W_IN_OUT):
        Ws = w_stored(p.W, lay).clone()
        b.lora_merge_adapter(pool, Ws, 17, w_layout=lay)
        torch.cuda.synchronize()
        ref = oracle.merge(f64(p.W), op, 0)
        assert_close(_stored_to_in_out(Ws, lay, b), ref, TOL[torch.bfloat16], f"layout {lay}")


def test_merge_argument_errors():
    b = binding()
    w = _case("bf16_uniform_r16")
    p = w.projections[0]
    pool = pool_of(p.pool)
    Ws = p.W.clone()
    for bad in (-1, p.pool.n_adapters):
        with pytest.raises(b.LoraError) as e:
            b.lora_merge_adapter(pool, Ws, bad, b.LORA_W_IN_OUT)
        assert e.value.status == b.LORA_E_ID_RANGE
    with pytest.raises(b.LoraError) as e:
        b.lora_merge_adapter(pool, Ws, 0, b.LORA_W_IN_OUT, sign=float("nan"))
    assert e.value.status == b.LORA_E_INVALID
    torch.cuda.synchronize()
    assert torch.equal(Ws, p.W), "a rejected call changed W"
