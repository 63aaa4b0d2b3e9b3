"""Decode over a 4-bit base weight (lora_decode_stream_q4 + lora_decode_finish)
against the fp64 oracle on the widened weight, through the C ABI.

The weight format is the reading stated in include/lora_mi355x.h (signed
nibbles, one fp32 scale per output and 128 inputs); the oracle widens it with
its own plain loop (pinned in test_oracle_pins.py).  x and the adapters are
bf16 with fp32 accumulation: |gpu - oracle| <= 2e-2 * max(1, |oracle|).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from _gpu import TOL, assert_close, binding, pool_of, requires_gpu, say
from _marshal import f64, oracle_pool
from lora_bgmv_shrink_amd import workloads as wl

pytestmark = [pytest.mark.gpu, requires_gpu]

DEV = "cuda"


def _run_q4(b, pool, x, Wq, sc, ids, with_lora):
    n = ids.numel()
    ws = torch.zeros(b.lora_decode_workspace(pool, n, with_lora), dtype=torch.uint8, device=DEV)
    y = torch.empty((n, pool.d_out), dtype=torch.bfloat16, device=DEV)
    b.lora_decode_stream_q4(pool, x, Wq, sc, ids, ws, with_lora)
    b.lora_decode_finish(pool, ids, ws, y, with_lora)
    torch.cuda.synchronize()
    return y


def _oracle_y(x, Wq, sc, ids_np, op, d_in, with_lora):
    W = oracle.dequant_q4(Wq.cpu().numpy(), sc.cpu().double().numpy(), d_in)
    ids_o = ids_np if with_lora else np.full_like(ids_np, -1)
    return oracle.layer(f64(x), W, ids_o, op, want=("y",))["y"]


@pytest.mark.parametrize("d_in,d_out", [(1024, 776), (4096, 1024), (1536, 2048)])
@pytest.mark.parametrize("n_rows", [1, 7, 32, 64])
@pytest.mark.parametrize("with_lora", [True, False])
def test_q4_decode_matches_oracle(d_in, d_out, n_rows, with_lora):
    say(f"q4 decode: {d_in}->{d_out}, {n_rows} rows, lora {with_lora}")
    b = binding()
    w = wl.small_batch(seed=11, n_rows=n_rows, d_in=d_in, d_out=d_out, n_adapters=6, ranks=16,
                       dtype=torch.bfloat16, device=DEV, frac_base=0.15)
    p = w.projections[0]
    pool = pool_of(p.pool)
    op, _ = oracle_pool(p.pool)
    Wq, sc = wl.q4_weight(1, d_in, d_out, DEV)
    ids = torch.as_tensor(w.ids, device=DEV)
    y = _run_q4(b, pool, p.x, Wq, sc, ids, with_lora)
    ref = _oracle_y(p.x, Wq, sc, w.ids, op, d_in, with_lora)
    assert_close(y, ref, TOL[torch.bfloat16], "q4 decode")


def test_q4_agrees_with_bf16_decode_on_exact_weights():
    """Power-of-two scales make every 4-bit weight exact in bf16: the 4-bit
    path and the bf16 decode path then compute the same layer."""
    b = binding()
    d_in, d_out, n = 2048, 1024, 24
    w = wl.small_batch(seed=12, n_rows=n, d_in=d_in, d_out=d_out, n_adapters=5, ranks=32,
                       dtype=torch.bfloat16, device=DEV, frac_base=0.1)
    p = w.projections[0]
    pool = pool_of(p.pool)
    Wq, sc = wl.q4_weight(2, d_in, d_out, DEV, pow2_scales=True)
    Wd = oracle.dequant_q4(Wq.cpu().numpy(), sc.cpu().double().numpy(), d_in)     # [d_in, d_out]
    Wb = torch.from_numpy(Wd.T.copy()).to(torch.bfloat16).to(DEV)                  # stored [d_out, d_in]
    assert np.array_equal(Wb.double().cpu().numpy().T, Wd)
    ids = torch.as_tensor(w.ids, device=DEV)
    y4 = _run_q4(b, pool, p.x, Wq, sc, ids, True)
    yb = b.lora_layer_apply(pool, p.x, Wb, ids, w_layout=b.LORA_W_OUT_IN, mode=b.LORA_MODE_BGMV)
    torch.cuda.synchronize()
    op, _ = oracle_pool(p.pool)
    ref = oracle.layer(f64(p.x), Wd, w.ids, op, want=("y",))["y"]
    assert_close(y4, ref, TOL[torch.bfloat16], "q4 vs oracle")
    assert_close(yb, ref, TOL[torch.bfloat16], "bf16 vs oracle")
    d = (y4.float() - yb.float()).abs().max().item()
    say(f"  max |q4 - bf16| = {d:.3e}")
    assert d <= 2e-2 * max(1.0, yb.float().abs().max().item())


def test_q4_decode_q_proj_full_size():
    """The 8B q projection decode batch (4096 -> 4096, 32 rows, 20 adapters,
    pool of 250) on a 4-bit base: every output against the oracle, and the
    run is bit-identical when repeated."""
    b = binding()
    w = wl.decode_q_proj(device=DEV)
    p = w.projections[0]
    pool = pool_of(p.pool)
    Wq, sc = wl.q4_weight(3, 4096, 4096, DEV)
    ids = torch.as_tensor(w.ids, device=DEV)
    y = _run_q4(b, pool, p.x, Wq, sc, ids, True)
    y2 = _run_q4(b, pool, p.x, Wq, sc, ids, True)
    assert torch.equal(y, y2)
    used = sorted(set(int(a) for a in w.ids if a >= 0))
    op, mp = oracle_pool(p.pool, used=used)
    from _marshal import remap_ids
    ref = _oracle_y(p.x, Wq, sc, remap_ids(w.ids, mp, p.pool.n_adapters), op, 4096, True)
    assert_close(y, ref, TOL[torch.bfloat16], "q4 q_proj")


def test_q4_argument_checks():
    b = binding()
    w = wl.small_batch(seed=1, n_rows=4, d_in=1024, d_out=256, n_adapters=2, ranks=16, dtype=torch.bfloat16,
                       device=DEV)
    p = w.projections[0]
    pool = pool_of(p.pool)
    Wq, sc = wl.q4_weight(4, 1024, 256, DEV)
    ids = torch.as_tensor(w.ids, device=DEV)
    ws = torch.zeros(b.lora_decode_workspace(pool, 4, True), dtype=torch.uint8, device=DEV)
    with pytest.raises(b.LoraError) as e:           # scales for fewer groups than d_in needs
        b.lora_decode_stream_q4(pool, p.x, Wq, sc[:, :4].contiguous(), ids, ws, True)
    assert e.value.status == b.LORA_E_INVALID
    with pytest.raises(b.LoraError) as e:           # rows shorter than d_in / 2 bytes
        b.lora_decode_stream_q4(pool, p.x, Wq[:, :511].contiguous(), sc, ids, ws, True)
    assert e.value.status == b.LORA_E_INVALID
    w2 = wl.small_batch(seed=1, n_rows=4, d_in=1000, d_out=256, n_adapters=2, ranks=16, dtype=torch.bfloat16,
                        device=DEV)
    pool2 = pool_of(w2.projections[0].pool)
    Wq2 = torch.zeros((256, 512), dtype=torch.uint8, device=DEV)
    sc2 = torch.ones((256, 8), dtype=torch.float32, device=DEV)
    with pytest.raises(b.LoraError) as e:           # d_in not a multiple of 128
        b.lora_decode_stream_q4(pool2, w2.projections[0].x, Wq2, sc2, ids, ws, True)
    assert e.value.status == b.LORA_E_UNSUPPORTED


def test_q4_decode_ragged_pool_fp32_y():
    """A ragged pool of ranks 8/16/32/64 and an fp32 y on the 4-bit base."""
    b = binding()
    d_in, d_out, n = 2048, 768, 40
    w = wl.small_batch(seed=13, n_rows=n, d_in=d_in, d_out=d_out, n_adapters=8, ranks=[8, 16, 32, 64] * 2,
                       layout=wl.RAGGED, dtype=torch.bfloat16, device=DEV, frac_base=0.1)
    p = w.projections[0]
    pool = pool_of(p.pool)
    op, _ = oracle_pool(p.pool)
    Wq, sc = wl.q4_weight(6, d_in, d_out, DEV)
    ids = torch.as_tensor(w.ids, device=DEV)
    ws = torch.zeros(b.lora_decode_workspace(pool, n, True), dtype=torch.uint8, device=DEV)
    y = torch.empty((n, d_out), dtype=torch.float32, device=DEV)
    b.lora_decode_stream_q4(pool, p.x, Wq, sc, ids, ws, True)
    b.lora_decode_finish(pool, ids, ws, y, True)
    torch.cuda.synchronize()
    ref = _oracle_y(p.x, Wq, sc, w.ids, op, d_in, True)
    assert_close(y, ref, TOL[torch.bfloat16], "q4 ragged, fp32 y")


# ---------------------------------------------------------------------------
# The layer over a 4-bit base at any batch size (lora_layer_apply_q4)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n_rows,d_in,d_out,layout,ranks,n_ad,runs", [
    (40, 1024, 776, wl.UNIFORM, 16, 6, None),                     # decode launches
    (65, 1024, 776, wl.UNIFORM, 16, 30, None),                    # segment-tile path
    (300, 2048, 1032, wl.RAGGED, [8, 16, 32, 64, 1, 3, 24, 40], 8, None),
    (700, 1536, 520, wl.UNIFORM, 64, 5, [300, 7, 200, 1, 64, 65, 63]),
    (1100, 1024, 640, wl.RAGGED, [8, 16, 32, 64] * 3, 12, [500, 1, 300, 299]),   # fused GEMM (past 1024 rows)
    (1500, 2048, 1000, wl.RAGGED, [1, 3, 24, 40, 64, 16], 6, [700, 2, 300, 1, 497]),   # odd ranks, ragged d_out
    (2100, 256, 6144, wl.UNIFORM, 32, 4, [1000, 600, 500]),     # 256 x 256 tiles of the fused GEMM
])
@pytest.mark.parametrize("ydt", [torch.bfloat16, torch.float32])
def test_q4_layer_matches_oracle(n_rows, d_in, d_out, layout, ranks, n_ad, runs, ydt):
    say(f"q4 layer: {n_rows} rows, {d_in}->{d_out}, y {ydt}")
    b = binding()
    w = wl.small_batch(seed=n_rows, n_rows=n_rows, d_in=d_in, d_out=d_out, n_adapters=n_ad, ranks=ranks,
                       layout=layout, dtype=torch.bfloat16, device=DEV, frac_base=0.1, run_lengths=runs,
                       scale=np.linspace(-2.0, 2.0, n_ad).astype(np.float32))
    p = w.projections[0]
    pool = pool_of(p.pool)
    op, _ = oracle_pool(p.pool)
    Wq, sc = wl.q4_weight(20 + n_rows, d_in, d_out, DEV)
    ids = torch.as_tensor(w.ids, device=DEV)
    y = b.lora_layer_apply_q4(pool, p.x, Wq, sc, ids, y_dtype=ydt)
    y2 = b.lora_layer_apply_q4(pool, p.x, Wq, sc, ids, y_dtype=ydt,
                               seg=b.lora_segments_build(ids, p.pool.n_adapters))
    torch.cuda.synchronize()
    assert torch.equal(y, y2), "caller's segments give other bits"
    ref = _oracle_y(p.x, Wq, sc, w.ids, op, d_in, True)
    assert_close(y, ref, TOL[torch.bfloat16], "q4 layer")


def test_q4_layer_agrees_with_bf16_layer_on_exact_weights():
    """Power-of-two scales: the 4-bit layer and the bf16 layer (W stored
    [d_out, d_in]) compute the same function at 300 rows."""
    b = binding()
    d_in, d_out, n = 2048, 1024, 300
    w = wl.small_batch(seed=14, n_rows=n, d_in=d_in, d_out=d_out, n_adapters=50, ranks=16,
                       dtype=torch.bfloat16, device=DEV, frac_base=0.1)
    p = w.projections[0]
    pool = pool_of(p.pool)
    Wq, sc = wl.q4_weight(7, d_in, d_out, DEV, pow2_scales=True)
    Wd = oracle.dequant_q4(Wq.cpu().numpy(), sc.cpu().double().numpy(), d_in)
    Wb = torch.from_numpy(Wd.T.copy()).to(torch.bfloat16).to(DEV)
    ids = torch.as_tensor(w.ids, device=DEV)
    y4 = b.lora_layer_apply_q4(pool, p.x, Wq, sc, ids, y_dtype=torch.float32)
    yb = b.lora_layer_apply(pool, p.x, Wb, ids, w_layout=b.LORA_W_OUT_IN, mode=b.LORA_MODE_BGMV,
                            y_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_close(y4, f64(yb), 1e-4, "q4 vs bf16 layer (fp32 y)")


def test_q4_layer_past_1024_rows_agrees_with_bf16_layer_on_exact_weights():
    """Past 1024 rows the 4-bit weight is widened to bf16(q * scale) in the
    fused GEMM's tiles; with power-of-two scales that widening is exact, so
    the 4-bit layer and the bf16 SGMV layer on the dequantized weight
    compute the same function."""
    b = binding()
    d_in, d_out, n = 1024, 1536, 1300
    w = wl.small_batch(seed=16, n_rows=n, d_in=d_in, d_out=d_out, n_adapters=6, ranks=64, dtype=torch.bfloat16,
                       device=DEV, frac_base=0.05, run_lengths=[400, 300, 1, 599])
    p = w.projections[0]
    pool = pool_of(p.pool)
    Wq, sc = wl.q4_weight(9, d_in, d_out, DEV, pow2_scales=True)
    Wd = oracle.dequant_q4(Wq.cpu().numpy(), sc.cpu().double().numpy(), d_in)
    Wb = torch.from_numpy(Wd.T.copy()).to(torch.bfloat16).to(DEV)
    ids = torch.as_tensor(w.ids, device=DEV)
    y4 = b.lora_layer_apply_q4(pool, p.x, Wq, sc, ids, y_dtype=torch.float32)
    yb = b.lora_layer_apply(pool, p.x, Wb, ids, w_layout=b.LORA_W_OUT_IN, mode=b.LORA_MODE_SGMV,
                            y_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_close(y4, f64(yb), 1e-4, "q4 vs bf16 SGMV layer (fp32 y)")


def test_q4_layer_small_batch_is_the_decode_pair():
    b = binding()
    w = wl.small_batch(seed=15, n_rows=33, d_in=1024, d_out=512, n_adapters=7, ranks=16,
                       dtype=torch.bfloat16, device=DEV, frac_base=0.1)
    p = w.projections[0]
    pool = pool_of(p.pool)
    Wq, sc = wl.q4_weight(8, 1024, 512, DEV)
    ids = torch.as_tensor(w.ids, device=DEV)
    y = b.lora_layer_apply_q4(pool, p.x, Wq, sc, ids)
    y2 = _run_q4(b, pool, p.x, Wq, sc, ids, True)
    assert torch.equal(y, y2)


@pytest.mark.parametrize("proj", ["q", "k", "down"])
def test_q4_layer_prefill_70b(proj):
    """The 70B prefill batch (16 requests, 8 rank-64 adapters, rows in
    arrival order) over a 4-bit base weight: sampled rows (every request
    boundary) x sampled columns against the oracle on the widened weight of
    those columns."""
    from _marshal import oracle_pool as opool, remap_ids
    say(f"q4 layer, 70B prefill {proj}: sampled rows x columns")
    b = binding()
    w = wl.prefill_70b(device=DEV, projections=[proj])
    p = w.projections[0]
    pool = pool_of(p.pool)
    Wq, sc = wl.q4_weight(30, p.d_in, p.d_out, DEV)
    ids = torch.as_tensor(w.ids, device=DEV)
    y = b.lora_layer_apply_q4(pool, p.x, Wq, sc, ids)
    torch.cuda.synchronize()
    rng = np.random.default_rng(31)
    n = w.n_rows
    rows = set(rng.choice(n, 40, replace=False).tolist()) | {0, n - 1}
    off = np.cumsum([0] + list(w.lengths))
    for o in off[1:-1]:
        rows |= {int(o) - 1, int(o)}
    rows = sorted(rows)
    cols = sorted(set(rng.choice(p.d_out, 160, replace=False).tolist()) | {0, p.d_out - 1})
    ci = torch.as_tensor(cols, device=DEV)
    Wd = oracle.dequant_q4(Wq[ci].cpu().numpy(), sc[ci].cpu().double().numpy(), p.d_in)   # [d_in, len(cols)]
    ids_r = w.ids[rows]
    op, mp = opool(p.pool, used=ids_r.tolist(), cols=cols)
    ref = oracle.layer(f64(p.x[torch.as_tensor(rows, device=DEV)]), Wd, remap_ids(ids_r, mp, p.pool.n_adapters),
                       op, want=("y",), threads=0)["y"]
    assert_close(y[rows][:, cols], ref, TOL[torch.bfloat16], "q4 prefill sampled")
