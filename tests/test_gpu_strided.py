"""Leading dimensions larger than the row width, through every entry point.

Inputs sit in wider buffers whose padding holds NaN (a value the result must
never depend on); outputs sit in wider buffers whose padding holds a canary
that must come back bit for bit.  Results are compared with the same call on
contiguous tensors (same kernels, so the same bits) and with the oracle.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from _gpu import TOL, assert_close, binding, ids_dev, pool_of, requires_gpu, say, w_stored
from _marshal import f64, run_oracle
from lora_bgmv_shrink_amd import workloads as wl

pytestmark = [pytest.mark.gpu, requires_gpu]

DEV = "cuda"
CANARY = 1234.5   # exact in bf16 and fp32


def padded(t: torch.Tensor, extra: int, fill) -> torch.Tensor:
    """A copy of 2-D ``t`` inside a [rows, cols + extra] buffer (padding = fill), as a view."""
    buf = torch.full((t.shape[0], t.shape[1] + extra), fill, dtype=t.dtype, device=t.device)
    buf[:, : t.shape[1]] = t
    return buf[:, : t.shape[1]]


def out_buf(rows, cols, extra, dtype):
    return torch.full((rows, cols + extra), CANARY, dtype=dtype, device=DEV)


def check_canary(buf: torch.Tensor, cols: int, what: str):
    pad = buf[:, cols:]
    assert bool((pad == CANARY).all()), f"{what}: padding columns were written"


def _batch(n, d_in, d_out, ranks=16, layout=wl.UNIFORM, n_ad=12, dtype=torch.bfloat16, runs=None, seed=0):
    return wl.small_batch(seed=seed, n_rows=n, d_in=d_in, d_out=d_out, n_adapters=n_ad, ranks=ranks, layout=layout,
                          dtype=dtype, device=DEV, frac_base=0.1, run_lengths=runs,
                          scale=np.linspace(-1.5, 2.0, n_ad).astype(np.float32))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_shrink_and_expand_strided(dtype):
    say(f"strided BGMV/SGMV shrink and expand ({dtype})")
    b = binding()
    w = _batch(150, 520, 776, ranks=[8, 16, 3, 64, 24, 1, 32, 40, 12, 16, 8, 64], layout=wl.RAGGED, dtype=dtype)
    p = w.projections[0]
    pool = pool_of(p.pool)
    ids = ids_dev(w)
    o = run_oracle(w)
    xs = padded(p.x, 24, float("nan"))
    seg = b.lora_segments_build(ids, p.pool.n_adapters)
    for mode in ("bgmv", "sgmv"):
        tb = out_buf(w.n_rows, p.pool.r_max, 12, torch.float32)
        t = tb[:, : p.pool.r_max]
        if mode == "bgmv":
            b.lora_bgmv_shrink(pool, xs, ids, t=t)
        else:
            b.lora_sgmv_shrink(pool, xs, seg, t=t)
        torch.cuda.synchronize()
        check_canary(tb, p.pool.r_max, f"t ({mode})")
        assert_close(t, o["t"], TOL[dtype], f"t strided ({mode})")
        tn = padded(t.clone(), 20, float("nan"))
        for ydt in (torch.float32, torch.bfloat16):
            for acc in (False, True):
                yb = out_buf(w.n_rows, p.d_out, 8 if ydt == torch.bfloat16 else 4, ydt)
                y = yb[:, : p.d_out]
                y.zero_()
                if mode == "bgmv":
                    b.lora_bgmv_expand(pool, tn, ids, y=y, accumulate=acc)
                else:
                    b.lora_sgmv_expand(pool, tn, seg, y=y, accumulate=acc)
                torch.cuda.synchronize()
                check_canary(yb, p.d_out, f"y ({mode}, {ydt}, acc {acc})")
                assert_close(y, o["lora"], TOL[torch.bfloat16], f"lora term strided ({mode}, {ydt}, acc {acc})")


# (rows, d_in, d_out, ranks, layout, W layout, mode): the decode launches,
# the few-hundred-row path, SGMV, the fused GEMM ([d_in, d_out] W)
LAYER = [
    (40, 1024, 776, 16, wl.UNIFORM, "out_in", "bgmv"),
    (300, 1000, 776, [8, 16, 3, 64, 24, 1, 32, 40, 12, 16, 8, 64], wl.RAGGED, "out_in", "bgmv"),
    (300, 1000, 776, [8, 16, 3, 64, 24, 1, 32, 40, 12, 16, 8, 64], wl.RAGGED, "out_in", "sgmv"),
    (300, 1000, 776, 16, wl.UNIFORM, "in_out", "bgmv"),
    (700, 512, 8200, 16, wl.UNIFORM, "out_in", "bgmv"),
]


@pytest.mark.parametrize("case", LAYER, ids=[f"{c[0]}-{c[5]}-{c[6]}" for c in LAYER])
@pytest.mark.parametrize("ydt", [torch.bfloat16, torch.float32])
def test_layer_strided(case, ydt):
    n, d_in, d_out, ranks, layout, wlay, mode = case
    say(f"strided layer: {n} x {d_in} -> {d_out}, W {wlay}, {mode}, y {ydt}")
    b = binding()
    w = _batch(n, d_in, d_out, ranks=ranks, layout=layout)
    p = w.projections[0]
    pool = pool_of(p.pool)
    ids = ids_dev(w)
    lay = b.LORA_W_OUT_IN if wlay == "out_in" else b.LORA_W_IN_OUT
    m = b.LORA_MODE_BGMV if mode == "bgmv" else b.LORA_MODE_SGMV
    Wc = w_stored(p.W, lay)
    y0 = b.lora_layer_apply(pool, p.x, Wc, ids, w_layout=lay, mode=m, y_dtype=ydt)
    xs = padded(p.x, 40, float("nan"))
    Ws = padded(Wc, 16, float("nan"))
    yb = out_buf(n, d_out, 8 if ydt == torch.bfloat16 else 4, ydt)
    y = yb[:, :d_out]
    b.lora_layer_apply(pool, xs, Ws, ids, w_layout=lay, mode=m, y=y)
    torch.cuda.synchronize()
    check_canary(yb, d_out, "layer y")
    assert torch.equal(y, y0), "strided call differs from the contiguous one"
    o = run_oracle(w, cols=None if d_out <= 1024 else list(range(0, d_out, 37)) + [d_out - 1])
    ys = y if d_out <= 1024 else y[:, list(range(0, d_out, 37)) + [d_out - 1]]
    assert_close(ys, o["y"], TOL[torch.bfloat16], "layer strided")
    # the no-allocation entry point on the same strided buffers
    yb2 = out_buf(n, d_out, 8 if ydt == torch.bfloat16 else 4, ydt)
    b.lora_layer_apply_noalloc(pool, xs, Ws, ids, lay, yb2[:, :d_out], mode=m)
    torch.cuda.synchronize()
    check_canary(yb2, d_out, "noalloc y")
    assert torch.equal(yb2[:, :d_out], y0)


def test_base_gemm_expand_strided():
    say("strided lora_base_gemm_expand")
    b = binding()
    w = _batch(200, 1000, 520, ranks=32)
    p = w.projections[0]
    pool = pool_of(p.pool)
    ids = ids_dev(w)
    o = run_oracle(w)
    t = b.lora_bgmv_shrink(pool, p.x, ids)
    for lay in (b.LORA_W_OUT_IN, b.LORA_W_IN_OUT):
        y0 = b.lora_base_gemm_expand(pool, p.x, w_stored(p.W, lay), ids, t, w_layout=lay, y_dtype=torch.float32)
        yb = out_buf(200, 520, 4, torch.float32)
        b.lora_base_gemm_expand(pool, padded(p.x, 8, float("nan")), padded(w_stored(p.W, lay), 8, float("nan")),
                                ids, padded(t, 12, float("nan")), w_layout=lay, y=yb[:, :520])
        torch.cuda.synchronize()
        check_canary(yb, 520, "base_gemm_expand y")
        assert torch.equal(yb[:, :520], y0)
        assert_close(y0, o["y"], TOL[torch.bfloat16], f"base_gemm_expand layout {lay}")


def test_decode_pair_and_q4_strided():
    say("strided decode launches, bf16 and 4-bit W")
    b = binding()
    n, d_in, d_out = 33, 1024, 640
    w = _batch(n, d_in, d_out, ranks=16)
    p = w.projections[0]
    pool = pool_of(p.pool)
    ids = ids_dev(w)
    ws = torch.zeros(b.lora_decode_workspace(pool, n, True), dtype=torch.uint8, device=DEV)
    Wt = w_stored(p.W, b.LORA_W_OUT_IN)
    y0 = torch.empty((n, d_out), dtype=torch.bfloat16, device=DEV)
    b.lora_decode_stream(pool, p.x, Wt, ids, ws, True)
    b.lora_decode_finish(pool, ids, ws, y0, True)
    yb = out_buf(n, d_out, 8, torch.bfloat16)
    b.lora_decode_stream(pool, padded(p.x, 16, float("nan")), padded(Wt, 8, float("nan")), ids, ws, True)
    b.lora_decode_finish(pool, ids, ws, yb[:, :d_out], True)
    torch.cuda.synchronize()
    check_canary(yb, d_out, "decode y")
    assert torch.equal(yb[:, :d_out], y0)
    # 4-bit: padded byte rows (ldq > d_in / 2) and scale rows (lds > d_in / 128)
    Wq, sc = wl.q4_weight(40, d_in, d_out, DEV)
    Wqp = torch.full((d_out, d_in // 2 + 16), 0x77, dtype=torch.uint8, device=DEV)
    Wqp[:, : d_in // 2] = Wq
    scp = padded(sc, 4, float("nan"))
    for nn in (n, 200):
        w2 = _batch(nn, d_in, d_out, ranks=16, seed=nn)
        p2 = w2.projections[0]
        pool2 = pool_of(p2.pool)
        ids2 = ids_dev(w2)
        yq0 = b.lora_layer_apply_q4(pool2, p2.x, Wq, sc, ids2)
        yqb = out_buf(nn, d_out, 8, torch.bfloat16)
        b.lora_layer_apply_q4(pool2, padded(p2.x, 24, float("nan")), Wqp[:, : d_in // 2], scp, ids2,
                              y=yqb[:, :d_out])
        torch.cuda.synchronize()
        check_canary(yqb, d_out, f"q4 layer y ({nn} rows)")
        assert torch.equal(yqb[:, :d_out], yq0)


def test_merge_strided_leaves_padding():
    say("strided merge: padding of W untouched")
    b = binding()
    w = _batch(8, 520, 776, ranks=16)
    p = w.projections[0]
    pool = pool_of(p.pool)
    for lay in (b.LORA_W_OUT_IN, b.LORA_W_IN_OUT):
        Wc = w_stored(p.W, lay).clone()
        Wb = torch.full((Wc.shape[0], Wc.shape[1] + 8), CANARY, dtype=Wc.dtype, device=DEV)
        Wb[:, : Wc.shape[1]] = Wc
        b.lora_merge_adapter(pool, Wc, 3, lay)
        b.lora_merge_adapter(pool, Wb[:, : Wc.shape[1]], 3, lay)
        torch.cuda.synchronize()
        check_canary(Wb, Wc.shape[1], "merged W")
        assert torch.equal(Wb[:, : Wc.shape[1]], Wc)
