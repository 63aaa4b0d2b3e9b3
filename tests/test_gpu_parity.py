"""HIP path vs the fp64 oracle, through the C ABI.

Segments are compared bit for bit; floats within |gpu - oracle| <=
tol * max(1, |oracle|) with tol 1e-4 (fp32) or 2e-2 (bf16 inputs, fp32
accumulation).  Mid-sized cases span several tiles and ragged tails; the
five workloads run at full size with outputs sampled where the oracle
would be too slow on every element.
"""
from __future__ import annotations

import json
import os

import numpy as np
import pytest
import torch

import oracle
from _gpu import TOL, assert_close, binding, ids_dev, pool_of, requires_gpu, say, scaled_err, w_stored
from _marshal import f64, run_oracle
from lora_bgmv_shrink_amd import workloads as wl

pytestmark = [pytest.mark.gpu, requires_gpu]

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
DEV = "cuda"


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# Segments (bit-exact)
# ---------------------------------------------------------------------------

def _check_segments(ids_np, n_adapters, what):
    b = binding()
    ids = torch.as_tensor(np.asarray(ids_np, np.int32), device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    seg = b.lora_segments_build(ids, n_adapters, status=status)
    perm, sid, soff = seg.host()
    rp, rs, ro, bad = oracle.segments(ids_np, n_adapters)
    assert perm[:len(rp)].tolist() == rp.tolist(), f"{what}: perm"
    assert sid.tolist() == rs.tolist(), f"{what}: seg_ids"
    assert soff.tolist() == ro.tolist(), f"{what}: seg_off"
    assert (int(status.item()) & 1) == (1 if bad else 0), f"{what}: status"


def test_segments_tiny_golden():
    say("segments: tiny batch (page script) golden")
    g = _golden("tiny_segments.json")
    w = wl.tiny_mixed_batch()
    seg = binding().lora_segments_build(ids_dev(w), 8)
    perm, sid, soff = seg.host()
    assert perm.tolist() == g["perm"]
    assert sid.tolist() == g["seg_ids"] and soff.tolist() == g["seg_off"]


def test_segments_walkthrough_golden():
    say("segments: T1,T2,T1,T3 golden")
    g = _golden("walkthrough_segments.json")
    seg = binding().lora_segments_build(torch.tensor(g["ids"], dtype=torch.int32, device=DEV), 8)
    perm, sid, soff = seg.host()
    assert perm.tolist() == g["perm"] and sid.tolist() == g["seg_ids"] and soff.tolist() == g["seg_off"]


@pytest.mark.parametrize("n,n_ad,mode", [
    (0, 5, "u"), (1, 1, "u"), (5, 3, "u"), (63, 10, "u"), (64, 10, "u"), (65, 10, "u"),
    (1000, 7, "runs"), (4097, 1000, "u"), (20000, 64, "runs"), (3000, 16383, "u"),
    (2500, 500, "bad"), (777, 1, "allbase"), (5000, 3, "u"),
])
def test_segments_random(n, n_ad, mode):
    say(f"segments: random n={n} n_adapters={n_ad} mode={mode}")
    rng = np.random.default_rng(n * 31 + n_ad)
    if mode == "runs":
        lens = rng.integers(1, 300, n)
        ids = np.concatenate([np.full(l, rng.integers(-1, n_ad)) for l in lens])[:n]
    elif mode == "allbase":
        ids = np.full(n, -1)
    else:
        ids = rng.integers(-1, n_ad, n)
    if mode == "bad" and n:
        ids[rng.integers(0, n, 20)] = rng.choice([-5, n_ad, n_ad + 100], 20)
    _check_segments(ids.astype(np.int32), n_ad, f"n={n}")


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_segments_workload_ids(cfg):
    say(f"segments: workload ids config {cfg}")
    ids = {1: lambda: wl.decode_q_proj_ids(), 2: lambda: wl.skewed_decode_ids(),
           3: lambda: wl.prefill_ids()[0], 4: lambda: wl.mixed_rank_ids()[0]}[cfg]()
    n_ad = {1: 250, 2: 1000, 3: 64, 4: 500}[cfg]
    _check_segments(ids, n_ad, f"config {cfg}")


# ---------------------------------------------------------------------------
# Mid-sized batches: several tiles, ragged K / N tails, every rank shape
# ---------------------------------------------------------------------------

RAGGED_RANKS = [1, 3, 4, 8, 12, 16, 24, 32, 40, 64, 8, 16]

CASES = {
    "f32_uniform": dict(dtype=torch.float32, layout=wl.UNIFORM, ranks=16, d_in=320, d_out=288, n_adapters=12),
    "bf16_uniform": dict(dtype=torch.bfloat16, layout=wl.UNIFORM, ranks=16, d_in=320, d_out=288, n_adapters=12),
    "bf16_ragged": dict(dtype=torch.bfloat16, layout=wl.RAGGED, ranks=RAGGED_RANKS, d_in=1000, d_out=776,
                        n_adapters=12),
    "f32_ragged": dict(dtype=torch.float32, layout=wl.RAGGED, ranks=RAGGED_RANKS, d_in=1000, d_out=772,
                       n_adapters=12),
    "bf16_r64_prefill": dict(dtype=torch.bfloat16, layout=wl.UNIFORM, ranks=64, d_in=512, d_out=384,
                             n_adapters=5, run_lengths=[130, 7, 300, 1, 64, 65, 200]),
}


def _case(name, seed=0):
    kw = dict(CASES[name])
    scale = np.linspace(-1.5, 2.5, kw["n_adapters"]).astype(np.float32)
    w = wl.small_batch(seed=seed, n_rows=333, device=DEV, frac_base=0.1, scale=scale, **kw)
    return w


_cache = {}


def _oracle(name):
    if name not in _cache:
        w = _case(name)
        _cache[name] = (w, run_oracle(w))
    return _cache[name]


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("mode", ["bgmv", "sgmv"])
def test_shrink(name, mode):
    say(f"shrink {mode}: {name}")
    b = binding()
    w, o = _oracle(name)
    p = w.projections[0]
    pool = pool_of(p.pool)
    ids = ids_dev(w)
    if mode == "bgmv":
        t = b.lora_bgmv_shrink(pool, p.x, ids)
    else:
        seg = b.lora_segments_build(ids, p.pool.n_adapters)
        t = b.lora_sgmv_shrink(pool, p.x, seg)
    torch.cuda.synchronize()
    assert_close(t, o["t"], TOL[w.dtype], f"t ({mode}, {name})")
    base = w.ids == -1
    assert np.all(t.cpu().numpy()[base] == 0)


@pytest.mark.parametrize("ranks", [16, [8, 16, 32, 64, 24, 8]])
@pytest.mark.parametrize("split", [True, False])
def test_sgmv_shrink_split_and_unsplit(ranks, split):
    """The standalone SGMV shrink with its K-split workspace and without
    (ws = NULL), on a shape where the split gives 4 slices: both match the
    oracle, columns past each rank and base-only rows are exactly 0, and a
    repeated call is bit-identical."""
    say(f"sgmv shrink split={split} ranks={ranks}")
    b = binding()
    layout = wl.UNIFORM if isinstance(ranks, int) else wl.RAGGED
    w = wl.small_batch(seed=21, n_rows=300, d_in=4096, d_out=256, n_adapters=6, ranks=ranks, layout=layout,
                       dtype=torch.bfloat16, device="cuda", run_lengths=[40, 3, 77, 1, 120, 59])
    p = w.projections[0]
    pool = pool_of(p.pool)
    ids = ids_dev(w)
    if split:
        assert b.lora_sgmv_shrink_workspace(pool, w.n_rows) > 0
    seg = b.lora_segments_build(ids, p.pool.n_adapters)
    t = b.lora_sgmv_shrink(pool, p.x, seg, split=split)
    t2 = b.lora_sgmv_shrink(pool, p.x, seg, split=split)
    torch.cuda.synchronize()
    assert torch.equal(t, t2)
    o = run_oracle(w, want=("t",))
    assert_close(t, o["t"], TOL[torch.bfloat16], f"t split={split}")
    tn = t.cpu().numpy()
    assert np.all(tn[w.ids == -1] == 0)
    for i, a in enumerate(w.ids.tolist()):
        if a >= 0:
            assert np.all(tn[i, int(p.pool.ranks[a]):] == 0)


@pytest.mark.parametrize("case", [
    # long runs at rank 64 (prefill-like), whole K-blocks
    dict(seed=31, d_in=4096, n_adapters=5, ranks=64, layout=wl.UNIFORM,
         runs=[700, 1, 530, 129, 128, 2, 300]),
    # ranks that are multiples of 8 but not powers of two, a ragged K tail
    # (2104 = 32 x 64 + 56) and base-only rows inside the runs
    dict(seed=32, d_in=2104, n_adapters=6, ranks=[8, 24, 64, 40, 16, 56], layout=wl.RAGGED,
         runs=[260, 3, 129, 1, 400, 77, 64]),
    # hundreds of short runs over 600 adapters: more tiles than workgroups
    # the GPU holds, so workgroups take several tiles of different ranks
    dict(seed=33, d_in=2048, n_adapters=600, ranks=([8, 16, 32, 64, 24] * 120), layout=wl.RAGGED,
         runs=None, n_rows=2000),
])
def test_sgmv_shrink_long_segments(case):
    """The split-K SGMV shrink on pools whose ranks are multiples of 8 (the
    transpose-read kernel): t matches the oracle, columns past each rank and
    base-only rows are exactly 0, a repeated call is bit-identical, and the
    unsplit shrink (ws = NULL, other kernel) agrees within the tolerance."""
    say(f"sgmv shrink, long segments: seed {case['seed']} d_in {case['d_in']}")
    b = binding()
    w = wl.small_batch(seed=case["seed"], n_rows=case.get("n_rows", 200), d_in=case["d_in"], d_out=128,
                       n_adapters=case["n_adapters"], ranks=case["ranks"], layout=case["layout"],
                       dtype=torch.bfloat16, device="cuda", run_lengths=case["runs"], frac_base=0.05)
    p = w.projections[0]
    pool = pool_of(p.pool)
    ids = ids_dev(w)
    assert b.lora_sgmv_shrink_workspace(pool, w.n_rows) > 0
    seg = b.lora_segments_build(ids, p.pool.n_adapters)
    t = b.lora_sgmv_shrink(pool, p.x, seg, split=True)
    t2 = b.lora_sgmv_shrink(pool, p.x, seg, split=True)
    tu = b.lora_sgmv_shrink(pool, p.x, seg, split=False)
    torch.cuda.synchronize()
    assert torch.equal(t, t2)
    o = run_oracle(w, want=("t",))
    assert_close(t, o["t"], TOL[torch.bfloat16], "t split")
    assert_close(tu, o["t"], TOL[torch.bfloat16], "t unsplit")
    tn = t.cpu().numpy()
    assert np.all(tn[w.ids == -1] == 0)
    for i, a in enumerate(w.ids.tolist()):
        if a >= 0:
            assert np.all(tn[i, int(p.pool.ranks[a]):] == 0)


@pytest.mark.parametrize("n_rows,d_out", [(64, 256), (20, 128), (300, 1024)])
@pytest.mark.parametrize("ydt", [torch.float32, torch.bfloat16])
def test_sgmv_expand_small_grids(n_rows, d_out, ydt):
    """The streaming SGMV expand deals equal runs of pieces to its
    workgroups XCD by XCD; with fewer pieces than XCDs (a grid of fewer than
    8 workgroups) every piece must still be written.  Accumulating into a
    random y, against the oracle."""
    say(f"sgmv expand, small grid: {n_rows} rows -> {d_out}, y {ydt}")
    b = binding()
    w = wl.small_batch(seed=n_rows + d_out, n_rows=n_rows, d_in=128, d_out=d_out, n_adapters=2, ranks=[16, 64],
                       layout=wl.RAGGED, dtype=torch.bfloat16, device="cuda", frac_base=0.0,
                       run_lengths=[n_rows // 2, n_rows - n_rows // 2])
    p = w.projections[0]
    pool = pool_of(p.pool)
    ids = ids_dev(w)
    o = run_oracle(w, want=("t", "lora"))
    t = torch.as_tensor(o["t"], dtype=torch.float32, device=DEV)
    y0 = torch.randn(w.n_rows, p.d_out, device=DEV).to(ydt)
    seg = b.lora_segments_build(ids, p.pool.n_adapters)
    y = b.lora_sgmv_expand(pool, t, seg, y=y0.clone(), y_dtype=ydt, accumulate=True)
    torch.cuda.synchronize()
    assert_close(y, o["lora"] + f64(y0), TOL[torch.bfloat16], f"y ({n_rows} x {d_out}, {ydt})")


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("mode", ["bgmv", "sgmv"])
@pytest.mark.parametrize("ydt", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("accumulate", [False, True])
def test_expand(name, mode, ydt, accumulate):
    say(f"expand {mode}: {name} y={ydt} accumulate={accumulate}")
    b = binding()
    w, o = _oracle(name)
    p = w.projections[0]
    if ydt == torch.bfloat16 and p.d_out % 8:
        pytest.skip("bf16 y rows need 16-byte aligned leading dimension")
    pool = pool_of(p.pool)
    ids = ids_dev(w)
    t = torch.as_tensor(o["t"], dtype=torch.float32, device=DEV)
    y0 = torch.randn(w.n_rows, p.d_out, device=DEV).to(ydt) if accumulate else None
    y = y0.clone() if accumulate else None
    if mode == "bgmv":
        y = b.lora_bgmv_expand(pool, t, ids, y=y, y_dtype=ydt, accumulate=accumulate)
    else:
        seg = b.lora_segments_build(ids, p.pool.n_adapters)
        y = b.lora_sgmv_expand(pool, t, seg, y=y, y_dtype=ydt, accumulate=accumulate)
    torch.cuda.synchronize()
    ref = o["lora"] + (f64(y0) if accumulate else 0.0)
    assert_close(y, ref, TOL[torch.bfloat16 if ydt == torch.bfloat16 else w.dtype], f"expand {mode}")
    if accumulate:
        base = w.ids == -1
        assert torch.equal(y[torch.as_tensor(base, device=DEV)], y0[torch.as_tensor(base, device=DEV)])


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("mode", ["bgmv", "sgmv"])
@pytest.mark.parametrize("wl_layout", ["in_out", "out_in"])
def test_layer(name, mode, wl_layout):
    say(f"layer {mode} W {wl_layout}: {name}")
    b = binding()
    w, o = _oracle(name)
    p = w.projections[0]
    pool = pool_of(p.pool)
    lay = b.LORA_W_IN_OUT if wl_layout == "in_out" else b.LORA_W_OUT_IN
    m = b.LORA_MODE_BGMV if mode == "bgmv" else b.LORA_MODE_SGMV
    y = b.lora_layer_apply(pool, p.x, w_stored(p.W, lay), ids_dev(w), w_layout=lay, mode=m,
                           y_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_close(y, o["y"], TOL[w.dtype], f"y ({mode}, {name})")
    if p.d_out % 8 == 0:
        yb = b.lora_layer_apply(pool, p.x, w_stored(p.W, lay), ids_dev(w), w_layout=lay, mode=m,
                                y_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert_close(yb, o["y"], TOL[torch.bfloat16], f"y bf16 ({mode}, {name})")


# ---------------------------------------------------------------------------
# The page's tiny batch and the walk-through
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mode", ["bgmv", "sgmv"])
def test_tiny_batch_layer(mode):
    say(f"tiny batch (page script, fp32) layer {mode}")
    b = binding()
    w = wl.tiny_mixed_batch(DEV)
    o = run_oracle(w)
    p = w.projections[0]
    pool = pool_of(p.pool)
    m = b.LORA_MODE_BGMV if mode == "bgmv" else b.LORA_MODE_SGMV
    for lay in (b.LORA_W_IN_OUT, b.LORA_W_OUT_IN):
        y = b.lora_layer_apply(pool, p.x, w_stored(p.W, lay), ids_dev(w), w_layout=lay, mode=m)
        torch.cuda.synchronize()
        assert_close(y, o["y"], 1e-4, f"tiny y {mode} layout {lay}")
        d = float(np.abs(y.cpu().double().numpy() - o["y"]).max())
        say(f"  page bound atol 1e-5: max |gpu - oracle| = {d:.2e} ({'met' if d <= 1e-5 else 'not met'})")
    t = b.lora_bgmv_shrink(pool, p.x, ids_dev(w)) if mode == "bgmv" else \
        b.lora_sgmv_shrink(pool, p.x, b.lora_segments_build(ids_dev(w), 8))
    torch.cuda.synchronize()
    assert_close(t, o["t"], 1e-4, "tiny t")


def test_walkthrough_shared_adapter():
    say("walk-through T1,T2,T1,T3 with row 2 = row 0")
    b = binding()
    w = wl.walkthrough_batch(DEV, repeat_row0=True)
    o = run_oracle(w)
    p = w.projections[0]
    pool = pool_of(p.pool)
    for m in (b.LORA_MODE_BGMV, b.LORA_MODE_SGMV):
        y = b.lora_layer_apply(pool, p.x, p.W, ids_dev(w), w_layout=b.LORA_W_IN_OUT, mode=m)
        torch.cuda.synchronize()
        assert_close(y, o["y"], 1e-4, f"walk-through mode {m}")
        assert torch.equal(y[0], y[2]), "rows sharing T1 with equal inputs differ"


# ---------------------------------------------------------------------------
# Properties
# ---------------------------------------------------------------------------

def test_permutation_and_determinism():
    say("properties: permutation equivariance, BGMV == SGMV, determinism")
    b = binding()
    w, o = _oracle("bf16_ragged")
    p = w.projections[0]
    pool = pool_of(p.pool)
    ids = ids_dev(w)
    Wt = w_stored(p.W, b.LORA_W_OUT_IN)
    ys = {}
    for m in (b.LORA_MODE_BGMV, b.LORA_MODE_SGMV):
        y1 = b.lora_layer_apply(pool, p.x, Wt, ids, w_layout=b.LORA_W_OUT_IN, mode=m, y_dtype=torch.float32)
        y2 = b.lora_layer_apply(pool, p.x, Wt, ids, w_layout=b.LORA_W_OUT_IN, mode=m, y_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(y1, y2), f"mode {m} not run-to-run identical"
        ys[m] = y1
        pi = torch.as_tensor(np.random.default_rng(5).permutation(w.n_rows), device=DEV)
        yp = b.lora_layer_apply(pool, p.x[pi].contiguous(), Wt, ids[pi].contiguous(), w_layout=b.LORA_W_OUT_IN,
                                mode=m, y_dtype=torch.float32)
        torch.cuda.synchronize()
        assert_close(yp, ys[m][pi].cpu().double().numpy(), TOL[w.dtype], f"permuted mode {m}")
        say(f"  mode {m}: permuted output bit-identical: {torch.equal(yp, ys[m][pi])}")
    assert_close(ys[b.LORA_MODE_BGMV], ys[b.LORA_MODE_SGMV].cpu().double().numpy(), TOL[w.dtype], "BGMV vs SGMV")


def test_layer_with_prebuilt_segments():
    """A segments descriptor built once for the batch and handed to the layer
    gives the same bits as the layer building its own."""
    say("layer with a prebuilt segments descriptor")
    b = binding()
    for name in ("bf16_ragged", "bf16_r64_prefill", "f32_uniform"):
        w, o = _oracle(name)
        p = w.projections[0]
        pool = pool_of(p.pool)
        ids = ids_dev(w)
        seg = b.lora_segments_build(ids, p.pool.n_adapters)
        for lay in (b.LORA_W_OUT_IN, b.LORA_W_IN_OUT):
            Ws = w_stored(p.W, lay)
            y0 = b.lora_layer_apply(pool, p.x, Ws, ids, w_layout=lay, mode=b.LORA_MODE_SGMV, y_dtype=torch.float32)
            y1 = b.lora_layer_apply(pool, p.x, Ws, ids, w_layout=lay, seg=seg, mode=b.LORA_MODE_SGMV,
                                    y_dtype=torch.float32)
            torch.cuda.synchronize()
            assert torch.equal(y0, y1), f"{name} layout {lay}: prebuilt segments change the result"
            assert_close(y1, o["y"], TOL[w.dtype], f"{name} layout {lay}")


def test_base_only_rows_and_all_base():
    say("properties: base-only rows equal the all-base product")
    b = binding()
    w, o = _oracle("bf16_uniform")
    p = w.projections[0]
    pool = pool_of(p.pool)
    ids = ids_dev(w)
    y = b.lora_layer_apply(pool, p.x, p.W, ids, w_layout=b.LORA_W_IN_OUT, y_dtype=torch.float32)
    allbase = torch.full_like(ids, -1)
    y0 = b.lora_layer_apply(pool, p.x, p.W, allbase, w_layout=b.LORA_W_IN_OUT, y_dtype=torch.float32)
    torch.cuda.synchronize()
    base_ref = f64(p.x) @ f64(p.W)
    assert_close(y0, base_ref, TOL[w.dtype], "all base-only = x W")
    mask = torch.as_tensor(w.ids == -1, device=DEV)
    assert torch.equal(y[mask], y0[mask]), "base-only rows depend on other rows' adapters"
    # bf16 y in BGMV mode (200 rows: base product in fp32 partials, then the
    # expand adds the term and rounds once; base-only rows take the partials)
    yb = b.lora_layer_apply(pool, p.x, p.W, ids, w_layout=b.LORA_W_IN_OUT, mode=b.LORA_MODE_BGMV, y_dtype=torch.bfloat16)
    yb0 = b.lora_layer_apply(pool, p.x, p.W, allbase, w_layout=b.LORA_W_IN_OUT, mode=b.LORA_MODE_BGMV, y_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert_close(yb0, base_ref, TOL[torch.bfloat16], "all base-only = x W (bf16 y)")
    assert torch.equal(yb[mask], yb0[mask]), "base-only rows depend on other rows' adapters (bf16 y)"
    assert_close(yb, o["y"], TOL[torch.bfloat16], "y bf16, BGMV")
    t = b.lora_bgmv_shrink(pool, p.x, allbase)
    torch.cuda.synchronize()
    assert torch.count_nonzero(t).item() == 0


def test_out_of_range_ids_flag_and_base_only():
    say("errors: ids outside [-1, n_adapters) set the pool flag and act as base-only")
    b = binding()
    w, o = _oracle("bf16_uniform")
    p = w.projections[0]
    pool = pool_of(p.pool)
    bad = w.ids.copy()
    bad[[3, 50, 100]] = [12, -4, 1 << 20]
    ids = torch.as_tensor(bad, device=DEV)
    assert b.lora_pool_last_error(pool) == 0
    for m in (b.LORA_MODE_BGMV, b.LORA_MODE_SGMV):
        y = b.lora_layer_apply(pool, p.x, p.W, ids, w_layout=b.LORA_W_IN_OUT, mode=m, y_dtype=torch.float32)
        assert b.lora_pool_last_error(pool) & 1 == 1
        assert b.lora_pool_last_error(pool) == 0
        base_ref = f64(p.x[[3, 50, 100]]) @ f64(p.W)
        assert_close(y[[3, 50, 100]], base_ref, TOL[w.dtype], f"invalid rows base-only mode {m}")
    # bf16 y in BGMV mode: the expand that adds the fp32 base partials flags too
    y = b.lora_layer_apply(pool, p.x, p.W, ids, w_layout=b.LORA_W_IN_OUT, mode=b.LORA_MODE_BGMV, y_dtype=torch.bfloat16)
    assert b.lora_pool_last_error(pool) & 1 == 1
    assert b.lora_pool_last_error(pool) == 0
    assert_close(y[[3, 50, 100]], f64(p.x[[3, 50, 100]]) @ f64(p.W), TOL[torch.bfloat16], "invalid rows, bf16 y")


def test_empty_and_single_row():
    say("edges: zero rows, one row, one adapter for every row")
    b = binding()
    w, o = _oracle("bf16_uniform")
    p = w.projections[0]
    pool = pool_of(p.pool)
    ids0 = torch.zeros(0, dtype=torch.int32, device=DEV)
    y0 = b.lora_layer_apply(pool, p.x[:0], p.W, ids0, w_layout=b.LORA_W_IN_OUT)
    seg0 = b.lora_segments_build(ids0, p.pool.n_adapters)
    torch.cuda.synchronize()
    assert y0.shape[0] == 0 and int(seg0.n_seg.item()) == 0
    for r in (0, 7):
        y1 = b.lora_layer_apply(pool, p.x[r:r + 1], p.W, ids_dev(w)[r:r + 1], w_layout=b.LORA_W_IN_OUT, y_dtype=torch.float32)
        torch.cuda.synchronize()
        assert_close(y1, o["y"][r:r + 1], TOL[w.dtype], f"single row {r}")
    one = torch.full_like(ids_dev(w), 4)
    ref = run_oracle(wl.Workload("one", w.dtype, np.full(w.n_rows, 4, np.int32), w.projections))
    for m in (b.LORA_MODE_BGMV, b.LORA_MODE_SGMV):
        y = b.lora_layer_apply(pool, p.x, p.W, one, w_layout=b.LORA_W_IN_OUT, mode=m, y_dtype=torch.float32)
        torch.cuda.synchronize()
        assert_close(y, ref["y"], TOL[w.dtype], f"single adapter mode {m}")


def test_workspace_reuse_and_clear():
    say("workspace: repeated calls on one workspace, explicit clear")
    b = binding()
    w, o = _oracle("bf16_uniform")
    p = w.projections[0]
    pool = pool_of(p.pool)
    ids = ids_dev(w)
    n = b.lora_layer_workspace(pool, w.n_rows, b.LORA_MODE_BGMV)
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)
    b.lora_workspace_clear(ws)
    outs = [b.lora_layer_apply(pool, p.x, p.W, ids, w_layout=b.LORA_W_IN_OUT, mode=b.LORA_MODE_BGMV, ws=ws, y_dtype=torch.float32)
            for _ in range(3)]
    torch.cuda.synchronize()
    for y in outs[1:]:
        assert torch.equal(y, outs[0])
    assert_close(outs[0], o["y"], TOL[w.dtype], "layer with reused workspace")


# ---------------------------------------------------------------------------
# The five workloads at full size
# ---------------------------------------------------------------------------

def test_decode_q_proj_full():
    say("decode q_proj 4096->4096, r16, pool 250, 32 rows: full parity")
    b = binding()
    w = wl.decode_q_proj(device=DEV)
    p = w.projections[0]
    o = run_oracle(w)
    pool = pool_of(p.pool)
    ids = ids_dev(w)
    t = b.lora_bgmv_shrink(pool, p.x, ids)
    torch.cuda.synchronize()
    assert_close(t, o["t"], TOL[w.dtype], "t bgmv")
    for lay in (b.LORA_W_OUT_IN, b.LORA_W_IN_OUT):
        Ws = w_stored(p.W, lay)
        for m in (b.LORA_MODE_BGMV, b.LORA_MODE_SGMV):
            y = b.lora_layer_apply(pool, p.x, Ws, ids, w_layout=lay, mode=m)
            torch.cuda.synchronize()
            assert_close(y, o["y"], TOL[w.dtype], f"y layout {lay} mode {m}")


def _sample_rows(w, k, rng):
    n = w.n_rows
    rows = set(rng.choice(n, min(k, n), replace=False).tolist())
    rows |= {0, n - 1}
    if w.lengths:
        off = np.cumsum([0] + list(w.lengths))
        for o in off[1:-1]:
            rows |= {int(o) - 1, int(o)}
    return sorted(rows)


@pytest.mark.parametrize("proj", [p[0] for p in wl.PROJ_8B])
def test_skewed_decode_8b(proj):
    """All 256 rows of the skewed batch (110 adapters) against the oracle on
    sampled columns (rows and columns are independent, so the sampled values
    are exact), in BGMV mode (the few-hundred-row path: shrink and finish per
    segment tile, split-K base product) and SGMV mode; t on every row."""
    say(f"skewed decode 8B {proj}: y on all rows x sampled columns, t on all rows")
    b = binding()
    w = wl.skewed_decode_8b(device=DEV, projections=[proj])
    p = w.projections[0]
    pool = pool_of(p.pool)
    ids = ids_dev(w)
    ot = run_oracle(w, want=("t",))
    rng = np.random.default_rng(2)
    cols = sorted(set(rng.choice(p.d_out, 256, replace=False).tolist()) | {0, p.d_out - 1})
    oy = run_oracle(w, cols=cols, want=("y",), threads=0)
    Ws = w_stored(p.W, b.LORA_W_OUT_IN)
    ys = {}
    for m in (b.LORA_MODE_BGMV, b.LORA_MODE_SGMV):
        y = b.lora_layer_apply(pool, p.x, Ws, ids, w_layout=b.LORA_W_OUT_IN, mode=m)
        torch.cuda.synchronize()
        assert_close(y[:, cols], oy["y"], TOL[w.dtype], f"y mode {m}, all rows")
        ys[m] = y
    seg = b.lora_segments_build(ids, p.pool.n_adapters)
    y2 = b.lora_layer_apply(pool, p.x, Ws, ids, w_layout=b.LORA_W_OUT_IN, mode=b.LORA_MODE_BGMV, seg=seg)
    torch.cuda.synchronize()
    assert torch.equal(y2, ys[b.LORA_MODE_BGMV]), "caller's segments give other bits"
    t = b.lora_bgmv_shrink(pool, p.x, ids)
    torch.cuda.synchronize()
    assert_close(t, ot["t"], TOL[w.dtype], "t bgmv")
    t = b.lora_sgmv_shrink(pool, p.x, seg)
    torch.cuda.synchronize()
    assert_close(t, ot["t"], TOL[w.dtype], "t sgmv")


# Batches of a few hundred rows in BGMV mode (W stored [d_out, d_in], bf16
# pool): segment-tile shrink and finish around a split-K base product.
ROWS_CASES = [
    # n_rows, d_in, d_out, layout, ranks, n_adapters, id pattern
    (65, 512, 384, wl.UNIFORM, 16, 40, "zipf"),
    (128, 1000, 776, wl.RAGGED, RAGGED_RANKS, 12, "uniform"),
    (257, 2056, 328, wl.UNIFORM, 64, 9, "runs"),
    (300, 1024, 8200, wl.RAGGED, RAGGED_RANKS, 12, "zipf"),       # 256 x 128 tiles, 2 row tiles
    (1024, 8264, 264, wl.UNIFORM, 8, 600, "zipf"),                # long, ragged K: 256 x 128 tiles, split K
    (200, 768, 520, wl.UNIFORM, 16, 150, "allbase"),
    (200, 768, 520, wl.UNIFORM, 16, 150, "one"),
    (200, 768, 520, wl.UNIFORM, 16, 150, "distinct"),
]


def _rows_ids(pattern, n, n_ad, rng):
    if pattern == "zipf":
        k = np.arange(1, n_ad + 1)
        p = k ** -1.1
        ids = rng.choice(n_ad, n, p=p / p.sum())
    elif pattern == "runs":
        ids = np.repeat(rng.integers(0, n_ad, 20), -(-n // 20))[:n]
    elif pattern == "allbase":
        ids = np.full(n, -1)
    elif pattern == "one":
        ids = np.full(n, n_ad // 2)
    elif pattern == "distinct":
        ids = rng.permutation(n_ad)[:n] if n <= n_ad else rng.integers(0, n_ad, n)
    else:
        ids = rng.integers(0, n_ad, n)
    if pattern not in ("allbase", "one"):
        ids = np.where(rng.random(n) < 0.08, -1, ids)
    return ids.astype(np.int32)


@pytest.mark.parametrize("case", ROWS_CASES, ids=[f"{c[0]}x{c[1]}x{c[2]}-{c[6]}" for c in ROWS_CASES])
def test_rows_path(case):
    n, d_in, d_out, layout, ranks, n_ad, pattern = case
    say(f"few-hundred-row path: {n} x {d_in} -> {d_out}, {pattern}")
    b = binding()
    rng = np.random.default_rng(n + d_out)
    w = wl.small_batch(seed=n, n_rows=n, device=DEV, dtype=torch.bfloat16, d_in=d_in, d_out=d_out,
                       n_adapters=n_ad, layout=layout, ranks=ranks, frac_base=0.0,
                       scale=np.linspace(-2.0, 2.0, n_ad).astype(np.float32))
    w = wl.Workload(w.name, w.dtype, _rows_ids(pattern, n, n_ad, rng), w.projections)
    p = w.projections[0]
    pool = pool_of(p.pool)
    ids = ids_dev(w)
    cols = None if d_out <= 1024 else sorted(set(rng.choice(d_out, 300, replace=False).tolist()) | {0, d_out - 1})
    o = run_oracle(w, cols=cols, threads=0)
    Ws = w_stored(p.W, b.LORA_W_OUT_IN)
    for ydt in (torch.bfloat16, torch.float32):
        y = b.lora_layer_apply(pool, p.x, Ws, ids, w_layout=b.LORA_W_OUT_IN, mode=b.LORA_MODE_BGMV, y_dtype=ydt)
        torch.cuda.synchronize()
        ys = y if cols is None else y[:, cols]
        assert_close(ys, o["y"], TOL[torch.bfloat16], f"y {ydt}")
    y2 = b.lora_layer_apply(pool, p.x, Ws, ids, w_layout=b.LORA_W_OUT_IN, mode=b.LORA_MODE_BGMV,
                            y_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y, y2), "run-to-run bits"


# The fused layer's 128x128 launches with few tiles and a long K run split K
# (fp32 partial sums, then a finish that adds them and s t B_a): all rows of
# a 1,536-row batch (1,024 x 2,048 -> 1,024 columns, two slices), and the 170
# rows past the 256x256 rounds of a 2,218-row batch (8,192 columns, two slices),
# in SGMV (rows visited grouped by adapter) and BGMV order, against the oracle.
SPLIT_CASES = [
    # n_rows, d_in, d_out, rows checked: "all" or "tail" (past the 256x256 rounds)
    (1536, 2048, 1024, "all"),
    (2218, 2048, 8192, "tail"),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[f"{c[0]}x{c[1]}x{c[2]}-{c[3]}" for c in SPLIT_CASES])
def test_layer_split_k_launches(case):
    n, d_in, d_out, which = case
    say(f"split-K layer launches: {n} x {d_in} -> {d_out}, rows {which}")
    b = binding()
    rng = np.random.default_rng(n + d_out)
    n_ad = 12
    w = wl.small_batch(seed=n, n_rows=n, device=DEV, dtype=torch.bfloat16, d_in=d_in, d_out=d_out,
                       n_adapters=n_ad, layout=wl.RAGGED, ranks=RAGGED_RANKS, frac_base=0.0,
                       scale=np.linspace(-2.0, 2.0, n_ad).astype(np.float32))
    w = wl.Workload(w.name, w.dtype, _rows_ids("runs", n, n_ad, rng), w.projections)
    p = w.projections[0]
    pool = pool_of(p.pool)
    ids = ids_dev(w)
    Ws = w_stored(p.W, b.LORA_W_OUT_IN)
    seg = b.lora_segments_build(ids, n_ad)
    torch.cuda.synchronize()
    if which == "all":
        rows = np.arange(n)
        cols = None
    else:
        # rows in the order each mode visits them: SGMV by segments, BGMV as given
        perm = seg.perm[:n].cpu().numpy()
        tail_sgmv = perm[2048:]
        tail_bgmv = np.arange(2048, n)
        rows = np.unique(np.concatenate([tail_sgmv, tail_bgmv, rng.choice(2048, 16, replace=False)]))
        cols = sorted(set(rng.choice(d_out, 160, replace=False).tolist()) | {0, d_out - 1})
    o = run_oracle(w, rows=rows.tolist(), cols=cols, threads=0)
    for mode in (b.LORA_MODE_SGMV, b.LORA_MODE_BGMV):
        for ydt in (torch.bfloat16, torch.float32):
            y = b.lora_layer_apply(pool, p.x, Ws, ids, w_layout=b.LORA_W_OUT_IN, mode=mode, y_dtype=ydt,
                                   seg=seg if mode == b.LORA_MODE_SGMV else None)
            torch.cuda.synchronize()
            ys = y[torch.as_tensor(rows, device=y.device)]
            if cols is not None:
                ys = ys[:, cols]
            assert_close(ys, o["y"], TOL[torch.bfloat16], f"y mode {mode} {ydt}")


def test_rows_path_invalid_ids():
    say("few-hundred-row path: invalid ids flagged and run as base-only rows")
    b = binding()
    w = wl.small_batch(seed=11, n_rows=150, device=DEV, dtype=torch.bfloat16, d_in=512, d_out=640,
                       n_adapters=70, ranks=16, frac_base=0.1)
    p = w.projections[0]
    pool = pool_of(p.pool)
    bad = w.ids.copy()
    bad[[3, 77, 149]] = [70, -2, 1000]
    ids = torch.as_tensor(bad, device=DEV)
    y = b.lora_layer_apply(pool, p.x, w_stored(p.W, b.LORA_W_OUT_IN), ids, w_layout=b.LORA_W_OUT_IN,
                           mode=b.LORA_MODE_BGMV)
    assert b.lora_pool_last_error(pool) & 1 == 1
    o = run_oracle(wl.Workload("bad", w.dtype, bad, w.projections))
    assert o["bad"] == 3
    assert_close(y, o["y"], TOL[torch.bfloat16], "y with invalid ids")


@pytest.mark.parametrize("proj", [p[0] for p in wl.PROJ_70B])
def test_prefill_70b(proj):
    say(f"prefill 70B {proj} r64: sampled rows x columns, both W layouts")
    b = binding()
    w = wl.prefill_70b(device=DEV, projections=[proj])
    p = w.projections[0]
    pool = pool_of(p.pool)
    ids = ids_dev(w)
    rng = np.random.default_rng(3)
    rows = _sample_rows(w, 40, rng)
    cols = sorted(set(rng.choice(p.d_out, 192, replace=False).tolist()) | {0, p.d_out - 1})
    o = run_oracle(w, rows=rows, cols=cols, threads=0)
    y = b.lora_layer_apply(pool, p.x, w_stored(p.W, b.LORA_W_OUT_IN), ids, w_layout=b.LORA_W_OUT_IN,
                           mode=b.LORA_MODE_SGMV)
    torch.cuda.synchronize()
    ys = y[rows][:, cols]
    assert_close(ys, o["y"], TOL[w.dtype], "y sampled")
    # W stored [d_in, d_out]: other loaders, the same products in the same
    # order, so the same bits on every row and column
    yi = b.lora_layer_apply(pool, p.x, w_stored(p.W, b.LORA_W_IN_OUT), ids, w_layout=b.LORA_W_IN_OUT,
                            mode=b.LORA_MODE_SGMV)
    torch.cuda.synchronize()
    assert torch.equal(yi, y), "W layouts differ"
    seg = b.lora_segments_build(ids, p.pool.n_adapters)
    t = b.lora_sgmv_shrink(pool, p.x, seg)
    torch.cuda.synchronize()
    assert_close(t[rows], o["t"], TOL[w.dtype], "t sampled")


@pytest.mark.parametrize("proj", [p[0] for p in wl.PROJ_70B])
def test_mixed_rank_70b(proj):
    say(f"mixed-rank 70B {proj}: ragged vs padded, sampled vs oracle")
    b = binding()
    w = wl.mixed_rank_70b(device=DEV, projections=[proj])
    p = w.projections[0]
    ids = ids_dev(w)
    Ws = w_stored(p.W, b.LORA_W_OUT_IN)
    pr = pool_of(p.pool)
    pp = pool_of(p.pool_padded)
    yr = b.lora_layer_apply(pr, p.x, Ws, ids, w_layout=b.LORA_W_OUT_IN, y_dtype=torch.float32)
    yp = b.lora_layer_apply(pp, p.x, Ws, ids, w_layout=b.LORA_W_OUT_IN, y_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_close(yr, yp.double().cpu().numpy(), 1e-4, "ragged vs padded (fp32 y)")
    rng = np.random.default_rng(4)
    rows = _sample_rows(w, 48, rng)
    cols = sorted(set(rng.choice(p.d_out, 160, replace=False).tolist()) | {0, p.d_out - 1})
    o = run_oracle(w, rows=rows, cols=cols)
    assert_close(yr[rows][:, cols], o["y"], TOL[w.dtype], "ragged y sampled")
    op = run_oracle(w, rows=rows, cols=cols, padded=True)
    assert np.array_equal(op["y"], o["y"]), "oracle: padded differs from ragged"


# ---------------------------------------------------------------------------
# Decode layer in two launches (bf16, <= 64 rows, W stored [d_out, d_in])
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n_rows", [1, 7, 16, 17, 32, 33, 64])
@pytest.mark.parametrize("layout", ["uniform", "ragged"])
def test_decode_two_launch(n_rows, layout):
    say(f"decode two-launch path: {n_rows} rows, {layout} pool")
    b = binding()
    kw = dict(dtype=torch.bfloat16, d_in=1000, d_out=776, n_adapters=12)
    if layout == "uniform":
        kw.update(layout=wl.UNIFORM, ranks=16)
    else:
        kw.update(layout=wl.RAGGED, ranks=RAGGED_RANKS)
    w = wl.small_batch(seed=n_rows, n_rows=n_rows, device=DEV, frac_base=0.15,
                       scale=np.linspace(-2.0, 2.0, 12).astype(np.float32), **kw)
    p = w.projections[0]
    o = run_oracle(w)
    pool = pool_of(p.pool)
    ids = ids_dev(w)
    Wt = w_stored(p.W, b.LORA_W_OUT_IN)
    for ydt in (torch.float32, torch.bfloat16):
        y = b.lora_layer_apply(pool, p.x, Wt, ids, w_layout=b.LORA_W_OUT_IN, mode=b.LORA_MODE_BGMV, y_dtype=ydt)
        torch.cuda.synchronize()
        assert_close(y, o["y"], TOL[torch.bfloat16], f"decode layer y={ydt}")
    # the exported phases give the same bits as the layer call
    ws = torch.empty(b.lora_decode_workspace(pool, n_rows, True), dtype=torch.uint8, device=DEV)
    b.lora_decode_stream(pool, p.x, Wt, ids, ws, True)
    y2 = b.lora_decode_finish(pool, ids, ws, torch.empty_like(y), True)
    torch.cuda.synchronize()
    assert torch.equal(y2, y)
    # base-only form: y = x W
    wsb = torch.empty(b.lora_decode_workspace(pool, n_rows, False), dtype=torch.uint8, device=DEV)
    b.lora_decode_stream(pool, p.x, Wt, ids, wsb, False)
    yb = b.lora_decode_finish(pool, ids, wsb, torch.empty(n_rows, p.d_out, device=DEV), False)
    torch.cuda.synchronize()
    assert_close(yb, f64(p.x) @ f64(p.W), TOL[torch.bfloat16], "decode base-only")


@pytest.mark.parametrize("n_rows", [1, 16, 33, 64])
@pytest.mark.parametrize("ranks", ["pow2", "odd"])
def test_decode_whole_slices(n_rows, ranks):
    """d_in 4096 splits into whole 512-row quarters (the branch-free stream
    form: 2 or 4 quarters per slice); d_out 4104 leaves a ragged last column
    tile; odd ranks take the any-rank shrink."""
    say(f"decode two-launch path, whole K slices: {n_rows} rows, {ranks} ranks")
    b = binding()
    rk = [8, 16, 32, 64, 16, 8] if ranks == "pow2" else [3, 16, 40, 64, 12, 1]
    w = wl.small_batch(seed=100 + n_rows, n_rows=n_rows, device=DEV, dtype=torch.bfloat16, d_in=4096,
                       d_out=4104, n_adapters=6, layout=wl.RAGGED, ranks=rk, frac_base=0.1)
    p = w.projections[0]
    o = run_oracle(w)
    pool = pool_of(p.pool)
    ids = ids_dev(w)
    Wt = w_stored(p.W, b.LORA_W_OUT_IN)
    for ydt in (torch.float32, torch.bfloat16):
        y = b.lora_layer_apply(pool, p.x, Wt, ids, w_layout=b.LORA_W_OUT_IN, mode=b.LORA_MODE_BGMV, y_dtype=ydt)
        torch.cuda.synchronize()
        assert_close(y, o["y"], TOL[torch.bfloat16], f"decode layer y={ydt}")


@pytest.mark.parametrize("n_rows,d_in,d_out", [(4, 256, 264), (20, 512, 1024), (9, 2056, 328)])
def test_decode_small_shapes(n_rows, d_in, d_out):
    """Shapes whose plan cuts the stream into one-quarter slices (8 column
    blocks per workgroup) with ragged K and column tails."""
    say(f"decode two-launch path, small shape: {n_rows} rows, {d_in} -> {d_out}")
    b = binding()
    w = wl.small_batch(seed=200 + n_rows, n_rows=n_rows, device=DEV, dtype=torch.bfloat16, d_in=d_in,
                       d_out=d_out, n_adapters=5, ranks=[16, 8, 64, 32, 16], layout=wl.RAGGED, frac_base=0.2)
    p = w.projections[0]
    o = run_oracle(w)
    pool = pool_of(p.pool)
    ids = ids_dev(w)
    Wt = w_stored(p.W, b.LORA_W_OUT_IN)
    y = b.lora_layer_apply(pool, p.x, Wt, ids, w_layout=b.LORA_W_OUT_IN, mode=b.LORA_MODE_BGMV,
                           y_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_close(y, o["y"], TOL[torch.bfloat16], "decode layer")


@pytest.mark.parametrize("d_in", [2104, 3104])
def test_sgmv_layer_split_k_shrink(d_in):
    """SGMV layer with d_in >= 2048 and few row tiles: the shrink runs in K
    slices (the last one ragged) whose partial sums a reduce pass adds."""
    say(f"SGMV layer, split-K shrink: d_in {d_in}")
    b = binding()
    w = wl.small_batch(seed=d_in, device=DEV, dtype=torch.bfloat16, d_in=d_in, d_out=272, n_adapters=7,
                       layout=wl.RAGGED, ranks=[3, 16, 64, 8, 40, 1, 32], frac_base=0.1,
                       run_lengths=[1, 37, 64, 5, 1, 90, 2, 17])
    p = w.projections[0]
    o = run_oracle(w)
    pool = pool_of(p.pool)
    ids = ids_dev(w)
    for lay in (b.LORA_W_OUT_IN, b.LORA_W_IN_OUT):
        y = b.lora_layer_apply(pool, p.x, w_stored(p.W, lay), ids, w_layout=lay, mode=b.LORA_MODE_SGMV,
                               y_dtype=torch.float32)
        torch.cuda.synchronize()
        assert_close(y, o["y"], TOL[torch.bfloat16], f"y layout {lay}")


@pytest.mark.parametrize("d_in,d_out,layout,runs", [
    (136, 200, wl.RAGGED, None),        # K shorter than one 256-deep block
    (776, 1032, wl.RAGGED, None),       # whole blocks plus a ragged K tail
    (1000, 776, wl.UNIFORM, [1, 2, 1, 40, 3, 1, 1, 90, 1, 2, 5, 1, 60, 1, 1, 91]),
])
def test_layer_many_adapters_per_tile(d_in, d_out, layout, runs):
    """Row tiles that hold many different adapters add the LoRA term row by
    row after the K loop; tiles of one or two long runs in the same launch
    keep the K-extension.  Both W layouts, both modes, fp32 and bf16 y."""
    say(f"layer, many adapters per tile: d_in {d_in} d_out {d_out} runs {runs is not None}")
    b = binding()
    ranks = (RAGGED_RANKS * 4)[:40] if layout == wl.RAGGED else 16
    w = wl.small_batch(seed=d_in + d_out, n_rows=257, device=DEV, dtype=torch.bfloat16, d_in=d_in,
                       d_out=d_out, n_adapters=40, layout=layout, ranks=ranks, frac_base=0.1,
                       run_lengths=runs, scale=np.linspace(-2.0, 2.0, 40).astype(np.float32))
    p = w.projections[0]
    o = run_oracle(w)
    pool = pool_of(p.pool)
    ids = ids_dev(w)
    for lay in (b.LORA_W_OUT_IN, b.LORA_W_IN_OUT):
        for m in (b.LORA_MODE_BGMV, b.LORA_MODE_SGMV, b.LORA_MODE_AUTO):
            for ydt in (torch.float32, torch.bfloat16):
                y = b.lora_layer_apply(pool, p.x, w_stored(p.W, lay), ids, w_layout=lay, mode=m, y_dtype=ydt)
                torch.cuda.synchronize()
                assert_close(y, o["y"], TOL[torch.bfloat16], f"y layout {lay} mode {m} {ydt}")


def test_bgmv_split_form_medium_batch():
    """600 rows x 512 -> 2560 in BGMV mode.  W stored [d_out, d_in] takes the
    few-hundred-row path (base product in fp32 partials, added with the
    expand by the finish, one rounding); W stored [d_in, d_out] the fused
    GEMM.  Both y dtypes, every row against the oracle, and bf16 y within
    one bf16 rounding of fp32 y."""
    say("layer, BGMV 600 x 512 -> 2560: few-hundred-row path and fused GEMM, both W layouts")
    b = binding()
    w = wl.small_batch(seed=600, n_rows=600, device=DEV, dtype=torch.bfloat16, d_in=512, d_out=2560,
                       n_adapters=40, layout=wl.RAGGED, ranks=(RAGGED_RANKS * 4)[:40], frac_base=0.1,
                       scale=np.linspace(-2.0, 2.0, 40).astype(np.float32))
    p = w.projections[0]
    o = run_oracle(w)
    pool = pool_of(p.pool)
    ids = ids_dev(w)
    for lay in (b.LORA_W_OUT_IN, b.LORA_W_IN_OUT):
        yb = b.lora_layer_apply(pool, p.x, w_stored(p.W, lay), ids, w_layout=lay, mode=b.LORA_MODE_BGMV,
                                y_dtype=torch.bfloat16)
        yf = b.lora_layer_apply(pool, p.x, w_stored(p.W, lay), ids, w_layout=lay, mode=b.LORA_MODE_BGMV,
                                y_dtype=torch.float32)
        torch.cuda.synchronize()
        assert_close(yb, o["y"], TOL[torch.bfloat16], f"y bf16, layout {lay}")
        assert_close(yf, o["y"], TOL[torch.bfloat16], f"y fp32, layout {lay}")
        assert_close(yb, f64(yf), TOL[torch.bfloat16], f"bf16 vs fp32 y, layout {lay}")


def test_layer_tail_rows_split_launch():
    """520 rows x 22,016 columns: 258 tiles of 256x256 would leave a last
    round of two; rows [0, 512) take the 256x256 launch and rows [512, 520)
    a launch of 128x128 tiles.  Every row checked, both W layouts and modes."""
    say("layer, 256x256 launch plus a tail launch: 520 x 136 -> 22016")
    b = binding()
    w = wl.small_batch(seed=520, n_rows=520, device=DEV, dtype=torch.bfloat16, d_in=136, d_out=22016,
                       n_adapters=12, layout=wl.RAGGED, ranks=RAGGED_RANKS, frac_base=0.1,
                       run_lengths=[1, 3, 200, 5, 1, 290, 2, 7, 1, 10])
    p = w.projections[0]
    o = run_oracle(w)
    pool = pool_of(p.pool)
    ids = ids_dev(w)
    for lay in (b.LORA_W_OUT_IN, b.LORA_W_IN_OUT):
        for m in (b.LORA_MODE_BGMV, b.LORA_MODE_SGMV):
            y = b.lora_layer_apply(pool, p.x, w_stored(p.W, lay), ids, w_layout=lay, mode=m, y_dtype=torch.float32)
            torch.cuda.synchronize()
            assert_close(y, o["y"], TOL[torch.bfloat16], f"y layout {lay} mode {m}")
        # bf16 y in BGMV mode (W [d_out, d_in]: the few-hundred-row path)
        y = b.lora_layer_apply(pool, p.x, w_stored(p.W, lay), ids, w_layout=lay, mode=b.LORA_MODE_BGMV,
                               y_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert_close(y, o["y"], TOL[torch.bfloat16], f"y bf16 layout {lay} BGMV")
    yb = b.lora_base_gemm_expand(pool, p.x, w_stored(p.W, b.LORA_W_OUT_IN), ids, None, w_layout=b.LORA_W_OUT_IN,
                                 y_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_close(yb, o["y"] - o["lora"], TOL[torch.bfloat16], "base-only y")


def test_decode_invalid_ids_and_determinism():
    say("decode two-launch path: invalid ids flagged, run-to-run identical")
    b = binding()
    w = wl.small_batch(seed=3, n_rows=40, device=DEV, dtype=torch.bfloat16, d_in=512, d_out=640,
                       n_adapters=9, ranks=32, frac_base=0.1)
    p = w.projections[0]
    pool = pool_of(p.pool)
    bad = w.ids.copy()
    bad[[1, 20]] = [9, -3]
    ids = torch.as_tensor(bad, device=DEV)
    Wt = w_stored(p.W, b.LORA_W_OUT_IN)
    y1 = b.lora_layer_apply(pool, p.x, Wt, ids, w_layout=b.LORA_W_OUT_IN, mode=b.LORA_MODE_BGMV)
    y2 = b.lora_layer_apply(pool, p.x, Wt, ids, w_layout=b.LORA_W_OUT_IN, mode=b.LORA_MODE_BGMV)
    assert b.lora_pool_last_error(pool) & 1 == 1
    assert torch.equal(y1, y2)
    w2 = wl.Workload("bad", w.dtype, bad, w.projections)
    o = run_oracle(w2)
    assert o["bad"] == 2
    assert_close(y1, o["y"], TOL[torch.bfloat16], "decode with invalid ids")


@pytest.mark.parametrize("name", ["bf16_ragged", "f32_uniform", "bf16_r64_prefill"])
@pytest.mark.parametrize("wl_layout", ["in_out", "out_in"])
def test_base_gemm_expand_entry(name, wl_layout):
    say(f"lora_base_gemm_expand with a given t: {name}, W {wl_layout}")
    b = binding()
    w, o = _oracle(name)
    p = w.projections[0]
    pool = pool_of(p.pool)
    lay = b.LORA_W_IN_OUT if wl_layout == "in_out" else b.LORA_W_OUT_IN
    t = torch.as_tensor(o["t"], dtype=torch.float32, device=DEV)
    for rows in (slice(0, w.n_rows), slice(5, 37)):   # tiled path, and <= 64 rows
        ids = ids_dev(w)[rows].contiguous()
        y = b.lora_base_gemm_expand(pool, p.x[rows].contiguous(), w_stored(p.W, lay), ids, t[rows].contiguous(),
                                    w_layout=lay, y_dtype=torch.float32)
        yb = b.lora_base_gemm_expand(pool, p.x[rows].contiguous(), w_stored(p.W, lay), ids, None,
                                     w_layout=lay, y_dtype=torch.float32)
        torch.cuda.synchronize()
        assert_close(y, o["y"][rows], TOL[w.dtype], f"y rows {rows}")
        assert_close(yb, o["y"][rows] - o["lora"][rows], TOL[w.dtype], f"base only rows {rows}")
