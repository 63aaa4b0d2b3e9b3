"""Pins of the fp64 oracle to what the pages and the mathematics fix.

Each ``pin_*`` takes the oracle's ctypes library so that
``test_oracle_mutations.py`` can run the same pins against deliberately
broken copies of the oracle and show that every planted mistake is caught.

Sources (page title -- section):
  [P1] Multi-LoRA batching and adapter paging -- Walking through a batch
  [P3] Serving multiple LoRAs: segmented matrix multiplies and adapter
       scheduling -- Self-test; Not merging the weights, computing in batches
  [P4] Serving many LoRA adapters (blog.ecitis.org) -- Low-rank structure and
       additivity; Merge or keep separate; Replay
"""
from __future__ import annotations

import json
import os

import numpy as np
import pytest
import torch

import oracle
from _marshal import f64, oracle_pool, run_oracle
from lora_bgmv_shrink_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _tiny():
    w = wl.tiny_mixed_batch()
    p = w.projections[0]
    op, _ = oracle_pool(p.pool)
    return w, p, op


def _close(a, b, rel, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    err = np.abs(a - b) / np.maximum(1.0, np.abs(b))
    assert a.shape == b.shape, what
    assert np.all(np.isfinite(a)), what
    assert err.max() <= rel, f"{what}: max scaled err {err.max():.3e} > {rel:.1e}"


# --------------------------------------------------------------------------
# Segments
# --------------------------------------------------------------------------

def pin_tiny_segments_golden(lib):
    """[P3] the page's tiny batch: 53 rows, 4 segments (hand-derived perm/offsets)."""
    g = _golden("tiny_segments.json")
    w = wl.tiny_mixed_batch()
    assert w.n_rows == g["n_rows"] == sum(g["lengths"])
    assert len(g["lengths"]) == g["per_request_calls"]
    perm, seg_ids, seg_off, bad = oracle.segments(w.ids, 8, lib=lib)
    assert bad == 0
    assert perm.tolist() == g["perm"]
    assert seg_ids.tolist() == g["seg_ids"]
    assert seg_off.tolist() == g["seg_off"]
    assert len(seg_ids) == g["n_segments"] == len(set(g["adapters"]))
    assert np.diff(seg_off).tolist() == g["seg_counts"]


def pin_walkthrough_segments_golden(lib):
    """[P1] T1,T2,T1,T3: three distinct adapters, rows 0 and 2 share T1."""
    g = _golden("walkthrough_segments.json")
    perm, seg_ids, seg_off, bad = oracle.segments(np.array(g["ids"], np.int32), 8, lib=lib)
    assert bad == 0
    assert perm.tolist() == g["perm"]
    assert seg_ids.tolist() == g["seg_ids"]
    assert seg_off.tolist() == g["seg_off"]


def pin_segments_vs_numpy_stable_sort(lib):
    """Special case that reduces to a library routine: numpy's stable argsort
    followed by run-length encoding; invalid ids are grouped with -1."""
    rng = np.random.default_rng(7)
    for trial in range(40):
        n = int(rng.integers(0, 300))
        n_ad = int(rng.integers(1, 40))
        ids = rng.integers(-1, n_ad, n).astype(np.int32)
        if trial % 5 == 0 and n:
            ids[rng.integers(0, n, 3)] = rng.choice([-7, n_ad, n_ad + 3])
        key = np.where((ids >= 0) & (ids < n_ad), ids, -1)
        ref_perm = np.argsort(key, kind="stable").astype(np.int32)
        sk = key[ref_perm]
        starts = [0] + [i for i in range(1, n) if sk[i] != sk[i - 1]] if n else []
        ref_ids = [int(sk[s]) for s in starts]
        ref_off = starts + [n] if n else [0]
        perm, seg_ids, seg_off, bad = oracle.segments(ids, n_ad, lib=lib)
        assert perm.tolist() == ref_perm.tolist()
        assert seg_ids.tolist() == ref_ids
        assert seg_off.tolist() == ref_off
        assert bad == int(np.sum((ids < -1) | (ids >= n_ad)))


# --------------------------------------------------------------------------
# The layer
# --------------------------------------------------------------------------

def _page_formulations(w, p):
    """The page's three fp32 formulations, restated: per-request products,
    per-token gathered einsums (BGMV) and sort-grouped segment products (SGMV)."""
    x, W = p.x, p.W
    A = p.pool.A.view(8, 256, 16)
    B = p.pool.B.view(8, 16, 256)
    s = 2.0
    outs, row = [], 0
    for a, n in zip(w.request_ids, w.lengths):
        xi = x[row:row + n]
        outs.append(xi @ W + s * (xi @ A[a]) @ B[a])
        row += n
    per_request = torch.cat(outs)
    tok = torch.as_tensor(w.ids.astype(np.int64))
    t = torch.einsum("ti,tir->tr", x, A[tok])
    bgmv = x @ W + s * torch.einsum("tr,tro->to", t, B[tok])
    order = torch.argsort(tok, stable=True)
    xs = x[order]
    seg_out = torch.empty(len(x), 256)
    uniq, counts = torch.unique_consecutive(tok[order], return_counts=True)
    st = 0
    for a, n in zip(uniq.tolist(), counts.tolist()):
        seg_out[st:st + n] = s * (xs[st:st + n] @ A[a]) @ B[a]
        st += n
    lora = torch.empty_like(seg_out)
    lora[order] = seg_out
    sgmv = x @ W + lora
    return per_request, bgmv, sgmv


def pin_page_script_agreement(lib):
    """[P3] the page checks BGMV and SGMV against the per-request loop with
    allclose(atol=1e-5) in fp32 on its seed-0 tensors; the fp64 oracle must
    sit within that bound of all three."""
    w, p, op = _tiny()
    o = oracle.layer(f64(p.x), f64(p.W), w.ids, op, lib=lib)
    assert o["bad"] == 0
    pr, bg, sg = _page_formulations(w, p)
    for name, v in (("per_request", pr), ("bgmv", bg), ("sgmv", sg)):
        d = np.abs(o["y"] - v.double().numpy()).max()
        assert d <= 1e-5, f"oracle vs page {name}: {d:.3e}"


def pin_merged_weights(lib):
    """[P3 Self-test; P4 Merge or keep separate] y_i = x_i (W + s A_a B_a)."""
    for layout in (wl.UNIFORM, wl.RAGGED):
        ranks = 12 if layout == wl.UNIFORM else [3, 16, 8, 1, 24, 5]
        w = wl.small_batch(seed=3, n_rows=60, d_in=40, d_out=36, n_adapters=6, ranks=ranks,
                           layout=layout, dtype=torch.float64, frac_base=0.2,
                           scale=[2.0, 0.5, -1.0, 3.0, 1.0, 0.25])
        p = w.projections[0]
        op, _ = oracle_pool(p.pool)
        o = oracle.layer(f64(p.x), f64(p.W), w.ids, op, lib=lib)
        x, W = f64(p.x), f64(p.W)
        for i, a in enumerate(w.ids.tolist()):
            if a < 0:
                Wm = W
            else:
                Wm = W + p.pool.scales[a] * f64(p.pool.a_block(a)) @ f64(p.pool.b_block(a))
            _close(o["y"][i], x[i] @ Wm, 1e-12, f"merged row {i}")


def pin_additivity_base_only(lib):
    """[P4 Low-rank structure and additivity; Replay] base-only rows are x W;
    every row's y - xW is the LoRA term; the shrink output is x A."""
    w = wl.small_batch(seed=5, n_rows=80, d_in=48, d_out=40, n_adapters=5, ranks=[4, 16, 9, 2, 7],
                       layout=wl.RAGGED, dtype=torch.float64, frac_base=0.3)
    p = w.projections[0]
    op, _ = oracle_pool(p.pool)
    o = oracle.layer(f64(p.x), f64(p.W), w.ids, op, lib=lib)
    base = f64(p.x) @ f64(p.W)
    assert (w.ids == -1).sum() >= 5
    assert o["bad"] == 0
    for i, a in enumerate(w.ids.tolist()):
        if a == -1:
            _close(o["y"][i], base[i], 1e-12, f"base-only row {i}")
            assert np.all(o["lora"][i] == 0) and np.all(o["t"][i] == 0)
        else:
            _close(o["y"][i] - base[i], o["lora"][i], 1e-12, f"lora term row {i}")
            r = int(p.pool.ranks[a])
            _close(o["t"][i, :r], f64(p.x)[i] @ f64(p.pool.a_block(a)), 1e-12, f"t row {i}")
            assert np.all(o["t"][i, r:] == 0)


def pin_einsum_gather_formulation(lib):
    """Per-token gather + einsum (numpy) on a uniform pool, including the
    LoRA term alone and the intermediate t."""
    w = wl.small_batch(seed=11, n_rows=33, d_in=24, d_out=20, n_adapters=4, ranks=8,
                       dtype=torch.float64, frac_base=0.15, scale=[1.5, -2.0, 0.75, 4.0])
    p = w.projections[0]
    op, _ = oracle_pool(p.pool)
    o = oracle.layer(f64(p.x), f64(p.W), w.ids, op, lib=lib)
    A = f64(p.pool.A).reshape(4, 24, 8)
    B = f64(p.pool.B).reshape(4, 8, 20)
    valid = w.ids >= 0
    g = np.where(valid, w.ids, 0)
    t = np.einsum("ti,tir->tr", f64(p.x), A[g]) * valid[:, None]
    lora = np.einsum("tr,tro->to", t, B[g]) * p.pool.scales[g][:, None]
    _close(o["t"], t, 1e-12, "t")
    _close(o["lora"], lora, 1e-12, "lora")
    _close(o["y"], f64(p.x) @ f64(p.W) + lora, 1e-12, "y")


def pin_permutation_equivariance(lib):
    """Reordering rows (and their ids) reorders the outputs identically
    ("both match per-request computation", [P3] Summary)."""
    w, p, op = _tiny()
    x, W = f64(p.x), f64(p.W)
    o = oracle.layer(x, W, w.ids, op, lib=lib)
    pi = np.random.default_rng(1).permutation(w.n_rows)
    o2 = oracle.layer(x[pi], W, w.ids[pi], op, lib=lib)
    for k in ("t", "lora", "y"):
        assert np.array_equal(o2[k], o[k][pi]), k


def pin_walkthrough_shared_adapter(lib):
    """[P1] rows 1 and 3 of the walk-through use T1: with equal inputs they
    produce equal outputs; T2 and T3 rows differ from them."""
    w = wl.walkthrough_batch(repeat_row0=True)
    p = w.projections[0]
    op, _ = oracle_pool(p.pool)
    o = oracle.layer(f64(p.x), f64(p.W), w.ids, op, lib=lib)
    assert np.array_equal(o["y"][0], o["y"][2])
    assert not np.allclose(o["y"][1], o["y"][0])
    merged = f64(p.x)[3] @ (f64(p.W) + 2.0 * f64(p.pool.a_block(3)) @ f64(p.pool.b_block(3)))
    _close(o["y"][3], merged, 1e-12, "T3 row")


def pin_special_cases_plain_gemm(lib):
    """All rows base-only, or every scale 0, reduce to a plain matmul; one
    adapter for every row reduces to one matmul with merged weights."""
    w = wl.small_batch(seed=13, n_rows=50, d_in=32, d_out=28, n_adapters=3, ranks=6,
                       dtype=torch.float64, frac_base=0.0)
    p = w.projections[0]
    x, W = f64(p.x), f64(p.W)
    op, _ = oracle_pool(p.pool)
    o = oracle.layer(x, W, np.full(50, -1, np.int32), op, lib=lib)
    _close(o["y"], x @ W, 1e-12, "all base-only")
    op0, _ = oracle_pool(p.pool)
    op0.scales = np.zeros_like(op0.scales)
    o = oracle.layer(x, W, w.ids, op0, lib=lib)
    _close(o["y"], x @ W, 1e-12, "zero scales")
    o = oracle.layer(x, W, np.full(50, 2, np.int32), op, lib=lib)
    Wm = W + p.pool.scales[2] * f64(p.pool.a_block(2)) @ f64(p.pool.b_block(2))
    _close(o["y"], x @ Wm, 1e-12, "single adapter")


def pin_linearity_in_scale(lib):
    """The LoRA term is linear in s ([P4] the alpha/r factor scales the
    adapter's strength): doubling every scale doubles the term exactly."""
    w = wl.small_batch(seed=17, n_rows=40, d_in=20, d_out=16, n_adapters=4, ranks=5,
                       dtype=torch.float64, frac_base=0.2)
    p = w.projections[0]
    op, _ = oracle_pool(p.pool)
    o1 = oracle.layer(f64(p.x), f64(p.W), w.ids, op, lib=lib)
    op.scales = op.scales * 2.0
    o2 = oracle.layer(f64(p.x), f64(p.W), w.ids, op, lib=lib)
    assert np.array_equal(o2["lora"], 2.0 * o1["lora"])
    assert np.array_equal(o2["t"], o1["t"])


def pin_ragged_equals_padded(lib):
    """Zero padding to the maximum rank adds exact zeros ([P4] Batching across
    different adapters: padding vs ragged indexing)."""
    w = wl.small_batch(seed=19, n_rows=70, d_in=36, d_out=30, n_adapters=7,
                       ranks=[8, 16, 32, 64, 8, 16, 3], layout=wl.RAGGED,
                       dtype=torch.float64, frac_base=0.1)
    p = w.projections[0]
    padded = wl.pad_pool(p.pool, 64)
    op_r, _ = oracle_pool(p.pool)
    op_p, _ = oracle_pool(padded)
    o_r = oracle.layer(f64(p.x), f64(p.W), w.ids, op_r, lib=lib)
    o_p = oracle.layer(f64(p.x), f64(p.W), w.ids, op_p, lib=lib)
    for k in ("t", "lora", "y"):
        assert np.array_equal(o_r[k], o_p[k]), k


def pin_invalid_ids(lib):
    """Ids outside [-1, n_adapters) are counted and treated as base-only."""
    w = wl.small_batch(seed=23, n_rows=30, d_in=16, d_out=12, n_adapters=4, ranks=4,
                       dtype=torch.float64, frac_base=0.0)
    p = w.projections[0]
    ids = w.ids.copy()
    ids[[3, 9, 17]] = [4, -2, 1000]
    op, _ = oracle_pool(p.pool)
    o = oracle.layer(f64(p.x), f64(p.W), ids, op, lib=lib)
    assert o["bad"] == 3
    base = f64(p.x) @ f64(p.W)
    for i in (3, 9, 17):
        _close(o["y"][i], base[i], 1e-12, f"invalid row {i}")
        assert np.all(o["t"][i] == 0)


def _merge_case(layout):
    ranks = 12 if layout == wl.UNIFORM else [3, 16, 8, 1, 24, 5]
    w = wl.small_batch(seed=11, n_rows=24, d_in=40, d_out=36, n_adapters=6, ranks=ranks, layout=layout,
                       dtype=torch.float64, frac_base=0.0, scale=[2.0, 0.5, -1.0, 3.0, 1.0, 0.25])
    p = w.projections[0]
    op, _ = oracle_pool(p.pool)
    return w, p, op


def pin_merge_serves_the_adapter(lib):
    """[P4 Merge or keep separate] the merged weight serves the adapter's
    requests as a plain product: x (W + s A_a B_a) equals the layer with
    every row on adapter a."""
    for layout in (wl.UNIFORM, wl.RAGGED):
        w, p, op = _merge_case(layout)
        x, W = f64(p.x), f64(p.W)
        for a in range(op.n_adapters):
            Wm = oracle.merge(W, op, a, lib=lib)
            ids = np.full(x.shape[0], a, np.int32)
            o = oracle.layer(x, W, ids, op, want=("y",), lib=lib)
            _close(x @ Wm, o["y"], 1e-12, f"merged adapter {a} ({layout})")


def pin_merge_then_unmerge(lib):
    """[P4 Merge or keep separate] taking the adapter back out (sign -1)
    restores the base weight; merging twice adds the term twice."""
    w, p, op = _merge_case(wl.RAGGED)
    W = f64(p.W)
    for a in (0, 3, 5):
        Wm = oracle.merge(W, op, a, 1.0, lib=lib)
        _close(oracle.merge(Wm, op, a, -1.0, lib=lib), W, 1e-12, f"unmerge adapter {a}")
        _close(oracle.merge(Wm, op, a, 1.0, lib=lib) - W, 2.0 * (Wm - W), 1e-12, f"merge twice {a}")
    with pytest.raises(ValueError):
        oracle.merge(W, op, op.n_adapters, lib=lib)


def pin_merge_rank_one_outer_product(lib):
    """Closed form: a rank-1 adapter adds s * outer(A[:, 0], B[0, :])."""
    rng = np.random.default_rng(7)
    d_in, d_out = 9, 7
    A = rng.standard_normal((2, d_in, 1))
    B = rng.standard_normal((2, 1, d_out))
    op = oracle.OraclePool.uniform(A, B, [1.5, -0.75])
    W = rng.standard_normal((d_in, d_out))
    for a, s in ((0, 1.5), (1, -0.75)):
        _close(oracle.merge(W, op, a, lib=lib), W + s * np.outer(A[a, :, 0], B[a, 0, :]), 1e-14,
               f"rank-1 merge {a}")


def pin_empty_batch(lib):
    """Zero rows: nothing computed, no error."""
    _, p, op = _tiny()
    o = oracle.layer(np.zeros((0, 256)), f64(p.W), np.zeros(0, np.int32), op, lib=lib)
    assert o["y"].shape == (0, 256) and o["bad"] == 0
    perm, seg_ids, seg_off, bad = oracle.segments(np.zeros(0, np.int32), 8, lib=lib)
    assert perm.size == 0 and seg_ids.size == 0 and seg_off.tolist() == [0]


def pin_dequant_q4_golden(lib):
    """The oracle's 4-bit base weight against entries worked out by hand
    (tests/golden/q4_dequant.json): nibble order, sign, group index and
    orientation."""
    g = json.load(open(os.path.join(GOLDEN, "q4_dequant.json")))
    q = np.array(g["q_rows"], np.uint8)
    W = oracle.dequant_q4(q, np.array(g["scales"]), g["d_in"], group=g["group"], lib=lib)
    assert W.shape == (g["d_in"], g["d_out"])
    want = np.zeros_like(W)
    for k, n, v in g["nonzero"]:
        want[k, n] = v
    assert np.array_equal(W, want)


def pin_q4_values_are_scaled_integers(lib):
    """With power-of-two scales every 4-bit weight is exact in bf16 (so a
    bf16 layer can serve as a cross-check of a 4-bit one), and every weight
    is an integer in [-8, 7] times its group's scale, both ends reached."""
    import torch
    rng = np.random.default_rng(3)
    d_in, d_out = 256, 64
    q = rng.integers(0, 256, size=(d_out, d_in // 2), dtype=np.uint8)
    sc = 2.0 ** rng.integers(-8, -4, size=(d_out, d_in // 128))
    W = oracle.dequant_q4(q, sc, d_in, lib=lib)
    Wb = torch.from_numpy(W).to(torch.bfloat16).double().numpy()
    assert np.array_equal(W, Wb)
    # the nibbles decode to integers in [-8, 7] times the group's scale
    ratio = W.T / np.repeat(sc, 128, axis=1)
    assert np.array_equal(ratio, np.round(ratio)) and ratio.min() >= -8 and ratio.max() <= 7
    assert ratio.min() == -8 and ratio.max() == 7


PINS = [pin_dequant_q4_golden, pin_q4_values_are_scaled_integers, pin_tiny_segments_golden, pin_walkthrough_segments_golden, pin_segments_vs_numpy_stable_sort,
        pin_page_script_agreement, pin_merged_weights, pin_additivity_base_only,
        pin_einsum_gather_formulation, pin_permutation_equivariance, pin_walkthrough_shared_adapter,
        pin_special_cases_plain_gemm, pin_linearity_in_scale, pin_ragged_equals_padded,
        pin_invalid_ids, pin_empty_batch, pin_merge_serves_the_adapter, pin_merge_then_unmerge,
        pin_merge_rank_one_outer_product]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(oracle.load())


def test_param_count_closed_form():
    """[P4 Low-rank structure and additivity] An adapter of rank r on a
    d -> k projection holds r(d+k) numbers; at d=k=4096, r=16 the golden file
    gives that count, the dense d*k count and their ratio in percent."""
    g = _golden("param_count.json")
    assert g["r"] * (g["d"] + g["k"]) == g["adapter_params"]
    assert g["d"] * g["k"] == g["dense_params"]
    assert round(100 * g["adapter_params"] / g["dense_params"], 1) == g["ratio_percent_about"]


def test_sampled_rows_match_full_batch():
    """Computing a subset of rows gives exactly the full batch's values for them."""
    w = wl.tiny_mixed_batch()
    full = run_oracle(w)
    rows = [52, 0, 39, 17]
    part = run_oracle(w, rows=rows)
    for k in ("t", "lora", "y"):
        assert np.array_equal(part[k], full[k][rows]), k

