"""Property test: lora_layer_apply against the fp64 oracle on batches drawn
by hypothesis (derandomized, bounded: the same examples every run).

Drawn: 0..300 rows; ids with base-only rows, all base-only, one adapter, or
uniform over the pool; uniform or ragged pools with ranks 1..64; bf16 or
fp32; both W layouts; AUTO, BGMV and SGMV; bf16 or fp32 y; and a random row
permutation, under which the layer must permute its rows (each row is its
own request: "Serving multiple LoRAs: segmented matrix multiplies and
adapter scheduling", section "Summary").
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

hyp = pytest.importorskip("hypothesis")
from hypothesis import given, settings, HealthCheck, strategies as st  # noqa: E402

from _gpu import TOL, binding, pool_of, requires_gpu, say, scaled_err, w_stored  # noqa: E402
from _marshal import run_oracle  # noqa: E402
from lora_bgmv_shrink_amd import workloads as wl  # noqa: E402

pytestmark = [pytest.mark.gpu, requires_gpu]

DEV = "cuda"


@st.composite
def batches(draw):
    n = draw(st.sampled_from([0, 1, 5, 33, 64, 65, 130, 300]))
    d_in = 8 * draw(st.integers(8, 96))
    d_out = 8 * draw(st.integers(1, 100))
    n_ad = draw(st.integers(1, 20))
    dtype = draw(st.sampled_from([torch.bfloat16, torch.float32]))
    ragged = draw(st.booleans())
    if ragged:
        ranks = draw(st.lists(st.integers(1, 64), min_size=n_ad, max_size=n_ad))
    else:
        ranks = draw(st.sampled_from([1, 4, 8, 16, 32, 64]))
    pattern = draw(st.sampled_from(["mixed", "allbase", "one", "uniform"]))
    seed = draw(st.integers(0, 2 ** 16))
    mode = draw(st.sampled_from(["auto", "bgmv", "sgmv"]))
    wlay = draw(st.sampled_from(["out_in", "in_out"]))
    ydt = draw(st.sampled_from([torch.bfloat16, torch.float32]))
    return dict(n=n, d_in=d_in, d_out=d_out, n_ad=n_ad, dtype=dtype, ragged=ragged, ranks=ranks,
                pattern=pattern, seed=seed, mode=mode, wlay=wlay, ydt=ydt)


@settings(max_examples=40, deadline=None, derandomize=True, database=None,
          suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])
@given(batches())
def test_layer_property(c):
    b = binding()
    say(f"property: {c}")
    rng = np.random.default_rng(c["seed"])
    n, n_ad = c["n"], c["n_ad"]
    w = wl.small_batch(seed=c["seed"], n_rows=max(n, 1), d_in=c["d_in"], d_out=c["d_out"], n_adapters=n_ad,
                       ranks=c["ranks"], layout=wl.RAGGED if c["ragged"] else wl.UNIFORM, dtype=c["dtype"],
                       device=DEV, frac_base=0.0, scale=rng.uniform(-2.0, 2.0, n_ad).astype(np.float32))
    ids = {"mixed": np.where(rng.random(n) < 0.2, -1, rng.integers(0, n_ad, n)),
           "allbase": np.full(n, -1), "one": np.full(n, int(rng.integers(0, n_ad))),
           "uniform": rng.integers(0, n_ad, n)}[c["pattern"]].astype(np.int32)
    p = w.projections[0]
    x = p.x[:n]
    w = wl.Workload("prop", w.dtype, ids, [wl.Projection("p", p.d_in, p.d_out, x, p.W, p.pool)])
    pool = pool_of(p.pool)
    lay = b.LORA_W_OUT_IN if c["wlay"] == "out_in" else b.LORA_W_IN_OUT
    m = {"auto": b.LORA_MODE_AUTO, "bgmv": b.LORA_MODE_BGMV, "sgmv": b.LORA_MODE_SGMV}[c["mode"]]
    ydt = c["ydt"] if c["d_out"] % 8 == 0 else torch.float32
    Ws = w_stored(p.W, lay)
    ids_d = torch.as_tensor(ids, device=DEV)
    y = b.lora_layer_apply(pool, x, Ws, ids_d, w_layout=lay, mode=m, y_dtype=ydt)
    torch.cuda.synchronize()
    if n == 0:
        assert y.shape[0] == 0
        return
    o = run_oracle(w)
    tol = TOL[c["dtype"]] if ydt == torch.float32 or c["dtype"] == torch.bfloat16 else TOL[torch.bfloat16]
    e = scaled_err(y, o["y"])
    assert float(e.max()) <= tol, f"max scaled err {e.max():.3e}"
    # a row permutation permutes the rows of y (within tolerance: grouping may change the order of sums)
    perm = rng.permutation(n)
    pt = torch.as_tensor(perm, device=DEV)
    yp = b.lora_layer_apply(pool, x[pt].contiguous(), Ws, ids_d[pt].contiguous(), w_layout=lay, mode=m, y_dtype=ydt)
    torch.cuda.synchronize()
    ep = scaled_err(yp, o["y"][perm])
    assert float(ep.max()) <= tol, f"permuted: max scaled err {ep.max():.3e}"
