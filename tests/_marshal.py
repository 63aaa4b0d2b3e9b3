"""Argument marshalling shared by the tests: torch tensors -> fp64 numpy for the
oracle, and compaction of big pools to the adapters a batch actually uses.
No arithmetic of the layer lives here."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from lora_bgmv_shrink_amd import workloads as wl


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening to fp64 (bf16 -> fp32 -> fp64 are both exact)."""
    return t.detach().to("cpu").to(torch.float32).to(torch.float64).numpy()


def oracle_pool(pool: wl.Pool, used=None, cols=None):
    """fp64 copy of ``pool``.  With ``used`` only those adapters are kept and
    the returned map sends old ids to new ones (-1 stays -1).  With ``cols``
    only those output columns of every B block are kept (d_out = len(cols))."""
    if used is None and cols is None:
        return oracle.OraclePool(pool.n_adapters, pool.d_in, pool.d_out, pool.r_max,
                                 pool.ranks.astype(np.int32), pool.a_off.astype(np.int64),
                                 pool.b_off.astype(np.int64), f64(pool.A), f64(pool.B),
                                 pool.scales.astype(np.float64)), None
    if used is None:
        used = range(pool.n_adapters)
    used = sorted(int(u) for u in set(used) if 0 <= int(u) < pool.n_adapters)
    d_out = pool.d_out if cols is None else len(cols)
    cidx = None if cols is None else torch.as_tensor(np.asarray(cols), device=pool.B.device)
    As, Bs, a_off, b_off, ranks = [], [], [], [], []
    pa = pb = 0
    for u in used:
        A = f64(pool.a_block(u)).reshape(-1)
        Bb = pool.b_block(u)
        if cidx is not None:
            Bb = Bb[:, cidx]
        B = f64(Bb).reshape(-1)
        a_off.append(pa)
        b_off.append(pb)
        pa += A.size
        pb += B.size
        As.append(A)
        Bs.append(B)
        ranks.append(int(pool.ranks[u]))
    n = len(used)
    mp = {u: i for i, u in enumerate(used)}
    op = oracle.OraclePool(max(n, 1), pool.d_in, d_out, pool.r_max,
                           np.array(ranks if n else [1], np.int32),
                           np.array(a_off if n else [0], np.int64), np.array(b_off if n else [0], np.int64),
                           np.concatenate(As) if As else np.zeros(pool.d_in),
                           np.concatenate(Bs) if Bs else np.zeros(d_out),
                           pool.scales[used].astype(np.float64) if n else np.zeros(1))
    if n == 0:
        mp = {}
    return op, mp


def remap_ids(ids: np.ndarray, mp, n_adapters_old: int) -> np.ndarray:
    """Apply a compaction map; invalid ids map to a value the compact pool also rejects."""
    out = np.empty_like(ids)
    for i, a in enumerate(ids.tolist()):
        if a == -1:
            out[i] = -1
        elif 0 <= a < n_adapters_old and a in mp:
            out[i] = mp[a]
        else:
            out[i] = -2
    return out


def run_oracle(w: wl.Workload, proj: int = 0, rows=None, cols=None, want=("t", "lora", "y"),
               padded: bool = False, threads: int = 0):
    """Oracle outputs for projection ``proj`` of workload ``w``.

    With ``rows`` only those rows are computed, in the order given (rows of
    the layer are independent, so a sub-batch is computed exactly as inside
    the full batch); with ``cols`` only those output columns (columns are
    independent too).  Big pools are compacted to the adapters the selected
    rows use; ids outside the pool map to an id the compact pool also
    rejects."""
    p = w.projections[proj]
    pool = p.pool_padded if padded else p.pool
    ids = w.ids if rows is None else w.ids[np.asarray(rows)]
    if pool.n_adapters > 64 or cols is not None:
        op, mp = oracle_pool(pool, used=ids.tolist(), cols=cols)
        ids = remap_ids(ids, mp, pool.n_adapters)
    else:
        op, _ = oracle_pool(pool)
    if rows is None:
        x = f64(p.x)
    else:
        x = f64(p.x[torch.as_tensor(np.asarray(rows), device=p.x.device)])
    W = None
    if "y" in want:
        Wt = p.W if cols is None else p.W[:, torch.as_tensor(np.asarray(cols), device=p.W.device)]
        W = f64(Wt)
    return oracle.layer(x, W, ids, op, want=want, threads=threads)
