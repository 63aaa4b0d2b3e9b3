"""Seeded synthetic workloads for the multi-LoRA batched layer.

This module only draws random numbers and lays them out; it holds none of
the layer's arithmetic.  Both the HIP path and the fp64 CPU oracle receive
the tensors built here, so it imports neither of them.

Shapes and value distributions follow the pages:

* the tiny mixed batch is the script of "Serving multiple LoRAs: segmented
  matrix multiplies and adapter scheduling", section "Not merging the
  weights, computing in batches" (seed 0, d=256, r=16, 8 adapters, scale 2,
  lengths [1,1,37,1,12,1], adapters [3,5,3,0,7,5]; 53 rows);
* the four-request T1,T2,T1,T3 decode step of "Multi-LoRA batching and
  adapter paging", section "Walking through a batch";
* 32 decode requests on 20 distinct adapters ("Serving many LoRA adapters",
  blog.ecitis.org, section "Batching across different adapters"), a pool of
  about 250 hot adapters ("Multi-LoRA batching and adapter paging", section
  "Packing math");
* 8B and 70B projection shapes, ranks 8-64 and Zipf-skewed adapter mixes.

Values are drawn in fp32 from N(0,1), divided by a per-tensor constant and,
for bf16 workloads, rounded to bf16 by torch (round to nearest even).
Structure (ids, lengths, ranks) comes from ``numpy.random.default_rng(seed)``;
values from a ``torch.Generator`` on the requested device (one generator per
projection, seeded ``1000*seed + index``, so any subset of projections draws
the same values), so a workload made on ``cuda`` differs numerically from one
made on ``cpu`` but is equally seeded.  Tests always hand the oracle the exact tensors the GPU sees.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np
import torch

UNIFORM = 0
RAGGED = 1

# 8B-shaped layer (d_model 4096, 8 KV heads of 128, MLP 14336).
PROJ_8B = [("q", 4096, 4096), ("k", 4096, 1024), ("v", 4096, 1024), ("o", 4096, 4096),
           ("gate", 4096, 14336), ("up", 4096, 14336), ("down", 14336, 4096)]
# 70B-shaped layer (d_model 8192, 8 KV heads of 128, MLP 28672).
PROJ_70B = [("q", 8192, 8192), ("k", 8192, 1024), ("v", 8192, 1024), ("o", 8192, 8192),
            ("gate", 8192, 28672), ("up", 8192, 28672), ("down", 28672, 8192)]

# Value scales shared by the bf16 workloads: x~N(0,1), W~N(0,1)/64,
# A~N(0,1)/64, B~N(0,1)/16.
X_DIV, W_DIV, A_DIV, B_DIV = 1.0, 64.0, 64.0, 16.0

# Ragged adapter blocks start on a multiple of this many elements (256 B in
# bf16) so that vector loads of any adapter stay aligned.
RAGGED_ALIGN_ELEMS = 128


@dataclass
class Pool:
    """A packed adapter pool for one projection.

    ``A`` and ``B`` are flat 1-D tensors.  Adapter ``u`` occupies
    ``A[a_off[u] : a_off[u] + d_in*ranks[u]]`` as a row-major
    ``[d_in, ranks[u]]`` matrix and ``B[b_off[u] : b_off[u] + ranks[u]*d_out]``
    as a row-major ``[ranks[u], d_out]`` matrix.  For the uniform layout the
    offsets are ``u*d_in*r`` and ``u*r*d_out`` (a dense ``[n, d_in, r]`` /
    ``[n, r, d_out]`` tensor).
    """

    layout: int
    n_adapters: int
    d_in: int
    d_out: int
    r_max: int
    ranks: np.ndarray   # int32 [n_adapters]
    a_off: np.ndarray   # int64 [n_adapters], elements
    b_off: np.ndarray   # int64 [n_adapters], elements
    scales: np.ndarray  # float32 [n_adapters]
    A: torch.Tensor
    B: torch.Tensor

    def a_block(self, u: int) -> torch.Tensor:
        r = int(self.ranks[u])
        o = int(self.a_off[u])
        return self.A[o:o + self.d_in * r].view(self.d_in, r)

    def b_block(self, u: int) -> torch.Tensor:
        r = int(self.ranks[u])
        o = int(self.b_off[u])
        return self.B[o:o + r * self.d_out].view(r, self.d_out)


@dataclass
class Projection:
    name: str
    d_in: int
    d_out: int
    x: torch.Tensor      # [n_rows, d_in]
    W: torch.Tensor      # [d_in, d_out] row-major (the math object y = xW)
    pool: Pool
    pool_padded: Optional[Pool] = None   # same adapters zero-padded to r_max


@dataclass
class Workload:
    name: str
    dtype: torch.dtype
    ids: np.ndarray                  # int32 [n_rows]; -1 = base only
    projections: List[Projection]
    lengths: Optional[List[int]] = None          # request lengths (rows per request)
    request_ids: Optional[List[int]] = None      # adapter id per request
    notes: dict = field(default_factory=dict)

    @property
    def n_rows(self) -> int:
        return int(self.ids.shape[0])


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn(g, shape, div, dtype, device) -> torch.Tensor:
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if div != 1.0:
        t = t / div
    return t.to(dtype)


def zipf_probs(n: int, s: float = 1.1) -> np.ndarray:
    """P(k) proportional to k^-s over k = 1..n (id = k-1)."""
    k = np.arange(1, n + 1, dtype=np.float64)
    p = k ** (-s)
    return p / p.sum()


def ragged_layout(ranks: np.ndarray, d_in: int, d_out: int, align: int = RAGGED_ALIGN_ELEMS):
    """Element offsets of a ragged pool; each block starts ``align``-aligned."""
    n = len(ranks)
    a_off = np.zeros(n, np.int64)
    b_off = np.zeros(n, np.int64)
    pa = pb = 0
    for u in range(n):
        a_off[u] = pa
        b_off[u] = pb
        pa += -(-int(d_in) * int(ranks[u]) // align) * align
        pb += -(-int(ranks[u]) * int(d_out) // align) * align
    return a_off, b_off, pa, pb


def make_uniform_pool(g, device, dtype, n_adapters, d_in, d_out, r, scale=2.0,
                      a_div=A_DIV, b_div=B_DIV) -> Pool:
    A = _randn(g, (n_adapters * d_in * r,), a_div, dtype, device)
    B = _randn(g, (n_adapters * r * d_out,), b_div, dtype, device)
    u = np.arange(n_adapters, dtype=np.int64)
    return Pool(UNIFORM, n_adapters, d_in, d_out, r,
                np.full(n_adapters, r, np.int32), u * d_in * r, u * r * d_out,
                np.full(n_adapters, scale, np.float32), A, B)


def make_ragged_pool(g, device, dtype, ranks, d_in, d_out, scale=2.0,
                     a_div=A_DIV, b_div=B_DIV) -> Pool:
    ranks = np.asarray(ranks, np.int32)
    a_off, b_off, ta, tb = ragged_layout(ranks, d_in, d_out)
    A = _randn(g, (ta,), a_div, dtype, device)
    B = _randn(g, (tb,), b_div, dtype, device)
    return Pool(RAGGED, len(ranks), d_in, d_out, int(ranks.max()), ranks, a_off, b_off,
                np.full(len(ranks), scale, np.float32), A, B)


def pad_pool(p: Pool, r_pad: int) -> Pool:
    """The same adapters in a uniform pool of rank ``r_pad``, exact zeros past each true rank."""
    n, d_in, d_out = p.n_adapters, p.d_in, p.d_out
    A = torch.zeros((n, d_in, r_pad), dtype=p.A.dtype, device=p.A.device)
    B = torch.zeros((n, r_pad, d_out), dtype=p.B.dtype, device=p.B.device)
    for u in range(n):
        r = int(p.ranks[u])
        A[u, :, :r] = p.a_block(u)
        B[u, :r, :] = p.b_block(u)
    u = np.arange(n, dtype=np.int64)
    return Pool(UNIFORM, n, d_in, d_out, r_pad, np.full(n, r_pad, np.int32),
                u * d_in * r_pad, u * r_pad * d_out, p.scales.copy(),
                A.view(-1), B.view(-1))


# --------------------------------------------------------------------------
# The tiny mixed batch and the T1,T2,T1,T3 walk-through
# --------------------------------------------------------------------------

TINY_LENGTHS = [1, 1, 37, 1, 12, 1]
TINY_ADAPTERS = [3, 5, 3, 0, 7, 5]


def tiny_mixed_batch(device="cpu") -> Workload:
    """The page's fp32 script inputs, drawn in the page's order from seed 0.

    W = randn(256,256)/16, A = randn(8,256,16)/16, B = randn(8,16,256)/4,
    x = randn(sum(lengths), 256); scale 2.0.  Drawn on the CPU (so the values
    are those of the page's script) and then moved to ``device``.
    """
    g = _gen("cpu", 0)
    d, r, n_ad = 256, 16, 8
    W = torch.randn(d, d, generator=g) / 16
    A = torch.randn(n_ad, d, r, generator=g) / 16
    B = torch.randn(n_ad, r, d, generator=g) / 4
    x = torch.randn(sum(TINY_LENGTHS), d, generator=g)
    ids = np.array([a for a, n in zip(TINY_ADAPTERS, TINY_LENGTHS) for _ in range(n)], np.int32)
    u = np.arange(n_ad, dtype=np.int64)
    pool = Pool(UNIFORM, n_ad, d, d, r, np.full(n_ad, r, np.int32), u * d * r, u * r * d,
                np.full(n_ad, 2.0, np.float32), A.reshape(-1).to(device), B.reshape(-1).to(device))
    proj = Projection("tiny", d, d, x.to(device), W.to(device), pool)
    return Workload("tiny_mixed_fp32", torch.float32, ids, [proj],
                    lengths=list(TINY_LENGTHS), request_ids=list(TINY_ADAPTERS))


def walkthrough_batch(device="cpu", repeat_row0=False) -> Workload:
    """T1,T2,T1,T3 as adapter ids 1,2,1,3 on the tiny pool; x from seed 1.

    With ``repeat_row0`` the third row is a copy of the first, so the two T1
    rows must produce the same output.
    """
    base = tiny_mixed_batch(device)
    g = _gen("cpu", 1)
    x = torch.randn(4, 256, generator=g)
    if repeat_row0:
        x[2] = x[0]
    p = base.projections[0]
    proj = Projection("walkthrough", 256, 256, x.to(device), p.W, p.pool)
    return Workload("walkthrough_T1T2T1T3", torch.float32, np.array([1, 2, 1, 3], np.int32), [proj],
                    lengths=[1, 1, 1, 1], request_ids=[1, 2, 1, 3])


# --------------------------------------------------------------------------
# Decode / prefill workloads
# --------------------------------------------------------------------------

def decode_q_proj_ids(seed=1) -> np.ndarray:
    """32 rows: 20 distinct ids drawn without replacement from 250, each used
    once plus 9 more uniform draws among them, 3 base-only rows; shuffled."""
    rng = np.random.default_rng(seed)
    n_rows, n_pool, n_distinct = 32, 250, 20
    n_base = int(round(0.1 * n_rows))
    chosen = rng.choice(n_pool, n_distinct, replace=False)
    extra = rng.choice(chosen, n_rows - n_base - n_distinct)
    ids = np.concatenate([chosen, extra, np.full(n_base, -1)]).astype(np.int32)
    rng.shuffle(ids)
    return ids


def skewed_decode_ids(seed=2) -> np.ndarray:
    """256 rows with ids ~ Zipf(1.1) over a pool of 1000."""
    rng = np.random.default_rng(seed)
    return rng.choice(1000, 256, p=zipf_probs(1000)).astype(np.int32)


def prefill_ids(seed=3, lengths=None):
    """16 requests, lengths ~ U{128..2048}, 8 distinct ids from 64, two
    requests each, arrival order shuffled; rows request after request."""
    rng = np.random.default_rng(seed)
    n_pool, n_req = 64, 16
    if lengths is None:
        lengths = rng.integers(128, 2049, n_req).tolist()
    else:
        rng.integers(128, 2049, n_req)
    distinct = rng.choice(n_pool, 8, replace=False)
    req_ids = np.repeat(distinct, 2)
    rng.shuffle(req_ids)
    ids = np.concatenate([np.full(n, a) for a, n in zip(req_ids, lengths)]).astype(np.int32)
    return ids, list(lengths), req_ids


def mixed_rank_ids(seed=4):
    """Ranks of a ragged pool of 500 and the 2218-row chunked-prefill batch."""
    rng = np.random.default_rng(seed)
    n_pool = 500
    ranks = rng.choice([8, 16, 32, 64], n_pool, p=[0.4, 0.3, 0.2, 0.1]).astype(np.int32)
    p = zipf_probs(n_pool)
    dec_ids = rng.choice(n_pool, 64, p=p)
    pre_ids = rng.choice(n_pool, 4, p=p)
    n_base = int(round(0.05 * (64 + 4 * 512)))
    block = np.full(64 + n_base, -1, np.int64)
    pos = np.sort(rng.choice(64 + n_base, 64, replace=False))
    block[pos] = dec_ids
    ids = np.concatenate([block] + [np.full(512, a) for a in pre_ids]).astype(np.int32)
    return ids, ranks, block, pre_ids


def decode_q_proj(device="cuda", dtype=torch.bfloat16, seed=1, value_seed=None) -> Workload:
    """32 decode rows, 20 distinct adapters out of a uniform rank-16 pool of 250,
    3 base-only rows (10%), one 4096->4096 projection.  ``value_seed`` draws
    other values for the same batch (replicas of the layer)."""
    ids = decode_q_proj_ids(seed)
    n_rows, n_pool, n_distinct, n_base = len(ids), 250, 20, int((ids == -1).sum())
    g = _gen(device, seed if value_seed is None else value_seed)
    d_in = d_out = 4096
    x = _randn(g, (n_rows, d_in), X_DIV, dtype, device)
    W = _randn(g, (d_in, d_out), W_DIV, dtype, device)
    pool = make_uniform_pool(g, device, dtype, n_pool, d_in, d_out, 16)
    return Workload("decode_bgmv_q4096_r16_pool250_rows32", dtype, ids,
                    [Projection("q", d_in, d_out, x, W, pool)],
                    notes={"distinct": n_distinct, "base_rows": n_base})


def skewed_decode_8b(device="cuda", dtype=torch.bfloat16, seed=2, projections=None) -> Workload:
    """256 decode rows, ids ~ Zipf(1.1) over a rank-16 pool of 1000, all seven 8B projections."""
    ids = skewed_decode_ids(seed)
    n_rows, n_pool = len(ids), 1000
    projs = []
    for pi, (name, d_in, d_out) in enumerate(PROJ_8B):
        if projections is not None and name not in projections:
            continue
        g = _gen(device, 1000 * seed + pi)
        x = _randn(g, (n_rows, d_in), X_DIV, dtype, device)
        W = _randn(g, (d_in, d_out), W_DIV, dtype, device)
        pool = make_uniform_pool(g, device, dtype, n_pool, d_in, d_out, 16)
        projs.append(Projection(name, d_in, d_out, x, W, pool))
    return Workload("skewed_decode_8b_r16_pool1000_rows256", dtype, ids, projs,
                    notes={"distinct": int(len(set(ids.tolist())))})


def prefill_70b(device="cuda", dtype=torch.bfloat16, seed=3, projections=None,
                lengths=None) -> Workload:
    """16 prefill requests, lengths ~ U{128..2048}, 8 distinct rank-64 adapters
    (two requests each) from a pool of 64; rows in arrival order."""
    ids, lengths, req_ids = prefill_ids(seed, lengths)
    n_pool = 64
    projs = []
    for pi, (name, d_in, d_out) in enumerate(PROJ_70B):
        if projections is not None and name not in projections:
            continue
        g = _gen(device, 1000 * seed + pi)
        x = _randn(g, (len(ids), d_in), X_DIV, dtype, device)
        W = _randn(g, (d_in, d_out), W_DIV, dtype, device)
        pool = make_uniform_pool(g, device, dtype, n_pool, d_in, d_out, 64)
        projs.append(Projection(name, d_in, d_out, x, W, pool))
    return Workload("prefill_sgmv_70b_r64_pool64_req16", dtype, ids, projs,
                    lengths=list(lengths), request_ids=req_ids.tolist())


def mixed_rank_70b(device="cuda", dtype=torch.bfloat16, seed=4, projections=None,
                   with_padded=True) -> Workload:
    """Chunked-prefill batch on a ragged pool of 500 (ranks 8/16/32/64 with
    weights .4/.3/.2/.1): 64 Zipf decode rows with 106 base-only rows
    interleaved, then 4 prefill segments of 512 rows; 2218 rows."""
    ids, ranks, block, pre_ids = mixed_rank_ids(seed)
    projs = []
    for pi, (name, d_in, d_out) in enumerate(PROJ_70B):
        if projections is not None and name not in projections:
            continue
        g = _gen(device, 1000 * seed + pi)
        x = _randn(g, (len(ids), d_in), X_DIV, dtype, device)
        W = _randn(g, (d_in, d_out), W_DIV, dtype, device)
        pool = make_ragged_pool(g, device, dtype, ranks, d_in, d_out)
        padded = pad_pool(pool, 64) if with_padded else None
        projs.append(Projection(name, d_in, d_out, x, W, pool, padded))
    return Workload("mixed_rank_70b_ragged_pool500_rows2218", dtype, ids, projs,
                    lengths=[1] * len(block) + [512] * 4,
                    request_ids=block.tolist() + pre_ids.tolist())


def small_batch(seed=0, n_rows=200, d_in=320, d_out=288, n_adapters=12, ranks=16,
                layout=UNIFORM, dtype=torch.float32, device="cpu", frac_base=0.1,
                run_lengths=None, scale=None) -> Workload:
    """A mid-sized mixed batch for parity tests: several tiles plus ragged tails.

    ``ranks`` is an int (uniform pool) or a list (ragged pool).  ``run_lengths``
    lays rows out as consecutive requests (prefill-like); otherwise every row
    is its own request (decode-like).  ``scale`` overrides the per-adapter
    scale (a float or an array).
    """
    rng = np.random.default_rng(seed)
    if run_lengths is None:
        ids = rng.integers(0, n_adapters, n_rows)
        lengths = [1] * n_rows
    else:
        lengths = list(run_lengths)
        req = rng.integers(0, n_adapters, len(lengths))
        ids = np.concatenate([np.full(n, a) for a, n in zip(req, lengths)])
        n_rows = len(ids)
    base = rng.random(n_rows) < frac_base
    ids = np.where(base, -1, ids).astype(np.int32)
    g = _gen(device, seed)
    x = _randn(g, (n_rows, d_in), X_DIV, dtype, device)
    W = _randn(g, (d_in, d_out), float(np.sqrt(d_in)), dtype, device)
    if layout == UNIFORM:
        pool = make_uniform_pool(g, device, dtype, n_adapters, d_in, d_out, int(ranks),
                                 a_div=float(np.sqrt(d_in)), b_div=4.0)
    else:
        pool = make_ragged_pool(g, device, dtype, ranks, d_in, d_out,
                                a_div=float(np.sqrt(d_in)), b_div=4.0)
    if scale is not None:
        pool.scales = np.broadcast_to(np.asarray(scale, np.float32), (n_adapters,)).copy()
    return Workload(f"small_s{seed}", dtype, ids, [Projection("p", d_in, d_out, x, W, pool)],
                    lengths=lengths)


CONFIG_BUILDERS = {
    0: tiny_mixed_batch,
    1: decode_q_proj,
    2: skewed_decode_8b,
    3: prefill_70b,
    4: mixed_rank_70b,
}


# --------------------------------------------------------------------------
# Adapter sets for the slot cache (host tier)
# --------------------------------------------------------------------------

@dataclass
class AdapterSet:
    """Adapters of several projections each, kept on the host: adapter u has
    rank ranks[u], scale scales[u] and, for part p, A[u][p] [d_in_p, r_u]
    and B[u][p] [r_u, d_out_p]."""
    parts: List[Tuple[int, int]]
    ranks: np.ndarray
    scales: np.ndarray
    A: List[List[torch.Tensor]]
    B: List[List[torch.Tensor]]


def adapter_set(parts, ranks, scales, dtype=torch.bfloat16, seed=0, a_div=64.0, b_div=16.0) -> AdapterSet:
    """Host (CPU) adapters with this module's value distributions: A ~
    N(0,1)/a_div, B ~ N(0,1)/b_div, drawn per adapter from a generator
    seeded ``1000*seed + u``."""
    ranks = np.asarray(ranks, np.int32)
    scales = np.asarray(scales, np.float32)
    As, Bs = [], []
    for u, r in enumerate(ranks):
        g = _gen("cpu", 1000 * seed + u)
        As.append([_randn(g, (di, int(r)), a_div, dtype, "cpu") for di, _ in parts])
        Bs.append([_randn(g, (int(r), do), b_div, dtype, "cpu") for _, do in parts])
    return AdapterSet([(int(a), int(b)) for a, b in parts], ranks, scales, As, Bs)


def eight_b_parts(layers: int = 32):
    """(d_in, d_out) of every projection of an 8B-shaped model, layer by
    layer: q, k, v, o, gate, up, down."""
    one = [(4096, 4096), (4096, 1024), (4096, 1024), (4096, 4096), (4096, 14336), (4096, 14336),
           (14336, 4096)]
    return one * layers


def q4_weight(seed: int, d_in: int, d_out: int, device="cuda", pow2_scales: bool = False):
    """A 4-bit base weight in the layout lora_decode_stream_q4 reads: bytes
    Wq [d_out, d_in / 2] with uniformly drawn nibbles (signed values -8..7)
    and fp32 scales [d_out, d_in / 128] drawn so that q * scale has about the
    spread of the bf16 weights here (std ~ 1/64).  With ``pow2_scales`` every
    scale is a power of two (each weight is then exact in bf16)."""
    g = _gen(device, 5000 + seed)
    Wq = torch.randint(0, 256, (d_out, d_in // 2), generator=g, device=device, dtype=torch.int32).to(torch.uint8)
    n_g = d_in // 128
    if pow2_scales:
        e = torch.randint(-10, -7, (d_out, n_g), generator=g, device=device, dtype=torch.int32)
        sc = torch.pow(2.0, e.to(torch.float32))
    else:
        u = torch.rand((d_out, n_g), generator=g, device=device, dtype=torch.float32)
        sc = (0.5 + u) / (64.0 * 4.6)
    return Wq.contiguous(), sc.contiguous()
