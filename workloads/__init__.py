"""Seeded synthetic inputs for the N-gram embedding layer: shapes, token ids and tables.

This module is shared by the tests, the benchmark and the smoke check. It feeds both the
HIP library and the CPU oracle, so it holds none of the layer's arithmetic: no hashing, no
row lookup, no projection. It only says how big things are and draws random numbers.

Sources (web notes on "Scaling Embeddings Outperforms Scaling Experts in Language Models"):
  * table shapes E_0 [V0, D], E_{n,k} [V_{n,k}, D/((N-1)K)], W_{n,k} [D, D/((N-1)K)]:
    section A2 (the final Over-Encoding form and the sentence after it);
  * sub-table sizes are kept well away from integer multiples of V0: section 3.2.2 and the
    2-gram collision plot (Fig. 3b). Every size below sits half-way between two multiples.
  * N in 3..5 and K >= 2 are the robust range: section 3.2.3 (Fig. 4).
  * the basic form (section A2, Eq. 1) has one full-width table E_n [V_n, D] per order and
    no projection; its workloads keep K = 1 and give the tables about the parameter count of
    the final-form workload of the same size.
The pages name no token-id distribution; uniform and Zipf(1.1) ids stand in for real text.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "workload", "mid_gap_primes",
    "uniform_ids", "zipf_ids", "token_batch", "cu_seqlens_from_lengths",
    "host_tables", "device_tables", "split_stacked_w", "collision_study",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    """One layer configuration plus the batch it is exercised on."""
    name: str
    dtype: str                 # "f32" or "bf16": tables, projection and output
    V0: int                    # base vocabulary
    D: int                     # hidden size
    N: int                     # largest n-gram order
    K: int                     # sub-tables per order
    V: Tuple[int, ...]         # V_{n,k}, n-major, k-minor: s = (n-2)*K + (k-1)
    batch: int                 # sequences
    seqlen: int                # tokens per sequence
    ids: str                   # "uniform" or "zipf1.1"
    seed: int
    mode: str = "prefill"      # "prefill" or "decode"
    decode_steps: int = 0      # decode: steps per run
    decode_new: int = 0        # decode: new tokens per sequence per step (1 + drafts)
    form: str = "final"        # "final" (projected sub-tables) or "basic" (Eq. 1)
    layers: int = 1            # per-layer embeddings: layers with tables of their own

    @property
    def S(self) -> int:
        return (self.N - 1) * self.K

    @property
    def d(self) -> int:
        if not self.S:
            return 0
        return self.D if self.form == "basic" else self.D // self.S

    @property
    def T(self) -> int:
        return self.batch * self.seqlen

    @property
    def esz(self) -> int:
        return 4 if self.dtype == "f32" else 2


def _w(name, dtype, V0, D, N, K, V, batch, seqlen, ids, seed, **kw) -> Workload:
    return Workload(name, dtype, V0, D, N, K, tuple(V), batch, seqlen, ids, seed, **kw)


# Sub-table sizes for the bf16 workloads: primes just above (floor(target/V0) + 1/2) * V0,
# consecutive primes where one start point serves several sub-tables.
_V2 = (1008001, 1104017, 1200007, 1296007)
_V3 = (2031671, 2031691, 2031703, 2031713, 2031749, 2031767, 2031779, 2031791,
       2031811, 2031839, 2031851, 2031863, 2031893, 2031907, 2031937, 2031961)
_V4 = (9764873, 9764897, 9764899, 9764921, 9764939, 9764957, 9764959, 9764971,
       9764977, 9764981, 9765001, 9765017)
_V5 = (983063, 983069, 983083, 983113)       # per-layer workload, V0 = 131072
_VB2 = (1104017, 1104041)                 # basic form, V0 = 32000
_VB4 = (3211279, 3211289, 3211291)        # basic form, V0 = 131072: 3 x 3.2M x 3072 = 29.6B

WORKLOADS = {
    "tiny_f32": _w("tiny_f32", "f32", 1000, 64, 3, 2, (5003, 7001, 6007, 8009), 2, 128,
                   "uniform", 0),
    "bf16_d1024": _w("bf16_d1024", "bf16", 32000, 1024, 3, 2, _V2, 8, 2048, "uniform", 2),
    "bf16_d2048_n5k4": _w("bf16_d2048_n5k4", "bf16", 131072, 2048, 5, 4, _V3, 16, 4096,
                          "zipf1.1", 3),
    "prefill_64k_30b": _w("prefill_64k_30b", "bf16", 131072, 3072, 4, 4, _V4, 8, 8192,
                          "zipf1.1", 4),
    "decode_spec5_30b": _w("decode_spec5_30b", "bf16", 131072, 3072, 4, 4, _V4, 256, 8192,
                           "zipf1.1", 5, mode="decode", decode_steps=1000, decode_new=5),
    # the basic form (Eq. 1)
    "basic_tiny_f32": _w("basic_tiny_f32", "f32", 1000, 64, 3, 1, (5003, 7001), 2, 128,
                         "uniform", 6, form="basic"),
    "basic_bf16_d1024": _w("basic_bf16_d1024", "bf16", 32000, 1024, 3, 1, _VB2, 8, 2048,
                           "uniform", 7, form="basic"),
    # per-layer N-gram embedding (section 5.2): 8 layers, 2.0B n-gram parameters each
    "plne_8x_d2048": _w("plne_8x_d2048", "bf16", 131072, 2048, 3, 2, _V5, 8, 8192, "zipf1.1", 9,
                        layers=8),
    "prefill_64k_basic_30b": _w("prefill_64k_basic_30b", "bf16", 131072, 3072, 4, 1, _VB4, 8,
                                8192, "zipf1.1", 8, form="basic"),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def _is_prime(x: int) -> bool:
    if x < 2:
        return False
    if x % 2 == 0:
        return x == 2
    f = 3
    while f * f <= x:
        if x % f == 0:
            return False
        f += 2
    return True


def mid_gap_primes(V0: int, target: int, count: int) -> List[int]:
    """`count` consecutive primes starting at (floor(target/V0) + 1/2) * V0.

    Puts every size about half-way between two multiples of V0, the collision-safe region
    of section 3.2.2."""
    x = (target // V0) * V0 + V0 // 2
    out = []
    while len(out) < count:
        x += 1
        if _is_prime(x):
            out.append(x)
    return out


# ---------------------------------------------------------------- token ids

def _rng(seed: int, purpose: int) -> np.random.Generator:
    return np.random.default_rng([0, seed, purpose])


def uniform_ids(rng: np.random.Generator, V0: int, shape) -> np.ndarray:
    return rng.integers(0, V0, size=shape, dtype=np.int64).astype(np.int32)


def zipf_ids(rng: np.random.Generator, V0: int, shape, s: float = 1.1) -> np.ndarray:
    """Ids with rank frequency proportional to r^-s over ranks 1..V0 (inverse CDF), mapped
    through a seeded permutation so the most frequent id is not id 0."""
    ranks = np.arange(1, V0 + 1, dtype=np.float64)
    cdf = np.cumsum(ranks ** (-s))
    cdf /= cdf[-1]
    perm = rng.permutation(V0)
    u = rng.random(size=int(np.prod(shape)))
    r = np.minimum(np.searchsorted(cdf, u, side="right"), V0 - 1)
    return perm[r].astype(np.int32).reshape(shape)


def token_batch(w: Workload, purpose: int = 0, batch: Optional[int] = None,
                seqlen: Optional[int] = None) -> np.ndarray:
    """int32 [batch, seqlen] token ids for workload `w`; `purpose` selects an independent
    stream (0 = the workload's own batch, others for rotations and decode steps)."""
    b = w.batch if batch is None else batch
    L = w.seqlen if seqlen is None else seqlen
    rng = _rng(w.seed, purpose)
    if w.ids == "uniform":
        return uniform_ids(rng, w.V0, (b, L))
    return zipf_ids(rng, w.V0, (b, L))


def cu_seqlens_from_lengths(lengths: Sequence[int]) -> np.ndarray:
    out = np.zeros(len(lengths) + 1, dtype=np.int32)
    out[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return out


# ---------------------------------------------------------------- tables

def _torch_dtype(w: Workload):
    import torch
    return torch.float32 if w.dtype == "f32" else torch.bfloat16


def _shapes(w: Workload):
    # the basic form has no projection W
    return [(w.V0, w.D)] + [(v, w.d) for v in w.V] + ([] if w.form == "basic" else [(w.D, w.D)])


def _split(w: Workload, mats):
    if w.form == "basic":
        return mats[0], mats[1:], None
    return mats[0], mats[1:-1], mats[-1]


def host_tables(w: Workload, seed: Optional[int] = None, std: float = 0.02):
    """CPU tables (E0, [E_s], W_stack) drawn N(0, std) in fp32 and rounded to the workload
    dtype (round-to-nearest-even for bf16). W_stack[o, s*d + c] holds W_{n,k}[o, c]; None
    in the basic form."""
    import torch
    g = torch.Generator().manual_seed(1000 * w.seed + (0 if seed is None else seed))
    dt = _torch_dtype(w)
    mats = [torch.empty(sh, dtype=torch.float32).normal_(0.0, std, generator=g).to(dt)
            for sh in _shapes(w)]
    return _split(w, mats)


def device_tables(w: Workload, device="cuda", seed: Optional[int] = None, std: float = 0.02,
                  chunk_rows: int = 1 << 20):
    """Device tables with the same shapes and distribution as host_tables, drawn by torch's
    device generator in row chunks (the 30B-parameter workload is 60 GB)."""
    import torch
    g = torch.Generator(device=device).manual_seed(1000 * w.seed + (0 if seed is None else seed))
    dt = _torch_dtype(w)
    mats = []
    for (r, c) in _shapes(w):
        t = torch.empty((r, c), dtype=dt, device=device)
        for r0 in range(0, r, chunk_rows):
            r1 = min(r, r0 + chunk_rows)
            t[r0:r1].copy_(torch.empty((r1 - r0, c), dtype=torch.float32, device=device)
                           .normal_(0.0, std, generator=g))
        mats.append(t)
    return _split(w, mats)


def split_stacked_w(W_stack, S: int):
    """The S blocks W_{n,k} [D, d] of a stacked [D, S*d] projection (a view per block)."""
    d = W_stack.shape[1] // S
    return [W_stack[:, s * d:(s + 1) * d] for s in range(S)]


# ---------------------------------------------------------------- hash-collision study

def collision_study(V0: int = 131072, nseq: int = 100, seqlen: int = 8192, seed: int = 10,
                    lo: int = 30, hi: int = 33):
    """Inputs of the collision measurement of section 3.2.2 (Fig. 3b): 100 sequences of
    Zipf(1.1) ids over a 128K base vocabulary stand in for the pretraining sequences, and
    table sizes between 30x and 33x the base vocabulary, sampled densely around the integer
    multiples of V0 (offsets 0, +-1, +-8, +-64, +-1024) and every 3*V0/32 elsewhere.
    Returns (ids int32 [nseq, seqlen], sorted table sizes)."""
    rng = _rng(seed, 0)
    ids = zipf_ids(rng, V0, (nseq, seqlen))
    sizes = set()
    for m in range(lo, hi + 1):
        for off in (-1024, -64, -8, -1, 0, 1, 8, 64, 1024):
            v = m * V0 + off
            if lo * V0 <= v <= hi * V0:
                sizes.add(v)
    for k in range(0, 32 * (hi - lo) // 3 + 1):
        sizes.add(lo * V0 + k * 3 * V0 // 32)
    return ids, sorted(sizes)
