"""CPU oracle for the N-gram embedding forward pass.

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of
bench.py may import this module. The library (gram_embedding_layer_amd) never imports it and
shares no code, table or helper with it.

Source: the deep-notes page on "Scaling Embeddings Outperforms Scaling Experts in Language
Models" (Meituan LongCat team), section A2 "N-gram embedding layer":
  * the polynomial rolling hash  H_n(t_{i-n+1..i}) = (sum_{j=0}^{n-1} t_{i-j} * V0^j) mod V_n;
  * the final (Over-Encoding) form
        e_i = ( E_0(t_i) + sum_{n=2}^{N} sum_{k=1}^{K} W_{n,k} E_{n,k}(H_{n,k}(t_{i-n+1..i})) )
              / ((N-1)K + 1),
    with E_{n,k} in R^{V_{n,k} x D/((N-1)K)} and W_{n,k} in R^{D x D/((N-1)K)};
  * K hash functions per order that differ only in their modulus V_{n,k} (same section, and
    section 3.2.3 on K as the number of distinct hash functions).
Section 4.2 (N-gram cache) motivates the decode oracle; its semantics are a reading:
the cache holds committed ids, a decode step's outputs equal a prefill over the whole
history followed by the new ids, and a commit appends accepted ids.

The same section's basic form (Eq. 1), e_i = (E_0(t_i) + sum_{n=2}^{N} E_n(H_n(...))) / N with
one full-width table E_n in R^{V_n x D} per order and no projection: embed_basic(). Its hash
H_n is the rolling hash above with one modulus per order (hash_indices with K = 1);
backward_basic() gives its plain gradients.
Per-layer N-gram embedding (PLNE, section 5.2 of the same page): every layer l computes the
final form with tables and projections of its own; the oracle of layer l is prefill() with
layer l's parameters (no new arithmetic).
Hash collisions and vocabulary hit rate (section 3.2.2, Fig. 3): hash_slot_stats().

Readings where the pages are silent:
  * positions before a sequence's first token take the pad id 0, never ids of another
    sequence packed in the same batch;
  * sub-table order s = (n-2)*K + (k-1), n-major;
  * N = 1 has no sub-tables: e_i = E_0(t_i);
  * token ids must lie in [0, V0) (the hash reads them as base-V0 digits).

Backward (training, which the pages do but do not spell out): backward() gives the plain
gradients of the final form, duplicates accumulated.

Embedding amplification (section 3.2.4 of the same page, outside the final form itself):
amplify() applies the output scale or the layer normalisation the pages describe; the
reading of the latter is stated there.

Arithmetic: hashes are exact Python integers (the n-gram value is formed as a sum of powers,
not by Horner's rule, and reduced once); embeddings are computed in float64.
Parity pins: tests/test_oracle_pins.py. Nothing here is "parity unpinned".
"""
from __future__ import annotations

from typing import Callable, List, Sequence

import numpy as np

PAD_ID = 0


def num_subtables(N: int, K: int) -> int:
    """(N-1)K sub-tables: K for each order n = 2..N (section A2, final form)."""
    return (N - 1) * K


def subtable_order(N: int, K: int) -> List[tuple]:
    """(n, k) for s = 0..S-1, n-major."""
    return [(n, k) for n in range(2, N + 1) for k in range(1, K + 1)]


def check_config(V0: int, D: int, N: int, K: int, V: Sequence[int]) -> None:
    if N < 1 or K < 1 or V0 < 1 or D < 1:
        raise ValueError("N, K, V0 and D must be positive")
    S = num_subtables(N, K)
    if len(V) != S:
        raise ValueError(f"need {S} sub-table sizes, got {len(V)}")
    if any(int(v) < 1 for v in V):
        raise ValueError("sub-table sizes must be positive")
    if S and D % S:
        raise ValueError("D must be a multiple of (N-1)K (sub-table width D/((N-1)K))")


def context(seq: Sequence[int], i: int, n: int) -> List[int]:
    """[t_i, t_{i-1}, ..., t_{i-n+1}] of one sequence, pad id 0 before its start."""
    return [int(seq[i - j]) if i - j >= 0 else PAD_ID for j in range(n)]


def ngram_value(ctx: Sequence[int], n: int, V0: int) -> int:
    """sum_{j=0}^{n-1} t_{i-j} * V0^j as an unbounded integer (t_i is the lowest digit)."""
    return sum(int(ctx[j]) * V0 ** j for j in range(n))


def hash_indices(V0: int, N: int, K: int, V: Sequence[int], tokens: Sequence[int],
                 cu_seqlens: Sequence[int]) -> np.ndarray:
    """int64 [T, (N-1)K]: H_{n,k} of every position of every packed sequence.

    tokens: all sequences back to back; cu_seqlens: offsets [B+1], cu_seqlens[0] = 0."""
    S = num_subtables(N, K)
    tokens = [int(t) for t in tokens]
    T = len(tokens)
    if any(t < 0 or t >= V0 for t in tokens):
        raise ValueError("token id outside [0, V0)")
    if int(cu_seqlens[0]) != 0 or int(cu_seqlens[-1]) != T:
        raise ValueError("cu_seqlens must run from 0 to the token count")
    idx = np.zeros((T, S), dtype=np.int64)
    order = subtable_order(N, K)
    for b in range(len(cu_seqlens) - 1):
        lo, hi = int(cu_seqlens[b]), int(cu_seqlens[b + 1])
        if hi < lo:
            raise ValueError("cu_seqlens must be non-decreasing")
        seq = tokens[lo:hi]
        for i in range(hi - lo):
            ctx = context(seq, i, N)
            for s, (n, k) in enumerate(order):
                idx[lo + i, s] = ngram_value(ctx, n, V0) % int(V[s])
    return idx


RowFetch = Callable[[int, np.ndarray], np.ndarray]
"""fetch(s, rows) -> float array [len(rows), width]; s = -1 means E_0, else sub-table s."""


def embed_from_indices(D: int, N: int, K: int, tokens: Sequence[int], idx: np.ndarray,
                       fetch: RowFetch, W_blocks: Sequence[np.ndarray]) -> np.ndarray:
    """float64 [T, D]: the final form of section A2 given the hash indices.

    W_blocks[s] is W_{n,k} [D, d] for s = (n-2)K + (k-1)."""
    S = num_subtables(N, K)
    tok = np.asarray(tokens, dtype=np.int64)
    acc = np.asarray(fetch(-1, tok), dtype=np.float64).copy()              # E_0(t_i)
    if acc.shape != (len(tok), D):
        raise ValueError("E_0 rows must be [T, D]")
    for s in range(S):
        rows = np.asarray(fetch(s, idx[:, s]), dtype=np.float64)           # E_{n,k}(H_{n,k})
        Wnk = np.asarray(W_blocks[s], dtype=np.float64)                     # [D, d]
        if rows.shape[1] != D // S or Wnk.shape != (D, D // S):
            raise ValueError("sub-table rows must be [T, D/S] and W_{n,k} [D, D/S]")
        acc += rows @ Wnk.T                                                 # W_{n,k} E_{n,k}(.)
    return acc / float(S + 1)                                               # / ((N-1)K + 1)


def embed_basic(D: int, N: int, tokens: Sequence[int], idx: np.ndarray,
                fetch: RowFetch) -> np.ndarray:
    """float64 [T, D]: the basic N-gram embedding (section A2, Eq. 1) given the hash indices,
        e_i = ( E_0(t_i) + sum_{n=2}^{N} E_n(H_n(t_{i-n+1..i})) ) / N,
    with one full-width table E_n [V_n, D] per order and no projection. idx[:, n-2] holds
    H_n (hash_indices with K = 1); fetch(n-2, rows) reads E_n."""
    tok = np.asarray(tokens, dtype=np.int64)
    acc = np.asarray(fetch(-1, tok), dtype=np.float64).copy()              # E_0(t_i)
    if acc.shape != (len(tok), D):
        raise ValueError("E_0 rows must be [T, D]")
    for n in range(2, N + 1):
        rows = np.asarray(fetch(n - 2, idx[:, n - 2]), dtype=np.float64)   # E_n(H_n)
        if rows.shape != (len(tok), D):
            raise ValueError("basic-form tables have full rows [T, D]")
        acc += rows
    return acc / float(N)


def table_fetch(E0, E_list) -> RowFetch:
    """Row fetch over in-memory tables (numpy arrays or anything np.asarray accepts)."""
    E0 = np.asarray(E0, dtype=np.float64)
    E_list = [np.asarray(e, dtype=np.float64) for e in E_list]

    def fetch(s: int, rows: np.ndarray) -> np.ndarray:
        table = E0 if s < 0 else E_list[s]
        return table[np.asarray(rows, dtype=np.int64)]
    return fetch


def prefill(V0: int, D: int, N: int, K: int, V: Sequence[int], tokens: Sequence[int],
            cu_seqlens: Sequence[int], fetch: RowFetch, W_blocks: Sequence[np.ndarray]):
    """(idx int64 [T, S], e float64 [T, D]) for packed sequences."""
    check_config(V0, D, N, K, V)
    idx = hash_indices(V0, N, K, V, tokens, cu_seqlens)
    return idx, embed_from_indices(D, N, K, tokens, idx, fetch, W_blocks)


class DecodeOracle:
    """Decode with an N-gram cache, as plain bookkeeping over each sequence's full history.

    step(new) gives, for each sequence b, the indices and embeddings of the positions that
    `new[b]` would occupy after the history, as a prefill of history + new would.
    commit(new, n_accept) appends the first n_accept[b] of them to the history."""

    def __init__(self, V0: int, D: int, N: int, K: int, V: Sequence[int],
                 histories: Sequence[Sequence[int]]):
        check_config(V0, D, N, K, V)
        self.V0, self.D, self.N, self.K, self.V = V0, D, N, K, [int(v) for v in V]
        self.hist = [[int(t) for t in h] for h in histories]

    def step_indices(self, new: Sequence[Sequence[int]]) -> List[np.ndarray]:
        out = []
        order = subtable_order(self.N, self.K)
        for b, toks in enumerate(new):
            seq = self.hist[b] + [int(t) for t in toks]
            if any(t < 0 or t >= self.V0 for t in toks):
                raise ValueError("token id outside [0, V0)")
            base = len(self.hist[b])
            idx = np.zeros((len(toks), len(order)), dtype=np.int64)
            for j in range(len(toks)):
                ctx = context(seq, base + j, self.N)
                for s, (n, k) in enumerate(order):
                    idx[j, s] = ngram_value(ctx, n, self.V0) % self.V[s]
            out.append(idx)
        return out

    def step(self, new: Sequence[Sequence[int]], fetch: RowFetch,
             W_blocks: Sequence[np.ndarray]):
        idxs = self.step_indices(new)
        embs = [embed_from_indices(self.D, self.N, self.K, list(toks), idx, fetch, W_blocks)
                for toks, idx in zip(new, idxs)]
        return idxs, embs

    def commit(self, new: Sequence[Sequence[int]], n_accept: Sequence[int]) -> None:
        for b, toks in enumerate(new):
            a = int(n_accept[b])
            if a < 0 or a > len(toks):
                raise ValueError("n_accept outside [0, n_new]")
            self.hist[b].extend(int(t) for t in toks[:a])


AMP_MODES = ("none", "scale", "layernorm")


def amplify(e: np.ndarray, mode: str = "none", scale: float = 1.0, eps: float = 1e-5,
            weight=None, bias=None) -> np.ndarray:
    """Embedding amplification of section 3.2.4 of the deep-notes page ("effective training
    through embedding amplification"), applied to the layer output e [T, D] before it joins
    the residual stream. Two strategies are described there:
      * "scale": multiply the output by a factor (sqrt(D) in the pages);
      * "layernorm": layer normalisation over the hidden dimension D. The pages give no
        formula; the reading here is the usual one: per row, mean m and biased variance v of
        the D values, (e - m) / sqrt(v + eps), then the optional elementwise affine
        weight * x + bias (weight 1 and bias 0 when absent).
    float64 throughout."""
    e = np.asarray(e, dtype=np.float64)
    if mode == "none":
        return e.copy()
    if mode == "scale":
        return e * float(scale)
    if mode == "layernorm":
        if not eps > 0:
            raise ValueError("layernorm needs eps > 0")
        D = e.shape[-1]
        m = e.sum(axis=-1, keepdims=True) / D
        c = e - m
        v = (c * c).sum(axis=-1, keepdims=True) / D
        y = c / np.sqrt(v + float(eps))
        if weight is not None:
            y = y * np.asarray(weight, dtype=np.float64)
        if bias is not None:
            y = y + np.asarray(bias, dtype=np.float64)
        return y
    raise ValueError(f"amplification mode must be one of {AMP_MODES}")


def backward(D: int, N: int, K: int, tokens: Sequence[int], idx: np.ndarray, dout: np.ndarray,
             fetch: RowFetch, W_blocks: Sequence[np.ndarray], V0: int, V: Sequence[int],
             scale: float = 1.0):
    """Gradients of the final form (section A2) for one batch, float64.

    The pages train the model but give no backward; this is the plain reading: the layer is
    e_i = c (E_0(t_i) + sum_s W_s E_s(h_{i,s})) with c = scale / ((N-1)K + 1) (scale 1, or the
    amplification factor of section 3.2.4), so for the upstream gradient dout = dL/de [T, D]:
      dE_0[t]    = c * sum over positions i with t_i = t of dout_i,
      dW_s       = c * sum_i dout_i E_s(h_{i,s})^T                     ([D, d] each),
      dE_s[r]    = c * sum over positions i with h_{i,s} = r of W_s^T dout_i.
    Repeated ids and indices accumulate. Returns (dE0 [V0, D], [dE_s [V_s, d]], [dW_s])."""
    S = num_subtables(N, K)
    d = D // S if S else 0
    tok = np.asarray(tokens, dtype=np.int64)
    g = np.asarray(dout, dtype=np.float64)
    if g.shape != (len(tok), D):
        raise ValueError("dout must be [T, D]")
    c = float(scale) / float(S + 1)
    dE0 = np.zeros((V0, D))
    np.add.at(dE0, tok, c * g)                                      # E_0(t_i) appears once
    dE, dW = [], []
    for s in range(S):
        rows = np.asarray(fetch(s, idx[:, s]), dtype=np.float64)    # E_s(h_{i,s}) [T, d]
        Ws = np.asarray(W_blocks[s], dtype=np.float64)              # [D, d]
        dW.append(c * (g.T @ rows))                                 # sum_i dout_i rows_i^T
        grad_rows = c * (g @ Ws)                                    # W_s^T dout_i, [T, d]
        dEs = np.zeros((int(V[s]), d))
        np.add.at(dEs, np.asarray(idx[:, s], dtype=np.int64), grad_rows)
        dE.append(dEs)
    return dE0, dE, dW


def backward_basic(D: int, N: int, tokens: Sequence[int], idx: np.ndarray, dout: np.ndarray,
                   V0: int, V: Sequence[int], scale: float = 1.0):
    """Gradients of the basic form (section A2, Eq. 1) for one batch, float64: with
    e_i = c (E_0(t_i) + sum_n E_n(h_{i,n})), c = scale / N and dout = dL/de [T, D],
      dE_0[t] = c * sum over positions i with t_i = t of dout_i,
      dE_n[r] = c * sum over positions i with h_{i,n} = r of dout_i   (no projection).
    Returns (dE0 [V0, D], [dE_n [V_n, D] for n = 2..N])."""
    tok = np.asarray(tokens, dtype=np.int64)
    g = np.asarray(dout, dtype=np.float64)
    if g.shape != (len(tok), D):
        raise ValueError("dout must be [T, D]")
    c = float(scale) / float(N)
    dE0 = np.zeros((V0, D))
    np.add.at(dE0, tok, c * g)
    dE = []
    for n in range(2, N + 1):
        dEn = np.zeros((int(V[n - 2]), D))
        np.add.at(dEn, np.asarray(idx[:, n - 2], dtype=np.int64), c * g)
        dE.append(dEn)
    return dE0, dE


def param_count(V0: int, D: int, N: int, K: int, V: Sequence[int]) -> dict:
    """Parameter counts of the layer's tables (section A2: E_0, E_{n,k}, W_{n,k} shapes)."""
    S = num_subtables(N, K)
    d = D // S if S else 0
    return {"E0": V0 * D, "ngram_tables": sum(int(v) * d for v in V), "projections": S * D * d}


def hash_slot_stats(V0: int, n: int, tokens: Sequence[int], cu_seqlens: Sequence[int],
                    vocab_sizes: Sequence[int]):
    """Hash collisions of the n-gram hash (section 3.2.2 and Fig. 3 of the deep-notes page).

    Over every position of the packed sequences (the n-grams the layer hashes, pad id 0
    before a sequence's start), returns (distinct, slots): `distinct` is the number of
    different n-grams, and slots[v] the number of different table rows H_n = (n-gram value)
    mod vocab_sizes[v] that they occupy. The pages count collisions as the unique n-grams
    lost to the modulo (reading: distinct - slots) and the hit rate as the share of table
    rows used at least once (slots / V)."""
    tokens = [int(t) for t in tokens]
    if any(t < 0 or t >= V0 for t in tokens):
        raise ValueError("token id outside [0, V0)")
    if n < 1:
        raise ValueError("n must be positive")
    values = set()
    for b in range(len(cu_seqlens) - 1):
        seq = tokens[int(cu_seqlens[b]):int(cu_seqlens[b + 1])]
        for i in range(len(seq)):
            values.add(ngram_value(context(seq, i, n), n, V0))
    slots = [len({x % int(V) for x in values}) for V in vocab_sizes]
    return len(values), slots
