"""Pins of the CPU oracle to facts fixed by the pages and by mathematics, not by itself.

Hash (section A2, polynomial rolling hash): hand-worked values, decimal and binary digit
strings, an exhaustive base-7 count, Horner's rule as an independent algorithm, the pad
convention at sequence starts, and packing independence.
Final form (section A2): hand-worked rational values, special cases that reduce to plain
indexing (N = 1, identity and zero projections), the stacked-matrix form, linearity,
locality, the parameter-count identity, and decode == prefill.
test_pins_catch_planted_mistakes plants plausible mistakes in the oracle and checks that
these pins fail.
"""
import json
import os
from collections import Counter
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from oracle import ngram_oracle as O
from workloads import cu_seqlens_from_lengths

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _one_seq(tokens):
    return [0, len(tokens)]


# ------------------------------------------------------------------ hash

def check_hash_golden():
    g = _load("hash_handworked_v1000.json")
    idx = oracle.hash_indices(g["V0"], g["N"], g["K"], g["V"], g["tokens"], _one_seq(g["tokens"]))
    np.testing.assert_array_equal(idx, np.array(g["idx"]))


def test_hash_handworked_v1000():
    check_hash_golden()


def _digits_to_int(digits, base):
    """Most significant digit first; uses Python's own base parser (no arithmetic of ours)."""
    alphabet = "0123456789abcdefghijklmnopqrstuvwxyz"
    return int("".join(alphabet[d] for d in digits), base)


def check_hash_decimal():
    # V0 = 10: the n-gram ending at t_i is the decimal number t_{i-n+1} ... t_{i-1} t_i.
    rng = np.random.default_rng(1)
    seq = [int(x) for x in rng.integers(0, 10, size=40)]
    seq[10:13] = [3, 1, 4]
    N, K = 4, 1
    V = [10 ** n + 7 for n in range(2, N + 1)]      # larger than any n-digit value
    idx = oracle.hash_indices(10, N, K, V, seq, _one_seq(seq))
    assert idx[12, 1] == 314                         # 3-gram (3, 1, 4)
    for i in range(len(seq)):
        for n in range(2, N + 1):
            window = [seq[i - j] if i - j >= 0 else 0 for j in range(n - 1, -1, -1)]
            assert idx[i, n - 2] == _digits_to_int(window, 10) % V[n - 2]


def test_hash_decimal_digits():
    check_hash_decimal()


def test_hash_power_of_two_base_is_bit_packing():
    bits, N, K = 5, 4, 2
    V0 = 1 << bits
    V = [(1 << 40) + 15, (1 << 40) + 21, (1 << 40) + 31, (1 << 40) + 33, 97, 101]
    rng = np.random.default_rng(2)
    seq = [int(x) for x in rng.integers(0, V0, size=30)]
    idx = oracle.hash_indices(V0, N, K, V, seq, _one_seq(seq))
    for i in range(len(seq)):
        for s, (n, k) in enumerate(oracle.subtable_order(N, K)):
            x = 0
            for j in range(n):
                if i - j >= 0:
                    x |= seq[i - j] << (bits * j)
            assert idx[i, s] == x % V[s]


def test_hash_exhaustive_base7_trigrams():
    # All 343 trigrams over V0 = 7 as separate length-3 sequences: with a large modulus the
    # 3-gram index is the base-7 number (a bijection onto 0..342); with modulus 13 the bucket
    # counts equal a direct count.
    trigrams = [(a, b, c) for a in range(7) for b in range(7) for c in range(7)]
    tokens = [t for tri in trigrams for t in tri]
    cu = cu_seqlens_from_lengths([3] * len(trigrams))
    idx = oracle.hash_indices(7, 3, 1, [101, 1000], tokens, cu)
    last = idx[2::3, 1]
    assert sorted(last.tolist()) == list(range(343))
    for tri, v in zip(trigrams, last):
        assert v == _digits_to_int(list(tri), 7)
    idx13 = oracle.hash_indices(7, 3, 1, [101, 13], tokens, cu)[2::3, 1]
    direct = Counter(_digits_to_int(list(tri), 7) % 13 for tri in trigrams)
    assert Counter(idx13.tolist()) == direct


def _horner_mod(ctx_oldest_first, V0, m):
    x = 0
    for t in ctx_oldest_first:
        x = (x * V0 + t) % m
    return x


@settings(max_examples=60, deadline=None)
@given(V0=st.integers(2, 300), N=st.integers(1, 5), K=st.integers(1, 4),
       data=st.data())
def test_hash_matches_horner(V0, N, K, data):
    S = (N - 1) * K
    V = data.draw(st.lists(st.integers(1, 5000), min_size=S, max_size=S))
    lengths = data.draw(st.lists(st.integers(0, 9), min_size=1, max_size=4))
    tokens = data.draw(st.lists(st.integers(0, V0 - 1), min_size=sum(lengths),
                                max_size=sum(lengths)))
    cu = cu_seqlens_from_lengths(lengths)
    idx = oracle.hash_indices(V0, N, K, V, tokens, cu)
    assert idx.shape == (len(tokens), S)
    for b in range(len(lengths)):
        lo = cu[b]
        for i in range(lengths[b]):
            for s, (n, k) in enumerate(oracle.subtable_order(N, K)):
                ctx = [tokens[lo + i - j] if i - j >= 0 else 0 for j in range(n - 1, -1, -1)]
                assert idx[lo + i, s] == _horner_mod(ctx, V0, V[s])


def test_hash_sequence_start_uses_pad_zero():
    V0, N, K, V = 50, 4, 2, [7, 11, 13, 17, 19, 23]
    seqs = [[9, 3, 48], [1], [0, 0, 5, 7, 49]]
    cu = cu_seqlens_from_lengths([len(s) for s in seqs])
    idx = oracle.hash_indices(V0, N, K, V, sum(seqs, []), cu)
    for b, seq in enumerate(seqs):
        first = idx[cu[b]]
        # every n-gram at position 0 is (pad, ..., pad, t_0) = t_0
        assert first.tolist() == [seq[0] % v for v in V]


def test_hash_packing_independence():
    V0, N, K, V = 1000, 3, 2, [5003, 7001, 6007, 8009]
    rng = np.random.default_rng(3)
    seqs = [[int(x) for x in rng.integers(0, V0, size=L)] for L in (5, 1, 12, 0, 3)]
    cu = cu_seqlens_from_lengths([len(s) for s in seqs])
    packed = oracle.hash_indices(V0, N, K, V, sum(seqs, []), cu)
    for b, seq in enumerate(seqs):
        alone = oracle.hash_indices(V0, N, K, V, seq, _one_seq(seq))
        np.testing.assert_array_equal(packed[cu[b]:cu[b + 1]], alone)


def test_hash_rejects_bad_ids():
    with pytest.raises(ValueError):
        oracle.hash_indices(10, 2, 1, [7], [3, 10], [0, 2])
    with pytest.raises(ValueError):
        oracle.hash_indices(10, 2, 1, [7], [3, -1], [0, 2])


# ------------------------------------------------------------------ final form

def _case_arrays(c):
    E0 = np.array(c["E0"], dtype=np.float64)
    E = [np.array(e, dtype=np.float64) for e in c["E"]]
    W = [np.array(w, dtype=np.float64) for w in c["W"]]
    return E0, E, W


def check_embed_golden():
    g = _load("embed_handworked_small.json")
    for c in g["cases"]:
        E0, E, W = _case_arrays(c)
        idx, e = oracle.prefill(c["V0"], c["D"], c["N"], c["K"], c["V"], c["tokens"],
                                _one_seq(c["tokens"]), oracle.table_fetch(E0, E), W)
        np.testing.assert_array_equal(idx, np.array(c["idx"]))
        want = np.array([[float(Fraction(p, q)) for p, q in row] for row in c["e"]])
        np.testing.assert_allclose(e, want, rtol=0, atol=1e-14)


def test_embed_handworked():
    check_embed_golden()


def _random_case(rng, V0=40, D=24, N=3, K=2, lengths=(7, 1, 5)):
    S = (N - 1) * K
    d = D // S if S else 0
    V = [int(v) for v in rng.integers(3, 200, size=S)]
    E0 = rng.standard_normal((V0, D))
    E = [rng.standard_normal((v, d)) for v in V]
    W = [rng.standard_normal((D, d)) for _ in range(S)]
    tokens = [int(x) for x in rng.integers(0, V0, size=sum(lengths))]
    return V0, D, N, K, V, E0, E, W, tokens, cu_seqlens_from_lengths(lengths)


def test_embed_N1_is_plain_lookup():
    rng = np.random.default_rng(4)
    E0 = rng.standard_normal((30, 8))
    tokens = [int(x) for x in rng.integers(0, 30, size=17)]
    idx, e = oracle.prefill(30, 8, 1, 3, [], tokens, [0, 17], oracle.table_fetch(E0, []), [])
    assert idx.shape == (17, 0)
    np.testing.assert_array_equal(e, np.take(E0, tokens, axis=0))


def test_embed_identity_projection_is_concatenation():
    # W_{n,k} = the s-th column block of I_D: the final form becomes
    # (E_0[t] + [E_s[idx_s] for s in order]) / (S+1), pure indexing (exact in float64).
    rng = np.random.default_rng(5)
    V0, D, N, K, V, E0, E, _, tokens, cu = _random_case(rng, D=24, N=4, K=2)
    S, d = (N - 1) * K, D // ((N - 1) * K)
    I = np.eye(D)
    W = [I[:, s * d:(s + 1) * d] for s in range(S)]
    idx, e = oracle.prefill(V0, D, N, K, V, tokens, cu, oracle.table_fetch(E0, E), W)
    concat = np.concatenate([np.take(E[s], idx[:, s], axis=0) for s in range(S)], axis=1)
    np.testing.assert_array_equal(e, (np.take(E0, tokens, axis=0) + concat) / (S + 1))


def test_embed_zero_projection():
    rng = np.random.default_rng(6)
    V0, D, N, K, V, E0, E, W, tokens, cu = _random_case(rng)
    W = [np.zeros_like(w) for w in W]
    _, e = oracle.prefill(V0, D, N, K, V, tokens, cu, oracle.table_fetch(E0, E), W)
    np.testing.assert_array_equal(e, np.take(E0, tokens, axis=0) / ((N - 1) * K + 1))


def test_embed_equals_stacked_matrix_form():
    # sum_s W_{n,k} row_s == [W_{2,1} | W_{2,2} | ...] @ concat(row_s)
    rng = np.random.default_rng(7)
    V0, D, N, K, V, E0, E, W, tokens, cu = _random_case(rng, D=32, N=5, K=2)
    S = (N - 1) * K
    idx, e = oracle.prefill(V0, D, N, K, V, tokens, cu, oracle.table_fetch(E0, E), W)
    g = np.concatenate([E[s][idx[:, s]] for s in range(S)], axis=1)
    stacked = np.concatenate(W, axis=1)
    np.testing.assert_allclose(e, (E0[tokens] + g @ stacked.T) / (S + 1), rtol=1e-12, atol=1e-12)


def test_embed_linearity_exact():
    rng = np.random.default_rng(8)
    V0, D, N, K, V, E0, E, W, tokens, cu = _random_case(rng)
    _, e1 = oracle.prefill(V0, D, N, K, V, tokens, cu, oracle.table_fetch(E0, E), W)
    _, e2 = oracle.prefill(V0, D, N, K, V, tokens, cu,
                           oracle.table_fetch(2 * E0, [2 * x for x in E]), W)
    np.testing.assert_array_equal(e2, 2 * e1)


def test_embed_locality():
    # Changing t_j may change only e_j .. e_{j+N-1} of the same sequence, and changes e_j.
    rng = np.random.default_rng(9)
    V0, D, N, K, V, E0, E, W, tokens, cu = _random_case(rng, N=3, lengths=(12, 9))
    fetch = oracle.table_fetch(E0, E)
    _, base = oracle.prefill(V0, D, N, K, V, tokens, cu, fetch, W)
    for j in (0, 4, 11, 12, 15):
        t2 = list(tokens)
        t2[j] = (t2[j] + 1) % V0
        _, e = oracle.prefill(V0, D, N, K, V, t2, cu, fetch, W)
        changed = np.nonzero(np.any(e != base, axis=1))[0].tolist()
        seq_end = 12 if j < 12 else 21
        allowed = set(range(j, min(j + N, seq_end)))
        assert set(changed) <= allowed and j in changed


def test_param_count_invariant_in_N_and_K():
    # Sub-table width D/((N-1)K): with every V_{n,k} = V the n-gram tables hold V*D
    # parameters and the projections D*D, whatever N and K (section A2).
    D, V = 240, 1009
    for N in range(2, 7):
        for K in range(1, 6):
            S = (N - 1) * K
            if D % S:
                continue
            pc = oracle.param_count(100, D, N, K, [V] * S)
            assert pc["ngram_tables"] == V * D
            assert pc["projections"] == D * D
            assert pc["E0"] == 100 * D


# ------------------------------------------------------------------ decode

def test_decode_equals_prefill():
    rng = np.random.default_rng(10)
    V0, D, N, K, V, E0, E, W, _, _ = _random_case(rng, N=4, K=1, D=12)
    fetch = oracle.table_fetch(E0, E)
    full = [[int(x) for x in rng.integers(0, V0, size=L)] for L in (14, 2, 9)]
    hist_len = [5, 0, 1]
    dec = oracle.DecodeOracle(V0, D, N, K, V, [f[:h] for f, h in zip(full, hist_len)])
    pos = list(hist_len)
    want = [oracle.prefill(V0, D, N, K, V, f, _one_seq(f), fetch, W) for f in full]
    while any(p < len(f) for p, f in zip(pos, full)):
        take = [min(int(rng.integers(1, 6)), len(f) - p) for p, f in zip(pos, full)]
        new = [f[p:p + t] for f, p, t in zip(full, pos, take)]
        idxs, embs = dec.step(new, fetch, W)
        for b in range(3):
            np.testing.assert_array_equal(idxs[b], want[b][0][pos[b]:pos[b] + take[b]])
            np.testing.assert_allclose(embs[b], want[b][1][pos[b]:pos[b] + take[b]],
                                       rtol=0, atol=1e-13)
        # accept a prefix only, then re-propose the rest: rejected drafts leave no trace
        acc = [int(rng.integers(0, t + 1)) for t in take]
        dec.commit(new, acc)
        pos = [p + a for p, a in zip(pos, acc)]


def test_decode_handworked():
    g = _load("embed_handworked_small.json")
    c = [c for c in g["cases"] if c["name"] == "N3_K1"][0]
    E0, E, W = _case_arrays(c)
    dec = oracle.DecodeOracle(c["V0"], c["D"], c["N"], c["K"], c["V"], [c["tokens"][:1]])
    idxs, embs = dec.step([c["tokens"][1:]], oracle.table_fetch(E0, E), W)
    np.testing.assert_array_equal(idxs[0], np.array(c["idx"][1:]))
    want = np.array([[float(Fraction(p, q)) for p, q in row] for row in c["e"][1:]])
    np.testing.assert_allclose(embs[0], want, rtol=0, atol=1e-14)


# ------------------------------------------------------------------ planted mistakes

def _fails(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


@pytest.mark.parametrize("mistake", ["digits_reversed", "drop_high_digit", "norm_over_N",
                                     "drop_E0", "no_pad", "transpose_W"])
def test_pins_catch_planted_mistakes(monkeypatch, mistake):
    if mistake == "digits_reversed":
        monkeypatch.setattr(O, "ngram_value",
                            lambda ctx, n, V0: sum(int(ctx[n - 1 - j]) * V0 ** j for j in range(n)))
    elif mistake == "drop_high_digit":
        monkeypatch.setattr(O, "ngram_value",
                            lambda ctx, n, V0: sum(int(ctx[j]) * V0 ** j for j in range(n - 1)))
    elif mistake == "no_pad":
        monkeypatch.setattr(O, "context",
                            lambda seq, i, n: [int(seq[(i - j) % len(seq)]) for j in range(n)])
    else:
        real = O.embed_from_indices

        def planted(D, N, K, tokens, idx, fetch, W_blocks):
            S = (N - 1) * K
            if mistake == "norm_over_N":
                return real(D, N, K, tokens, idx, fetch, W_blocks) * (S + 1) / N
            if mistake == "drop_E0":
                zero = lambda s, rows: (np.zeros((len(rows), D)) if s < 0 else fetch(s, rows))
                return real(D, N, K, tokens, idx, zero, W_blocks)
            if mistake == "transpose_W":
                Wt = [np.asarray(w)[::-1] for w in W_blocks]
                return real(D, N, K, tokens, idx, fetch, Wt)
            raise AssertionError
        # oracle.prefill resolves embed_from_indices in its module at call time
        monkeypatch.setattr(O, "embed_from_indices", planted)
    if mistake in ("digits_reversed", "drop_high_digit", "no_pad"):
        assert _fails(check_hash_golden) or _fails(check_hash_decimal)
    else:
        assert _fails(check_embed_golden)


# ------------------------------------------------------------------ embedding amplification
# Section 3.2.4 of the deep-notes page: the output scaled (by sqrt(D)) or layer-normalised
# before it joins the residual stream. The layer normalisation is pinned to closed forms
# worked by hand, to its defining invariants and to torch's own layer_norm.

def check_layernorm_closed_form():
    e = np.array([[1.0, 2.0, 3.0, 4.0]])
    r5 = np.sqrt(5.0)
    # mean 5/2 and biased variance 5/4, so (e - 5/2) / sqrt(5/4) = (2e - 5) / sqrt(5)
    np.testing.assert_allclose(O.amplify(e, "layernorm", eps=1e-300),
                               [[-3 / r5, -1 / r5, 1 / r5, 3 / r5]], rtol=1e-12)
    # eps = 3/4 makes the denominator sqrt(5/4 + 3/4) = sqrt(2)
    np.testing.assert_allclose(O.amplify(e, "layernorm", eps=0.75),
                               [[-1.5 / np.sqrt(2), -0.5 / np.sqrt(2), 0.5 / np.sqrt(2),
                                 1.5 / np.sqrt(2)]], rtol=1e-12)
    # elementwise affine: weight * x + bias
    w, b = np.array([2.0, 0.0, -1.0, 1.0]), np.array([0.0, 1.0, 0.0, -3.0])
    np.testing.assert_allclose(O.amplify(e, "layernorm", eps=0.75, weight=w, bias=b),
                               [[-3 / np.sqrt(2), 1.0, -0.5 / np.sqrt(2), 1.5 / np.sqrt(2) - 3]],
                               rtol=1e-12)
    # a constant row has zero variance: the output is the bias alone
    np.testing.assert_allclose(O.amplify(np.full((1, 4), 7.0), "layernorm", eps=1e-5, bias=b),
                               [b], rtol=0, atol=1e-12)


def test_layernorm_closed_form():
    check_layernorm_closed_form()


def test_layernorm_invariants_and_library():
    import torch
    rng = np.random.default_rng(11)
    e = rng.normal(0.3, 0.02, size=(9, 96))
    y = O.amplify(e, "layernorm", eps=1e-300)
    np.testing.assert_allclose(y.mean(axis=1), 0, atol=1e-12)
    np.testing.assert_allclose((y * y).mean(axis=1), 1, rtol=1e-10)
    # shift and positive scale invariance of the normalised rows
    np.testing.assert_allclose(O.amplify(5 * e - 2, "layernorm", eps=1e-300), y, atol=1e-10)
    w, b = rng.normal(size=96), rng.normal(size=96)
    want = torch.nn.functional.layer_norm(torch.tensor(e), (96,), torch.tensor(w),
                                          torch.tensor(b), eps=1e-5).numpy()
    np.testing.assert_allclose(O.amplify(e, "layernorm", eps=1e-5, weight=w, bias=b), want,
                               rtol=1e-12, atol=1e-12)


def test_scale_amplification():
    rng = np.random.default_rng(12)
    e = rng.normal(size=(5, 16))
    np.testing.assert_array_equal(O.amplify(e, "scale", 4.0), 4.0 * e)
    np.testing.assert_array_equal(O.amplify(e, "scale", 1.0), e)
    np.testing.assert_array_equal(O.amplify(e, "none"), e)
    with pytest.raises(ValueError):
        O.amplify(e, "rms")


@pytest.mark.parametrize("mistake", ["unbiased_var", "eps_outside_sqrt", "no_center",
                                     "affine_swapped"])
def test_layernorm_pins_catch_planted_mistakes(monkeypatch, mistake):
    def planted(e, mode="none", scale=1.0, eps=1e-5, weight=None, bias=None):
        e = np.asarray(e, dtype=np.float64)
        D = e.shape[-1]
        m = e.mean(axis=-1, keepdims=True)
        c = e - m
        if mistake == "no_center":
            c = e
        v = (c * c).sum(axis=-1, keepdims=True) / (D - 1 if mistake == "unbiased_var" else D)
        y = c / (np.sqrt(v) + eps) if mistake == "eps_outside_sqrt" else c / np.sqrt(v + eps)
        w = np.ones(D) if weight is None else np.asarray(weight, dtype=np.float64)
        b = np.zeros(D) if bias is None else np.asarray(bias, dtype=np.float64)
        return y * b + w if mistake == "affine_swapped" else y * w + b
    monkeypatch.setattr(O, "amplify", planted)
    assert _fails(check_layernorm_closed_form)


# ------------------------------------------------------------------ backward (training)
# The gradients of the final form, pinned to the oracle's own forward by finite differences:
# L = sum(dout * e) is linear in E_0, in each E_s and in each W_s, so a central difference in
# float64 is exact up to rounding, whatever the step.

def _bw_case(seed=3, V0=9, D=12, N=3, K=2, lengths=(7, 1, 6)):
    rng = np.random.default_rng(seed)
    S = (N - 1) * K
    d = D // S
    V = [5, 7, 6, 11][:S]
    seqs = [rng.integers(0, V0, size=L) for L in lengths]
    tokens = np.concatenate(seqs)
    cu = cu_seqlens_from_lengths(lengths)
    E0 = rng.normal(size=(V0, D))
    E = [rng.normal(size=(V[s], d)) for s in range(S)]
    Wb = [rng.normal(size=(D, d)) for _ in range(S)]
    dout = rng.normal(size=(len(tokens), D))
    return dict(V0=V0, D=D, N=N, K=K, V=V, tokens=tokens, cu=cu, E0=E0, E=E, W=Wb, dout=dout)


def _loss(c, E0, E, Wb, scale):
    idx = O.hash_indices(c["V0"], c["N"], c["K"], c["V"], c["tokens"], c["cu"])
    e = O.embed_from_indices(c["D"], c["N"], c["K"], c["tokens"], idx, O.table_fetch(E0, E), Wb)
    return float(np.sum(c["dout"] * e * scale))


def check_backward_fd(scale=1.0):
    c = _bw_case()
    idx = O.hash_indices(c["V0"], c["N"], c["K"], c["V"], c["tokens"], c["cu"])
    dE0, dE, dW = O.backward(c["D"], c["N"], c["K"], c["tokens"], idx, c["dout"],
                             O.table_fetch(c["E0"], c["E"]), c["W"], c["V0"], c["V"], scale)
    rng = np.random.default_rng(4)
    h = 0.5

    def fd(kind, s, pos):
        def shifted(delta):
            E0, E, Wb = c["E0"].copy(), [e.copy() for e in c["E"]], [w.copy() for w in c["W"]]
            tgt = E0 if kind == "E0" else (E[s] if kind == "E" else Wb[s])
            tgt[pos] += delta
            return _loss(c, E0, E, Wb, scale)
        return (shifted(h) - shifted(-h)) / (2 * h)

    for _ in range(12):
        pos = (int(rng.integers(c["V0"])), int(rng.integers(c["D"])))
        np.testing.assert_allclose(dE0[pos], fd("E0", None, pos), rtol=1e-9, atol=1e-9)
    for s in range(len(c["E"])):
        for _ in range(6):
            pos = (int(rng.integers(c["V"][s])), int(rng.integers(c["D"] // len(c["E"]))))
            np.testing.assert_allclose(dE[s][pos], fd("E", s, pos), rtol=1e-9, atol=1e-9)
            pos = (int(rng.integers(c["D"])), int(rng.integers(c["D"] // len(c["E"]))))
            np.testing.assert_allclose(dW[s][pos], fd("W", s, pos), rtol=1e-9, atol=1e-9)


def test_backward_matches_finite_differences():
    check_backward_fd()
    check_backward_fd(scale=np.sqrt(12.0))


def test_backward_identity_projection_closed_form():
    """N = 2, K = 1 (S = 1, d = D) with W = I: dE_1[h] and dE_0[t] are the scattered sums of
    dout / 2, and dW = (1/2) sum_i dout_i E_1(h_i)^T."""
    rng = np.random.default_rng(8)
    V0, D, V = 5, 4, [3]
    tokens = np.array([1, 1, 4, 1, 0, 2])
    cu = np.array([0, 6])
    idx = O.hash_indices(V0, 2, 1, V, tokens, cu)
    E1 = rng.normal(size=(3, D))
    dout = rng.normal(size=(6, D))
    dE0, dE, dW = O.backward(D, 2, 1, tokens, idx, dout, O.table_fetch(np.zeros((V0, D)), [E1]),
                             [np.eye(D)], V0, V)
    want0 = np.zeros((V0, D))
    want1 = np.zeros((3, D))
    wantW = np.zeros((D, D))
    for i in range(6):
        want0[tokens[i]] += dout[i] / 2
        want1[idx[i, 0]] += dout[i] / 2
        wantW += np.outer(dout[i], E1[idx[i, 0]]) / 2
    np.testing.assert_allclose(dE0, want0, atol=1e-15)
    np.testing.assert_allclose(dE[0], want1, atol=1e-15)
    np.testing.assert_allclose(dW[0], wantW, atol=1e-14)
    # token 1 appears three times: its gradient row is the sum of three upstream rows
    np.testing.assert_allclose(dE0[1], (dout[0] + dout[1] + dout[3]) / 2, atol=1e-15)


@pytest.mark.parametrize("mistake", ["no_scale", "W_rows_flipped", "overwrite_duplicates"])
def test_backward_pins_catch_planted_mistakes(monkeypatch, mistake):
    real = O.backward

    def planted(D, N, K, tokens, idx, dout, fetch, W_blocks, V0, V, scale=1.0):
        S = (N - 1) * K
        if mistake == "no_scale":
            return real(D, N, K, tokens, idx, dout, fetch, W_blocks, V0, V, scale * (S + 1))
        if mistake == "W_rows_flipped":
            return real(D, N, K, tokens, idx, dout, fetch,
                        [np.asarray(w)[::-1] for w in W_blocks], V0, V, scale)
        dE0, dE, dW = real(D, N, K, tokens, idx, dout, fetch, W_blocks, V0, V, scale)
        c = scale / (S + 1)
        dE0 = np.zeros_like(dE0)
        dE0[np.asarray(tokens)] = c * np.asarray(dout)       # last write wins: no accumulation
        return dE0, dE, dW
    monkeypatch.setattr(O, "backward", planted)
    assert _fails(check_backward_fd)
