"""Pins of the oracle's variants of the layer to facts fixed by the pages and by mathematics.

Basic form (section A2, Eq. 1: full-width tables, no projection, divided by N): hand-worked
rational values, N = 1, the special case N = 2 where the final form with K = 1 and an
identity projection is the same layer, linearity, and planted mistakes; its backward
against finite differences and the final form's backward in that special case.
Hash collisions and hit counts (section 3.2.2, Fig. 3): hand-worked counts, brute force over
context tuples, the closed form at table sizes that are multiples of V0 (the spikes of
Fig. 3b), sizes above every n-gram value, and planted mistakes.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import ngram_oracle as O
from workloads import cu_seqlens_from_lengths

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _fails(check):
    try:
        check()
    except (AssertionError, IndexError, ValueError):
        return True
    return False


# ------------------------------------------------------------------ basic form (Eq. 1)

def basic_prefill(V0, D, N, V, tokens, cu, fetch):
    idx = oracle.hash_indices(V0, N, 1, V, tokens, cu)
    return idx, O.embed_basic(D, N, tokens, idx, fetch)


def check_basic_golden():
    g = _load("basic_form_handworked.json")
    for c in g["cases"]:
        fetch = oracle.table_fetch(np.array(c["E0"], float), [np.array(e, float) for e in c["E"]])
        idx, e = basic_prefill(c["V0"], c["D"], c["N"], c["V"], c["tokens"], c["cu_seqlens"],
                               fetch)
        np.testing.assert_array_equal(idx, np.array(c["idx"]))
        want = np.array([[float(Fraction(p, q)) for p, q in row] for row in c["e"]])
        np.testing.assert_allclose(e, want, rtol=0, atol=1e-13)


def test_basic_form_handworked():
    check_basic_golden()


def _basic_case(rng, V0=30, D=12, N=4, lengths=(6, 1, 9)):
    V = [int(v) for v in rng.integers(3, 90, size=N - 1)]
    E0 = rng.standard_normal((V0, D))
    E = [rng.standard_normal((v, D)) for v in V]
    tokens = [int(x) for x in rng.integers(0, V0, size=sum(lengths))]
    return V0, D, N, V, E0, E, tokens, cu_seqlens_from_lengths(lengths)


def test_basic_form_N1_is_lookup():
    rng = np.random.default_rng(2)
    E0 = rng.standard_normal((20, 8))
    tokens = [3, 19, 0, 3]
    _, e = basic_prefill(20, 8, 1, [], tokens, [0, 4], oracle.table_fetch(E0, []))
    np.testing.assert_array_equal(e, E0[tokens])


def test_basic_form_N2_equals_final_form_with_identity_projection():
    """With N = 2 and K = 1 the final form has one sub-table of full width D; with W = I it
    is the basic form (both divide by 2)."""
    rng = np.random.default_rng(3)
    V0, D, N, V, E0, E, tokens, cu = _basic_case(rng, N=2)
    fetch = oracle.table_fetch(E0, E)
    idx, e = basic_prefill(V0, D, N, V, tokens, cu, fetch)
    idx3, e3 = oracle.prefill(V0, D, 2, 1, V, tokens, cu, fetch, [np.eye(D)])
    np.testing.assert_array_equal(idx, idx3)
    np.testing.assert_allclose(e, e3, rtol=0, atol=1e-14)


def test_basic_form_linearity_and_mean():
    rng = np.random.default_rng(4)
    V0, D, N, V, E0, E, tokens, cu = _basic_case(rng)
    _, e = basic_prefill(V0, D, N, V, tokens, cu, oracle.table_fetch(E0, E))
    _, e2 = basic_prefill(V0, D, N, V, tokens, cu,
                          oracle.table_fetch(3 * E0, [3 * t for t in E]))
    np.testing.assert_allclose(e2, 3 * e, rtol=1e-13, atol=1e-14)
    # all tables constant c: the output is the mean of N copies of c
    c = rng.standard_normal(D)
    ones = lambda r: np.tile(c, (r, 1))
    _, ec = basic_prefill(V0, D, N, V, tokens, cu,
                          oracle.table_fetch(ones(V0), [ones(v) for v in V]))
    np.testing.assert_allclose(ec, np.tile(c, (len(tokens), 1)), rtol=1e-14)


@pytest.mark.parametrize("mistake", ["norm_over_N_minus_1", "drop_E0", "orders_swapped"])
def test_basic_pins_catch_planted_mistakes(monkeypatch, mistake):
    real = O.embed_basic

    def planted(D, N, tokens, idx, fetch):
        if mistake == "norm_over_N_minus_1":
            return real(D, N, tokens, idx, fetch) * N / max(N - 1, 1)
        if mistake == "drop_E0":
            zero = lambda s, rows: (np.zeros((len(rows), D)) if s < 0 else fetch(s, rows))
            return real(D, N, tokens, idx, zero)
        swapped = lambda s, rows: fetch(s if s < 0 else N - 2 - s, rows)
        return real(D, N, tokens, idx, swapped)
    monkeypatch.setattr(O, "embed_basic", planted)
    assert _fails(check_basic_golden)


def check_basic_backward():
    """Directional finite differences of L = <dout, e> through embed_basic (exact for a
    linear map, up to rounding), and the final form's backward with N = 2, K = 1, W = I."""
    rng = np.random.default_rng(8)
    V0, D, N, V, E0, E, tokens, cu = _basic_case(rng, V0=9, N=4, lengths=(30, 2, 11))
    idx = oracle.hash_indices(V0, N, 1, V, tokens, cu)
    dout = rng.standard_normal((len(tokens), D))
    scale = 1.7
    dE0, dE = O.backward_basic(D, N, tokens, idx, dout, V0, V, scale)

    def loss(E0_, E_):
        return float((dout * scale * O.embed_basic(D, N, tokens, idx,
                                                   oracle.table_fetch(E0_, E_))).sum())
    P0 = rng.standard_normal(E0.shape)
    P = [rng.standard_normal(e.shape) for e in E]
    h = 1e-3
    fd = (loss(E0 + h * P0, [e + h * p for e, p in zip(E, P)]) -
          loss(E0 - h * P0, [e - h * p for e, p in zip(E, P)])) / (2 * h)
    an = float((dE0 * P0).sum() + sum((g * p).sum() for g, p in zip(dE, P)))
    assert abs(fd - an) <= 1e-8 * max(1.0, abs(an)), (fd, an)
    # per table, not only in sum: each table alone
    for n in range(N - 1):
        Pn = [np.zeros_like(e) for e in E]
        Pn[n] = P[n]
        fdn = (loss(E0, [e + h * p for e, p in zip(E, Pn)]) -
               loss(E0, [e - h * p for e, p in zip(E, Pn)])) / (2 * h)
        assert abs(fdn - float((dE[n] * P[n]).sum())) <= 1e-8 * max(1.0, abs(fdn)), n
    # N = 2: the final form with K = 1 and W = I has the same table gradients
    V0, D, N, V, E0, E, tokens, cu = _basic_case(rng, V0=9, N=2, lengths=(25,))
    idx = oracle.hash_indices(V0, 2, 1, V, tokens, cu)
    dout = rng.standard_normal((len(tokens), D))
    a0, a = O.backward_basic(D, 2, tokens, idx, dout, V0, V, scale)
    b0, b, _ = oracle.backward(D, 2, 1, tokens, idx, dout, oracle.table_fetch(E0, E),
                               [np.eye(D)], V0, V, scale)
    np.testing.assert_allclose(a0, b0, rtol=0, atol=1e-13)
    np.testing.assert_allclose(a[0], b[0], rtol=0, atol=1e-13)


def test_basic_backward():
    check_basic_backward()


@pytest.mark.parametrize("mistake", ["norm_over_N_minus_1", "orders_swapped", "no_repeats"])
def test_basic_backward_pins_catch_planted_mistakes(monkeypatch, mistake):
    real = O.backward_basic

    def planted(D, N, tokens, idx, dout, V0, V, scale=1.0):
        if mistake == "norm_over_N_minus_1":
            return real(D, N, tokens, idx, dout, V0, V, scale * N / max(N - 1, 1))
        if mistake == "orders_swapped":
            dE0, dE = real(D, N, tokens, idx, dout, V0, V, scale)
            return dE0, dE[::-1]
        # duplicates overwrite instead of accumulating
        dE0, dE = real(D, N, tokens, idx, dout, V0, V, scale)
        c = scale / N
        for n in range(N - 1):
            dE[n][:] = 0
            dE[n][np.asarray(idx[:, n])] = c * np.asarray(dout)
        return dE0, dE
    monkeypatch.setattr(O, "backward_basic", planted)
    assert _fails(check_basic_backward)


# ------------------------------------------------------------------ collisions (section 3.2.2)

def check_collisions_golden():
    g = _load("hash_collisions_handworked.json")
    for c in g["cases"]:
        distinct, slots = O.hash_slot_stats(g["V0"], c["n"], g["tokens"], g["cu_seqlens"],
                                            c["V"])
        assert distinct == c["distinct"], c["n"]
        assert slots == c["slots"], c["n"]


def test_collisions_handworked():
    check_collisions_golden()


def _contexts(tokens, cu, n):
    """Every position's n-gram as a tuple (t_i, t_{i-1}, ...), pad 0 before the start."""
    out = []
    for b in range(len(cu) - 1):
        seq = list(tokens[cu[b]:cu[b + 1]])
        for i in range(len(seq)):
            out.append(tuple(seq[i - j] if i - j >= 0 else 0 for j in range(n)))
    return out


def check_collisions_closed_forms():
    rng = np.random.default_rng(7)
    V0 = 23
    lengths = (40, 1, 17, 90)
    tokens = [int(x) for x in rng.integers(0, V0, size=sum(lengths))]
    cu = [int(x) for x in cu_seqlens_from_lengths(lengths)]
    ctx2 = _contexts(tokens, cu, 2)
    # distinct 2-grams are distinct (t_{i-1}, t_i) pairs; a table of size m*V0 keeps t_i and
    # t_{i-1} mod m (the value is t_i + V0 t_{i-1}), which is why multiples of V0 collide
    for m in (1, 2, 3, 5):
        distinct, slots = O.hash_slot_stats(V0, 2, tokens, cu, [m * V0])
        assert distinct == len(set(ctx2))
        assert slots == [len({(a, b % m) for a, b in ctx2})], m
    # sizes above every 2-gram value (V0^2) lose nothing; a one-row table keeps one row
    distinct, slots = O.hash_slot_stats(V0, 2, tokens, cu, [V0 * V0, V0 * V0 + 7, 1])
    assert slots == [distinct, distinct, 1]
    # order 3: brute force over context tuples, and the one-digit table V = V0
    ctx3 = _contexts(tokens, cu, 3)
    distinct3, slots3 = O.hash_slot_stats(V0, 3, tokens, cu, [V0, V0 ** 3])
    assert distinct3 == len(set(ctx3))
    assert slots3 == [len({c[0] for c in ctx3}), distinct3]


def test_collisions_closed_forms():
    check_collisions_closed_forms()


@pytest.mark.parametrize("mistake", ["digits_reversed", "no_pad", "count_positions"])
def test_collision_pins_catch_planted_mistakes(monkeypatch, mistake):
    if mistake == "digits_reversed":
        monkeypatch.setattr(O, "ngram_value",
                            lambda ctx, n, V0: sum(int(ctx[n - 1 - j]) * V0 ** j for j in range(n)))
    elif mistake == "no_pad":
        monkeypatch.setattr(O, "context",
                            lambda seq, i, n: [int(seq[(i - j) % len(seq)]) for j in range(n)])
    else:
        real = O.hash_slot_stats

        def planted(V0, n, tokens, cu, vocab_sizes):
            distinct, slots = real(V0, n, tokens, cu, vocab_sizes)
            return len(tokens), slots
        monkeypatch.setattr(O, "hash_slot_stats", planted)
    assert _fails(check_collisions_golden) or _fails(check_collisions_closed_forms)
