"""Host checks of the synthetic-input module: sizes, primes, id generators, determinism."""
import numpy as np
import pytest

import workloads as W


def _is_prime(x):
    from sympy import isprime
    return isprime(x)


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_workload_shapes(name):
    w = W.workload(name)
    assert len(w.V) == w.S and len(set(w.V)) == w.S
    if w.form == "final":
        assert w.D % w.S == 0
    else:                                   # Eq. 1: one full-width table per order
        assert w.K == 1 and w.d == w.D
    # sub-table width D/((N-1)K) (D in the basic form); 16-byte rows: whole-vector loads
    assert (w.d * w.esz) % 16 == 0
    assert w.V0 * max(w.V) < 2 ** 63


@pytest.mark.parametrize("name", [n for n in W.WORKLOADS if "tiny" not in n])
def test_subtable_sizes_are_mid_gap_primes(name):
    # Section 3.2.2: keep V_{n,k} away from integer multiples of V0.
    w = W.workload(name)
    for v in w.V:
        assert _is_prime(v)
        frac = (v % w.V0) / w.V0
        assert 0.45 < frac < 0.55


def test_tiny_sizes_match_spec():
    w = W.workload("tiny_f32")
    assert (w.V0, w.D, w.N, w.K, w.V, w.batch, w.seqlen, w.seed) == \
        (1000, 64, 3, 2, (5003, 7001, 6007, 8009), 2, 128, 0)
    assert all(_is_prime(v) for v in w.V)


def test_param_scale_of_30b_workload():
    w = W.workload("prefill_64k_30b")
    n_params = sum(v * w.d for v in w.V)
    assert 29.9e9 < n_params < 30.1e9
    assert w.T == 65536


def test_param_scale_of_basic_30b_workload():
    w = W.workload("prefill_64k_basic_30b")
    assert sum(v * w.D for v in w.V) == pytest.approx(29.6e9, rel=0.01)
    assert w.T == 65536 and w.form == "basic"
    assert W.mid_gap_primes(131072, 3260000, 3) == list(w.V)


def test_basic_tables_have_no_projection():
    E0, E, Wm = W.host_tables(W.workload("basic_tiny_f32"))
    assert Wm is None and tuple(E0.shape) == (1000, 64)
    assert [tuple(e.shape) for e in E] == [(5003, 64), (7001, 64)]


def test_per_layer_workload():
    w = W.workload("plne_8x_d2048")
    assert w.layers == 8 and w.S == 4 and w.d == 512
    assert W.mid_gap_primes(131072, 1000000, 4) == list(w.V)
    assert sum(v * w.d for v in w.V) == pytest.approx(2.0e9, rel=0.01)


def test_mid_gap_primes_rule():
    ps = W.mid_gap_primes(131072, int(9.8e6), 12)
    assert ps == list(W.workload("prefill_64k_30b").V)
    assert W.mid_gap_primes(131072, int(2.0e6), 16) == list(W.workload("bf16_d2048_n5k4").V)


def test_ids_in_range_and_deterministic():
    for name in ("tiny_f32", "bf16_d2048_n5k4"):
        w = W.workload(name)
        a = W.token_batch(w, 0, batch=3, seqlen=500)
        b = W.token_batch(w, 0, batch=3, seqlen=500)
        c = W.token_batch(w, 1, batch=3, seqlen=500)
        assert a.dtype == np.int32 and a.min() >= 0 and a.max() < w.V0
        np.testing.assert_array_equal(a, b)
        assert not np.array_equal(a, c)


def test_zipf_is_heavy_tailed_and_not_pad():
    rng = np.random.default_rng(0)
    ids = W.zipf_ids(rng, 131072, (200000,))
    counts = np.bincount(ids, minlength=131072)
    top = np.sort(counts)[::-1]
    # rank-1 probability of Zipf(1.1) over ranks 1..V0 is 1 / sum_r r^-1.1
    p1 = 1.0 / np.sum(np.arange(1, 131073, dtype=np.float64) ** -1.1)
    assert abs(top[0] / ids.size - p1) < 5 * np.sqrt(p1 / ids.size)
    assert top[0] / max(top[99], 1) > 50
    assert counts[0] < top[0]


def test_host_tables_shapes_and_scale():
    w = W.workload("tiny_f32")
    E0, E, Wst = W.host_tables(w)
    assert tuple(E0.shape) == (w.V0, w.D)
    assert [tuple(e.shape) for e in E] == [(v, w.d) for v in w.V]
    assert tuple(Wst.shape) == (w.D, w.D)
    assert abs(float(E0.float().std()) - 0.02) < 0.002
    blocks = W.split_stacked_w(Wst, w.S)
    assert all(tuple(b.shape) == (w.D, w.d) for b in blocks)
