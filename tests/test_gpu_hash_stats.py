"""GPU parity of the hash statistics (collisions and table hit counts, section 3.2.2 and
Fig. 3 of the deep-notes page), through the C ABI, against oracle.hash_slot_stats: exact
integers, compared for equality.

Cases: the hand-worked counts of tests/golden (decimal digits, V0 = 10), random small batches
with empty and one-token sequences for n = 1..4 and table sizes around multiples of V0, more
sizes than one launch takes, an order whose exact values exceed 64 bits (rows only), bad ids,
and the study's own scale: 100 sequences x 8192 Zipf(1.1) ids, 59 table sizes between 30x and
33x V0 = 131072, where the collisions spike at the integer multiples of V0 (Fig. 3b) and
stay near the birthday count at sizes coprime to V0."""
import json
import os

import numpy as np
import pytest

import gram_embedding_layer_amd as g
import oracle
import workloads as WL
from tests.gpu_helpers import packed
from tests.test_gpu_prefill import dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def gpu_stats(V0, n, tokens, cu, sizes, with_distinct=True):
    rows = torch.full((max(1, len(sizes)),), -7, dtype=torch.int64, device="cuda")
    distinct = torch.full((1,), -7, dtype=torch.int64, device="cuda") if with_distinct else None
    ws = g.ngram_hash_stats(V0, n, dev(tokens), dev(cu), sizes, rows, distinct)
    torch.cuda.synchronize()
    flags = g.ngram_embed_read_error_flag(ws)
    d = int(distinct.item()) if with_distinct else None
    return d, [int(x) for x in rows[:len(sizes)].cpu()], flags


def test_hash_stats_handworked(lib):
    with open(os.path.join(GOLDEN, "hash_collisions_handworked.json")) as f:
        gold = json.load(f)
    toks = np.array(gold["tokens"], np.int32)
    cu = np.array(gold["cu_seqlens"], np.int32)
    for c in gold["cases"]:
        d, rows, flags = gpu_stats(gold["V0"], c["n"], toks, cu, c["V"])
        assert (d, rows, flags) == (c["distinct"], c["slots"], 0), c["n"]


@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_hash_stats_small_random(lib, n):
    rng = np.random.default_rng(n)
    V0 = 23
    tokens, cu = packed([rng.integers(0, V0, size=L).astype(np.int32)
                         for L in (40, 1, 0, 17, 90, 300)])
    sizes = [1, 2, 23, 46, 69, 70, 115, 529, 530, 12167, 97, 1000003, 2 ** 31 - 1]
    d, rows, flags = gpu_stats(V0, n, tokens, cu, sizes)
    wd, wrows = oracle.hash_slot_stats(V0, n, tokens, cu, sizes)
    assert flags == 0
    assert d == wd and rows == wrows


def test_hash_stats_many_sizes_and_rows_only(lib):
    """70 table sizes (three launches of the size groups); order 5 over V0 = 2^17 has exact
    values up to 2^85, so only the rows are asked for."""
    rng = np.random.default_rng(9)
    V0 = 131072
    tokens, cu = packed([rng.integers(0, V0, size=L).astype(np.int32) for L in (3000, 5, 900)])
    sizes = [int(x) for x in rng.integers(1, 3 * V0, size=70)] + [V0, 2 * V0, 7]
    d, rows, flags = gpu_stats(V0, 2, tokens, cu, sizes)
    wd, wrows = oracle.hash_slot_stats(V0, 2, tokens, cu, sizes)
    assert (d, rows, flags) == (wd, wrows, 0)
    _, rows5, flags5 = gpu_stats(V0, 5, tokens, cu, sizes, with_distinct=False)
    _, wrows5 = oracle.hash_slot_stats(V0, 5, tokens, cu, sizes)
    assert (rows5, flags5) == (wrows5, 0)
    with pytest.raises(g.NgramError):
        gpu_stats(V0, 5, tokens, cu, sizes, with_distinct=True)   # 2^85 > 2^63


def test_hash_stats_bad_ids_flagged(lib):
    tokens = np.array([1, 2, 3, 1000, 4], np.int32)
    _, _, flags = gpu_stats(10, 2, tokens, np.array([0, 5], np.int32), [7])
    assert flags & g.NGRAM_FLAG_BAD_TOKEN


def test_hash_stats_collision_study(lib):
    """The study's scale: every count equal to the oracle's, and the collisions of the
    2-gram hash far higher at integer multiples of V0 than at sizes coprime to V0."""
    V0 = 131072
    ids, sizes = WL.collision_study(V0)
    tokens = ids.reshape(-1)
    cu = np.arange(ids.shape[0] + 1, dtype=np.int32) * ids.shape[1]
    d, rows, flags = gpu_stats(V0, 2, tokens, cu, sizes)
    wd, wrows = oracle.hash_slot_stats(V0, 2, tokens, cu, sizes)
    assert flags == 0
    assert d == wd and rows == wrows
    coll = {v: d - r for v, r in zip(sizes, rows)}
    at_multiples = [coll[m * V0] for m in range(30, 34)]
    # odd sizes share no factor with V0 = 2^17: about the birthday count d^2 / 2V
    coprime = [c for v, c in coll.items() if v % 2 == 1]
    print(f"  distinct 2-grams {d}; collisions at multiples {at_multiples}, at odd sizes "
          f"{min(coprime)}..{max(coprime)} (birthday ~{d * d // (2 * 31 * V0)})", flush=True)
    assert min(at_multiples) > 5 * max(coprime)
    # hit counts of orders 3 and 4 at 30 x V0 (Fig. 3a's table size)
    for n in (3, 4):
        _, r, f = gpu_stats(V0, n, tokens, cu, [30 * V0 + 1], with_distinct=(n == 3))
        _, wr = oracle.hash_slot_stats(V0, n, tokens, cu, [30 * V0 + 1])
        assert (r, f) == (wr, 0), n
