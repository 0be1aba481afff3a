"""GPU check of ngram_embed_decode_noalloc (the decode step for callers that cannot allocate:
its scratch is the library's fixed per-GPU array) against ngram_embed_decode, through the C
ABI: the same kernels on the same inputs, so outputs and cache updates must be equal bit for
bit, on calls in a row whose inputs shrink (the array keeps the previous call's contents).
The layer has the speculative-verify decode shape of the 30B layer (D = 3072, 12 sub-tables of
width 256, 256 sequences x 5 ids) on smaller tables."""
import numpy as np
import pytest

import gram_embedding_layer_amd as g
import workloads as WL

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def dev(a):
    return torch.as_tensor(np.asarray(a)).to("cuda")


@pytest.fixture(scope="module")
def layer():
    V0 = 32000
    w = WL.Workload("noalloc_d3072", "bf16", V0, 3072, 4, 4,
                    tuple(WL.mid_gap_primes(V0, 3 * V0, 12)), 1, 1, "uniform", 31)
    E0, E, W = WL.device_tables(w)
    return w, g.Tables(E0, E, W)


def caches(cfg, hists):
    """Two identical caches filled from the same histories."""
    tokens = np.concatenate(hists).astype(np.int32)
    cu = np.zeros(len(hists) + 1, np.int32)
    cu[1:] = np.cumsum([len(h) for h in hists])
    out = []
    for _ in range(2):
        c = g.Cache.empty(cfg, len(hists))
        g.ngram_cache_init(cfg, c, dev(tokens), dev(cu))
        out.append(c)
    return out


def both(cfg, tables, ca, cb, new, n_new, n_commit):
    """One step through each entry point on its own cache; returns the two outputs."""
    nseq, tmax = new.shape
    oa = torch.full((nseq, tmax, cfg.D), 5.0, dtype=torch.bfloat16, device="cuda")
    ob = torch.full((nseq, tmax, cfg.D), -5.0, dtype=torch.bfloat16, device="cuda")
    ws = g.alloc_workspace(cfg, nseq * tmax)
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    commit = None if n_commit is None else dev(n_commit)
    g.ngram_embed_decode(cfg, tables, ca, dev(new), dev(n_new), oa, ws, n_commit=commit)
    g.ngram_embed_decode_noalloc(cfg, tables, cb, dev(new), dev(n_new), ob, n_commit=commit,
                                 err_flags=flags)
    torch.cuda.synchronize()
    assert g.ngram_embed_read_error_flag(ws) == int(flags.item())
    return oa, ob, int(flags.item())


def same(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("amp", ["none", "layernorm"])
def test_noalloc_equals_decode_on_calls_in_a_row(lib, layer, amp):
    w, tables = layer
    cfg = g.Config(w.N, w.K, w.D, w.dtype, w.V0, list(w.V), amp=amp)
    rng = np.random.default_rng(3 if amp == "none" else 4)
    nseq = 256
    hists = [rng.integers(0, w.V0, size=int(L)).astype(np.int32)
             for L in rng.integers(0, 40, size=nseq)]
    ca, cb = caches(cfg, hists)
    # 1: the speculative-verify shape, every id committed
    new = rng.integers(0, w.V0, size=(nseq, 5)).astype(np.int32)
    n5 = np.full(nseq, 5, np.int32)
    oa, ob, fl = both(cfg, tables, ca, cb, new, n5, n5)
    assert fl == 0 and same(oa, ob)
    assert torch.equal(ca.len, cb.len) and torch.equal(ca.ring, cb.ring)
    # 2: a smaller step on the same caches: 3-id windows, partial counts and commits
    new = rng.integers(0, w.V0, size=(nseq, 3)).astype(np.int32)
    n_new = rng.integers(0, 4, size=nseq).astype(np.int32)
    n_commit = np.minimum(n_new, rng.integers(0, 4, size=nseq)).astype(np.int32)
    oa, ob, fl = both(cfg, tables, ca, cb, new, n_new, n_commit)
    assert fl == 0 and same(oa, ob)
    assert torch.equal(ca.len, cb.len) and torch.equal(ca.ring, cb.ring)
    # 3: smaller still, fewer sequences, no commit, one bad count (flagged, clamped alike)
    few = hists[:7]
    ca2, cb2 = caches(cfg, few)
    new = rng.integers(0, w.V0, size=(7, 2)).astype(np.int32)
    n_new = np.array([2, 1, 0, 2, 9, 1, 2], np.int32)
    oa, ob, fl = both(cfg, tables, ca2, cb2, new, n_new, None)
    assert fl & g.NGRAM_FLAG_BAD_COUNT and same(oa, ob)
    assert torch.equal(ca2.len, cb2.len)


def test_noalloc_rejects_a_step_beyond_its_scratch(lib, layer):
    w, tables = layer
    cfg = g.Config(w.N, w.K, w.D, w.dtype, w.V0, list(w.V), amp="layernorm")
    nseq = 200
    cache = g.Cache.empty(cfg, nseq)
    new = torch.zeros((nseq, 8), dtype=torch.int32, device="cuda")     # 1600 fp32 rows: 19.7 MB
    n8 = torch.full((nseq,), 8, dtype=torch.int32, device="cuda")
    out = torch.empty((nseq, 8, w.D), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(g.NgramError) as e:
        g.ngram_embed_decode_noalloc(cfg, tables, cache, new, n8, out)
    assert e.value.status == g.NGRAM_ESCRATCH
    assert int(cache.len.abs().sum().item()) == 0                      # nothing enqueued
