"""GPU parity of kernel 4 (decode with the device N-gram cache) against the decode oracle.

A decode step's rows must equal, index for index, what a prefill of the committed history
followed by the new ids gives those positions; rows beyond n_new are zero; commits advance
the cache like the oracle's histories. Also: decode == prefill bitwise on the GPU, the
30B-parameter layer at the speculative-verify shape (256 sequences, 8192-token histories,
5 ids per step), and replays of a captured HIP graph of several steps."""
import numpy as np
import pytest

import gram_embedding_layer_amd as g
import oracle
import workloads as WL
from tests.gpu_helpers import (assert_close, cfg_of, device_fetch, packed, to_f64, w_blocks,
                               ws_indices)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def dev(a):
    return torch.as_tensor(np.asarray(a)).to("cuda")


def decode_workload(N=4, K=2, D=1536, V0=32000, dtype="bf16"):
    S = (N - 1) * K
    V = WL.mid_gap_primes(V0, 3 * V0, S)
    return WL.Workload(f"dec_{N}_{K}_{D}", dtype, V0, D, N, K, tuple(V), 1, 1, "uniform", 21)


def init_cache(cfg, histories):
    tokens, cu = packed(histories)
    cache = g.Cache.empty(cfg, len(histories))
    g.ngram_cache_init(cfg, cache, dev(tokens), dev(cu))
    return cache


def check_cache(cfg, cache, hist):
    ring = cache.ring.cpu().numpy()
    ln = cache.len.cpu().numpy()
    nm1 = cfg.N - 1
    for b, h in enumerate(hist):
        assert ln[b] == len(h)
        for p in range(max(0, len(h) - nm1), len(h)):
            assert ring[b, p % nm1] == h[p]


def decode_step(cfg, tables, cache, new, n_new, n_commit, ws, dtype):
    nseq, tmax = new.shape
    out = torch.full((nseq, tmax, cfg.D), 7.0, dtype=dtype, device="cuda")
    g.ngram_embed_decode(cfg, tables, cache, dev(new), dev(n_new), out, ws,
                         n_commit=None if n_commit is None else dev(n_commit))
    torch.cuda.synchronize()
    return out


# (5, 16, 512) with 8-id windows: 8 x 64 (row, sub-table) hashes per entry, exactly one entry
# per block of the decode hash; N = 1: no sub-tables, the rows are E_0 rows
@pytest.mark.parametrize("N,K,D,dtype,tmax", [(4, 2, 1536, "bf16", 5), (3, 2, 64, "f32", 5),
                                              (2, 1, 256, "bf16", 5), (6, 1, 320, "bf16", 5),
                                              (5, 16, 512, "bf16", 8), (1, 1, 256, "bf16", 8)])
def test_decode_matches_oracle(lib, N, K, D, dtype, tmax):
    w = decode_workload(N=N, K=K, D=D, dtype=dtype)
    cfg = cfg_of(w)
    E0, E, W = WL.host_tables(w) if dtype == "f32" else WL.device_tables(w)
    E0, E, W = E0.cuda(), [e.cuda() for e in E], W.cuda()
    tables = g.Tables(E0, E, W)
    tdt = E0.dtype
    rng = np.random.default_rng([N, K, D])
    hist = [list(rng.integers(0, w.V0, size=L)) for L in (0, 1, 2, 3, 10, 100, N - 1, 5)]
    nseq = len(hist)
    cache = init_cache(cfg, hist)
    check_cache(cfg, cache, hist)
    orc = oracle.DecodeOracle(w.V0, w.D, w.N, w.K, w.V, hist)
    ws = g.alloc_workspace(cfg, nseq * tmax)
    fetch, Wb = device_fetch(E0, E), w_blocks(W, w.S)
    for step in range(6):
        new = rng.integers(0, w.V0, size=(nseq, tmax)).astype(np.int32)
        n_new = rng.integers(0, tmax + 1, size=nseq).astype(np.int32)
        if step == 0:
            n_new[:] = tmax
        n_commit = np.array([rng.integers(0, n + 1) for n in n_new], dtype=np.int32)
        separate = step % 3 == 2     # commit through ngram_cache_commit instead
        out = decode_step(cfg, tables, cache, new, n_new, None if separate else n_commit,
                          ws, tdt)
        tok, idx = ws_indices(ws, cfg, nseq * tmax)
        props = [list(new[b, :n_new[b]]) for b in range(nseq)]
        want_idx = orc.step_indices(props)
        got = to_f64(out)
        act_rows, act_tok, act_idx = [], [], []
        for b in range(nseq):
            for j in range(tmax):
                r = b * tmax + j
                if j < n_new[b]:
                    assert tok[r] == new[b, j]
                    np.testing.assert_array_equal(idx[r], want_idx[b][j])
                    act_rows.append((b, j))
                    act_tok.append(new[b, j])
                    act_idx.append(want_idx[b][j])
                else:
                    assert tok[r] == -1
                    assert np.all(got[b, j] == 0)
        if act_rows:
            e = oracle.embed_from_indices(w.D, w.N, w.K, act_tok, np.array(act_idx), fetch, Wb)
            assert_close(np.stack([got[b, j] for b, j in act_rows]), e, dtype, f"step {step}")
        if separate:
            g.ngram_cache_commit(cfg, cache, dev(new), dev(n_commit))
        orc.commit(props, n_commit)
        check_cache(cfg, cache, orc.hist)
    assert g.ngram_embed_read_error_flag(ws) == 0


def test_decode_equals_prefill_bitwise(lib):
    w = decode_workload()
    cfg = cfg_of(w)
    E0, E, W = WL.device_tables(w)
    tables = g.Tables(E0, E, W)
    rng = np.random.default_rng(8)
    full = [list(rng.integers(0, w.V0, size=L)) for L in (40, 9, 17, 3)]
    hist_len = [30, 0, 12, 1]
    cache = init_cache(cfg, [f[:h] for f, h in zip(full, hist_len)])
    tmax = 5
    new = np.zeros((4, tmax), np.int32)
    n_new = np.zeros(4, np.int32)
    for b, (f, h) in enumerate(zip(full, hist_len)):
        k = min(tmax, len(f) - h)
        new[b, :k] = f[h:h + k]
        n_new[b] = k
    ws = g.alloc_workspace(cfg, 4 * tmax)
    out = decode_step(cfg, tables, cache, new, n_new, None, ws, torch.bfloat16)
    tokens, cu = packed(full)
    pre = torch.empty((len(tokens), w.D), dtype=torch.bfloat16, device="cuda")
    ws2 = g.alloc_workspace(cfg, len(tokens))
    g.ngram_embed_prefill(cfg, tables, dev(tokens), dev(cu), pre, ws2)
    torch.cuda.synchronize()
    for b in range(4):
        for j in range(n_new[b]):
            p = int(cu[b]) + hist_len[b] + j
            assert torch.equal(out[b, j].view(torch.int16), pre[p].view(torch.int16)), (b, j)


def test_bad_counts_set_flag(lib):
    w = decode_workload(N=3, K=2, D=64, dtype="f32")
    cfg = cfg_of(w)
    E0, E, W = WL.host_tables(w)
    tables = g.Tables(E0.cuda(), [e.cuda() for e in E], W.cuda())
    cache = init_cache(cfg, [[1, 2, 3], [4]])
    ws = g.alloc_workspace(cfg, 2 * 3)
    new = np.array([[5, 6, 7], [8, 9, 10]], np.int32)
    out = decode_step(cfg, tables, cache, new, np.array([9, 1], np.int32), None, ws,
                      torch.float32)
    assert g.ngram_embed_read_error_flag(ws) & g.NGRAM_FLAG_BAD_COUNT
    assert torch.isfinite(out).all()
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    g.ngram_cache_commit(cfg, cache, dev(new), dev(np.array([-2, 1], np.int32)), flags)
    torch.cuda.synchronize()
    assert int(flags.item()) & g.NGRAM_FLAG_BAD_COUNT
    check_cache(cfg, cache, [[1, 2, 3], [4, 8]])


def test_decode_30b_spec_verify_shape(lib, tables_30b):
    """256 sequences with 8192-token histories in the cache, 5 ids (1 + 4 drafts) per step,
    all committed, on the 30B-parameter tables: every index and every embedding row."""
    w = WL.workload("decode_spec5_30b")
    cfg = cfg_of(w)
    E0, E, W = tables_30b
    tables = g.Tables(E0, E, W)
    hist2d = WL.token_batch(w, purpose=0)
    hist = [list(h) for h in hist2d]
    cache = init_cache(cfg, hist)
    orc = oracle.DecodeOracle(w.V0, w.D, w.N, w.K, w.V, hist)
    nseq, tmax = w.batch, w.decode_new
    ws = g.alloc_workspace(cfg, nseq * tmax)
    fetch, Wb = device_fetch(E0, E), w_blocks(W, w.S)
    steps = WL.token_batch(w, purpose=1, batch=3 * nseq, seqlen=tmax).reshape(3, nseq, tmax)
    n_new = np.full(nseq, tmax, np.int32)
    for step in range(3):
        new = steps[step]
        out = decode_step(cfg, tables, cache, new, n_new, n_new, ws, torch.bfloat16)
        tok, idx = ws_indices(ws, cfg, nseq * tmax)
        props = [list(new[b]) for b in range(nseq)]
        want = np.concatenate(orc.step_indices(props), axis=0)
        np.testing.assert_array_equal(idx, want)
        e = oracle.embed_from_indices(w.D, w.N, w.K, new.reshape(-1), want, fetch, Wb)
        assert_close(to_f64(out).reshape(nseq * tmax, w.D), e, "bf16", f"step {step}")
        orc.commit(props, n_new)
    check_cache(cfg, cache, orc.hist)


def test_decode_30b_1000_steps(lib, tables_30b):
    """The speculative-verify workload end to end: 1000 steps of 256 x 5 ids, all committed,
    on the 30B-parameter tables (the ids the benchmark times). Every index of every step
    (15.36M) bit for bit against the oracle's hash of the sequences (history followed by all
    committed ids: a decode step's rows are the prefill rows of those positions), and
    the embeddings of 34 steps (first, last, 32 seeded) against the oracle."""
    wd = WL.workload("decode_spec5_30b")
    cfg = cfg_of(wd)
    E0, E, W = tables_30b
    tables = g.Tables(E0, E, W)
    nseq, tmax, nsteps, L = wd.batch, wd.decode_new, wd.decode_steps, wd.seqlen
    hist = WL.token_batch(wd, purpose=0)                                   # [256, 8192]
    ids = WL.token_batch(wd, purpose=1, batch=nsteps * nseq, seqlen=tmax).reshape(
        nsteps, nseq, tmax)
    cache = g.Cache.empty(cfg, nseq)
    cu_h = np.arange(nseq + 1, dtype=np.int32) * L
    g.ngram_cache_init(cfg, cache, dev(hist.reshape(-1)), dev(cu_h))
    ws = g.alloc_workspace(cfg, nseq * tmax)
    _, idx_off = g.ngram_embed_workspace_layout(cfg, nseq * tmax)
    idx_ws = ws[idx_off:idx_off + nseq * tmax * wd.S * 4].view(torch.int32)
    rng = np.random.default_rng(8)
    check = sorted({0, nsteps - 1} | set(int(x) for x in rng.choice(nsteps, 32, replace=False)))
    all_idx = torch.empty((nsteps, nseq * tmax * wd.S), dtype=torch.int32, device="cuda")
    outs = {}
    n_new = dev(np.full(nseq, tmax, np.int32))
    ids_dev = dev(ids)
    out = torch.empty((nseq, tmax, wd.D), dtype=torch.bfloat16, device="cuda")
    for step in range(nsteps):
        g.ngram_embed_decode(cfg, tables, cache, ids_dev[step], n_new, out, ws, n_commit=n_new)
        all_idx[step].copy_(idx_ws)
        if step in check:
            outs[step] = out.clone()
    torch.cuda.synchronize()
    assert g.ngram_embed_read_error_flag(ws) == 0
    assert bool((cache.len == L + nsteps * tmax).all())
    # the oracle: every sequence = history + the 5000 committed ids, hashed once. Only the
    # last N-1 history ids reach a decode position's context, so each sequence is cut to
    # them plus the committed ids (the cut's own first N-1 positions are not compared)
    h = wd.N - 1
    full = np.concatenate([hist[:, L - h:], ids.transpose(1, 0, 2).reshape(nseq, nsteps * tmax)],
                          axis=1)
    cu = np.arange(nseq + 1, dtype=np.int64) * full.shape[1]
    want = oracle.hash_indices(wd.V0, wd.N, wd.K, wd.V, full.reshape(-1), cu)
    want = want.reshape(nseq, full.shape[1], wd.S)[:, h:, :]               # decode positions
    want = want.reshape(nseq, nsteps, tmax, wd.S).transpose(1, 0, 2, 3)   # [step, b, j, s]
    got = all_idx.cpu().numpy().reshape(nsteps, nseq, tmax, wd.S)
    np.testing.assert_array_equal(got, want)
    fetch, Wb = device_fetch(E0, E), w_blocks(W, wd.S)
    for step in check:
        e = oracle.embed_from_indices(wd.D, wd.N, wd.K, ids[step].reshape(-1),
                                      want[step].reshape(-1, wd.S), fetch, Wb)
        assert_close(to_f64(outs[step]).reshape(nseq * tmax, wd.D), e, "bf16", f"step {step}")
    del outs, all_idx


def test_decode_graph_replays(lib):
    """Four decode+commit steps captured in one HIP graph, replayed three times from the
    same cache snapshot with eager work in between; every replay equals the eager run."""
    w = decode_workload()
    cfg = cfg_of(w)
    E0, E, W = WL.device_tables(w)
    tables = g.Tables(E0, E, W)
    rng = np.random.default_rng(13)
    nseq, tmax, nsteps = 16, 5, 4
    hist = [list(rng.integers(0, w.V0, size=int(rng.integers(0, 50)))) for _ in range(nseq)]
    cache = init_cache(cfg, hist)
    torch.cuda.synchronize()
    ring0, len0 = cache.ring.clone(), cache.len.clone()
    new = dev(rng.integers(0, w.V0, size=(nsteps, nseq, tmax)).astype(np.int32))
    n_new = dev(rng.integers(1, tmax + 1, size=(nsteps, nseq)).astype(np.int32))
    n_commit = torch.minimum(n_new, dev(rng.integers(0, tmax + 1, size=(nsteps, nseq))
                                        .astype(np.int32)))
    ws = g.alloc_workspace(cfg, nseq * tmax)
    outs = torch.zeros((nsteps, nseq, tmax, w.D), dtype=torch.bfloat16, device="cuda")

    def run():
        for s in range(nsteps):
            g.ngram_embed_decode(cfg, tables, cache, new[s], n_new[s], outs[s], ws,
                                 n_commit=n_commit[s])

    run()
    torch.cuda.synchronize()
    ref = outs.clone()
    ref_ring, ref_len = cache.ring.clone(), cache.len.clone()
    graph = torch.cuda.CUDAGraph()
    cache.ring.copy_(ring0)
    cache.len.copy_(len0)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        run()
    for rep in range(3):
        cache.ring.copy_(ring0)
        cache.len.copy_(len0)
        outs.zero_()
        junk = torch.randn(1000, 1000, device="cuda") @ torch.randn(1000, 1000, device="cuda")
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        del junk
        assert torch.equal(outs.view(torch.int16), ref.view(torch.int16)), rep
        assert torch.equal(cache.ring, ref_ring) and torch.equal(cache.len, ref_len), rep


@pytest.mark.parametrize("N", [1, 2, 4, 6])
def test_prefill_fills_the_cache(lib, N):
    """ngram_embed_prefill with a cache fills it in the same call exactly as ngram_cache_init
    does (lengths and the last N-1 ids, pad id 0 before short sequences, empty sequences
    included), and its outputs are those of the call without a cache; decoding on from that
    cache follows the decode oracle."""
    w = decode_workload(N=N, K=1, D=480)       # S = 0, 1, 3, 5 all divide 480
    cfg = cfg_of(w)
    E0, E, W = WL.host_tables(w)
    E0, E, W = E0.cuda(), [e.cuda() for e in E], W.cuda()
    tables = g.Tables(E0, E, W)
    rng = np.random.default_rng(N)
    hists = [rng.integers(0, w.V0, size=L).astype(np.int32) for L in (0, 1, N - 1, 37, 2, 0, 300)]
    tokens, cu = packed(hists)
    T = len(tokens)
    outs, caches = [], []
    for with_cache in (False, True):
        cache = g.Cache(torch.full((len(hists), max(N - 1, 0)), -5, dtype=torch.int32,
                                   device="cuda"),
                        torch.full((len(hists),), -9, dtype=torch.int64, device="cuda"))
        out = torch.empty((T, w.D), dtype=torch.bfloat16, device="cuda")
        ws = g.alloc_workspace(cfg, T)
        g.ngram_embed_prefill(cfg, tables, dev(tokens), dev(cu), out, ws,
                              cache=cache if with_cache else None)
        torch.cuda.synchronize()
        assert g.ngram_embed_read_error_flag(ws) == 0
        outs.append(out)
        caches.append(cache)
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    ref = init_cache(cfg, hists)
    assert torch.equal(caches[1].len, ref.len)
    assert torch.equal(caches[1].ring, ref.ring)
    check_cache(cfg, caches[1], [list(h) for h in hists])
    # one decode step on the prefill-filled cache against the oracle
    nseq, tmax = len(hists), 5
    new = rng.integers(0, w.V0, size=(nseq, tmax)).astype(np.int32)
    n_new = np.full(nseq, tmax, np.int32)
    ws = g.alloc_workspace(cfg, nseq * tmax)
    out = decode_step(cfg, tables, caches[1], new, n_new, n_new, ws, torch.bfloat16)
    orc = oracle.DecodeOracle(w.V0, w.D, w.N, w.K, w.V, hists)
    _, embs = orc.step([list(r) for r in new], device_fetch(E0, E), w_blocks(W, w.S))
    assert_close(to_f64(out).reshape(nseq * tmax, w.D), np.concatenate(embs), "bf16",
                 f"decode after prefill N={N}")


def test_prefill_cache_only_when_no_tokens(lib):
    """A batch of empty sequences still fills the cache (lengths 0, pad ids)."""
    w = decode_workload(N=3, K=2, D=256)
    cfg = cfg_of(w)
    E0, E, W = WL.host_tables(w)
    tables = g.Tables(E0.cuda(), [e.cuda() for e in E], W.cuda())
    cache = g.Cache(torch.full((3, 2), 4, dtype=torch.int32, device="cuda"),
                    torch.full((3,), 11, dtype=torch.int64, device="cuda"))
    out = torch.empty((0, w.D), dtype=torch.bfloat16, device="cuda")
    ws = g.alloc_workspace(cfg, 0)
    g.ngram_embed_prefill(cfg, tables, torch.zeros(0, dtype=torch.int32, device="cuda"),
                          dev(np.zeros(4, np.int32)), out, ws, cache=cache)
    torch.cuda.synchronize()
    assert int(cache.len.abs().sum().item()) == 0
    assert int(cache.ring.abs().sum().item()) == 0
