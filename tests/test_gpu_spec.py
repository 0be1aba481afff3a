"""GPU tests of the pooled N-gram cache and decode row windows (speculative decoding: rows
computed while the draft model proposes ids are reused at verify time; dynamic batches over a
pool of cache slots), through the C ABI.

Exact where the method is exact: a row computed alone equals the same row computed in a full
decode step bit for bit (the projection's sum order does not depend on which rows share a
call), and rows outside a window keep their bytes. Against the decode oracle within the bf16
tolerance of gpu_helpers.TOL."""
import numpy as np
import pytest

import gram_embedding_layer_amd as g
import oracle
import workloads as WL
from tests.gpu_helpers import assert_close, device_fetch, packed, to_f64, w_blocks
from tests.test_gpu_prefill import dev, host_to_dev_tables, small_workload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def bits(t):
    return t.view(torch.int16)


def setup_small(amp="none", nseq=6, tmax=5, seed=31):
    w = small_workload("bf16", D=1024, N=3, K=2, V0=32000)
    E0, E, W = host_to_dev_tables(w)
    cfg = g.Config(w.N, w.K, w.D, w.dtype, w.V0, list(w.V), amp=amp)
    rng = np.random.default_rng(seed)
    hists = [rng.integers(0, w.V0, size=L).astype(np.int32) for L in (0, 1, 2, 7, 40, 3)[:nseq]]
    new = rng.integers(0, w.V0, size=(nseq, tmax)).astype(np.int32)
    n_new = rng.integers(1, tmax + 1, size=nseq).astype(np.int32)
    return w, cfg, g.Tables(E0, E, W), hists, new, n_new


def fresh_cache(cfg, hists):
    htok, hcu = packed(hists)
    cache = g.Cache.empty(cfg, len(hists))
    g.ngram_cache_init(cfg, cache, dev(htok), dev(hcu))
    return cache


@pytest.mark.parametrize("amp", ["none", "layernorm"])
def test_full_window_equals_decode_and_leaves_other_rows(lib, amp):
    w, cfg, tables, hists, new, n_new = setup_small(amp)
    nseq, tmax = new.shape
    ws = g.alloc_workspace(cfg, nseq * tmax)
    ref = torch.empty((nseq, tmax, w.D), dtype=torch.bfloat16, device="cuda")
    g.ngram_embed_decode(cfg, tables, fresh_cache(cfg, hists), dev(new), dev(n_new), ref, ws)
    out = torch.full((nseq, tmax, w.D), 1.5, dtype=torch.bfloat16, device="cuda")
    g.ngram_embed_decode_rows(cfg, tables, fresh_cache(cfg, hists), dev(new), dev(n_new), out, ws)
    torch.cuda.synchronize()
    for b in range(nseq):
        k = int(n_new[b])
        assert torch.equal(bits(out[b, :k]), bits(ref[b, :k])), b
        assert bool((out[b, k:] == 1.5).all()), b            # untouched, not zeroed
    assert g.ngram_embed_read_error_flag(ws) == 0


@pytest.mark.parametrize("amp", ["none", "layernorm"])
def test_draft_phase_rows_equal_one_shot(lib, amp):
    """Rows filled one at a time as the draft ids appear (later ids still garbage) equal the
    rows of one decode step over all of them."""
    w, cfg, tables, hists, new, n_new = setup_small(amp)
    nseq, tmax = new.shape
    n_new[:] = tmax
    ws = g.alloc_workspace(cfg, nseq * tmax)
    ref = torch.empty((nseq, tmax, w.D), dtype=torch.bfloat16, device="cuda")
    g.ngram_embed_decode(cfg, tables, fresh_cache(cfg, hists), dev(new), dev(n_new), ref, ws)
    cache = fresh_cache(cfg, hists)
    out = torch.full((nseq, tmax, w.D), -2.0, dtype=torch.bfloat16, device="cuda")
    rng = np.random.default_rng(5)
    for j in range(tmax):
        draft = new.copy()
        draft[:, j + 1:] = rng.integers(0, w.V0, size=(nseq, tmax - j - 1))   # not known yet
        nn = np.full(nseq, j + 1, dtype=np.int32)
        g.ngram_embed_decode_rows(cfg, tables, cache, dev(draft), dev(nn), out, ws,
                                  row_begin=j, row_end=j + 1)
        torch.cuda.synchronize()
        assert bool((out[:, j + 1:] == -2.0).all())          # later rows not yet written
    assert torch.equal(bits(out), bits(ref))
    assert g.ngram_embed_read_error_flag(ws) == 0


def test_slot_pool_follows_the_oracle(lib):
    """Four sequences in a pool of ten slots, batches in varying slot order, commits through
    the slots; untouched slots keep their state."""
    w, cfg, tables, hists4, _, _ = setup_small(nseq=4)
    pool = 10
    slots0 = np.array([7, 2, 5, 0], dtype=np.int32)
    cache = g.Cache.empty(cfg, pool)
    cache.ring.fill_(11)
    cache.len.fill_(3)
    htok, hcu = packed(hists4)
    g.ngram_cache_init_slots(cfg, cache, dev(slots0), dev(htok), dev(hcu))
    torch.cuda.synchronize()
    untouched = [s for s in range(pool) if s not in slots0]
    ring_before = cache.ring[untouched].clone()
    len_before = cache.len[untouched].clone()
    orc = oracle.DecodeOracle(w.V0, w.D, w.N, w.K, w.V, hists4)    # history i <-> slots0[i]
    fetch, Wb = device_fetch(tables.E0, tables.E), w_blocks(tables.W, w.S)
    rng = np.random.default_rng(9)
    tmax = 4
    ws = g.alloc_workspace(cfg, 4 * tmax)
    for step in range(4):
        order = rng.permutation(4)                    # batch entry b is history order[b]
        slots = slots0[order]
        new = rng.integers(0, w.V0, size=(4, tmax)).astype(np.int32)
        n_new = rng.integers(1, tmax + 1, size=4).astype(np.int32)
        n_acc = np.array([rng.integers(0, n + 1) for n in n_new], dtype=np.int32)
        out = torch.zeros((4, tmax, w.D), dtype=torch.bfloat16, device="cuda")
        g.ngram_embed_decode_rows(cfg, tables, cache, dev(new), dev(n_new), out, ws,
                                  slots=dev(slots))
        g.ngram_cache_commit_slots(cfg, cache, dev(slots), dev(new), dev(n_acc))
        torch.cuda.synchronize()
        per_hist = [None] * 4
        for b in range(4):
            per_hist[order[b]] = list(new[b, :n_new[b]])
        _, embs = orc.step(per_hist, fetch, Wb)
        got = to_f64(out)
        for b in range(4):
            k = int(n_new[b])
            assert_close(got[b, :k], embs[order[b]], "bf16", f"step {step} entry {b}")
        acc = [0] * 4
        for b in range(4):
            acc[order[b]] = int(n_acc[b])
        orc.commit(per_hist, acc)
    lens = cache.len.cpu().numpy()
    for i, s in enumerate(slots0):
        assert lens[s] == len(orc.hist[i])
    assert torch.equal(cache.ring[untouched], ring_before)
    assert torch.equal(cache.len[untouched], len_before)
    assert g.ngram_embed_read_error_flag(ws) == 0


def test_bad_slot_sets_flag_and_writes_nothing(lib):
    w, cfg, tables, hists, new, n_new = setup_small(nseq=3)
    cache = fresh_cache(cfg, hists[:3])
    len_before = cache.len.clone()
    ws = g.alloc_workspace(cfg, 3 * new.shape[1])
    out = torch.full((3, new.shape[1], w.D), 4.0, dtype=torch.bfloat16, device="cuda")
    slots = np.array([0, 3, 1], dtype=np.int32)                    # 3 is outside the pool
    g.ngram_embed_decode_rows(cfg, tables, cache, dev(new[:3]), dev(n_new[:3]), out, ws,
                              slots=dev(slots), n_commit=dev(n_new[:3]))
    torch.cuda.synchronize()
    assert g.ngram_embed_read_error_flag(ws) & g.NGRAM_FLAG_BAD_SLOT
    assert bool((out[1] == 4.0).all())
    assert int(cache.len[1]) == int(len_before[1]) + int(n_new[2])   # entry 2 -> slot 1
    assert int(cache.len[0]) == int(len_before[0]) + int(n_new[0])


def test_draft_rows_30b_spec_shape(lib, tables_30b):
    """256 sequences with 8192-token histories, 5 ids per step: the verify step's rows,
    filled one draft id at a time, equal one decode step's rows bit for bit."""
    wd = WL.workload("decode_spec5_30b")
    w = WL.workload("prefill_64k_30b")
    E0, E, W = tables_30b
    cfg = g.Config(w.N, w.K, w.D, w.dtype, w.V0, list(w.V))
    tables = g.Tables(E0, E, W)
    nseq, tmax = wd.batch, wd.decode_new
    hist = torch.as_tensor(WL.token_batch(wd, purpose=0).reshape(-1)).cuda()
    cu = torch.as_tensor(np.arange(nseq + 1, dtype=np.int32) * wd.seqlen).cuda()
    new = torch.as_tensor(WL.token_batch(wd, purpose=1, batch=nseq, seqlen=tmax)).cuda()
    n_new = torch.full((nseq,), tmax, dtype=torch.int32, device="cuda")
    ws = g.alloc_workspace(cfg, nseq * tmax)
    caches = []
    for _ in range(2):
        c = g.Cache.empty(cfg, nseq)
        g.ngram_cache_init(cfg, c, hist, cu)
        caches.append(c)
    ref = torch.empty((nseq, tmax, w.D), dtype=torch.bfloat16, device="cuda")
    g.ngram_embed_decode(cfg, tables, caches[0], new, n_new, ref, ws)
    out = torch.empty_like(ref)
    for j in range(tmax):
        nn = torch.full((nseq,), j + 1, dtype=torch.int32, device="cuda")
        g.ngram_embed_decode_rows(cfg, tables, caches[1], new, nn, out, ws, row_begin=j,
                                  row_end=j + 1)
    torch.cuda.synchronize()
    assert torch.equal(bits(out), bits(ref))
    assert g.ngram_embed_read_error_flag(ws) == 0


def test_duplicate_slots_are_flagged_and_skipped(lib):
    """A slot that an earlier batch entry of the call already uses: the later entry is
    ignored (no rows, no commit, NGRAM_FLAG_DUP_SLOT), the earlier one is served exactly as in
    a call without the repeat; the same for commit_slots and init_slots."""
    w, cfg, tables, hists, new, n_new = setup_small(nseq=6)
    nseq, tmax = new.shape
    slots = np.array([3, 1, 3, 0, 1, 5], dtype=np.int32)       # entries 2 and 4 repeat
    keep = [0, 1, 3, 5]
    # reference: the same call without the repeated entries
    ref_cache = fresh_cache(cfg, hists)
    ws = g.alloc_workspace(cfg, nseq * tmax)
    ref = torch.full((len(keep), tmax, w.D), 2.5, dtype=torch.bfloat16, device="cuda")
    g.ngram_embed_decode_rows(cfg, tables, ref_cache, dev(new[keep]), dev(n_new[keep]), ref, ws,
                              slots=dev(slots[keep]), n_commit=dev(n_new[keep]))
    torch.cuda.synchronize()
    assert g.ngram_embed_read_error_flag(ws) == 0
    cache = fresh_cache(cfg, hists)
    ws2 = g.alloc_workspace(cfg, nseq * tmax)
    out = torch.full((nseq, tmax, w.D), 2.5, dtype=torch.bfloat16, device="cuda")
    g.ngram_embed_decode_rows(cfg, tables, cache, dev(new), dev(n_new), out, ws2,
                              slots=dev(slots), n_commit=dev(n_new))
    torch.cuda.synchronize()
    fl = g.ngram_embed_read_error_flag(ws2)
    assert fl & g.NGRAM_FLAG_DUP_SLOT and not fl & g.NGRAM_FLAG_BAD_SLOT
    for i, b in enumerate(keep):
        assert torch.equal(bits(out[b]), bits(ref[i])), b
    for b in (2, 4):
        assert bool((out[b] == 2.5).all()), b                   # nothing written
    assert torch.equal(cache.len, ref_cache.len) and torch.equal(cache.ring, ref_cache.ring)
    # commit_slots: the repeat is flagged and not appended
    c1, c2 = fresh_cache(cfg, hists), fresh_cache(cfg, hists)
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    g.ngram_cache_commit_slots(cfg, c1, dev(slots), dev(new), dev(n_new), err_flags=flags)
    g.ngram_cache_commit_slots(cfg, c2, dev(slots[keep]), dev(new[keep]), dev(n_new[keep]))
    torch.cuda.synchronize()
    assert int(flags.item()) == g.NGRAM_FLAG_DUP_SLOT
    assert torch.equal(c1.len, c2.len) and torch.equal(c1.ring, c2.ring)
    # init_slots: the first sequence given a slot fills it
    seqs = [np.arange(L, dtype=np.int32) + 7 * L for L in (5, 9, 2, 4, 1, 6)]
    tok, cu = packed(seqs)
    d1, d2 = fresh_cache(cfg, hists), fresh_cache(cfg, hists)
    flags.zero_()
    g.ngram_cache_init_slots(cfg, d1, dev(slots), dev(tok), dev(cu), err_flags=flags)
    tk, ck = packed([seqs[i] for i in keep])
    g.ngram_cache_init_slots(cfg, d2, dev(slots[keep]), dev(tk), dev(ck))
    torch.cuda.synchronize()
    assert int(flags.item()) == g.NGRAM_FLAG_DUP_SLOT
    assert torch.equal(d1.len, d2.len) and torch.equal(d1.ring, d2.ring)


def test_duplicate_check_across_blocks(lib):
    """Repeats far apart in a large batch (the check runs over every earlier entry, across
    the kernels' blocks): only the later copies are dropped."""
    w = small_workload("bf16", D=256, N=3, K=2, V0=500)
    E0, E, W = host_to_dev_tables(w)
    cfg = g.Config(w.N, w.K, w.D, w.dtype, w.V0, list(w.V))
    tables = g.Tables(E0, E, W)
    nbatch, pool = 3000, 4000
    rng = np.random.default_rng(8)
    slots = rng.permutation(pool)[:nbatch].astype(np.int32)
    dups = [(10, 2999), (700, 1500), (2048, 2049)]            # (earlier, later) entries
    for a_, b_ in dups:
        slots[b_] = slots[a_]
    new = rng.integers(0, w.V0, size=(nbatch, 2)).astype(np.int32)
    n_new = np.full(nbatch, 2, np.int32)
    cache = g.Cache.empty(cfg, pool)
    ws = g.alloc_workspace(cfg, nbatch * 2)
    out = torch.full((nbatch, 2, w.D), 9.0, dtype=torch.bfloat16, device="cuda")
    g.ngram_embed_decode_rows(cfg, tables, cache, dev(new), dev(n_new), out, ws,
                              slots=dev(slots), n_commit=dev(n_new))
    torch.cuda.synchronize()
    assert g.ngram_embed_read_error_flag(ws) & g.NGRAM_FLAG_DUP_SLOT
    written = (out != 9.0).flatten(1).any(dim=1).cpu().numpy()
    later = {b_ for _, b_ in dups}
    assert all(written[b] == (b not in later) for b in range(nbatch))
    lens = cache.len.cpu().numpy()
    assert int((lens == 2).sum()) == nbatch - len(dups)       # one commit per distinct slot
