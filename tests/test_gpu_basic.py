"""GPU parity of the basic form of the layer (section A2, Eq. 1: one full-width table per
order, no projection, divided by N), through the C ABI, against oracle.embed_basic and
oracle.backward_basic on the same seeded inputs.

Hash indices are compared bit for bit. Embeddings use the tolerances of gpu_helpers.TOL
(fp32 sums, one rounding); the amplified outputs the scale-aware bound of the amplification
tests; gradients relative L2 <= 1e-5 (fp32 sums of exact inputs). Covered: every row of the
small cases (ragged, empty and one-token sequences, N = 1, 2, 3, 5, fp32 and bf16), ids
outside the vocabulary, both amplifications, decode with the N-gram cache (one-shot and
row windows), the stand-alone gather, the backward, and the ~30B-parameter basic-form layer
at its 64K-token shape (every row)."""
import numpy as np
import pytest

import gram_embedding_layer_amd as g
import oracle
import workloads as WL
from tests.gpu_helpers import assert_close, device_fetch, packed, rel_l2, to_f64, ws_indices
from tests.test_gpu_amp import assert_close as assert_close_amp, ln_params
from tests.test_gpu_prefill import dev, host_to_dev_tables

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def basic_workload(dtype="bf16", V0=1000, D=256, N=3, seed=11):
    V = WL.mid_gap_primes(V0, 3 * V0, N - 1) if N > 1 else []
    return WL.Workload(f"basic_{dtype}_{D}_{N}", dtype, V0, D, N, 1, tuple(V), 1, 1, "uniform",
                       seed, form="basic")


def cfg_of(w, **kw):
    return g.Config(w.N, 1, w.D, w.dtype, w.V0, list(w.V), form="basic", **kw)


def tdtype(w):
    return torch.float32 if w.dtype == "f32" else torch.bfloat16


def expected(w, E0, E, tokens, idx, rows):
    return oracle.embed_basic(w.D, w.N, tokens[rows], idx[rows], device_fetch(E0, E))


def run_prefill(cfg, tables, tokens, cu, dtype, fill=3.0):
    T = len(tokens)
    out = torch.full((T, cfg.D), fill, dtype=dtype, device="cuda")
    ws = g.alloc_workspace(cfg, T)
    g.ngram_embed_prefill(cfg, tables, dev(tokens), dev(cu), out, ws)
    torch.cuda.synchronize()
    return out, ws


CASES = [
    ("f32_tiny", WL.workload("basic_tiny_f32"), None),
    ("bf16_d1024", WL.workload("basic_bf16_d1024"), None),
    ("bf16_ragged_n4", basic_workload("bf16", D=256, N=4), (300, 1, 0, 77, 2)),
    ("bf16_n5_d512", basic_workload("bf16", D=512, N=5, V0=5000), (600, 3)),
    ("f32_n2", basic_workload("f32", D=64, N=2), (50, 9)),
    ("bf16_n1", basic_workload("bf16", D=128, N=1), (40, 9)),
    # more than 4 orders after the first (the kernel's id registers sized for up to 16)
    ("bf16_n9", basic_workload("bf16", D=256, N=9), (200, 5)),
    ("bf16_n16_max", basic_workload("bf16", D=128, N=16), (100, 2)),
]


def case_tokens(w, lengths, name):
    if lengths is None:
        return packed(list(WL.token_batch(w)))
    rng = np.random.default_rng(len(name))
    return packed([rng.integers(0, w.V0, size=L).astype(np.int32) for L in lengths])


@pytest.mark.parametrize("name,w,lengths", CASES, ids=[c[0] for c in CASES])
def test_basic_prefill_matches_oracle(lib, name, w, lengths):
    E0, E, _ = host_to_dev_tables(w)
    cfg = cfg_of(w)
    tokens, cu = case_tokens(w, lengths, name)
    T = len(tokens)
    out, ws = run_prefill(cfg, g.Tables(E0, E, None), tokens, cu, tdtype(w))
    idx = oracle.hash_indices(w.V0, w.N, 1, w.V, tokens, cu)
    if w.N > 1:
        _, got_idx = ws_indices(ws, cfg, T)
        np.testing.assert_array_equal(got_idx, idx)                  # bit-exact hash
    rows = np.arange(T)
    assert_close(to_f64(out), expected(w, E0, E, tokens, idx, rows), w.dtype, name)
    assert g.ngram_embed_read_error_flag(ws) == 0


@pytest.mark.parametrize("mode,scale,affine", [("scale", None, False), ("scale", -0.5, False),
                                               ("layernorm", None, False),
                                               ("layernorm", None, True)],
                         ids=["sqrtD", "neg_factor", "ln_plain", "ln_affine"])
def test_basic_amplification(lib, mode, scale, affine):
    w = basic_workload("bf16", D=256, N=4)
    E0, E, _ = host_to_dev_tables(w)
    wt, bs = ln_params(w, affine)
    cfg = cfg_of(w, amp=mode, amp_scale=scale)
    tokens, cu = case_tokens(w, (300, 1, 0, 77), "amp")
    out, ws = run_prefill(cfg, g.Tables(E0, E, None, wt, bs), tokens, cu, torch.bfloat16)
    idx = oracle.hash_indices(w.V0, w.N, 1, w.V, tokens, cu)
    e = expected(w, E0, E, tokens, idx, np.arange(len(tokens)))
    if mode == "scale":
        want = oracle.amplify(e, "scale", scale=np.sqrt(w.D) if scale is None else scale)
    else:
        want = oracle.amplify(e, "layernorm", eps=1e-5,
                              weight=None if wt is None else to_f64(wt),
                              bias=None if bs is None else to_f64(bs))
    assert_close_amp(to_f64(out), want, "bf16", f"basic {mode}")
    assert g.ngram_embed_read_error_flag(ws) == 0


@pytest.mark.parametrize("amp", ["none", "layernorm"])
def test_basic_bad_tokens_give_zero_rows(lib, amp):
    w = basic_workload("bf16", D=256, N=3)
    E0, E, _ = host_to_dev_tables(w)
    cfg = cfg_of(w, amp=amp)
    rng = np.random.default_rng(3)
    tokens = rng.integers(0, w.V0, size=200).astype(np.int32)
    tokens[[4, 150]] = [w.V0, -7]
    out, ws = run_prefill(cfg, g.Tables(E0, E, None), tokens, np.array([0, 200], np.int32),
                          torch.bfloat16)
    got = to_f64(out)
    assert np.all(got[[4, 150]] == 0)
    assert g.ngram_embed_read_error_flag(ws) & g.NGRAM_FLAG_BAD_TOKEN
    good = np.setdiff1d(np.arange(200), [4, 5, 6, 150, 151, 152])    # contexts of bad ids aside
    ok = tokens.copy()
    ok[[4, 150]] = 0
    idx = oracle.hash_indices(w.V0, w.N, 1, w.V, ok, [0, 200])
    if amp == "none":
        assert_close(got[good], expected(w, E0, E, ok, idx, good), "bf16", "basic good rows")


def test_basic_gather_is_table_rows(lib):
    w = basic_workload("bf16", D=256, N=4)
    E0, E, _ = host_to_dev_tables(w)
    cfg = cfg_of(w)
    tokens, cu = case_tokens(w, (500, 3), "gather")
    idx = oracle.hash_indices(w.V0, w.N, 1, w.V, tokens, cu)
    G = torch.empty((len(tokens), w.S * w.D), dtype=torch.bfloat16, device="cuda")
    g.ngram_embed_gather(cfg, g.Tables(E0, E, None), dev(idx.astype(np.int32)), G)
    torch.cuda.synchronize()
    want = torch.cat([E[s][torch.as_tensor(idx[:, s], device="cuda")] for s in range(w.S)], 1)
    assert torch.equal(G, want)


def test_basic_decode_matches_oracle_and_windows(lib):
    w = basic_workload("bf16", D=768, N=4, V0=5000)
    E0, E, _ = host_to_dev_tables(w)
    cfg = cfg_of(w)
    tables = g.Tables(E0, E, None)
    rng = np.random.default_rng(12)
    hists = [rng.integers(0, w.V0, size=L).astype(np.int32) for L in (0, 1, 2, 9, 40)]
    nseq, tmax = len(hists), 5
    htok, hcu = packed(hists)
    caches = [g.Cache.empty(cfg, nseq) for _ in range(2)]
    for c in caches:
        g.ngram_cache_init(cfg, c, dev(htok), dev(hcu))
    orc = oracle.DecodeOracle(w.V0, w.D, w.N, 1, w.V, hists)
    fetch = device_fetch(E0, E)
    ws = g.alloc_workspace(cfg, nseq * tmax)
    for step in range(3):
        new = rng.integers(0, w.V0, size=(nseq, tmax)).astype(np.int32)
        n_new = rng.integers(1, tmax + 1, size=nseq).astype(np.int32)
        n_acc = np.array([rng.integers(0, n + 1) for n in n_new], dtype=np.int32)
        out = torch.full((nseq, tmax, w.D), 3.0, dtype=torch.bfloat16, device="cuda")
        g.ngram_embed_decode(cfg, tables, caches[0], dev(new), dev(n_new), out, ws,
                             n_commit=dev(n_acc))
        win = torch.full_like(out, -1.0)
        for j in range(tmax):                      # rows filled one draft id at a time
            g.ngram_embed_decode_rows(cfg, tables, caches[1], dev(new),
                                      dev(np.minimum(n_new, j + 1)), win, ws, row_begin=j,
                                      row_end=j + 1)
        g.ngram_cache_commit(cfg, caches[1], dev(new), dev(n_acc))
        torch.cuda.synchronize()
        per = [list(new[b, :n_new[b]]) for b in range(nseq)]
        idxs = orc.step_indices(per)
        got = to_f64(out)
        for b in range(nseq):
            k = int(n_new[b])
            assert np.all(got[b, k:] == 0), (step, b)
            want = oracle.embed_basic(w.D, w.N, per[b], idxs[b], fetch)
            assert_close(got[b, :k], want, "bf16", f"step {step} seq {b}")
            assert torch.equal(win[b, :k].view(torch.int16), out[b, :k].view(torch.int16))
            assert bool((win[b, k:] == -1.0).all())
        orc.commit(per, n_acc)
    assert torch.equal(caches[0].len, caches[1].len)
    assert g.ngram_embed_read_error_flag(ws) == 0


BW_CASES = [
    ("bf16_dups", basic_workload("bf16", D=256, N=3, V0=60), (700, 1, 0, 90), 1.0),
    ("bf16_n5_scaled", basic_workload("bf16", D=512, N=5, V0=5000), (900, 30), None),
    ("f32_tiny", WL.workload("basic_tiny_f32"), None, 1.0),
]


@pytest.mark.parametrize("name,w,lengths,scale", BW_CASES, ids=[c[0] for c in BW_CASES])
def test_basic_backward_matches_oracle(lib, name, w, lengths, scale):
    E0, E, _ = host_to_dev_tables(w)
    amp = "none" if scale == 1.0 else "scale"
    cfg = cfg_of(w, amp=amp)
    tokens, cu = case_tokens(w, lengths, name)
    T = len(tokens)
    rng = np.random.default_rng(5)
    dout = torch.as_tensor(rng.normal(0.0, 1.0, size=(T, w.D))).to(tdtype(w)).cuda()
    dE0 = torch.zeros((w.V0, w.D), dtype=torch.float32, device="cuda")
    dE = [torch.zeros((v, w.D), dtype=torch.float32, device="cuda") for v in w.V]
    ws = g.alloc_backward_workspace(cfg, T)
    g.ngram_embed_backward(cfg, g.Tables(E0, E, None), dev(tokens), dev(cu), dout, dE0, dE,
                           None, ws)
    torch.cuda.synchronize()
    assert g.ngram_embed_read_error_flag(ws) == 0
    idx = oracle.hash_indices(w.V0, w.N, 1, w.V, tokens, cu)
    c = np.sqrt(w.D) if scale is None else 1.0
    want0, want = oracle.backward_basic(w.D, w.N, tokens, idx, to_f64(dout), w.V0, w.V, c)
    for nm, got, ref in [("dE0", dE0, want0)] + [(f"dE[{s}]", dE[s], want[s])
                                                  for s in range(w.S)]:
        r = rel_l2(to_f64(got), ref)
        print(f"  {name} {nm}: rel_l2={r:.3e}", flush=True)
        assert r <= 1e-5, (nm, r)


def test_basic_30b_prefill_every_row(lib):
    """The basic form with ~30B parameters (3 tables of 3.2M x 3072 bf16, 59 GB) at the
    64K-token shape: hash indices of every position bit for bit, every embedding row element
    by element."""
    w = WL.workload("prefill_64k_basic_30b")
    E0, E, _ = WL.device_tables(w)
    cfg = cfg_of(w)
    tokens, cu = packed(list(WL.token_batch(w)))
    T = len(tokens)
    out, ws = run_prefill(cfg, g.Tables(E0, E, None), tokens, cu, torch.bfloat16)
    idx = oracle.hash_indices(w.V0, w.N, 1, w.V, tokens, cu)
    _, got_idx = ws_indices(ws, cfg, T)
    np.testing.assert_array_equal(got_idx, idx)
    got = to_f64(out)
    del out
    assert_close(got, expected(w, E0, E, tokens, idx, np.arange(T)), "bf16", "basic 30b")
    assert g.ngram_embed_read_error_flag(ws) == 0
    del E0, E, ws, got
    torch.cuda.empty_cache()
