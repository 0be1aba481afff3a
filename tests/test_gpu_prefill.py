"""GPU parity of kernels 1-3 (hash, gather, fused projection) and of prefill, through the C
ABI, against the CPU oracle on the same seeded inputs.

Hash indices must match bit for bit; gathered rows byte for byte; embeddings within the
tolerances in gpu_helpers (relative L2 overall and per row, and for bf16 every element within
the one-rounding bound). Every case compares every row: the small ones (several tiles and a
ragged tail, each tile shape of the matrix-core kernel) and the full-size workloads in the
launch configuration the benchmark times."""
import json
import os

import numpy as np
import pytest

import gram_embedding_layer_amd as g
import oracle
import workloads as WL
from tests.gpu_helpers import (assert_close, cfg_of, device_fetch, gathered_words,
                               oracle_rows, packed, row_checksums, to_f64, w_blocks)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def dev(a, dtype=None):
    t = torch.as_tensor(np.asarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to("cuda")


def small_workload(dtype="bf16", V0=1000, D=256, N=3, K=2, seed=11):
    S = (N - 1) * K
    V = WL.mid_gap_primes(V0, 3 * V0, S) if S else []
    return WL.Workload(f"small_{dtype}_{D}_{N}_{K}", dtype, V0, D, N, K, tuple(V), 1, 1,
                       "uniform", seed)


def host_to_dev_tables(w):
    """Seeded tables on the device: drawn on the host when small, else on the device (W is
    None in the basic form)."""
    n = w.V0 * w.D + sum(w.V) * w.d + (w.D * w.D if w.form == "final" else 0)
    if n <= 8_000_000:
        E0, E, W = WL.host_tables(w)
        return E0.cuda(), [e.cuda() for e in E], (W.cuda() if W is not None else None)
    return WL.device_tables(w)


def run_prefill(cfg, E0, E, W, tokens, cu, dtype):
    T = len(tokens)
    out = torch.empty((T, cfg.D), dtype=dtype, device="cuda")
    ws = g.alloc_workspace(cfg, T)
    g.ngram_embed_prefill(cfg, g.Tables(E0, E, W), dev(tokens), dev(cu), out, ws)
    torch.cuda.synchronize()
    return out, ws


def test_hash_handworked_golden(lib):
    gd = json.load(open(os.path.join(GOLDEN, "hash_handworked_v1000.json")))
    cfg = g.Config(gd["N"], gd["K"], 64, "f32", gd["V0"], gd["V"])
    toks = dev(np.array(gd["tokens"], dtype=np.int32))
    cu = dev(np.array([0, len(gd["tokens"])], dtype=np.int32))
    idx = torch.full((len(gd["tokens"]), cfg.S), -7, dtype=torch.int32, device="cuda")
    g.ngram_embed_hash(cfg, toks, cu, idx)
    np.testing.assert_array_equal(idx.cpu().numpy(), np.array(gd["idx"]))


@pytest.mark.parametrize("N,K,V0", [(3, 2, 1000), (2, 1, 7), (5, 4, 131072), (8, 1, 50),
                                    (4, 3, 32000), (16, 1, 3)])
def test_hash_bit_exact_ragged(lib, N, K, V0):
    rng = np.random.default_rng([N, K, V0])
    S = (N - 1) * K
    V = [int(v) for v in rng.integers(2, 2 ** 31 - 1, size=S)]
    lengths = [0, 1, 2, N - 1, N, 333, 0, 1000, 7]
    seqs = [rng.integers(0, V0, size=L).astype(np.int32) for L in lengths]
    tokens, cu = packed(seqs)
    cfg = g.Config(N, K, 16 * S, "f32", V0, V)
    idx = torch.full((len(tokens), S), -7, dtype=torch.int32, device="cuda")
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    g.ngram_embed_hash(cfg, dev(tokens), dev(cu), idx, flags)
    want = oracle.hash_indices(V0, N, K, V, tokens, cu)
    np.testing.assert_array_equal(idx.cpu().numpy(), want)
    assert int(flags.item()) == 0


def test_hash_extreme_moduli(lib):
    """Largest accepted V0 and V_{n,k}, V = 1, and ids at V0 - 1: exact residues."""
    V0 = 2 ** 31 - 1
    N, K = 4, 2
    V = [1, 2, 3, 2 ** 31 - 1, 2 ** 31 - 2, 65536]
    rng = np.random.default_rng(77)
    seqs = [np.full(9, V0 - 1, np.int32), rng.integers(V0 - 1000, V0, size=300).astype(np.int32),
            rng.integers(0, V0, size=500).astype(np.int32), np.zeros(5, np.int32)]
    tokens, cu = packed(seqs)
    cfg = g.Config(N, K, 16 * len(V), "f32", V0, V)
    idx = torch.full((len(tokens), len(V)), -7, dtype=torch.int32, device="cuda")
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    g.ngram_embed_hash(cfg, dev(tokens), dev(cu), idx, flags)
    np.testing.assert_array_equal(idx.cpu().numpy(), oracle.hash_indices(V0, N, K, V, tokens, cu))
    assert int(flags.item()) == 0


@pytest.mark.parametrize("w", [small_workload("f32", D=64), small_workload("bf16", D=256),
                               small_workload("bf16", D=192, N=4, K=1)], ids=lambda w: w.name)
def test_gather_bytes_exact(lib, w):
    cfg = cfg_of(w)
    E0, E, W = host_to_dev_tables(w)
    rng = np.random.default_rng(5)
    seqs = [rng.integers(0, w.V0, size=L).astype(np.int32) for L in (130, 1, 257)]
    tokens, cu = packed(seqs)
    idx = torch.empty((len(tokens), w.S), dtype=torch.int32, device="cuda")
    g.ngram_embed_hash(cfg, dev(tokens), dev(cu), idx)
    G = torch.empty((len(tokens), w.D), dtype=E0.dtype, device="cuda")
    g.ngram_embed_gather(cfg, g.Tables(E0, E, W), idx, G)
    want_idx = oracle.hash_indices(w.V0, w.N, w.K, w.V, tokens, cu)
    want = np.concatenate([to_f64(E[s].cpu()[torch.as_tensor(want_idx[:, s])])
                           for s in range(w.S)], axis=1)
    np.testing.assert_array_equal(to_f64(G), want)


# Small configurations: every row against the oracle. Row counts pick each tile shape of
# the matrix-core kernel (the tile whose busiest CU loads the fewest bytes; D=1024 has 4
# output tiles of 256): 64 x 64 with its load-only waves (bm64_bn64: 12 row tiles x 16 output
# tiles, one round of the CUs), 64 x 128 (bm64), 128 x 256 (bm128), 256 x 256 (bm256),
# 128 x 128 (n5k4); 64 x 256 where 32 sub-tables' indices do not fit a 128-row tile and
# 64 x 128 tiles would take two rounds of the CUs (s32); and ragged tails.
SMALL = [
    ("tiny_f32_full", WL.workload("tiny_f32"), None),
    ("f32_odd", small_workload("f32", D=96, N=4, K=2), (50, 1, 0, 201)),
    ("bf16_generic_d32", small_workload("bf16", D=128, N=3, K=2), (300, 2, 77)),
    ("bf16_mfma_bm64_bn64", small_workload("bf16", D=1024, N=3, K=2, V0=32000), (300, 1, 0, 450)),
    ("bf16_mfma_bm64", small_workload("bf16", D=1024, N=3, K=2, V0=32000), (700, 1, 0, 1301)),
    ("bf16_mfma_bm128", small_workload("bf16", D=1024, N=3, K=2, V0=32000), (4000, 4100, 3)),
    ("bf16_mfma_bm256", small_workload("bf16", D=1024, N=3, K=2, V0=32000),
     (16384, 16384, 999)),
    ("bf16_mfma_n5k4", small_workload("bf16", D=2048, N=5, K=4, V0=131072), (1000, 37)),
    ("bf16_mfma_bm64_s32", small_workload("bf16", D=2048, N=3, K=16, V0=4000), (900, 1, 500)),
]


@pytest.mark.parametrize("name,w,lengths", SMALL, ids=[s[0] for s in SMALL])
def test_prefill_parity_small(lib, name, w, lengths):
    cfg = cfg_of(w)
    E0, E, W = host_to_dev_tables(w)
    if lengths is None:
        tok2d = WL.token_batch(w)
        seqs = list(tok2d)
    else:
        rng = np.random.default_rng(len(name))
        seqs = [rng.integers(0, w.V0, size=L).astype(np.int32) for L in lengths]
    tokens, cu = packed(seqs)
    T = len(tokens)
    out, ws = run_prefill(cfg, E0, E, W, tokens, cu, E0.dtype)
    _, e = oracle_rows(w, E0, E, W, tokens, cu, np.arange(T))     # every row
    assert_close(to_f64(out), e, w.dtype, name)
    assert g.ngram_embed_read_error_flag(ws) == 0


def test_prefill_handworked_golden(lib):
    """The hand-worked rational examples, scaled so every value is exact in fp32."""
    gd = json.load(open(os.path.join(GOLDEN, "embed_handworked_small.json")))
    for c in gd["cases"]:
        D, S = c["D"], (c["N"] - 1) * c["K"]
        # pad D to 4 fp32 columns (16-byte rows): extra columns are zero tables / W rows
        Dp = 4 * S
        d = Dp // S
        E0 = np.zeros((c["V0"], Dp), np.float32)
        E0[:, :D] = c["E0"]
        E = []
        for s in range(S):
            e = np.zeros((c["V"][s], d), np.float32)
            e[:, :1] = c["E"][s]
            E.append(e)
        Wst = np.zeros((Dp, Dp), np.float32)
        for s in range(S):
            Wst[:D, s * d:s * d + 1] = c["W"][s]
        cfg = g.Config(c["N"], c["K"], Dp, "f32", c["V0"], c["V"])
        tokens, cu = packed([c["tokens"]])
        out, _ = run_prefill(cfg, dev(E0), [dev(e) for e in E], dev(Wst), tokens, cu,
                             torch.float32)
        want = np.array([[p / q for p, q in row] for row in c["e"]])
        np.testing.assert_allclose(out.cpu().numpy()[:, :D], want, rtol=1e-6, atol=1e-6)
        assert np.all(out.cpu().numpy()[:, D:] == 0)


@pytest.mark.parametrize("name", ["bf16_d1024", "bf16_d2048_n5k4", "prefill_64k_30b"])
def test_prefill_parity_workload(lib, request, name):
    w = WL.workload(name)
    print(f"  {name}: {sum(v * w.d for v in w.V) * 2 / 1e9:.1f} GB of sub-tables", flush=True)
    if name == "prefill_64k_30b":
        E0, E, W = request.getfixturevalue("tables_30b")
    else:
        E0, E, W = WL.device_tables(w)
    cfg = cfg_of(w)
    tok2d = WL.token_batch(w)
    tokens, cu = packed(list(tok2d))
    T = len(tokens)
    out, ws = run_prefill(cfg, E0, E, W, tokens, cu, torch.bfloat16)
    # every index, bit for bit (prefill leaves them in the workspace)
    _, idx_off = g.ngram_embed_workspace_layout(cfg, T)
    got_idx = ws[idx_off:idx_off + T * w.S * 4].view(torch.int32).cpu().numpy().reshape(T, w.S)
    # every row of the launch the benchmark times, element by element (the oracle contracts
    # the whole batch in float64)
    idx, e = oracle_rows(w, E0, E, W, tokens, cu, np.arange(T))
    np.testing.assert_array_equal(got_idx, idx)
    got = to_f64(out)
    del out
    assert_close(got, e, "bf16", name)
    del got, e
    # the stand-alone gather agrees byte for byte with torch indexing on every row
    G = torch.empty((T, w.D), dtype=torch.bfloat16, device="cuda")
    g.ngram_embed_gather(cfg, g.Tables(E0, E, W), ws[idx_off:].view(torch.int32), G)
    torch.cuda.synchronize()
    for s in range(w.S):
        want = E[s].index_select(0, torch.as_tensor(idx[:, s], device="cuda"))
        assert torch.equal(G[:, s * w.d:(s + 1) * w.d].view(torch.int16),
                           want.view(torch.int16)), s
    del G
    # the gather into LDS (the projection's loader) delivers every byte of every row
    sums = torch.empty(T, dtype=torch.int32, device="cuda")
    g.ngram_embed_gather_checksum(cfg, g.Tables(E0, E, W), ws[idx_off:].view(torch.int32), sums)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(sums.cpu().numpy().view(np.uint32),
                                  row_checksums(gathered_words(E, idx)))
    assert g.ngram_embed_read_error_flag(ws) == 0
    del E0, E, W, ws
    torch.cuda.empty_cache()


def test_prefill_is_deterministic(lib):
    w = small_workload("bf16", D=1024, N=3, K=2, V0=32000)
    cfg = cfg_of(w)
    E0, E, W = host_to_dev_tables(w)
    rng = np.random.default_rng(3)
    tokens, cu = packed([rng.integers(0, w.V0, size=5000).astype(np.int32)])
    a, _ = run_prefill(cfg, E0, E, W, tokens, cu, torch.bfloat16)
    b, _ = run_prefill(cfg, E0, E, W, tokens, cu, torch.bfloat16)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_n1_is_plain_lookup(lib):
    for dtype, tdt in (("f32", torch.float32), ("bf16", torch.bfloat16)):
        cfg = g.Config(1, 1, 64, dtype, 500, [])
        E0 = torch.randn(500, 64).to(tdt).cuda()
        rng = np.random.default_rng(2)
        tokens, cu = packed([rng.integers(0, 500, size=L).astype(np.int32) for L in (3, 90)])
        out, _ = run_prefill(cfg, E0, [], E0[:64].contiguous(), tokens, cu, tdt)
        assert torch.equal(out, E0[torch.as_tensor(tokens.astype(np.int64), device="cuda")])


def test_empty_batch_is_a_no_op(lib):
    w = small_workload("bf16")
    cfg = cfg_of(w)
    E0, E, W = host_to_dev_tables(w)
    out = torch.empty((0, w.D), dtype=torch.bfloat16, device="cuda")
    ws = g.alloc_workspace(cfg, 0)
    g.ngram_embed_prefill(cfg, g.Tables(E0, E, W), torch.zeros(0, dtype=torch.int32,
                          device="cuda"), dev(np.array([0, 0], np.int32)), out, ws)
    torch.cuda.synchronize()


def test_bad_token_sets_flag_and_zero_row(lib):
    w = small_workload("bf16", D=256)
    cfg = cfg_of(w)
    E0, E, W = host_to_dev_tables(w)
    rng = np.random.default_rng(9)
    tokens = rng.integers(0, w.V0, size=300).astype(np.int32)
    tokens[100] = w.V0 + 5
    cu = np.array([0, 300], np.int32)
    out, ws = run_prefill(cfg, E0, E, W, tokens, cu, torch.bfloat16)
    assert g.ngram_embed_read_error_flag(ws) & g.NGRAM_FLAG_BAD_TOKEN
    assert torch.count_nonzero(out[100]).item() == 0
    good = tokens.copy()
    good[100] = 0
    # rows whose context does not reach position 100 are unaffected
    _, e = oracle_rows(w, E0, E, W, good, cu, np.arange(0, 100))
    assert_close(to_f64(out[:100]), e, "bf16", "rows before the bad id")
    g.ngram_embed_clear_error_flag(ws)
    assert g.ngram_embed_read_error_flag(ws) == 0


def test_bad_seqlens_sets_flag(lib):
    w = small_workload("f32", D=64)
    cfg = cfg_of(w)
    tokens = np.arange(40, dtype=np.int32)
    idx = torch.empty((40, w.S), dtype=torch.int32, device="cuda")
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    g.ngram_embed_hash(cfg, dev(tokens), dev(np.array([0, 30, 20, 40], np.int32)), idx, flags)
    assert int(flags.item()) & g.NGRAM_FLAG_BAD_SEQLENS


def test_out_of_range_indices_are_clamped(lib):
    """project() clamps each index into its table: V_s + 5 and -1 read row V_s - 1."""
    w = small_workload("bf16", D=1024, N=3, K=2, V0=32000)
    cfg = cfg_of(w)
    E0, E, W = host_to_dev_tables(w)
    T = 100
    rng = np.random.default_rng(4)
    tok = rng.integers(0, w.V0, size=T).astype(np.int32)
    idx = np.stack([rng.integers(0, v, size=T) for v in w.V], axis=1).astype(np.int32)
    bad = idx.copy()
    bad[::3, 0] = w.V[0] + 5
    bad[1::3, 1] = -1
    fixed = bad.copy()
    fixed[::3, 0] = w.V[0] - 1
    fixed[1::3, 1] = w.V[1] - 1
    outs = []
    for ix in (bad, fixed):
        o = torch.empty((T, w.D), dtype=torch.bfloat16, device="cuda")
        g.ngram_embed_project(cfg, g.Tables(E0, E, W), dev(ix), dev(tok), o)
        outs.append(o)
    torch.cuda.synchronize()
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    e = oracle.embed_from_indices(w.D, w.N, w.K, tok, fixed.astype(np.int64),
                                  device_fetch(E0, E), w_blocks(W, w.S))
    assert_close(to_f64(outs[1]), e, "bf16", "clamped")


# Each path of the LDS gather: batches of whole rows (1, 2 and 4 KB rows, 16 sub-tables),
# rows longer than a wave's 10 KB buffer taken in pieces (the basic form's 3 x 6 KB rows),
# fp32 rows, ragged batch sizes, indices past their table (clamped as ngram_embed_gather).
LDS_CASES = [
    ("f32_d64", small_workload("f32", D=64), 257),
    ("bf16_d1024", small_workload("bf16", D=1024, N=3, K=2, V0=32000), 1001),
    ("bf16_d2048_s16", small_workload("bf16", D=2048, N=5, K=4, V0=131072), 333),
    ("bf16_d3072_s12", small_workload("bf16", D=3072, N=4, K=4, V0=131072), 4097),
    # more groups of 5 rows than waves (2048): several groups per wave, a ragged last group
    ("bf16_d3072_s12_multi", small_workload("bf16", D=3072, N=4, K=4, V0=131072), 24003),
    ("bf16_d3072_s12_one_row", small_workload("bf16", D=3072, N=4, K=4, V0=131072), 1),
    ("bf16_d1024_three_rows", small_workload("bf16", D=1024, N=3, K=2, V0=32000), 3),
    ("basic_d3072", WL.Workload("basic_lds", "bf16", 5000, 3072, 4, 1,
                                tuple(WL.mid_gap_primes(5000, 15000, 3)), 1, 1, "uniform", 12,
                                form="basic"), 130),
]


@pytest.mark.parametrize("name,w,T", LDS_CASES, ids=[c[0] for c in LDS_CASES])
def test_gather_checksum_every_row(lib, name, w, T):
    cfg = g.Config(w.N, w.K, w.D, w.dtype, w.V0, list(w.V), form=w.form)
    E0, E, W = host_to_dev_tables(w)
    rng = np.random.default_rng(T)
    idx = np.stack([rng.integers(0, v, size=T) for v in w.V], axis=1).astype(np.int32)
    idx[::97, 0] = w.V[0] + 3                     # past the table: clamped to its last row
    sums = torch.full((T,), 7, dtype=torch.int32, device="cuda")
    g.ngram_embed_gather_checksum(cfg, g.Tables(E0, E, W), dev(idx), sums)
    torch.cuda.synchronize()
    ref_idx = np.minimum(idx, np.asarray(w.V) - 1)
    want = row_checksums(gathered_words(E, ref_idx))
    np.testing.assert_array_equal(sums.cpu().numpy().view(np.uint32), want)
