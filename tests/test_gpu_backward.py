"""GPU parity of the backward (training gradients), through the C ABI, against
oracle.backward on the same seeded inputs.

The inputs (tables, W, upstream gradient) are exact in the config dtype, so the only error is
fp32 accumulation: about u * sqrt(n) relative for n summed terms (u = 2^-24). Bounds: relative
L2 <= 1e-5 for the small cases (n up to a few thousand), <= 1e-4 at the 64K-token batch.
Small cases compare every gradient entry; repeated ids and hash indices are forced with small
vocabularies and tables. Also: bitwise-repeatable results (no atomics), accumulation into the
buffers, N = 1, the sqrt(D) factor, and the 30B-parameter layer at its 64K-token shape
(every gradient row the batch touches, through a relabelled copy of the problem)."""
import numpy as np
import pytest

import gram_embedding_layer_amd as g
import oracle
import workloads as WL
from tests.gpu_helpers import device_fetch, packed, rel_l2, to_f64, w_blocks
from tests.test_gpu_prefill import dev, host_to_dev_tables, small_workload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def grad_buffers(w, dtype=torch.float32):
    dE0 = torch.zeros((w.V0, w.D), dtype=dtype, device="cuda")
    dE = [torch.zeros((v, w.d), dtype=dtype, device="cuda") for v in w.V]
    dW = torch.zeros((w.D, w.D), dtype=dtype, device="cuda")
    return dE0, dE, dW


def upstream(w, T, seed):
    rng = np.random.default_rng(seed)
    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    return torch.as_tensor(rng.normal(0.0, 1.0, size=(T, w.D))).to(dt).cuda()


def run_backward(cfg, tables, tokens, cu, dout, bufs):
    ws = g.alloc_backward_workspace(cfg, len(tokens))
    dE0, dE, dW = bufs
    g.ngram_embed_backward(cfg, tables, dev(tokens), dev(cu), dout, dE0, dE, dW, ws)
    torch.cuda.synchronize()
    return ws


def check(name, got, want, tol):
    r = rel_l2(to_f64(got), want)
    print(f"  {name}: rel_l2={r:.3e}", flush=True)
    assert np.all(np.isfinite(to_f64(got)))
    assert r <= tol, (name, r)


CASES = [
    ("f32_generic", WL.workload("tiny_f32"), None, None),
    ("bf16_dup_d256", small_workload("bf16", D=256, N=3, K=2, V0=50), (300, 1, 0, 77, 1000), None),
    ("bf16_d1024", small_workload("bf16", D=1024, N=3, K=2, V0=32000), (3000, 2100, 5), None),
    ("bf16_n5k4_d2048", small_workload("bf16", D=2048, N=5, K=4, V0=131072), (700, 60), None),
    ("bf16_scaled", small_workload("bf16", D=768, N=4, K=2, V0=300), (500, 400), "scale"),
    ("f32_n1", small_workload("f32", D=64, N=1, K=1), (40, 9), None),
    ("bf16_n1", small_workload("bf16", D=256, N=1, K=1, V0=20), (400, 9), None),
]


@pytest.mark.parametrize("name,w,lengths,amp", CASES, ids=[c[0] for c in CASES])
def test_backward_matches_oracle(lib, name, w, lengths, amp):
    E0, E, W = host_to_dev_tables(w)
    cfg = g.Config(w.N, w.K, w.D, w.dtype, w.V0, list(w.V), amp=amp or "none")
    if lengths is None:
        seqs = list(WL.token_batch(w))
    else:
        rng = np.random.default_rng(len(name))
        seqs = [rng.integers(0, w.V0, size=L).astype(np.int32) for L in lengths]
    tokens, cu = packed(seqs)
    T = len(tokens)
    dout = upstream(w, T, 17)
    bufs = grad_buffers(w)
    ws = run_backward(cfg, g.Tables(E0, E, W), tokens, cu, dout, bufs)
    assert g.ngram_embed_read_error_flag(ws) == 0
    idx = oracle.hash_indices(w.V0, w.N, w.K, w.V, tokens, cu)
    scale = np.sqrt(w.D) if amp == "scale" else 1.0
    dE0_r, dE_r, dW_r = oracle.backward(w.D, w.N, w.K, tokens, idx, to_f64(dout),
                                         device_fetch(E0, E), w_blocks(W, w.S), w.V0, w.V,
                                         scale)
    dE0, dE, dW = bufs
    check(f"{name} dE0", dE0, dE0_r, 1e-5)
    for s in range(w.S):
        check(f"{name} dE[{s}]", dE[s], dE_r[s], 1e-5)
    if w.S:
        dW_ref = np.concatenate(dW_r, axis=1)          # the stacked layout [D, S*d]
        check(f"{name} dW", dW, dW_ref, 1e-5)


def test_backward_runs_ending_on_chunk_boundaries(lib):
    """Repeated ids are summed in chunks of sorted entries (64 for E_0, 32 for sub-tables);
    a run that crosses chunks is finished by the chunk it starts in. Token counts are chosen so
    that E_0 runs end exactly at chunk ends (32 + 96 entries, then 64, then 66 whole chunks,
    which is also longer than the 64 chunks probed at once), and a tiny vocabulary gives long
    sub-table runs that cross many chunks."""
    w = small_workload("bf16", D=256, N=3, K=2, V0=8)
    E0, E, W = host_to_dev_tables(w)
    cfg = g.Config(w.N, w.K, w.D, w.dtype, w.V0, list(w.V))
    counts = {1: 32, 2: 96, 3: 64, 4: 64 * 66, 5: 100, 6: 7}
    multiset = np.concatenate([np.full(c, t, dtype=np.int32) for t, c in counts.items()])
    rng = np.random.default_rng(21)
    rng.shuffle(multiset)
    half = len(multiset) // 2
    tokens, cu = packed([multiset[:half], multiset[half:]])
    dout = upstream(w, len(tokens), 23)
    bufs = grad_buffers(w)
    run_backward(cfg, g.Tables(E0, E, W), tokens, cu, dout, bufs)
    idx = oracle.hash_indices(w.V0, w.N, w.K, w.V, tokens, cu)
    dE0_r, dE_r, dW_r = oracle.backward(w.D, w.N, w.K, tokens, idx, to_f64(dout),
                                         device_fetch(E0, E), w_blocks(W, w.S), w.V0, w.V, 1.0)
    dE0, dE, dW = bufs
    check("aligned dE0", dE0, dE0_r, 1e-5)
    for s in range(w.S):
        check(f"aligned dE[{s}]", dE[s], dE_r[s], 1e-5)


def test_backward_is_repeatable_and_accumulates(lib):
    w = small_workload("bf16", D=256, N=3, K=2, V0=50)
    E0, E, W = host_to_dev_tables(w)
    cfg = g.Config(w.N, w.K, w.D, w.dtype, w.V0, list(w.V))
    rng = np.random.default_rng(4)
    tokens, cu = packed([rng.integers(0, w.V0, size=L).astype(np.int32) for L in (900, 130)])
    dout = upstream(w, len(tokens), 5)
    a, b = grad_buffers(w), grad_buffers(w)
    run_backward(cfg, g.Tables(E0, E, W), tokens, cu, dout, a)
    run_backward(cfg, g.Tables(E0, E, W), tokens, cu, dout, b)
    for x, y in zip([a[0], a[2]] + a[1], [b[0], b[2]] + b[1]):
        assert torch.equal(x, y)                        # no atomics: same bits every run
    run_backward(cfg, g.Tables(E0, E, W), tokens, cu, dout, b)
    for x, y in zip([a[0], a[2]] + a[1], [b[0], b[2]] + b[1]):
        assert torch.equal(2 * x, y)                    # accumulated: x + x, exactly


def test_backward_skips_only_requested_buffers(lib):
    w = small_workload("bf16", D=256, N=3, K=2, V0=50)
    E0, E, W = host_to_dev_tables(w)
    cfg = g.Config(w.N, w.K, w.D, w.dtype, w.V0, list(w.V))
    rng = np.random.default_rng(6)
    tokens, cu = packed([rng.integers(0, w.V0, size=600).astype(np.int32)])
    dout = upstream(w, len(tokens), 7)
    full = grad_buffers(w)
    run_backward(cfg, g.Tables(E0, E, W), tokens, cu, dout, full)
    dE0, dE, dW = grad_buffers(w)
    ws = g.alloc_backward_workspace(cfg, len(tokens))
    g.ngram_embed_backward(cfg, g.Tables(E0, E, W), dev(tokens), dev(cu), dout, None, dE, None, ws)
    g.ngram_embed_backward(cfg, g.Tables(E0, E, W), dev(tokens), dev(cu), dout, dE0, None, dW, ws)
    torch.cuda.synchronize()
    assert torch.equal(dE0, full[0]) and torch.equal(dW, full[2])
    for x, y in zip(dE, full[1]):
        assert torch.equal(x, y)


def test_backward_30b_every_touched_row(lib, tables_30b):
    """The 30B-parameter layer at its 64K-token shape, against oracle.backward on every gradient
    row the batch touches. The batch uses about 13K distinct tokens and 44K distinct rows per
    sub-table of 9.76M, so the oracle runs on a relabelled copy of the problem: ids and hash
    indices are renumbered densely (np.unique), which leaves each position's rows and every sum
    unchanged, and the oracle's rows come back to their table rows through the same map. All of
    dW, every touched row of dE0 and of each dE_s is compared; every other row must stay zero."""
    w = WL.workload("prefill_64k_30b")
    E0, E, W = tables_30b
    cfg = g.Config(w.N, w.K, w.D, w.dtype, w.V0, list(w.V))
    tokens, cu = packed(list(WL.token_batch(w)))
    T = len(tokens)
    dout = upstream(w, T, 23)
    bufs = grad_buffers(w)
    print(f"  backward of {T} tokens: gradient buffers {sum(b.numel() for b in bufs[1]) * 4 / 1e9:.0f} GB",
          flush=True)
    ws = run_backward(cfg, g.Tables(E0, E, W), tokens, cu, dout, bufs)
    assert g.ngram_embed_read_error_flag(ws) == 0
    dE0, dE, dW = bufs
    idx = oracle.hash_indices(w.V0, w.N, w.K, w.V, tokens, cu)
    tok_rows, tok_c = np.unique(tokens, return_inverse=True)
    sub = [np.unique(idx[:, s], return_inverse=True) for s in range(w.S)]
    idx_c = np.stack([inv for _, inv in sub], axis=1)
    fetch = device_fetch(E0, E)

    def fetch_c(s, rows_c):                      # dense row number -> the table's own row
        return fetch(s, sub[s][0][np.asarray(rows_c, dtype=np.int64)])

    dE0_r, dE_r, dW_r = oracle.backward(w.D, w.N, w.K, tok_c, idx_c, to_f64(dout), fetch_c,
                                         w_blocks(W, w.S), len(tok_rows),
                                         [len(rows) for rows, _ in sub], 1.0)

    def touched_rows(t):                         # rows with any nonzero entry, ascending
        norms = torch.linalg.vector_norm(t, dim=1)
        return torch.nonzero(norms).flatten().cpu().numpy()

    def check_rows(name, t, rows, want):
        got = t.index_select(0, torch.as_tensor(rows.astype(np.int64), device=t.device))
        check(name, got, want, 1e-4)
        err = np.abs(to_f64(got) - want).max()
        rms = np.sqrt(np.mean(want * want))
        assert err <= 1e-3 * rms, (name, err, rms)
        extra = np.setdiff1d(touched_rows(t), rows)
        assert extra.size == 0, (name, "rows outside the batch were written", extra[:8])

    dW_ref = np.concatenate(dW_r, axis=1)                # the stacked layout [D, S*d]
    check("30b dW", dW, dW_ref, 1e-4)
    assert np.abs(to_f64(dW) - dW_ref).max() <= 1e-3 * np.sqrt(np.mean(dW_ref * dW_ref))
    check_rows("30b dE0", dE0, tok_rows, dE0_r)
    for s in range(w.S):
        check_rows(f"30b dE[{s}]", dE[s], sub[s][0], dE_r[s])
    del bufs, dE0, dE, dW, ws, dE0_r, dE_r, dW_r, dW_ref
    torch.cuda.empty_cache()
