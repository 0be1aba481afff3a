"""GPU parity of the embedding amplification (section 3.2.4 of the deep-notes page: the layer
output scaled, or layer-normalised over D, before it joins the residual stream), through the
C ABI, against oracle.amplify applied to the float64 oracle of the layer.

Every kernel path is covered: the fp32 and bf16 generic projections, each matrix-core tile
height (64, 128, 256 rows) with ragged tails, N = 1, decode, and the 30B-parameter layer at
its full 64K-token shape (every row). Tolerances as for the plain layer (gpu_helpers.TOL):
both modes round once, from fp32 values; the bf16 elementwise bound scales with the value
(see assert_close)."""
import numpy as np
import pytest

import gram_embedding_layer_amd as g
import oracle
import workloads as WL
from tests.gpu_helpers import (ROW_TOL, TOL, device_fetch, oracle_rows, packed, rel_l2,
                               row_rel_l2, to_f64, w_blocks)
from tests.test_gpu_prefill import dev, host_to_dev_tables, small_workload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def assert_close(out, ref, dtype, what=""):
    """Relative L2 as for the plain layer (gpu_helpers.TOL), and for bf16 an elementwise
    bound that scales with the value, since amplified outputs are O(1)..O(10) rather than
    O(0.01): one rounding to bf16 moves a value by at most half an ulp, 2^-8 of it; 1e-3 of
    the output's RMS allows for the fp32 error before that rounding."""
    rl2 = rel_l2(out, ref)
    err = np.abs(out - ref)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    rows = row_rel_l2(out, ref) if ref.size else np.zeros(0)
    rmax = float(rows.max()) if rows.size else 0.0
    print(f"  {what}: rel_l2={rl2:.3e} max_abs={float(err.max()) if err.size else 0:.3e} "
          f"rms={rms:.3e} worst_row_rel_l2={rmax:.3e}", flush=True)
    assert np.all(np.isfinite(out))
    assert rl2 <= TOL[dtype][0], (what, rl2)
    assert rmax <= ROW_TOL[dtype], (what, "row", int(np.argmax(rows)), rmax)
    if dtype == "bf16":
        bound = 2.0 ** -8 * np.abs(ref) + 1e-3 * rms
        assert bool(np.all(err <= bound)), (what, float((err - bound).max()))


def amp_cfg(w, mode, scale=None, eps=1e-5):
    return g.Config(w.N, w.K, w.D, w.dtype, w.V0, list(w.V), amp=mode, amp_scale=scale,
                    ln_eps=eps)


def ln_params(w, affine, seed=5):
    """Seeded layer-norm weight and bias [D] in the layer's dtype, or (None, None)."""
    if not affine:
        return None, None
    rng = np.random.default_rng(seed)
    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    wt = torch.as_tensor(rng.normal(1.0, 0.5, size=w.D)).to(dt).cuda()
    bs = torch.as_tensor(rng.normal(0.0, 0.5, size=w.D)).to(dt).cuda()
    return wt, bs


def expected(e, mode, D, scale, eps, wt, bs):
    if mode == "scale":
        return oracle.amplify(e, "scale", scale=np.sqrt(D) if scale is None else scale)
    return oracle.amplify(e, "layernorm", eps=eps,
                          weight=None if wt is None else to_f64(wt),
                          bias=None if bs is None else to_f64(bs))


def run(cfg, tables, tokens, cu, dtype):
    T = len(tokens)
    out = torch.full((T, cfg.D), 3.0, dtype=dtype, device="cuda")
    ws = g.alloc_workspace(cfg, T)
    g.ngram_embed_prefill(cfg, tables, dev(tokens), dev(cu), out, ws)
    torch.cuda.synchronize()
    return out, ws


CASES = [
    ("f32_generic", small_workload("f32", D=96, N=4, K=2), (50, 1, 0, 201)),
    ("bf16_generic_d32", small_workload("bf16", D=128, N=3, K=2), (300, 2, 77)),
    ("bf16_mfma_bm64_bn64", small_workload("bf16", D=1024, N=3, K=2, V0=32000), (300, 1, 0, 450)),
    ("bf16_mfma_bm64", small_workload("bf16", D=1024, N=3, K=2, V0=32000), (700, 1, 0, 1301)),
    ("bf16_mfma_bm128", small_workload("bf16", D=1024, N=3, K=2, V0=32000), (4000, 4100, 3)),
    ("bf16_mfma_bm256", small_workload("bf16", D=1024, N=3, K=2, V0=32000),
     (16384, 16384, 999)),
    ("f32_n1", small_workload("f32", D=64, N=1, K=1), (40, 9)),
    ("bf16_n1", small_workload("bf16", D=256, N=1, K=1), (40, 9)),
    # rows wider than the normalisation pass keeps its parameters in registers for (bf16 past
    # D = 3072, fp32 past D = 1024): the parameters are loaded where they are used
    ("bf16_wide_d4096", small_workload("bf16", D=4096, N=3, K=2), (300, 7)),
    ("f32_wide_d2048", small_workload("f32", D=2048, N=2, K=1), (90, 3)),
    # the widest rows of the pass: 24 and 32 vectors per lane (up to D = 8192)
    ("f32_wide_d5120", small_workload("f32", D=5120, N=3, K=2), (20, 3)),
    ("bf16_wide_d6144", small_workload("bf16", D=6144, N=3, K=2), (40, 7)),
    ("bf16_wide_d8192", small_workload("bf16", D=8192, N=3, K=2), (30, 5)),
]
MODES = [("scale", None, False), ("scale", -0.75, False), ("layernorm", None, False),
         ("layernorm", None, True)]


@pytest.mark.parametrize("mode,scale,affine", MODES,
                         ids=["sqrtD", "neg_factor", "ln_plain", "ln_affine"])
@pytest.mark.parametrize("name,w,lengths", CASES, ids=[c[0] for c in CASES])
def test_amp_prefill_parity(lib, name, w, lengths, mode, scale, affine):
    E0, E, W = host_to_dev_tables(w)
    wt, bs = ln_params(w, affine)
    cfg = amp_cfg(w, mode, scale, eps=1e-5)
    rng = np.random.default_rng(len(name))
    seqs = [rng.integers(0, w.V0, size=L).astype(np.int32) for L in lengths]
    tokens, cu = packed(seqs)
    T = len(tokens)
    out, ws = run(cfg, g.Tables(E0, E, W, wt, bs), tokens, cu, E0.dtype)
    _, e = oracle_rows(w, E0, E, W, tokens, cu, np.arange(T))       # every row
    want = expected(e, mode, w.D, scale, 1e-5, wt, bs)
    assert_close(to_f64(out), want, w.dtype, f"{name} {mode}")
    assert g.ngram_embed_read_error_flag(ws) == 0


def test_amp_bad_token_row_is_zero(lib):
    """Rows of ids outside [0, V0) stay zero after the normalisation (not the bias)."""
    w = small_workload("bf16", D=1024, N=3, K=2, V0=32000)
    E0, E, W = host_to_dev_tables(w)
    wt, bs = ln_params(w, True)
    cfg = amp_cfg(w, "layernorm")
    rng = np.random.default_rng(9)
    tokens = rng.integers(0, w.V0, size=300).astype(np.int32)
    tokens[[5, 123]] = [w.V0, -4]
    out, ws = run(cfg, g.Tables(E0, E, W, wt, bs), tokens, np.array([0, 300], np.int32),
                  torch.bfloat16)
    got = to_f64(out)
    assert np.all(got[[5, 123]] == 0)
    assert g.ngram_embed_read_error_flag(ws) & g.NGRAM_FLAG_BAD_TOKEN
    assert np.all(np.isfinite(got))


@pytest.mark.parametrize("mode", ["scale", "layernorm"])
def test_amp_decode_matches_oracle(lib, mode):
    w = small_workload("bf16", D=1024, N=3, K=2, V0=32000)
    E0, E, W = host_to_dev_tables(w)
    wt, bs = ln_params(w, mode == "layernorm")
    cfg = amp_cfg(w, mode)
    tables = g.Tables(E0, E, W, wt, bs)
    rng = np.random.default_rng(21)
    hists = [rng.integers(0, w.V0, size=L).astype(np.int32) for L in (0, 1, 5, 40, 2, 9)]
    nseq, tmax = len(hists), 5
    htok, hcu = packed(hists)
    cache = g.Cache.empty(cfg, nseq)
    g.ngram_cache_init(cfg, cache, dev(htok), dev(hcu))
    orc = oracle.DecodeOracle(w.V0, w.D, w.N, w.K, w.V, hists)
    fetch, Wb = device_fetch(E0, E), w_blocks(W, w.S)
    ws = g.alloc_workspace(cfg, nseq * tmax)
    for step in range(3):
        n_new = rng.integers(0, tmax + 1, size=nseq).astype(np.int32)
        new = rng.integers(0, w.V0, size=(nseq, tmax)).astype(np.int32)
        out = torch.full((nseq, tmax, w.D), 3.0, dtype=torch.bfloat16, device="cuda")
        g.ngram_embed_decode(cfg, tables, cache, dev(new), dev(n_new), out, ws,
                             n_commit=dev(n_new))
        torch.cuda.synchronize()
        _, embs = orc.step([list(new[b, :n_new[b]]) for b in range(nseq)], fetch, Wb)
        got = to_f64(out)
        for b in range(nseq):
            k = int(n_new[b])
            assert np.all(got[b, k:] == 0), (step, b)
            if k:
                want = expected(embs[b], mode, w.D, None, 1e-5, wt, bs)
                assert_close(got[b, :k], want, "bf16", f"step {step} seq {b}")
        orc.commit([list(new[b, :n_new[b]]) for b in range(nseq)], n_new)
    assert g.ngram_embed_read_error_flag(ws) == 0


def test_amp_layernorm_30b_prefill(lib, tables_30b):
    """The 30B-parameter layer at its 64K-token shape (256-row tiles writing fp32 rows,
    then the normalisation): every row, element by element."""
    w = WL.workload("prefill_64k_30b")
    E0, E, W = tables_30b
    wt, bs = ln_params(w, True)
    cfg = amp_cfg(w, "layernorm")
    tokens, cu = packed(list(WL.token_batch(w)))
    T = len(tokens)
    out, ws = run(cfg, g.Tables(E0, E, W, wt, bs), tokens, cu, torch.bfloat16)
    assert T == 65536
    _, e = oracle_rows(w, E0, E, W, tokens, cu, np.arange(T))
    want = expected(e, "layernorm", w.D, None, 1e-5, wt, bs)
    del e
    got = to_f64(out)
    del out
    assert_close(got, want, "bf16", "30b ln")
    assert g.ngram_embed_read_error_flag(ws) == 0
    del ws, got, want
    torch.cuda.empty_cache()
