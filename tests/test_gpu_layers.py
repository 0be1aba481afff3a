"""GPU tests of the per-layer N-gram embedding (PLNE, section 5.2 of the deep-notes page):
several layers, each with embedding tables and projections of its own, computed from one
hash of the token ids with the layers' projections batched into shared launches, through the
C ABI.

Exact where the method is exact: each layer's output equals a single-layer call with that
layer's tables bit for bit (same kernels, same sum order per output), and against
oracle.prefill with that layer's tables within gpu_helpers.TOL. Covered: the matrix-core
path at every tile height, more layers than one launch holds (sub-table pointer and layer
limits), the generic fp32 path, N = 1, the basic form, layer normalisation (layers in turn),
and decode with one commit for all layers."""
import numpy as np
import pytest

import gram_embedding_layer_amd as g
import oracle
import workloads as WL
from tests.gpu_helpers import assert_close, device_fetch, packed, to_f64, w_blocks
from tests.test_gpu_amp import assert_close as close_amp
from tests.test_gpu_basic import basic_workload
from tests.test_gpu_prefill import dev, small_workload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def layer_tables(w, n, amp=None):
    """n layers of seeded tables (a different seed per layer), as g.Tables."""
    out = []
    for l in range(n):
        E0, E, W = WL.host_tables(w, seed=l + 1)
        wt = bs = None
        if amp == "layernorm":
            rng = np.random.default_rng(100 + l)
            dt = E0.dtype
            wt = torch.as_tensor(rng.normal(1.0, 0.5, size=w.D)).to(dt).cuda()
            bs = torch.as_tensor(rng.normal(0.0, 0.5, size=w.D)).to(dt).cuda()
        out.append(g.Tables(E0.cuda(), [e.cuda() for e in E],
                            W.cuda() if W is not None else None, wt, bs))
    return out


def cfg_of(w, amp="none"):
    return g.Config(w.N, w.K, w.D, w.dtype, w.V0, list(w.V), amp=amp, form=w.form)


def tdtype(w):
    return torch.float32 if w.dtype == "f32" else torch.bfloat16


CASES = [
    # name, workload, layers, sequence lengths, amplification
    ("bf16_bm64", small_workload("bf16", D=1024, N=3, K=2, V0=3000), 3, (500, 1, 0, 77), "none"),
    ("bf16_bm128", small_workload("bf16", D=1024, N=3, K=2, V0=3000), 3, (9000, 11), "none"),
    ("bf16_bm256_scaled", small_workload("bf16", D=1024, N=3, K=2, V0=3000), 3,
     (16384, 16384, 5), "scale"),
    ("bf16_s16_9layers", small_workload("bf16", D=2048, N=5, K=4, V0=2000), 9, (700, 3), "none"),
    ("f32_generic", small_workload("f32", D=96, N=4, K=2), 3, (50, 1, 201), "none"),
    ("bf16_n1", small_workload("bf16", D=256, N=1, K=1), 3, (40, 9), "none"),
    ("bf16_n1_scaled", small_workload("bf16", D=256, N=1, K=1), 2, (40, 9), "scale"),
    ("basic_bf16", basic_workload("bf16", D=256, N=4), 2, (300, 2), "none"),
    ("bf16_layernorm", small_workload("bf16", D=1024, N=3, K=2, V0=3000), 3, (900, 7),
     "layernorm"),
]


@pytest.mark.parametrize("name,w,nl,lengths,amp", CASES, ids=[c[0] for c in CASES])
def test_layers_prefill(lib, name, w, nl, lengths, amp):
    tabs = layer_tables(w, nl, amp)
    cfg = cfg_of(w, amp)
    rng = np.random.default_rng(len(name))
    tokens, cu = packed([rng.integers(0, w.V0, size=L).astype(np.int32) for L in lengths])
    T = len(tokens)
    dt = tdtype(w)
    ws = g.alloc_workspace(cfg, T)
    outs = [torch.full((T, w.D), 7.0, dtype=dt, device="cuda") for _ in range(nl)]
    g.ngram_embed_prefill_layers(cfg, tabs, dev(tokens), dev(cu), outs, ws)
    single = torch.empty((T, w.D), dtype=dt, device="cuda")
    rows = np.arange(T) if T <= 2000 else np.unique(np.concatenate(
        [cu[:-1][np.diff(cu) > 0], cu[1:] - 1, rng.choice(T, 600, replace=False)]))
    rows = rows[(rows >= 0) & (rows < T)]
    idx = oracle.hash_indices(w.V0, w.N, w.K, w.V, tokens, cu)
    for l, tab in enumerate(tabs):
        g.ngram_embed_prefill(cfg, tab, dev(tokens), dev(cu), single, ws)
        torch.cuda.synchronize()
        assert torch.equal(bits(outs[l]), bits(single)), f"layer {l}"
        fetch = device_fetch(tab.E0, tab.E)
        if w.form == "basic":
            e = oracle.embed_basic(w.D, w.N, tokens[rows], idx[rows], fetch)
        else:
            e = oracle.embed_from_indices(w.D, w.N, w.K, tokens[rows], idx[rows], fetch,
                                          w_blocks(tab.W, w.S))
        if amp == "scale":
            e = oracle.amplify(e, "scale", scale=np.sqrt(w.D))
        if amp == "layernorm":
            want = oracle.amplify(e, "layernorm", eps=1e-5, weight=to_f64(tab.ln_weight),
                                  bias=to_f64(tab.ln_bias))
            close_amp(to_f64(outs[l])[rows], want, w.dtype, f"{name} layer {l}")
        elif amp == "scale":
            close_amp(to_f64(outs[l])[rows], e, w.dtype, f"{name} layer {l}")
        else:
            assert_close(to_f64(outs[l])[rows], e, w.dtype, f"{name} layer {l}")
    assert g.ngram_embed_read_error_flag(ws) == 0


@pytest.mark.parametrize("nl,nseq", [(3, 6), (8, 40)], ids=["3layers", "8layers_bm64"])
def test_layers_decode(lib, nl, nseq):
    w = small_workload("bf16", D=1024, N=3, K=2, V0=3000)
    tabs = layer_tables(w, nl)
    cfg = cfg_of(w)
    rng = np.random.default_rng(nl)
    hists = [rng.integers(0, w.V0, size=int(L)).astype(np.int32)
             for L in rng.integers(0, 50, size=nseq)]
    htok, hcu = packed(hists)
    tmax = 5
    caches = [g.Cache.empty(cfg, nseq) for _ in range(2)]
    for c in caches:
        g.ngram_cache_init(cfg, c, dev(htok), dev(hcu))
    orc = oracle.DecodeOracle(w.V0, w.D, w.N, w.K, w.V, hists)
    ws = g.alloc_workspace(cfg, nseq * tmax)
    for step in range(2):
        new = rng.integers(0, w.V0, size=(nseq, tmax)).astype(np.int32)
        n_new = rng.integers(0, tmax + 1, size=nseq).astype(np.int32)
        n_acc = np.array([rng.integers(0, n + 1) for n in n_new], dtype=np.int32)
        outs = [torch.full((nseq, tmax, w.D), 7.0, dtype=torch.bfloat16, device="cuda")
                for _ in range(nl)]
        g.ngram_embed_decode_layers(cfg, tabs, caches[0], dev(new), dev(n_new), outs, ws,
                                    n_commit=dev(n_acc))
        per = [list(new[b, :n_new[b]]) for b in range(nseq)]
        for l, tab in enumerate(tabs):
            single = torch.empty_like(outs[0])
            # the reference cache advances only after the last layer
            g.ngram_embed_decode(cfg, tab, caches[1], dev(new), dev(n_new), single, ws,
                                 n_commit=dev(n_acc) if l == nl - 1 else None)
            torch.cuda.synchronize()
            assert torch.equal(bits(outs[l]), bits(single)), (step, l)
        _, embs = orc.step(per, device_fetch(tabs[0].E0, tabs[0].E), w_blocks(tabs[0].W, w.S))
        got = to_f64(outs[0])
        for b in range(nseq):
            k = int(n_new[b])
            assert np.all(got[b, k:] == 0)
            if k:
                assert_close(got[b, :k], embs[b], "bf16", f"step {step} seq {b}")
        orc.commit(per, n_acc)
        assert torch.equal(caches[0].len, caches[1].len)
        assert torch.equal(caches[0].ring, caches[1].ring)
    assert g.ngram_embed_read_error_flag(ws) == 0
