"""Shared pieces of the GPU parity tests: oracle inputs from the same seeded data the HIP
library reads, tolerances, and comparison helpers. Expected values come only from oracle/."""
import numpy as np

import gram_embedding_layer_amd as g
import oracle

# Tolerances of the output embeddings against the float64 oracle.
#  fp32 paths: relative L2 <= 1e-5.
#  bf16 paths: relative L2 <= 2e-3 and max |error| <= 3e-2. The max-abs bound is loose at
#  these init scales (|e| ~ 0.01), so relative L2 is the binding check. One rounding to bf16
#  (8 significant bits: error up to half an ulp, an ulp being 2^-7..2^-8 of the value) costs
#  about 1.6e-3 relative L2 on normally distributed values; fp32 accumulation adds ~1e-6.
#  So the output must be rounded exactly once, after the E_0 add and the scale.
TOL = {"f32": (1e-5, None), "bf16": (2e-3, 3e-2)}


def cfg_of(w):
    return g.Config(w.N, w.K, w.D, w.dtype, w.V0, list(w.V))


def to_f64(t):
    """Exact widening of a bf16/fp32 tensor to a float64 numpy array."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def device_fetch(E0, E):
    """Row fetch for the oracle: torch indexing of the device tables (not the library)."""
    import torch

    def fetch(s, rows):
        tab = E0 if s < 0 else E[s]
        r = torch.as_tensor(np.asarray(rows, dtype=np.int64), device=tab.device)
        return to_f64(tab.index_select(0, r))
    return fetch


def w_blocks(W, S):
    if S == 0:                     # N = 1: no sub-tables, no projections
        return []
    Wh = to_f64(W)
    d = Wh.shape[1] // S
    return [Wh[:, s * d:(s + 1) * d] for s in range(S)]


def rel_l2(out, ref):
    n = np.linalg.norm(ref)
    return float(np.linalg.norm(out - ref) / (n if n > 0 else 1.0))


def assert_close(out, ref, dtype, what=""):
    rl2_tol, abs_tol = TOL[dtype]
    rl2 = rel_l2(out, ref)
    mabs = float(np.max(np.abs(out - ref))) if out.size else 0.0
    print(f"  {what}: rel_l2={rl2:.3e} max_abs={mabs:.3e}", flush=True)
    assert np.all(np.isfinite(out))
    assert rl2 <= rl2_tol, (what, rl2)
    if abs_tol is not None:
        assert mabs <= abs_tol, (what, mabs)


def packed(seqs):
    tokens = np.concatenate([np.asarray(s, dtype=np.int32) for s in seqs]) if seqs else \
        np.zeros(0, np.int32)
    cu = np.zeros(len(seqs) + 1, dtype=np.int32)
    cu[1:] = np.cumsum([len(s) for s in seqs])
    return tokens, cu


def ws_indices(ws, cfg, rows):
    """(tok, idx) that a decode call left in the workspace (layout from the library)."""
    import torch
    tok_off, idx_off = g.ngram_embed_workspace_layout(cfg, rows)
    tok = ws[tok_off:tok_off + rows * 4].view(torch.int32).cpu().numpy()
    idx = ws[idx_off:idx_off + rows * cfg.S * 4].view(torch.int32).cpu().numpy()
    return tok, idx.reshape(rows, cfg.S)


def oracle_rows(w, E0, E, W, tokens, cu, rows):
    """Oracle indices for every position and embeddings for the chosen rows."""
    idx = oracle.hash_indices(w.V0, w.N, w.K, w.V, tokens, cu)
    rows = np.asarray(rows, dtype=np.int64)
    e = oracle.embed_from_indices(w.D, w.N, w.K, tokens[rows], idx[rows],
                                  device_fetch(E0, E), w_blocks(W, w.S))
    return idx, e
