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


# Element by element (bf16 outputs): the kernel computes v = (E_0 row + product) * scale in
# fp32 and rounds v once to bf16, which moves it by at most half an ulp: for v in
# [2^e, 2^(e+1)) an ulp of bf16's 8 significant bits is 2^(e-7), so |out - v| <= 2^-8 |v|.
# The fp32 accumulation of a 3072-term product (MFMA products are exact; the sums round) is
# about 2^-24 * sqrt(3072 / 16) * |acc| ~ 1e-5 of the output's RMS, so |v - ref| is bounded by
# ELEM_C * rms(ref) with a tenfold margin, and
#     |out - ref| <= 2^-8 |ref| + ELEM_C * rms(ref)     (rms over the compared values).
ELEM_C = 1e-4
# Per row: the relative L2 of each row alone; a row error that a norm over many rows would
# dilute shows here. The element bound above caps it at about 2^-8; bf16 rounding alone gives
# ~1.6e-3 on average.
ROW_TOL = {"f32": 1e-5, "bf16": 3e-3}


def row_rel_l2(out, ref):
    """Relative L2 error of every row (rows with a zero reference use norm 1)."""
    out2 = out.reshape(-1, out.shape[-1]) if out.ndim else out
    ref2 = ref.reshape(-1, ref.shape[-1]) if ref.ndim else ref
    num = np.sqrt(np.sum((out2 - ref2) ** 2, axis=1))
    den = np.sqrt(np.sum(ref2 * ref2, axis=1))
    return num / np.where(den > 0, den, 1.0)


def assert_close(out, ref, dtype, what=""):
    """Relative L2 over everything compared (the targets in TOL), relative L2 of every row
    (ROW_TOL), every element within the bf16 rounding bound (bf16), and max |error|."""
    rl2_tol, abs_tol = TOL[dtype]
    assert out.shape == ref.shape, (what, out.shape, ref.shape)
    assert np.all(np.isfinite(out))
    err = np.abs(out - ref)
    rl2 = rel_l2(out, ref)
    mabs = float(err.max()) if out.size else 0.0
    rows = row_rel_l2(out, ref) if out.size else np.zeros(0)
    rmax = float(rows.max()) if rows.size else 0.0
    msg = f"  {what}: rel_l2={rl2:.3e} max_abs={mabs:.3e} worst_row_rel_l2={rmax:.3e}"
    if dtype == "bf16" and out.size:
        rms = float(np.sqrt(np.mean(ref * ref)))
        excess = err - (2.0 ** -8 * np.abs(ref) + ELEM_C * rms)
        worst = int(np.argmax(excess))
        msg += f" elems={out.size} worst_elem_margin={float(excess.flat[worst]):.2e}"
    print(msg, flush=True)
    assert rl2 <= rl2_tol, (what, rl2)
    if abs_tol is not None:
        assert mabs <= abs_tol, (what, mabs)
    assert rmax <= ROW_TOL[dtype], (what, "row", int(np.argmax(rows)), rmax)
    if dtype == "bf16" and out.size:
        assert float(excess.flat[worst]) <= 0.0, (
            what, "element", np.unravel_index(worst, out.shape), float(out.flat[worst]),
            float(ref.flat[worst]))


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


def row_checksums(words):
    """sum_k w_k (2k + 1) mod 2^32 of every row of a uint32 array [rows, M] (the checksum that
    ngram_embed_gather_checksum takes of each gathered row where it lands)."""
    w = np.asarray(words, dtype=np.uint32).astype(np.uint64)
    k = 2 * np.arange(w.shape[1], dtype=np.uint64) + 1
    return ((w * k).sum(axis=1) % (1 << 32)).astype(np.uint32)


def gathered_words(E, idx):
    """The gathered rows [E_s[idx[:, s]] for every s] as uint32 words, by torch indexing of the
    device tables (not the library)."""
    import torch
    parts = [E[s].index_select(0, torch.as_tensor(np.asarray(idx[:, s], dtype=np.int64),
                                                  device=E[s].device))
             for s in range(len(E))]
    G = torch.cat(parts, dim=1).contiguous()
    return G.view(torch.int32).cpu().numpy().view(np.uint32)
