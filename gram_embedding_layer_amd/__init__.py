"""MI355X (gfx950) N-gram embedding forward pass: Python binding of libngram_embed.so.

Argument marshalling only: every step of the layer runs in the HIP kernels behind the C ABI
declared in include/ngram_embed.h; PyTorch supplies device memory and streams. There is no
fallback: if the library is missing, load() raises.

The layer (section A2 of the deep-notes page on "Scaling Embeddings Outperforms Scaling
Experts in Language Models"): e_i = (E_0(t_i) + sum_{n,k} W_{n,k} E_{n,k}(H_{n,k})) / ((N-1)K+1)
with H_{n,k} the polynomial rolling hash modulo V_{n,k}; optionally amplified (section 3.2.4:
an output factor such as sqrt(D), or a layer normalisation over D).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

__all__ = [
    "LIB_PATH", "NgramError", "Config", "Tables", "Cache", "load",
    "NGRAM_OK", "NGRAM_F32", "NGRAM_BF16", "AMP_MODES",
    "NGRAM_FLAG_BAD_TOKEN", "NGRAM_FLAG_BAD_SEQLENS", "NGRAM_FLAG_BAD_COUNT",
    "NGRAM_FLAG_BAD_SLOT", "NGRAM_FLAG_DUP_SLOT", "ngram_embed_decode_rows", "ngram_cache_init_slots",
    "ngram_cache_commit_slots", "ngram_embed_prefill_layers", "ngram_embed_decode_layers",
    "NGRAM_FORM_FINAL", "NGRAM_FORM_BASIC", "FORMS", "ngram_hash_stats_workspace_size",
    "ngram_hash_stats",
    "ngram_embed_workspace_size", "ngram_embed_workspace_layout", "ngram_embed_hash",
    "ngram_embed_gather", "ngram_embed_gather_checksum", "ngram_embed_project", "ngram_embed_prefill", "ngram_cache_init",
    "ngram_embed_decode", "ngram_cache_commit", "ngram_embed_read_error_flag",
    "ngram_embed_clear_error_flag", "ngram_embed_status_string", "alloc_workspace",
    "ngram_embed_backward_workspace_size", "ngram_embed_backward", "alloc_backward_workspace",
    "ngram_embed_decode_noalloc", "NGRAM_ESCRATCH", "NGRAM_NOALLOC_SCRATCH_BYTES",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libngram_embed.so")

NGRAM_OK = 0
NGRAM_ESCRATCH = -7                       # the step needs more than the fixed scratch
NGRAM_NOALLOC_SCRATCH_BYTES = 16 << 20    # scratch of ngram_embed_decode_noalloc, per GPU
NGRAM_F32, NGRAM_BF16 = 0, 1
NGRAM_FLAG_BAD_TOKEN, NGRAM_FLAG_BAD_SEQLENS, NGRAM_FLAG_BAD_COUNT = 1, 2, 4
NGRAM_FLAG_BAD_SLOT = 8
NGRAM_FLAG_DUP_SLOT = 16
NGRAM_MAX_DECODE_TOKENS = 8
# amp_scale value that makes the library use sqrt(D) (NGRAM_AMP_SCALE_SQRT_D)
NGRAM_AMP_SCALE_SQRT_D = 0.0
# embedding amplification modes (NGRAM_AMP_NONE / SCALE / LAYERNORM)
AMP_MODES = {"none": 0, "scale": 1, "layernorm": 2}
# forms of the layer (NGRAM_FORM_FINAL / NGRAM_FORM_BASIC)
NGRAM_FORM_FINAL, NGRAM_FORM_BASIC = 0, 1
FORMS = {"final": NGRAM_FORM_FINAL, "basic": NGRAM_FORM_BASIC}


class NgramError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: status {status} ({ngram_embed_status_string(status)})")


class _CConfig(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int32), ("K", ctypes.c_int32), ("D", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("V0", ctypes.c_int64),
                ("V", ctypes.POINTER(ctypes.c_int64)), ("amp", ctypes.c_int32),
                ("amp_scale", ctypes.c_float), ("ln_eps", ctypes.c_float),
                ("form", ctypes.c_int32)]


class _CTables(ctypes.Structure):
    _fields_ = [("E0", ctypes.c_void_p), ("E", ctypes.POINTER(ctypes.c_void_p)),
                ("W", ctypes.c_void_p), ("ln_weight", ctypes.c_void_p),
                ("ln_bias", ctypes.c_void_p)]


class _CCache(ctypes.Structure):
    _fields_ = [("ring", ctypes.c_void_p), ("len", ctypes.c_void_p), ("nseq", ctypes.c_int32)]


_lib = None


def load():
    """Load libngram_embed.so (after torch, so both use the same HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    try:
        import torch  # noqa: F401  (binds libamdhip64 first)
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m gram_embedding_layer_amd.build` (no fallback exists)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    cfgp = ctypes.POINTER(_CConfig)
    tabp = ctypes.POINTER(_CTables)
    cachep = ctypes.POINTER(_CCache)
    sig = {
        "ngram_embed_workspace_size": (SZ, [cfgp, I64]),
        "ngram_embed_workspace_layout": (ctypes.c_int, [cfgp, I64, ctypes.POINTER(SZ),
                                                        ctypes.POINTER(SZ)]),
        "ngram_embed_hash": (ctypes.c_int, [cfgp, P, P, I32, I64, P, P, P]),
        "ngram_embed_gather": (ctypes.c_int, [cfgp, tabp, P, I64, P, P]),
        "ngram_embed_gather_checksum": (ctypes.c_int, [cfgp, tabp, P, I64, P, P]),
        "ngram_embed_project": (ctypes.c_int, [cfgp, tabp, P, P, I64, P, P]),
        "ngram_embed_prefill": (ctypes.c_int, [cfgp, tabp, P, P, I32, I64, P, cachep, P,
                                                SZ, P]),
        "ngram_cache_init": (ctypes.c_int, [cfgp, cachep, P, P, I64, P]),
        "ngram_embed_decode": (ctypes.c_int, [cfgp, tabp, cachep, P, P, I32, P, P, P, SZ, P]),
        "ngram_cache_commit": (ctypes.c_int, [cfgp, cachep, P, P, I32, P, P]),
        "ngram_embed_decode_rows": (ctypes.c_int, [cfgp, tabp, cachep, P, I32, P, P, I32, I32,
                                                   I32, P, P, P, SZ, P]),
        "ngram_cache_init_slots": (ctypes.c_int, [cfgp, cachep, P, I32, P, P, I64, P, P]),
        "ngram_cache_commit_slots": (ctypes.c_int, [cfgp, cachep, P, I32, P, P, I32, P, P]),
        "ngram_embed_prefill_layers": (ctypes.c_int, [cfgp, tabp, I32, P, P, I32, I64,
                                                      ctypes.POINTER(P), P, SZ, P]),
        "ngram_embed_decode_layers": (ctypes.c_int, [cfgp, tabp, I32, cachep, P, P, I32, P,
                                                     ctypes.POINTER(P), P, SZ, P]),
        "ngram_hash_stats_workspace_size": (SZ, [I64, I32, I64, ctypes.POINTER(I64), I32]),
        "ngram_hash_stats": (ctypes.c_int, [I64, I32, P, P, I32, I64, ctypes.POINTER(I64), I32,
                                            P, P, P, SZ, P]),
        "ngram_embed_backward_workspace_size": (SZ, [cfgp, I64]),
        "ngram_embed_backward": (ctypes.c_int, [cfgp, tabp, P, P, I32, I64, P, P,
                                                ctypes.POINTER(P), P, P, SZ, P]),
        "ngram_embed_decode_noalloc": (ctypes.c_int, [cfgp, tabp, cachep, P, P, I32, P, P, P,
                                                      P]),
        "ngram_embed_read_error_flag": (ctypes.c_int, [P, ctypes.POINTER(I32), P]),
        "ngram_embed_clear_error_flag": (ctypes.c_int, [P, P]),
        "ngram_embed_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    _lib = lib
    return lib


# ------------------------------------------------------------------ argument objects

@dataclass
class Config:
    """Mirror of ngram_embed_config: N, K, D, dtype ("f32"/"bf16" or 0/1), V0, V_{n,k}, the
    amplification (amp in AMP_MODES, amp_scale (None: the library applies sqrt(D)), ln_eps)
    and the form
    ("final", or "basic": Eq. 1 with K = 1, full-width tables, no projection)."""
    N: int
    K: int
    D: int
    dtype: object
    V0: int
    V: Sequence[int]
    amp: object = "none"
    amp_scale: Optional[float] = None    # None: the library's sqrt(D)
    ln_eps: float = 1e-5
    form: object = "final"

    @property
    def S(self) -> int:
        return (self.N - 1) * self.K

    @property
    def form_code(self) -> int:
        return FORMS[self.form] if isinstance(self.form, str) else int(self.form)

    @property
    def d(self) -> int:
        if not self.S:
            return 0
        return self.D if self.form_code == NGRAM_FORM_BASIC else self.D // self.S

    @property
    def dtype_code(self) -> int:
        if self.dtype in ("f32", "float32", NGRAM_F32):
            return NGRAM_F32
        if self.dtype in ("bf16", "bfloat16", NGRAM_BF16):
            return NGRAM_BF16
        return int(self.dtype) if isinstance(self.dtype, int) else -1

    @property
    def amp_code(self) -> int:
        return AMP_MODES[self.amp] if isinstance(self.amp, str) else int(self.amp)

    def _c(self):
        arr = (ctypes.c_int64 * max(1, len(self.V)))(*[int(v) for v in self.V])
        # None: the C side's sentinel 0, which selects the pages' factor sqrt(D)
        scale = NGRAM_AMP_SCALE_SQRT_D if self.amp_scale is None else float(self.amp_scale)
        c = _CConfig(int(self.N), int(self.K), int(self.D), self.dtype_code, int(self.V0),
                     ctypes.cast(arr, ctypes.POINTER(ctypes.c_int64)), self.amp_code, scale,
                     float(self.ln_eps), self.form_code)
        return c, arr


@dataclass
class Tables:
    """E0 [V0, D], E = S sub-tables [V_s, d], W [D, D] stacked; optional layer-norm weight
    and bias [D] (device tensors)."""
    E0: object
    E: Sequence[object]
    W: object
    ln_weight: object = None
    ln_bias: object = None

    def _c(self):
        arr = (ctypes.c_void_p * max(1, len(self.E)))(*[_ptr(e) for e in self.E])
        return _CTables(_ptr(self.E0), ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)),
                        _ptr(self.W), _ptr(self.ln_weight), _ptr(self.ln_bias)), arr


@dataclass
class Cache:
    """N-gram cache: ring int32 [nseq, N-1], len int64 [nseq] (device tensors)."""
    ring: object
    len: object

    @staticmethod
    def empty(cfg: Config, nseq: int, device="cuda") -> "Cache":
        import torch
        return Cache(torch.zeros((nseq, max(cfg.N - 1, 0)), dtype=torch.int32, device=device),
                     torch.zeros((nseq,), dtype=torch.int64, device=device))

    @property
    def nseq(self) -> int:
        return int(self.len.shape[0])

    def _c(self):
        ring = _ptr(self.ring) if self.ring is not None and self.ring.numel() else None
        return _CCache(ring, _ptr(self.len), self.nseq)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return int(t.data_ptr())


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return int(getattr(stream, "cuda_stream", stream))
    import torch
    return int(torch.cuda.current_stream().cuda_stream)


def _check(fn: str, rc: int):
    if rc != NGRAM_OK:
        raise NgramError(fn, rc)


def _torch_dtype(code: int):
    import torch
    return torch.float32 if code == NGRAM_F32 else torch.bfloat16


def _arg(fn: str, name: str, t, dtype=None, shape=None, min_numel=None, min_bytes=None,
         optional=False):
    """Check a tensor argument before its pointer crosses the C ABI: the C side sees only
    addresses, so a wrong dtype (int64 ids read as pairs of int32), a short buffer or a host
    tensor would otherwise read or write out of bounds. Checks, in this order: a tensor (or
    None when optional), dtype, shape (None entries match any size) or a minimum element
    count / byte size, contiguity, a CUDA device. Raises ValueError naming fn and the
    argument."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{fn}: {name} is required")
    if not hasattr(t, "data_ptr") or not hasattr(t, "is_contiguous"):
        raise ValueError(f"{fn}: {name} must be a torch tensor, got {type(t).__name__}")
    if dtype is not None:
        allowed = dtype if isinstance(dtype, (tuple, list)) else (dtype,)
        if t.dtype not in allowed:
            raise ValueError(f"{fn}: {name} must have dtype "
                             f"{' or '.join(str(d) for d in allowed)}, got {t.dtype}")
    if shape is not None:
        if t.dim() != len(shape) or any(w is not None and int(n) != int(w)
                                         for n, w in zip(t.shape, shape)):
            want = ", ".join("*" if w is None else str(w) for w in shape)
            raise ValueError(f"{fn}: {name} must have shape "
                             f"({want}{',' if len(shape) == 1 else ''}), got {tuple(t.shape)}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{fn}: {name} needs at least {min_numel} elements, has {t.numel()}")
    if min_bytes is not None and t.numel() * t.element_size() < min_bytes:
        raise ValueError(f"{fn}: {name} needs at least {min_bytes} bytes")
    if not t.is_contiguous():
        raise ValueError(f"{fn}: {name} must be contiguous")
    if not t.is_cuda:
        raise ValueError(f"{fn}: {name} must be on a CUDA (HIP) device, got {t.device}")


def _i32():
    import torch
    return torch.int32


def _i64():
    import torch
    return torch.int64


def _ids_arg(fn, tokens, cu_seqlens):
    """tokens int32 [ntok], cu_seqlens int32 [nseq + 1]."""
    _arg(fn, "tokens", tokens, _i32(), shape=(None,))
    _arg(fn, "cu_seqlens", cu_seqlens, _i32(), shape=(None,), min_numel=1)


def _flags_arg(fn, name, t):
    """An int32 flag word, or a workspace whose first 4 bytes are the flags."""
    import torch
    _arg(fn, name, t, (torch.int32, torch.uint8), min_bytes=4, optional=True)


def _ws_arg(fn, ws):
    _arg(fn, "ws", ws, min_bytes=1)


def _tables_arg(fn, cfg, tables, layer=""):
    """E0 [>= V0, D], E[s] [>= V_s, d], W [D, D] (final form with sub-tables), optional
    layer-norm weight / bias [D], all in the config's dtype."""
    dt = _torch_dtype(cfg.dtype_code)
    if cfg.dtype_code not in (NGRAM_F32, NGRAM_BF16):
        return                       # the C side reports the dtype
    _arg(fn, f"tables{layer}.E0", tables.E0, dt, shape=(None, cfg.D))
    if tables.E0.shape[0] < cfg.V0:
        raise ValueError(f"{fn}: tables{layer}.E0 needs {cfg.V0} rows")
    if len(tables.E) < cfg.S:
        raise ValueError(f"{fn}: tables{layer}.E needs {cfg.S} sub-tables")
    for s in range(cfg.S):
        _arg(fn, f"tables{layer}.E[{s}]", tables.E[s], dt, shape=(None, cfg.d))
        if tables.E[s].shape[0] < int(cfg.V[s]):
            raise ValueError(f"{fn}: tables{layer}.E[{s}] needs {int(cfg.V[s])} rows")
    if cfg.form_code == NGRAM_FORM_FINAL:       # W: read only when there are sub-tables
        _arg(fn, f"tables{layer}.W", tables.W, dt, shape=(cfg.D, cfg.D) if cfg.S else None)
    _arg(fn, f"tables{layer}.ln_weight", tables.ln_weight, dt, shape=(cfg.D,), optional=True)
    _arg(fn, f"tables{layer}.ln_bias", tables.ln_bias, dt, shape=(cfg.D,), optional=True)


def _cache_arg(fn, cfg, cache):
    """ring int32 [nseq, N-1] (absent when N = 1), len int64 [nseq]."""
    _arg(fn, "cache.len", cache.len, _i64(), shape=(None,))
    if cfg.N > 1:
        _arg(fn, "cache.ring", cache.ring, _i32(), shape=(cache.nseq, cfg.N - 1))


def _out_arg(fn, cfg, out, shape, name="out"):
    if cfg.dtype_code in (NGRAM_F32, NGRAM_BF16):
        _arg(fn, name, out, _torch_dtype(cfg.dtype_code), shape=shape)


# ------------------------------------------------------------------ entry points

def _shapes_ok(cfg: Config) -> bool:
    """Whether the config's derived widths are meaningful (else the C side reports it)."""
    if cfg.N < 1 or cfg.K < 1 or cfg.D < 1 or len(cfg.V) < cfg.S:
        return False
    return not (cfg.S and cfg.form_code == NGRAM_FORM_FINAL and cfg.D % cfg.S)


def ngram_embed_status_string(status: int) -> str:
    return load().ngram_embed_status_string(int(status)).decode()


def ngram_embed_workspace_size(cfg: Config, max_rows: int) -> int:
    c, keep = cfg._c()
    return int(load().ngram_embed_workspace_size(ctypes.byref(c), int(max_rows)))


def ngram_embed_workspace_layout(cfg: Config, max_rows: int):
    c, keep = cfg._c()
    tok, idx = ctypes.c_size_t(), ctypes.c_size_t()
    _check("ngram_embed_workspace_layout", load().ngram_embed_workspace_layout(
        ctypes.byref(c), int(max_rows), ctypes.byref(tok), ctypes.byref(idx)))
    return tok.value, idx.value


def alloc_workspace(cfg: Config, max_rows: int, device="cuda"):
    """Zero-filled uint8 device workspace for up to max_rows rows."""
    import torch
    n = ngram_embed_workspace_size(cfg, max_rows)
    if n == 0:
        raise NgramError("ngram_embed_workspace_size", -1)
    return torch.zeros((n,), dtype=torch.uint8, device=device)


def ngram_embed_backward_workspace_size(cfg: Config, ntok: int) -> int:
    c, keep = cfg._c()
    return int(load().ngram_embed_backward_workspace_size(ctypes.byref(c), int(ntok)))


def alloc_backward_workspace(cfg: Config, ntok: int, device="cuda"):
    """Zero-filled uint8 device workspace for the backward of ntok tokens."""
    import torch
    n = ngram_embed_backward_workspace_size(cfg, ntok)
    if n == 0:
        raise NgramError("ngram_embed_backward_workspace_size", -1)
    return torch.zeros((n,), dtype=torch.uint8, device=device)


def ngram_embed_backward(cfg: Config, tables: Tables, tokens, cu_seqlens, dout, dE0, dE, dW,
                         ws, stream=None):
    """Accumulate the gradients of one batch into fp32 buffers dE0 [V0, D], dE (S tensors
    [V_s, d]) and dW [D, D]; any may be None."""
    import torch
    fn = "ngram_embed_backward"
    _ids_arg(fn, tokens, cu_seqlens)
    if _shapes_ok(cfg):
        _tables_arg(fn, cfg, tables)
        _out_arg(fn, cfg, dout, (tokens.numel(), cfg.D), "dout")
        _arg(fn, "dE0", dE0, torch.float32, shape=(cfg.V0, cfg.D), optional=True)
        _arg(fn, "dW", dW, torch.float32, shape=(cfg.D, cfg.D), optional=True)
        if dE is not None:
            if len(dE) < cfg.S:
                raise ValueError(f"{fn}: dE needs {cfg.S} gradient buffers")
            for s in range(cfg.S):
                _arg(fn, f"dE[{s}]", dE[s], torch.float32, shape=(int(cfg.V[s]), cfg.d))
    _ws_arg(fn, ws)
    c, keep = cfg._c()
    t, keep2 = tables._c()
    dE_arr = None
    if dE is not None:
        dE_arr = (ctypes.c_void_p * max(1, len(dE)))(*[_ptr(e) for e in dE])
    _check(fn, load().ngram_embed_backward(
        ctypes.byref(c), ctypes.byref(t), _ptr(tokens), _ptr(cu_seqlens),
        int(cu_seqlens.numel()) - 1, int(tokens.numel()), _ptr(dout), _ptr(dE0),
        dE_arr, _ptr(dW), _ptr(ws), int(ws.numel() * ws.element_size()), _stream(stream)))


def ngram_embed_hash(cfg: Config, tokens, cu_seqlens, idx, err_flags=None, stream=None):
    """idx (int32, >= ntok * S elements) = the hash indices of every position."""
    fn = "ngram_embed_hash"
    _ids_arg(fn, tokens, cu_seqlens)
    _arg(fn, "idx", idx, _i32(), min_numel=tokens.numel() * max(cfg.S, 0))
    _flags_arg(fn, "err_flags", err_flags)
    c, keep = cfg._c()
    _check(fn, load().ngram_embed_hash(
        ctypes.byref(c), _ptr(tokens), _ptr(cu_seqlens), int(cu_seqlens.numel()) - 1,
        int(tokens.numel()), _ptr(idx), _ptr(err_flags), _stream(stream)))


def ngram_embed_gather(cfg: Config, tables: Tables, idx, G, stream=None):
    """G [nrows, S * d] (the config's dtype) = the concatenated sub-table rows idx names."""
    fn = "ngram_embed_gather"
    if _shapes_ok(cfg):
        _tables_arg(fn, cfg, tables)
        _out_arg(fn, cfg, G, (None, cfg.S * cfg.d), "G")
    else:
        _arg(fn, "G", G)
    _arg(fn, "idx", idx, _i32(), min_numel=G.shape[0] * max(cfg.S, 0))
    c, keep = cfg._c()
    t, keep2 = tables._c()
    _check(fn, load().ngram_embed_gather(
        ctypes.byref(c), ctypes.byref(t), _ptr(idx), int(G.shape[0]), _ptr(G), _stream(stream)))


def ngram_embed_gather_checksum(cfg: Config, tables: Tables, idx, sums, stream=None):
    """sums [nrows] (uint32 stored in an int32 tensor) = the checksum of each gathered row as
    it lands in LDS: sum_k w_k (2k + 1) mod 2^32 over the row's 32-bit words."""
    fn = "ngram_embed_gather_checksum"
    if _shapes_ok(cfg):
        _tables_arg(fn, cfg, tables)
    _arg(fn, "sums", sums, _i32(), shape=(None,))
    _arg(fn, "idx", idx, _i32(), min_numel=sums.shape[0] * max(cfg.S, 0))
    c, keep = cfg._c()
    t, keep2 = tables._c()
    _check(fn, load().ngram_embed_gather_checksum(
        ctypes.byref(c), ctypes.byref(t), _ptr(idx), int(sums.shape[0]), _ptr(sums),
        _stream(stream)))


def ngram_embed_project(cfg: Config, tables: Tables, idx, tok, out, stream=None):
    """out [nrows, D] = the layer's rows for hash indices idx and E_0 tokens tok."""
    fn = "ngram_embed_project"
    if _shapes_ok(cfg):
        _tables_arg(fn, cfg, tables)
        _out_arg(fn, cfg, out, (None, cfg.D))
    else:
        _arg(fn, "out", out)
    nrows = int(out.shape[0])
    _arg(fn, "idx", idx, _i32(), min_numel=nrows * max(cfg.S, 0))
    _arg(fn, "tok", tok, _i32(), min_numel=nrows)
    c, keep = cfg._c()
    t, keep2 = tables._c()
    _check(fn, load().ngram_embed_project(
        ctypes.byref(c), ctypes.byref(t), _ptr(idx), _ptr(tok), nrows, _ptr(out),
        _stream(stream)))


def ngram_embed_prefill(cfg: Config, tables: Tables, tokens, cu_seqlens, out, ws,
                        cache: Optional["Cache"] = None, stream=None):
    """out [ntok, D] = the layer over packed sequences; with a cache (one slot per
    sequence), the same call also fills it from the sequences' last N-1 ids."""
    fn = "ngram_embed_prefill"
    _ids_arg(fn, tokens, cu_seqlens)
    if _shapes_ok(cfg):
        _tables_arg(fn, cfg, tables)
        _out_arg(fn, cfg, out, (tokens.numel(), cfg.D))
    _ws_arg(fn, ws)
    cc = None
    if cache is not None:
        _cache_arg(fn, cfg, cache)
        if cache.nseq != cu_seqlens.numel() - 1:
            raise ValueError(f"{fn}: the cache needs one slot per sequence")
        cc = cache._c()
    c, keep = cfg._c()
    t, keep2 = tables._c()
    _check(fn, load().ngram_embed_prefill(
        ctypes.byref(c), ctypes.byref(t), _ptr(tokens), _ptr(cu_seqlens),
        int(cu_seqlens.numel()) - 1, int(tokens.numel()), _ptr(out),
        ctypes.byref(cc) if cc is not None else None, _ptr(ws),
        int(ws.numel() * ws.element_size()), _stream(stream)))


def ngram_cache_init(cfg: Config, cache: Cache, tokens, cu_seqlens, stream=None):
    fn = "ngram_cache_init"
    _ids_arg(fn, tokens, cu_seqlens)
    _cache_arg(fn, cfg, cache)
    if cu_seqlens.numel() != cache.nseq + 1:
        raise ValueError(f"{fn}: cu_seqlens must have cache.nseq + 1 = {cache.nseq + 1} "
                         f"entries, has {cu_seqlens.numel()}")
    c, keep = cfg._c()
    cc = cache._c()
    _check(fn, load().ngram_cache_init(
        ctypes.byref(c), ctypes.byref(cc), _ptr(tokens), _ptr(cu_seqlens), int(tokens.numel()),
        _stream(stream)))


def _step_args(fn, cfg, nbatch, new_tokens, counts, count_names):
    """new_tokens int32 [nbatch, tmax]; each count int32 [nbatch] (None allowed for the
    optional ones, whose names end in '?')."""
    _arg(fn, "new_tokens", new_tokens, _i32(), shape=(nbatch, None))
    for t, name in zip(counts, count_names):
        _arg(fn, name.rstrip("?"), t, _i32(), shape=(nbatch,), optional=name.endswith("?"))


def ngram_embed_decode(cfg: Config, tables: Tables, cache: Cache, new_tokens, n_new, out, ws,
                       n_commit=None, stream=None):
    fn = "ngram_embed_decode"
    _cache_arg(fn, cfg, cache)
    _step_args(fn, cfg, cache.nseq, new_tokens, (n_new, n_commit), ("n_new", "n_commit?"))
    if _shapes_ok(cfg):
        _tables_arg(fn, cfg, tables)
        _out_arg(fn, cfg, out, (cache.nseq, new_tokens.shape[1], cfg.D))
    _ws_arg(fn, ws)
    c, keep = cfg._c()
    t, keep2 = tables._c()
    cc = cache._c()
    _check(fn, load().ngram_embed_decode(
        ctypes.byref(c), ctypes.byref(t), ctypes.byref(cc), _ptr(new_tokens), _ptr(n_new),
        int(new_tokens.shape[1]), _ptr(n_commit), _ptr(out), _ptr(ws),
        int(ws.numel() * ws.element_size()), _stream(stream)))


def ngram_embed_decode_noalloc(cfg: Config, tables: Tables, cache: Cache, new_tokens, n_new,
                               out, n_commit=None, err_flags=None, stream=None):
    """ngram_embed_decode without a workspace: the step's scratch is the library's fixed
    per-GPU array (for callers that cannot allocate; calls overlapping on one GPU race).
    err_flags: optional device int32 the step's flags are OR-ed into."""
    fn = "ngram_embed_decode_noalloc"
    _cache_arg(fn, cfg, cache)
    _step_args(fn, cfg, cache.nseq, new_tokens, (n_new, n_commit), ("n_new", "n_commit?"))
    if _shapes_ok(cfg):
        _tables_arg(fn, cfg, tables)
        _out_arg(fn, cfg, out, (cache.nseq, new_tokens.shape[1], cfg.D))
    _arg(fn, "err_flags", err_flags, _i32(), min_numel=1, optional=True)
    c, keep = cfg._c()
    t, keep2 = tables._c()
    cc = cache._c()
    _check(fn, load().ngram_embed_decode_noalloc(
        ctypes.byref(c), ctypes.byref(t), ctypes.byref(cc), _ptr(new_tokens), _ptr(n_new),
        int(new_tokens.shape[1]), _ptr(n_commit), _ptr(out), _ptr(err_flags),
        _stream(stream)))


def _layer_args(fn, cfg, tables, outs, out_shape):
    """C arrays of the layers' tables and output pointers (kept alive by the caller)."""
    if len(tables) != len(outs) or not tables:
        raise ValueError("one output per layer, at least one layer")
    if _shapes_ok(cfg):
        for l, (tb, o) in enumerate(zip(tables, outs)):
            _tables_arg(fn, cfg, tb, layer=f"[{l}]")
            _out_arg(fn, cfg, o, out_shape, name=f"outs[{l}]")
    cts = [t._c() for t in tables]
    tarr = (_CTables * len(cts))(*[ct for ct, _ in cts])
    oarr = (ctypes.c_void_p * len(outs))(*[_ptr(o) for o in outs])
    return tarr, oarr, cts


def ngram_embed_prefill_layers(cfg: Config, tables, tokens, cu_seqlens, outs, ws, stream=None):
    """Per-layer embeddings: outs[l] = the layer with tables[l], hash computed once."""
    fn = "ngram_embed_prefill_layers"
    _ids_arg(fn, tokens, cu_seqlens)
    _ws_arg(fn, ws)
    c, keep = cfg._c()
    tarr, oarr, keep2 = _layer_args(fn, cfg, tables, outs, (tokens.numel(), cfg.D))
    _check(fn, load().ngram_embed_prefill_layers(
        ctypes.byref(c), tarr, len(tables), _ptr(tokens), _ptr(cu_seqlens),
        int(cu_seqlens.numel()) - 1, int(tokens.numel()), oarr, _ptr(ws),
        int(ws.numel() * ws.element_size()), _stream(stream)))


def ngram_embed_decode_layers(cfg: Config, tables, cache: Cache, new_tokens, n_new, outs, ws,
                              n_commit=None, stream=None):
    fn = "ngram_embed_decode_layers"
    _cache_arg(fn, cfg, cache)
    _step_args(fn, cfg, cache.nseq, new_tokens, (n_new, n_commit), ("n_new", "n_commit?"))
    _ws_arg(fn, ws)
    c, keep = cfg._c()
    tarr, oarr, keep2 = _layer_args(fn, cfg, tables, outs,
                                    (cache.nseq, new_tokens.shape[1], cfg.D))
    cc = cache._c()
    _check(fn, load().ngram_embed_decode_layers(
        ctypes.byref(c), tarr, len(tables), ctypes.byref(cc), _ptr(new_tokens), _ptr(n_new),
        int(new_tokens.shape[1]), _ptr(n_commit), oarr, _ptr(ws),
        int(ws.numel() * ws.element_size()), _stream(stream)))


def _vocab_arr(vocab):
    return (ctypes.c_int64 * max(1, len(vocab)))(*[int(v) for v in vocab])


def ngram_hash_stats_workspace_size(V0: int, n: int, ntok: int, vocab) -> int:
    arr = _vocab_arr(vocab)
    return int(load().ngram_hash_stats_workspace_size(int(V0), int(n), int(ntok), arr,
                                                      len(vocab)))


def ngram_hash_stats(V0: int, n: int, tokens, cu_seqlens, vocab, rows, distinct=None,
                     ws=None, stream=None):
    """rows[v] (device int64 [len(vocab)]) = distinct table rows of size vocab[v] that the
    order-n hash of every position uses; distinct (device int64 [1], optional) = distinct
    n-grams. ws: None allocates a zero-filled workspace."""
    import torch
    fn = "ngram_hash_stats"
    _ids_arg(fn, tokens, cu_seqlens)
    _arg(fn, "rows", rows, _i64(), min_numel=len(vocab), optional=len(vocab) == 0)
    _arg(fn, "distinct", distinct, _i64(), shape=(1,), optional=True)
    arr = _vocab_arr(vocab)
    if ws is None:
        nbytes = ngram_hash_stats_workspace_size(V0, n, tokens.numel(), vocab)
        if nbytes == 0:
            raise NgramError("ngram_hash_stats_workspace_size", -1)
        ws = torch.zeros((nbytes,), dtype=torch.uint8, device=tokens.device)
    _ws_arg(fn, ws)
    _check(fn, load().ngram_hash_stats(
        int(V0), int(n), _ptr(tokens), _ptr(cu_seqlens), int(cu_seqlens.numel()) - 1,
        int(tokens.numel()), arr, len(vocab), _ptr(rows), _ptr(distinct), _ptr(ws),
        int(ws.numel() * ws.element_size()), _stream(stream)))
    return ws


def ngram_embed_decode_rows(cfg: Config, tables: Tables, cache: Cache, new_tokens, n_new, out,
                            ws, row_begin=0, row_end=None, slots=None, n_commit=None,
                            stream=None):
    """Rows [row_begin, min(row_end, n_new[b])) of every batch entry b (batch entry b uses
    cache slot slots[b], or b); other rows of out are left as they are."""
    fn = "ngram_embed_decode_rows"
    _cache_arg(fn, cfg, cache)
    nbatch = int(new_tokens.shape[0]) if hasattr(new_tokens, "shape") else 0
    _step_args(fn, cfg, nbatch, new_tokens, (n_new, n_commit, slots),
               ("n_new", "n_commit?", "slots?"))
    tmax = int(new_tokens.shape[1])
    if _shapes_ok(cfg):
        _tables_arg(fn, cfg, tables)
        _out_arg(fn, cfg, out, (nbatch, tmax, cfg.D))
    _ws_arg(fn, ws)
    c, keep = cfg._c()
    t, keep2 = tables._c()
    cc = cache._c()
    _check(fn, load().ngram_embed_decode_rows(
        ctypes.byref(c), ctypes.byref(t), ctypes.byref(cc), _ptr(slots),
        nbatch, _ptr(new_tokens), _ptr(n_new), tmax, int(row_begin),
        int(tmax if row_end is None else row_end), _ptr(n_commit), _ptr(out), _ptr(ws),
        int(ws.numel() * ws.element_size()), _stream(stream)))


def ngram_cache_init_slots(cfg: Config, cache: Cache, slots, tokens, cu_seqlens,
                           err_flags=None, stream=None):
    fn = "ngram_cache_init_slots"
    _ids_arg(fn, tokens, cu_seqlens)
    _cache_arg(fn, cfg, cache)
    nbatch = int(cu_seqlens.numel()) - 1
    _arg(fn, "slots", slots, _i32(), shape=(nbatch,), optional=True)
    _flags_arg(fn, "err_flags", err_flags)
    c, keep = cfg._c()
    cc = cache._c()
    _check(fn, load().ngram_cache_init_slots(
        ctypes.byref(c), ctypes.byref(cc), _ptr(slots), nbatch,
        _ptr(tokens), _ptr(cu_seqlens), int(tokens.numel()), _ptr(err_flags), _stream(stream)))


def ngram_cache_commit_slots(cfg: Config, cache: Cache, slots, new_tokens, n_accept,
                             err_flags=None, stream=None):
    fn = "ngram_cache_commit_slots"
    _cache_arg(fn, cfg, cache)
    nbatch = int(new_tokens.shape[0]) if hasattr(new_tokens, "shape") else 0
    _step_args(fn, cfg, nbatch, new_tokens, (n_accept, slots), ("n_accept", "slots?"))
    _flags_arg(fn, "err_flags", err_flags)
    c, keep = cfg._c()
    cc = cache._c()
    _check(fn, load().ngram_cache_commit_slots(
        ctypes.byref(c), ctypes.byref(cc), _ptr(slots), nbatch,
        _ptr(new_tokens), _ptr(n_accept), int(new_tokens.shape[1]), _ptr(err_flags),
        _stream(stream)))


def ngram_cache_commit(cfg: Config, cache: Cache, new_tokens, n_accept, err_flags=None,
                       stream=None):
    fn = "ngram_cache_commit"
    _cache_arg(fn, cfg, cache)
    _step_args(fn, cfg, cache.nseq, new_tokens, (n_accept,), ("n_accept",))
    _flags_arg(fn, "err_flags", err_flags)
    c, keep = cfg._c()
    cc = cache._c()
    _check(fn, load().ngram_cache_commit(
        ctypes.byref(c), ctypes.byref(cc), _ptr(new_tokens), _ptr(n_accept),
        int(new_tokens.shape[1]), _ptr(err_flags), _stream(stream)))


def ngram_embed_read_error_flag(ws, stream=None) -> int:
    _flags_arg("ngram_embed_read_error_flag", "ws", ws)
    v = ctypes.c_int32(0)
    _check("ngram_embed_read_error_flag", load().ngram_embed_read_error_flag(
        _ptr(ws), ctypes.byref(v), _stream(stream)))
    return int(v.value)


def ngram_embed_clear_error_flag(ws, stream=None):
    _flags_arg("ngram_embed_clear_error_flag", "ws", ws)
    _check("ngram_embed_clear_error_flag",
           load().ngram_embed_clear_error_flag(_ptr(ws), _stream(stream)))
