"""CPU checks of the C ABI: the library loads, exports what include/ngram_embed.h declares,
and rejects bad arguments on the host before any HIP call (no GPU is touched here: every
call below carries at least one argument that validation refuses)."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

import gram_embedding_layer_amd as g

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ngram_embed.h")

FAKE = 0x100000  # 1 MiB: aligned, never dereferenced because validation fails first


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(g.LIB_PATH):
        pytest.fail("libngram_embed.so not built (python -m gram_embedding_layer_amd.build)")
    return g.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(ngram_[a-z_]+)\s*\(", text, re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("ngram_embed_prefill", "ngram_embed_decode", "ngram_embed_hash",
              "ngram_embed_gather", "ngram_embed_project", "ngram_cache_init",
              "ngram_cache_commit", "ngram_embed_backward",
              "ngram_embed_backward_workspace_size"):
        assert n in names
    assert len(names) == 23


def test_library_exports_every_declared_symbol(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_binding_names_match_header():
    for n in declared_functions():
        assert callable(getattr(g, n)), n


def tiny_cfg(**kw):
    args = dict(N=3, K=2, D=64, dtype="bf16", V0=1000, V=[5003, 7001, 6007, 8009])
    args.update(kw)
    return g.Config(**args)


def test_status_strings(lib):
    assert g.ngram_embed_status_string(0) == "ok"
    for s in range(-7, 0):
        assert g.ngram_embed_status_string(s) != "unknown status"
    assert g.ngram_embed_status_string(-99) == "unknown status"


def test_workspace_size_and_layout(lib):
    cfg = tiny_cfg()
    rows = 1000
    tok_off, idx_off = g.ngram_embed_workspace_layout(cfg, rows)
    assert tok_off == 256
    assert idx_off == 256 + ((rows * 4 + 255) // 256) * 256
    size = g.ngram_embed_workspace_size(cfg, rows)
    assert size == idx_off + ((rows * cfg.S * 4 + 255) // 256) * 256
    assert size % 256 == 0
    assert g.ngram_embed_workspace_size(cfg, -1) == 0
    assert g.ngram_embed_workspace_size(tiny_cfg(D=63), 10) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(D=62), -1),                       # D not a multiple of (N-1)K
    (dict(D=36, V=[5, 7, 11, 13]), -1),     # d = 9 bf16 = 18 bytes: not whole 16-byte rows
    (dict(N=0), -1),
    (dict(K=0), -1),
    (dict(N=17), -1),
    (dict(N=3, K=33, D=66 * 64, V=[7] * 66), -1),   # more than 64 sub-tables
    (dict(dtype=7), -2),
    (dict(V0=0), -1),
    (dict(V0=2 ** 31), -1),
    (dict(V=[5003, 0, 6007, 8009]), -1),
    (dict(V=[5003, 2 ** 31, 6007, 8009]), -1),
    (dict(form="basic"), -1),               # the basic form has K = 1
    (dict(form=2), -1),
])
def test_config_validation(lib, kw, status):
    cfg = tiny_cfg(**kw)
    c, keep = cfg._c()
    rc = lib.ngram_embed_prefill(ctypes.byref(c), None, FAKE, FAKE, 1, 16, FAKE, None, FAKE, 1 << 20, 0)
    assert rc == status
    assert lib.ngram_embed_workspace_size(ctypes.byref(c), 16) == 0


def _tables_c(n_sub, e0=FAKE, w=FAKE, sub=FAKE):
    arr = (ctypes.c_void_p * max(1, n_sub))(*([sub] * n_sub))
    return g._CTables(e0, ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)), w), arr


def test_prefill_argument_checks(lib):
    cfg = tiny_cfg()
    c, keep = cfg._c()
    T, keep2 = _tables_c(4)
    ws_need = g.ngram_embed_workspace_size(cfg, 16)
    P = ctypes.byref
    # workspace too small / misaligned
    assert lib.ngram_embed_prefill(P(c), P(T), FAKE, FAKE, 1, 16, FAKE, None, FAKE, ws_need - 1, 0) == -4
    assert lib.ngram_embed_prefill(P(c), P(T), FAKE, FAKE, 1, 16, FAKE, None, FAKE + 64, ws_need, 0) == -4
    # negative sizes, no sequences for tokens
    assert lib.ngram_embed_prefill(P(c), P(T), FAKE, FAKE, 1, -1, FAKE, None, FAKE, ws_need, 0) == -1
    assert lib.ngram_embed_prefill(P(c), P(T), FAKE, FAKE, 0, 16, FAKE, None, FAKE, ws_need, 0) == -1
    # misaligned table / output / token pointers
    Tb, k3 = _tables_c(4, e0=FAKE + 8)
    assert lib.ngram_embed_prefill(P(c), P(Tb), FAKE, FAKE, 1, 16, FAKE, None, FAKE, ws_need, 0) == -3
    Tb, k4 = _tables_c(4, sub=FAKE + 2)
    assert lib.ngram_embed_prefill(P(c), P(Tb), FAKE, FAKE, 1, 16, FAKE, None, FAKE, ws_need, 0) == -3
    assert lib.ngram_embed_prefill(P(c), P(T), FAKE, FAKE, 1, 16, FAKE + 8, None, FAKE, ws_need, 0) == -3
    assert lib.ngram_embed_prefill(P(c), P(T), FAKE + 1, FAKE, 1, 16, FAKE, None, FAKE, ws_need, 0) == -3
    assert lib.ngram_embed_prefill(P(c), None, FAKE, FAKE, 1, 16, FAKE, None, FAKE, ws_need, 0) == -3


def test_layers_argument_checks(lib):
    """Per-layer entry points: at least one layer, every layer's tables and output checked."""
    cfg = tiny_cfg()
    c, keep = cfg._c()
    P = ctypes.byref
    ws_need = g.ngram_embed_workspace_size(cfg, 16)
    good, k1 = _tables_c(4)
    bad, k2 = _tables_c(4, sub=FAKE + 2)
    two = (g._CTables * 2)(good, good)
    mixed = (g._CTables * 2)(good, bad)
    outs = (ctypes.c_void_p * 2)(FAKE, FAKE)
    outs_bad = (ctypes.c_void_p * 2)(FAKE, FAKE + 8)
    pf = lib.ngram_embed_prefill_layers
    assert pf(P(c), two, 0, FAKE, FAKE, 1, 16, outs, FAKE, ws_need, 0) == -1
    assert pf(P(c), two, 2, FAKE, FAKE, 1, 16, outs, FAKE, ws_need - 1, 0) == -4
    assert pf(P(c), mixed, 2, FAKE, FAKE, 1, 16, outs, FAKE, ws_need, 0) == -3
    assert pf(P(c), two, 2, FAKE, FAKE, 1, 16, outs_bad, FAKE, ws_need, 0) == -3
    assert pf(P(c), None, 2, FAKE, FAKE, 1, 16, outs, FAKE, ws_need, 0) == -3
    assert pf(P(c), two, 2, FAKE, FAKE, 1, 16, None, FAKE, ws_need, 0) == -3
    assert pf(P(c), two, 2, FAKE, FAKE, 1, 0, outs, FAKE, ws_need, 0) == 0      # no tokens
    cache = g._CCache(FAKE, FAKE, 4)
    ws_dec = g.ngram_embed_workspace_size(cfg, 4 * 5)
    dl = lib.ngram_embed_decode_layers
    assert dl(P(c), two, -1, P(cache), FAKE, FAKE, 5, None, outs, FAKE, ws_dec, 0) == -1
    assert dl(P(c), two, 2, P(cache), FAKE, FAKE, 9, None, outs, FAKE, ws_dec, 0) == -1
    assert dl(P(c), two, 2, P(cache), FAKE, FAKE, 5, None, outs, FAKE, ws_dec - 1, 0) == -4
    assert dl(P(c), mixed, 2, P(cache), FAKE, FAKE, 5, None, outs, FAKE, ws_dec, 0) == -3
    assert dl(P(c), two, 2, P(cache), FAKE, FAKE, 5, None, outs_bad, FAKE, ws_dec, 0) == -3


def test_hash_stats_checks(lib):
    """Hash statistics: workspace sizes, exact-value limit, argument checks."""
    P = ctypes.byref
    vocab = [5003, 32, 1, 2 ** 31 - 1]
    n1 = g.ngram_hash_stats_workspace_size(1000, 2, 100, vocab)
    n2 = g.ngram_hash_stats_workspace_size(1000, 2, 10000, vocab)
    assert 0 < n1 < n2 and n1 % 256 == 0
    # the bitmaps of one group of sizes: 2^31 - 1 rows need 2^26 words
    assert n1 >= (5003 + 31) // 32 * 4 + 32 // 32 * 4 + 4 + (2 ** 26) * 4
    assert g.ngram_hash_stats_workspace_size(1000, 2, 100, [0]) == 0
    assert g.ngram_hash_stats_workspace_size(1000, 2, 100, [2 ** 31]) == 0
    assert g.ngram_hash_stats_workspace_size(0, 2, 100, vocab) == 0
    assert g.ngram_hash_stats_workspace_size(1000, 0, 100, vocab) == 0
    assert g.ngram_hash_stats_workspace_size(1000, 17, 100, vocab) == 0
    # no sort buffers once the exact values do not fit: V0 = 2^17, n = 4 is 2^68
    big = g.ngram_hash_stats_workspace_size(131072, 4, 10 ** 6, [7])
    small = g.ngram_hash_stats_workspace_size(131072, 3, 10 ** 6, [7])
    assert big < small
    hs = lib.ngram_hash_stats
    arr = (ctypes.c_int64 * 1)(7)
    ws = g.ngram_hash_stats_workspace_size(131072, 4, 16, [7])
    assert hs(131072, 4, FAKE, FAKE, 1, 16, arr, 1, FAKE, FAKE, FAKE, ws, 0) == -5
    assert hs(131072, 4, FAKE, FAKE, 1, 16, arr, 1, FAKE + 4, None, FAKE, ws, 0) == -3
    assert hs(131072, 4, FAKE, FAKE, 1, 16, arr, 1, FAKE, None, FAKE, ws - 1, 0) == -4
    assert hs(131072, 4, FAKE, FAKE, 0, 16, arr, 1, FAKE, None, FAKE, ws, 0) == -1
    assert hs(131072, 4, FAKE, FAKE, 1, 16, None, 1, FAKE, None, FAKE, ws, 0) == -1
    assert hs(131072, 4, FAKE, FAKE, 1, 16, arr, 0, None, None, FAKE, ws, 0) == 0


def test_decode_and_cache_argument_checks(lib):
    cfg = tiny_cfg()
    c, keep = cfg._c()
    T, keep2 = _tables_c(4)
    P = ctypes.byref
    cache = g._CCache(FAKE, FAKE, 4)
    ws_need = g.ngram_embed_workspace_size(cfg, 4 * 5)
    for tmax in (0, 9):
        assert lib.ngram_embed_decode(P(c), P(T), P(cache), FAKE, FAKE, tmax, None, FAKE, FAKE,
                                      ws_need, 0) == -1
    assert lib.ngram_embed_decode(P(c), P(T), P(cache), FAKE, FAKE, 5, None, FAKE, FAKE,
                                  ws_need - 256, 0) == -4
    assert lib.ngram_embed_decode(P(c), P(T), None, FAKE, FAKE, 5, None, FAKE, FAKE,
                                  ws_need, 0) == -1
    bad_len = g._CCache(FAKE, FAKE + 4, 4)
    assert lib.ngram_embed_decode(P(c), P(T), P(bad_len), FAKE, FAKE, 5, None, FAKE, FAKE,
                                  ws_need, 0) == -3
    assert lib.ngram_embed_decode(P(c), P(T), P(cache), FAKE, FAKE, 5, FAKE + 2, FAKE, FAKE,
                                  ws_need, 0) == -3
    assert lib.ngram_cache_commit(P(c), P(cache), FAKE, FAKE, 9, None, 0) == -1
    assert lib.ngram_cache_commit(P(c), P(bad_len), FAKE, FAKE, 5, None, 0) == -3
    assert lib.ngram_cache_init(P(c), None, FAKE, FAKE, 10, 0) == -1
    assert lib.ngram_cache_init(P(c), P(bad_len), FAKE, FAKE, 10, 0) == -3
    neg = g._CCache(FAKE, FAKE, -1)
    assert lib.ngram_cache_init(P(c), P(neg), FAKE, FAKE, 10, 0) == -1


def test_hash_gather_project_argument_checks(lib):
    cfg = tiny_cfg()
    c, keep = cfg._c()
    T, keep2 = _tables_c(4)
    P = ctypes.byref
    assert lib.ngram_embed_hash(P(c), FAKE, FAKE, 1, -5, FAKE, None, 0) == -1
    assert lib.ngram_embed_hash(P(c), FAKE + 2, FAKE, 1, 5, FAKE, None, 0) == -3
    assert lib.ngram_embed_hash(P(c), FAKE, FAKE, 1, 5, FAKE, FAKE + 1, 0) == -3
    assert lib.ngram_embed_gather(P(c), P(T), FAKE, -1, FAKE, 0) == -1
    assert lib.ngram_embed_gather(P(c), P(T), FAKE, 5, FAKE + 4, 0) == -3
    assert lib.ngram_embed_project(P(c), P(T), FAKE, FAKE, 5, FAKE + 4, 0) == -3
    Tb, k3 = _tables_c(4, w=0)
    assert lib.ngram_embed_project(P(c), P(Tb), FAKE, FAKE, 5, FAKE, 0) == -3
    assert lib.ngram_embed_read_error_flag(FAKE + 16, None, 0) == -3
    assert lib.ngram_embed_clear_error_flag(FAKE + 16, 0) == -3


def test_amplification_checks(lib):
    """Embedding amplification: the layer normalisation keeps the fp32 rows in the
    workspace, needs that workspace (so the bare projection refuses it), a positive epsilon
    and 16-byte aligned parameters; the scale needs a finite factor."""
    P = ctypes.byref
    plain, ln = tiny_cfg(), tiny_cfg(amp="layernorm")
    assert g.ngram_embed_workspace_size(ln, 1000) == \
        g.ngram_embed_workspace_size(plain, 1000) + ((1000 * 64 * 4 + 255) // 256) * 256
    assert g.ngram_embed_workspace_size(tiny_cfg(amp="scale"), 1000) == \
        g.ngram_embed_workspace_size(plain, 1000)
    for kw in (dict(amp="layernorm", ln_eps=0.0), dict(amp="layernorm", ln_eps=-1e-5),
               dict(amp="layernorm", ln_eps=float("nan")), dict(amp="scale", amp_scale=float("inf")),
               dict(amp="scale", amp_scale=float("nan")), dict(amp=3), dict(amp=-1),
               dict(amp="layernorm", N=2, K=1, D=8192 + 64, V=[5003])):
        c, keep = tiny_cfg(**kw)._c()
        assert lib.ngram_embed_workspace_size(P(c), 16) == 0, kw
        assert lib.ngram_embed_prefill(P(c), None, FAKE, FAKE, 1, 16, FAKE, None, FAKE, 1 << 20, 0) == -1
    c, keep = ln._c()
    T, keep2 = _tables_c(4)
    assert lib.ngram_embed_project(P(c), P(T), FAKE, FAKE, 5, FAKE, 0) == -1
    ws_need = g.ngram_embed_workspace_size(ln, 16)
    arr = (ctypes.c_void_p * 4)(*([FAKE] * 4))
    for wt, bs in ((FAKE + 2, None), (None, FAKE + 8)):
        Tb = g._CTables(FAKE, ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)), FAKE, wt, bs)
        assert lib.ngram_embed_prefill(P(c), P(Tb), FAKE, FAKE, 1, 16, FAKE, None, FAKE, ws_need,
                                       0) == -3


def test_backward_argument_checks(lib):
    """Backward: its workspace grows with the batch, layer normalisation is refused, and
    bad workspaces, sizes and pointers are rejected before any launch."""
    P = ctypes.byref
    cfg = tiny_cfg()
    n1, n2 = g.ngram_embed_backward_workspace_size(cfg, 100), \
        g.ngram_embed_backward_workspace_size(cfg, 1000)
    assert 0 < n1 < n2 and n1 % 256 == 0 and n2 % 256 == 0
    assert g.ngram_embed_backward_workspace_size(tiny_cfg(amp="layernorm"), 100) == 0
    assert g.ngram_embed_backward_workspace_size(cfg, -1) == 0
    c, keep = cfg._c()
    T, keep2 = _tables_c(4)
    ws = g.ngram_embed_backward_workspace_size(cfg, 16)
    bw = lib.ngram_embed_backward
    assert bw(P(c), P(T), FAKE, FAKE, 1, 16, FAKE, FAKE, None, FAKE, FAKE, ws - 1, 0) == -4
    assert bw(P(c), P(T), FAKE, FAKE, 1, 16, FAKE, FAKE, None, FAKE, FAKE + 64, ws, 0) == -4
    assert bw(P(c), P(T), FAKE, FAKE, 1, -1, FAKE, FAKE, None, FAKE, FAKE, ws, 0) == -1
    assert bw(P(c), P(T), FAKE, FAKE, 0, 16, FAKE, FAKE, None, FAKE, FAKE, ws, 0) == -1
    assert bw(P(c), P(T), FAKE, FAKE, 1, 16, FAKE + 8, FAKE, None, FAKE, FAKE, ws, 0) == -3
    assert bw(P(c), P(T), FAKE, FAKE, 1, 16, FAKE, FAKE + 4, None, FAKE, FAKE, ws, 0) == -3
    assert bw(P(c), P(T), FAKE, FAKE, 1, 16, FAKE, None, None, FAKE + 4, FAKE, ws, 0) == -3
    arr = (ctypes.c_void_p * 4)(FAKE, FAKE, FAKE + 4, FAKE)
    assert bw(P(c), P(T), FAKE, FAKE, 1, 16, FAKE, None, arr, None, FAKE, ws, 0) == -3
    assert bw(P(c), None, FAKE, FAKE, 1, 16, FAKE, None, None, None, FAKE, ws, 0) == -3
    cl, keep3 = tiny_cfg(amp="layernorm")._c()
    assert bw(P(cl), P(T), FAKE, FAKE, 1, 16, FAKE, None, None, None, FAKE, ws, 0) == -1
    # an empty batch succeeds without touching the device
    assert bw(P(c), P(T), FAKE, FAKE, 0, 0, FAKE, FAKE, None, FAKE, FAKE, ws, 0) == 0
    # the basic form has no projection: dW must be NULL; W itself is never read
    cb, keep4 = tiny_cfg(form="basic", K=1, V=[5003, 7001])._c()
    Tb, keep5 = _tables_c(2, w=None)
    wsb = g.ngram_embed_backward_workspace_size(tiny_cfg(form="basic", K=1, V=[5003, 7001]), 16)
    assert 0 < wsb < ws
    assert bw(P(cb), P(Tb), FAKE, FAKE, 1, 16, FAKE, None, None, FAKE, FAKE, wsb, 0) == -1
    assert bw(P(cb), P(Tb), FAKE, FAKE, 1, 16, FAKE + 8, None, None, None, FAKE, wsb, 0) == -3


def test_zero_sized_calls_enqueue_nothing(lib):
    # ntok = 0 / nrows = 0 / nseq = 0 succeed without touching the device.
    cfg = tiny_cfg()
    c, keep = cfg._c()
    T, keep2 = _tables_c(4)
    P = ctypes.byref
    ws = g.ngram_embed_workspace_size(cfg, 0)
    assert lib.ngram_embed_prefill(P(c), P(T), FAKE, FAKE, 0, 0, FAKE, None, FAKE, ws, 0) == 0
    assert lib.ngram_embed_hash(P(c), FAKE, FAKE, 0, 0, FAKE, None, 0) == 0
    assert lib.ngram_embed_gather(P(c), P(T), FAKE, 0, FAKE, 0) == 0
    assert lib.ngram_embed_project(P(c), P(T), FAKE, FAKE, 0, FAKE, 0) == 0
    empty = g._CCache(FAKE, FAKE, 0)
    assert lib.ngram_embed_decode(P(c), P(T), P(empty), FAKE, FAKE, 5, None, FAKE, FAKE, ws, 0) == 0
    assert lib.ngram_cache_commit(P(c), P(empty), FAKE, FAKE, 5, None, 0) == 0
    assert lib.ngram_cache_init(P(c), P(empty), FAKE, FAKE, 0, 0) == 0


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not installed")
def test_host_validation_under_sanitizers(tmp_path):
    """The HIP-free validation unit, built with g++ under ASan/UBSan and exercised."""
    csrc = os.path.join(ROOT, "gram_embedding_layer_amd", "csrc")
    exe = tmp_path / "validate_test"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", f"-I{os.path.join(ROOT, 'include')}", f"-I{csrc}",
           os.path.join(csrc, "validate.cpp"), os.path.join(ROOT, "tests", "validate_test.cpp"),
           "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "all passed" in res.stdout


def test_prefill_cache_argument_checks(lib):
    """cache_or_null of ngram_embed_prefill: one slot per sequence, aligned ring and len."""
    cfg = tiny_cfg()
    c, keep = cfg._c()
    T, keep2 = _tables_c(4)
    P = ctypes.byref
    ws = g.ngram_embed_workspace_size(cfg, 16)
    other = g._CCache(FAKE, FAKE, 3)                        # 3 slots for 2 sequences
    assert lib.ngram_embed_prefill(P(c), P(T), FAKE, FAKE, 2, 16, FAKE, P(other), FAKE, ws,
                                   0) == -1
    bad_len = g._CCache(FAKE, FAKE + 4, 2)                  # int64 lengths, 4-byte aligned
    assert lib.ngram_embed_prefill(P(c), P(T), FAKE, FAKE, 2, 16, FAKE, P(bad_len), FAKE, ws,
                                   0) == -3
    bad_ring = g._CCache(FAKE + 2, FAKE, 2)
    assert lib.ngram_embed_prefill(P(c), P(T), FAKE, FAKE, 2, 16, FAKE, P(bad_ring), FAKE, ws,
                                   0) == -3
    # the workspace is still checked first
    ok = g._CCache(FAKE, FAKE, 2)
    assert lib.ngram_embed_prefill(P(c), P(T), FAKE, FAKE, 2, 16, FAKE, P(ok), FAKE, ws - 1,
                                   0) == -4


def test_binding_rejects_bad_tensors():
    """The binding checks every tensor before its address crosses the C ABI (no GPU needed:
    dtype and shape are checked before the device). int64 token ids, torch's default integer
    type, would otherwise be read as pairs of int32."""
    torch = pytest.importorskip("torch")

    class OnDevice:
        """A host tensor that reports a CUDA device, so that the checks after the device
        check of one argument are reached (every call below still fails a check before any
        pointer is passed to the library)."""
        def __init__(self, t):
            self._t = t
            self.is_cuda = True

        def __getattr__(self, k):
            v = getattr(self._t, k)
            if k in ("long", "float", "int", "t", "__getitem__"):
                return lambda *a: OnDevice(v(*a))
            return v

        def __getitem__(self, i):
            return OnDevice(self._t[i])

    _zeros = torch.zeros

    def zeros(*a, **kw):
        return OnDevice(_zeros(*a, **kw))

    def tensor(*a, **kw):
        return OnDevice(torch.tensor(*a, **kw))

    def full(*a, **kw):
        return OnDevice(torch.full(*a, **kw))

    cfg = tiny_cfg()
    E0 = zeros((1000, 64), dtype=torch.bfloat16)
    E = [zeros((v, 16), dtype=torch.bfloat16) for v in cfg.V]
    W = zeros((64, 64), dtype=torch.bfloat16)
    tables = g.Tables(E0, E, W)
    tok32 = zeros(16, dtype=torch.int32)
    cu = tensor([0, 16], dtype=torch.int32)
    out = zeros((16, 64), dtype=torch.bfloat16)
    ws = zeros(g.ngram_embed_workspace_size(cfg, 16), dtype=torch.uint8)

    def rejects(match, f, *a, **kw):
        with pytest.raises(ValueError, match=match):
            f(*a, **kw)

    rejects("tokens must have dtype torch.int32", g.ngram_embed_prefill, cfg, tables,
            tok32.long(), cu, out, ws)
    rejects("cu_seqlens must have dtype", g.ngram_embed_prefill, cfg, tables, tok32,
            cu.long(), out, ws)
    rejects(r"out must have shape \(16, 64\)", g.ngram_embed_prefill, cfg, tables, tok32, cu,
            out[:15], ws)
    rejects("out must have dtype", g.ngram_embed_prefill, cfg, tables, tok32, cu,
            out.float(), ws)
    rejects("out must be contiguous", g.ngram_embed_prefill, cfg, tables, tok32, cu,
            OnDevice(_zeros((64, 16), dtype=torch.bfloat16).t()), ws)
    rejects("out must be on a CUDA", g.ngram_embed_prefill, cfg, tables, tok32, cu,
            out._t, ws)
    rejects(r"E\[2\] needs 6007 rows", g.ngram_embed_prefill, cfg,
            g.Tables(E0, E[:2] + [E[2][:100]] + E[3:], W), tok32, cu, out, ws)
    rejects(r"W must have shape \(64, 64\)", g.ngram_embed_prefill, cfg,
            g.Tables(E0, E, W[:32]), tok32, cu, out, ws)
    rejects("E0 must have dtype", g.ngram_embed_project, cfg, g.Tables(E0.float(), E, W),
            zeros((16, 4), dtype=torch.int32), tok32, out)
    rejects("idx needs at least 64 elements", g.ngram_embed_project, cfg, tables,
            zeros(63, dtype=torch.int32), tok32, out)
    rejects("tok needs at least 16 elements", g.ngram_embed_project, cfg, tables,
            zeros(64, dtype=torch.int32), tok32[:8], out)
    rejects("idx needs at least", g.ngram_embed_hash, cfg, tok32, cu,
            zeros(10, dtype=torch.int32))
    # decode: per-sequence arrays must have one entry per cache slot
    cache = g.Cache(zeros((4, 2), dtype=torch.int32), zeros(4, dtype=torch.int64))
    new = zeros((4, 5), dtype=torch.int32)
    n4 = full((4,), 5, dtype=torch.int32)
    dout = zeros((4, 5, 64), dtype=torch.bfloat16)
    rejects(r"new_tokens must have shape \(4, \*\)", g.ngram_embed_decode, cfg, tables, cache,
            new[:3], n4, dout, ws)
    rejects(r"n_new must have shape \(4,\)", g.ngram_embed_decode, cfg, tables, cache, new,
            n4[:2], dout, ws)
    rejects(r"n_commit must have shape \(4,\)", g.ngram_embed_decode, cfg, tables, cache, new,
            n4, dout, ws, n_commit=n4[:3])
    rejects(r"out must have shape \(4, 5, 64\)", g.ngram_embed_decode, cfg, tables, cache, new,
            n4, dout[:, :4], ws)
    rejects(r"cache.len must have dtype torch.int64", g.ngram_embed_decode, cfg, tables,
            g.Cache(cache.ring, cache.len.int()), new, n4, dout, ws)
    rejects(r"cache.ring must have shape \(4, 2\)", g.ngram_embed_decode, cfg, tables,
            g.Cache(cache.ring[:, :1], cache.len), new, n4, dout, ws)
    rejects("cu_seqlens must have cache.nseq", g.ngram_cache_init, cfg, cache, tok32, cu)
    rejects(r"n_accept must have shape \(4,\)", g.ngram_cache_commit, cfg, cache, new, n4[:1])
    rejects("one slot per sequence", g.ngram_embed_prefill, cfg, tables, tok32, cu, out, ws,
            cache=cache)
    rejects(r"slots must have shape \(4,\)", g.ngram_embed_decode_rows, cfg, tables, cache,
            new, n4, dout, ws, slots=n4[:2])
    rejects(r"dE\[0\] must have shape \(5003, 16\)", g.ngram_embed_backward, cfg, tables,
            tok32, cu, out, None, [zeros((5003, 8))] * 4, None, ws)
    rejects("dW must have dtype torch.float32", g.ngram_embed_backward, cfg, tables, tok32, cu,
            out, None, None, W, ws)


def test_lds_dma_m0_is_an_operand():
    """The LDS-DMA loads (projection, LDS gather) take their LDS address in m0 as an asm input operand
    ("{m0}"), so the compiler writes m0 itself and keeps no other value there across them.
    Checked on the gfx950 assembly of this repository's source: no reserved-register clobber
    warning, every DMA load preceded by an m0 write and the hazard nop, and no instruction that
    reads m0 for another purpose (movrel, sendmsg) in the projection kernels."""
    from gram_embedding_layer_amd import build
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not installed")
    lines = []
    for src in ("project.hip", "gather.hip"):
        cmd = [build.hipcc(), f"--offload-arch={build.ARCH}", "-O3", "-std=c++17",
               "--cuda-device-only", "-S", "-Xclang", "-target-feature", "-Xclang",
               "-packed-fp32-ops", f"-I{build.INCLUDE}", f"-I{build.CSRC}", "-o", "-",
               os.path.join(build.CSRC, src)]
        res = subprocess.run(cmd, capture_output=True, text=True, check=True)
        assert "reserved registers" not in res.stderr, src
        lines += [ln.strip() for ln in res.stdout.splitlines()]
    dma = [i for i, ln in enumerate(lines) if ln.startswith("global_load_lds_dword")]
    assert dma, "no LDS-DMA loads found"
    for i in dma:
        assert lines[i - 1] == "s_nop 0", lines[i - 3:i + 1]
        prev = [ln for ln in lines[max(0, i - 40):i] if "m0" in ln and not ln.startswith(";")]
        # the compiler's own write of the operand (s_mov, or an address computed into m0)
        assert prev and prev[-1].split()[0].startswith("s_") and \
            prev[-1].split()[1].rstrip(",") == "m0", lines[i - 5:i + 1]
    body = "\n".join(lines)
    for op in ("s_movrel", "v_movrel", "s_sendmsg"):
        assert op not in body, op


def test_noalloc_decode_rejects_before_any_device_call(lib):
    """The allocation-free decode checks its sizes against the fixed scratch (and every
    argument) on the host before touching the device."""
    cfg = tiny_cfg()
    c, keep = cfg._c()
    T, keep2 = _tables_c(4)
    P = ctypes.byref
    per_row = 4 + 4 * cfg.S              # token and indices: 20 bytes per row
    big = g._CCache(FAKE, FAKE, (g.NGRAM_NOALLOC_SCRATCH_BYTES // per_row) // 8 + 64)
    assert lib.ngram_embed_decode_noalloc(P(c), P(T), P(big), FAKE, FAKE, 8, None, FAKE, None,
                                          0) == g.NGRAM_ESCRATCH
    assert g.ngram_embed_status_string(g.NGRAM_ESCRATCH) != "unknown status"
    # the layer normalisation keeps fp32 rows: 64 columns x 4 bytes more per row
    ln = tiny_cfg(amp="layernorm")
    cl, keep3 = ln._c()
    mid = g._CCache(FAKE, FAKE, (g.NGRAM_NOALLOC_SCRATCH_BYTES // (per_row + 256)) // 8 + 64)
    assert lib.ngram_embed_decode_noalloc(P(cl), P(T), P(mid), FAKE, FAKE, 8, None, FAKE,
                                          None, 0) == g.NGRAM_ESCRATCH
    small = g._CCache(FAKE, FAKE, 4)
    assert lib.ngram_embed_decode_noalloc(P(c), P(T), P(small), FAKE, FAKE, 9, None, FAKE,
                                          None, 0) == -1                   # tmax > 8
    assert lib.ngram_embed_decode_noalloc(P(c), P(T), P(small), FAKE + 2, FAKE, 5, None, FAKE,
                                          None, 0) == -3                   # new_tokens
    assert lib.ngram_embed_decode_noalloc(P(c), P(T), P(small), FAKE, FAKE, 5, None, FAKE,
                                          FAKE + 1, 0) == -3               # err_flags
    assert lib.ngram_embed_decode_noalloc(P(c), None, P(small), FAKE, FAKE, 5, None, FAKE,
                                          None, 0) == -3                   # no tables
    empty = g._CCache(FAKE, FAKE, 0)
    assert lib.ngram_embed_decode_noalloc(P(c), P(T), P(empty), FAKE, FAKE, 5, None, FAKE,
                                          None, 0) == 0


def test_gather_checksum_argument_checks(lib):
    cfg = tiny_cfg()
    c, keep = cfg._c()
    T, keep2 = _tables_c(4)
    P = ctypes.byref
    assert lib.ngram_embed_gather_checksum(P(c), P(T), FAKE, -1, FAKE, 0) == -1
    assert lib.ngram_embed_gather_checksum(P(c), P(T), FAKE, 0, FAKE, 0) == 0
    assert lib.ngram_embed_gather_checksum(P(c), P(T), FAKE + 2, 8, FAKE, 0) == -3
    assert lib.ngram_embed_gather_checksum(P(c), P(T), FAKE, 8, FAKE + 1, 0) == -3
    Tb, k3 = _tables_c(4, sub=FAKE + 8)
    assert lib.ngram_embed_gather_checksum(P(c), P(Tb), FAKE, 8, FAKE, 0) == -3
    bad = tiny_cfg(D=62)
    cb, k4 = bad._c()
    assert lib.ngram_embed_gather_checksum(P(cb), P(T), FAKE, 8, FAKE, 0) == -1
