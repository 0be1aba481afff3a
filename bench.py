"""Benchmark of the N-gram embedding forward pass on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--no-decode]

A step is one pass of the whole path over one 64K-token batch of the 30B-parameter layer
(V0=131072, D=3072, N=4, K=4: 12 sub-tables of width 256, ~60 GB, Zipf(1.1) ids, 8 x 8192):
kernel 1 (hash) then kernels 2+3 (gather fused into the bf16 matrix-core projection, E_0
epilogue), the two launches ngram_embed_prefill makes. Inputs are resident in HBM; four
pre-drawn id batches rotate so no batch finds its rows cached.
Besides the JSON line's `value` (tokens/s) it reports:
  roofline      the projection kernel (dominant) against the bf16 matrix-core peak, with
                HIP-event kernel times taken on the launch stream inside the timed region;
  gather        the stand-alone gather kernel against the 8 TB/s HBM peak;
  decode        1000 speculative-verify steps (256 sequences x 5 ids) replayed as a HIP graph;
  cpu_baseline  the CPU oracle timed on this host's cores on a bounded sample.
Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "N-gram embed tokens/sec + achieved HBM GB/s (64K-tok prefill, spec decode)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores
FP32_PEAK_TFLOPS = 157.3        # MI355X fp32 vector (the fp32 configuration's FMA path)
WORKLOAD = "prefill_64k_30b"
DECODE_WORKLOAD = "decode_spec5_30b"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_prefill_64k_30b.txt")
TRAFFIC_DECODE = os.path.join(ROOT, "profiles", "traffic_decode_spec5_30b.txt")
TRAFFIC_BASIC = os.path.join(ROOT, "profiles", "traffic_prefill_64k_basic_30b.txt")
# the three smaller configurations, timed as parity-sized calls of the same path
CONFIG_LEGS = (("tiny_f32", 100), ("bf16_d1024", 20), ("bf16_d2048_n5k4", 20))


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_digest(name):
    p = os.path.join(ROOT, "gram_embedding_layer_amd", "csrc", name)
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def counter_traffic(kernel, source, path=None):
    """HBM bytes per launch of `kernel` from a committed rocprofv3 counter summary (default
    the prefill one; FETCH_SIZE + WRITE_SIZE, each scaled by what it reads for a plain copy of
    known size), or None when it is missing or was taken on a different kernel source."""
    path = TRAFFIC_FILE if path is None else path
    if not os.path.exists(path):
        return None
    kv = {}
    for ln in open(path):
        # "key: value" lines; keys may hold a colon themselves ("project.hip sha256[:16]")
        if ": " in ln and not ln.lstrip().startswith(("#", "|", "-")):
            k, v = ln.rsplit(": ", 1)
            kv[k.strip()] = v.strip()
    if kv.get(f"{source} sha256[:16]") != source_digest(source):
        return None
    try:
        return float(kv[f"{kernel} hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def blas_info():
    from threadpoolctl import threadpool_info
    blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    threads = max([p.get("num_threads", 1) for p in blas] or [1])
    return blas, int(threads)


def cpu_baseline(w, E0, E, W, batches):
    """The oracle as it stands, on whole benchmark batches ([batch, seqlen] token ids). Table
    rows the oracle asks for are copied from HBM first (not timed)."""
    import numpy as np
    import torch

    import oracle
    from threadpoolctl import threadpool_info

    Wh = W.float().cpu().numpy().astype(np.float64)
    Wb = [Wh[:, s * w.d:(s + 1) * w.d] for s in range(w.S)]
    t_hash = t_embed = t_copy = 0.0
    n = 0
    for tokens2d in batches:
        tokens = tokens2d.reshape(-1)
        cu = np.arange(tokens2d.shape[0] + 1, dtype=np.int64) * tokens2d.shape[1]
        t0 = time.perf_counter()
        idx = oracle.hash_indices(w.V0, w.N, w.K, w.V, tokens, cu)
        t_hash += time.perf_counter() - t0
        c0 = time.perf_counter()
        rows = {-1: E0.index_select(0, torch.as_tensor(tokens.astype(np.int64),
                                                       device=E0.device))
                .float().cpu().numpy().astype(np.float64)}
        for s in range(w.S):
            r = torch.as_tensor(idx[:, s], device=E0.device)
            rows[s] = E[s].index_select(0, r).float().cpu().numpy().astype(np.float64)
        t_copy += time.perf_counter() - c0

        def fetch(s, r, rows=rows):
            return rows[s]          # rows already in the oracle's order
        t1 = time.perf_counter()
        oracle.embed_from_indices(w.D, w.N, w.K, tokens, idx, fetch, Wb)
        t_embed += time.perf_counter() - t1
        n += len(tokens)
        del rows
    blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    blas_threads = max([p.get("num_threads", 1) for p in blas] or [1])
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f
                              if ln.startswith("model name")), "")
    except OSError:
        pass
    return {
        "value": round(n / (t_hash + t_embed), 1),
        "unit": "tokens/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": (f"{len(batches)} benchmark batch(es) of {batches[0].shape[0]} x "
                   f"{batches[0].shape[1]} tokens ({n} tokens); "
                   f"python-int hash {t_hash:.2f} s on 1 thread + float64 contraction "
                   f"{t_embed:.2f} s on {blas_threads} BLAS threads; host copy of the named "
                   f"table rows {t_copy:.2f} s not timed"),
        "host_cpus": len(os.sched_getaffinity(0)),
        "host_cpu_model": cpu_model,
        "blas": ", ".join(sorted({f"{p.get('internal_api')} {p.get('version')}" for p in blas})),
        "seconds": {"hash_python_int": round(t_hash, 3), "contraction_float64": round(t_embed, 3),
                    "row_copy_not_timed": round(t_copy, 3)},
    }


def profile_launches(g, WL, cfg, tables, toks, cu, idx, out, stream, dev):
    """A few launches of each kernel, in a fixed order, plus a plain device copy of known size,
    for rocprofv3 counter passes (the copy calibrates FETCH_SIZE / WRITE_SIZE). Prints the
    launch order as one JSON line, so that a pass's dispatches can be told apart."""
    import numpy as np
    import torch
    T, D = out.shape
    w = WL.workload(WORKLOAD)
    order = []
    G = torch.empty_like(out)
    src = torch.empty_like(out).fill_(1.0)
    sums = torch.empty(T, dtype=torch.int32, device=dev)
    uni = [torch.as_tensor(WL.uniform_ids(np.random.default_rng([7, p]), w.V0, (T,))).to(dev)
           for p in range(3)]
    idx_u = torch.empty_like(idx)
    for k in range(3):
        g.ngram_embed_hash(cfg, toks[k], cu, idx, None, stream=stream)
        g.ngram_embed_project(cfg, tables, idx, toks[k], out, stream=stream)
        g.ngram_embed_gather(cfg, tables, idx, G, stream=stream)
        g.ngram_embed_gather_checksum(cfg, tables, idx, sums, stream=stream)
        G.copy_(src)               # plain copy: T*D*2 bytes read, the same written
        g.ngram_embed_hash(cfg, uni[k], cu, idx_u, None, stream=stream)
        g.ngram_embed_gather_checksum(cfg, tables, idx_u, sums, stream=stream)
        order += ["hash", "project", "gather", "gather_lds", "copy", "hash (uniform ids)",
                  "gather_lds (uniform ids)"]
    # decode: 256 sequences x 5 ids on caches of 8192-token histories (no commit), and the
    # draft-phase calls of one row per sequence
    wd = WL.workload(DECODE_WORKLOAD)
    nseq, tmax = wd.batch, wd.decode_new
    hist = torch.as_tensor(WL.token_batch(wd, purpose=0).reshape(-1)).to(dev)
    hcu = torch.as_tensor(np.arange(nseq + 1, dtype=np.int32) * wd.seqlen).to(dev)
    cache = g.Cache.empty(cfg, nseq, device=dev)
    g.ngram_cache_init(cfg, cache, hist, hcu, stream=stream)
    new = torch.as_tensor(WL.token_batch(wd, purpose=1, batch=nseq, seqlen=tmax)).to(dev)
    n_new = torch.full((nseq,), tmax, dtype=torch.int32, device=dev)
    n_one = torch.ones((nseq,), dtype=torch.int32, device=dev)
    dout = torch.empty((nseq, tmax, D), dtype=torch.bfloat16, device=dev)
    dws = g.alloc_workspace(cfg, nseq * tmax, device=dev)
    for k in range(3):
        g.ngram_embed_decode(cfg, tables, cache, new, n_new, dout, dws, stream=stream)
        g.ngram_embed_decode_rows(cfg, tables, cache, new, n_one, dout, dws, row_begin=0,
                                  row_end=1, stream=stream)
        order += ["decode hash", "decode project (1280 rows)", "draft-row hash",
                  "draft-row project (256 rows)"]
    torch.cuda.synchronize()
    del G, src, dout, dws
    # the basic form (Eq. 1) at ~30B parameters: Zipf and uniform ids
    wb = WL.workload("prefill_64k_basic_30b")
    cb = g.Config(wb.N, wb.K, wb.D, wb.dtype, wb.V0, list(wb.V), form="basic")
    E0b, Eb, _ = WL.device_tables(wb, device=dev)
    tb = g.Tables(E0b, Eb, None)
    btok = torch.as_tensor(WL.token_batch(wb, purpose=0).reshape(-1)).to(dev)
    bcu = torch.as_tensor(np.arange(wb.batch + 1, dtype=np.int32) * wb.seqlen).to(dev)
    buni = torch.as_tensor(WL.uniform_ids(np.random.default_rng([8, 0]), wb.V0, (wb.T,))).to(dev)
    bidx = torch.empty((wb.T, wb.S), dtype=torch.int32, device=dev)
    bout = torch.empty((wb.T, wb.D), dtype=torch.bfloat16, device=dev)
    for k in range(3):
        for name, t in (("basic_sum", btok), ("basic_sum (uniform ids)", buni)):
            g.ngram_embed_hash(cb, t, bcu, bidx, None, stream=stream)
            g.ngram_embed_project(cb, tb, bidx, t, bout, stream=stream)
            order += ["basic hash", name]
    torch.cuda.synchronize()
    print(json.dumps({"profile": f"copy bytes {T * D * 2}", "order": order}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward (training gradients) timing")
    ap.add_argument("--no-amp", action="store_true",
                    help="skip the amplified (scale / layer-norm) prefill timings")
    ap.add_argument("--no-layers", action="store_true",
                    help="skip the per-layer (PLNE) batched-launch timing")
    ap.add_argument("--no-stats", action="store_true",
                    help="skip the hash-collision statistics timing")
    ap.add_argument("--no-basic", action="store_true",
                    help="skip the basic-form (Eq. 1) prefill timing")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the three smaller configurations (tiny fp32, D=1024, D=2048)")
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--cpu-batches", type=int, default=4,
                    help="benchmark batches of 64K tokens the CPU oracle is timed on")
    ap.add_argument("--profile", action="store_true",
                    help="only launch each kernel a few times (for rocprofv3 counter runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the layer's data-parallel path needs no second GPU "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gram_embedding_layer_amd as g
    import workloads as WL

    g.load()
    dev = torch.device("cuda:0")
    w = WL.workload(WORKLOAD)
    cfg = g.Config(w.N, w.K, w.D, w.dtype, w.V0, list(w.V))
    T = w.T
    log(f"generating tables: {sum(w.V) * w.d * 2 / 1e9:.1f} GB sub-tables + E0 + W")
    E0, E, W = WL.device_tables(w, device=dev)
    tables = g.Tables(E0, E, W)
    nrot = 4
    tok_host = [WL.token_batch(w, purpose=p) for p in range(nrot)]
    toks = [torch.as_tensor(t.reshape(-1)).to(dev) for t in tok_host]
    cu = torch.as_tensor(np.arange(w.batch + 1, dtype=np.int32) * w.seqlen).to(dev)
    out = torch.empty((T, w.D), dtype=torch.bfloat16, device=dev)
    ws = g.alloc_workspace(cfg, T, device=dev)
    _, idx_off = g.ngram_embed_workspace_layout(cfg, T)
    idx_ws = ws[idx_off:].view(torch.int32)
    idx_rot = [torch.empty((T, w.S), dtype=torch.int32, device=dev) for _ in range(nrot)]
    stream = torch.cuda.current_stream(dev)
    if args.profile:
        profile_launches(g, WL, cfg, tables, toks, cu, idx_rot[0], out, stream, dev)
        return

    def step(k, ev=None):
        r = k % nrot
        if ev is not None:
            ev[0].record(stream)
        g.ngram_embed_hash(cfg, toks[r], cu, idx_ws, ws, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        g.ngram_embed_project(cfg, tables, idx_ws, toks[r], out, stream=stream)
        if ev is not None:
            ev[2].record(stream)

    log(f"warmup {args.warmup} steps")
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize(dev)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(k, evs[k])
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    if g.ngram_embed_read_error_flag(ws, stream=stream) != 0:
        raise RuntimeError("device error flags set during the benchmark")
    t_hash = float(np.mean([e[0].elapsed_time(e[1]) for e in evs])) * 1e-3
    t_proj = float(np.mean([e[1].elapsed_time(e[2]) for e in evs])) * 1e-3
    ms_per_step = wall / args.steps * 1e3
    value = T * args.steps / wall

    esz = 2
    flops = 2.0 * T * w.D * w.D
    alg_bytes_proj = T * (w.S * w.d * esz + w.D * esz + w.D * esz + w.S * 4 + 4) + w.D * w.D * esz
    tflops = flops / t_proj / 1e12
    traffic = counter_traffic("project", "project.hip")
    roofline = {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": traffic, "kernel": "proj_mfma_kernel<256, 0, 256>",
                "kernel_us": round(t_proj * 1e6, 1),
                "algorithmic_hbm_GBps": round(alg_bytes_proj / t_proj / 1e9, 1)}
    if traffic is not None:
        roofline["counter_hbm_GBps"] = round(traffic / t_proj / 1e9, 1)
        roofline["counter_hbm_frac"] = round(traffic / t_proj / 1e9 / HBM_PEAK_GBS, 4)
    log(f"step {ms_per_step:.3f} ms: hash {t_hash*1e6:.1f} us, project {t_proj*1e6:.1f} us "
        f"({tflops:.0f} TFLOP/s)")

    # stand-alone gather: HBM gate (read T*S*d*2 bytes of random rows, write the same)
    G = torch.empty((T, w.D), dtype=torch.bfloat16, device=dev)
    for r in range(nrot):
        g.ngram_embed_hash(cfg, toks[r], cu, idx_rot[r], None, stream=stream)
    for k in range(3):
        g.ngram_embed_gather(cfg, tables, idx_rot[k % nrot], G, stream=stream)
    gev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for k in range(args.steps):
        gev[k][0].record(stream)
        g.ngram_embed_gather(cfg, tables, idx_rot[k % nrot], G, stream=stream)
        gev[k][1].record(stream)
    torch.cuda.synchronize(dev)
    t_g = float(np.mean([a.elapsed_time(b) for a, b in gev])) * 1e-3
    read_b = T * w.S * w.d * esz
    gather = {"kernel": "gather_kernel", "kernel_us": round(t_g * 1e6, 1),
              "read_GBps": round(read_b / t_g / 1e9, 1),
              "read_write_GBps": round(2 * read_b / t_g / 1e9, 1),
              "frac_of_hbm_peak": round(2 * read_b / t_g / 1e9 / HBM_PEAK_GBS, 4),
              "read_only_frac_of_hbm_peak": round(read_b / t_g / 1e9 / HBM_PEAK_GBS, 4),
              "bytes_read": read_b, "bytes_written": read_b,
              "traffic": counter_traffic("gather", "gather.hip"),
              "note": ("HBM -> HBM copy through registers (G written back); the projection "
                       "gathers into LDS instead: see gather_lds")}
    log(f"gather {t_g*1e6:.1f} us: {2*read_b/t_g/1e9:.0f} GB/s read+write")
    # control: uniform ids (no Zipf repeats, so no reuse of rows within a batch)
    uni = [torch.as_tensor(WL.uniform_ids(np.random.default_rng([7, p]), w.V0, (T,))).to(dev)
           for p in range(nrot)]
    for r in range(nrot):
        g.ngram_embed_hash(cfg, uni[r], cu, idx_rot[r], None, stream=stream)
    for k in range(3):
        g.ngram_embed_gather(cfg, tables, idx_rot[k % nrot], G, stream=stream)
    for k in range(args.steps):
        gev[k][0].record(stream)
        g.ngram_embed_gather(cfg, tables, idx_rot[k % nrot], G, stream=stream)
        gev[k][1].record(stream)
    torch.cuda.synchronize(dev)
    t_u = float(np.mean([a.elapsed_time(b) for a, b in gev])) * 1e-3
    gather["uniform_ids_control"] = {
        "kernel_us": round(t_u * 1e6, 1), "read_write_GBps": round(2 * read_b / t_u / 1e9, 1),
        "frac_of_hbm_peak": round(2 * read_b / t_u / 1e9 / HBM_PEAK_GBS, 4)}
    log(f"gather, uniform ids: {t_u*1e6:.1f} us: {2*read_b/t_u/1e9:.0f} GB/s read+write")
    del G, uni

    gather_lds = bench_gather_lds(g, WL, w, cfg, tables, toks, cu, dev, stream, args.steps)

    amp = None
    if not args.no_amp:
        amp = bench_amplification(g, w, tables, toks, cu, dev, stream, args.steps)

    backward = None
    if not args.no_backward:
        backward = bench_backward(g, w, cfg, tables, toks, cu, dev, stream, min(args.steps, 10))

    decode = None
    if not args.no_decode:
        decode = bench_decode(g, WL, cfg, tables, dev, stream, args.decode_steps,
                              with_cpu=not args.no_cpu_baseline)

    basic = None
    if not args.no_basic:
        basic = bench_basic(g, WL, dev, stream, args.steps)

    layers = None
    if not args.no_layers:
        layers = bench_layers(g, WL, dev, stream, min(args.steps, 10))

    stats = None
    if not args.no_stats:
        stats = bench_hash_stats(g, WL, dev, stream, min(args.steps, 10))

    configs = None
    if not args.no_configs:
        configs = bench_configs(g, WL, dev, stream, with_cpu=not args.no_cpu_baseline)

    cpu = None
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on {args.cpu_batches} batches")
        cpu = cpu_baseline(w, E0, E, W, tok_host[:max(1, min(args.cpu_batches, nrot))])
        log(f"cpu baseline {cpu['value']:.0f} tokens/s")

    step_bytes = alg_bytes_proj + T * 4 * (1 + w.S)   # + hash: ids in, indices out
    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "V0": w.V0, "D": w.D, "N": w.N, "K": w.K,
                   "subtables": w.S, "subtable_width": w.d, "ngram_params": sum(w.V) * w.d,
                   "batch": w.batch, "seq_len": w.seqlen, "tokens_per_step": T,
                   "ids": "zipf1.1"},
        "hbm_GBps_algorithmic": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "kernels_us": {"hash": round(t_hash * 1e6, 1), "project": round(t_proj * 1e6, 1)},
        "roofline": roofline,
        "gather": gather,
        "gather_lds": gather_lds,
        "configs": configs,
        "amplification": amp,
        "backward": backward,
        "decode": decode,
        "basic_form": basic,
        "per_layer": layers,
        "hash_stats": stats,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


def bench_amplification(g, w, tables, toks, cu, dev, stream, steps):
    """The prefill entry point on the same batches, plain and with each embedding
    amplification (output factor sqrt(D); layer normalisation with seeded bf16 weight and
    bias), HIP events around each call. The layer normalisation adds an fp32 row write in the
    projection's epilogue and a second, HBM-bound pass (the trace shows its own duration)."""
    import numpy as np
    import torch

    T = int(toks[0].shape[0])
    out = torch.empty((T, w.D), dtype=torch.bfloat16, device=dev)
    rng = np.random.default_rng(7)
    lw = torch.as_tensor(rng.normal(1.0, 0.1, size=w.D)).to(torch.bfloat16).to(dev)
    lb = torch.as_tensor(rng.normal(0.0, 0.1, size=w.D)).to(torch.bfloat16).to(dev)
    res = {"workload": WORKLOAD, "entry": "ngram_embed_prefill"}
    modes = ("none", "scale", "layernorm")
    runs = {}
    for mode in modes:
        cfg = g.Config(w.N, w.K, w.D, w.dtype, w.V0, list(w.V), amp=mode)
        runs[mode] = (cfg, g.Tables(tables.E0, tables.E, tables.W, lw, lb),
                      g.alloc_workspace(cfg, T, device=dev))
    for k in range(3):
        for mode in modes:
            cfg, tab, ws = runs[mode]
            g.ngram_embed_prefill(cfg, tab, toks[k % len(toks)], cu, out, ws, stream=stream)
    # modes interleaved call by call, so clock ramps and cache state treat them alike
    ev = {m: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)] for m in modes}
    for k in range(steps):
        for mode in modes:
            cfg, tab, ws = runs[mode]
            ev[mode][k][0].record(stream)
            g.ngram_embed_prefill(cfg, tab, toks[k % len(toks)], cu, out, ws, stream=stream)
            ev[mode][k][1].record(stream)
    torch.cuda.synchronize(dev)
    for mode in modes:
        if g.ngram_embed_read_error_flag(runs[mode][2], stream=stream) != 0:
            raise RuntimeError(f"device error flags set in the {mode} prefill")
        t = float(np.mean([a.elapsed_time(b) for a, b in ev[mode]])) * 1e-3
        res[mode] = {"us_per_step": round(t * 1e6, 1), "tokens_per_s": round(T / t, 1)}
    del runs
    for mode in ("scale", "layernorm"):
        res[mode]["extra_us_vs_plain"] = round(res[mode]["us_per_step"] -
                                               res["none"]["us_per_step"], 1)
    # the normalisation pass alone moves 4D bytes in (fp32 rows) and 2D out per token
    res["layernorm"]["norm_pass_bytes"] = T * w.D * (4 + 2)
    log(f"prefill: plain {res['none']['us_per_step']:.0f} us, x sqrt(D) "
        f"{res['scale']['us_per_step']:.0f} us, layer norm {res['layernorm']['us_per_step']:.0f} us")
    return res


def bench_basic(g, WL, dev, stream, steps):
    """The basic form (section A2, Eq. 1) with ~30B parameters (3 full-width tables of
    3.2M x 3072 bf16) on 64K-token batches: hash, then the gather-sum kernel, HIP events
    around each on the launch stream. No contraction: the sum kernel is bound by HBM, with
    N rows read and one written per token."""
    import numpy as np
    import torch

    torch.cuda.empty_cache()
    w = WL.workload("prefill_64k_basic_30b")
    cfg = g.Config(w.N, w.K, w.D, w.dtype, w.V0, list(w.V), form="basic")
    log(f"basic form: generating {sum(w.V) * w.D * 2 / 1e9:.1f} GB of tables")
    E0, E, _ = WL.device_tables(w, device=dev)
    tables = g.Tables(E0, E, None)
    T = w.T
    toks = [torch.as_tensor(WL.token_batch(w, purpose=p).reshape(-1)).to(dev) for p in range(4)]
    cu = torch.as_tensor(np.arange(w.batch + 1, dtype=np.int32) * w.seqlen).to(dev)
    out = torch.empty((T, w.D), dtype=torch.bfloat16, device=dev)
    ws = g.alloc_workspace(cfg, T, device=dev)
    _, idx_off = g.ngram_embed_workspace_layout(cfg, T)
    idx = ws[idx_off:].view(torch.int32)
    for k in range(3):
        g.ngram_embed_prefill(cfg, tables, toks[k % 4], cu, out, ws, stream=stream)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for k in range(steps):
        ev[k][0].record(stream)
        g.ngram_embed_hash(cfg, toks[k % 4], cu, idx, ws, stream=stream)
        ev[k][1].record(stream)
        g.ngram_embed_project(cfg, tables, idx, toks[k % 4], out, stream=stream)
        ev[k][2].record(stream)
    torch.cuda.synchronize(dev)
    wall = (time.perf_counter() - t0) / steps
    if g.ngram_embed_read_error_flag(ws, stream=stream) != 0:
        raise RuntimeError("device error flags set in the basic-form prefill")
    t_hash = float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) * 1e-3
    t_sum = float(np.mean([e[1].elapsed_time(e[2]) for e in ev])) * 1e-3
    # per token: N rows of D bf16 read (E_0 and the N-1 tables), one written, the ids
    per_tok = w.N * w.D * 2 + w.D * 2 + w.S * 4 + 4
    gbs = T * per_tok / t_sum / 1e9
    res = {"workload": w.name, "form": "basic (Eq. 1)", "ngram_params": sum(w.V) * w.D,
           "tokens_per_s": round(T / wall, 1), "ms_per_step": round(wall * 1e3, 4),
           "kernels_us": {"hash": round(t_hash * 1e6, 1), "sum": round(t_sum * 1e6, 1)},
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                        "kernel": "basic_sum_kernel<unsigned short, unsigned short>",
                        "bytes_per_token": per_tok}}
    # control: uniform ids (rows repeat far less, so fewer reads hit in cache)
    uni = [torch.as_tensor(WL.uniform_ids(np.random.default_rng([8, p]), w.V0, (T,))).to(dev)
           for p in range(4)]
    idx_u = [torch.empty((T, w.S), dtype=torch.int32, device=dev) for _ in range(4)]
    for p in range(4):
        g.ngram_embed_hash(cfg, uni[p], cu, idx_u[p], ws, stream=stream)
    for k in range(3):
        g.ngram_embed_project(cfg, tables, idx_u[k % 4], uni[k % 4], out, stream=stream)
    (t_u,) = time_launches(lambda k, e: (g.ngram_embed_project(
        cfg, tables, idx_u[k % 4], uni[k % 4], out, stream=stream), e[1].record(stream)),
        stream, steps)
    gbs_u = T * per_tok / t_u / 1e9
    res["uniform_ids_control"] = {"sum_us": round(t_u * 1e6, 1), "achieved_GBps": round(gbs_u, 1),
                                  "frac": round(gbs_u / HBM_PEAK_GBS, 4)}
    tr_u = counter_traffic("basic_sum_uniform", "basic.hip", TRAFFIC_BASIC)
    if tr_u is not None:
        res["uniform_ids_control"]["traffic"] = tr_u
        res["uniform_ids_control"]["counter_hbm_frac"] = round(tr_u / t_u / 1e9 / HBM_PEAK_GBS, 4)
    traffic = counter_traffic("basic_sum", "basic.hip", TRAFFIC_BASIC)
    res["roofline"]["traffic"] = traffic
    if traffic is not None:
        res["roofline"]["counter_hbm_GBps"] = round(traffic / t_sum / 1e9, 1)
        res["roofline"]["counter_hbm_frac"] = round(traffic / t_sum / 1e9 / HBM_PEAK_GBS, 4)
    log(f"basic form: step {wall*1e6:.0f} us, hash {t_hash*1e6:.1f} us, sum {t_sum*1e6:.1f} us "
        f"({gbs:.0f} GB/s); uniform ids {t_u*1e6:.1f} us ({gbs_u:.0f} GB/s)")
    del uni, idx_u
    del E0, E, tables, out, ws, idx
    torch.cuda.empty_cache()
    return res


def bench_layers(g, WL, dev, stream, steps):
    """Per-layer N-gram embedding (section 5.2): 8 layers with tables of their own (D = 2048,
    N = 3, K = 2, 2.0B n-gram parameters each, 38 GB in all). Each layer's embeddings in one
    call per layer, against all 8 layers in one call (hash once, the projections of the 8
    layers in one launch): 64K-token prefill batches, and speculative-verify decode steps
    (256 sequences x 5 ids, no commit so every step does the same work), each captured in
    HIP graphs so that host launch gaps do not count."""
    import numpy as np
    import torch

    torch.cuda.empty_cache()
    w = WL.workload("plne_8x_d2048")
    cfg = g.Config(w.N, w.K, w.D, w.dtype, w.V0, list(w.V))
    log(f"per-layer: generating {w.layers} x {(sum(w.V) * w.d + w.V0 * w.D) * 2 / 1e9:.1f} GB")
    tabs = []
    for l in range(w.layers):
        E0, E, W = WL.device_tables(w, device=dev, seed=l + 1)
        tabs.append(g.Tables(E0, E, W))
    T = w.T
    toks = torch.as_tensor(WL.token_batch(w).reshape(-1)).to(dev)
    cu = torch.as_tensor(np.arange(w.batch + 1, dtype=np.int32) * w.seqlen).to(dev)
    outs = [torch.empty((T, w.D), dtype=torch.bfloat16, device=dev) for _ in range(w.layers)]
    ws = g.alloc_workspace(cfg, T, device=dev)

    def separate(cs):
        for l in range(w.layers):
            g.ngram_embed_prefill(cfg, tabs[l], toks, cu, outs[l], ws, stream=cs)

    def batched(cs):
        g.ngram_embed_prefill_layers(cfg, tabs, toks, cu, outs, ws, stream=cs)

    def graph_us(body, reps):
        """GPU time of `reps` calls captured in one HIP graph (no host gaps), per call."""
        body(stream)
        torch.cuda.synchronize(dev)
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            cs = torch.cuda.current_stream()
            for _ in range(reps):
                body(cs)
        ts = []
        for _ in range(3):
            torch.cuda.synchronize(dev)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            gr.replay()
            b.record(stream)
            torch.cuda.synchronize(dev)
            ts.append(a.elapsed_time(b) * 1e-3 / reps)
        del gr
        return float(np.median(ts))

    t_sep = graph_us(separate, steps)
    t_bat = graph_us(batched, steps)
    flops = 2.0 * T * w.D * w.D * w.layers
    res = {"workload": w.name, "layers": w.layers,
           "prefill": {"tokens": T, "us_separate_calls": round(t_sep * 1e6, 1),
                       "us_one_call": round(t_bat * 1e6, 1),
                       "tflops_one_call": round(flops / t_bat / 1e12, 1)}}
    del outs, ws
    # decode: 256 sequences x 5 ids per step, histories of 8192 ids
    nseq, tmax, nsteps = 256, 5, 200
    hist = torch.as_tensor(WL.token_batch(w, purpose=2, batch=nseq, seqlen=8192).reshape(-1)
                           ).to(dev)
    hcu = torch.as_tensor(np.arange(nseq + 1, dtype=np.int32) * 8192).to(dev)
    cache = g.Cache.empty(cfg, nseq, device=dev)
    g.ngram_cache_init(cfg, cache, hist, hcu, stream=stream)
    ids = torch.as_tensor(WL.token_batch(w, purpose=3, batch=nsteps * nseq, seqlen=tmax)
                          .reshape(nsteps, nseq, tmax)).to(dev)
    n_new = torch.full((nseq,), tmax, dtype=torch.int32, device=dev)
    douts = [torch.empty((nseq, tmax, w.D), dtype=torch.bfloat16, device=dev)
             for _ in range(w.layers)]
    dws = g.alloc_workspace(cfg, nseq * tmax, device=dev)

    def graph_time(body):
        gr = torch.cuda.CUDAGraph()
        torch.cuda.synchronize(dev)
        with torch.cuda.graph(gr):
            cs = torch.cuda.current_stream()
            for s in range(nsteps):
                body(s, cs)
        ts = []
        for _ in range(3):
            torch.cuda.synchronize(dev)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            gr.replay()
            b.record(stream)
            torch.cuda.synchronize(dev)
            ts.append(a.elapsed_time(b) * 1e-3)
        return float(np.median(ts)) / nsteps

    def dec_separate(s, cs):
        for l in range(w.layers):
            g.ngram_embed_decode(cfg, tabs[l], cache, ids[s], n_new, douts[l], dws, stream=cs)

    def dec_batched(s, cs):
        g.ngram_embed_decode_layers(cfg, tabs, cache, ids[s], n_new, douts, dws, stream=cs)

    d_sep = graph_time(dec_separate)
    d_bat = graph_time(dec_batched)
    if g.ngram_embed_read_error_flag(dws, stream=stream) != 0:
        raise RuntimeError("device error flags set in the per-layer timing")
    res["decode"] = {"seqs": nseq, "ids_per_step": tmax, "steps": nsteps,
                     "us_per_step_separate_calls": round(d_sep * 1e6, 2),
                     "us_per_step_one_call": round(d_bat * 1e6, 2)}
    log(f"per-layer ({w.layers} layers): prefill {t_sep*1e6:.0f} us in separate calls, "
        f"{t_bat*1e6:.0f} us in one; decode {d_sep*1e6:.1f} vs {d_bat*1e6:.1f} us/step")
    del tabs, douts, dws, cache
    torch.cuda.empty_cache()
    return res


def bench_hash_stats(g, WL, dev, stream, steps):
    """Hash collisions of the 2-gram hash (section 3.2.2, Fig. 3b): 100 sequences x 8192
    Zipf(1.1) ids, 59 table sizes between 30x and 33x V0 = 131072; rows in use per size and
    the distinct 2-grams, exact, on the device."""
    import numpy as np
    import torch

    V0 = 131072
    ids, sizes = WL.collision_study(V0)
    toks = torch.as_tensor(ids.reshape(-1)).to(dev)
    cu = torch.as_tensor(np.arange(ids.shape[0] + 1, dtype=np.int32) * ids.shape[1]).to(dev)
    rows = torch.empty((len(sizes),), dtype=torch.int64, device=dev)
    distinct = torch.empty((1,), dtype=torch.int64, device=dev)
    ws = g.ngram_hash_stats(V0, 2, toks, cu, sizes, rows, distinct, stream=stream)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        a.record(stream)
        g.ngram_hash_stats(V0, 2, toks, cu, sizes, rows, distinct, ws=ws, stream=stream)
        b.record(stream)
    torch.cuda.synchronize(dev)
    if g.ngram_embed_read_error_flag(ws, stream=stream) != 0:
        raise RuntimeError("device error flags set in the hash statistics")
    t = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e-3
    d = int(distinct.item())
    coll = {v: d - int(r) for v, r in zip(sizes, rows.cpu())}
    res = {"positions": int(toks.numel()), "table_sizes": len(sizes), "n": 2,
           "us_per_call": round(t * 1e6, 1),
           "position_sizes_per_s": round(toks.numel() * len(sizes) / t, 1),
           "distinct_2grams": d,
           "collisions_at_multiples": {f"{m}xV0": coll[m * V0] for m in range(30, 34)},
           "collisions_coprime_sizes": [min(c for v, c in coll.items() if v % 2),
                                        max(c for v, c in coll.items() if v % 2)]}
    log(f"hash stats: {t*1e6:.0f} us for {toks.numel()} positions x {len(sizes)} sizes; "
        f"collisions at multiples {list(res['collisions_at_multiples'].values())}, "
        f"coprime {res['collisions_coprime_sizes']}")
    return res


def bench_backward(g, w, cfg, tables, toks, cu, dev, stream, steps):
    """Gradients of the 64K-token batch for every parameter (fp32 buffers: 120 GB for the
    sub-tables, 3.2 GB for E_0, 38 MB for W), accumulated, HIP events around each call. Its two
    products (dout W and dout^T G) are 2 x 2*T*D^2 flops on the matrix cores; the rest is
    the hash, transposes, sorts and segmented sums."""
    import numpy as np
    import torch

    T = int(toks[0].shape[0])
    rng = np.random.default_rng(11)
    dout = torch.as_tensor(rng.normal(0.0, 1.0, size=(T, w.D)).astype(np.float32)).to(
        torch.bfloat16).to(dev)
    dE0 = torch.zeros((w.V0, w.D), dtype=torch.float32, device=dev)
    dE = [torch.zeros((v, w.d), dtype=torch.float32, device=dev) for v in w.V]
    dW = torch.zeros((w.D, w.D), dtype=torch.float32, device=dev)
    ws = g.alloc_backward_workspace(cfg, T, device=dev)
    log(f"backward: {steps} steps, workspace {ws.numel() / 1e9:.2f} GB")
    for k in range(2):
        g.ngram_embed_backward(cfg, tables, toks[k % len(toks)], cu, dout, dE0, dE, dW, ws,
                               stream=stream)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for k in range(steps):
        ev[k][0].record(stream)
        g.ngram_embed_backward(cfg, tables, toks[k % len(toks)], cu, dout, dE0, dE, dW, ws,
                               stream=stream)
        ev[k][1].record(stream)
    torch.cuda.synchronize(dev)
    if g.ngram_embed_read_error_flag(ws, stream=stream) != 0:
        raise RuntimeError("device error flags set during the backward")
    t = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e-3
    flops = 2 * 2.0 * T * w.D * w.D
    res = {"workload": WORKLOAD, "steps": steps, "us_per_step": round(t * 1e6, 1),
           "tokens_per_s": round(T / t, 1), "product_flops": flops,
           "tflops_over_step": round(flops / t / 1e12, 1),
           "workspace_bytes": int(ws.numel())}
    log(f"backward {t * 1e6:.0f} us per 64K-token step ({flops / t / 1e12:.0f} TFLOP/s of "
        "products over the whole step)")
    del dE0, dE, dW, ws, dout
    torch.cuda.empty_cache()
    return res


def bench_decode(g, WL, cfg, tables, dev, stream, nsteps, with_cpu=False):
    """Speculative-verify decode: 256 sequences with 8192-token histories in the device
    cache; each step proposes 5 ids per sequence (1 + 4 drafts), all committed. The loop is
    captured once as a HIP graph and replayed; the cache is restored before each replay."""
    import numpy as np
    import torch

    wd = WL.workload(DECODE_WORKLOAD)
    nseq, tmax = wd.batch, wd.decode_new
    log(f"decode: {nsteps} steps x {nseq} sequences x {tmax} ids")
    hist_host = WL.token_batch(wd, purpose=0)
    hist = torch.as_tensor(hist_host.reshape(-1)).to(dev)
    cu = torch.as_tensor(np.arange(nseq + 1, dtype=np.int32) * wd.seqlen).to(dev)
    cache = g.Cache.empty(cfg, nseq, device=dev)
    g.ngram_cache_init(cfg, cache, hist, cu, stream=stream)
    ring0, len0 = cache.ring.clone(), cache.len.clone()
    ids_host = WL.token_batch(wd, purpose=1, batch=nsteps * nseq, seqlen=tmax).reshape(
        nsteps, nseq, tmax)
    ids = torch.as_tensor(ids_host).to(dev)
    n_new = torch.full((nseq,), tmax, dtype=torch.int32, device=dev)
    out = torch.empty((nseq, tmax, cfg.D), dtype=torch.bfloat16, device=dev)
    ws = g.alloc_workspace(cfg, nseq * tmax, device=dev)
    # eager warmup of a few steps, then restore the cache
    for s in range(3):
        g.ngram_embed_decode(cfg, tables, cache, ids[s], n_new, out, ws, n_commit=n_new,
                             stream=stream)
    torch.cuda.synchronize(dev)
    # eager steps (host launch path included): best of three rounds of 50, so that a one-off
    # stall (the freeing of the previous leg's buffers) is not read as the step time
    eager_steps = 50
    rounds = []
    for _ in range(3):
        cache.ring.copy_(ring0)
        cache.len.copy_(len0)
        torch.cuda.synchronize(dev)
        t0 = time.perf_counter()
        for s in range(eager_steps):
            g.ngram_embed_decode(cfg, tables, cache, ids[s], n_new, out, ws, n_commit=n_new,
                                 stream=stream)
        torch.cuda.synchronize(dev)
        rounds.append((time.perf_counter() - t0) / eager_steps * 1e6)
    eager_us = min(rounds)
    graph = torch.cuda.CUDAGraph()
    cache.ring.copy_(ring0)
    cache.len.copy_(len0)
    torch.cuda.synchronize(dev)
    with torch.cuda.graph(graph):
        cs = torch.cuda.current_stream()
        for s in range(nsteps):
            g.ngram_embed_decode(cfg, tables, cache, ids[s], n_new, out, ws, n_commit=n_new,
                                 stream=cs)
    times = []
    for rep in range(3):
        cache.ring.copy_(ring0)
        cache.len.copy_(len0)
        torch.cuda.synchronize(dev)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        graph.replay()
        b.record(stream)
        torch.cuda.synchronize(dev)
        times.append(a.elapsed_time(b) * 1e-3)
    t = float(np.median(times))
    if int(cache.len[0].item()) != wd.seqlen + nsteps * tmax:
        raise RuntimeError("decode cache length mismatch after the graph replay")
    if g.ngram_embed_read_error_flag(ws, stream=stream) != 0:
        raise RuntimeError("device error flags set during decode")
    toks = nsteps * nseq * tmax
    log(f"decode graph: {t/nsteps*1e6:.1f} us/step, eager {eager_us:.1f} us/step")

    # Speculative decoding with the rows computed while the draft ids appear (the deep notes'
    # section 4.2): each draft id's row is one call (ngram_embed_decode_rows, window of one
    # row); verify then only commits. Graphs of the same 1000 steps: rows one at a time +
    # commit (all N-gram work of a step), and the commit alone (what stays on the verify
    # step's path).
    n_j = [torch.full((nseq,), j + 1, dtype=torch.int32, device=dev) for j in range(tmax)]

    def graph_time(body):
        gr = torch.cuda.CUDAGraph()
        cache.ring.copy_(ring0)
        cache.len.copy_(len0)
        torch.cuda.synchronize(dev)
        with torch.cuda.graph(gr):
            cs = torch.cuda.current_stream()
            for s in range(nsteps):
                body(s, cs)
        ts = []
        for rep in range(3):
            cache.ring.copy_(ring0)
            cache.len.copy_(len0)
            torch.cuda.synchronize(dev)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            gr.replay()
            b.record(stream)
            torch.cuda.synchronize(dev)
            ts.append(a.elapsed_time(b) * 1e-3)
        return float(np.median(ts)) / nsteps

    def rows_then_commit(s, cs):
        for j in range(tmax):
            g.ngram_embed_decode_rows(cfg, tables, cache, ids[s], n_j[j], out, ws, row_begin=j,
                                      row_end=j + 1, stream=cs)
        g.ngram_cache_commit(cfg, cache, ids[s], n_new, stream=cs)

    def commit_only(s, cs):
        g.ngram_cache_commit(cfg, cache, ids[s], n_new, stream=cs)

    t_rows = graph_time(rows_then_commit)
    t_commit = graph_time(commit_only)
    if g.ngram_embed_read_error_flag(ws, stream=stream) != 0:
        raise RuntimeError("device error flags set during the draft-phase decode")
    draft = {"us_per_step_rows_one_at_a_time": round(t_rows * 1e6, 2),
             "us_per_row_call": round((t_rows - t_commit) / tmax * 1e6, 2),
             "us_verify_path_commit_only": round(t_commit * 1e6, 2)}
    log(f"draft-phase rows: {t_rows*1e6:.1f} us/step in {tmax} calls, verify path "
        f"{t_commit*1e6:.1f} us (one-shot decode {t/nsteps*1e6:.1f} us)")
    # both rooflines of a step: algorithmic bytes (the rows' sub-table pieces, E_0 rows and
    # outputs, ids, W once, the ring read and written) and the product's flops
    rows = nseq * tmax
    step_bytes = (rows * (wd.S * wd.d * 2 + wd.D * 2 + wd.D * 2 + wd.S * 4 + 8)
                  + wd.D * wd.D * 2 + nseq * (2 * (wd.N - 1) * 4 + 16))
    step_flops = 2.0 * rows * wd.D * wd.D
    t_step = t / nsteps
    fractions = {"bytes_per_step": step_bytes, "flops_per_step": step_flops,
                 "hbm_GBps": round(step_bytes / t_step / 1e9, 1),
                 "hbm_frac": round(step_bytes / t_step / 1e9 / HBM_PEAK_GBS, 4),
                 "mfma_TFLOPs": round(step_flops / t_step / 1e12, 1),
                 "mfma_frac": round(step_flops / t_step / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
    cpu = None
    if with_cpu:
        # steps 0 and the last plus 32 seeded ones
        rest = np.random.default_rng(5).choice(np.arange(1, max(2, nsteps - 1)),
                                               size=min(32, max(0, nsteps - 2)), replace=False)
        check = sorted({0, nsteps - 1, *[int(x) for x in rest]})
        log(f"decode cpu baseline: oracle hash of {nsteps} steps, embeddings of {len(check)}")
        cpu = cpu_baseline_decode(wd, tables.E0, tables.E, tables.W,
                                  hist_host[:, wd.seqlen - (wd.N - 1):], ids_host, set(check))
        log(f"decode cpu baseline {cpu['value']:.0f} tokens/s")
    fractions["traffic_decode_projection"] = counter_traffic(
        "decode_project", "project.hip", TRAFFIC_DECODE)
    draft["traffic_row_call_projection"] = counter_traffic("draft_project", "project.hip",
                                                           TRAFFIC_DECODE)
    return {"workload": DECODE_WORKLOAD, "steps": nsteps, "seqs": nseq, "ids_per_step": tmax,
            "tokens_per_s": round(toks / t, 1), "us_per_step_graph": round(t_step * 1e6, 2),
            "us_per_step_eager": round(eager_us, 2), "replays": len(times),
            "roofline_fractions": fractions, "draft_phase": draft, "cpu_baseline": cpu}


def time_launches(fn, stream, reps, nev=2):
    """HIP events on the launch stream around each call of fn(k, ev) (fn records ev[1..]
    between its launches); returns the mean of every interval, in seconds."""
    import numpy as np
    import torch
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(reps)]
    for k in range(reps):
        evs[k][0].record(stream)
        fn(k, evs[k])
    torch.cuda.synchronize()
    return [float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])) * 1e-3
            for i in range(nev - 1)]


def bench_gather_lds(g, WL, w, cfg, tables, toks, cu, dev, stream, steps):
    """Kernel 2 in the form the projection runs it: the sub-table rows of a 64K-token batch
    from HBM straight into LDS with the projection's 16-byte-per-lane LDS loads, reduced
    there to one checksum per row (4 bytes written per row). Zipf(1.1) ids (the workload)
    and uniform ids (no repeats within a batch to hit in cache), four batches rotated; and
    contiguous rows, the loader's ceiling on this layout (a control, not the workload)."""
    import numpy as np
    import torch

    T = int(toks[0].shape[0])
    idx = [torch.empty((T, w.S), dtype=torch.int32, device=dev) for _ in toks]
    uni = [torch.as_tensor(WL.uniform_ids(np.random.default_rng([7, p]), w.V0, (T,))).to(dev)
           for p in range(len(toks))]
    sums = torch.empty(T, dtype=torch.int32, device=dev)
    read_b = T * w.S * w.d * 2
    alg_b = read_b + T * w.S * 4 + T * 4            # rows, indices read, checksums written
    res = {"kernel": "gather_lds_kernel", "loader": "global_load_lds_dwordx4 (HBM -> LDS)",
           "bytes_read_rows": read_b, "bytes_algorithmic": alg_b,
           "traffic": counter_traffic("gather_lds", "gather.hip"),
           "traffic_uniform_ids": counter_traffic("gather_lds_uniform", "gather.hip")}
    # the loader's own ceiling: every sub-table read as one contiguous run of rows (row
    # r + k T of each sub-table in batch k, so the four batches share no line)
    seq = [torch.stack([torch.arange(k * T, (k + 1) * T, dtype=torch.int32, device=dev)] * w.S,
                       dim=1).contiguous() for k in range(len(toks))]
    for name, ids in (("zipf", toks), ("uniform_ids_control", uni),
                      ("sequential_rows_control", None)):
        if ids is None:
            for r in range(len(seq)):
                idx[r].copy_(seq[r])
        for r in range(len(ids) if ids is not None else 0):
            g.ngram_embed_hash(cfg, ids[r], cu, idx[r], None, stream=stream)
        for k in range(3):
            g.ngram_embed_gather_checksum(cfg, tables, idx[k % len(idx)], sums, stream=stream)
        (t,) = time_launches(lambda k, ev: (g.ngram_embed_gather_checksum(
            cfg, tables, idx[k % len(idx)], sums, stream=stream), ev[1].record(stream)),
            stream, steps)
        res[name] = {"kernel_us": round(t * 1e6, 1),
                     "read_GBps": round(read_b / t / 1e9, 1),
                     "algorithmic_GBps": round(alg_b / t / 1e9, 1),
                     "frac_of_hbm_peak": round(alg_b / t / 1e9 / HBM_PEAK_GBS, 4)}
        tr = {"zipf": res["traffic"], "uniform_ids_control": res["traffic_uniform_ids"]}.get(name)
        if tr is not None:
            res[name]["counter_hbm_frac"] = round(tr / t / 1e9 / HBM_PEAK_GBS, 4)
        log(f"gather into LDS, {name}: {t*1e6:.1f} us = {alg_b/t/1e9:.0f} GB/s "
            f"({alg_b/t/1e9/HBM_PEAK_GBS:.1%} of HBM peak)")
    res["frac_of_hbm_peak"] = res["zipf"]["frac_of_hbm_peak"]
    return res


def bench_configs(g, WL, dev, stream, with_cpu):
    """The three smaller configurations through the same entry points the 30B layer uses
    (hash, then the fused gather + projection), each on its own seeded batch: tokens/s, the
    kernels' HIP-event times, and both rooflines (algorithmic bytes and flops per call); the
    CPU oracle on the same whole batch beside each."""
    import numpy as np
    import torch

    out = {}
    for name, reps in CONFIG_LEGS:
        torch.cuda.empty_cache()
        w = WL.workload(name)
        cfg = g.Config(w.N, w.K, w.D, w.dtype, w.V0, list(w.V))
        if w.dtype == "f32":
            E0, E, W = WL.host_tables(w)
            E0, E, W = E0.to(dev), [e.to(dev) for e in E], W.to(dev)
        else:
            E0, E, W = WL.device_tables(w, device=dev)
        tables = g.Tables(E0, E, W)
        tok2d = WL.token_batch(w)
        T = w.T
        toks = torch.as_tensor(tok2d.reshape(-1)).to(dev)
        cu = torch.as_tensor(np.arange(w.batch + 1, dtype=np.int32) * w.seqlen).to(dev)
        out_t = torch.empty((T, w.D), dtype=E0.dtype, device=dev)
        ws = g.alloc_workspace(cfg, T, device=dev)
        _, idx_off = g.ngram_embed_workspace_layout(cfg, T)
        idx = ws[idx_off:].view(torch.int32)
        for _ in range(5):
            g.ngram_embed_prefill(cfg, tables, toks, cu, out_t, ws, stream=stream)
        torch.cuda.synchronize(dev)
        t0 = time.perf_counter()

        def step(k, ev):
            g.ngram_embed_hash(cfg, toks, cu, idx, ws, stream=stream)
            ev[1].record(stream)
            g.ngram_embed_project(cfg, tables, idx, toks, out_t, stream=stream)
            ev[2].record(stream)
        t_hash, t_proj = time_launches(step, stream, reps, nev=3)
        wall = (time.perf_counter() - t0) / reps
        # the same two launches captured `reps` times in one HIP graph: GPU time per call
        # without host launch gaps (small calls finish before the host issues the next)
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            cs = torch.cuda.current_stream()
            for _ in range(reps):
                g.ngram_embed_hash(cfg, toks, cu, idx, ws, stream=cs)
                g.ngram_embed_project(cfg, tables, idx, toks, out_t, stream=cs)
        gts = []
        for _ in range(3):
            torch.cuda.synchronize(dev)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            gr.replay()
            e1.record(stream)
            torch.cuda.synchronize(dev)
            gts.append(e0.elapsed_time(e1) * 1e-3 / reps)
        t_graph = float(np.median(gts))
        del gr
        if g.ngram_embed_read_error_flag(ws, stream=stream) != 0:
            raise RuntimeError(f"device error flags set in the {name} prefill")
        esz = w.esz
        flops = 2.0 * T * w.D * w.D
        alg = (T * (w.S * w.d * esz + 2 * w.D * esz + w.S * 4 + 4) + w.D * w.D * esz
               + T * 4 * (1 + w.S))
        t = t_graph
        peak_f = MFMA_BF16_PEAK_TFLOPS if w.dtype == "bf16" else FP32_PEAK_TFLOPS
        res = {"dtype": w.dtype, "V0": w.V0, "D": w.D, "N": w.N, "K": w.K, "tokens": T,
               "reps": reps, "ids": w.ids,
               "tokens_per_s": round(T / t, 1), "us_per_call": round(t * 1e6, 2),
               "timing": "HIP graph of reps calls (hash + project), median of 3 replays",
               "us_per_call_eager_host_wall": round(wall * 1e6, 2),
               "kernels_us_eager_events": {"hash": round(t_hash * 1e6, 2),
                                           "project": round(t_proj * 1e6, 2)},
               "bytes_algorithmic": int(alg), "flops": flops,
               "hbm_GBps": round(alg / t / 1e9, 1),
               "hbm_frac": round(alg / t / 1e9 / HBM_PEAK_GBS, 4),
               "TFLOPs": round(flops / t / 1e12, 2),
               "compute_peak_TFLOPs": peak_f,
               "compute_frac": round(flops / t / 1e12 / peak_f, 4)}
        if with_cpu:
            res["cpu_baseline"] = cpu_baseline(w, E0, E, W, [tok2d])
        log(f"{name}: {t*1e6:.1f} us per call ({T / t / 1e6:.1f} M tokens/s; "
            f"{res['hbm_frac']:.1%} of HBM, {res['compute_frac']:.1%} of compute peak)"
            + (f"; oracle {res['cpu_baseline']['value']:.0f} tokens/s" if with_cpu else ""))
        out[name] = res
        del E0, E, W, tables, out_t, ws, idx
    torch.cuda.empty_cache()
    return out


def cpu_baseline_decode(wd, E0, E, W, hist_tail, ids, check_steps):
    """The decode oracle on the benchmark's own decode run: every hash index of every step
    (the histories' last N-1 ids, then each step's ids committed in turn) and the embeddings
    of the rows of `check_steps`; the time of the whole run at the measured rate per step is
    reported as extrapolated."""
    import numpy as np
    import torch

    import oracle
    nsteps, nseq, tmax = ids.shape
    orc = oracle.DecodeOracle(wd.V0, wd.D, wd.N, wd.K, wd.V, [list(h) for h in hist_tail])
    kept = {}
    t0 = time.perf_counter()
    for s in range(nsteps):
        step_ids = [list(r) for r in ids[s]]
        idxs = orc.step_indices(step_ids)
        if s in check_steps:
            kept[s] = np.concatenate(idxs)
        orc.commit(step_ids, [tmax] * nseq)
    t_hash = time.perf_counter() - t0
    Wh = W.float().cpu().numpy().astype(np.float64)
    Wb = [Wh[:, q * wd.d:(q + 1) * wd.d] for q in range(wd.S)]
    t_embed = t_copy = 0.0
    for s in sorted(kept):
        tok = ids[s].reshape(-1)
        c0 = time.perf_counter()
        rows = {-1: E0.index_select(0, torch.as_tensor(tok.astype(np.int64), device=E0.device))
                .float().cpu().numpy().astype(np.float64)}
        for q in range(wd.S):
            rows[q] = E[q].index_select(0, torch.as_tensor(kept[s][:, q], device=E0.device)
                                        ).float().cpu().numpy().astype(np.float64)
        t_copy += time.perf_counter() - c0
        t1 = time.perf_counter()
        oracle.embed_from_indices(wd.D, wd.N, wd.K, tok, kept[s], lambda q, r, rows=rows: rows[q],
                                  Wb)
        t_embed += time.perf_counter() - t1
    per_step = t_hash / nsteps + t_embed / len(kept)
    blas, threads = blas_info()
    return {"value": round(nseq * tmax / per_step, 1), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": (f"hash indices of all {nsteps} steps x {nseq} sequences x {tmax} ids "
                       f"({t_hash:.2f} s, python ints, 1 thread); float64 embeddings of "
                       f"{len(kept)} of the steps ({t_embed:.2f} s, {threads} BLAS threads); "
                       f"the {nsteps}-step run at that rate is extrapolated"),
            "seconds": {"hash_all_steps": round(t_hash, 3),
                        "embeddings_sampled_steps": round(t_embed, 3),
                        "row_copy_not_timed": round(t_copy, 3),
                        "whole_run_extrapolated": round(per_step * nsteps, 2)}}


if __name__ == "__main__":
    main()
