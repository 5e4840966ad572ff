"""Prefill attention benchmark: CRISP layer ms and speedup over the dense kernel.

One step = one layer's whole path (proxy -> route -> select -> block-sparse
attention) on one batch of seeded synthetic inputs already resident in HBM.
The proxy emits per-block masses instead of the full proxy map; routing and
selection read those.
The headline workload is the Llama-3.1-8B-shaped 512k-token layer (32 query
heads, 8 KV heads, head dim 128); the Qwen2.5-7B-shaped 128k layer is
reported beside it.  The dense causal kernel, the forced Vertical-Slash
chain and the gamma-cumulative comparison chains are timed separately.

Prints one JSON line (rank 0, N = 1).
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

TILE_FLOP = 4 * 128 * 128 * 128  # QK^T + PV of one 128x128 (query block, key block) tile
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
METRIC = "prefill attn ms/layer + speedup vs own dense kernel at 128k/512k, 1 GPU"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10, help="timed steps of the CRISP chain and of the dense kernel")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--compare-steps", type=int, default=3,
                    help="timed steps of each supplementary chain (forced-VS, gamma)")
    ap.add_argument("--workload", default="llama3.1-8b-512k")
    ap.add_argument("--secondary", default="qwen2.5-7b-128k", help="extra workload reported beside ('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-compare", action="store_true", help="skip the gamma comparison chains")
    ap.add_argument("--only-crisp", action="store_true", help="time the CRISP chain only (profiling runs)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one 1 GiB device-to-device copy first (HBM counter calibration)")
    ap.add_argument("--route", choices=["auto", "vs", "pe"], default="auto",
                    help="route override of the timed CRISP chain (the reported value uses auto)")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the MFMA ceiling probe")
    ap.add_argument("--sweep", action="store_true",
                    help="length sweep instead of the benchmark line: CRISP (route auto, and forced-VS at several "
                         "alpha) against dense from 8k to 512k on the Llama-3.1-8B shape; prints a markdown table")
    ap.add_argument("--sweep-out", default="", help="also write the sweep as JSON to this path")
    ap.add_argument("--agreement", action="store_true",
                    help="C_struct vs JSD routing agreement and routing cost on the five synthetic layers")
    ap.add_argument("--agreement-out", default="", help="also write the agreement report as JSON to this path")
    ap.add_argument("--tau-jsd", type=float, default=0.1, help="JSD distance threshold of the agreement report")
    ap.add_argument("--counts", action="store_true",
                    help="selected-block counts of the noise floor and gamma-cumulative selection per head and "
                         "direction on --counts-workload, with the tiles and time of each chain")
    ap.add_argument("--counts-workload", default="llama3.1-8b-256k")
    ap.add_argument("--counts-out", default="", help="also write the counts report as JSON to this path")
    ap.add_argument("--token-chain", action="store_true",
                    help="time only the token-granular chain (forced VS, alpha 1.25) on --workload (profiling runs)")
    return ap.parse_args()


def kernel_sha():
    h = hashlib.sha256()
    for f in ("attn.hip", "common.h"):
        with open(os.path.join(ROOT, "dynamic_sparse_attention_proxy_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


class Timer:
    """HIP events on torch's current stream, which is the stream every
    libcrisp call is enqueued on."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def __enter__(self):
        self.a = self.torch.cuda.Event(enable_timing=True)
        self.b = self.torch.cuda.Event(enable_timing=True)
        self.a.record()
        return self

    def __exit__(self, *exc):
        self.b.record()
        self.pairs.append((self.a, self.b))

    def ms(self):
        return [a.elapsed_time(b) for a, b in self.pairs]


def _two_block_pays(own, bound):
    return 2000 * bound <= 1035 * own


def attn_schedule(torch, ws):
    """Which attention kernel took the items of the last sparse call on the
    workspace `ws`: the decision words after the schedule sums (bytes
    80..127) give each kernel the pair its own launch test reads."""
    w = [int(t) for t in ws[80:128].view(torch.int64).cpu().tolist()]
    pays = [_two_block_pays(a, b) for a, b in (w[0:2], w[2:4], w[4:6])]
    names = [n for n, p in zip(("two-block", "one-block", "one-block, runs of 16 blocks per XCD"),
                                (pays[0], not pays[1], not pays[2])) if p]
    return names[0] if len(names) == 1 else "unknown"


def run_workload(torch, B, synth, wname, args, cfg_kw, compare):
    w = synth.workload(wname)
    log(f"generating {w.name} on the GPU")
    t0 = time.time()
    x = synth.make_inputs(w, device="cuda")
    torch.cuda.synchronize()
    log(f"generated in {time.time() - t0:.1f}s")
    dims = B.make_dims(w.num_q_heads, w.num_kv_heads, w.seq_len)
    N = w.seq_len // 128
    bufs = B.CrispBuffers(dims, out_dtype=torch.bfloat16)
    override = {"auto": B.ROUTE_AUTO, "vs": B.ROUTE_FORCE_VS, "pe": B.ROUTE_FORCE_PE}[args.route]
    cfg = B.make_cfg(**dict(cfg_kw, route_override=override))
    res = {"workload": w.name}

    # The proxy emits the block masses only (no 4 * 128 * n * Hq-byte map);
    # routing and selection read them.
    mass = bufs.block_mass

    def ev():
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def chain(c, gamma, marks=None):
        """One layer; `marks` collects an event after each stage."""
        t = [ev()] if marks is not None else None
        B.crisp_proxy(dims, x.q, x.k, None, bufs.row_lse, bufs.partials, block_mass=mass)
        if t is not None:
            t.append(ev())
        B.crisp_route(dims, c, None, bufs.c_struct, bufs.route, block_mass=mass)
        if t is not None:
            t.append(ev())
        if gamma is None:
            B.crisp_select(dims, c, x.q, x.k, None, bufs.route, bufs.blocks, bufs.workspace, block_mass=mass)
        else:
            B.crisp_select_gamma(dims, c, gamma, x.q, x.k, None, bufs.route, bufs.blocks, bufs.workspace,
                                 block_mass=mass)
        if t is not None:
            t.append(ev())
        B.crisp_sparse_attn(dims, x.q, x.k, x.v, bufs.blocks["count"], bufs.blocks["idx"], bufs.out, bufs.lse,
                            workspace=bufs.attn_workspace)
        if t is not None:
            t.append(ev())
            marks.append(t)

    def stats(xs):
        ys = sorted(xs)
        return {"median": ys[len(ys) // 2], "min": ys[0], "mean": sum(ys) / len(ys)}

    def timed_chain(c, gamma, steps, warmup):
        for _ in range(warmup):
            chain(c, gamma)
        torch.cuda.synchronize()
        marks = []
        t0 = time.perf_counter()
        ev0 = ev()
        for _ in range(steps):
            chain(c, gamma, marks)
        ev1 = ev()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3 / steps
        step_ms = ev0.elapsed_time(ev1) / steps
        stage = {name: [m[i].elapsed_time(m[i + 1]) for m in marks]
                 for i, name in enumerate(("proxy", "route", "select", "attn"))}
        tiles = int(bufs.blocks["count"].sum().item())
        routes = bufs.route.cpu().tolist()
        attn = stage["attn"]
        return {"ms_per_layer": step_ms, "wall_ms_per_layer": wall, "attn_ms": sum(attn) / len(attn),
                "attn_ms_all": attn, "stage_ms": {k: {kk: round(vv, 4) for kk, vv in stats(v).items()}
                                                  for k, v in stage.items()},
                "tiles": tiles, "tile_frac": tiles / (w.num_q_heads * N * (N + 1) / 2),
                "heads_vs": int(sum(routes)), "heads_pe": len(routes) - int(sum(routes)),
                "attn_kernel": attn_schedule(torch, bufs.attn_workspace)}

    log(f"{w.name}: CRISP chain (route {args.route}), warmup {args.warmup}, steps {args.steps}")
    res["crisp"] = timed_chain(cfg, None, args.steps, args.warmup)
    res["crisp"]["c_struct"] = [round(float(c), 6) for c in bufs.c_struct.cpu().tolist()]
    log(f"{w.name}: crisp {res['crisp']['ms_per_layer']:.2f} ms")
    if args.only_crisp:
        return res, x, dims
    res["map_path"] = time_map_path(torch, B, x, dims, cfg, args.compare_steps)
    log(f"{w.name}: map path proxy {res['map_path']['proxy_ms']:.3f} ms, select {res['map_path']['select_ms']:.3f} ms")
    # dense baseline
    for _ in range(args.warmup):
        B.crisp_dense_attn(dims, x.q, x.k, x.v, bufs.out, workspace=bufs.attn_workspace)
    torch.cuda.synchronize()
    dt = Timer(torch)
    for _ in range(args.steps):
        with dt:
            B.crisp_dense_attn(dims, x.q, x.k, x.v, bufs.out, workspace=bufs.attn_workspace)
    torch.cuda.synchronize()
    d_ms = dt.ms()
    # the dense call takes the rule the schedule pass applies to full lists
    own = sum((qa + 1) + (qa + 2 if qa + 1 < N else 0) for qa in range(0, N, 2))
    bound = sum(qa + 2 if qa + 1 < N else qa + 1 for qa in range(0, N, 2))
    res["dense"] = {"ms_per_layer": sum(d_ms) / len(d_ms), "ms_all": d_ms,
                    "ms": {kk: round(vv, 4) for kk, vv in stats(d_ms).items()},
                    "tiles": w.num_q_heads * N * (N + 1) // 2,
                    "attn_kernel": "two-block" if _two_block_pays(own, bound) else "one-block"}
    log(f"{w.name}: dense {res['dense']['ms_per_layer']:.2f} ms")
    # forced Vertical-Slash: the noise-floor selection on every head
    for alpha in (1.25, 1.0):
        c = B.make_cfg(**dict(cfg_kw, route_override=B.ROUTE_FORCE_VS, alpha=alpha))
        r = timed_chain(c, None, args.compare_steps, 1)
        r["n_v_mean"] = float(bufs.blocks["n_v"].float().mean())
        r["n_s_mean"] = float(bufs.blocks["n_s"].float().mean())
        res[f"forced_vs_alpha{alpha}"] = r
        log(f"{w.name}: forced-VS alpha {alpha}: {r['ms_per_layer']:.2f} ms, {r['tiles']} tiles")
    # token-granular vertical selection, forced VS
    tb = B.CrispBuffers(dims, tokens=True)
    for alpha in (1.25,):
        c = B.make_cfg(**dict(cfg_kw, route_override=B.ROUTE_FORCE_VS, alpha=alpha))
        r = timed_token_chain(torch, B, x, dims, tb, c, args.compare_steps, 1)
        r["tiles"] = int(tb.blocks["count"].sum().item())
        r["tile_frac"] = r["tiles"] / (w.num_q_heads * N * (N + 1) / 2)
        r["kept_columns_mean"] = float(tb.ncols.float().mean())
        r["gathered_columns"] = int(tb.col_below.sum().item())
        r["needle_recall_last_block"] = needle_recall(x, tb, N, tokens=True)
        res[f"forced_vs_tokens_alpha{alpha}"] = r
        log(f"{w.name}: forced-VS tokens alpha {alpha}: {r['ms_per_layer']:.2f} ms, {r['tiles']} tiles + "
            f"{r['gathered_columns']} gathered columns, needle recall {r['needle_recall_last_block']:.3f}")
    del tb
    torch.cuda.empty_cache()
    c = B.make_cfg(**dict(cfg_kw, route_override=B.ROUTE_FORCE_VS, alpha=1.25))
    chain(c, None)
    torch.cuda.synchronize()
    res["forced_vs_alpha1.25"]["needle_recall_last_block"] = needle_recall(x, bufs, N, tokens=False)
    if compare:
        for gamma in (0.95, 0.97):
            c = B.make_cfg(**dict(cfg_kw, route_override=B.ROUTE_FORCE_VS))
            r = timed_chain(c, gamma, args.compare_steps, 1)
            r["n_v_mean"] = float(bufs.blocks["n_v"].float().mean())
            r["n_s_mean"] = float(bufs.blocks["n_s"].float().mean())
            res[f"gamma{gamma}_forced_vs"] = r
            log(f"{w.name}: gamma {gamma} (VS heads): {r['ms_per_layer']:.2f} ms, {r['tiles']} tiles")
    dense_ms = res["dense"]["ms_per_layer"]
    for key in list(res):
        if isinstance(res[key], dict) and "ms_per_layer" in res[key] and key != "dense":
            res[key]["speedup_vs_dense"] = dense_ms / res[key]["ms_per_layer"]
    return res, x, dims


def timed_token_chain(torch, B, x, dims, tb, cfg, steps, warmup):
    """The token-granular chain (forced route in cfg): per-stage event times."""
    names = ("proxy_cols", "route", "select_tokens", "attn_tiles", "attn_cols")

    def one(marks=None):
        t = []

        def mark():
            if marks is not None:
                e = torch.cuda.Event(enable_timing=True)
                e.record()
                t.append(e)

        mark()
        B.crisp_proxy_cols(dims, x.q, x.k, tb.block_mass, tb.col_mass, tb.row_lse, tb.partials)
        mark()
        B.crisp_route(dims, cfg, None, tb.c_struct, tb.route, block_mass=tb.block_mass)
        mark()
        B.crisp_select_tokens(dims, cfg, x.q, x.k, tb.block_mass, tb.col_mass, tb.route, tb.blocks, tb.cols,
                              tb.ncols, tb.col_below, tb.workspace)
        mark()
        B.crisp_sparse_attn(dims, x.q, x.k, x.v, tb.blocks["count"], tb.blocks["idx"], tb.out, tb.lse,
                            workspace=tb.attn_workspace)
        mark()
        B.crisp_sparse_attn_cols(dims, x.q, x.k, x.v, tb.blocks["count"], tb.blocks["idx"], tb.cols, tb.col_below,
                                 tb.out, tb.lse, workspace=tb.attn_workspace)
        mark()
        if marks is not None:
            marks.append(t)

    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    marks = []
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        one(marks)
    e1.record()
    torch.cuda.synchronize()
    stage = {nm: sorted(m[i].elapsed_time(m[i + 1]) for m in marks)[len(marks) // 2] for i, nm in enumerate(names)}
    return {"ms_per_layer": e0.elapsed_time(e1) / steps, "stage_ms_median": {k: round(v, 4) for k, v in stage.items()}}


def needle_recall(x, bufs, N, tokens):
    """Share of (sink head, needle) pairs whose key the last query block
    attends: its key block is listed, or (token chain) it is a kept column."""
    qpg = x.q.shape[0] // x.k.shape[0]
    count = bufs.blocks["count"].cpu().numpy()
    idx = bufs.blocks["idx"].cpu().numpy()
    if tokens:
        cols = bufs.cols.cpu().numpy()
        ncols = bufs.ncols.cpu().numpy()
    hit = tot = 0
    base_last = (N - 1) * N // 2
    for h in x.sink_heads:
        g = h // qpg
        s = h * (N * (N + 1) // 2) + base_last
        listed = set(idx[s:s + int(count[h, N - 1])].tolist())
        kept = set(cols[h, :int(ncols[h])].tolist()) if tokens else set()
        for p in x.needle_pos.get(g, []):
            tot += 1
            hit += int((p // 128) in listed or p in kept)
    return hit / tot if tot else None


def time_map_path(torch, B, x, dims, cfg, steps):
    """The proxy writing the full map and selection reading it (the ABI's map
    path, off the default chain): stage times and the map store's HBM rate."""
    bufs = B.CrispBuffers(dims, out_dtype=torch.bfloat16, diagnostics=False, with_map=True)
    ts = {"proxy": [], "route": [], "select": []}
    for it in range(steps + 1):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        e[0].record()
        B.crisp_proxy(dims, x.q, x.k, bufs.attn_map, bufs.row_lse, bufs.partials)
        e[1].record()
        B.crisp_route(dims, cfg, bufs.attn_map, bufs.c_struct, bufs.route)
        e[2].record()
        B.crisp_select(dims, cfg, x.q, x.k, bufs.attn_map, bufs.route, bufs.blocks, bufs.workspace)
        e[3].record()
        torch.cuda.synchronize()
        if it > 0:
            for i, k in enumerate(ts):
                ts[k].append(e[i].elapsed_time(e[i + 1]))
    med = {k: sorted(v)[len(v) // 2] for k, v in ts.items()}
    map_bytes = 4 * dims.block * dims.seq_len * dims.num_q_heads
    del bufs
    torch.cuda.empty_cache()
    return {"proxy_ms": round(med["proxy"], 4), "route_ms": round(med["route"], 4),
            "select_ms": round(med["select"], 4), "map_bytes": map_bytes}


def mfma_ceiling(torch):
    """Sustained bf16 MFMA rate of this GPU on N(0,1) operands (the data the
    attention kernels see; the clock under load depends on it), measured by
    the probe library: median of 5 launches of ~20 ms."""
    import ctypes

    path = os.path.join(ROOT, "dynamic_sparse_attention_proxy_amd", "libcrisp_probe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not found: build it with `python -m dynamic_sparse_attention_proxy_amd.build`")
    probe = ctypes.CDLL(path)
    probe.crisp_probe_mfma_bf16.restype = ctypes.c_int
    probe.crisp_probe_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_void_p]
    probe.crisp_probe_mfma_bf16_flops.restype = ctypes.c_double
    probe.crisp_probe_mfma_bf16_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    gen = torch.Generator(device="cuda").manual_seed(11)
    ops = torch.randn(16 * 64 * 8, generator=gen, device="cuda").to(torch.bfloat16)
    nblocks, iters = 256 * 2 * 8, 4096
    sink = torch.empty(nblocks * 256, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def launch():
        st = probe.crisp_probe_mfma_bf16(ctypes.c_void_p(ops.data_ptr()), ctypes.c_void_p(sink.data_ptr()), nblocks,
                                         iters, stream)
        if st != 0:
            raise RuntimeError(f"MFMA probe failed ({st})")

    launch()
    torch.cuda.synchronize()
    ms = []
    for _ in range(5):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        launch()
        b.record()
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    ms.sort()
    return probe.crisp_probe_mfma_bf16_flops(nblocks, iters) / (ms[2] * 1e-3) / 1e12


def _host_cpu():
    """CPU model, logical CPU count and BLAS thread pools of the host."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    try:
        import numpy  # noqa: F401  (loads the BLAS whose pools are listed)
        from threadpoolctl import threadpool_info
        blas = [f"{i.get('internal_api')}:{i.get('num_threads')}" for i in threadpool_info()]
    except Exception:  # pragma: no cover
        blas = []
    return {"cpu_model": model, "logical_cpus": os.cpu_count(), "blas_threads": blas}


def cpu_baseline(q, k, v, dims, res, cfg_kw):
    """The fp64 oracle on a bounded sample of the same layer (head 0), scaled
    to ms/layer: per-head proxy/route/scores x Hq, pooled-estimation rows by
    their length, attention by the tiles the GPU chain computed."""
    from oracle import crisp_oracle as O

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    hq, n = dims.num_q_heads, dims.seq_len
    N = n // 128
    ocfg = O.OracleConfig(**{kk: vv for kk, vv in cfg_kw.items() if kk in ("tau", "alpha", "gamma_pe")})
    t0 = time.perf_counter()
    A, _ = O.proxy_map(q[-128:], k, dims.scale)
    c = O.c_struct(A)
    O.route(c, ocfg.tau)
    ct, dg = O.token_scores(A)
    O.pooled_scores(ct, dg)
    t_head = time.perf_counter() - t0
    del A
    t0 = time.perf_counter()
    qbar, kbar = O.pe_pool(q), O.pe_pool(k)
    rows = [N - 1 - 7 * i for i in range(48)]
    lists = {qb: O.pe_row_select(qbar, kbar, qb, dims.scale, ocfg.gamma_pe) for qb in rows}
    t_rows = time.perf_counter() - t0
    t_pe_head = t_rows / sum(qb + 1 for qb in rows) * (N * (N + 1) / 2)
    # attention of sampled query blocks, one at a time, until about 10 s of CPU work
    att_rows, t_att = [], 0.0
    for qb in rows:
        t0 = time.perf_counter()
        O.attention_rows(q, k, v, lists, dims.scale, [qb])
        t_att += time.perf_counter() - t0
        att_rows.append(qb)
        if t_att >= 10.0:
            break
    tiles_sampled = sum(len(lists[qb]) for qb in att_rows)
    tiles = res["crisp"]["tiles"]
    total_s = t_head * hq + t_pe_head * res["crisp"]["heads_pe"] + t_att / tiles_sampled * tiles
    return {"value": round(total_s * 1e3, 1), "unit": "ms", "cores": int(threads), "kind": "oracle",
            "host": _host_cpu(),
            "sample": (f"head 0 of {res['workload']}: proxy map, C_struct and vertical/slash scores in full, "
                       f"{len(rows)} pooled-estimation rows, attention of query blocks {att_rows} "
                       f"({tiles_sampled} tiles); scaled to {hq} heads, N(N+1)/2 pooled pairs per PE head "
                       f"and the {tiles} tiles the GPU chain computed"),
            "measured_s": round(t_head + t_rows + t_att, 2)}


SWEEP_LENGTHS = (8192, 16384, 32768, 65536, 131072, 262144, 524288)
SWEEP_ALPHAS = (1.0, 1.25, 1.5)


def sweep(torch, B, synth, args):
    """CRISP vs dense across context lengths (Llama-3.1-8B shape, the 512k
    workload's generator at each length): median of `--compare-steps` runs."""
    base = synth.workload("llama3.1-8b-512k")
    rows = []

    def med(fn, steps):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        ms = []
        for _ in range(steps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b))
        return sorted(ms)[len(ms) // 2]

    for n in SWEEP_LENGTHS:
        x = synth.make_inputs(base, device="cuda", seq_len=n)
        dims = B.make_dims(base.num_q_heads, base.num_kv_heads, n)
        bufs = B.CrispBuffers(dims, out_dtype=torch.bfloat16)
        N = n // 128
        dense_tiles = base.num_q_heads * N * (N + 1) // 2
        row = {"seq_len": n, "dense_ms": med(lambda: B.crisp_dense_attn(dims, x.q, x.k, x.v, bufs.out,
                                                                         workspace=bufs.attn_workspace),
                                             args.compare_steps)}
        chains = [("auto", B.make_cfg())] + [(f"vs_alpha{a}", B.make_cfg(route_override=B.ROUTE_FORCE_VS, alpha=a))
                                             for a in SWEEP_ALPHAS]
        for name, cfg in chains:
            t = med(lambda: B.crisp_prefill(dims, cfg, x.q, x.k, x.v, bufs, dense_below=0), args.compare_steps)
            tiles = int(bufs.blocks["count"].sum().item())
            row[name] = {"ms": t, "tiles": tiles, "tile_frac": tiles / dense_tiles, "speedup": row["dense_ms"] / t}
        del bufs
        tb = B.CrispBuffers(dims, tokens=True)
        ct = B.make_cfg(route_override=B.ROUTE_FORCE_VS, alpha=1.25)
        t = med(lambda: B.crisp_prefill_tokens(dims, ct, x.q, x.k, x.v, tb), args.compare_steps)
        row["tokens_alpha1.25"] = {"ms": t, "tiles": int(tb.blocks["count"].sum().item()),
                                   "gathered_columns": int(tb.col_below.sum().item()),
                                   "tile_frac": int(tb.blocks["count"].sum().item()) / dense_tiles,
                                   "speedup": row["dense_ms"] / t}
        log(f"sweep n={n}: dense {row['dense_ms']:.3f} ms, " +
            ", ".join(f"{nm} {row[nm]['ms']:.3f} ms" for nm, _ in chains) +
            f", tokens {row['tokens_alpha1.25']['ms']:.3f} ms")
        rows.append(row)
        del x, tb
        torch.cuda.empty_cache()
    names = ["auto"] + [f"vs_alpha{a}" for a in SWEEP_ALPHAS] + ["tokens_alpha1.25"]
    print("| n | dense ms | " + " | ".join(f"{nm} ms (speedup, tiles)" for nm in names) + " |")
    print("|---|---|" + "---|" * len(names))
    for r in rows:
        cells = [f"{r[nm]['ms']:.3f} ({r[nm]['speedup']:.2f}x, {100 * r[nm]['tile_frac']:.1f}%)" for nm in names]
        print(f"| {r['seq_len']} | {r['dense_ms']:.3f} | " + " | ".join(cells) + " |")
    if args.sweep_out:
        with open(args.sweep_out, "w") as f:
            json.dump(rows, f, indent=1)
    return rows


COUNT_CHAINS = (("route auto", None, None, None), ("noise floor alpha 1.25", 1.25, None, "vs"),
                ("noise floor alpha 1.0", 1.0, None, "vs"), ("gamma 0.95", 1.25, 0.95, "vs"),
                ("gamma 0.97", 1.25, 0.97, "vs"))


def counts(torch, B, synth, args):
    """Selected-block counts, noise floor against gamma-cumulative coverage.

    Both rules run on every head's vertical and slash block scores (route
    forced to Vertical-Slash), beside the route-auto chain: per head and
    direction the kept blocks, and per chain the tiles the attention
    computes and the layer's time.  The O(n) claim (ai.info "Key
    Contributions" 3) shows as the gamma counts covering most of the N
    blocks while the noise floor keeps a handful."""
    w = synth.workload(args.counts_workload)
    log(f"generating {w.name} on the GPU")
    x = synth.make_inputs(w, device="cuda")
    dims = B.make_dims(w.num_q_heads, w.num_kv_heads, w.seq_len)
    bufs = B.CrispBuffers(dims, out_dtype=torch.bfloat16)
    N = -(-w.seq_len // 128)
    dense_tiles = w.num_q_heads * N * (N + 1) // 2
    dense_ms = _med_ms(torch, lambda: B.crisp_dense_attn(dims, x.q, x.k, x.v, bufs.out, workspace=bufs.attn_workspace),
                       args.compare_steps)
    rows = []
    for name, alpha, gamma, route in COUNT_CHAINS:
        kw = {} if route is None else {"route_override": B.ROUTE_FORCE_VS, "alpha": alpha}
        cfg = B.make_cfg(**kw)
        t = _med_ms(torch, lambda: B.crisp_prefill(dims, cfg, x.q, x.k, x.v, bufs, gamma=gamma, dense_below=0),
                    args.compare_steps)
        tiles = int(bufs.blocks["count"].sum().item())
        routes = bufs.route.cpu().tolist()
        r = {"chain": name, "ms": t, "tiles": tiles, "tile_frac": tiles / dense_tiles, "speedup": dense_ms / t,
             "heads_vs": int(sum(routes)), "n_v": bufs.blocks["n_v"].cpu().tolist(),
             "n_s": bufs.blocks["n_s"].cpu().tolist()}
        rows.append(r)
        log(f"counts {w.name} {name}: {t:.2f} ms, {tiles} tiles ({100 * r['tile_frac']:.1f}%)")
    sink = set(range(w.num_sink_heads))
    print(f"Workload {w.name}: {w.num_q_heads} query / {w.num_kv_heads} KV heads, n = {w.seq_len}, N = {N} "
          f"blocks of 128; dense causal tiles {dense_tiles}; dense kernel {dense_ms:.2f} ms\n")
    print("| chain | VS heads | ms | speedup vs dense | tiles | of causal | mean vertical blocks | "
          "mean slash blocks |")
    print("|---|---|---|---|---|---|---|---|")
    for r in rows:
        # vertical/slash counts mean something only when every head took the VS route
        cells = ("-", "-") if r["chain"] == "route auto" else \
            (f"{sum(r['n_v']) / len(r['n_v']):.1f}", f"{sum(r['n_s']) / len(r['n_s']):.1f}")
        print(f"| {r['chain']} | {r['heads_vs']} | {r['ms']:.2f} | {r['speedup']:.2f}x | {r['tiles']} | "
              f"{100 * r['tile_frac']:.2f}% | {cells[0]} | {cells[1]} |")
    per = [r for r in rows if r["chain"] != "route auto"]
    print("\nKept blocks per head, vertical / slash (of N = %d per direction)\n" % N)
    print("| head | kind | " + " | ".join(r["chain"] for r in per) + " |")
    print("|---|---|" + "---|" * len(per))
    for h in range(w.num_q_heads):
        kind = "sink" if h in sink else "diffuse"
        print(f"| {h} | {kind} | " + " | ".join(f"{r['n_v'][h]} / {r['n_s'][h]}" for r in per) + " |")
    if args.counts_out:
        with open(args.counts_out, "w") as f:
            json.dump({"workload": w.name, "dense_ms": dense_ms, "dense_tiles": dense_tiles, "rows": rows}, f,
                      indent=1)
    return rows


AGREEMENT_WORKLOADS = (0, 1, 2, 3, 4, "family-32k", "family-512k")
AGREEMENT_TAUS = (0.2, 0.5)
AGREEMENT_TAU_JSDS = (0.1, 0.2, 0.3, 0.4, 0.5)


def _med_ms(torch, fn, steps):
    for _ in range(2):
        fn()
    torch.cuda.synchronize()
    ms = []
    for _ in range(steps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    return sorted(ms)[len(ms) // 2]


def _ranks(xs):
    order = sorted(range(len(xs)), key=lambda i: xs[i])
    r = [0.0] * len(xs)
    i = 0
    while i < len(order):
        j = i
        while j + 1 < len(order) and xs[order[j + 1]] == xs[order[i]]:
            j += 1
        for t in range(i, j + 1):
            r[order[t]] = (i + j) / 2.0
        i = j + 1
    return r


def _spearman(a, b):
    if len(a) < 3:
        return None
    ra, rb = _ranks(a), _ranks(b)
    ma, mb = sum(ra) / len(ra), sum(rb) / len(rb)
    num = sum((x - ma) * (y - mb) for x, y in zip(ra, rb))
    den = math.sqrt(sum((x - ma) ** 2 for x in ra) * sum((y - mb) ** 2 for y in rb))
    return num / den if den > 0 else None


def agreement_stats(c, d, tau, tau_jsds):
    """Share of heads on which 'C_struct >= tau' and 'JSD distance >= t'
    agree, for each t in tau_jsds and for the best t over all thresholds."""
    vs_c = [x >= tau for x in c]
    h = len(c)
    at = {t: sum(int((dd >= t) == v) for dd, v in zip(d, vs_c)) / h for t in tau_jsds}
    best, best_t = -1.0, None
    for t in sorted(set(d)) + [float("inf")]:
        acc = sum(int((dd >= t) == v) for dd, v in zip(d, vs_c)) / h
        if acc > best:
            best, best_t = acc, t
    return {"tau": tau, "vs_heads_cstruct": int(sum(vs_c)), "agreement_at": at, "best_agreement": best,
            "best_tau_jsd": None if best_t == float("inf") else best_t}


def agreement(torch, B, synth, args):
    """Routing agreement between C_struct and the JSD signal on every head of
    the five synthetic layers and of the graded-structure family, and the
    cost of each routing step on top of the proxy (median of --steps runs)."""
    rows = []
    for wid in AGREEMENT_WORKLOADS:
        if isinstance(wid, int):
            x = synth.make_inputs(synth.workload(wid), device="cuda")
        else:
            x = synth.make_routing_family(seq_len=32768 if wid == "family-32k" else 524288, device="cuda")
        w = x.workload
        hq, hkv, n = w.num_q_heads, w.num_kv_heads, w.seq_len
        dims = B.make_dims(hq, hkv, n)
        cfg = B.make_cfg()
        N = B.num_blocks(n)
        mass = torch.empty((4, hq, N), dtype=torch.float32, device="cuda")
        partials = torch.empty(B.crisp_proxy_scratch_bytes(dims), dtype=torch.uint8, device="cuda")
        cs = torch.empty(hq, dtype=torch.float32, device="cuda")
        rt = torch.empty(hq, dtype=torch.int32, device="cuda")
        ws = torch.empty(B.crisp_route_jsd_workspace_bytes(dims), dtype=torch.uint8, device="cuda")
        jd = torch.empty(hq, dtype=torch.float32, device="cuda")
        jr = torch.empty(hq, dtype=torch.int32, device="cuda")

        def proxy():
            B.crisp_proxy(dims, x.q, x.k, None, partials=partials, block_mass=mass)

        def route_c():
            B.crisp_route(dims, cfg, None, cs, rt, block_mass=mass)

        def route_j():
            B.crisp_route_jsd(dims, args.tau_jsd, x.q, x.k, mass, jd, jr, ws)

        t_proxy = _med_ms(torch, proxy, args.steps)
        t_c = _med_ms(torch, route_c, args.steps)
        t_j = _med_ms(torch, route_j, args.steps)
        torch.cuda.synchronize()
        c, d = cs.cpu().tolist(), jd.cpu().tolist()
        k_bytes = hkv * n * 128 * 2
        row = {"workload": w.name, "heads": hq, "seq_len": n,
               "stats": [agreement_stats(c, d, tau, AGREEMENT_TAU_JSDS) for tau in AGREEMENT_TAUS],
               "spearman": _spearman(c, d),
               "proxy_ms": t_proxy, "route_cstruct_ms": t_c, "route_jsd_ms": t_j,
               "route_jsd_k_bytes": k_bytes, "route_jsd_gbs": k_bytes / (t_j * 1e-3) / 1e9,
               "c_struct": c, "js_dist": d}
        log(f"agreement {w.name}: C_struct in [{min(c):.3f}, {max(c):.3f}], JSD distance in "
            f"[{min(d):.3f}, {max(d):.3f}]; proxy {t_proxy:.3f} ms, route C {t_c * 1e3:.1f} us, "
            f"route JSD {t_j * 1e3:.1f} us")
        rows.append(row)
        del x
        torch.cuda.empty_cache()
    for si, tau in enumerate(AGREEMENT_TAUS):
        print(f"\nC_struct tau = {tau}: share of heads routed alike, by JSD-distance threshold\n")
        print("| workload | heads | VS by C_struct | " + " | ".join(f"tau_jsd {t}" for t in AGREEMENT_TAU_JSDS) +
              " | best (at tau_jsd) | Spearman(C, JSD) |")
        print("|---|---|---|" + "---|" * len(AGREEMENT_TAU_JSDS) + "---|---|")
        for r in rows:
            st = r["stats"][si]
            bt = "-" if st["best_tau_jsd"] is None else f"{st['best_tau_jsd']:.3f}"
            sp = "-" if r["spearman"] is None else f"{r['spearman']:.3f}"
            print(f"| {r['workload']} | {r['heads']} | {st['vs_heads_cstruct']} | " +
                  " | ".join(f"{100 * st['agreement_at'][t]:.1f}%" for t in AGREEMENT_TAU_JSDS) +
                  f" | {100 * st['best_agreement']:.1f}% ({bt}) | {sp} |")
    print("\nRouting cost on top of the proxy (median, ms)\n")
    print("| workload | proxy (block masses) | route from C_struct | route from JSD | JSD K read GB/s |")
    print("|---|---|---|---|---|")
    for r in rows:
        print(f"| {r['workload']} | {r['proxy_ms']:.3f} | {r['route_cstruct_ms']:.4f} | {r['route_jsd_ms']:.4f} | "
              f"{r['route_jsd_gbs']:.0f} |")
    if args.agreement_out:
        with open(args.agreement_out, "w") as f:
            json.dump({"taus": AGREEMENT_TAUS, "tau_jsds": AGREEMENT_TAU_JSDS, "rows": rows}, f, indent=1)
    return rows


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the CRISP layer is timed on a single MI355X "
              "(a multi-GPU run would shard whole KV groups with no communication; not built).", file=sys.stderr)
        sys.exit(2)
    import torch

    from dynamic_sparse_attention_proxy_amd import binding as B
    from dynamic_sparse_attention_proxy_amd import synth

    B.lib()
    torch.cuda.set_device(0)
    if args.sweep:
        sweep(torch, B, synth, args)
        return
    if args.agreement:
        agreement(torch, B, synth, args)
        return
    if args.counts:
        counts(torch, B, synth, args)
        return
    if args.token_chain:
        w = synth.workload(args.workload)
        x = synth.make_inputs(w, device="cuda")
        dims = B.make_dims(w.num_q_heads, w.num_kv_heads, w.seq_len)
        tb = B.CrispBuffers(dims, tokens=True)
        c = B.make_cfg(tau=0.5, alpha=1.25, gamma_pe=0.95, route_override=B.ROUTE_FORCE_VS)
        r = timed_token_chain(torch, B, x, dims, tb, c, args.steps, args.warmup)
        r["gathered_columns"] = int(tb.col_below.sum().item())
        print(json.dumps({"workload": w.name, "token_chain": r}))
        return
    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copy: 1 GiB read + 1 GiB written")
        del src, dst
    cfg_kw = dict(tau=0.5, alpha=1.25, gamma_pe=0.95)
    t_start = time.time()
    main_res, x, dims = run_workload(torch, B, synth, args.workload, args, cfg_kw, compare=not args.no_compare)
    crisp = main_res["crisp"]
    value = crisp["ms_per_layer"]
    achieved = TILE_FLOP * crisp["tiles"] / (crisp["attn_ms"] * 1e-3) / 1e12
    traffic = None
    tfile = os.path.join(ROOT, "profiles", "sparse_attn_traffic.json")
    if os.path.exists(tfile):
        with open(tfile) as f:
            t = json.load(f)
        if t.get("kernel_sha") == kernel_sha() and t.get("workload") == main_res["workload"]:
            traffic = t.get("hbm_bytes_per_launch")
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                "kernel": "fa_fwd_kernel<false> (crisp_sparse_attn)", "kernel_ms": round(crisp["attn_ms"], 3),
                "flop_per_launch": TILE_FLOP * crisp["tiles"]}
    if not args.no_ceiling:
        log("measuring the MFMA ceiling on N(0,1) bf16 operands")
        ceil = mfma_ceiling(torch)
        roofline["ceiling_measured"] = {
            "value": round(ceil, 1), "unit": "TFLOP/s", "frac": round(achieved / ceil, 4),
            "probe": "independent v_mfma_f32_32x32x16_bf16 chains on N(0,1) bf16 operands, 2 workgroups of "
                     "4 waves per CU (libcrisp_probe.so)"}
    cpu_inputs = None
    if not args.no_cpu_baseline and not args.only_crisp:
        g0 = 0
        cpu_inputs = tuple(t.double().cpu().numpy() for t in (x.q[0], x.k[g0], x.v[g0]))
    secondary = None
    if args.secondary and not args.only_crisp:
        del x
        torch.cuda.empty_cache()
        sres, sx, _ = run_workload(torch, B, synth, args.secondary, args, cfg_kw, compare=False)
        del sx
        secondary = sres
    cpu = None
    if cpu_inputs is not None:
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(*cpu_inputs, dims, main_res, cfg_kw)
    speed = main_res.get("dense", {}).get("ms_per_layer")
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(value, 3),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Gaussians with planted sink and needles, RoPE; shapes of the named model)",
        "config": {"workload": main_res["workload"], "num_q_heads": dims.num_q_heads,
                   "num_kv_heads": dims.num_kv_heads, "seq_len": dims.seq_len, "head_dim": 128, "block": 128,
                   "route": args.route, "proxy_output": "block_mass", **cfg_kw},
        "speedup_vs_dense": round(speed / value, 4) if speed else None,
        "dense_ms": round(speed, 3) if speed else None,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "detail": main_res,
        "secondary": secondary,
        "wall_s": round(time.time() - t_start, 1),
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
