#!/usr/bin/env python3
"""Benchmark of the binarized linear layers on one MI355X (gfx950).

Headline (one JSON line on stdout): BitLinear W1A8 decode of one token through
a 4096 x 11008 layer -- LayerNorm + absmax-quant prologue, then the packed
1-bit GEMV with its epilogue -- as whole-step throughput in GB/s of algorithmic
bytes, with the weights rotated over enough distinct copies (> 512 MB) that
every step streams its packed signs from HBM rather than the 256 MB MALL.
The timed region replays a HIP graph of exactly K captured steps.

Extra objects on the same line:
  roofline      the decode GEMV kernel: algorithmic bytes per launch over its
                average launch duration (one launch per step, so the timed
                region's HIP-event time over the K launches), against 8 TB/s.
  cpu_baseline  the CPU oracle on the same workload (one thread, bounded sample).
  legs          every other hot-path row at its workload: the two weight
                conversions, W1A16 decode over a 7B-shaped layer (B = 1, 4, 16),
                the W1A16 and W1A8 prefill GEMMs at 4096 x 4096 x 11008, a
                1.3B-shaped 24-layer stack (decode B = 64, prefill 2 x 1024),
                and BitNet b1.58 ternary weights (decode and prefill at the
                BitLinear shapes).
Progress lines go to stderr.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
INT8_PEAK_TOPS = 5000.0
METRIC = "packed-W1 GEMV HBM GB/s (% of peak); W1 GEMM TFLOP/s/TOP/s (% MFMA peak)"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000, help="timed steps of the headline workload")
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--rotate-mb", type=float, default=640.0, help="packed weight bytes in the rotation")
    ap.add_argument("--legs", default="all", help="comma list of extra legs, 'all' or 'none'")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="bound on the one-core CPU-oracle samples (split over the workloads)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--ceilings", action="store_true",
                    help="also run the ceiling microbenchmarks (part of --legs all)")
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="processes for the all-core CPU oracle timing (0: min(16, cores))")
    ap.add_argument("--calib-copy-mb", type=float, default=0.0,
                    help="only run a plain device copy of this many MB (HBM counter calibration) and exit")
    return ap.parse_args()


# ----------------------------------------------------------------- timing ----

MALL_FLUSH_BYTES = 1 << 30          # read before a timed region: 4x the 256 MB Infinity Cache
_flush_buf = None


def flush_buffer(torch):
    """The 1 GiB buffer flush_mall reads, allocated on first use."""
    global _flush_buf
    if _flush_buf is None:
        _flush_buf = torch.ones(MALL_FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
    return _flush_buf


def flush_mall(torch):
    """Stream 1 GiB through the memory-side cache (a read-only reduction), so
    that nothing a timed region reads is left in the 256 MB MALL or the L2s."""
    flush_buffer(torch).sum()
    torch.cuda.synchronize()


GRAPH_WARM_S = 0.1                  # untimed replays before a timed one: at least this much GPU work


def graph_time(torch, body, steps, warmup, flush=True):
    """Capture `steps` calls of body(i) into one HIP graph; replay it untimed
    until at least GRAPH_WARM_S has passed (warm-up, also `warmup` eager calls
    before capture), stream 1 GiB through the MALL (flush=True), then replay
    once timed. The clocks climb for some milliseconds after an idle spell: a
    3 ms window of prefill GEMMs read up to 25% slow right after one idle
    second, and the same at any length once the GPU had been busy for 50 ms.
    The flush buffer is allocated before the warm-up, so that no idle spell
    falls between the warm-up and the timed replay.
    Returns milliseconds for the timed replay."""
    if flush:
        flush_buffer(torch)
    for i in range(warmup):
        body(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            body(i)
    t0 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    while time.perf_counter() - t0 < GRAPH_WARM_S:
        g.replay()
        torch.cuda.synchronize()
    if flush:
        flush_mall(torch)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    del g
    return ms


def per_launch_ms(torch, launch, n, busy_mb=1024):  # pragma: no cover - diagnostic
    """Average device duration of launch(i) from event pairs around each call.
    A long copy is queued first so all n calls are enqueued before the GPU
    reaches them: each event pair then brackets only the kernel(s)."""
    a = torch.empty(int(busy_mb * 2**20) // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    for _ in range(max(16, n // 10)):          # ~0.4 ms each: longer than enqueueing n calls
        b.copy_(a)
    for i in range(n):
        ev[i][0].record()
        launch(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    d = sorted(s.elapsed_time(e) for s, e in ev)
    del a, b
    return sum(d) / n, d[len(d) // 2]


# ---------------------------------------------------------- headline leg ----

def headline_host_state(syn):
    """The headline workload's host inputs (numpy only: no GPU is touched)."""
    cfg = syn.CONFIGS["bitlinear_decode_4096x11008"]
    K, N, M, seed = cfg["K"], cfg["N"], cfg["M"], cfg["seed"]
    W = syn.normal_f32(seed, 0, (K, N), mean=cfg["w_mean"], std=cfg["w_std"])
    x = syn.normal_f32(seed, 1, (M, K))
    pbytes = 16 * ((K + 127) // 128) * N          # the packed format: one 16-byte tile per 128 rows per column
    return dict(W=W, x=x, K=K, N=N, M=M, step_bytes=pbytes + M * K * 4 + M * N * 4)


def headline(torch, bgb, syn, args):
    cfg = syn.CONFIGS["bitlinear_decode_4096x11008"]
    K, N, M, seed = cfg["K"], cfg["N"], cfg["M"], cfg["seed"]
    host = headline_host_state(syn)
    W_host, x_host = host["W"], host["x"]
    P0, beta, centre = bgb.binarize_pack(torch.from_numpy(W_host).cuda(), bgb.MODE_BITNET)
    pbytes = bgb.packed_bytes(K, N)
    R = max(2, math.ceil(args.rotate_mb * 1e6 / pbytes))
    Ps = [P0] + [P0.clone() for _ in range(R - 1)]
    x = torch.from_numpy(x_host).cuda()
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(bgb.workspace_bytes(bgb.OP_BITLINEAR, M, K, N), 256), dtype=torch.uint8, device="cuda")

    def step(i):
        bgb.bitlinear_w1a8(x, Ps[i % R], beta, N, y=y, ws=ws)

    log(f"headline: BitLinear W1A8 decode M={M} K={K} N={N}, {R} weight copies ({R * pbytes / 1e6:.0f} MB)")
    # the MALL is flushed between the warm and the timed replay, so each copy
    # the timed replay reads comes from HBM at any --steps; a copy is read
    # again only after the other R - 1 (643 MB) have been
    ms = graph_time(torch, step, args.steps, args.warmup)
    ms_step = ms / args.steps
    step_bytes = pbytes + M * K * 4 + M * N * 4          # packed signs + x (f32) + y (f32)
    assert step_bytes == host["step_bytes"]
    value = step_bytes / (ms_step * 1e-3) / 1e9
    log(f"headline: {ms_step * 1e3:.2f} us/step, {value:.1f} GB/s")

    # roofline of the dominant kernel: for one token the whole step is a single
    # launch of the fused decode kernel, so its average launch duration is the
    # timed region's HIP-event time over the K launches (same stream, no gaps
    # other than the hardware's own dispatch of dependent kernels)
    kbytes = step_bytes
    achieved = value
    roof = {"kernel": "bitlinear_decode1_kernel", "bound": "hbm", "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic_bytes("bitlinear_decode1_kernel"), "bytes_per_launch": kbytes,
            "avg_launch_us": round(ms_step * 1e3, 3), "launches": args.steps}

    # correctness spot check of the timed configuration against the first copy
    y_ref = bgb.bitlinear_w1a8(x, P0, beta, N)
    bgb.bitlinear_w1a8(x, Ps[R - 1], beta, N, y=y, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref), "rotated copy disagrees"

    state = dict(W=W_host, x=x_host, K=K, N=N, M=M, step_bytes=step_bytes,
                 distinct_bytes=min(args.steps, R) * pbytes)
    del Ps
    return ms_step, value, roof, R, state


def traffic_bytes(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE runs, each scaled by a plain copy's reading),
    or None if the kernel source has changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(kernel)
    if not rec:
        return None
    h = hashlib.sha256()
    for rel in rec["sources"]:                   # the kernel's source file and the headers it includes
        src = os.path.join(ROOT, rel)
        if not os.path.exists(src):
            return None
        h.update(open(src, "rb").read())
    if h.hexdigest() != rec["sources_sha256"]:
        return None
    return int(round((rec["fetch_kib"] * rec["fetch_scale"] + rec["write_kib"] * rec["write_scale"]) * 1024))


# ------------------------------------------------------------ cpu baseline ----

def host_info():
    """CPU model, logical CPUs and whether SMT is on (Linux /proc and /sys)."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    smt = None
    try:
        smt = open("/sys/devices/system/cpu/smt/active").read().strip() == "1"
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(), "smt": smt}


_JOBS = []          # per-worker closures, inherited by forked workers


def _run_job(i):
    t0 = time.perf_counter()
    _JOBS[i]()
    return time.perf_counter() - t0


def _oracle_cases(state):
    """The oracle on each workload, as (name, unit work, fn(cols) -> callable,
    columns, work per full config, sample note). fn(cols) returns a closure
    that computes the sample for output columns `cols` only; run over all
    columns it is the whole sample."""
    import numpy as np
    import oracle
    import bgb_synth as syn
    cases = []
    # 768 x 768 FBI-linear, 8 bf16 tokens (whole workload)
    c = syn.CONFIGS["fbi_768"]
    W1 = syn.normal_f32(c["seed"], 0, (c["K"], c["N"]), std=c["w_std"])
    x1 = syn.f32_to_bf16_bits(syn.normal_f32(c["seed"], 1, (c["M"], c["K"])))
    a1 = oracle.fbi_alpha(W1)
    cases.append(("fbi_w1a16_768x768_m8", lambda cols: (lambda: oracle.fbi_linear(
        x1, np.ascontiguousarray(W1[:, cols]), a1[cols])), c["N"], 1.0, "the whole workload"))
    # BitLinear decode 4096 x 11008 (whole workload: LN + quant, product, output)
    W2, xf2 = state["W"], state["x"]
    c2, b2 = oracle.bitnet_scalars(W2)

    def bl(cols):
        Wc = np.ascontiguousarray(W2[:, cols])

        def f():
            q, g, _, _ = oracle.ln_absmax_quant(xf2)
            acc = oracle.bitlinear_acc(q, Wc, c2)
            oracle.bitlinear_out(acc, b2, g)
        return f
    cases.append(("bitlinear_w1a8_decode_4096x11008", bl, W2.shape[1], 1.0, "the whole workload"))
    # 7B layer at one token: the q (4096 x 4096) and gate (4096 x 11008) shapes;
    # a layer is 4 of the first (q, k, v, o) and 3 of the second's size (gate, up, down)
    Wq = syn.normal_f32(2, 0, (4096, 4096), std=0.02)
    Wg = syn.normal_f32(2, 4, (4096, 11008), std=0.02)
    xq = syn.f32_to_bf16_bits(syn.normal_f32(2, 100, (1, 4096)))
    aq, ag = oracle.fbi_alpha(Wq), oracle.fbi_alpha(Wg)

    def layer7b(cols):
        cq = cols[cols < 4096]
        Wqc, Wgc = np.ascontiguousarray(Wq[:, cq]), np.ascontiguousarray(Wg[:, cols])

        def f():
            oracle.fbi_linear(xq, Wqc, aq[cq])
            oracle.fbi_linear(xq, Wgc, ag[cols])
        return f
    layer_adds = 4 * 4096 * 4096 + 3 * 4096 * 11008
    cases.append(("w1a16_decode_7b_layer_b1", layer7b, 11008, layer_adds / (4096 * 4096 + 4096 * 11008),
                  "one q-shaped and one gate-shaped linear at one token, scaled to the layer's 7 linears"))
    # 4096 x 4096 x 11008 prefill, W1A16: 8 of the 4096 token rows, scaled by 512
    xp = syn.f32_to_bf16_bits(syn.normal_f32(3, 1, (8, 4096)))
    Wp = syn.normal_f32(3, 0, (4096, 11008), std=0.02)
    ap_ = oracle.fbi_alpha(Wp)
    cases.append(("w1a16_prefill_4096x4096x11008", lambda cols: (lambda: oracle.fbi_linear(
        xp, np.ascontiguousarray(Wp[:, cols]), ap_[cols])), 11008, 4096 / 8,
        "8 of the 4096 token rows, scaled by 512"))
    # 1.3B stack decode at batch 64: one layer's q and gate shapes for 8 tokens, scaled to 7 linears x 24 layers x 64 tokens
    Wq5 = syn.normal_f32(4, 0, (2048, 2048), std=0.02)
    Wg5 = syn.normal_f32(4, 4, (2048, 5632), std=0.02)
    x5 = syn.f32_to_bf16_bits(syn.normal_f32(4, 100, (8, 2048)))
    aq5, ag5 = oracle.fbi_alpha(Wq5), oracle.fbi_alpha(Wg5)

    def stack(cols):
        cq = cols[cols < 2048]
        Wqc, Wgc = np.ascontiguousarray(Wq5[:, cq]), np.ascontiguousarray(Wg5[:, cols])

        def f():
            oracle.fbi_linear(x5, Wqc, aq5[cq])
            oracle.fbi_linear(x5, Wgc, ag5[cols])
        return f
    stack_adds = 24 * 64 * (4 * 2048 * 2048 + 3 * 2048 * 5632)
    cases.append(("w1a16_1p3b_stack_decode_b64", stack, 5632, stack_adds / (8 * (2048 * 2048 + 2048 * 5632)),
                  "8 tokens through one q-shaped and one gate-shaped linear, scaled to 7 linears x 24 layers x 64 tokens"))
    return cases


def cpu_baseline(state, seconds, workers):
    """The oracle as it stands (plain single-threaded C), timed on this host:
    every workload on one core, and on `workers` cores by running the same
    oracle in forked processes on disjoint slices of the output columns (each
    output is computed exactly as in the one-core run). The headline's value
    is the one-core BitLinear decode rate."""
    import concurrent.futures as cf
    import multiprocessing as mp
    import numpy as np
    cases = _oracle_cases(state)
    info = host_info()
    budget = seconds / len(cases)
    per = {}
    head = None
    for name, fn, ncols, scale, note in cases:
        allc = np.arange(ncols)
        f = fn(allc)
        n, t0 = 0, time.perf_counter()
        while True:
            f()
            n += 1
            if time.perf_counter() - t0 >= budget:
                break
        t1 = (time.perf_counter() - t0) / n
        rec = {"ms_1core": round(t1 * scale * 1e3, 3), "sample": note, "sample_ms_1core": round(t1 * 1e3, 3),
               "repeats": n}
        if workers > 1:
            global _JOBS
            _JOBS = [fn(sl) for sl in np.array_split(allc, workers)]
            with cf.ProcessPoolExecutor(workers, mp_context=mp.get_context("fork")) as ex:
                list(ex.map(_run_job, range(workers)))              # warm the workers
                reps = max(1, n)
                tw = []
                for _ in range(reps):
                    w0 = time.perf_counter()
                    list(ex.map(_run_job, range(workers)))
                    tw.append(time.perf_counter() - w0)
            _JOBS = []
            tmin = min(tw)
            rec.update({"ms_all_cores": round(tmin * scale * 1e3, 3), "cores": workers,
                        "speedup": round(t1 / tmin, 2)})
        per[name] = rec
        log(f"cpu oracle {name}: {rec['ms_1core']:.1f} ms on 1 core"
            + (f", {rec['ms_all_cores']:.1f} ms on {workers}" if workers > 1 else ""))
        if name == "bitlinear_w1a8_decode_4096x11008":
            head = (t1, n)
    dt, n = head
    value = state["step_bytes"] / dt / 1e9
    return {"value": round(value, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} full decode steps (M=1, K=4096, N=11008: LN+quant, integer product, output) "
                      f"in {n * dt:.1f} s, plain single-thread C oracle", "ms_per_step": round(dt * 1e3, 2),
            **info, "all_core_workers": workers, "per_config": per}


# ------------------------------------------------------------------ legs ----

def leg_pack(torch, bgb, syn):
    out = {}
    K, N = 4096, 11008
    W = syn.gpu_normal(3, 0, (K, N), mean=0.001, std=0.02)
    pbytes = bgb.packed_bytes(K, N)
    for name, mode in (("pack_fbi_4096x11008", bgb.MODE_FBI), ("pack_bitnet_4096x11008", bgb.MODE_BITNET)):
        ws = torch.empty(max(bgb.workspace_bytes(mode, 0, K, N), 256), dtype=torch.uint8, device="cuda")
        P = torch.empty(pbytes // 4, dtype=torch.int32, device="cuda")
        alpha = torch.empty(N, dtype=torch.float32, device="cuda")
        beta = torch.empty(4, dtype=torch.float32, device="cuda")
        cen = torch.empty(4, dtype=torch.float32, device="cuda")

        def body(i):
            bgb.binarize_pack(W, mode, P=P, alpha=alpha, beta=beta, centre=cen, ws=ws)

        steps = 20
        ms = graph_time(torch, body, steps, 3) / steps
        reads = K * N * 4 * (1 if mode == bgb.MODE_FBI else 2)
        nbytes = reads + pbytes + (N * 4 if mode == bgb.MODE_FBI else 8)
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"ms": round(ms, 4), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                     "bytes": nbytes, "bound": "hbm"}
        log(f"{name}: {ms * 1e3:.1f} us, {gbs:.0f} GB/s")
    return out


def leg_fbi_768(torch, bgb, syn):
    """The 768 x 768 FBI-linear (130M-class hidden size): 8 bf16 tokens, fp32
    output, fp32 alpha. 113,664 algorithmic bytes per call: bound by launch
    latency, so it reports microseconds per call (back-to-back in a graph,
    and one call at a time between HIP events)."""
    c = syn.CONFIGS["fbi_768"]
    K, N, M = c["K"], c["N"], c["M"]
    W = torch.from_numpy(syn.normal_f32(c["seed"], 0, (K, N), std=c["w_std"])).cuda()
    xb = syn.f32_to_bf16_bits(syn.normal_f32(c["seed"], 1, (M, K)))
    import numpy as np
    x = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)
    P, alpha = bgb.binarize_pack(W, bgb.MODE_FBI)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(bgb.workspace_bytes(bgb.OP_FBI_LINEAR, M, K, N), 256), dtype=torch.uint8, device="cuda")

    def body(i):
        bgb.fbi_linear_w1a16(x, P, alpha, N, y=y, ws=ws)

    n = 1000
    ms = graph_time(torch, body, n, 20) / n
    avg, med = per_launch_ms(torch, body, 200)
    nbytes = bgb.packed_bytes(K, N) + 4 * N + 2 * M * K + 4 * M * N
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"fbi 768x768 M=8: {ms * 1e3:.2f} us/call back-to-back, {med * 1e3:.2f} us one call at a time")
    return {"fbi_w1a16_768x768_m8": {"us_per_call": round(ms * 1e3, 3), "us_single_call_median": round(med * 1e3, 3),
                                     "us_single_call_mean": round(avg * 1e3, 3), "GB/s": round(gbs, 1),
                                     "frac_hbm": round(gbs / HBM_PEAK_GBS, 5), "bytes": nbytes,
                                     "bound": "launch latency (113,664 B per call)"}}


def cold_step_ms(torch, body, n):
    """Milliseconds of one step (body(0), captured once as a HIP graph) with
    the MALL flushed before each of n timed replays: the median and the
    spread over the replays."""
    body(0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body(0)
    g.replay()
    torch.cuda.synchronize()
    t = []
    for _ in range(n):
        flush_mall(torch)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        t.append(e0.elapsed_time(e1))
    del g
    t.sort()
    return t[len(t) // 2], t[0], t[-1]


def build_layer(torch, bgb, syn, seed, shapes, layer, alpha_dtype):
    Ps, alphas = [], []
    for li, (_, K, N) in enumerate(shapes):
        W = syn.gpu_normal(seed, 100 * layer + li, (K, N), std=0.02)
        P, a = bgb.binarize_pack(W, bgb.MODE_FBI, alpha_dtype)
        Ps.append(P)
        alphas.append(a)
        del W
    return Ps, alphas


def leg_decode_7b(torch, bgb, syn, steps):
    cfg = syn.CONFIGS["w1a16_decode_7b_layer"]
    shapes = cfg["shapes"]
    L = 32                                              # distinct layer copies: 809 MB of signs
    P1, A1 = build_layer(torch, bgb, syn, cfg["seed"], shapes, 0, torch.float16)
    layers = [(P1, A1)] + [([p.clone() for p in P1], A1) for _ in range(L - 1)]
    pbytes = sum(bgb.packed_bytes(K, N) for _, K, N in shapes)
    abytes = sum(2 * N for _, K, N in shapes)
    out = {}
    for B in cfg["batches"]:
        xs = {K: torch.randn((B, K), device="cuda").to(torch.bfloat16) for K in (4096, 11008)}
        ys = {N: torch.empty((B, N), dtype=torch.bfloat16, device="cuda") for N in (4096, 11008)}
        wsz = max(bgb.workspace_bytes(bgb.OP_FBI_LINEAR, B, K, N) for _, K, N in shapes)
        ws = torch.empty(max(wsz, 256), dtype=torch.uint8, device="cuda")

        def body(i, B=B, xs=xs, ys=ys, ws=ws):
            Ps, As = layers[i % L]
            for li, (_, K, N) in enumerate(shapes):
                bgb.fbi_linear_w1a16(xs[K], Ps[li], As[li], N, y=ys[N], ws=ws)

        n = steps
        ms = graph_time(torch, body, n, 4) / n
        xb = sum(2 * B * K for _, K, N in shapes)
        yb = sum(2 * B * N for _, K, N in shapes)
        nbytes = pbytes + abytes + xb + yb
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[f"w1a16_decode_7b_layer_b{B}"] = {
            "us_per_layer": round(ms * 1e3, 2), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
            "bytes_per_layer": nbytes, "bound": "hbm", "layer_copies": L, "launches_per_layer": 14}
        log(f"decode 7B layer B={B}: {ms * 1e3:.1f} us/layer, {gbs:.0f} GB/s")
    del layers
    torch.cuda.empty_cache()
    # same layer with the same-input linears concatenated column-wise before
    # packing (q|k|v -> N = 12288, gate|up -> N = 22016): 4 launches per layer
    fshapes = [("qkv", 4096, 12288), ("o", 4096, 4096), ("gate_up", 4096, 22016), ("down", 11008, 4096)]
    F1, FA = build_layer(torch, bgb, syn, cfg["seed"], fshapes, 50, torch.float16)
    flayers = [(F1, FA)] + [([p.clone() for p in F1], FA) for _ in range(L - 1)]
    for B in cfg["batches"]:
        xs = {K: torch.randn((B, K), device="cuda").to(torch.bfloat16) for K in (4096, 11008)}
        ys = {N: torch.empty((B, N), dtype=torch.bfloat16, device="cuda") for _, _, N in fshapes}
        wsz = max(bgb.workspace_bytes(bgb.OP_FBI_LINEAR, B, K, N) for _, K, N in fshapes)
        ws = torch.empty(max(wsz, 256), dtype=torch.uint8, device="cuda")

        def fbody(i, xs=xs, ys=ys, ws=ws):
            Ps, As = flayers[i % L]
            for li, (_, K, N) in enumerate(fshapes):
                bgb.fbi_linear_w1a16(xs[K], Ps[li], As[li], N, y=ys[N], ws=ws)

        ms = graph_time(torch, fbody, steps, 4) / steps
        xb = sum(2 * B * K for _, K, N in fshapes)
        yb = sum(2 * B * N for _, K, N in fshapes)
        nbytes = pbytes + abytes + xb + yb
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[f"w1a16_decode_7b_layer_fused_b{B}"] = {
            "us_per_layer": round(ms * 1e3, 2), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
            "bytes_per_layer": nbytes, "bound": "hbm", "layer_copies": L, "linears": "qkv, o, gate_up, down"}
        log(f"decode 7B layer fused B={B}: {ms * 1e3:.1f} us/layer, {gbs:.0f} GB/s")
        # the 4 linears of the layer as one group: one launch for 1 and 4
        # tokens; at 16 the down projection's tokens do not fit in LDS, and
        # the other three run as one launch, down alone (the linears' inputs
        # are independent synthetic tensors here)
        gys = [torch.empty((B, N), dtype=torch.bfloat16, device="cuda") for _, _, N in fshapes]

        def gbody(i, xs=xs, gys=gys):
            Ps, As = flayers[i % L]
            bgb.fbi_linear_w1a16_group([(xs[K], Ps[li], As[li], N) for li, (_, K, N) in enumerate(fshapes)],
                                       ys=gys)

        ms = graph_time(torch, gbody, steps, 4) / steps
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[f"w1a16_decode_7b_layer_grouped_b{B}"] = {
            "us_per_layer": round(ms * 1e3, 2), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
            "bytes_per_layer": nbytes, "bound": "hbm", "layer_copies": L, "linears": "qkv, o, gate_up, down",
            "launches_per_layer": 1 if B <= 4 else "3 (qkv, o, gate_up as one; down and its reduce pass)"}
        log(f"decode 7B layer grouped B={B}: {ms * 1e3:.1f} us/layer, {gbs:.0f} GB/s")
    del flayers
    return out


def leg_prefill(torch, bgb, syn):
    cfg = syn.CONFIGS["w1_prefill_4096x4096x11008"]
    M, K, N, seed = cfg["M"], cfg["K"], cfg["N"], cfg["seed"]
    W = syn.gpu_normal(seed, 0, (K, N), std=cfg["w_std"])
    x = syn.gpu_normal(seed, 1, (M, K)).to(torch.bfloat16)
    flops = 2 * M * K * N
    out = {}
    P, alpha = bgb.binarize_pack(W, bgb.MODE_FBI)
    y16 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def f16(i):
        bgb.fbi_linear_w1a16(x, P, alpha, N, y=y16)

    ms = graph_time(torch, f16, 10, 3) / 10
    tf = flops / (ms * 1e-3) / 1e12
    out["w1a16_prefill_gemm_4096x4096x11008"] = {"ms": round(ms, 4), "TFLOP/s": round(tf, 1),
                                                 "frac_mfma_bf16": round(tf / BF16_PEAK_TFLOPS, 4),
                                                 "flops": flops, "bound": "mfma"}
    log(f"W1A16 prefill GEMM: {ms * 1e3:.0f} us, {tf:.0f} TFLOP/s")
    Pb, beta, _ = bgb.binarize_pack(W, bgb.MODE_BITNET)
    y32 = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(bgb.workspace_bytes(bgb.OP_BITLINEAR, M, K, N), dtype=torch.uint8, device="cuda")

    def f8(i):
        bgb.bitlinear_w1a8(x, Pb, beta, N, y=y32, ws=ws)

    ms = graph_time(torch, f8, 10, 3) / 10
    bgb.bitlinear_quantize(x, ws=ws)

    def m8(i):
        bgb.bitlinear_matmul(M, K, Pb, beta, N, ws=ws, y=y32)

    ms_mm = graph_time(torch, m8, 10, 3) / 10
    t8 = flops / (ms_mm * 1e-3) / 1e12
    out["w1a8_prefill_gemm_4096x4096x11008"] = {
        "ms_gemm": round(ms_mm, 4), "TOP/s": round(t8, 1), "frac_mfma_int8": round(t8 / INT8_PEAK_TOPS, 4),
        "ms_with_prologue": round(ms, 4), "ops": flops, "bound": "mfma"}
    log(f"W1A8 prefill GEMM: {ms_mm * 1e3:.0f} us ({ms * 1e3:.0f} with prologue), {t8:.0f} TOP/s")
    return out


def leg_ternary(torch, bgb, syn, rotate_mb):
    """BitNet b1.58 ternary weights (two sign planes) at the BitLinear shapes:
    decode of one token through 4096 x 11008 (rotated copies, as the headline)
    and the prefill product at 4096 x 4096 x 11008."""
    cfg = syn.CONFIGS["bitlinear_decode_4096x11008"]
    K, N, seed = cfg["K"], cfg["N"], cfg["seed"]
    W = syn.gpu_normal(seed, 0, (K, N), mean=cfg["w_mean"], std=cfg["w_std"])
    P0, beta, _ = bgb.binarize_pack(W, bgb.MODE_TERNARY)
    pbytes = 2 * bgb.packed_bytes(K, N)
    R = max(2, math.ceil(rotate_mb * 1e6 / pbytes))
    Ps = [P0] + [P0.clone() for _ in range(R - 1)]
    x1 = syn.gpu_normal(seed, 1, (1, K))
    y1 = torch.empty((1, N), dtype=torch.float32, device="cuda")
    ws1 = torch.empty(max(bgb.workspace_bytes(bgb.OP_BITLINEAR158, 1, K, N), 256), dtype=torch.uint8, device="cuda")

    def dec(i):
        bgb.bitlinear158_w1a8(x1, Ps[i % R], beta, N, y=y1, ws=ws1)

    ms = graph_time(torch, dec, 2000, 200) / 2000
    step_bytes = pbytes + K * 4 + N * 4
    gbs = step_bytes / (ms * 1e-3) / 1e9
    out = {"ternary_decode_4096x11008": {"us_per_step": round(ms * 1e3, 3), "GB/s": round(gbs, 1),
                                         "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "bytes": step_bytes,
                                         "weight_copies": R, "bound": "hbm"}}
    log(f"ternary decode 4096x11008: {ms * 1e3:.2f} us/step, {gbs:.0f} GB/s")
    del Ps
    pc = syn.CONFIGS["w1_prefill_4096x4096x11008"]
    M = pc["M"]
    x = syn.gpu_normal(pc["seed"], 1, (M, K)).to(torch.bfloat16)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(bgb.workspace_bytes(bgb.OP_BITLINEAR158, M, K, N), dtype=torch.uint8, device="cuda")
    bgb.bitlinear_quantize(x, ws=ws)

    def mm(i):
        bgb.bitlinear158_matmul(M, K, P0, beta, N, ws=ws, y=y)

    ms_mm = graph_time(torch, mm, 10, 3) / 10
    ops = 2 * M * K * N
    t = ops / (ms_mm * 1e-3) / 1e12
    out["ternary_prefill_gemm_4096x4096x11008"] = {"ms_gemm": round(ms_mm, 4), "TOP/s": round(t, 1),
                                                   "frac_mfma_int8": round(t / INT8_PEAK_TOPS, 4), "ops": ops,
                                                   "mfma_per_weight_bit_plane": 2, "bound": "mfma"}
    log(f"ternary prefill product: {ms_mm * 1e3:.0f} us, {t:.0f} TOP/s")
    return out


def leg_backward(torch, bgb, syn):
    """FBI-linear backward at the prefill shape (4096 tokens, 4096 x 11008): dX, dalpha and dW
    (identity straight-through estimator) from a synthetic output gradient."""
    cfg = syn.CONFIGS["w1_prefill_4096x4096x11008"]
    M, K, N, seed = cfg["M"], cfg["K"], cfg["N"], cfg["seed"]
    W = syn.gpu_normal(seed, 0, (K, N), std=cfg["w_std"])
    x = syn.gpu_normal(seed, 1, (M, K)).to(torch.bfloat16)
    dy = syn.gpu_normal(seed, 5, (M, N)).to(torch.bfloat16)
    P, alpha = bgb.binarize_pack(W, bgb.MODE_FBI)
    del W
    PT = bgb.fbi_pack_transposed(P, K, N)
    ms = graph_time(torch, lambda i: bgb.fbi_pack_transposed(P, K, N, PT=PT), 10, 2) / 10
    out = {"fbi_pack_transposed_4096x11008": {"us": round(ms * 1e3, 2)}}
    ws = torch.empty(bgb.workspace_bytes(bgb.OP_FBI_BACKWARD, M, K, N), dtype=torch.uint8, device="cuda")
    flops = 2 * M * K * N
    for name, want in (("dx", ("dx",)), ("dalpha", ("dalpha",)), ("dw", ("dw",)), ("all", ("dx", "dalpha", "dw"))):
        ms = graph_time(torch, lambda i, want=want: bgb.fbi_linear_w1a16_backward(dy, x, P, PT, alpha, want=want,
                                                                                  ws=ws), 5, 2) / 5
        f = flops * len(want)
        tf = f / (ms * 1e-3) / 1e12
        out[f"fbi_backward_{name}_4096x4096x11008"] = {"ms": round(ms, 4), "TFLOP/s": round(tf, 1),
                                                       "frac_mfma_bf16": round(tf / BF16_PEAK_TFLOPS, 4),
                                                       "flops": f, "bound": "mfma"}
        log(f"FBI backward {name}: {ms * 1e3:.0f} us, {tf:.0f} TFLOP/s")
    return out


def leg_stack_1p3b(torch, bgb, syn, only_grouped=False):
    """only_grouped: just the grouped batch-64 decode step (a focused run for
    kernel traces)."""
    cfg = syn.CONFIGS["w1a16_1p3b_stack"]
    shapes, L = cfg["shapes"], cfg["layers"]
    layers = [] if only_grouped else [build_layer(torch, bgb, syn, cfg["seed"], shapes, l, torch.float16)
                                      for l in range(L)]
    out = {}
    for name, M in (() if only_grouped else
                    (("decode_b64", cfg["decode_batch"]), ("prefill_2x1024", cfg["prefill_tokens"]))):
        xs = {K: torch.randn((M, K), device="cuda").to(torch.bfloat16) for K in (2048, 5632)}
        ys = {N: torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for N in (2048, 5632)}
        wsz = max(bgb.workspace_bytes(bgb.OP_FBI_LINEAR, M, K, N) for _, K, N in shapes)
        ws = torch.empty(max(wsz, 256), dtype=torch.uint8, device="cuda")

        def body(i, xs=xs, ys=ys, ws=ws):
            for Ps, As in layers:
                for li, (_, K, N) in enumerate(shapes):
                    bgb.fbi_linear_w1a16(xs[K], Ps[li], As[li], N, y=ys[N], ws=ws)

        n = 10 if M <= 64 else 3
        # warm: the 154 MB of signs stay in the MALL from step to step (no
        # flush); cold: the MALL is flushed before each timed step
        ms = graph_time(torch, body, n, 2, flush=False) / n
        cold, cmin, cmax = cold_step_ms(torch, body, 5 if M <= 64 else 3)
        flops = 2 * M * sum(K * N for _, K, N in shapes) * L
        tf = flops / (ms * 1e-3) / 1e12
        out[f"w1a16_1p3b_stack_{name}"] = {"ms_per_step": round(ms, 4), "TFLOP/s": round(tf, 1),
                                           "frac_mfma_bf16": round(tf / BF16_PEAK_TFLOPS, 4),
                                           "ms_per_step_cold_mall": round(cold, 4),
                                           "cold_range_ms": [round(cmin, 4), round(cmax, 4)],
                                           "frac_mfma_bf16_cold": round(flops / (cold * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                                           "flops": flops, "linears": L * len(shapes), "bound": "mfma"}
        log(f"1.3B stack {name}: {ms * 1e3:.0f} us/step warm, {cold * 1e3:.0f} cold, {tf:.0f} TFLOP/s")
    del layers
    torch.cuda.empty_cache()
    # the same stack with each layer's same-input linears concatenated column-wise
    # before packing (q|k|v -> N = 6144, gate|up -> N = 11264): 4 launches per layer
    H, F = 2048, 5632
    fshapes = [("qkv", H, 3 * H), ("o", H, H), ("gate_up", H, 2 * F), ("down", F, H)]
    flayers = [build_layer(torch, bgb, syn, cfg["seed"], fshapes, 50 + l, torch.float16) for l in range(L)]
    for name, M in ((("decode_b64", cfg["decode_batch"]),) if only_grouped else
                    (("decode_b64", cfg["decode_batch"]), ("prefill_2x1024", cfg["prefill_tokens"]))):
        xs = {K: torch.randn((M, K), device="cuda").to(torch.bfloat16) for K in (H, F)}
        ys = {N: torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for _, _, N in fshapes}
        wsz = max(bgb.workspace_bytes(bgb.OP_FBI_LINEAR, M, K, N) for _, K, N in fshapes)
        ws = torch.empty(max(wsz, 256), dtype=torch.uint8, device="cuda")

        def fbody(i, xs=xs, ys=ys, ws=ws):
            for Ps, As in flayers:
                for li, (_, K, N) in enumerate(fshapes):
                    bgb.fbi_linear_w1a16(xs[K], Ps[li], As[li], N, y=ys[N], ws=ws)

        n = 10 if M <= 64 else 3
        flops = 2 * M * sum(K * N for _, K, N in fshapes) * L
        if not only_grouped:
            ms = graph_time(torch, fbody, n, 2, flush=False) / n
            cold, cmin, cmax = cold_step_ms(torch, fbody, 5 if M <= 64 else 3)
            tf = flops / (ms * 1e-3) / 1e12
            out[f"w1a16_1p3b_stack_fused_{name}"] = {
                "ms_per_step": round(ms, 4), "TFLOP/s": round(tf, 1), "frac_mfma_bf16": round(tf / BF16_PEAK_TFLOPS, 4),
                "ms_per_step_cold_mall": round(cold, 4), "cold_range_ms": [round(cmin, 4), round(cmax, 4)],
                "frac_mfma_bf16_cold": round(flops / (cold * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4), "flops": flops,
                "linears": L * len(fshapes), "bound": "mfma"}
            log(f"1.3B stack fused {name}: {ms * 1e3:.0f} us/step warm, {cold * 1e3:.0f} cold, {tf:.0f} TFLOP/s")
        if M > 64:
            continue
        # the layer's four fused linears as one group call: one launch per
        # layer (the linears' inputs are independent synthetic tensors here)
        gys = [torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for _, _, N in fshapes]
        glin0 = [(xs[K], flayers[0][0][li], flayers[0][1][li], N) for li, (_, K, N) in enumerate(fshapes)]
        gws = torch.empty(max(bgb.group_workspace_bytes([(x, P, a, y) for (x, P, a, _), y in zip(glin0, gys)], M),
                              256), dtype=torch.uint8, device="cuda")

        def gbody(i, xs=xs, gys=gys, gws=gws):
            for Ps, As in flayers:
                bgb.fbi_linear_w1a16_group([(xs[K], Ps[li], As[li], N) for li, (_, K, N) in enumerate(fshapes)],
                                           ys=gys, ws=gws)

        ms = graph_time(torch, gbody, n, 2, flush=False) / n
        cold, cmin, cmax = cold_step_ms(torch, gbody, 5)
        tf = flops / (ms * 1e-3) / 1e12
        out[f"w1a16_1p3b_stack_grouped_{name}"] = {
            "ms_per_step": round(ms, 4), "TFLOP/s": round(tf, 1), "frac_mfma_bf16": round(tf / BF16_PEAK_TFLOPS, 4),
            "ms_per_step_cold_mall": round(cold, 4), "cold_range_ms": [round(cmin, 4), round(cmax, 4)],
            "frac_mfma_bf16_cold": round(flops / (cold * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4), "flops": flops,
            "launches": L * (2 if gws.numel() > 256 else 1),
            "linears": "qkv, o, gate_up, down as one group per layer (GEMM + reduce of the K parts)", "bound": "mfma"}
        log(f"1.3B stack grouped {name}: {ms * 1e3:.0f} us/step warm, {cold * 1e3:.0f} cold, {tf:.0f} TFLOP/s")
    del flayers
    return out


def leg_ceilings(torch):
    """Ceilings measured on this GPU (include/bgb_ceilings.h): streaming-read
    bandwidth per launch size (each launch reads a window of a 2 GiB buffer
    that no recent launch has read), the empty-kernel launch cost, and the
    sustained dense MFMA rates on random operand values (bf16 16x16x32, int8
    16x16x64), each a HIP graph of back-to-back launches."""
    import ctypes
    path = os.path.join(ROOT, "bit_gemm_binarize_amd", "ceilings", "libbgb_ceilings.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built (python -m bit_gemm_binarize_amd.build)")
    lib = ctypes.CDLL(path)
    V, SZ, I = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.ceil_stream_read.argtypes = [V, SZ, I, V, V]
    lib.ceil_empty.argtypes = [I, I, V]
    lib.ceil_mfma_bf16.argtypes = [V, I, I, V, V]
    lib.ceil_mfma_i8.argtypes = [V, I, I, V, V]
    for f in (lib.ceil_stream_read, lib.ceil_empty, lib.ceil_mfma_bf16, lib.ceil_mfma_i8):
        f.restype = I

    def ok(rc):
        if rc != 0:
            raise RuntimeError(f"ceiling kernel failed: {rc} (hip {lib.ceil_last_hip_error()})")

    st = lambda: torch.cuda.current_stream().cuda_stream
    out = {}
    big = torch.empty((2 << 30) // 4, dtype=torch.int32, device="cuda").random_()
    blocks = 2048
    sink = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
    for label, nbytes in (("2MB", 2 << 20), ("5.6MB", 5636096), ("25MB", 25296896), ("800MB", 800 << 20)):
        nbytes -= nbytes % 16
        windows = max(1, (2 << 30) // nbytes)
        n = min(400, max(4, windows * 2))

        def body(i, nbytes=nbytes, windows=windows):
            ok(lib.ceil_stream_read(big.data_ptr() + (i % windows) * nbytes, nbytes, blocks, sink.data_ptr(), st()))

        ms = graph_time(torch, body, n, 2) / n
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[f"stream_read_{label}"] = {"us_per_launch": round(ms * 1e3, 3), "GB/s": round(gbs, 1),
                                       "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "bytes": nbytes}
        log(f"ceiling stream read {label}: {ms * 1e3:.2f} us/launch, {gbs:.0f} GB/s")
    del big
    ms = graph_time(torch, lambda i: ok(lib.ceil_empty(256, 512, st())), 2000, 20, flush=False) / 2000
    out["empty_kernel_256x512"] = {"us_per_launch": round(ms * 1e3, 3)}
    log(f"ceiling empty kernel: {ms * 1e3:.2f} us/launch")
    # operands: N(0,1) bf16 values (finite, every mantissa bit toggling) and
    # uniform int8 values, 8192 x 16 bytes each
    rnd_bf16 = torch.randn(8192 * 8, device="cuda").to(torch.bfloat16)
    rnd_i8 = torch.randint(-128, 128, (8192 * 16,), dtype=torch.int8, device="cuda")
    fsink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    for name, fn, opd, per, peak in (("mfma_bf16_16x16x32", lib.ceil_mfma_bf16, rnd_bf16, 16384, BF16_PEAK_TFLOPS),
                                     ("mfma_i8_16x16x64", lib.ceil_mfma_i8, rnd_i8, 32768, INT8_PEAK_TOPS)):
        iters = 2000
        n = 20

        def body(i, fn=fn, opd=opd, iters=iters):
            ok(fn(opd.data_ptr(), blocks, iters, fsink.data_ptr(), st()))

        ms = graph_time(torch, body, n, 2, flush=False) / n
        work = blocks * 4 * iters * 8 * per
        rate = work / (ms * 1e-3) / 1e12
        out[name] = {"T_per_s": round(rate, 1), "frac_peak": round(rate / peak, 4), "ms_per_launch": round(ms, 4),
                     "operands": "random values, fixed per lane"}
        log(f"ceiling {name}: {rate:.0f} T/s ({rate / peak:.2f} of peak)")
    return {"ceilings": out}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported (this build has no "
              f"multi-GPU path; see DESIGN.md for how the layer would shard).", file=sys.stderr)
        sys.exit(2)
    # the CPU oracle first, before anything touches the GPU: its all-core leg
    # forks worker processes, which must not inherit a HIP context
    cpu = None
    if not args.no_cpu_baseline and args.calib_copy_mb <= 0:
        import bgb_synth as syn
        workers = args.cpu_workers or min(16, os.cpu_count() or 1)
        cpu = cpu_baseline(headline_host_state(syn), args.cpu_seconds, workers)

    import torch

    if args.calib_copy_mb > 0:
        n = int(args.calib_copy_mb * 1e6) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"copy calibration: 5 copies of {n * 4} bytes")
        return

    import bgb_synth as syn
    import bit_gemm_binarize_amd as bgb
    bgb.load()
    torch.cuda.set_device(0)
    torch.backends.cuda.matmul.allow_tf32 = False

    ms_step, value, roof, R, state = headline(torch, bgb, syn, args)

    legs = {}
    want = set() if args.legs == "none" else (
        {"fbi768", "pack", "decode7b", "prefill", "stack", "ternary", "backward", "ceilings"} if args.legs == "all"
        else set(args.legs.split(",")))
    if args.ceilings:
        want.add("ceilings")
    if "fbi768" in want:
        legs.update(leg_fbi_768(torch, bgb, syn))
    if "pack" in want:
        legs.update(leg_pack(torch, bgb, syn))
        torch.cuda.empty_cache()
    if "decode7b" in want:
        legs.update(leg_decode_7b(torch, bgb, syn, 64))
        torch.cuda.empty_cache()
    if "prefill" in want:
        legs.update(leg_prefill(torch, bgb, syn))
        torch.cuda.empty_cache()
    if "stack" in want:
        legs.update(leg_stack_1p3b(torch, bgb, syn))
    elif "stack_grouped" in want:
        legs.update(leg_stack_1p3b(torch, bgb, syn, only_grouped=True))
    if "ternary" in want:
        legs.update(leg_ternary(torch, bgb, syn, args.rotate_mb))
        torch.cuda.empty_cache()
    if "backward" in want:
        legs.update(leg_backward(torch, bgb, syn))
        torch.cuda.empty_cache()
    if "ceilings" in want:
        legs.update(leg_ceilings(torch))
        torch.cuda.empty_cache()


    rec = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8",
        "data": "synthetic: seeded N(0.001, 0.02) fp32 weights packed to 1 bit, N(0,1) fp32 activations",
        "config": {"workload": "bitlinear_w1a8_decode_4096x11008", "M": state["M"], "K": state["K"],
                   "N": state["N"], "x_dtype": "f32", "weight_copies": R,
                   "distinct_weight_bytes_timed": state["distinct_bytes"], "mall_flush_bytes": MALL_FLUSH_BYTES,
                   "step": "one fused kernel: LN + absmax quant prologue, packed GEMV, epilogue (HIP graph of all steps)"},
        "roofline": roof, "cpu_baseline": cpu, "legs": legs,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
