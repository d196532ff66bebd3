"""Benchmark of the TurboQuant hot path on one MI355X.

Default workload (`--workload serving`, one "step" = one pass of the whole hot
path over one batch): batched serving step with 64 sequences x 8192-token
context, 8 KV heads, 32 query heads, head_dim 128, bf16 K/V; prefill quantize
of all 64 x 8 x 8192 K and V vectors (keys b=4: 3-bit Lloyd-Max + 1-bit QJL;
values 3-bit), then 128 decode steps, each appending one quantized token per
sequence and running decode attention over the packed cache.

Prints ONE JSON line. For the serving step `value` = attention-score keys/s of
the whole step (KV-head tokens scored by decode attention divided by the step
time, prefill included). Inputs are resident in HBM before the timed region.

Other workloads (`--workload gqa|single|search|tiny`) measure the other
shapes with the same reporting; `--workload prefill` measures chunked prefill
(quantize each chunk into the cache, then causal attention of its query
positions over the cache); `--workload logits` times the attention logits alone
over the serving cache against fp32 and bf16 keys scored by a library GEMM.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "attention-score keys/s over packed KV (% HBM peak); quantize vectors/s"
HBM_PEAK_GBS = 8000.0
FP32_PEAK_TFLOPS = 157.3
VAL_B3 = 52   # 3-bit value record at d=128 (48 code + 4 norm bytes; 50 with fp16 norms)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", choices=["serving", "gqa", "single", "search", "tiny", "prefill", "polar", "logits"],
                    default="serving")
    ap.add_argument("--data", choices=["outlier", "gaussian"], default="outlier")
    ap.add_argument("--kbits", type=int, default=3, help="MSE bits of the keys (b = kbits + 1)")
    ap.add_argument("--key-format", choices=["turboquant", "mse", "qjl"], default="turboquant",
                    help="keys: TurboQuant (codes + QJL signs), MSE-only (codes), or pure QJL (signs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--separate-append", action="store_true",
                    help="serving step: tq_append_token then tq_attention_decode instead of tq_decode_step")
    ap.add_argument("--norms", choices=["f32", "f16"], default="f32",
                    help="decode workloads: record norms as fp32, or fp16 (compact records)")
    ap.add_argument("--page-tokens", type=int, default=0,
                    help="decode workloads: paged cache with pages of this many tokens (a multiple of 256) in a "
                         "shuffled pool, instead of the contiguous layout")
    ap.add_argument("--graph", action="store_true",
                    help="decode workloads: also capture one whole step in a HIP graph (torch.cuda.graph) and "
                         "time its replays (graph_ms_per_step)")
    ap.add_argument("--no-gaussian-pass", action="store_true",
                    help="serving / gqa with outlier data: skip the second pass on Gaussian data (reported "
                         "under \"gaussian\" in the same JSON line)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run 5 device-to-device copies of this many MiB (a plain copy kernel of known size, "
                         "the calibration of the rocprofv3 FETCH_SIZE / WRITE_SIZE counters) and exit")
    return ap.parse_args()


def copy_probe(torch, mib):
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4, "copies": 5}), flush=True)


def threads_used():
    try:
        n = int(os.environ.get("OMP_NUM_THREADS", "0"))
        return n or len(os.sched_getaffinity(0))
    except Exception:
        return os.cpu_count()


def cpu_info():
    """The host CPU model and the BLAS thread count the oracle's numpy runs with."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        import threadpoolctl
        pools = [p for p in threadpoolctl.threadpool_info() if p.get("user_api") == "blas"]
        if pools:
            blas = {"library": pools[0].get("internal_api"), "threads": pools[0].get("num_threads")}
    except Exception:
        pass
    return {"cpu_model": model, "blas": blas, "affinity_cpus": len(os.sched_getaffinity(0))}


class Timer:
    """HIP-event timing on torch's current stream (the stream every tq_* call runs on)."""

    def __init__(self, torch):
        self.torch = torch
        self.stream = torch.cuda.current_stream()

    def __call__(self, fn):
        t = self.torch
        e0, e1 = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        fn()
        e1.record(self.stream)
        return (e0, e1)


def ms(ev):
    return ev[0].elapsed_time(ev[1])


KERNEL_SOURCE = os.path.join(ROOT, "kv_cache_vector_turboquant_amd", "csrc", "tq_kernels.hip")


def cold_cache_decode(torch, tq, ctx, K, V, q, B, H, Hq, L, cap, kbits, vbits, kqjl, mib=600):
    """Decode with a cold cache: the same records prefilled into enough distinct
    caches to exceed the 256 MB Infinity Cache twice over, decoded round-robin.
    Returns (caches, mean decode_kernel ms, mean call ms)."""
    d = K.shape[-1]
    per = cap * B * H * (tq.Packed(32, d, kbits, True, qjl=kqjl).words[0].numel() * 4 + 8 + d * vbits // 8 + 4)
    n = max(2, -(-mib * 1024 * 1024 // per))
    caches = []
    kwork = torch.empty(tq.quantize_ws_bytes(ctx, B * H, L, True), dtype=torch.uint8, device="cuda")
    for _ in range(n):
        c = tq.KVCache(B, H, cap, d, kbits, vbits, key_qjl=kqjl)
        tq.quantize_kv(ctx, K.view(B * H, L, d), c.k, out_stream_stride=cap, work=kwork)
        tq.quantize_kv(ctx, V.view(B * H, L, d), c.v, out_stream_stride=cap)
        c.seq_len.fill_(L)
        c.host_max_len = L
        caches.append(c)
    ws = torch.empty(caches[0].decode_ws_bytes(ctx, Hq), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    for c in caches[:2]:
        c.decode(ctx, q, out=out, ws=ws)
    reps = 2 * n
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for pair in kev:
        for e in pair:
            e.record()
    torch.cuda.synchronize()
    for i in range(reps):
        tq.time_next_decode(*kev[i])
        cev[i][0].record()
        caches[i % n].decode(ctx, q, out=out, ws=ws)
        cev[i][1].record()
    torch.cuda.synchronize()
    kms = sum(a.elapsed_time(b) for a, b in kev) / reps
    cms = sum(a.elapsed_time(b) for a, b in cev) / reps
    del caches
    return n, kms, cms


def read_ceiling(torch, tq, mib=2048, grid=8192, reps=10):
    """Practical HBM read ceiling on this GPU, measured live: the library's
    read-bandwidth probe streaming `mib` MiB (GB/s, best grid of a small sweep)."""
    src = torch.empty(mib * 1024 * 1024, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    best = 0.0
    for g in (4096, grid, 16384):
        sink = torch.empty(g * 256, dtype=torch.int32, device="cuda")
        for _ in range(2):
            tq.read_probe(src, g, sink)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            tq.read_probe(src, g, sink)
        e1.record()
        torch.cuda.synchronize()
        best = max(best, src.numel() / (e0.elapsed_time(e1) / reps / 1e3) / 1e9)
    del src
    return best


def measured_traffic(tag):
    """HBM bytes per launch of a kernel from its committed counter summary
    (profiles/<tag>_traffic.md: FETCH_SIZE and WRITE_SIZE per dispatch, scaled
    by the copy-kernel calibration), or None when there is none or the kernel
    source has changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{tag}_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and line.startswith("- "):
                k, v = line[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    with open(KERNEL_SOURCE, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    if fields.get("kernel_source_sha256") != sha or "traffic_bytes_per_launch" not in fields:
        return None
    return float(fields["traffic_bytes_per_launch"])


# ---------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on a bounded sample of the workload
# ---------------------------------------------------------------------------

def key_format(args):
    """(MSE bits B, QJL flag, text) of the keys the run uses."""
    if args.key_format == "mse":
        return args.kbits, False, f"MSE-only keys {args.kbits}-bit"
    if args.key_format == "qjl":
        return 0, True, "pure QJL keys (1 sign bit)"
    return args.kbits, True, f"keys b={args.kbits + 1}"


def key_record_bytes(d, B, qjl, norm_f16=False):
    return (d // 32) * (B + int(qjl)) * 4 + (2 if norm_f16 else 4) * (1 + int(qjl))


def oracle_stream_rates(d, L, group, kbits, vbits, seconds, data, kqjl=True):
    """Encode L K + L V vectors of whole streams and run their decode for
    `group` query heads, until `seconds` of CPU work; returns rates."""
    import synth
    from oracle import turboquant as T
    Pi = T.rotation_from_gaussian(synth.gaussian_matrix(0, synth.TAG_ROTATION, d, d))
    S = T.sketch_from_gaussian(synth.gaussian_matrix(0, synth.TAG_SKETCH, d, d))
    cbk = T.codebook(d, kbits) if kbits > 0 else None
    cbv = T.codebook(d, vbits)
    t_enc = t_dec = 0.0
    n_enc = n_dec = streams = 0
    t_start = time.perf_counter()
    while time.perf_counter() - t_start < seconds or streams == 0:
        if data == "outlier":
            K = synth.outlier_kv(0, (streams, 91), synth.TAG_SCALES_K, (L, d))
            V = synth.outlier_kv(0, (streams, 92), synth.TAG_SCALES_V, (L, d))
        else:
            K = synth.gaussian(0, (streams, 91), (L, d), "bf16")
            V = synth.gaussian(0, (streams, 92), (L, d), "bf16")
        Q = synth.outlier_kv(0, (streams, 93), synth.TAG_SCALES_K, (group, d))
        t0 = time.perf_counter()
        keys = T.pack_keys(T.encode(K, Pi, cbk, S if kqjl else None), kbits, kqjl)
        vals = T.pack_values(T.encode(V, Pi, cbv), vbits)
        t1 = time.perf_counter()
        T.attention_decode(Q, Pi, S, cbk, cbv, keys, vals, L, 1 / math.sqrt(d), kqjl)
        t2 = time.perf_counter()
        t_enc += t1 - t0
        t_dec += t2 - t1
        n_enc += 2 * L
        n_dec += L
        streams += 1
    return n_enc / t_enc, n_dec / t_dec, streams, t_enc + t_dec


# ---------------------------------------------------------------------------
# Workloads
# ---------------------------------------------------------------------------

def kv_inputs(torch, synth, args, shape, tags, scale_tag):
    if args.data == "outlier":
        return synth.torch_outlier_kv(0, tags, scale_tag, shape, torch.bfloat16, "cuda")
    return synth.torch_gaussian(0, tags, shape, torch.bfloat16, "cuda")


def decode_spans(B, H, Hq, cap, page_tokens):
    """Whether the decode launch takes the kernel whose chunks span several pages.

    The library picks the chunk per launch: 1024 tokens, halved (not below 256)
    while the launch would have fewer than 2048 work-groups, then, for a paged
    cache, halved until it and the page size divide one another; chunks longer
    than a page span several pages. This only labels the bench line.
    """
    if not page_tokens:
        return False
    streams = B * H * ((Hq // H + 3) // 4)
    chunk = 1024
    while chunk > 256 and streams * ((cap + chunk - 1) // chunk) < 2048:
        chunk >>= 1
    while page_tokens % chunk and chunk % page_tokens:
        chunk >>= 1
    return chunk > page_tokens


def run_decode_workload(args, torch, tq, synth, B, H, Hq, L, NS, name, cfg_text):
    """Prefill quantize of B x H x L K/V, then NS x (append + decode)."""
    d, vbits = 128, 3
    kbits, kqjl, _ = key_format(args)
    nf16 = args.norms == "f16"
    cap = ((L + NS + 31) // 32) * 32
    ctx = tq.Context(d, 0)
    K = kv_inputs(torch, synth, args, (B, H, L, d), (3, synth.TAG_KEYS), synth.TAG_SCALES_K)
    V = kv_inputs(torch, synth, args, (B, H, L, d), (3, synth.TAG_VALUES), synth.TAG_SCALES_V)
    KA = kv_inputs(torch, synth, args, (max(NS, 1), B, H, d), (3, synth.TAG_APPEND_K), synth.TAG_SCALES_K)
    VA = kv_inputs(torch, synth, args, (max(NS, 1), B, H, d), (3, synth.TAG_APPEND_V), synth.TAG_SCALES_V)
    QS = kv_inputs(torch, synth, args, (max(NS, 1), B, Hq, d), (3, synth.TAG_QUERIES), synth.TAG_SCALES_K)
    if args.page_tokens:
        # paged cache: whole pages per sequence, handed out in a shuffled order
        Pt = args.page_tokens
        cap = ((L + NS + Pt - 1) // Pt) * Pt
        cols = cap // Pt
        g = torch.Generator(device="cpu")
        g.manual_seed(7)
        perm = torch.randperm(B * cols + 8, generator=g)[:B * cols].to(torch.int32).view(B, cols).to("cuda")
        cache = tq.KVCache(B, H, cap, d, kbits, vbits, key_qjl=kqjl, page_tokens=Pt, n_pages=B * cols + 8,
                           block_table=perm, norm_f16=nf16)
    else:
        cache = tq.KVCache(B, H, cap, d, kbits, vbits, key_qjl=kqjl, norm_f16=nf16)
    kwork = torch.empty(tq.quantize_ws_bytes(ctx, B * H, L, True), dtype=torch.uint8, device="cuda")
    cache.host_max_len = cap
    fused = NS > 0 and not args.separate_append
    dws = torch.empty(max(cache.decode_ws_bytes(ctx, Hq), cache.decode_step_ws_bytes(ctx, Hq)), dtype=torch.uint8,
                      device="cuda")
    cache.host_max_len = 0
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    timer = Timer(torch)
    n_dec = max(NS, 1)

    def prefill():
        cache.prefill(ctx, K, V, work=kwork)  # tq_cache_write: keys and values of every stream

    dec_events = []
    kev = []  # per timed call: events around its score/attention kernel

    def step(record):
        prefill()
        for i in range(n_dec):
            n = L + (i + 1 if NS > 0 else 0)
            if fused:
                # one serving step: append the new K/V token and decode with it (tq_decode_step)
                call = lambda: cache.decode_step(ctx, KA[i], VA[i], QS[i], out=out, ws=dws)  # noqa: E731
            else:
                if NS > 0:
                    cache.append(ctx, KA[i], VA[i])
                call = lambda: cache.decode(ctx, QS[i], out=out, ws=dws)  # noqa: E731
            if record:
                k_ev = kev[len(dec_events)]
                tq.time_next_decode(*k_ev)
                dec_events.append((timer(call), k_ev, n))
            else:
                call()

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    pre_ev = timer(prefill)
    torch.cuda.synchronize()
    prefill_ms = ms(pre_ev)
    # timed region: K whole steps, events only around them (an event recorded
    # between the launches of a call would stall the launches behind it)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    whole = timer(lambda: [step(False) for _ in range(args.steps)])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = ms(whole) / args.steps
    # launch timing, right after: one more identical step with events around
    # each call and around each call's decode_kernel (created beforehand)
    for _ in range(n_dec):
        pair = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        for e in pair:
            e.record()
        kev.append(pair)
    torch.cuda.synchronize()
    step(True)
    torch.cuda.synchronize()
    graph = None
    if args.graph:
        # the whole step captured once; replays start from the captured host state
        eager_out = out.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(False)
        torch.cuda.synchronize()
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        same = bool(torch.equal(out, eager_out))
        gw = timer(lambda: [g.replay() for _ in range(args.steps)])
        torch.cuda.synchronize()
        graph = {"graph_ms_per_step": ms(gw) / args.steps, "graph_replay_matches_eager": same}
    keys_per_step = sum(B * H * (L + (i + 1 if NS > 0 else 0)) for i in range(n_dec))
    rec_bytes = key_record_bytes(d, kbits, kqjl, nf16) + VAL_B3 - (2 if nf16 else 0)
    dec_ms = np.array([ms(e) for e, _, _ in dec_events])
    kern_ms = np.array([ms(k) for _, k, _ in dec_events])
    dec_bytes = np.array([B * H * n * rec_bytes for _, _, n in dec_events], dtype=np.float64)
    avg_ms = float(dec_ms.mean())
    kern_avg_ms = float(kern_ms.mean())
    achieved = float(dec_bytes.mean()) / (kern_avg_ms / 1e3) / 1e9
    fmt_tag = "" if (args.key_format == "turboquant" and args.kbits == 3) else f"_{args.key_format}{kbits}"
    fmt_tag += ("_f16norms" if nf16 else "") + (f"_paged{args.page_tokens}" if args.page_tokens else "")
    traffic = measured_traffic(f"decode_kernel_{name}{fmt_tag}")
    cold = cold_cache_decode(torch, tq, ctx, K, V, QS[0], B, H, Hq, L, cap, kbits, vbits, kqjl) \
        if name == "single" else None
    ceiling = read_ceiling(torch, tq)
    vectors = 2 * B * H * L
    if cold is not None:
        rec_total = B * H * L * rec_bytes
        extra_cold = {"cold_cache": {
            "caches": cold[0], "bytes_per_cache": rec_total, "decode_kernel_us": cold[1] * 1e3,
            "gbs": rec_total / (cold[1] / 1e3) / 1e9, "decode_call_us": cold[2] * 1e3,
            "note": ("decode rotated over distinct caches totalling more than twice the 256 MB Infinity Cache, so "
                     "every launch reads its records from HBM")}}
    else:
        extra_cold = {}
    res = {
        "metric": METRIC, "value": keys_per_step / (ms_per_step / 1e3), "unit": "keys/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32+fp6/fp4/i8 exact-digit MFMA",
        "data": ("synthetic (outlier-channel bf16 K/V, seeded)" if args.data == "outlier" else "synthetic (i.i.d. N(0,1) bf16 K/V, seeded)"),
        "config": {"workload": cfg_text, "batch": B, "context": L, "decode_steps": NS, "kv_heads": H,
                   "q_heads": Hq, "head_dim": d, "key_bits": kbits + int(kqjl), "key_format": args.key_format,
                   "value_bits": vbits, "norms": args.norms, "cache_layout": (f"paged, {args.page_tokens}-token pages in a shuffled pool"
                                                         if args.page_tokens else "contiguous"),
                   "parallelism": "none (1 GPU)"},
        "quantize_vectors_per_s": vectors / (prefill_ms / 1e3), "prefill_ms": prefill_ms,
        "decode_keys_per_s": float(B * H * sum(n for _, _, n in dec_events) / (dec_ms.sum() / 1e3)),
        "decode_call_ms": avg_ms, "wall_s_timed": wall, **extra_cold, **(graph or {}),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": (f"decode_kernel<{kbits}, {vbits}, {str(kqjl).lower()}, "
                                f"{str(decode_spans(B, H, Hq, cap, args.page_tokens)).lower()}, {str(nf16).lower()}> "
                                "(score/attention over the packed cache; template arguments: key MSE bits, value bits, "
                                "QJL signs, chunks spanning several pages, fp16 norms)"),
                     "algorithmic_bytes_per_launch": float(dec_bytes.mean()), "avg_launch_ms": kern_avg_ms,
                     "bytes_per_kv_token": rec_bytes,
                     "call": ("tq_decode_step: decode_prep_kernel (query prep + append), decode_kernel, "
                              "decode_merge_kernel" if fused else
                              "tq_attention_decode: decode_prep_kernel, decode_kernel, decode_merge_kernel"),
                     "call_ms": avg_ms, "call_gbs": float(dec_bytes.mean()) / (avg_ms / 1e3) / 1e9,
                     "timing": ("HIP events on the launch stream around every decode_kernel launch of one "
                                "step run right after the timed steps, same inputs and launch configuration"),
                     "read_ceiling_gbs": ceiling, "frac_of_read_ceiling": achieved / ceiling,
                     "read_ceiling": ("tq_read_probe: best of grids 4096/8192/16384 x 256 threads streaming 2 GiB "
                                      "(a contiguous slice per work-group, 16-byte non-temporal loads), "
                                      "timed live in this run")},
    }
    if not args.no_cpu_baseline:
        enc_rate, dec_rate, streams, secs = oracle_stream_rates(d, min(L, 8192), Hq // H, kbits, vbits,
                                                               args.cpu_seconds, args.data, kqjl)
        step_s = vectors / enc_rate + keys_per_step / dec_rate
        res["cpu_baseline"] = {
            "value": keys_per_step / step_s, "unit": "keys/s", "cores": threads_used(), "kind": "oracle", **cpu_info(),
            "sample": f"{streams} whole (sequence, KV head) streams of {min(L, 8192)} tokens: oracle encode of "
                      f"their K and V vectors and decode for {Hq // H} query heads, {secs:.1f} s of CPU work; "
                      f"extrapolated to the step at {enc_rate:.0f} vectors/s and {dec_rate:.0f} keys/s",
            "quantize_vectors_per_s": enc_rate, "decode_keys_per_s": dec_rate}
    return res


def oracle_prefill_rate(d, L, nq, group, kbits, vbits, seconds, data, kqjl=True):
    """Oracle causal attention of chunks of nq query positions x `group` heads
    over streams of L packed tokens (records encoded beforehand, untimed), until
    `seconds` of CPU work; returns (query position, KV-head token) pairs/s."""
    import synth
    from oracle import turboquant as T
    Pi = T.rotation_from_gaussian(synth.gaussian_matrix(0, synth.TAG_ROTATION, d, d))
    S = T.sketch_from_gaussian(synth.gaussian_matrix(0, synth.TAG_SKETCH, d, d))
    cbk = T.codebook(d, kbits) if kbits > 0 else None
    cbv = T.codebook(d, vbits)
    gen = (lambda t, sc: synth.outlier_kv(0, t, sc, (L, d))) if data == "outlier" else \
        (lambda t, sc: synth.gaussian(0, t, (L, d), "bf16"))
    K, V = gen((0, 94), synth.TAG_SCALES_K), gen((0, 95), synth.TAG_SCALES_V)
    keys = T.pack_keys(T.encode(K, Pi, cbk, S if kqjl else None), kbits, kqjl)
    vals = T.pack_values(T.encode(V, Pi, cbv), vbits)
    t = 0.0
    pairs = chunks = 0
    while t < seconds or chunks == 0:
        Q = synth.gaussian(0, (chunks, 96), (nq, group, d), "bf16")
        t0 = time.perf_counter()
        T.attention_prefill(Q, Pi, S, cbk, cbv, keys, vals, L, 1 / math.sqrt(d), True, kqjl)
        t += time.perf_counter() - t0
        pairs += sum(L - nq + i + 1 for i in range(nq))
        chunks += 1
    return pairs / t, chunks, t


def run_prefill(args, torch, tq, synth):
    """Chunked prefill: the prompt's K/V are quantized into the cache chunk by
    chunk, and each chunk's query positions attend causally over the cache."""
    B, H, Hq, P, C, d, vbits = 1, 8, 32, 16384, 1024, 128, 3
    kbits, kqjl, ktext = key_format(args)
    nch = P // C
    ctx = tq.Context(d, 0)
    K = kv_inputs(torch, synth, args, (nch, B, H, C, d), (4, synth.TAG_KEYS), synth.TAG_SCALES_K)
    V = kv_inputs(torch, synth, args, (nch, B, H, C, d), (4, synth.TAG_VALUES), synth.TAG_SCALES_V)
    Q = synth.torch_gaussian(0, (4, synth.TAG_QUERIES), (nch, B, C, Hq, d), torch.bfloat16, "cuda")
    cache = tq.KVCache(B, H, P, d, kbits, vbits, key_qjl=kqjl)
    cache.host_max_len = P
    ws = torch.empty(cache.prefill_ws_bytes(ctx, C, Hq), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, C, Hq, d), dtype=torch.float32, device="cuda")
    timer = Timer(torch)
    kev = []

    def step(record):
        cache.seq_len.zero_()
        cache.host_max_len = 0
        for j in range(nch):
            cache.extend(ctx, K[j], V[j])
            if record:
                tq.time_next_decode(*kev[j][1])
                kev[j] = (timer(lambda: cache.attend(ctx, Q[j], True, out=out, ws=ws)), kev[j][1])
            else:
                cache.attend(ctx, Q[j], True, out=out, ws=ws)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    whole = timer(lambda: [step(False) for _ in range(args.steps)])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = ms(whole) / args.steps
    for _ in range(nch):
        pair = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        for e in pair:
            e.record()
        kev.append((None, pair))
    torch.cuda.synchronize()
    step(True)
    torch.cuda.synchronize()
    # (query position, KV-head token) pairs: position i of chunk j sees j*C + i + 1 tokens
    pairs_chunk = [B * H * sum(j * C + i + 1 for i in range(C)) for j in range(nch)]
    call_ms = np.array([ms(c) for c, _ in kev])
    kern_ms = np.array([ms(k) for _, k in kev])
    # MFMA work of prefill_kernel (16 virtual heads per work-group): per 16 tokens
    # x 16 heads, (Walsh masks + sign mask) x 6 query digits of 16x16x128 fp6 x fp4
    # MFMAs; per 512 tokens x 16 heads, 4 waves x 2 coordinate halves x 4 groups x
    # value masks x 4 weight digits x 2 (token halves) 16x16x64 int8 MFMAs
    km = (1 << (kbits - 1)) if kbits > 0 else 0
    vm = 1 << (vbits - 1)
    k_ops = (km + int(kqjl)) * 6 * 16 * 16 * 128 * 2 / (16 * 16)        # per (virtual head, token)
    v_ops = 4 * 2 * 4 * vm * 4 * 2 * 16 * 16 * 64 * 2 / (512 * 16)
    vheads = Hq // H
    vh_tokens = np.array([p * vheads for p in pairs_chunk], dtype=np.float64)
    tput = vh_tokens * (k_ops + v_ops) / (kern_ms / 1e3) / 1e12
    # the peak of this mix: fp6 x fp4 MFMAs at 10.1 PFLOP/s, int8 MFMAs at 5.0 POP/s
    mix_peak = (k_ops + v_ops) / (k_ops / 10100.0 + v_ops / 5000.0)
    # the method's own arithmetic: a d-term dot product per score and a d-term
    # weighted sum per value, at fp32 accuracy
    alg = vh_tokens * 4 * d / (kern_ms / 1e3) / 1e12
    res = {
        "metric": METRIC, "value": sum(pairs_chunk) / (ms_per_step / 1e3), "unit": "keys/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32+fp6/fp4/i8 exact-digit MFMA",
        "data": f"synthetic ({args.data}-channel bf16 K/V, Gaussian bf16 queries, seeded)",
        "config": {"workload": (f"chunked_prefill: batch {B} x {P}-token prompt in {C}-token chunks, {H} KV heads, "
                                f"{Hq} q heads, d={d}, {ktext}, values 3-bit; per chunk quantize its K/V into the "
                                f"cache, then causal attention of its {C} query positions over the cache"),
                   "batch": B, "prompt": P, "chunk": C, "kv_heads": H, "q_heads": Hq, "head_dim": d,
                   "key_bits": kbits + int(kqjl), "key_format": args.key_format, "value_bits": vbits,
                   "parallelism": "none (1 GPU)"},
        "value_note": "keys/s = (query position, KV-head token) pairs scored per second over the whole prompt",
        "wall_s_timed": wall,
        "attend_call_ms": call_ms.tolist(), "attend_kernel_ms": kern_ms.tolist(),
        "roofline": {"bound": "mfma", "achieved": float(tput[-1]), "peak": mix_peak, "unit": "TFLOP/s",
                     "frac": float(tput[-1]) / mix_peak, "traffic": None,
                     "kernel": f"prefill_kernel<{kbits}, {vbits}, {str(kqjl).lower()}> on the last chunk "
                               f"({P} tokens visible to its last position; template arguments: key MSE bits, value "
                               "bits, QJL signs)",
                     "ops_per_vhead_token": k_ops + v_ops, "k_ops_per_vhead_token": k_ops,
                     "v_ops_per_vhead_token": v_ops, "avg_launch_ms": float(kern_ms[-1]),
                     "peak_note": ("executed exact-digit MFMA work (fp6 x fp4 score MFMAs, int8 value MFMAs) "
                                   "against the peak of that mix: 10.1 PFLOP/s fp6/fp4 and 5.0 POP/s int8 dense"),
                     "algorithmic_fp32_tflops": float(alg[-1]), "algorithmic_fp32_frac": float(alg[-1]) / FP32_PEAK_TFLOPS,
                     "algorithmic_note": ("4 d flops per (virtual head, visible token): the score's and the value "
                                          "sum's dot products at fp32 accuracy, against the 157.3 TFLOP/s fp32 peak"),
                     "timing": "HIP events on the launch stream around each chunk's prefill_kernel launch"},
    }
    if not args.no_cpu_baseline:
        rate, chunks, secs = oracle_prefill_rate(d, 2048, 64, Hq // H, kbits, vbits, args.cpu_seconds, args.data,
                                                 kqjl)
        res["cpu_baseline"] = {
            "value": rate, "unit": "keys/s", "cores": threads_used(), "kind": "oracle", **cpu_info(),
            "sample": f"{chunks} chunks of 64 causal query positions x {Hq // H} heads over one 2048-token packed "
                      f"stream (records encoded beforehand), {secs:.1f} s of CPU work"}
    return res


def run_polar(args, torch, tq, synth):
    """Decode attention with PolarQuant keys (b1 = 4, b2 = 3) and 3-bit stage-1
    values on the serving shape: prefill quantize of all K/V, then 32 decode
    calls over the cache."""
    B, H, Hq, L, NS, d = 64, 8, 32, 8192, 32, 128
    ctx = tq.Context(d, 0)
    K = kv_inputs(torch, synth, args, (B, H, L, d), (5, synth.TAG_KEYS), synth.TAG_SCALES_K)
    V = kv_inputs(torch, synth, args, (B, H, L, d), (5, synth.TAG_VALUES), synth.TAG_SCALES_V)
    QS = synth.torch_gaussian(0, (5, synth.TAG_QUERIES), (NS, B, Hq, d), torch.bfloat16, "cuda")
    cache = tq.PolarKVCache(B, H, L)
    cache.host_max_len = L
    ws = torch.empty(cache.decode_ws_bytes(ctx, Hq), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    timer = Timer(torch)
    kev, cev = [], []

    def step(record):
        cache.prefill(ctx, K, V)
        for i in range(NS):
            if record:
                tq.time_next_decode(*kev[i])
                cev.append(timer(lambda: cache.decode(ctx, QS[i], out=out, ws=ws)))
            else:
                cache.decode(ctx, QS[i], out=out, ws=ws)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    pre = timer(lambda: cache.prefill(ctx, K, V))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    whole = timer(lambda: [step(False) for _ in range(args.steps)])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = ms(whole) / args.steps
    for _ in range(NS):
        pair = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        for e in pair:
            e.record()
        kev.append(pair)
    torch.cuda.synchronize()
    step(True)
    torch.cuda.synchronize()
    kern_ms = float(np.mean([ms(k) for k in kev]))
    call_ms = float(np.mean([ms(c) for c in cev]))
    keys = B * H * L * NS
    # the scoring kernel's arithmetic per (token, query head), in its evaluation
    # order: a multiply and an fma (3 flops) at each of the 63 internal tree nodes;
    # the 64 leaves come from a per-block table (64 pairs x 16 level-1 codes x 3
    # flops per 256 tokens: 12); per level-4 subtree the ancestors' product (3
    # multiplies shared by the 4 heads) and an fma into the sum (2); the radius scale
    flops_per = 3 * 63 + 12 + (8 * 3) // 4 + 8 * 2 + 1
    tflops = B * Hq * L * flops_per / (kern_ms / 1e3) / 1e12
    rec = 60 + VAL_B3
    res = {
        "metric": METRIC, "value": keys / (ms_per_step / 1e3), "unit": "keys/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32 (PolarQuant tree evaluation) + i8 MFMA values",
        "data": f"synthetic ({args.data}-channel bf16 K/V, Gaussian bf16 queries, seeded)",
        "config": {"workload": (f"polar_decode: {B} seq x {L} ctx, {H} KV heads, {Hq} q heads, d={d}, PolarQuant "
                                f"keys (4-bit level-1 and 3-bit higher angles, fp32 radius: 60 B), values 3-bit; "
                                f"prefill quantize + {NS} decode calls"),
                   "batch": B, "context": L, "decode_calls": NS, "kv_heads": H, "q_heads": Hq, "head_dim": d,
                   "key_format": "polarquant(4,3)", "value_bits": 3, "parallelism": "none (1 GPU)"},
        "quantize_vectors_per_s": 2 * B * H * L / (ms(pre) / 1e3), "prefill_ms": ms(pre),
        "decode_call_ms": call_ms, "decode_keys_per_s": B * H * L / (call_ms / 1e3),
        "decode_call_gbs": B * H * L * rec / (call_ms / 1e3) / 1e9, "bytes_per_kv_token": rec,
        "wall_s_timed": wall,
        "roofline": {"bound": "alu", "achieved": tflops, "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / FP32_PEAK_TFLOPS, "traffic": None,
                     "kernel": "polar_logits_kernel (PolarQuant tree evaluation of every cached key for 4 heads)",
                     "flops_per_token_head": flops_per, "avg_launch_ms": kern_ms,
                     "timing": "HIP events on the launch stream around the scoring kernel of every decode call",
                     "peak_note": "157.3 TFLOP/s counts packed fp32 FMA; this path issues unpacked fp32 ops (half that)"},
    }
    if not args.no_cpu_baseline:
        from oracle import polarquant as PQ
        from oracle import turboquant as T
        Pi = T.rotation_from_gaussian(synth.gaussian_matrix(0, synth.TAG_ROTATION, d, d))
        pcb = PQ.polar_codebooks(d, 4, 3)
        cbv = T.codebook(d, 3)
        Ls = 4096
        Kh = synth.outlier_kv(0, (5, 1), synth.TAG_SCALES_K, (Ls, d))
        Vh = synth.outlier_kv(0, (5, 2), synth.TAG_SCALES_V, (Ls, d))
        t0c = time.perf_counter()
        kr = PQ.pack_polar(PQ.polar_encode(Kh, Pi, pcb), pcb)
        vr = T.pack_values(T.encode(Vh, Pi, cbv), 3)
        t_enc = time.perf_counter() - t0c
        n_dec, t_dec = 0, 0.0
        while t_dec < args.cpu_seconds / 2 or n_dec == 0:
            q = synth.gaussian(0, (5, 3, n_dec), (Hq // H, d), "bf16")
            t1 = time.perf_counter()
            PQ.polar_attention_decode(q, Pi, pcb, cbv, kr, vr, Ls, 1 / math.sqrt(d), T.unpack_values)
            t_dec += time.perf_counter() - t1
            n_dec += 1
        enc_rate, dec_rate = 2 * Ls / t_enc, Ls * n_dec / t_dec
        step_s = 2 * B * H * L / enc_rate + keys / dec_rate
        res["cpu_baseline"] = {
            "value": keys / step_s, "unit": "keys/s", "cores": threads_used(), "kind": "oracle", **cpu_info(),
            "sample": f"one stream of {Ls} tokens: oracle encode of its K and V, then {n_dec} decodes for "
                      f"{Hq // H} query heads ({t_enc + t_dec:.1f} s of CPU work), extrapolated to the step",
            "quantize_vectors_per_s": enc_rate, "decode_keys_per_s": dec_rate}
    return res


def run_search(args, torch, tq, synth):
    """Vector search: 1e6 unit-norm Gaussian vectors at d=1536 quantized at b=4,
    1000 queries scored against all of them, top-10 each."""
    d, N, NQ, K = 1536, 1_000_000, 1000, 10
    ctx = tq.Context(d, 0)
    X = synth.torch_unit_gaussian(0, (4, synth.TAG_DB), (N, d), "cuda")
    Qd = synth.torch_unit_gaussian(0, (4, synth.TAG_QUERIES), (NQ, d), "cuda")
    keys = tq.Packed(N, d, 3, True)
    work = torch.empty(tq.quantize_ws_bytes(ctx, 1, N, True), dtype=torch.uint8, device="cuda")
    sws = torch.empty(tq.scores_ws_bytes(ctx, NQ, N, K, False), dtype=torch.uint8, device="cuda")
    timer = Timer(torch)
    ev = {"q": [], "s": []}

    def step(record):
        a = timer(lambda: tq.quantize_kv(ctx, X, keys, work=work))
        b = timer(lambda: tq.scores(ctx, Qd, keys, want_scores=False, topk=K, ws=sws))
        if record:
            ev["q"].append(a)
            ev["s"].append(b)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    whole = timer(lambda: [step(True) for _ in range(args.steps)])
    torch.cuda.synchronize()
    ms_per_step = ms(whole) / args.steps
    q_ms = float(np.mean([ms(e) for e in ev["q"]]))
    s_ms = float(np.mean([ms(e) for e in ev["s"]]))
    _, ti, _ = tq.scores(ctx, Qd, keys, want_scores=False, topk=K, ws=sws)
    exact = torch.empty((NQ, K), dtype=torch.int64, device="cuda")
    for q0 in range(0, NQ, 100):
        exact[q0:q0 + 100] = torch.topk(Qd[q0:q0 + 100] @ X.T, K, dim=1).indices
    hits = sum(len(set(a) & set(b)) for a, b in zip(ti.cpu().numpy().tolist(), exact.cpu().numpy().tolist()))
    score_flops = 2.0 * NQ * N * 2 * d            # fp32-equivalent algorithmic flops of the scores
    score_mfma_ops = 10240.0 * (d // 128) * NQ * N  # fp6 x fp4 MFMA ops issued: 5 masks x 2 digit halves x 2*16*16*128 per 4x16 pairs per block
    quant_flops = 2.0 * N * d * (d + d)
    res = {
        "metric": "vector search pair-scores/s (top-10 fused); quantize vectors/s", "value": NQ * N / (ms_per_step / 1e3),
        "unit": "pair-scores/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic (unit-norm Gaussian, seeded)",
        "config": {"workload": "vector_search: 1e6 x d=1536 unit Gaussian, b=4, 1000 queries, top-10", "n": N, "d": d, "queries": NQ},
        "quantize_vectors_per_s": N / (q_ms / 1e3), "quantize_ms": q_ms, "scores_topk_ms": s_ms,
        "recall_at_10": hits / (NQ * K),
        # the step's dominant kernel: the quantize GEMM (fp32 input: fp32 MFMA)
        "roofline": {"bound": "mfma", "achieved": quant_flops / (q_ms / 1e3) / 1e12, "peak": FP32_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": quant_flops / (q_ms / 1e3) / 1e12 / FP32_PEAK_TFLOPS, "traffic": None,
                     "kernel": ("gemm_kernel<MODE_KEY_CODES> + gemm_kernel<MODE_KEY_SIGNS> (tq_quantize_kv, fp32 input: "
                                "Y = X Pi^T and Z = R S^T on v_mfma_f32_32x32x2_f32; algorithmic 2 N d (d + m) flops)"),
                     "timing": "HIP events around each tq_quantize_kv call of the timed steps"},
        "scores_roofline": {"bound": "mfma", "achieved": score_mfma_ops / (s_ms / 1e3) / 1e12, "peak": 10100.0,
                            "unit": "TFLOP/s", "frac": score_mfma_ops / (s_ms / 1e3) / 1e12 / 10100.0,
                            "fp32_equivalent_tflops": score_flops / (s_ms / 1e3) / 1e12,
                            "kernel": ("tq_scores: query prep (fp32 GEMMs, fp6 digits), search_kernel<3, true> "
                                       "(v_mfma_scale_f32_16x16x128_f8f6f4, fp6 query digits x fp4 bit masks, fused "
                                       "top-10), search_merge_kernel; timed as the whole call"),
                            "ops_per_pair": 10240.0 * (d // 128)},
    }
    if not args.no_cpu_baseline:
        import synth as sy
        from oracle import turboquant as T
        Pi = T.rotation_from_gaussian(sy.gaussian_matrix(0, sy.TAG_ROTATION, d, d))
        S = T.sketch_from_gaussian(sy.gaussian_matrix(0, sy.TAG_SKETCH, d, d))
        cb = T.codebook(d, 3)
        Xs = sy.unit_gaussian(0, (4, 99), (4096, d))
        Qs = sy.unit_gaussian(0, (4, 98), (100, d))
        t0 = time.perf_counter()
        enc = T.encode(Xs, Pi, cb, S)
        t1 = time.perf_counter()
        q_rot, q_s = T.query_prep(Qs, Pi, S)
        sc = T.scores_from_parts(q_rot, q_s, enc.idx, enc.sigma, enc.norm, enc.rho, cb, d)
        [T.topk(r, K) for r in sc]
        t2 = time.perf_counter()
        enc_rate, pair_rate = 4096 / (t1 - t0), 100 * 4096 / (t2 - t1)
        res["cpu_baseline"] = {"value": NQ * N / (N / enc_rate + NQ * N / pair_rate), "unit": "pair-scores/s",
                               "cores": threads_used(), "kind": "oracle", **cpu_info(),
                               "sample": f"encode 4096 vectors and score/top-10 100 queries against them "
                                         f"({t2 - t0:.1f} s); extrapolated to the step",
                               "quantize_vectors_per_s": enc_rate, "pair_scores_per_s": pair_rate}
    return res


def run_logits(args, torch, tq, synth):
    """The attention-logit computation alone, which the pages compare for 4-bit keys
    against 32-bit keys: the serving cache (64 sequences x 8 KV heads x 8192 tokens,
    32 query heads in groups of 4, d = 128, keys b = 4) scored by the decode path's
    query prep and key phase (tq_decode_logits: scale * s_t for every token and
    head), against the same keys held as fp32 and as bf16 tensors and scored by
    torch.matmul (a library batched GEMM per KV stream, [8192 x 128] x [128 x 4];
    the softmax scale, a free epilogue, is left out of the library side)."""
    d, B, H, Hq, L = 128, 64, 8, 32, 8192
    g, S_ = Hq // H, B * H
    kbits, kqjl, kdesc = key_format(args)
    ctx = tq.Context(d, 0)
    K = kv_inputs(torch, synth, args, (B, H, L, d), (3, synth.TAG_KEYS), synth.TAG_SCALES_K)
    V = kv_inputs(torch, synth, args, (B, H, L, d), (3, synth.TAG_VALUES), synth.TAG_SCALES_V)
    Q = kv_inputs(torch, synth, args, (1, B, Hq, d), (3, synth.TAG_QUERIES), synth.TAG_SCALES_K)[0].contiguous()
    cache = tq.KVCache(B, H, L, d, kbits, 3, key_qjl=kqjl)
    cache.prefill(ctx, K, V)
    torch.cuda.synchronize()
    del V
    cache.host_max_len = L
    ws = torch.empty(cache.decode_ws_bytes(ctx, Hq), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, Hq, L), dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(d)
    K32 = K.float().view(S_, L, d)
    Kb = K.view(S_, L, d)
    Q32 = Q.float().view(S_, g, d).transpose(1, 2).contiguous()  # [stream, d, 4]: a contiguous right operand
    Qb = Q.view(S_, g, d).transpose(1, 2).contiguous()
    o32 = torch.empty((S_, L, g), dtype=torch.float32, device="cuda")
    ob = torch.empty((S_, L, g), dtype=torch.bfloat16, device="cuda")
    timer = Timer(torch)
    legs = {"turboquant": lambda: cache.decode_logits(ctx, Q, scale, ws=ws, out=out),
            "fp32": lambda: torch.matmul(K32, Q32, out=o32),
            "bf16": lambda: torch.matmul(Kb, Qb, out=ob)}
    t = {}
    for name, fn in legs.items():
        for _ in range(max(args.warmup, 1)):
            fn()
        torch.cuda.synchronize()
        evs = [timer(fn) for _ in range(max(args.steps, 3))]
        torch.cuda.synchronize()
        t[name] = float(np.median([ms(e) for e in evs]))
    keys = S_ * L
    rec_b = (d // 32) * 4 * (kbits + int(kqjl)) + 4 * (1 + int(kqjl))  # key words and norms per token
    alg = keys * (rec_b + 4 * g)  # key records read, 4 logits (fp32) written per token
    res = {
        "metric": "attention-logit keys/s (logits alone, packed keys vs fp32 and bf16 keys)",
        "value": keys / (t["turboquant"] / 1e3), "unit": "keys/s", "n_gpus": 1, "steps": max(args.steps, 3),
        "warmup": max(args.warmup, 1), "ms_per_step": t["turboquant"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32+fp6/fp4 exact-digit MFMA", "data": "synthetic (outlier-channel bf16 K, seeded)"
        if args.data == "outlier" else "synthetic (i.i.d. N(0,1) bf16 K, seeded)",
        "config": {"workload": f"attention_logits: 64 seq x 8192 ctx, 8 KV heads, 32 q heads, d=128, {kdesc}",
                   "batch": B, "context": L, "kv_heads": H, "q_heads": Hq, "head_dim": d},
        "turboquant_ms": t["turboquant"], "fp32_keys_ms": t["fp32"], "bf16_keys_ms": t["bf16"],
        "speedup_vs_fp32_keys": t["fp32"] / t["turboquant"], "speedup_vs_bf16_keys": t["bf16"] / t["turboquant"],
        "fp32_keys_hbm_floor_ms": keys * (4 * d + 4 * g) / 8e12 * 1e3,
        "speedup_vs_fp32_keys_hbm_floor": keys * (4 * d + 4 * g) / 8e12 * 1e3 / t["turboquant"],
        "roofline": {"bound": "hbm", "achieved": alg / (t["turboquant"] / 1e3) / 1e9, "peak": 8000.0, "unit": "GB/s",
                     "frac": alg / (t["turboquant"] / 1e3) / 1e9 / 8000.0, "traffic": None,
                     "kernel": "tq_decode_logits: decode_prep_kernel (query prep) + decode_kernel<..., LOGITS> (key phase)",
                     "bytes_per_kv_token": rec_b + 4 * g, "timing": "HIP events around each whole call, median"},
    }
    if not args.no_cpu_baseline:
        import synth as sy
        from oracle import turboquant as T
        Pi = T.rotation_from_gaussian(sy.gaussian_matrix(0, sy.TAG_ROTATION, d, d))
        Sk = T.sketch_from_gaussian(sy.gaussian_matrix(0, sy.TAG_SKETCH, d, d))
        cb = T.codebook(d, kbits) if kbits > 0 else None
        Qh = Q.float().cpu().numpy().astype(np.float64)
        el, n = 0.0, 0  # oracle time only (the copies of the records to the host are not timed)
        while el < min(args.cpu_seconds, 6.0) and n < S_:
            kw = cache.k.words[n * L:(n + 1) * L].cpu().numpy().view(np.uint32)
            kn = cache.k.norms[n * L:(n + 1) * L].cpu().numpy()
            t1 = time.perf_counter()
            T.scores(Qh[n // H, (n % H) * g:(n % H + 1) * g], Pi, Sk, cb, {"bits": kw, "norms": kn}, kqjl)
            el += time.perf_counter() - t1
            n += 1
        res["cpu_baseline"] = {"value": n * L / el, "unit": "keys/s", "cores": threads_used(), "kind": "oracle",
                               **cpu_info(), "sample": f"{n} whole KV streams of {L} tokens scored for their 4 query "
                                                       f"heads by the oracle ({el:.1f} s)"}
    return res


def run_tiny(args, torch, tq, synth):
    """4096 fp32 keys at d=128, b=3; 16 queries; the 16 x 4096 score matrix."""
    d = 128
    ctx = tq.Context(d, 0)
    X = torch.from_numpy(synth.gaussian(0, (0, synth.TAG_KEYS), (4096, d))).cuda()
    Q = torch.from_numpy(synth.gaussian(0, (0, synth.TAG_QUERIES), (16, d))).cuda()
    keys = tq.Packed(4096, d, 2, True)
    timer = Timer(torch)
    evs = []

    def step():
        tq.quantize_kv(ctx, X, keys)
        tq.scores(ctx, Q, keys)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    for _ in range(args.steps):
        evs.append(timer(step))
    torch.cuda.synchronize()
    ms_per_step = float(np.mean([ms(e) for e in evs]))
    return {"metric": "tiny reference: quantize + 16x4096 scores (cache-resident, launch-bound)", "value": 4096 / (ms_per_step / 1e3),
            "unit": "vectors/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": "tiny_reference: 4096 x d=128 fp32 N(0,1), b=3, 16 queries"}, "roofline": None}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (this path has no multi-GPU mode); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import kv_cache_vector_turboquant_amd as tq
    import synth

    torch.cuda.set_device(0)
    if args.copy_probe_mib > 0:
        copy_probe(torch, args.copy_probe_mib)
        return
    serving = (64, 8, 32, 8192, 128, "serving",
               "batched_serving_step: 64 seq x 8192 ctx, 8 KV heads, 32 q heads, d=128, "
               f"{key_format(args)[2]}, values 3-bit, prefill quantize + 128 x (append + decode)")
    gqa = (4, 8, 32, 131072, 0, "gqa",
           "gqa_layer: batch 4 x 131072 ctx, 8 KV heads, 32 q heads, d=128, "
           f"{key_format(args)[2]}, values 3-bit, prefill quantize + 1 decode")
    if args.workload in ("serving", "gqa"):
        shape = serving if args.workload == "serving" else gqa
        res = run_decode_workload(args, torch, tq, synth, *shape)
        if args.data == "outlier" and not args.no_gaussian_pass:
            # the same workload on i.i.d. Gaussian K/V: both data laws in one line
            import copy
            a2 = copy.copy(args)
            a2.data, a2.graph, a2.cpu_seconds = "gaussian", False, min(args.cpu_seconds, 6.0)
            g = run_decode_workload(a2, torch, tq, synth, *shape)
            rf = g["roofline"]
            res["gaussian"] = {
                "data": g["data"], "value": g["value"], "unit": g["unit"], "ms_per_step": g["ms_per_step"],
                "quantize_vectors_per_s": g["quantize_vectors_per_s"],
                "roofline": {k: rf[k] for k in ("bound", "achieved", "peak", "unit", "frac", "avg_launch_ms",
                                                 "read_ceiling_gbs", "frac_of_read_ceiling")},
                "cpu_baseline": g.get("cpu_baseline")}
    elif args.workload == "single":
        res = run_decode_workload(args, torch, tq, synth, 1, 1, 1, 32768, 0, "single",
                                  "single_head_decode: 32768 ctx, d=128, keys b=4, values 3-bit, quantize + 1 decode")
    elif args.workload == "search":
        res = run_search(args, torch, tq, synth)
    elif args.workload == "prefill":
        res = run_prefill(args, torch, tq, synth)
    elif args.workload == "polar":
        res = run_polar(args, torch, tq, synth)
    elif args.workload == "logits":
        res = run_logits(args, torch, tq, synth)
    else:
        res = run_tiny(args, torch, tq, synth)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
