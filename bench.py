"""Benchmark of the TurboQuant hot path on one MI355X.

Workload (one "step" = one pass of the whole hot path over one batch):
batched serving step with 64 sequences x 8192-token context, 8 KV heads,
32 query heads, head_dim 128, bf16 K/V; prefill quantize of all 64 x 8 x 8192
K and V vectors (keys b=4: 3-bit Lloyd-Max + 1-bit QJL; values 3-bit), then
128 decode steps, each appending one quantized token per sequence and running
decode attention over the packed cache.

Prints ONE JSON line. `value` = attention-score keys/s of the whole step
(KV-head tokens scored by decode attention, divided by the step time,
prefill included). Inputs are resident in HBM before the timed region.
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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--data", choices=["outlier", "gaussian"], default="outlier")
    ap.add_argument("--batch", type=int, default=64)
    ap.add_argument("--ctx", type=int, default=8192)
    ap.add_argument("--decode-steps", type=int, default=128)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    return ap.parse_args()


def cpu_baseline(args, d, kv_heads, group, kbits, vbits, total_keys_per_step, vectors_per_step, decode_tokens):
    """The oracle as it stands, on a bounded sample of the same workload: whole
    (sequence, KV head) streams of the prefill (encode 8192 K + 8192 V vectors)
    and their decode attention for the 4 query heads of that KV head over the
    full context. Extrapolated to the step: quantize all prefill vectors, plus
    128 decodes over every stream."""
    import synth
    from oracle import turboquant as T
    Pi = T.rotation_from_gaussian(synth.gaussian_matrix(0, synth.TAG_ROTATION, d, d))
    S = T.sketch_from_gaussian(synth.gaussian_matrix(0, synth.TAG_SKETCH, d, d))
    cbk, cbv = T.codebook(d, kbits), T.codebook(d, vbits)
    L = args.ctx
    t_enc = t_dec = 0.0
    n_enc = n_dec = 0
    streams = 0
    t_start = time.perf_counter()
    while time.perf_counter() - t_start < args.cpu_seconds:
        K = synth.outlier_kv(0, (streams, 91), synth.TAG_SCALES_K, (L, d))
        V = synth.outlier_kv(0, (streams, 92), synth.TAG_SCALES_V, (L, d))
        Q = synth.outlier_kv(0, (streams, 93), synth.TAG_SCALES_K, (group, d))
        t0 = time.perf_counter()
        keys = T.pack_keys(T.encode(K, Pi, cbk, S), kbits)
        vals = T.pack_values(T.encode(V, Pi, cbv), vbits)
        t1 = time.perf_counter()
        T.attention_decode(Q, Pi, S, cbk, cbv, keys, vals, L, 1 / math.sqrt(d))
        t2 = time.perf_counter()
        t_enc += t1 - t0
        t_dec += t2 - t1
        n_enc += 2 * L
        n_dec += L
        streams += 1
    enc_rate = n_enc / t_enc           # vectors/s
    dec_rate = n_dec / t_dec           # KV-head tokens/s (with `group` query heads each)
    step_s = vectors_per_step / enc_rate + decode_tokens / dec_rate
    try:
        threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    except Exception:
        threads = os.cpu_count()
    return {
        "value": total_keys_per_step / step_s, "unit": "keys/s", "cores": threads, "kind": "oracle",
        "sample": f"{streams} whole streams (encode {L} K + {L} V vectors, decode {group} query heads over {L} "
                  f"tokens) in {t_enc + t_dec:.1f} s; extrapolated to the step "
                  f"(oracle quantize {enc_rate:.0f} vectors/s, decode {dec_rate:.0f} keys/s)",
        "quantize_vectors_per_s": enc_rate, "decode_keys_per_s": dec_rate,
    }


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
    dev = "cuda"
    d, kv_heads, q_heads, kbits, vbits = 128, 8, 32, 3, 3
    B, L, NS = args.batch, args.ctx, args.decode_steps
    cap = ((L + NS + 31) // 32) * 32
    group = q_heads // kv_heads
    ctx = tq.Context(d, 0)

    # ---- inputs resident in HBM (seeded, synthetic) ----
    gen = synth.torch_outlier_kv if args.data == "outlier" else None

    def kv(tags, scale_tag, shape):
        if gen is not None:
            return gen(0, tags, scale_tag, shape, torch.bfloat16, dev)
        return synth.torch_gaussian(0, tags, shape, torch.bfloat16, dev)

    K = kv((3, synth.TAG_KEYS), synth.TAG_SCALES_K, (B, kv_heads, L, d))
    V = kv((3, synth.TAG_VALUES), synth.TAG_SCALES_V, (B, kv_heads, L, d))
    KA = kv((3, synth.TAG_APPEND_K), synth.TAG_SCALES_K, (NS, B, kv_heads, d))
    VA = kv((3, synth.TAG_APPEND_V), synth.TAG_SCALES_V, (NS, B, kv_heads, d))
    QS = kv((3, synth.TAG_QUERIES), synth.TAG_SCALES_K, (NS, B, q_heads, d))
    cache = tq.KVCache(B, kv_heads, cap, d, kbits, vbits)
    kwork = torch.empty(tq.quantize_ws_bytes(ctx, B * kv_heads, L, True), dtype=torch.uint8, device=dev)
    cache.host_max_len = L + NS
    dws = torch.empty(cache.decode_ws_bytes(ctx, q_heads), dtype=torch.uint8, device=dev)
    cache.host_max_len = 0
    out = torch.empty((B, q_heads, d), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def prefill():
        tq.quantize_kv(ctx, K.view(B * kv_heads, L, d), cache.k, out_stream_stride=cap, work=kwork)
        tq.quantize_kv(ctx, V.view(B * kv_heads, L, d), cache.v, out_stream_stride=cap)
        cache.seq_len.fill_(L)
        cache.host_max_len = L

    ev_dec = []

    def step(record=False):
        prefill()
        for i in range(NS):
            cache.append(ctx, KA[i], VA[i])
            if record:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                cache.decode(ctx, QS[i], out=out, ws=dws)
                e1.record(stream)
                ev_dec.append((e0, e1, L + i + 1))
            else:
                cache.decode(ctx, QS[i], out=out, ws=dws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # prefill-only timing (quantize vectors/s), outside the step loop
    pe0, pe1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    pe0.record(stream)
    prefill()
    pe1.record(stream)
    torch.cuda.synchronize()
    prefill_ms = pe0.elapsed_time(pe1)

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record(stream)
    for _ in range(args.steps):
        step(record=True)
    s1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = s0.elapsed_time(s1)
    ms_per_step = total_ms / args.steps

    keys_per_step = sum(B * kv_heads * (L + i + 1) for i in range(NS))
    value = keys_per_step / (ms_per_step / 1e3)
    vectors_per_step = 2 * B * kv_heads * L
    # dominant kernel: decode attention (prep + chunked score/softmax/value + merge launches)
    dec_ms = [e0.elapsed_time(e1) for (e0, e1, _) in ev_dec]
    dec_bytes = [B * kv_heads * n * (T_KEY_BYTES + T_VAL_BYTES) for (_, _, n) in ev_dec]
    avg_ms = float(np.mean(dec_ms))
    avg_bytes = float(np.mean(dec_bytes))
    achieved = avg_bytes / (avg_ms / 1e3) / 1e9
    roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": None,
            "kernel": "tq_attention_decode (decode_prep + decode_kernel<3,3> + decode_merge)",
            "algorithmic_bytes_per_launch": avg_bytes, "avg_launch_ms": avg_ms}
    res = {
        "metric": METRIC, "value": value, "unit": "keys/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32+i8", "data": f"synthetic ({args.data}-channel bf16 K/V, seeded)",
        "config": {"workload": f"batched_serving_step: {B} seq x {L} ctx, {kv_heads} KV heads, {q_heads} q heads, "
                               f"d={d}, keys b=4 (3+1 QJL), values 3-bit, prefill quantize + {NS} x "
                               f"(append + decode attention)",
                   "batch": B, "context": L, "decode_steps": NS, "kv_heads": kv_heads, "q_heads": q_heads,
                   "head_dim": d, "parallelism": "none (1 GPU)"},
        "quantize_vectors_per_s": vectors_per_step / (prefill_ms / 1e3),
        "prefill_ms": prefill_ms,
        "decode_keys_per_s": float(np.sum([B * kv_heads * n for (_, _, n) in ev_dec]) / (np.sum(dec_ms) / 1e3)),
        "wall_s_timed": wall,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        decode_tokens = keys_per_step
        res["cpu_baseline"] = cpu_baseline(args, d, kv_heads, group, kbits, vbits, keys_per_step,
                                           vectors_per_step, decode_tokens)
    print(json.dumps(res), flush=True)


# algorithmic bytes per KV-head token at d = 128: key record 72 B (48 B codes + 16 B signs + 8 B norms),
# value record 52 B (48 B codes + 4 B norm)
T_KEY_BYTES = 72
T_VAL_BYTES = 52

if __name__ == "__main__":
    main()
