"""Full-size GPU checks at the workloads' real shapes, in the launch
configuration the benchmark uses, on sampled outputs the oracle can compute.

* GQA decode layer: batch 4, 8 KV heads, 32 query heads, context 131072,
  bf16 outlier-channel K/V, keys b=3 and b=4, 3-bit values.
* Batched serving step: 64 sequences x 8192 tokens x 8 KV heads, 32 query
  heads, prefill quantize, 128 appends, decode at b=4.
* Vector search: 1,000,000 unit-norm Gaussian vectors at d=1536, b=4, 1000
  queries, scores and top-10.

Encode parity is checked on sampled records (inputs copied back from the
device). Decode parity is checked on sampled (sequence, KV head) streams whose
records are replaced by oracle-packed records of the same inputs, so the GPU
kernel and the oracle read identical bytes at full context length.
"""
import math

import numpy as np
import pytest

import synth
from oracle import turboquant as T
from tests import parity as P

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
tq = pytest.importorskip("kv_cache_vector_turboquant_amd")

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

DEV = "cuda"


def _oracle_tables(d, seed=0):
    Pi = T.rotation_from_gaussian(synth.gaussian_matrix(seed, synth.TAG_ROTATION, d, d))
    S = T.sketch_from_gaussian(synth.gaussian_matrix(seed, synth.TAG_SKETCH, d, d))
    return Pi, S


def _inject_stream(cache, s, Kh, Vh, Pi, S, cbk, cbv):
    """Replace stream s's records with oracle-packed records of Kh/Vh (host fp32)."""
    cap = cache.capacity
    pk = T.pack_keys(T.encode(Kh, Pi, cbk, S), cbk.bits)
    pv = T.pack_values(T.encode(Vh, Pi, cbv), cbv.bits)
    L = Kh.shape[0]
    cache.k.words[s * cap:s * cap + L].copy_(torch.from_numpy(pk["bits"].view(np.int32)).to(DEV))
    cache.k.norms[s * cap:s * cap + L].copy_(torch.from_numpy(pk["norms"]).to(DEV))
    nb = pv["bits"].shape[0]
    cache.v.words[s * cap // 32:s * cap // 32 + nb].copy_(torch.from_numpy(pv["bits"].view(np.int32)).to(DEV))
    cache.v.norms[s * cap:s * cap + L].copy_(torch.from_numpy(pv["norms"]).to(DEV))
    return pk, pv


def _check_sampled_records(cache, s, Kh, Vh, rows, Pi, S, cbk, cbv):
    cap = cache.capacity
    kw = cache.k.words[s * cap:s * cap + Kh.shape[0]].cpu().numpy().view(np.uint32)
    kn = cache.k.norms[s * cap:s * cap + Kh.shape[0]].cpu().numpy()
    P.check_key_records(kw[rows], kn[rows], T.encode(Kh[rows], Pi, cbk, S), cbk, cbk.bits, Kh.shape[1])
    vw = cache.v.words[s * cap // 32:(s * cap + cap) // 32].cpu().numpy().view(np.uint32)
    g_idx = T.unpack_values(vw, Kh.shape[1], cbv.bits, Vh.shape[0])[rows]
    P.check_codes(g_idx, T.encode(Vh[rows], Pi, cbv), cbv, "value codes")


@pytest.mark.parametrize("kbits", [2, 3])
def test_gqa_layer_131k(kbits):
    d, B, H, Hq, L = 128, 4, 8, 32, 131072
    Pi, S = _oracle_tables(d)
    cbk, cbv = T.codebook(d, kbits), T.codebook(d, 3)
    ctx = tq.Context(d, 0)
    K = synth.torch_outlier_kv(0, (2, synth.TAG_KEYS), synth.TAG_SCALES_K, (B, H, L, d), torch.bfloat16, DEV)
    V = synth.torch_outlier_kv(0, (2, synth.TAG_VALUES), synth.TAG_SCALES_V, (B, H, L, d), torch.bfloat16, DEV)
    Q = synth.torch_outlier_kv(0, (2, synth.TAG_QUERIES), synth.TAG_SCALES_K, (B, Hq, d), torch.bfloat16, DEV)
    cache = tq.KVCache(B, H, L, d, kbits, 3)
    cache.prefill(ctx, K, V)
    torch.cuda.synchronize()
    rng = np.random.default_rng(kbits)
    streams = [5, 30]
    for s in streams:
        b, h = divmod(s, H)
        Kh = K[b, h].float().cpu().numpy()
        Vh = V[b, h].float().cpu().numpy()
        rows = np.sort(rng.choice(L, 2048, replace=False))
        _check_sampled_records(cache, s, Kh, Vh, rows, Pi, S, cbk, cbv)
        _inject_stream(cache, s, Kh, Vh, Pi, S, cbk, cbv)
    out = cache.decode(ctx, Q).cpu().numpy()
    torch.cuda.synchronize()
    Qh = Q.float().cpu().numpy()
    for s in streams:
        b, h = divmod(s, H)
        Kh = K[b, h].float().cpu().numpy()
        Vh = V[b, h].float().cpu().numpy()
        keys = T.pack_keys(T.encode(Kh, Pi, cbk, S), kbits)
        vals = T.pack_values(T.encode(Vh, Pi, cbv), 3)
        ref = T.attention_decode(Qh[b, 4 * h:4 * h + 4], Pi, S, cbk, cbv, keys, vals, L, 1 / math.sqrt(d))
        err = np.max(np.abs(out[b, 4 * h:4 * h + 4] - ref))
        assert err <= 2e-3, f"stream {s}: {err}"


def test_serving_step_64x8192():
    d, B, H, Hq, L, NS = 128, 64, 8, 32, 8192, 128
    Pi, S = _oracle_tables(d)
    cbk, cbv = T.codebook(d, 3), T.codebook(d, 3)
    ctx = tq.Context(d, 0)
    cap = L + NS
    K = synth.torch_outlier_kv(0, (3, synth.TAG_KEYS), synth.TAG_SCALES_K, (B, H, L, d), torch.bfloat16, DEV)
    V = synth.torch_outlier_kv(0, (3, synth.TAG_VALUES), synth.TAG_SCALES_V, (B, H, L, d), torch.bfloat16, DEV)
    KA = synth.torch_outlier_kv(0, (3, synth.TAG_APPEND_K), synth.TAG_SCALES_K, (NS, B, H, d), torch.bfloat16, DEV)
    VA = synth.torch_outlier_kv(0, (3, synth.TAG_APPEND_V), synth.TAG_SCALES_V, (NS, B, H, d), torch.bfloat16, DEV)
    QS = synth.torch_outlier_kv(0, (3, synth.TAG_QUERIES), synth.TAG_SCALES_K, (NS, B, Hq, d), torch.bfloat16, DEV)
    cache = tq.KVCache(B, H, cap, d, 3, 3)
    tq.quantize_kv(ctx, K.view(B * H, L, d), cache.k, out_stream_stride=cap)
    tq.quantize_kv(ctx, V.view(B * H, L, d), cache.v, out_stream_stride=cap)
    cache.seq_len.fill_(L)
    cache.host_max_len = L
    out = None
    for i in range(NS):
        cache.append(ctx, KA[i], VA[i])
        out = cache.decode(ctx, QS[i])
    torch.cuda.synchronize()
    assert cache.seq_len.cpu().tolist() == [L + NS] * B
    streams = [0, 263, 511]
    rng = np.random.default_rng(7)
    Kfull = {}
    for s in streams:
        b, h = divmod(s, H)
        Kh = np.concatenate([K[b, h].float().cpu().numpy(), KA[:, b, h].float().cpu().numpy()])
        Vh = np.concatenate([V[b, h].float().cpu().numpy(), VA[:, b, h].float().cpu().numpy()])
        rows = np.sort(np.concatenate([rng.choice(L, 1024, replace=False), np.arange(L, L + NS)]))
        _check_sampled_records(cache, s, Kh, Vh, rows, Pi, S, cbk, cbv)
        _inject_stream(cache, s, Kh, Vh, Pi, S, cbk, cbv)
        Kfull[s] = (Kh, Vh)
    # decode once more with the last step's queries over the full, partly oracle-packed cache
    out = cache.decode(ctx, QS[NS - 1]).cpu().numpy()
    torch.cuda.synchronize()
    Qh = QS[NS - 1].float().cpu().numpy()
    for s in streams:
        b, h = divmod(s, H)
        Kh, Vh = Kfull[s]
        keys = T.pack_keys(T.encode(Kh, Pi, cbk, S), 3)
        vals = T.pack_values(T.encode(Vh, Pi, cbv), 3)
        ref = T.attention_decode(Qh[b, 4 * h:4 * h + 4], Pi, S, cbk, cbv, keys, vals, L + NS, 1 / math.sqrt(d))
        err = np.max(np.abs(out[b, 4 * h:4 * h + 4] - ref))
        assert err <= 2e-3, f"stream {s}: {err}"


def test_vector_search_1m_x_1536():
    d, N, NQ, K = 1536, 1_000_000, 1000, 10
    Pi, S = _oracle_tables(d)
    cb = T.codebook(d, 3)
    ctx = tq.Context(d, 0)
    X = synth.torch_unit_gaussian(0, (4, synth.TAG_DB), (N, d), DEV)
    Qd = synth.torch_unit_gaussian(0, (4, synth.TAG_QUERIES), (NQ, d), DEV)
    keys = tq.Packed(N, d, 3, True)
    tq.quantize_kv(ctx, X, keys)
    sc, ti, tv = tq.scores(ctx, Qd, keys, want_scores=False, topk=K)
    # exact fp32 brute force for recall@10 (reported quantity, computed with torch)
    exact = torch.empty((NQ, K), dtype=torch.int64, device=DEV)
    for q0 in range(0, NQ, 100):
        s = Qd[q0:q0 + 100] @ X.T
        exact[q0:q0 + 100] = torch.topk(s, K, dim=1).indices
    torch.cuda.synchronize()
    ti_h, tv_h = ti.cpu().numpy(), tv.cpu().numpy()
    recall = T.recall_at_k(ti_h, exact.cpu().numpy())
    assert recall > 0.5, recall
    rng = np.random.default_rng(4)
    # sampled encode parity
    rows = np.sort(rng.choice(N, 1000, replace=False))
    rows_t = torch.from_numpy(rows).to(DEV)
    kw = keys.words[rows_t].cpu().numpy().view(np.uint32)
    kn = keys.norms[rows_t].cpu().numpy()
    Xs = X[rows_t].cpu().numpy()
    P.check_key_records(kw, kn, T.encode(Xs, Pi, cb, S), cb, 3, d)
    # reported top-10 scores equal the oracle's scores of those (query, key) pairs,
    # and no sampled key beats the reported 10th score
    qs = rng.choice(NQ, 8, replace=False)
    sample = np.sort(rng.choice(N, 3000, replace=False))
    enc_sample = T.encode(X[torch.from_numpy(sample).to(DEV)].cpu().numpy(), Pi, cb, S)
    for q in qs:
        qv = Qd[q].cpu().numpy()[None, :]
        q_rot, q_s = T.query_prep(qv, Pi, S)
        enc_top = T.encode(X[ti[q].long()].cpu().numpy(), Pi, cb, S)
        ref_top = T.scores_from_parts(q_rot, q_s, enc_top.idx, enc_top.sigma, enc_top.norm.astype(np.float32),
                                      enc_top.rho.astype(np.float32), cb, d)[0]
        gpu_codes = T.unpack_keys(keys.words[ti[q].long()].cpu().numpy().view(np.uint32), d, 3)[0]
        same = np.all(gpu_codes == enc_top.idx, axis=1)  # skip keys with an excused code flip
        assert np.all(np.abs(tv_h[q][same] - ref_top[same]) <= 1e-3 * np.abs(ref_top[same]) + 1e-6)
        ref_s = T.scores_from_parts(q_rot, q_s, enc_sample.idx, enc_sample.sigma, enc_sample.norm.astype(np.float32),
                                    enc_sample.rho.astype(np.float32), cb, d)[0]
        outside = ~np.isin(sample, ti_h[q])
        assert np.max(ref_s[outside]) <= tv_h[q][K - 1] + 1e-3 * abs(tv_h[q][K - 1]) + 1e-6
    # full top-10 parity for 4 queries: oracle scores over all 10^6 GPU-encoded
    # records (identical packed bytes), chunked over threads; the GPU's top-10
    # set equals the oracle's up to near-ties, its values match the oracle's
    qf = rng.choice(NQ, 4, replace=False)
    q_rot, q_s = T.query_prep(Qd[torch.from_numpy(qf).to(DEV)].cpu().numpy(), Pi, S)
    CH = 25000

    def chunk_scores(i0):
        w = keys.words[i0:i0 + CH].cpu().numpy().view(np.uint32)
        nrm = keys.norms[i0:i0 + CH].cpu().numpy()
        idx, sig = T.unpack_keys(w, d, 3)
        return T.scores_from_parts(q_rot, q_s, idx, sig, nrm[:, 0], nrm[:, 1], cb, d)

    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(8) as ex:
        s_full = np.concatenate(list(ex.map(chunk_scores, range(0, N, CH))), axis=1)
    xnorm = keys.norms[:, 0].cpu().numpy().astype(np.float64)
    qn = np.linalg.norm(Qd[torch.from_numpy(qf).to(DEV)].cpu().numpy().astype(np.float64), axis=1)
    P.check_topk(ti_h[qf], tv_h[qf], s_full, K, qn, xnorm)
    print(f"recall@10 = {recall:.4f}")


def test_fused_step_bench_shape():
    """tq_decode_step in the serving benchmark's launch configuration: 64
    sequences x 8192 tokens x 8 KV heads, 32 query heads, b = 4 keys, 3-bit
    values, outlier-channel bf16 data with the benchmark's seeds, the workspace
    sized for the whole 128-step run. Three fused steps; after each, sampled
    streams' outputs against the oracle over the records the cache then holds
    (identical bytes), and their appended records against the oracle's encoding."""
    d, B, H, Hq, L, NS, NSTEP = 128, 64, 8, 32, 8192, 128, 3
    Pi, S = _oracle_tables(d)
    cbk, cbv = T.codebook(d, 3), T.codebook(d, 3)
    ctx = tq.Context(d, 0)
    cap = ((L + NS + 31) // 32) * 32
    gen = synth.torch_outlier_kv
    K = gen(0, (3, synth.TAG_KEYS), synth.TAG_SCALES_K, (B, H, L, d), torch.bfloat16, DEV)
    V = gen(0, (3, synth.TAG_VALUES), synth.TAG_SCALES_V, (B, H, L, d), torch.bfloat16, DEV)
    KA = gen(0, (3, synth.TAG_APPEND_K), synth.TAG_SCALES_K, (NS, B, H, d), torch.bfloat16, DEV)
    VA = gen(0, (3, synth.TAG_APPEND_V), synth.TAG_SCALES_V, (NS, B, H, d), torch.bfloat16, DEV)
    QS = gen(0, (3, synth.TAG_QUERIES), synth.TAG_SCALES_K, (NS, B, Hq, d), torch.bfloat16, DEV)
    cache = tq.KVCache(B, H, cap, d, 3, 3)
    cache.host_max_len = cap
    dws = torch.empty(max(cache.decode_ws_bytes(ctx, Hq), cache.decode_step_ws_bytes(ctx, Hq)), dtype=torch.uint8,
                      device=DEV)
    cache.prefill(ctx, K, V)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=DEV)
    streams = [0, 263, 511]
    scale = 1 / math.sqrt(d)
    for i in range(NSTEP):
        cache.decode_step(ctx, KA[i], VA[i], QS[i], out=out, ws=dws)
        torch.cuda.synchronize()
        n = L + i + 1
        assert cache.seq_len.cpu().tolist() == [n] * B and cache.host_max_len == n
        o = out.cpu().numpy()
        Qh = QS[i].float().cpu().numpy()
        for s in streams:
            b, h = divmod(s, H)
            kw = cache.k.words[s * cap:s * cap + n].cpu().numpy().view(np.uint32)
            kn = cache.k.norms[s * cap:s * cap + n].cpu().numpy()
            vw = cache.v.words[s * cap // 32:(s + 1) * cap // 32].cpu().numpy().view(np.uint32)
            vn = cache.v.norms[s * cap:s * cap + n].cpu().numpy()
            ref = T.attention_decode(Qh[b, 4 * h:4 * h + 4], Pi, S, cbk, cbv, {"bits": kw, "norms": kn},
                                     {"bits": vw, "norms": vn}, n, scale)
            err = np.max(np.abs(o[b, 4 * h:4 * h + 4] - ref))
            assert err <= 2e-3, f"step {i} stream {s}: {err}"
            # the appended record of this step
            ka = KA[i, b, h].float().cpu().numpy()[None]
            va = VA[i, b, h].float().cpu().numpy()[None]
            P.check_key_records(kw[n - 1:n], kn[n - 1:n], T.encode(ka, Pi, cbk, S), cbk, 3, d)
            g_idx = T.unpack_values(vw, d, 3, n)[n - 1:n]
            P.check_codes(g_idx, T.encode(va, Pi, cbv), cbv, "appended value codes")
