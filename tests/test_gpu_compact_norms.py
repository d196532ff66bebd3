"""GPU parity of compact records: every norm stored as fp16 (nearest even,
saturated at 65504) instead of fp32, two bytes less per norm. Records written
by both quantize paths and both appends match the oracle's encoding (codes
under the usual band rule; each norm the fp16 rounding of a value within the
fp32 norm tolerance); decode, prefill attention, the fused step and scores
over compact records match the oracle over the same records at the usual bars;
a paged compact cache equals a contiguous one bit for bit."""
import math

import numpy as np
import pytest

import synth
from oracle import turboquant as T
from tests import parity as P

torch = pytest.importorskip("torch")
tq = pytest.importorskip("kv_cache_vector_turboquant_amd")

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

pytestmark = pytest.mark.gpu
DEV = "cuda"
VARIANTS = [(3, True), (3, False), (0, True)]
IDS = ["tq4", "mse3", "qjl"]


@pytest.fixture(scope="module")
def c128():
    ctx = tq.Context(128, 0)
    Pi = T.rotation_from_gaussian(synth.gaussian_matrix(0, synth.TAG_ROTATION, 128, 128))
    S = T.sketch_from_gaussian(synth.gaussian_matrix(0, synth.TAG_SKETCH, 128, 128))
    return ctx, Pi, S


def _dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def _encode(X, Pi, S, bits, qjl):
    cb = T.codebook(Pi.shape[0], bits) if bits > 0 else None
    return T.encode(X, Pi, cb, S if qjl else None), cb


@pytest.mark.parametrize("bits,qjl", VARIANTS, ids=IDS)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_compact_records(c128, bits, qjl, dtype):
    """3 streams x 300 tokens of outlier-channel K/V (fused bf16 kernel or fp32
    GEMM path) into compact key and value arrays, stream stride 320."""
    ctx, Pi, S = c128
    ns, n, stride, d = 3, 300, 320, 128
    X = synth.outlier_kv(51, (bits, 1), synth.TAG_SCALES_K, (ns, n, d), dtype)
    keys = tq.Packed(ns * stride, d, bits, True, qjl=qjl, norm_f16=True)
    vals = tq.Packed(ns * stride, d, 3, False, norm_f16=True)
    xd = _dev(X, dtype)
    work = torch.empty(tq.quantize_ws_bytes(ctx, ns, n, True), dtype=torch.uint8, device=DEV)
    tq.quantize_kv(ctx, xd, keys, out_stream_stride=stride, work=work)
    tq.quantize_kv(ctx, xd, vals, out_stream_stride=stride)
    kw, kn = keys.host()
    vw, vn = vals.host()
    assert kn.dtype == np.float16 and vn.dtype == np.float16
    cbv = T.codebook(d, 3)
    for s in range(ns):
        enc, cb = _encode(X[s], Pi, S, bits, qjl)
        P.check_key_records(kw[s * stride:s * stride + n], kn[s * stride:s * stride + n], enc, cb, bits, d, qjl,
                            norm_f16=True)
        encv = T.encode(X[s], Pi, cbv)
        P.check_value_records(vw[s * stride // 32:(s + 1) * stride // 32], vn[s * stride:(s + 1) * stride], encv,
                              cbv, 3, d, n, norm_f16=True)


def _compact_cache(ctx, Pi, S, K, V, seq, bits, qjl, cap):
    """Oracle-packed compact records uploaded into a device cache."""
    B, H, L, d = K.shape
    cbv = T.codebook(d, 3)
    cache = tq.KVCache(B, H, cap, d, bits, 3, key_qjl=qjl, norm_f16=True)
    recs = {}
    cbk = None
    for b in range(B):
        for h in range(H):
            s = b * H + h
            enc, cbk = _encode(K[b, h], Pi, S, bits, qjl)
            pk = T.pack_keys(enc, bits, qjl, norm_f16=True)
            pv = T.pack_values(T.encode(V[b, h], Pi, cbv), 3, norm_f16=True)
            cache.k.words[s * cap:s * cap + L].copy_(torch.from_numpy(pk["bits"].view(np.int32)).to(DEV))
            cache.k.norms[s * cap:s * cap + L].copy_(torch.from_numpy(pk["norms"]).to(DEV))
            nb = pv["bits"].shape[0]
            cache.v.words[s * cap // 32:s * cap // 32 + nb].copy_(torch.from_numpy(pv["bits"].view(np.int32)).to(DEV))
            cache.v.norms[s * cap:s * cap + L].copy_(torch.from_numpy(pv["norms"]).to(DEV))
            recs[s] = (pk, pv)
    cache.seq_len.copy_(torch.tensor(seq, dtype=torch.int32))
    cache.host_max_len = int(max(seq))
    return cache, recs, cbk, cbv


@pytest.mark.parametrize("bits,qjl", VARIANTS, ids=IDS)
def test_attention_over_compact_records(c128, bits, qjl):
    """batch 3 (lengths 1500, 0, 777), 2 KV heads, 8 query heads: decode and a
    causal prefill of 6 positions over compact records within 2e-3 of the
    oracle; scores of 5 queries against one stream's compact keys within the
    score bar."""
    ctx, Pi, S = c128
    B, H, Hq, cap, L, d = 3, 2, 8, 1536, 1500, 128
    seq = [1500, 0, 777]
    K = synth.outlier_kv(52, (bits, 1), synth.TAG_SCALES_K, (B, H, L, d))
    V = synth.outlier_kv(52, (bits, 2), synth.TAG_SCALES_V, (B, H, L, d))
    cache, recs, cbk, cbv = _compact_cache(ctx, Pi, S, K, V, seq, bits, qjl, cap)
    q = synth.gaussian(52, (3,), (B, Hq, d), "bf16")
    qp = synth.gaussian(52, (4,), (B, 6, Hq, d), "bf16")
    scale = 1 / math.sqrt(d)
    out = cache.decode(ctx, _dev(q, "bf16"), scale).cpu().numpy()
    outp = cache.attend(ctx, _dev(qp, "bf16"), True, scale).cpu().numpy()
    g = Hq // H
    for b in range(B):
        for h in range(H):
            pk, pv = recs[b * H + h]
            n = seq[b]
            if n == 0:
                assert not out[b, h * g:(h + 1) * g].any() and not outp[b, :, h * g:(h + 1) * g].any()
                continue
            keys = {"bits": pk["bits"][:n], "norms": pk["norms"][:n]}
            vals = {"bits": pv["bits"], "norms": pv["norms"][:n]}
            ref = T.attention_decode(q[b, h * g:(h + 1) * g], Pi, S, cbk, cbv, keys, vals, n, scale, qjl)
            assert np.max(np.abs(out[b, h * g:(h + 1) * g] - ref)) <= 2e-3, f"decode b={b} h={h}"
            refp = T.attention_prefill(qp[b, :, h * g:(h + 1) * g], Pi, S, cbk, cbv, keys, vals, n, scale, True, qjl)
            assert np.max(np.abs(outp[b, :, h * g:(h + 1) * g] - refp)) <= 2e-3, f"prefill b={b} h={h}"
    # scores over one stream's compact keys (a standalone packed array)
    pk, _ = recs[0]
    arr = tq.Packed(L, d, bits, True, qjl=qjl, norm_f16=True)
    arr.words.copy_(torch.from_numpy(pk["bits"].view(np.int32)).to(DEV))
    arr.norms.copy_(torch.from_numpy(pk["norms"]).to(DEV))
    qs = synth.gaussian(52, (5,), (5, d))
    sc, _, _ = tq.scores(ctx, _dev(qs, "f32"), arr)
    ref = T.scores(qs, Pi, S, cbk, pk, qjl)
    P.check_scores(sc.cpu().numpy(), ref, np.linalg.norm(qs, axis=1), np.linalg.norm(K[0, 0], axis=1))


@pytest.mark.parametrize("fused", [False, True], ids=["append", "step"])
def test_appends_into_compact_cache(c128, fused):
    """Prefill 45 tokens into a compact cache (tq_cache_write), then 20 appends
    or fused steps: appended records match the oracle's encoding; the last fused
    step's output matches the oracle over the cache's records."""
    ctx, Pi, S = c128
    B, H, Hq, cap, L0, NA, d = 2, 2, 8, 96, 45, 20, 128
    K = synth.outlier_kv(53, (1,), synth.TAG_SCALES_K, (B, H, L0 + NA, d), "bf16")
    V = synth.outlier_kv(53, (2,), synth.TAG_SCALES_V, (B, H, L0 + NA, d), "bf16")
    Q = synth.gaussian(53, (3,), (NA, B, Hq, d), "bf16")
    cache = tq.KVCache(B, H, cap, d, 3, 3, norm_f16=True)
    cache.prefill(ctx, _dev(K[:, :, :L0], "bf16").contiguous(), _dev(V[:, :, :L0], "bf16").contiguous())
    out = None
    for t in range(NA):
        ka = _dev(K[:, :, L0 + t], "bf16").contiguous()
        va = _dev(V[:, :, L0 + t], "bf16").contiguous()
        if fused:
            out = cache.decode_step(ctx, ka, va, _dev(Q[t], "bf16"), 1 / math.sqrt(d))
        else:
            cache.append(ctx, ka, va)
    torch.cuda.synchronize()
    kw, kn = cache.k.host()
    vw, vn = cache.v.host()
    cbk, cbv = T.codebook(d, 3), T.codebook(d, 3)
    n = L0 + NA
    for b in range(B):
        for h in range(H):
            s = b * H + h
            enc = T.encode(K[b, h], Pi, cbk, S)
            P.check_key_records(kw[s * cap:s * cap + n], kn[s * cap:s * cap + n], enc, cbk, 3, d, norm_f16=True)
            encv = T.encode(V[b, h], Pi, cbv)
            P.check_value_records(vw[s * cap // 32:(s + 1) * cap // 32], vn[s * cap:(s + 1) * cap], encv, cbv, 3, d,
                                  n, norm_f16=True)
            if fused:
                keys = {"bits": kw[s * cap:s * cap + n], "norms": kn[s * cap:s * cap + n]}
                vals = {"bits": vw[s * cap // 32:(s + 1) * cap // 32], "norms": vn[s * cap:s * cap + n]}
                ref = T.attention_decode(Q[NA - 1, b, h * 4:h * 4 + 4], Pi, S, cbk, cbv, keys, vals, n,
                                         1 / math.sqrt(d))
                assert np.max(np.abs(out.cpu().numpy()[b, h * 4:h * 4 + 4] - ref)) <= 2e-3


def test_compact_paged_equals_contiguous(c128):
    """A compact cache in shuffled 256-token pages equals a contiguous compact
    cache bit for bit: records, decode and fused steps."""
    ctx, _, _ = c128
    B, H, Hq, cap, L, d = 2, 2, 8, 1024, 900, 128
    cols = cap // 256
    perm = np.random.default_rng(54).permutation(B * cols + 2)[:B * cols].astype(np.int32)
    table = torch.from_numpy(perm.reshape(B, cols)).to(DEV)
    K = synth.torch_outlier_kv(54, (1,), synth.TAG_SCALES_K, (B, H, L, d), torch.bfloat16, DEV)
    V = synth.torch_outlier_kv(54, (2,), synth.TAG_SCALES_V, (B, H, L, d), torch.bfloat16, DEV)
    flat = tq.KVCache(B, H, cap, d, 3, 3, norm_f16=True)
    paged = tq.KVCache(B, H, cap, d, 3, 3, norm_f16=True, page_tokens=256, n_pages=B * cols + 2, block_table=table)
    for c in (flat, paged):
        c.prefill(ctx, K, V)
    q = synth.torch_gaussian(54, (3,), (B, Hq, d), torch.bfloat16, DEV)
    assert torch.equal(flat.decode(ctx, q), paged.decode(ctx, q))
    for i in range(2):
        ka = synth.torch_outlier_kv(54, (4, i), synth.TAG_SCALES_K, (B, H, d), torch.bfloat16, DEV)
        va = synth.torch_outlier_kv(54, (5, i), synth.TAG_SCALES_V, (B, H, d), torch.bfloat16, DEV)
        assert torch.equal(flat.decode_step(ctx, ka, va, q), paged.decode_step(ctx, ka, va, q))
    fk, fn = flat.k.host()
    pk_, pn = paged.k.host()
    th = table.cpu().numpy()
    for b in range(B):
        for h in range(H):
            t = np.arange(L + 2)
            ridx = (th[b, t // 256].astype(np.int64) * H + h) * 256 + t % 256
            s = b * H + h
            assert np.array_equal(fk[s * cap:s * cap + L + 2], pk_[ridx])
            assert np.array_equal(fn[s * cap:s * cap + L + 2], pn[ridx])
