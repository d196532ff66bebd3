"""GPU parity of the key-format variants: MSE-only keys (stage 1 alone, the
codes and ||k||) and pure QJL keys (no code bits: the sign word of the sketched
rotated unit vector and both norms). Quantize (fused d = 128 bf16 kernel and the
GEMM path), standalone append, fused decode step, decode attention and scores
are compared with the oracle on the same records, at the parity bar of the
full TurboQuant keys."""
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
# (MSE bits, QJL): MSE-only keys at 2 and 3 bits, pure QJL keys
VARIANTS = [(2, False), (3, False), (0, True)]
IDS = ["mse2", "mse3", "qjl"]


def _ctx(d, seed=0):
    ctx = tq.Context(d, seed)
    Pi = T.rotation_from_gaussian(synth.gaussian_matrix(seed, synth.TAG_ROTATION, d, d))
    S = T.sketch_from_gaussian(synth.gaussian_matrix(seed, synth.TAG_SKETCH, d, d))
    return ctx, Pi, S


@pytest.fixture(scope="module")
def c128():
    return _ctx(128)


@pytest.fixture(scope="module")
def c256():
    return _ctx(256, seed=3)


def _dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def _encode(X, Pi, S, bits, qjl):
    cb = T.codebook(Pi.shape[0], bits) if bits > 0 else None
    return T.encode(X, Pi, cb, S if qjl else None), cb


def _upload(packed, words, norms):
    packed.words[:words.shape[0]].copy_(torch.from_numpy(np.ascontiguousarray(words).view(np.int32)).to(DEV))
    packed.norms[:norms.shape[0]].copy_(torch.from_numpy(np.ascontiguousarray(norms)).to(DEV))


@pytest.mark.parametrize("bits,qjl", VARIANTS, ids=IDS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_key_variants(c128, bits, qjl, dtype):
    """3 streams x 333 tokens (ragged tiles) at offset 17 of 400-record streams;
    records outside the written ranges stay zero. bf16 takes the fused kernel,
    fp32 the GEMM path."""
    ctx, Pi, S = c128
    X = synth.outlier_kv(2, (bits, int(qjl)), synth.TAG_SCALES_K, (3, 333, 128), "bf16") if dtype == "bf16" else \
        synth.gaussian(2, (bits, int(qjl)), (3, 333, 128))
    X[1, 5] = 0.0  # a zero vector
    out = tq.Packed(3 * 400, 128, bits, True, qjl=qjl)
    tq.quantize_kv(ctx, _dev(X, dtype), out, out_stream_stride=400, out_offset=17)
    torch.cuda.synchronize()
    words, norms = out.host()
    assert words.shape == (1200, 4, bits + int(qjl)) and norms.shape == (1200, 1 + int(qjl))
    for s in range(3):
        enc, cb = _encode(X[s], Pi, S, bits, qjl)
        sl = slice(s * 400 + 17, s * 400 + 17 + 333)
        P.check_key_records(words[sl], norms[sl], enc, cb, bits, 128, qjl)
        untouched = np.r_[s * 400:s * 400 + 17, s * 400 + 350:(s + 1) * 400]
        assert not words[untouched].any() and not norms[untouched].any()
    assert not words[400 + 17 + 5].any() and not norms[400 + 17 + 5].any()


@pytest.mark.parametrize("bits,qjl", VARIANTS, ids=IDS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_key_variants_d256(c256, bits, qjl, dtype):
    """d = 256 (the GEMM path for both input types), 2 streams x 200 tokens."""
    ctx, Pi, S = c256
    X = synth.gaussian(3, (bits, int(qjl)), (2, 200, 256))
    if dtype == "bf16":
        X = torch.from_numpy(X).to(torch.bfloat16).float().numpy()
    out = tq.Packed(2 * 200, 256, bits, True, qjl=qjl)
    tq.quantize_kv(ctx, _dev(X, dtype), out)
    torch.cuda.synchronize()
    words, norms = out.host()
    for s in range(2):
        enc, cb = _encode(X[s], Pi, S, bits, qjl)
        sl = slice(s * 200, (s + 1) * 200)
        P.check_key_records(words[sl], norms[sl], enc, cb, bits, 256, qjl)


def _oracle_cache(K, V, Pi, S, bits, qjl, vbits, cap):
    B, H, L, d = K.shape
    cbv = T.codebook(d, vbits)
    kw = np.zeros((B * H * cap, d // 32, bits + int(qjl)), np.uint32)
    kn = np.zeros((B * H * cap, 1 + int(qjl)), np.float32)
    vw = np.zeros((B * H * cap // 32, d, vbits), np.uint32)
    vn = np.zeros((B * H * cap,), np.float32)
    cbk = None
    for b in range(B):
        for h in range(H):
            s = b * H + h
            enc, cbk = _encode(K[b, h], Pi, S, bits, qjl)
            pk = T.pack_keys(enc, bits, qjl)
            pv = T.pack_values(T.encode(V[b, h], Pi, cbv), vbits)
            kw[s * cap:s * cap + L] = pk["bits"]
            kn[s * cap:s * cap + L] = pk["norms"]
            vw[s * cap // 32:s * cap // 32 + pv["bits"].shape[0]] = pv["bits"]
            vn[s * cap:s * cap + L] = pv["norms"]
    return cbk, cbv, kw, kn, vw, vn


@pytest.mark.parametrize("bits,qjl", VARIANTS, ids=IDS)
def test_decode_key_variants(c128, bits, qjl):
    """batch 3 (lengths 1500, 0, 777), 2 KV heads, 8 query heads (groups of 4),
    outlier-channel bf16 K/V, 3-bit values: attention within 2e-3 max-abs of the
    oracle over the same records."""
    ctx, Pi, S = c128
    cap, L = 1536, 1500
    seq = [1500, 0, 777]
    K = synth.outlier_kv(8, (bits, 1), synth.TAG_SCALES_K, (3, 2, L, 128))
    V = synth.outlier_kv(8, (bits, 2), synth.TAG_SCALES_V, (3, 2, L, 128))
    Q = synth.outlier_kv(8, (bits, 3), synth.TAG_SCALES_K, (3, 8, 128))
    cbk, cbv, kw, kn, vw, vn = _oracle_cache(K, V, Pi, S, bits, qjl, 3, cap)
    cache = tq.KVCache(3, 2, cap, 128, bits, 3, key_qjl=qjl)
    _upload(cache.k, kw, kn)
    _upload(cache.v, vw, vn)
    cache.seq_len.copy_(torch.tensor(seq, dtype=torch.int32))
    cache.host_max_len = max(seq)
    scale = 1.0 / math.sqrt(128)
    out = cache.decode(ctx, _dev(Q, "bf16"), scale).cpu().numpy()
    for b in range(3):
        for h in range(2):
            s, Lb = b * 2 + h, seq[b]
            if Lb == 0:
                assert not out[b, 4 * h:4 * h + 4].any()
                continue
            keys = {"bits": kw[s * cap:s * cap + Lb], "norms": kn[s * cap:s * cap + Lb]}
            vals = {"bits": vw[s * cap // 32:(s + 1) * cap // 32], "norms": vn[s * cap:s * cap + Lb]}
            ref = T.attention_decode(Q[b, 4 * h:4 * h + 4], Pi, S, cbk, cbv, keys, vals, Lb, scale, qjl)
            assert np.max(np.abs(out[b, 4 * h:4 * h + 4] - ref)) <= 2e-3, f"b={b} h={h}"


@pytest.mark.parametrize("bits,qjl", VARIANTS, ids=IDS)
@pytest.mark.parametrize("fused", [False, True], ids=["append", "step"])
def test_append_key_variants(c128, bits, qjl, fused):
    """Prefill 45 tokens, then 20 appends (tq_append_token) or 20 fused decode steps
    (tq_decode_step): appended key records match the oracle's encoding of the new
    tokens; the fused step's output at the last step matches the oracle over the
    cache's records."""
    ctx, Pi, S = c128
    B, H, cap, L0, NA, hq = 2, 2, 96, 45, 20, 8
    K = synth.outlier_kv(9, (bits, 1), synth.TAG_SCALES_K, (B, H, L0 + NA, 128), "bf16")
    V = synth.outlier_kv(9, (bits, 2), synth.TAG_SCALES_V, (B, H, L0 + NA, 128), "bf16")
    Q = synth.outlier_kv(9, (bits, 3), synth.TAG_SCALES_K, (NA, B, hq, 128), "bf16")
    cbk, cbv, kw, kn, vw, vn = _oracle_cache(K[:, :, :L0], V[:, :, :L0], Pi, S, bits, qjl, 3, cap)
    cache = tq.KVCache(B, H, cap, 128, bits, 3, key_qjl=qjl)
    _upload(cache.k, kw, kn)
    _upload(cache.v, vw, vn)
    cache.seq_len.fill_(L0)
    cache.host_max_len = L0
    scale = 1.0 / math.sqrt(128)
    out = None
    for t in range(NA):
        k = _dev(K[:, :, L0 + t], "bf16").contiguous()
        v = _dev(V[:, :, L0 + t], "bf16").contiguous()
        if fused:
            out = cache.decode_step(ctx, k, v, _dev(Q[t], "bf16").contiguous(), scale)
        else:
            cache.append(ctx, k, v)
    torch.cuda.synchronize()
    assert cache.seq_len.cpu().tolist() == [L0 + NA] * B and cache.host_max_len == L0 + NA
    gkw, gkn = cache.k.host()
    gvw, gvn = cache.v.host()
    n = L0 + NA
    for s in range(B * H):
        b, h = divmod(s, H)
        assert np.array_equal(gkw[s * cap:s * cap + L0], kw[s * cap:s * cap + L0])
        enc, cb = _encode(K[b, h, L0:], Pi, S, bits, qjl)
        P.check_key_records(gkw[s * cap + L0:s * cap + n], gkn[s * cap + L0:s * cap + n], enc, cb, bits, 128, qjl)
        if fused:
            keys = {"bits": gkw[s * cap:s * cap + n], "norms": gkn[s * cap:s * cap + n]}
            vals = {"bits": gvw[s * cap // 32:(s + 1) * cap // 32], "norms": gvn[s * cap:s * cap + n]}
            g = hq // H
            ref = T.attention_decode(Q[NA - 1, b, h * g:(h + 1) * g], Pi, S, cbk, cbv, keys, vals, n, scale, qjl)
            assert np.max(np.abs(out.cpu().numpy()[b, h * g:(h + 1) * g] - ref)) <= 2e-3


@pytest.mark.parametrize("bits,qjl", VARIANTS, ids=IDS)
def test_scores_key_variants(c128, bits, qjl):
    """tq_scores of 16 fp32 queries against 1000 packed keys of each variant, and
    their top-10, against the oracle's scores of the same records."""
    ctx, Pi, S = c128
    X = synth.gaussian(6, (bits, 1), (1000, 128))
    Qv = synth.gaussian(6, (bits, 2), (16, 128))
    keys = tq.Packed(1000, 128, bits, True, qjl=qjl)
    tq.quantize_kv(ctx, _dev(X, "f32"), keys)
    sc, ti, tv = tq.scores(ctx, _dev(Qv, "f32"), keys, want_scores=True, topk=10)
    torch.cuda.synchronize()
    words, norms = keys.host()
    cb = T.codebook(128, bits) if bits > 0 else None
    ref = T.scores(Qv, Pi, S, cb, {"bits": words, "norms": norms}, qjl)
    qn, xn = np.linalg.norm(Qv, axis=1), np.linalg.norm(X, axis=1)
    P.check_scores(sc.cpu().numpy(), ref, qn, xn)
    P.check_topk(ti.cpu().numpy(), tv.cpu().numpy(), ref, 10, qn, xn)
