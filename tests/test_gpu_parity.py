"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Encode tests compare GPU-packed records with the oracle's encoding of the same
inputs (bit-exact up to the boundary band). Score, top-k and attention tests
run the GPU kernels on oracle-packed bytes uploaded to the device, so both
sides see identical packed data.
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


def _ctx_and_oracle(d, seed=0):
    ctx = tq.Context(d, seed)
    Pi = T.rotation_from_gaussian(synth.gaussian_matrix(seed, synth.TAG_ROTATION, d, d))
    S = T.sketch_from_gaussian(synth.gaussian_matrix(seed, synth.TAG_SKETCH, d, d))
    return ctx, Pi, S


@pytest.fixture(scope="module")
def c128():
    return _ctx_and_oracle(128)


@pytest.fixture(scope="module")
def c1536():
    return _ctx_and_oracle(1536)


def _dev(x_f32, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32)).to(DEV)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def _upload(packed, words, norms, rec0=0):
    w = torch.from_numpy(np.ascontiguousarray(words).view(np.int32)).to(DEV)
    nrm = torch.from_numpy(np.ascontiguousarray(norms)).to(DEV)
    packed.words[rec0:rec0 + w.shape[0]].copy_(w)
    packed.norms[rec0:rec0 + nrm.shape[0]].copy_(nrm)


# ---------------------------------------------------------------------------
# setup tables
# ---------------------------------------------------------------------------

def test_context_tables_match_oracle(c128):
    ctx, Pi, S = c128
    rot, sk = ctx.export()
    assert np.max(np.abs(rot.view(np.int32).astype(np.int64) - Pi.view(np.int32))) <= 1
    assert np.array_equal(sk, S)
    for b in (1, 2, 3, 4):
        cb = ctx.codebook(b)
        o = T.codebook(128, b)
        assert np.array_equal(cb.centroids, o.centroids) and np.array_equal(cb.boundaries, o.boundaries)


# ---------------------------------------------------------------------------
# quantize
# ---------------------------------------------------------------------------

def test_quantize_keys_tiny_reference(c128):
    """4096 fp32 N(0,1) keys, d = 128, b = 3 (2-bit Lloyd-Max + 1-bit QJL), seed 0."""
    ctx, Pi, S = c128
    X = synth.gaussian(0, (0, synth.TAG_KEYS), (4096, 128))
    out = tq.Packed(4096, 128, 2, True)
    tq.quantize_kv(ctx, _dev(X, "f32"), out)
    torch.cuda.synchronize()
    words, norms = out.host()
    cb = T.codebook(128, 2)
    P.check_key_records(words, norms, T.encode(X, Pi, cb, S), cb, 2, 128)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_keys_streams_offsets(c128, bits, dtype):
    """3 streams x 333 tokens (ragged tiles), written at offset 17 of 400-record streams;
    records outside the written ranges must stay untouched (zero)."""
    ctx, Pi, S = c128
    X = synth.outlier_kv(1, (bits, 7), synth.TAG_SCALES_K, (3, 333, 128), "bf16") if dtype == "bf16" else \
        synth.gaussian(1, (bits, 7), (3, 333, 128))
    out = tq.Packed(3 * 400, 128, bits, True)
    tq.quantize_kv(ctx, _dev(X, dtype), out, out_stream_stride=400, out_offset=17)
    torch.cuda.synchronize()
    words, norms = out.host()
    cb = T.codebook(128, bits)
    for s in range(3):
        enc = T.encode(X[s], Pi, cb, S)
        sl = slice(s * 400 + 17, s * 400 + 17 + 333)
        P.check_key_records(words[sl], norms[sl], enc, cb, bits, 128)
        untouched = np.r_[s * 400:s * 400 + 17, s * 400 + 350:(s + 1) * 400]
        assert not words[untouched].any() and not norms[untouched].any()


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_values_token_major(c128, bits, dtype):
    ctx, Pi, S = c128
    X = synth.outlier_kv(2, (bits, 8), synth.TAG_SCALES_V, (2, 333, 128), "bf16") if dtype == "bf16" else \
        synth.gaussian(2, (bits, 8), (2, 333, 128))
    out = tq.Packed(2 * 416, 128, bits, False)
    tq.quantize_kv(ctx, _dev(X, dtype), out, out_stream_stride=416, out_offset=32)
    torch.cuda.synchronize()
    words, norms = out.host()
    cb = T.codebook(128, bits)
    for s in range(2):
        enc = T.encode(X[s], Pi, cb)
        b0 = (s * 416 + 32) // 32
        nb = (333 + 31) // 32
        P.check_value_records(words[b0:b0 + nb], norms[s * 416 + 32:s * 416 + 32 + 333], enc, cb, bits, 128, 333)
        assert not words[s * 13:b0].any() and not words[b0 + nb:(s + 1) * 13].any()
        assert not norms[s * 416:s * 416 + 32].any()


def test_zero_vectors_give_zero_records(c128):
    ctx, Pi, S = c128
    X = synth.gaussian(3, (1,), (64, 128))
    X[[0, 5, 63]] = 0.0
    kp = tq.Packed(64, 128, 3, True)
    vp = tq.Packed(64, 128, 3, False)
    tq.quantize_kv(ctx, _dev(X, "f32"), kp)
    tq.quantize_kv(ctx, _dev(X, "f32"), vp)
    torch.cuda.synchronize()
    kw, kn = kp.host()
    assert not kw[[0, 5, 63]].any() and not kn[[0, 5, 63]].any()
    cb = T.codebook(128, 3)
    P.check_key_records(kw, kn, T.encode(X, Pi, cb, S), cb, 3, 128)
    vw, vn = vp.host()
    P.check_value_records(vw, vn, T.encode(X, Pi, cb), cb, 3, 128, 64)


def test_quantize_empty_call_is_a_no_op(c128):
    ctx, _, _ = c128
    out = tq.Packed(32, 128, 3, True)
    x = torch.zeros((0, 128), device=DEV)
    tq.quantize_kv(ctx, x, out, n_tokens=0)
    torch.cuda.synchronize()
    assert not out.words.any()


def test_quantize_keys_d1536(c1536):
    ctx, Pi, S = c1536
    X = synth.unit_gaussian(4, (synth.TAG_DB,), (1500, 1536))
    out = tq.Packed(1500, 1536, 3, True)
    tq.quantize_kv(ctx, _dev(X, "f32"), out)
    torch.cuda.synchronize()
    words, norms = out.host()
    cb = T.codebook(1536, 3)
    P.check_key_records(words, norms, T.encode(X, Pi, cb, S), cb, 3, 1536)


# ---------------------------------------------------------------------------
# scores and top-k on identical packed bytes
# ---------------------------------------------------------------------------

def _packed_keys(X, Pi, S, bits):
    cb = T.codebook(Pi.shape[0], bits)
    enc = T.encode(X, Pi, cb, S)
    return cb, enc, T.pack_keys(enc, bits)


def test_scores_tiny_reference(c128):
    """16 fp32 queries against the 4096 packed keys: 16 x 4096 estimated q.k."""
    ctx, Pi, S = c128
    X = synth.gaussian(0, (0, synth.TAG_KEYS), (4096, 128))
    Qv = synth.gaussian(0, (0, synth.TAG_QUERIES), (16, 128))
    cb, enc, pk = _packed_keys(X, Pi, S, 2)
    kp = tq.Packed(4096, 128, 2, True)
    _upload(kp, pk["bits"], pk["norms"])
    sc, _, _ = tq.scores(ctx, _dev(Qv, "f32"), kp)
    torch.cuda.synchronize()
    ref = T.scores(Qv, Pi, S, cb, pk)
    P.check_scores(sc.cpu().numpy(), ref, np.linalg.norm(Qv, axis=1), enc.norm)


@pytest.mark.parametrize("k", [10, 33])
def test_topk_matches_oracle(c128, k):
    ctx, Pi, S = c128
    X = synth.unit_gaussian(5, (1,), (20000, 128))
    Qv = synth.unit_gaussian(5, (2,), (37, 128))
    cb, enc, pk = _packed_keys(X, Pi, S, 3)
    kp = tq.Packed(20000, 128, 3, True)
    _upload(kp, pk["bits"], pk["norms"])
    sc, ti, tv = tq.scores(ctx, _dev(Qv, "f32"), kp, want_scores=False, topk=k)
    torch.cuda.synchronize()
    assert sc is None
    ref = T.scores(Qv, Pi, S, cb, pk)
    P.check_topk(ti.cpu().numpy(), tv.cpu().numpy(), ref, k, np.linalg.norm(Qv, axis=1), enc.norm)


def test_scores_and_topk_d1536(c1536):
    ctx, Pi, S = c1536
    X = synth.unit_gaussian(6, (synth.TAG_DB,), (5000, 1536))
    Qv = synth.unit_gaussian(6, (synth.TAG_QUERIES,), (40, 1536))
    cb, enc, pk = _packed_keys(X, Pi, S, 3)
    kp = tq.Packed(5000, 1536, 3, True)
    _upload(kp, pk["bits"], pk["norms"])
    sc, ti, tv = tq.scores(ctx, _dev(Qv, "f32"), kp, want_scores=True, topk=10)
    torch.cuda.synchronize()
    ref = T.scores(Qv, Pi, S, cb, pk)
    qn = np.linalg.norm(Qv, axis=1)
    P.check_scores(sc.cpu().numpy(), ref, qn, enc.norm)
    P.check_topk(ti.cpu().numpy(), tv.cpu().numpy(), ref, 10, qn, enc.norm)


# ---------------------------------------------------------------------------
# decode attention on identical packed bytes
# ---------------------------------------------------------------------------

def _oracle_cache(K, V, Pi, S, kbits, vbits, cap):
    """K, V: [B, H, L, d] (L <= cap). Oracle-packed arrays in the cache layout."""
    B, H, L, d = K.shape
    cbk, cbv = T.codebook(d, kbits), T.codebook(d, vbits)
    kw = np.zeros((B * H * cap, d // 32, kbits + 1), np.uint32)
    kn = np.zeros((B * H * cap, 2), np.float32)
    vw = np.zeros((B * H * cap // 32, d, vbits), np.uint32)
    vn = np.zeros((B * H * cap,), np.float32)
    for b in range(B):
        for h in range(H):
            s = b * H + h
            pk = T.pack_keys(T.encode(K[b, h], Pi, cbk, S), kbits)
            pv = T.pack_values(T.encode(V[b, h], Pi, cbv), vbits)
            kw[s * cap:s * cap + L] = pk["bits"]
            kn[s * cap:s * cap + L] = pk["norms"]
            vw[s * cap // 32:s * cap // 32 + pv["bits"].shape[0]] = pv["bits"]
            vn[s * cap:s * cap + L] = pv["norms"]
    return cbk, cbv, kw, kn, vw, vn


def _run_decode_case(ctx, Pi, S, K, V, Q, seq, kbits, vbits, cap, qdtype="bf16"):
    B, H, L, d = K.shape
    Hq = Q.shape[1]
    g = Hq // H
    cbk, cbv, kw, kn, vw, vn = _oracle_cache(K, V, Pi, S, kbits, vbits, cap)
    cache = tq.KVCache(B, H, cap, d, kbits, vbits)
    _upload(cache.k, kw, kn)
    _upload(cache.v, vw, vn)
    cache.seq_len.copy_(torch.tensor(seq, dtype=torch.int32))
    cache.host_max_len = int(max(seq))
    scale = 1.0 / math.sqrt(d)
    out = cache.decode(ctx, _dev(Q, qdtype), scale).cpu().numpy()
    torch.cuda.synchronize()
    worst = 0.0
    for b in range(B):
        for h in range(H):
            s = b * H + h
            Lb = seq[b]
            qh = Q[b, h * g:(h + 1) * g]
            if Lb == 0:
                assert not out[b, h * g:(h + 1) * g].any()
                continue
            keys = {"bits": kw[s * cap:s * cap + Lb], "norms": kn[s * cap:s * cap + Lb]}
            vals = {"bits": vw[s * cap // 32:(s * cap + cap) // 32], "norms": vn[s * cap:s * cap + Lb]}
            ref = T.attention_decode(qh, Pi, S, cbk, cbv, keys, vals, Lb, scale)
            err = np.max(np.abs(out[b, h * g:(h + 1) * g] - ref))
            worst = max(worst, err)
            assert err <= 2e-3, f"decode mismatch b={b} h={h}: {err}"
    return worst


def test_decode_single_head_32k(c128):
    """Single-head decode: context 32768, outlier-channel bf16 K/V, b = 4 keys,
    3-bit values, one bf16 query, softmax(q K^T / sqrt(128)) V."""
    ctx, Pi, S = c128
    L = 32768
    K = synth.outlier_kv(0, (1, synth.TAG_KEYS), synth.TAG_SCALES_K, (1, 1, L, 128))
    V = synth.outlier_kv(0, (1, synth.TAG_VALUES), synth.TAG_SCALES_V, (1, 1, L, 128))
    Q = synth.outlier_kv(0, (1, synth.TAG_QUERIES), synth.TAG_SCALES_K, (1, 1, 128))
    _run_decode_case(ctx, Pi, S, K, V, Q, [L], 3, 3, L)


@pytest.mark.parametrize("kbits,vbits", [(2, 3), (3, 3), (3, 2), (1, 1), (4, 4)])
def test_decode_gqa_ragged(c128, kbits, vbits):
    """batch 3 (lengths 2000, 0, 777), 2 KV heads, 8 query heads (groups of 4)."""
    ctx, Pi, S = c128
    cap, L = 2048, 2000
    K = synth.outlier_kv(7, (kbits, 1), synth.TAG_SCALES_K, (3, 2, L, 128))
    V = synth.outlier_kv(7, (kbits, 2), synth.TAG_SCALES_V, (3, 2, L, 128))
    Q = synth.outlier_kv(7, (kbits, 3), synth.TAG_SCALES_K, (3, 8, 128))
    _run_decode_case(ctx, Pi, S, K, V, Q, [2000, 0, 777], kbits, vbits, cap)


@pytest.mark.parametrize("kbits", [3, 1])
def test_decode_full_cache_partial_chunk(c128, kbits):
    """The last sequence fills its cache (capacity 1056 = a 1024-token chunk + 32):
    the key loads of its last chunk (range-checked over the chunk's records) sit at
    the very end of the key, norm and value arrays; the other sequence ends at 1000
    tokens. b = kbits + 1 keys (records of 4 and 2 words per 32 coordinates), 3-bit
    values."""
    ctx, Pi, S = c128
    cap = 1056
    K = synth.outlier_kv(8, (kbits, 1), synth.TAG_SCALES_K, (2, 2, cap, 128))
    V = synth.outlier_kv(8, (kbits, 2), synth.TAG_SCALES_V, (2, 2, cap, 128))
    Q = synth.outlier_kv(8, (kbits, 3), synth.TAG_SCALES_K, (2, 8, 128))
    _run_decode_case(ctx, Pi, S, K, V, Q, [1000, cap], kbits, 3, cap)


def test_decode_uniform_softmax_long_context(c128):
    """A query of zero gives every token the same weight, so the output is the
    mean of the dequantized values over the whole context: the case where each
    chunk's value sums cancel the most (2 M_S - W for every Walsh mask, formed in
    fp32 from exact int32 digit sums). 3000 tokens (three chunks), outlier-channel
    V; the other heads of the group keep outlier-channel queries."""
    ctx, Pi, S = c128
    cap, L = 3072, 3000
    K = synth.outlier_kv(9, (1,), synth.TAG_SCALES_K, (1, 2, L, 128))
    V = synth.outlier_kv(9, (2,), synth.TAG_SCALES_V, (1, 2, L, 128))
    Q = np.array(synth.outlier_kv(9, (3,), synth.TAG_SCALES_K, (1, 8, 128)))
    Q[:, 0::2] = 0.0
    worst = _run_decode_case(ctx, Pi, S, K, V, Q, [L], 3, 3, cap)
    print(f"uniform softmax: max-abs error {worst:.2e}")


@pytest.mark.parametrize("L", [4096, 4097])
def test_decode_merge_group_boundary(c128, L):
    """Two KV streams give 256-token chunks: 4096 tokens are 16 chunks (the merge's
    two chunk groups of 8) and 4097 tokens 17 chunks (four groups, the last chunk
    one token)."""
    ctx, Pi, S = c128
    cap = 4352
    K = synth.outlier_kv(10, (L, 1), synth.TAG_SCALES_K, (1, 2, L, 128))
    V = synth.outlier_kv(10, (L, 2), synth.TAG_SCALES_V, (1, 2, L, 128))
    Q = synth.outlier_kv(10, (L, 3), synth.TAG_SCALES_K, (1, 8, 128))
    _run_decode_case(ctx, Pi, S, K, V, Q, [L], 3, 3, cap)


@pytest.mark.parametrize("hq,qdtype", [(2, "f32"), (4, "bf16"), (16, "f32"), (32, "bf16")])
def test_decode_group_sizes_gaussian(c128, hq, qdtype):
    """Gaussian K/V; 2 KV heads with query groups of 1, 2, 8 and 16 heads."""
    ctx, Pi, S = c128
    cap = 1024
    K = synth.gaussian(8, (hq, 1), (2, 2, 999, 128), "bf16")
    V = synth.gaussian(8, (hq, 2), (2, 2, 999, 128), "bf16")
    Q = synth.gaussian(8, (hq, 3), (2, hq, 128), qdtype)
    _run_decode_case(ctx, Pi, S, K, V, Q, [999, 640], 3, 3, cap, qdtype)


# ---------------------------------------------------------------------------
# append
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_append_tokens(c128, dtype):
    """Prefill 37 oracle-packed tokens, append 40 tokens one at a time on the GPU:
    appended records match the oracle's encoding, earlier records (including the
    other bits of a shared token-major value word) are untouched, lengths advance."""
    ctx, Pi, S = c128
    B, H, cap, L0, NA = 2, 2, 96, 37, 40
    K = synth.outlier_kv(9, (1,), synth.TAG_SCALES_K, (B, H, L0 + NA, 128), dtype)
    V = synth.outlier_kv(9, (2,), synth.TAG_SCALES_V, (B, H, L0 + NA, 128), dtype)
    cbk, cbv, kw, kn, vw, vn = _oracle_cache(K[:, :, :L0], V[:, :, :L0], Pi, S, 3, 3, cap)
    cache = tq.KVCache(B, H, cap, 128, 3, 3)
    _upload(cache.k, kw, kn)
    _upload(cache.v, vw, vn)
    cache.seq_len.fill_(L0)
    cache.host_max_len = L0
    for t in range(NA):
        cache.append(ctx, _dev(K[:, :, L0 + t], dtype).contiguous(), _dev(V[:, :, L0 + t], dtype).contiguous())
    torch.cuda.synchronize()
    assert cache.seq_len.cpu().tolist() == [L0 + NA] * B and cache.host_max_len == L0 + NA
    gkw, gkn = cache.k.host()
    gvw, gvn = cache.v.host()
    _, _, kw2, kn2, vw2, vn2 = _oracle_cache(K, V, Pi, S, 3, 3, cap)
    for s in range(B * H):
        b, h = divmod(s, H)
        assert np.array_equal(gkw[s * cap:s * cap + L0], kw[s * cap:s * cap + L0])
        enc_k = T.encode(K[b, h, L0:], Pi, cbk, S)
        P.check_key_records(gkw[s * cap + L0:s * cap + L0 + NA], gkn[s * cap + L0:s * cap + L0 + NA], enc_k, cbk, 3, 128)
        g_idx = T.unpack_values(gvw[s * cap // 32:(s + 1) * cap // 32], 128, 3, L0 + NA)
        o_idx = T.unpack_values(vw2[s * cap // 32:(s + 1) * cap // 32], 128, 3, L0 + NA)
        assert np.array_equal(g_idx[:L0], o_idx[:L0])
        enc_v = T.encode(V[b, h, L0:], Pi, cbv)
        P.check_codes(g_idx[L0:], enc_v, cbv, "appended value codes")
        assert np.all(np.abs(gvn[s * cap + L0:s * cap + L0 + NA] - enc_v.norm) <= 2e-6 * enc_v.norm)


@pytest.mark.parametrize("dtype,hq", [("bf16", 8), ("f32", 4)])
def test_decode_step_appends_and_attends(c128, dtype, hq):
    """Fused serving step: prefill 37 oracle-packed tokens, then 40 decode steps
    (append one token per sequence and attend with it). Appended records match
    the oracle's encoding, lengths advance, and sampled steps' outputs match the
    oracle attention over the records the cache holds after that step."""
    ctx, Pi, S = c128
    B, H, cap, L0, NA = 2, 2, 96, 37, 40
    g = hq // H
    K = synth.outlier_kv(11, (1,), synth.TAG_SCALES_K, (B, H, L0 + NA, 128), dtype)
    V = synth.outlier_kv(11, (2,), synth.TAG_SCALES_V, (B, H, L0 + NA, 128), dtype)
    Q = synth.outlier_kv(11, (3,), synth.TAG_SCALES_K, (NA, B, hq, 128), dtype)
    cbk, cbv, kw, kn, vw, vn = _oracle_cache(K[:, :, :L0], V[:, :, :L0], Pi, S, 3, 3, cap)
    cache = tq.KVCache(B, H, cap, 128, 3, 3)
    _upload(cache.k, kw, kn)
    _upload(cache.v, vw, vn)
    cache.seq_len.fill_(L0)
    cache.host_max_len = L0
    scale = 1.0 / math.sqrt(128)
    ws = torch.empty(cache.decode_step_ws_bytes(ctx, hq) + 1024, dtype=torch.uint8, device=DEV)
    for t in range(NA):
        out = cache.decode_step(ctx, _dev(K[:, :, L0 + t], dtype).contiguous(), _dev(V[:, :, L0 + t], dtype).contiguous(),
                                _dev(Q[t], dtype).contiguous(), scale, ws=ws)
        if t not in (0, 17, NA - 1):
            continue
        o = out.cpu().numpy()
        gkw, gkn = cache.k.host()
        gvw, gvn = cache.v.host()
        n = L0 + t + 1
        assert cache.seq_len.cpu().tolist() == [n] * B
        for s in range(B * H):
            b, h = divmod(s, H)
            keys = {"bits": gkw[s * cap:s * cap + n], "norms": gkn[s * cap:s * cap + n]}
            vals = {"bits": gvw[s * cap // 32:(s + 1) * cap // 32], "norms": gvn[s * cap:s * cap + n]}
            ref = T.attention_decode(Q[t, b, h * g:(h + 1) * g], Pi, S, cbk, cbv, keys, vals, n, scale)
            assert np.max(np.abs(o[b, h * g:(h + 1) * g] - ref)) <= 2e-3, f"step {t} b={b} h={h}"
    torch.cuda.synchronize()
    assert cache.seq_len.cpu().tolist() == [L0 + NA] * B and cache.host_max_len == L0 + NA
    gkw, gkn = cache.k.host()
    gvw, gvn = cache.v.host()
    for s in range(B * H):
        b, h = divmod(s, H)
        assert np.array_equal(gkw[s * cap:s * cap + L0], kw[s * cap:s * cap + L0])
        enc_k = T.encode(K[b, h, L0:], Pi, cbk, S)
        P.check_key_records(gkw[s * cap + L0:s * cap + L0 + NA], gkn[s * cap + L0:s * cap + L0 + NA], enc_k, cbk, 3, 128)
        g_idx = T.unpack_values(gvw[s * cap // 32:(s + 1) * cap // 32], 128, 3, L0 + NA)
        enc_v = T.encode(V[b, h, L0:], Pi, cbv)
        P.check_codes(g_idx[L0:], enc_v, cbv, "appended value codes")
        assert np.all(np.abs(gvn[s * cap + L0:s * cap + L0 + NA] - enc_v.norm) <= 2e-6 * enc_v.norm)


def test_decode_kernel_timing_events(c128):
    """tq_time_next_decode: the armed events bracket the score/attention kernel of
    the next decode call only (inside that call's own time), and the output is the
    same as an unarmed call's."""
    ctx, _, _ = c128
    B, H, hq, cap, L = 2, 2, 8, 2048, 2000
    K = synth.outlier_kv(12, (1,), synth.TAG_SCALES_K, (B, H, L, 128), "bf16")
    V = synth.outlier_kv(12, (2,), synth.TAG_SCALES_V, (B, H, L, 128), "bf16")
    Q = synth.outlier_kv(12, (3,), synth.TAG_SCALES_K, (B, hq, 128), "bf16")
    cache = tq.KVCache(B, H, cap, 128, 3, 3)
    tq.quantize_kv(ctx, _dev(K, "bf16").view(B * H, L, 128), cache.k, out_stream_stride=cap,
                   work=torch.empty(tq.quantize_ws_bytes(ctx, B * H, L, True), dtype=torch.uint8, device=DEV))
    tq.quantize_kv(ctx, _dev(V, "bf16").view(B * H, L, 128), cache.v, out_stream_stride=cap)
    cache.seq_len.fill_(L)
    cache.host_max_len = L
    q = _dev(Q, "bf16").contiguous()
    ref = cache.decode(ctx, q).clone()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    ev[0].record()
    tq.time_next_decode(ev[1], ev[2])
    out = cache.decode(ctx, q)
    ev[3].record()
    torch.cuda.synchronize()
    kern, call = ev[1].elapsed_time(ev[2]), ev[0].elapsed_time(ev[3])
    assert 0.0 < kern <= call
    assert torch.equal(out, ref)
    # the thread is disarmed: the next call records nothing into these events
    e_end = ev[2].elapsed_time(ev[3])
    cache.decode(ctx, q)
    torch.cuda.synchronize()
    assert ev[2].elapsed_time(ev[3]) == e_end


def test_read_probe_reads_everything():
    """The read-bandwidth probe touches every 16-byte granule: the XOR of the
    per-thread folds equals the XOR of all words of the buffer."""
    g = 40
    src = torch.randint(-2**31, 2**31 - 1, (1000 * 4 + 4 * 7,), dtype=torch.int32, device=DEV)
    sink = torch.zeros(g * 256, dtype=torch.int32, device=DEV)
    tq.read_probe(src, g, sink)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(src.cpu().numpy().view(np.uint32))
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == want


def test_append_rejects_full_cache(c128):
    ctx, _, _ = c128
    cache = tq.KVCache(1, 1, 32, 128, 3, 3)
    cache.seq_len.fill_(32)
    cache.host_max_len = 32
    x = torch.zeros((1, 1, 128), device=DEV)
    with pytest.raises(tq.TQError) as e:
        cache.append(ctx, x, x)
    assert e.value.status == tq.TQ_ERR_CAPACITY


def test_hot_path_argument_errors(c128):
    ctx, _, _ = c128
    kp = tq.Packed(64, 128, 3, True)
    x = torch.zeros((64, 128), device=DEV)
    with pytest.raises(tq.TQError):
        tq.quantize_kv(ctx, x, kp, out_offset=10)          # records past the end
    vp = tq.Packed(64, 128, 3, False)
    with pytest.raises(tq.TQError):
        tq.quantize_kv(ctx, x[:32], vp, out_offset=16)     # value offsets must be block aligned
    with pytest.raises(tq.TQError):
        tq.quantize_kv(ctx, x, kp, work=torch.empty(16, dtype=torch.uint8, device=DEV))  # workspace too small
    cache = tq.KVCache(1, 2, 64, 128, 3, 3)
    with pytest.raises(tq.TQError):
        cache.decode(ctx, torch.zeros((1, 3, 128), device=DEV))  # q_heads not a multiple of kv_heads
    with pytest.raises(tq.TQError):
        tq.scores(ctx, torch.zeros((2, 128), device=DEV), kp, want_scores=False, topk=65)
