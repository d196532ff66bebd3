"""GPU parity of attention over the packed cache for many query positions per
sequence (the cache part of chunked prefill): every query position i of n_q
attends to the tokens t < seq_len (non-causal) or t < seq_len - n_q + i + 1
(causal), with the keys' estimator scores and the values' stage-1 records.
The kernels run on oracle-packed records uploaded to the device; outputs are
within 2e-3 max-abs of the oracle (the decode bar).

Queries are Gaussian against outlier-channel K/V: logits of order ten. Queries
with the keys' own outlier channels give logits of order 10^3, where two keys
a logit apart share the softmax and the output moves by p1 p2 |v1 - v2| per
unit of logit error: a score error of 1e-6 relative (far inside the score bar)
then moves it by ~1e-2. n_q = 1 is bit-identical to decode either way."""
import math

import numpy as np
import pytest

import synth
from oracle import turboquant as T

torch = pytest.importorskip("torch")
tq = pytest.importorskip("kv_cache_vector_turboquant_amd")

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def c128():
    ctx = tq.Context(128, 0)
    Pi = T.rotation_from_gaussian(synth.gaussian_matrix(0, synth.TAG_ROTATION, 128, 128))
    S = T.sketch_from_gaussian(synth.gaussian_matrix(0, synth.TAG_SKETCH, 128, 128))
    return ctx, Pi, S


def _dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def _upload(packed, words, norms):
    packed.words[:words.shape[0]].copy_(torch.from_numpy(np.ascontiguousarray(words).view(np.int32)).to(DEV))
    packed.norms[:norms.shape[0]].copy_(torch.from_numpy(np.ascontiguousarray(norms)).to(DEV))


def _cache(ctx, Pi, S, K, V, seq, kbits, vbits, cap, qjl=True):
    """Oracle-encoded K, V [B, H, L, d] uploaded into a device cache of capacity cap."""
    B, H, L, d = K.shape
    cbk = T.codebook(d, kbits) if kbits > 0 else None
    cbv = T.codebook(d, vbits)
    kw = np.zeros((B * H * cap, d // 32, kbits + int(qjl)), np.uint32)
    kn = np.zeros((B * H * cap, 1 + int(qjl)), np.float32)
    vw = np.zeros((B * H * cap // 32, d, vbits), np.uint32)
    vn = np.zeros((B * H * cap,), np.float32)
    for b in range(B):
        for h in range(H):
            s = b * H + h
            pk = T.pack_keys(T.encode(K[b, h], Pi, cbk, S if qjl else None), kbits, qjl)
            pv = T.pack_values(T.encode(V[b, h], Pi, cbv), vbits)
            kw[s * cap:s * cap + L] = pk["bits"]
            kn[s * cap:s * cap + L] = pk["norms"]
            vw[s * cap // 32:s * cap // 32 + pv["bits"].shape[0]] = pv["bits"]
            vn[s * cap:s * cap + L] = pv["norms"]
    cache = tq.KVCache(B, H, cap, d, kbits, vbits, key_qjl=qjl)
    _upload(cache.k, kw, kn)
    _upload(cache.v, vw, vn)
    cache.seq_len.copy_(torch.tensor(seq, dtype=torch.int32))
    cache.host_max_len = int(max(seq))
    return cache, dict(cbk=cbk, cbv=cbv, kw=kw, kn=kn, vw=vw, vn=vn, cap=cap, H=H, qjl=qjl)


def _check(out, Q, Pi, S, o, seq, scale, causal, tol=2e-3):
    """out, Q: [B, n_q, Hq, d]."""
    B, nq, Hq, d = Q.shape
    H, cap = o["H"], o["cap"]
    g = Hq // H
    worst = 0.0
    for b in range(B):
        for h in range(H):
            s, Lb = b * H + h, seq[b]
            got = out[b, :, h * g:(h + 1) * g]
            keys = {"bits": o["kw"][s * cap:s * cap + Lb], "norms": o["kn"][s * cap:s * cap + Lb]}
            vals = {"bits": o["vw"][s * cap // 32:(s + 1) * cap // 32], "norms": o["vn"][s * cap:s * cap + Lb]}
            ref = T.attention_prefill(Q[b, :, h * g:(h + 1) * g], Pi, S, o["cbk"], o["cbv"], keys, vals, Lb, scale,
                                      causal, o["qjl"])
            blind = np.all(ref == 0, axis=2)            # positions that see no token
            assert not got[blind].any(), f"b={b} h={h}: a position with no visible token is nonzero"
            err = float(np.max(np.abs(got - ref))) if got.size else 0.0
            worst = max(worst, err)
            assert err <= tol, f"prefill mismatch b={b} h={h}: {err}"
    return worst


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("qdtype", ["bf16", "f32"])
def test_prefill_gqa_ragged(c128, causal, qdtype):
    """batch 4 (lengths 1000, 37, 20, 0), 2 KV heads, 8 query heads (groups of 4),
    37 query positions: the last position of each sequence sees it all, a
    sequence shorter than the chunk leaves its first positions blind."""
    ctx, Pi, S = c128
    B, H, cap, L, nq, hq = 4, 2, 1024, 1000, 37, 8
    seq = [1000, 37, 20, 0]
    K = synth.outlier_kv(21, (1,), synth.TAG_SCALES_K, (B, H, L, 128))
    V = synth.outlier_kv(21, (2,), synth.TAG_SCALES_V, (B, H, L, 128))
    Q = synth.gaussian(21, (3,), (B, nq, hq, 128), qdtype)
    cache, o = _cache(ctx, Pi, S, K, V, seq, 3, 3, cap)
    scale = 1.0 / math.sqrt(128)
    out = cache.attend(ctx, _dev(Q, qdtype), causal, scale).cpu().numpy()
    _check(out, Q, Pi, S, o, seq, scale, causal)


@pytest.mark.parametrize("seq", [[1026, 3], [3, 1026]])
def test_prefill_decode_path_heads_blind_in_a_chunk(c128, seq):
    """Causal attention of 5 query positions (groups of one query head: 5 virtual
    heads per KV head, so the decode kernels run, over head groups of 4). At
    length 1026 the last 256-token chunk holds 2 tokens: positions 0-2 see none of
    them while 3 and 4 do, in the same work-group (a head with no visible token
    in a chunk whose others see some). At length 3 positions 0 and 1 see nothing
    at all: their output is exactly zero."""
    ctx, Pi, S = c128
    B, H, cap, nq, hq = 2, 2, 1280, 5, 2
    L = max(seq)
    K = synth.outlier_kv(23, (1,), synth.TAG_SCALES_K, (B, H, L, 128))
    V = synth.outlier_kv(23, (2,), synth.TAG_SCALES_V, (B, H, L, 128))
    Q = synth.gaussian(23, (3,), (B, nq, hq, 128), "bf16")
    cache, o = _cache(ctx, Pi, S, K, V, seq, 3, 3, cap)
    scale = 1.0 / math.sqrt(128)
    out = cache.attend(ctx, _dev(Q, "bf16"), True, scale).cpu().numpy()
    _check(out, Q, Pi, S, o, seq, scale, True)


@pytest.mark.parametrize("hq,nq", [(2, 5), (6, 7), (32, 3), (4, 129)])
def test_prefill_group_sizes(c128, hq, nq):
    """Gaussian K/V, 2 KV heads; groups of 1, 3, 16 and 2 query heads times n_q
    positions give 5, 21, 48 and 258 virtual heads per KV head (partial groups
    of four at the end)."""
    ctx, Pi, S = c128
    B, H, cap, L = 2, 2, 640, 600
    seq = [600, 333]
    K = synth.gaussian(22, (hq, 1), (B, H, L, 128))
    V = synth.gaussian(22, (hq, 2), (B, H, L, 128))
    Q = synth.gaussian(22, (hq, 3), (B, nq, hq, 128), "bf16")
    cache, o = _cache(ctx, Pi, S, K, V, seq, 2, 4, cap)
    scale = 1.0 / math.sqrt(128)
    out = cache.attend(ctx, _dev(Q, "bf16"), True, scale).cpu().numpy()
    _check(out, Q, Pi, S, o, seq, scale, True)


@pytest.mark.parametrize("bits,qjl", [(2, False), (0, True), (4, True), (1, True)], ids=["mse2", "qjl", "tq4", "tq1"])
def test_prefill_key_formats(c128, bits, qjl):
    """MSE-only, pure QJL and B = 1, 4 TurboQuant keys, causal, n_q = 10."""
    ctx, Pi, S = c128
    B, H, cap, L, nq, hq = 2, 2, 512, 500, 10, 8
    seq = [500, 123]
    K = synth.outlier_kv(23, (bits, 1), synth.TAG_SCALES_K, (B, H, L, 128))
    V = synth.outlier_kv(23, (bits, 2), synth.TAG_SCALES_V, (B, H, L, 128))
    Q = synth.gaussian(23, (bits, 3), (B, nq, hq, 128), "bf16")
    cache, o = _cache(ctx, Pi, S, K, V, seq, bits, 3, cap, qjl)
    scale = 1.0 / math.sqrt(128)
    out = cache.attend(ctx, _dev(Q, "bf16"), True, scale).cpu().numpy()
    _check(out, Q, Pi, S, o, seq, scale, True)


def test_prefill_one_position_is_decode(c128):
    """n_q = 1 runs the decode kernels unchanged: the causal and full outputs are
    bit-identical to tq_attention_decode's."""
    ctx, Pi, S = c128
    B, H, cap, L = 3, 2, 2048, 2000
    seq = [2000, 0, 777]
    K = synth.outlier_kv(24, (1,), synth.TAG_SCALES_K, (B, H, L, 128))
    V = synth.outlier_kv(24, (2,), synth.TAG_SCALES_V, (B, H, L, 128))
    Q = synth.outlier_kv(24, (3,), synth.TAG_SCALES_K, (B, 1, 8, 128), "bf16")
    cache, o = _cache(ctx, Pi, S, K, V, seq, 3, 3, cap)
    q = _dev(Q, "bf16")
    dec = cache.decode(ctx, q[:, 0].contiguous())
    for causal in (True, False):
        assert torch.equal(cache.attend(ctx, q, causal)[:, 0], dec)


def test_chunked_prefill_end_to_end(c128):
    """Chunked prefill through the cache: quantize a 256-token prompt, then
    append a 96-token chunk (tq_quantize_kv at offset 256) and attend the
    chunk's queries causally over all 352 tokens. The appended records are the
    oracle's up to the boundary band; attention is checked on the records the
    GPU wrote."""
    ctx, Pi, S = c128
    B, H, cap, L0, nq, hq = 2, 2, 384, 256, 96, 8
    K = synth.outlier_kv(25, (1,), synth.TAG_SCALES_K, (B, H, L0 + nq, 128), "bf16")
    V = synth.outlier_kv(25, (2,), synth.TAG_SCALES_V, (B, H, L0 + nq, 128), "bf16")
    Q = synth.gaussian(25, (3,), (B, nq, hq, 128), "bf16")
    cache = tq.KVCache(B, H, cap, 128, 3, 3)
    cache.prefill(ctx, _dev(K[:, :, :L0], "bf16"), _dev(V[:, :, :L0], "bf16"))
    cache.extend(ctx, _dev(K[:, :, L0:], "bf16"), _dev(V[:, :, L0:], "bf16"))
    assert cache.host_max_len == L0 + nq
    scale = 1.0 / math.sqrt(128)
    out = cache.attend(ctx, _dev(Q, "bf16"), True, scale).cpu().numpy()
    kw, kn = cache.k.host()
    vw, vn = cache.v.host()
    cbk, cbv = T.codebook(128, 3), T.codebook(128, 3)
    L = L0 + nq
    for b in range(B):
        for h in range(H):
            s = b * H + h
            enc = T.encode(K[b, h].astype(np.float32), Pi, cbk, S)
            ref_idx = enc.idx
            got_idx, _ = T.unpack_keys(kw[s * cap:s * cap + L], 128, 3)
            assert np.mean(got_idx != ref_idx) < 1e-3
    o = dict(cbk=cbk, cbv=cbv, kw=kw, kn=kn, vw=vw, vn=vn, cap=cap, H=H, qjl=True)
    _check(out, Q, Pi, S, o, [L] * B, scale, True)


def test_prefill_argument_errors(c128):
    ctx, Pi, S = c128
    cache = tq.KVCache(1, 2, 64, 128, 3, 3)
    q = torch.zeros((1, 4, 8, 128), device=DEV)
    cc = cache.c()
    out = torch.empty((1, 4, 8, 128), device=DEV)
    need = cache.prefill_ws_bytes(ctx, 4, 8)
    assert need > 0 and cache.prefill_ws_bytes(ctx, 0, 8) == 0 and cache.prefill_ws_bytes(ctx, 4, 3) == 0
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    import ctypes
    L = tq.lib()
    args = lambda nq, hq, causal, wsb: (ctx.handle, ctypes.byref(cc), q.data_ptr(), 0, nq, hq, causal, 0.1,
                                        out.data_ptr(), ws.data_ptr(), wsb, None)
    assert L.tq_attention_prefill(*args(4, 8, 1, need)) == 0
    assert L.tq_attention_prefill(*args(0, 8, 1, need)) != 0
    assert L.tq_attention_prefill(*args(4, 8, 2, need)) != 0
    assert L.tq_attention_prefill(*args(4, 3, 1, need)) != 0
    assert L.tq_attention_prefill(*args(4, 8, 1, need - 1)) != 0
    assert L.tq_attention_prefill(*args(4, 64, 1, need)) != 0     # group 32 > 16
    torch.cuda.synchronize()


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_prefill_kernel_many_chunks(c128, causal):
    """The 16-virtual-head prefill kernel over a context split into several
    512-token chunks: 1 sequence of 2900 tokens (a ragged last block), 2 KV
    heads, 8 query heads, 64 query positions (256 virtual heads per KV head,
    16 work-group units), 3-bit keys with QJL signs, 3-bit values."""
    ctx, Pi, S = c128
    B, H, cap, L, nq, hq = 1, 2, 3072, 2900, 64, 8
    seq = [L]
    K = synth.outlier_kv(26, (1,), synth.TAG_SCALES_K, (B, H, L, 128))
    V = synth.outlier_kv(26, (2,), synth.TAG_SCALES_V, (B, H, L, 128))
    Q = synth.gaussian(26, (3,), (B, nq, hq, 128), "bf16")
    cache, o = _cache(ctx, Pi, S, K, V, seq, 3, 3, cap)
    scale = 1.0 / math.sqrt(128)
    out = cache.attend(ctx, _dev(Q, "bf16"), causal, scale).cpu().numpy()
    _check(out, Q, Pi, S, o, seq, scale, causal)


@pytest.mark.parametrize("kbits,qjl,vbits", [(4, True, 3), (2, True, 1), (4, False, 2), (0, True, 3)],
                         ids=["tq5-v3", "tq3-v1", "mse4-v2", "qjl-v3"])
def test_prefill_kernel_formats(c128, kbits, qjl, vbits):
    """Key formats (B = 0..4, with and without QJL signs) and value bits 1..3
    through the prefill kernel: 2 sequences (1100 and 513 tokens), 2 KV heads,
    16 query heads (groups of 8), 9 positions (72 virtual heads: a partial
    last unit of 8)."""
    ctx, Pi, S = c128
    B, H, cap, L, nq, hq = 2, 2, 1152, 1100, 9, 16
    seq = [1100, 513]
    K = synth.outlier_kv(27, (kbits, vbits, 1), synth.TAG_SCALES_K, (B, H, L, 128))
    V = synth.outlier_kv(27, (kbits, vbits, 2), synth.TAG_SCALES_V, (B, H, L, 128))
    Q = synth.gaussian(27, (kbits, vbits, 3), (B, nq, hq, 128), "f32")
    cache, o = _cache(ctx, Pi, S, K, V, seq, kbits, vbits, cap, qjl)
    scale = 1.0 / math.sqrt(128)
    out = cache.attend(ctx, _dev(Q, "f32"), True, scale).cpu().numpy()
    _check(out, Q, Pi, S, o, seq, scale, True)


def test_prefill_kernel_bench_shape_sampled(c128):
    """The chunked-prefill benchmark's last chunk at full size: 8 KV heads x
    16384 tokens quantized on the GPU, 1024 causal query positions x 32 query
    heads. Sampled outputs (2 KV heads x 3 positions x 4 heads) against the
    oracle over the records the GPU wrote, within 2e-3."""
    ctx, Pi, S = c128
    B, H, Hq, P, C, d = 1, 8, 32, 16384, 1024, 128
    K = synth.outlier_kv(28, (1,), synth.TAG_SCALES_K, (B, H, P, d), "bf16")
    V = synth.outlier_kv(28, (2,), synth.TAG_SCALES_V, (B, H, P, d), "bf16")
    Q = synth.gaussian(28, (3,), (B, C, Hq, d), "bf16")
    cache = tq.KVCache(B, H, P, d, 3, 3)
    cache.prefill(ctx, _dev(K, "bf16"), _dev(V, "bf16"))
    scale = 1.0 / math.sqrt(d)
    out = cache.attend(ctx, _dev(Q, "bf16"), True, scale).cpu().numpy()
    torch.cuda.synchronize()
    kw, kn = cache.k.host()
    vw, vn = cache.v.host()
    cbk, cbv = T.codebook(d, 3), T.codebook(d, 3)
    g = Hq // H
    worst = 0.0
    for h in (0, 5):
        keys = {"bits": kw[h * P:(h + 1) * P], "norms": kn[h * P:(h + 1) * P]}
        vals = {"bits": vw[h * P // 32:(h + 1) * P // 32], "norms": vn[h * P:(h + 1) * P]}
        for i in (0, 517, C - 1):
            vis = P - C + i + 1
            ref = T.attention_decode(Q[0, i, h * g:(h + 1) * g], Pi, S, cbk, cbv, keys, vals, vis, scale)
            err = float(np.max(np.abs(out[0, i, h * g:(h + 1) * g] - ref)))
            worst = max(worst, err)
            assert err <= 2e-3, f"h={h} position {i}: {err}"


def test_prefill_kernel_one_chunk_finishes_in_kernel(c128):
    """Enough units (8 sequences x 8 KV heads x 16 units) that one chunk covers
    each context: the prefill kernel writes the output itself (no partials,
    no merge). Lengths 700, 600, 0, 20, 64, 65, 1, 512: whole-unit blind
    positions (a sequence shorter than the chunk), a sequence with no token and
    one block boundary; 64 causal positions x 4 heads per KV head."""
    ctx, Pi, S = c128
    B, H, cap, L, nq, hq = 8, 8, 704, 700, 64, 32
    seq = [700, 600, 0, 20, 64, 65, 1, 512]
    K = synth.outlier_kv(29, (1,), synth.TAG_SCALES_K, (B, H, L, 128))
    V = synth.outlier_kv(29, (2,), synth.TAG_SCALES_V, (B, H, L, 128))
    Q = synth.gaussian(29, (3,), (B, nq, hq, 128), "bf16")
    cache, o = _cache(ctx, Pi, S, K, V, seq, 3, 3, cap)
    scale = 1.0 / math.sqrt(128)
    out = cache.attend(ctx, _dev(Q, "bf16"), True, scale).cpu().numpy()
    _check(out, Q, Pi, S, o, seq, scale, True)
