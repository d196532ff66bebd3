"""Paged KV cache: the pool of pages with a block table per sequence, through
every cache entry point (tq_cache_write, tq_attention_decode,
tq_attention_prefill, tq_decode_step, tq_append_token). With pages of 1024
tokens the paged cache holds, for every (sequence, KV head, position), the
record the contiguous cache holds, bit for bit, and every attention output is
bit-identical (same kernels, same chunking) -- with the pages in a shuffled
order and spare pages in the pool. With 256-token pages (the decode chunk
shrinks to the page) the records and the attention are checked against the
oracle on the logical streams."""
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


@pytest.fixture(scope="module")
def c128():
    ctx = tq.Context(128, 0)
    Pi = T.rotation_from_gaussian(synth.gaussian_matrix(0, synth.TAG_ROTATION, 128, 128))
    S = T.sketch_from_gaussian(synth.gaussian_matrix(0, synth.TAG_SKETCH, 128, 128))
    return ctx, Pi, S


def _dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def _shuffled_table(seed, batch, cols, spare):
    n_pages = batch * cols + spare
    perm = np.random.default_rng(seed).permutation(n_pages)[:batch * cols].astype(np.int32)
    return n_pages, torch.from_numpy(perm.reshape(batch, cols)).to(DEV)


def _rec_index(cache, table_h, b, h, t):
    """Record indices of positions t (array) of stream (b, h)."""
    t = np.asarray(t, dtype=np.int64)
    if cache.block_table is None:
        return (b * cache.kv_heads + h) * cache.capacity + t
    Pt = cache.page_tokens
    return (table_h[b, t // Pt].astype(np.int64) * cache.kv_heads + h) * Pt + t % Pt


def _stream_records(cache, b, h, L):
    """(key words, key norms, value block words, value norms) of the first L
    positions of stream (b, h), in logical order."""
    table_h = cache.block_table.cpu().numpy() if cache.block_table is not None else None
    kw, kn = cache.k.host()
    vw, vn = cache.v.host()
    idx = _rec_index(cache, table_h, b, h, np.arange(L))
    blk = _rec_index(cache, table_h, b, h, np.arange(0, L, 32)) >> 5
    return kw[idx], kn[idx], vw[blk], vn[idx]


def _assert_same_records(ca, cb, B, H, lens):
    for b in range(B):
        for h in range(H):
            ra, rb = _stream_records(ca, b, h, lens[b]), _stream_records(cb, b, h, lens[b])
            for x, y, what in zip(ra, rb, ("key words", "key norms", "value words", "value norms")):
                if what == "value words" and lens[b] % 32:
                    # the last block's bits past the length are not part of the stream
                    keep = np.uint32((1 << (lens[b] % 32)) - 1)
                    x, y = x.copy(), y.copy()
                    x[-1] &= keep
                    y[-1] &= keep
                assert np.array_equal(x, y), f"{what} differ at b={b} h={h}"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_paged_cache_matches_contiguous(c128, dtype):
    """batch 3, 2 KV heads, 8 query heads, capacity 4096, 1024-token pages in a
    shuffled pool with 3 spare pages: prefill of 3000 tokens (fused bf16 kernel /
    fp32 GEMM path), lengths 3000, 1500, 37; decode, causal prefill attention of
    7 positions, three fused decode steps and two standalone appends give the
    contiguous cache's records and outputs exactly."""
    ctx, _, _ = c128
    B, H, Hq, cap, Pt, L, d = 3, 2, 8, 4096, 1024, 3000, 128
    n_pages, table = _shuffled_table(41, B, cap // Pt, 3)
    K = synth.outlier_kv(41, (1,), synth.TAG_SCALES_K, (B, H, L, d), dtype)
    V = synth.outlier_kv(41, (2,), synth.TAG_SCALES_V, (B, H, L, d), dtype)
    flat = tq.KVCache(B, H, cap, d, 3, 3)
    paged = tq.KVCache(B, H, cap, d, 3, 3, page_tokens=Pt, n_pages=n_pages, block_table=table)
    for c in (flat, paged):
        c.prefill(ctx, _dev(K, dtype), _dev(V, dtype))
    torch.cuda.synchronize()
    _assert_same_records(flat, paged, B, H, [L] * B)
    lens = [3000, 1500, 37]
    for c in (flat, paged):
        c.seq_len.copy_(torch.tensor(lens, dtype=torch.int32))
        c.host_max_len = max(lens)
    q = _dev(synth.gaussian(41, (3,), (B, Hq, d)), dtype)
    assert torch.equal(flat.decode(ctx, q), paged.decode(ctx, q))
    qp = _dev(synth.gaussian(41, (4,), (B, 7, Hq, d)), dtype)
    assert torch.equal(flat.attend(ctx, qp, True), paged.attend(ctx, qp, True))
    for i in range(3):
        ka = _dev(synth.outlier_kv(41, (5, i), synth.TAG_SCALES_K, (B, H, d), dtype), dtype)
        va = _dev(synth.outlier_kv(41, (6, i), synth.TAG_SCALES_V, (B, H, d), dtype), dtype)
        qs = _dev(synth.gaussian(41, (7, i), (B, Hq, d)), dtype)
        assert torch.equal(flat.decode_step(ctx, ka, va, qs), paged.decode_step(ctx, ka, va, qs)), f"step {i}"
    for i in range(2):
        ka = _dev(synth.outlier_kv(41, (8, i), synth.TAG_SCALES_K, (B, H, d), dtype), dtype)
        va = _dev(synth.outlier_kv(41, (9, i), synth.TAG_SCALES_V, (B, H, d), dtype), dtype)
        for c in (flat, paged):
            c.append(ctx, ka, va)
    torch.cuda.synchronize()
    lens = [n + 5 for n in lens]
    assert flat.seq_len.cpu().tolist() == lens == paged.seq_len.cpu().tolist()
    _assert_same_records(flat, paged, B, H, lens)
    assert torch.equal(flat.decode(ctx, q), paged.decode(ctx, q))


def test_paged_small_pages_against_oracle(c128):
    """256-token pages (decode chunks of 256), shuffled, fp32 inputs through the
    GEMM quantize path: 2 sequences x 2 KV heads of 700 tokens, lengths 700 and
    300. Records match the oracle's encoding of the logical streams; decode and
    causal prefill attention match the oracle within 2e-3."""
    ctx, Pi, S = c128
    B, H, Hq, cap, Pt, L, d = 2, 2, 8, 1024, 256, 700, 128
    n_pages, table = _shuffled_table(42, B, cap // Pt, 1)
    K = synth.outlier_kv(42, (1,), synth.TAG_SCALES_K, (B, H, L, d))
    V = synth.outlier_kv(42, (2,), synth.TAG_SCALES_V, (B, H, L, d))
    cache = tq.KVCache(B, H, cap, d, 3, 3, page_tokens=Pt, n_pages=n_pages, block_table=table)
    cache.prefill(ctx, _dev(K, "f32"), _dev(V, "f32"))
    lens = [700, 300]
    cache.seq_len.copy_(torch.tensor(lens, dtype=torch.int32))
    cache.host_max_len = max(lens)
    q = synth.gaussian(42, (3,), (B, Hq, d), "bf16")
    qp = synth.gaussian(42, (4,), (B, 5, Hq, d), "bf16")
    out = cache.decode(ctx, _dev(q, "bf16"), 1 / math.sqrt(d)).cpu().numpy()
    outp = cache.attend(ctx, _dev(qp, "bf16"), True, 1 / math.sqrt(d)).cpu().numpy()
    cbk, cbv = T.codebook(d, 3), T.codebook(d, 3)
    g = Hq // H
    for b in range(B):
        for h in range(H):
            kw, kn, vw, vn = _stream_records(cache, b, h, L)
            enc_k = T.encode(K[b, h], Pi, cbk, S)
            P.check_key_records(kw, kn, enc_k, cbk, 3, d)
            enc_v = T.encode(V[b, h], Pi, cbv)
            P.check_codes(T.unpack_values(vw, d, 3, L), enc_v, cbv, "value codes")
            n = lens[b]
            keys = {"bits": kw[:n], "norms": kn[:n]}
            vals = {"bits": vw, "norms": vn[:n]}
            ref = T.attention_decode(q[b, h * g:(h + 1) * g], Pi, S, cbk, cbv, keys, vals, n, 1 / math.sqrt(d))
            assert np.max(np.abs(out[b, h * g:(h + 1) * g] - ref)) <= 2e-3, f"decode b={b} h={h}"
            refp = T.attention_prefill(qp[b, :, h * g:(h + 1) * g], Pi, S, cbk, cbv, keys, vals, n,
                                       1 / math.sqrt(d), True)
            assert np.max(np.abs(outp[b, :, h * g:(h + 1) * g] - refp)) <= 2e-3, f"prefill b={b} h={h}"


@pytest.mark.parametrize("page_tokens", [256, 512])
def test_paged_chunks_spanning_pages(c128, page_tokens):
    """Pages smaller than the decode chunk: 2 sequences x 8 KV heads x 32868
    tokens with 128 query heads (groups of 16) make 1024-token chunks, each
    spanning four or two shuffled pages. Decode and two fused steps equal the
    contiguous cache's outputs bit for bit (same chunking, so the same
    arithmetic). Causal prefill attention of 3 positions (48 virtual heads per
    KV head): with 512-token pages both caches run the 16-head prefill kernel
    and agree bit for bit; 256-token pages take the decode kernels, whose
    result agrees with the prefill kernel's within the attention bar (each is
    checked against the oracle on its own elsewhere)."""
    ctx, _, _ = c128
    B, H, Hq, L, d = 2, 8, 128, 32868, 128
    cap = ((L + 2 + 1023) // 1024) * 1024
    n_pages, table = _shuffled_table(43, B, cap // page_tokens, 5)
    K = synth.torch_outlier_kv(43, (1,), synth.TAG_SCALES_K, (B, H, L, d), torch.bfloat16, DEV)
    V = synth.torch_outlier_kv(43, (2,), synth.TAG_SCALES_V, (B, H, L, d), torch.bfloat16, DEV)
    flat = tq.KVCache(B, H, cap, d, 3, 3)
    paged = tq.KVCache(B, H, cap, d, 3, 3, page_tokens=page_tokens, n_pages=n_pages, block_table=table)
    for c in (flat, paged):
        c.prefill(ctx, K, V)
        c.seq_len.copy_(torch.tensor([L, L - 5000], dtype=torch.int32))
    del K, V
    q = synth.torch_gaussian(43, (3,), (B, Hq, d), torch.bfloat16, DEV)
    assert torch.equal(flat.decode(ctx, q), paged.decode(ctx, q))
    qp = synth.torch_gaussian(43, (4,), (B, 3, Hq, d), torch.bfloat16, DEV)
    of, op = flat.attend(ctx, qp, True), paged.attend(ctx, qp, True)
    if page_tokens % 512 == 0:
        assert torch.equal(of, op)
    else:
        assert float((of - op).abs().max()) <= 2e-3
    for i in range(2):
        ka = synth.torch_outlier_kv(43, (5, i), synth.TAG_SCALES_K, (B, H, d), torch.bfloat16, DEV)
        va = synth.torch_outlier_kv(43, (6, i), synth.TAG_SCALES_V, (B, H, d), torch.bfloat16, DEV)
        qs = synth.torch_gaussian(43, (7, i), (B, Hq, d), torch.bfloat16, DEV)
        assert torch.equal(flat.decode_step(ctx, ka, va, qs), paged.decode_step(ctx, ka, va, qs)), f"step {i}"
    chunk_ws = paged.decode_ws_bytes(ctx, Hq)
    assert chunk_ws == flat.decode_ws_bytes(ctx, Hq)  # same chunking


def test_paged_cache_argument_errors(c128):
    """Page sizes that are not multiples of 256 or do not divide the capacity, and
    pools that are not whole pages, are rejected before any launch."""
    ctx, _, _ = c128
    cache = tq.KVCache(2, 2, 1024, 128, 3, 3, page_tokens=256)
    q = torch.zeros((2, 8, 128), device=DEV)
    cache.decode(ctx, q)  # valid
    L = tq.lib()
    import ctypes
    ws = torch.empty(cache.decode_ws_bytes(ctx, 8), dtype=torch.uint8, device=DEV)
    out = torch.empty((2, 8, 128), device=DEV)
    for field, value in (("page_tokens", 128), ("page_tokens", 768), ("page_tokens", 0)):
        cc = cache.c()
        setattr(cc, field, value)
        st = L.tq_attention_decode(ctx.handle, ctypes.byref(cc), q.data_ptr(), 0, 8, 0.1, out.data_ptr(),
                                   ws.data_ptr(), ws.numel(), None)
        assert st == tq.TQ_ERR_ARG, (field, value)
    cc = cache.c()
    cc.k.n = cc.k.n - 32  # not a whole number of pages
    cc.v.n = cc.v.n - 32
    assert L.tq_attention_decode(ctx.handle, ctypes.byref(cc), q.data_ptr(), 0, 8, 0.1, out.data_ptr(),
                                 ws.data_ptr(), ws.numel(), None) == tq.TQ_ERR_ARG
    torch.cuda.synchronize()
