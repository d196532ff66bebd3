"""tq_attention_decode_noalloc: decode attention with the library-held scratch
instead of a caller workspace, through the C ABI. Two calls in a row (the
second on a smaller cache, so it reuses the scratch the first one left
behind) must give exactly the output of tq_attention_decode with a caller
workspace on the same inputs, and match the oracle within 2e-3."""
import ctypes
import math

import numpy as np
import pytest

import synth
from oracle import turboquant as T

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
tq = pytest.importorskip("kv_cache_vector_turboquant_amd")

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

DEV = "cuda"
D = 128


def _case(ctx, Pi, S, B, H, Hq, cap, seq, seed):
    """An oracle-packed cache and queries; returns (cache, q, host records)."""
    cbk, cbv = T.codebook(D, 3), T.codebook(D, 3)
    K = synth.outlier_kv(seed, (1,), synth.TAG_SCALES_K, (B, H, cap, D))
    V = synth.outlier_kv(seed, (2,), synth.TAG_SCALES_V, (B, H, cap, D))
    cache = tq.KVCache(B, H, cap, D, 3, 3)
    host = {}
    for b in range(B):
        for h in range(H):
            s = b * H + h
            pk = T.pack_keys(T.encode(K[b, h], Pi, cbk, S), 3)
            pv = T.pack_values(T.encode(V[b, h], Pi, cbv), 3)
            cache.k.words[s * cap:(s + 1) * cap].copy_(torch.from_numpy(pk["bits"].view(np.int32)).to(DEV))
            cache.k.norms[s * cap:(s + 1) * cap].copy_(torch.from_numpy(pk["norms"]).to(DEV))
            cache.v.words[s * cap // 32:(s + 1) * cap // 32].copy_(torch.from_numpy(pv["bits"].view(np.int32)).to(DEV))
            cache.v.norms[s * cap:(s + 1) * cap].copy_(torch.from_numpy(pv["norms"]).to(DEV))
            host[s] = (pk, pv)
    cache.seq_len.copy_(torch.tensor(seq, dtype=torch.int32))
    cache.host_max_len = int(max(seq))
    Q = synth.gaussian(seed, (3,), (B, Hq, D), "bf16")
    return cache, Q, host, cbk, cbv


def _noalloc(ctx, cache, q, Hq, scale, out):
    lib = tq.lib()
    cc = cache.c()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = lib.tq_attention_decode_noalloc(ctx.handle, ctypes.byref(cc), ctypes.c_void_p(q.data_ptr()), tq.TQ_BF16, Hq,
                                         ctypes.c_float(scale), ctypes.c_void_p(out.data_ptr()), st)
    assert rc == tq.TQ_OK, tq.last_error()


def test_noalloc_decode_matches_workspace_decode_twice():
    ctx = tq.Context(D, 0)
    Pi = T.rotation_from_gaussian(synth.gaussian_matrix(0, synth.TAG_ROTATION, D, D))
    S = T.sketch_from_gaussian(synth.gaussian_matrix(0, synth.TAG_SKETCH, D, D))
    scale = 1 / math.sqrt(D)
    # first call: 3 sequences x 2 KV heads x 8 query heads, up to 3000 tokens;
    # second call: smaller (1 sequence x 2 KV heads x 4 query heads, 700 tokens)
    for (B, H, Hq, cap, seq, seed) in [(3, 2, 8, 3008, [3000, 1, 2077], 31), (1, 2, 4, 704, [700], 32)]:
        cache, Q, host, cbk, cbv = _case(ctx, Pi, S, B, H, Hq, cap, seq, seed)
        q = torch.from_numpy(Q).to(DEV).to(torch.bfloat16).contiguous()
        ref_out = cache.decode(ctx, q, scale)  # tq_attention_decode with a caller workspace
        out = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device=DEV)
        _noalloc(ctx, cache, q, Hq, scale, out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), "noalloc output differs from the workspace entry point's"
        o = out.cpu().numpy()
        g = Hq // H
        for b in range(B):
            for h in range(H):
                pk, pv = host[b * H + h]
                ref = T.attention_decode(Q[b, h * g:(h + 1) * g], Pi, S, cbk, cbv, pk, pv, seq[b], scale)
                assert np.max(np.abs(o[b, h * g:(h + 1) * g] - ref)) <= 2e-3


def test_noalloc_rejects_a_call_larger_than_the_scratch():
    """A decode whose workspace would exceed TQ_SCRATCH_BYTES is refused with
    TQ_ERR_CAPACITY before any launch (the cache arrays are never touched)."""
    ctx = tq.Context(D, 0)
    B, H, Hq, cap = 64, 8, 128, 131072
    cc = tq.CCache(tq.CPacked(16, 16, B * H * cap, 3, 1, 1, 0), tq.CPacked(16, 16, B * H * cap, 3, 0, 0, 0), B, H, cap,
                   16, cap, None, 0)
    need = tq.lib().tq_attention_decode_ws_bytes(ctx.handle, ctypes.byref(cc), Hq)
    assert need > (32 << 20)
    out = torch.empty(4, device=DEV)
    rc = tq.lib().tq_attention_decode_noalloc(ctx.handle, ctypes.byref(cc), ctypes.c_void_p(out.data_ptr()), tq.TQ_BF16,
                                              Hq, ctypes.c_float(0.1), ctypes.c_void_p(out.data_ptr()), None)
    assert rc == tq.TQ_ERR_CAPACITY and "TQ_SCRATCH_BYTES" in tq.last_error()
