"""GPU regression tests: the decode kernels read no record outside a chunk's
valid tokens.

The key records of a decode chunk are fetched with range-checked buffer loads
whose range covers exactly the chunk's valid records, and the loads of a wave
run a round ahead of its compute, so near a chunk's end they ask for records
past it. Those must come back as zeros: the records past a sequence's length,
and past the end of the cache arrays, hold huge norms (1e30) and random bits
here, and any of them reaching the kernel would swamp the chunk's value scale
(its largest ||v||) or its logits. Decode, many-query attention and the fused
step are checked against the oracle on the valid records only.
"""
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
TAIL = 512  # records of garbage after the end of every cache array
HUGE = 1e30


def _garbage_tail_cache(B, H, cap, kbits, vbits):
    """A KVCache whose arrays are the heads of larger buffers; the rest of each
    buffer (TAIL records) holds random bits and norms of 1e30."""
    cache = tq.KVCache(B, H, cap, D, kbits, vbits)
    n = B * H * cap
    g = torch.Generator(device=DEV)
    g.manual_seed(99)

    def big(t, rows, fill_norm):
        shape = (t.shape[0] + rows,) + tuple(t.shape[1:])
        if t.dtype == torch.int32:
            x = torch.randint(-2 ** 31, 2 ** 31 - 1, shape, generator=g, device=DEV, dtype=torch.int32)
        else:
            x = torch.full(shape, fill_norm, dtype=t.dtype, device=DEV)
        return x

    kw = big(cache.k.words, TAIL, 0)
    kn = big(cache.k.norms, TAIL, HUGE)
    vw = big(cache.v.words, TAIL // 32, 0)
    vn = big(cache.v.norms, TAIL, HUGE)
    cache.k.words, cache.k.norms = kw[:n], kn[:n]
    cache.v.words, cache.v.norms = vw[:n // 32], vn[:n]
    return cache


def _fill(cache, K, V, Pi, S, kbits, vbits, seq):
    """Oracle-packed records of K/V for every stream; records at or past
    seq[b] (up to capacity) are overwritten with garbage."""
    B, H, cap = cache.batch, cache.kv_heads, cache.capacity
    cbk, cbv = T.codebook(D, kbits), T.codebook(D, vbits)
    host = {}
    rng = np.random.default_rng(5)
    for b in range(B):
        for h in range(H):
            s = b * H + h
            pk = T.pack_keys(T.encode(K[b, h], Pi, cbk, S), kbits)
            pv = T.pack_values(T.encode(V[b, h], Pi, cbv), vbits)
            kw, kn = pk["bits"].copy(), pk["norms"].copy()
            vn = pv["norms"].copy()
            L = seq[b]
            kw[L:] = rng.integers(0, 2 ** 32, size=kw[L:].shape, dtype=np.uint64).astype(np.uint32)
            kn[L:] = HUGE
            vn[L:] = HUGE
            cache.k.words[s * cap:(s + 1) * cap].copy_(torch.from_numpy(kw.view(np.int32)).to(DEV))
            cache.k.norms[s * cap:(s + 1) * cap].copy_(torch.from_numpy(kn).to(DEV))
            cache.v.words[s * cap // 32:(s + 1) * cap // 32].copy_(torch.from_numpy(pv["bits"].view(np.int32)).to(DEV))
            cache.v.norms[s * cap:(s + 1) * cap].copy_(torch.from_numpy(vn).to(DEV))
            host[s] = ({"bits": kw, "norms": kn}, {"bits": pv["bits"], "norms": vn})
    cache.seq_len.copy_(torch.tensor(seq, dtype=torch.int32))
    cache.host_max_len = int(max(seq))
    return cbk, cbv, host


@pytest.mark.parametrize("kbits", [3, 2])
def test_decode_ignores_records_past_length_and_array_end(kbits):
    """Capacity 1056: sequence 0 ends at 1000 with garbage in records
    1000..1055; sequence 1 is full, so its last chunk (32 tokens) ends at the
    end of the arrays, followed by the garbage tail. Decode (groups of 4) and
    many-query causal attention (4 positions) against the oracle over the valid
    records."""
    from tests.test_gpu_parity import _ctx_and_oracle
    ctx, Pi, S = _ctx_and_oracle(D)
    B, H, Hq, cap = 2, 2, 8, 1056
    seq = [1000, cap]
    K = synth.outlier_kv(21, (kbits, 1), synth.TAG_SCALES_K, (B, H, cap, D))
    V = synth.outlier_kv(21, (kbits, 2), synth.TAG_SCALES_V, (B, H, cap, D))
    cache = _garbage_tail_cache(B, H, cap, kbits, 3)
    cbk, cbv, host = _fill(cache, K, V, Pi, S, kbits, 3, seq)
    scale = 1 / math.sqrt(D)
    g = Hq // H
    Q = synth.gaussian(21, (kbits, 3), (B, Hq, D), "bf16")
    out = cache.decode(ctx, torch.from_numpy(Q).to(DEV).to(torch.bfloat16), scale).cpu().numpy()
    NQ = 4
    Qp = synth.gaussian(21, (kbits, 4), (B, NQ, Hq, D), "bf16")
    outp = cache.attend(ctx, torch.from_numpy(Qp).to(DEV).to(torch.bfloat16), True, scale).cpu().numpy()
    torch.cuda.synchronize()
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(outp))
    for b in range(B):
        for h in range(H):
            keys, vals = host[b * H + h]
            ref = T.attention_decode(Q[b, h * g:(h + 1) * g], Pi, S, cbk, cbv, keys, vals, seq[b], scale)
            err = np.max(np.abs(out[b, h * g:(h + 1) * g] - ref))
            assert err <= 2e-3, f"decode b={b} h={h}: {err}"
            refp = T.attention_prefill(Qp[b, :, h * g:(h + 1) * g], Pi, S, cbk, cbv, keys, vals, seq[b], scale, True)
            errp = np.max(np.abs(outp[b, :, h * g:(h + 1) * g] - refp))
            assert errp <= 2e-3, f"prefill b={b} h={h}: {errp}"


def test_decode_step_ignores_records_past_length():
    """Fused step on a cache whose records past each length hold garbage: the
    appended token overwrites record seq_len[b] and is attended; the garbage
    after it is not."""
    from tests.test_gpu_parity import _ctx_and_oracle
    ctx, Pi, S = _ctx_and_oracle(D)
    B, H, Hq, cap = 2, 2, 8, 1056
    seq = [700, cap - 1]
    K = synth.outlier_kv(23, (1,), synth.TAG_SCALES_K, (B, H, cap, D))
    V = synth.outlier_kv(23, (2,), synth.TAG_SCALES_V, (B, H, cap, D))
    cache = _garbage_tail_cache(B, H, cap, 3, 3)
    cbk, cbv, _ = _fill(cache, K, V, Pi, S, 3, 3, seq)
    scale = 1 / math.sqrt(D)
    g = Hq // H
    KA = synth.outlier_kv(23, (3,), synth.TAG_SCALES_K, (B, H, D))
    VA = synth.outlier_kv(23, (4,), synth.TAG_SCALES_V, (B, H, D))
    Q = synth.gaussian(23, (5,), (B, Hq, D), "bf16")
    bf = lambda x: torch.from_numpy(x).to(DEV).to(torch.bfloat16).contiguous()  # noqa: E731
    out = cache.decode_step(ctx, bf(KA), bf(VA), bf(Q), scale).cpu().numpy()
    torch.cuda.synchronize()
    assert cache.seq_len.cpu().tolist() == [s + 1 for s in seq]
    gkw, gkn = cache.k.host()
    gvw, gvn = cache.v.host()
    for b in range(B):
        for h in range(H):
            s = b * H + h
            n = seq[b] + 1
            keys = {"bits": gkw[s * cap:s * cap + n], "norms": gkn[s * cap:s * cap + n]}
            vals = {"bits": gvw[s * cap // 32:(s + 1) * cap // 32], "norms": gvn[s * cap:s * cap + n]}
            assert np.all(gkn[s * cap:s * cap + n] < 1e29), "the appended record was not written"
            ref = T.attention_decode(Q[b, h * g:(h + 1) * g], Pi, S, cbk, cbv, keys, vals, n, scale)
            err = np.max(np.abs(out[b, h * g:(h + 1) * g] - ref))
            assert err <= 2e-3, f"step b={b} h={h}: {err}"
