"""The decode path's logits measured directly (tq_decode_logits: the query
preparation and key phase of the decode kernels, writing scale * s_t instead
of feeding the softmax) against the oracle's scores on identical packed bytes.

The decode scores use fixed-point query digits (about 23 bits relative to each
query's largest rotated coordinate) and fp32 folds, so each logit is expected
within fp32-level error of the oracle: |dl| <= 1e-6 (|l| + scale |q| |k|).
Outlier-channel queries against outlier-channel keys (logits of order 10^3,
the case where an attention output is ill-conditioned) and Gaussian queries are
both measured; the largest relative errors are printed."""
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


@pytest.mark.parametrize("qlaw,kbits,qjl", [("outlier", 3, True), ("gaussian", 3, True), ("outlier", 2, True),
                                           ("outlier", 3, False)])
def test_decode_logits_match_oracle_scores(qlaw, kbits, qjl):
    ctx = tq.Context(D, 0)
    Pi = T.rotation_from_gaussian(synth.gaussian_matrix(0, synth.TAG_ROTATION, D, D))
    S = T.sketch_from_gaussian(synth.gaussian_matrix(0, synth.TAG_SKETCH, D, D))
    B, H, Hq, cap = 2, 2, 8, 3072
    seq = [3000, 1777]
    g = Hq // H
    cb = T.codebook(D, kbits)
    K = synth.outlier_kv(31, (1,), synth.TAG_SCALES_K, (B, H, cap, D))
    if qlaw == "outlier":
        Q = synth.outlier_kv(31, (3,), synth.TAG_SCALES_K, (B, Hq, D))
    else:
        Q = synth.gaussian(31, (3,), (B, Hq, D), "bf16")
    cache = tq.KVCache(B, H, cap, D, kbits, 3, key_qjl=qjl)
    packs = {}
    for b in range(B):
        for h in range(H):
            s = b * H + h
            pk = T.pack_keys(T.encode(K[b, h], Pi, cb, S if qjl else None), kbits, qjl)
            cache.k.words[s * cap:(s + 1) * cap].copy_(torch.from_numpy(pk["bits"].view(np.int32)).to(DEV))
            cache.k.norms[s * cap:(s + 1) * cap].copy_(torch.from_numpy(pk["norms"]).to(DEV))
            packs[s] = pk
    cache.seq_len.copy_(torch.tensor(seq, dtype=torch.int32))
    cache.host_max_len = max(seq)
    scale = 1 / math.sqrt(D)
    lg = cache.decode_logits(ctx, torch.from_numpy(Q).to(DEV).to(torch.bfloat16), scale).cpu().numpy()
    torch.cuda.synchronize()
    worst_rel, worst_abs_over_ql = 0.0, 0.0
    for b in range(B):
        for h in range(H):
            pk = packs[b * H + h]
            L = seq[b]
            qh = Q[b, h * g:(h + 1) * g].astype(np.float64)
            ref = scale * T.scores(qh, Pi, S, cb, {"bits": pk["bits"][:L], "norms": pk["norms"][:L]}, qjl)
            got = lg[b, h * g:(h + 1) * g, :L].astype(np.float64)
            assert np.all(np.isnan(lg[b, h * g:(h + 1) * g, L:]))  # nothing written past the length
            kn = pk["norms"][:L].reshape(L, -1)[:, 0].astype(np.float64)
            qk = scale * np.outer(np.linalg.norm(qh, axis=1), kn)
            err = np.abs(got - ref)
            assert np.all(err <= 1e-6 * (np.abs(ref) + qk)), f"b={b} h={h}: worst {np.max(err / (np.abs(ref) + qk))}"
            worst_rel = max(worst_rel, float(np.max(err / np.maximum(np.abs(ref), 1e-30))))
            worst_abs_over_ql = max(worst_abs_over_ql, float(np.max(err / qk)))
    print(f"{qlaw} queries, b={kbits + int(qjl)}: max |dl|/(scale|q||k|) = {worst_abs_over_ql:.2e}, "
          f"max logit magnitude {np.nanmax(np.abs(lg)):.1f}")


def test_decode_logits_into_a_callers_buffer():
    """decode_logits with a caller's output buffer gives the same logits as with its
    own, and leaves the entries past each length as the buffer held them."""
    ctx = tq.Context(D, 0)
    B, H, Hq, cap = 2, 2, 8, 1024
    seq = [1000, 333]
    K = synth.outlier_kv(32, (1,), synth.TAG_SCALES_K, (B, H, cap, D))
    V = synth.outlier_kv(32, (2,), synth.TAG_SCALES_V, (B, H, cap, D))
    Q = torch.from_numpy(synth.gaussian(32, (3,), (B, Hq, D), "bf16")).to(DEV).to(torch.bfloat16)
    cache = tq.KVCache(B, H, cap, D, 3, 3)
    cache.prefill(ctx, torch.from_numpy(K).to(DEV).to(torch.bfloat16), torch.from_numpy(V).to(DEV).to(torch.bfloat16))
    cache.seq_len.copy_(torch.tensor(seq, dtype=torch.int32))
    cache.host_max_len = max(seq)
    ref = cache.decode_logits(ctx, Q)
    out = torch.full((B, Hq, cap), 7.0, dtype=torch.float32, device=DEV)
    got = cache.decode_logits(ctx, Q, out=out)
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr()
    for b in range(B):
        assert torch.equal(got[b, :, :seq[b]], ref[b, :, :seq[b]])
        assert torch.all(got[b, :, seq[b]:] == 7.0)
