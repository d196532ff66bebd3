"""GPU parity of the PolarQuant keys (d = 128) against oracle/polarquant.py.

Records: every angle code equals the oracle's except where the oracle's angle
lies inside the band the fp32 rotation can move it by (1e-5 rad plus
1e-6 ||x|| / rho for a node of radius rho: a small radius makes its angle
sensitive) -- there the code may differ by one cell (or wrap around the
circle at level 1) -- and at most 1e-3 of the codes may be so excused;
||x|| within 2e-6 relative. Scores over identical records (oracle-packed,
uploaded): |ds| <= 1e-3 |s| or 1e-6 ||q|| ||x||."""
import math

import numpy as np
import pytest

import synth
from oracle import polarquant as PQ
from oracle import turboquant as T
from tests import parity as P

torch = pytest.importorskip("torch")
tq = pytest.importorskip("kv_cache_vector_turboquant_amd")

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

pytestmark = pytest.mark.gpu
DEV = "cuda"
CONFIGS = [(4, 3), (2, 2), (3, 1), (1, 4)]


@pytest.fixture(scope="module")
def ctx_pi():
    ctx = tq.Context(128, 0)
    Pi = T.rotation_from_gaussian(synth.gaussian_matrix(0, synth.TAG_ROTATION, 128, 128))
    return ctx, Pi


def _dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def _node_radii(Y):
    """Radii of the nodes whose angles each level holds: level 1 pair radii for
    level-1 angles, then for level l the radius of the node that owns the angle."""
    a, b = Y[:, 0::2], Y[:, 1::2]
    out = [np.hypot(a, b)]
    r = out[0]
    while r.shape[1] > 1:
        r = np.hypot(r[:, 0::2], r[:, 1::2])
        out.append(r)
    return out


def check_polar_records(words, norms, X, Pi, pcb):
    g = PQ.unpack_polar(words, pcb)
    enc = PQ.polar_encode(X, Pi, pcb)
    Y = X.astype(np.float64) @ Pi.astype(np.float64).T
    radii = _node_radii(Y)
    xn = np.linalg.norm(X.astype(np.float64), axis=1)
    total = excused = 0
    for lv in range(1, pcb.L + 1):
        gc, oc = g[lv - 1], enc.codes[lv - 1]
        cb = pcb.levels[lv - 1]
        diff = gc != oc
        total += gc.size
        if diff.any():
            psi = enc.angles[lv - 1]
            dist = np.min(np.abs(psi[..., None] - cb.boundaries.astype(np.float64)), axis=-1)
            if lv == 1:  # the circle's seam at -pi / pi
                dist = np.minimum(dist, math.pi - np.abs(psi))
            band = 1e-5 + 1e-6 * xn[:, None] / np.maximum(radii[lv - 1], 1e-300)
            bad = diff & ~(dist <= band)
            assert not bad.any(), f"level {lv}: {int(bad.sum())} code mismatches outside the band"
            step = np.abs(gc[diff] - oc[diff])
            L = 1 << cb.bits
            assert np.all((step == 1) | ((lv == 1) & (step == L - 1))), f"level {lv}: non-adjacent code"
            excused += int(diff.sum())
    assert excused <= 1e-3 * total, f"{excused} excused codes of {total}"
    assert np.all(np.abs(norms - enc.norm) <= 2e-6 * enc.norm + 1e-30), "||x|| mismatch"
    return excused


@pytest.mark.parametrize("b1,b2", CONFIGS)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_polar_quantize_records(ctx_pi, b1, b2, dtype):
    """1001 outlier-channel vectors (a ragged last block of 4) into records
    32 .. 1032 of a 1100-record array; three zero vectors among them."""
    ctx, Pi = ctx_pi
    n = 1001
    X = synth.outlier_kv(71, (b1, b2), synth.TAG_SCALES_K, (n, 128), dtype)
    X[[0, 500, 1000]] = 0.0
    out = tq.PolarPacked(1100, b1, b2)
    tq.polar_quantize(ctx, _dev(X, dtype), out, 32)
    words, norms = out.host()
    pcb = PQ.polar_codebooks(128, b1, b2)
    check_polar_records(words[32:32 + n], norms[32:32 + n], X, Pi, pcb)
    assert not words[:32].any() and not words[32 + n:].any()  # nothing outside the range written
    zero_rec = PQ.pack_polar(PQ.polar_encode(np.zeros((1, 128)), Pi, pcb), pcb)["bits"][0]
    for z in (0, 500, 1000):
        assert norms[32 + z] == 0 and np.array_equal(words[32 + z], zero_rec)


@pytest.mark.parametrize("b1,b2", CONFIGS)
def test_polar_scores(ctx_pi, b1, b2):
    """Scores of 37 bf16 queries against 3000 oracle-packed keys (identical
    records on both sides)."""
    ctx, Pi = ctx_pi
    n, nq = 3000, 37
    pcb = PQ.polar_codebooks(128, b1, b2)
    X = synth.outlier_kv(72, (b1, b2), synth.TAG_SCALES_K, (n, 128))
    Q = synth.gaussian(72, (b1, b2, 1), (nq, 128), "bf16")
    rec = PQ.pack_polar(PQ.polar_encode(X, Pi, pcb), pcb)
    keys = tq.PolarPacked(n, b1, b2)
    keys.words.copy_(torch.from_numpy(rec["bits"].view(np.int32)).to(DEV))
    keys.norms.copy_(torch.from_numpy(rec["norms"]).to(DEV))
    s = tq.polar_scores(ctx, _dev(Q, "bf16"), keys).cpu().numpy()
    ref = PQ.polar_scores(Q, Pi, pcb, rec)
    P.check_scores(s, ref, np.linalg.norm(Q, axis=1), np.linalg.norm(X, axis=1))


def test_polar_end_to_end_inner_products(ctx_pi):
    """GPU-encoded keys scored on the GPU estimate <q, x> about as well as the
    oracle's own encoding: the mean relative error of the inner products
    matches the oracle's within 5% (code flips inside the band are rare)."""
    ctx, Pi = ctx_pi
    n = 4000
    X = synth.gaussian(73, (1,), (n, 128))
    Q = synth.gaussian(73, (2,), (8, 128))
    keys = tq.PolarPacked(n)
    tq.polar_quantize(ctx, _dev(X, "f32"), keys)
    s = tq.polar_scores(ctx, _dev(Q, "f32"), keys).cpu().numpy()
    pcb = PQ.polar_codebooks(128, 4, 3)
    ref = PQ.polar_scores(Q, Pi, pcb, PQ.pack_polar(PQ.polar_encode(X, Pi, pcb), pcb))
    exact = Q.astype(np.float64) @ X.astype(np.float64).T
    scale = np.linalg.norm(Q, axis=1)[:, None] * np.linalg.norm(X, axis=1)[None, :]
    e_gpu = np.mean(np.abs(s - exact) / scale)
    e_ora = np.mean(np.abs(ref - exact) / scale)
    assert abs(e_gpu - e_ora) <= 0.05 * e_ora and e_ora < 0.05


def test_polar_argument_errors(ctx_pi):
    ctx, _ = ctx_pi
    keys = tq.PolarPacked(10)
    x = torch.zeros((20, 128), device=DEV)
    with pytest.raises(tq.TQError):
        tq.polar_quantize(ctx, x, keys)  # 20 records into a 10-record array
    bad = tq.PolarPacked(10, 5, 3)
    with pytest.raises(tq.TQError):
        tq.polar_quantize(ctx, x[:10], bad)  # b1 out of range
    c256 = tq.Context(256, 1)
    with pytest.raises(tq.TQError):
        tq.polar_quantize(c256, torch.zeros((4, 256), device=DEV), keys)  # d != 128
    torch.cuda.synchronize()


@pytest.mark.parametrize("hq", [8, 32])
def test_polar_attention_decode(ctx_pi, hq):
    """batch 3 (lengths 1500, 0, 777), 2 KV heads, groups of 4 or 16 query
    heads: decode attention over PolarQuant keys (oracle-packed, uploaded) and
    3-bit stage-1 values within 2e-3 max-abs of the oracle; a sequence with no
    tokens gives zeros."""
    ctx, Pi = ctx_pi
    B, H, cap, L, d = 3, 2, 1536, 1500, 128
    seq = [1500, 0, 777]
    pcb = PQ.polar_codebooks(128, 4, 3)
    cbv = T.codebook(d, 3)
    K = synth.outlier_kv(74, (hq, 1), synth.TAG_SCALES_K, (B, H, L, d))
    V = synth.outlier_kv(74, (hq, 2), synth.TAG_SCALES_V, (B, H, L, d))
    Q = synth.gaussian(74, (hq, 3), (B, hq, d), "bf16")
    cache = tq.PolarKVCache(B, H, cap)
    recs = {}
    for b in range(B):
        for h in range(H):
            s = b * H + h
            kr = PQ.pack_polar(PQ.polar_encode(K[b, h], Pi, pcb), pcb)
            vr = T.pack_values(T.encode(V[b, h], Pi, cbv), 3)
            cache.keys.words[s * cap:s * cap + L].copy_(torch.from_numpy(kr["bits"].view(np.int32)).to(DEV))
            cache.keys.norms[s * cap:s * cap + L].copy_(torch.from_numpy(kr["norms"]).to(DEV))
            nb = vr["bits"].shape[0]
            cache.values.v.words[s * cap // 32:s * cap // 32 + nb].copy_(torch.from_numpy(vr["bits"].view(np.int32)).to(DEV))
            cache.values.v.norms[s * cap:s * cap + L].copy_(torch.from_numpy(vr["norms"]).to(DEV))
            recs[s] = (kr, vr)
    cache.seq_len.copy_(torch.tensor(seq, dtype=torch.int32))
    cache.host_max_len = max(seq)
    scale = 1 / math.sqrt(d)
    out = cache.decode(ctx, _dev(Q, "bf16"), scale).cpu().numpy()
    g = hq // H
    for b in range(B):
        for h in range(H):
            kr, vr = recs[b * H + h]
            n = seq[b]
            if n == 0:
                assert not out[b, h * g:(h + 1) * g].any()
                continue
            ref = PQ.polar_attention_decode(Q[b, h * g:(h + 1) * g], Pi, pcb, cbv, kr,
                                            {"bits": vr["bits"], "norms": vr["norms"][:n]}, n, scale,
                                            T.unpack_values)
            assert np.max(np.abs(out[b, h * g:(h + 1) * g] - ref)) <= 2e-3, f"b={b} h={h}"


@pytest.mark.parametrize("b1,b2,qdtype", [(2, 2, "f32"), (3, 1, "bf16"), (1, 4, "f32"), (4, 4, "bf16")])
def test_polar_attention_decode_code_widths(ctx_pi, b1, b2, qdtype):
    """Decode attention over PolarQuant keys of other code widths (the scoring
    kernel is compiled per width pair) and fp32 or bf16 queries: batch 2
    (lengths 700, 333), 2 KV heads, groups of 4, within 2e-3 max-abs of the oracle."""
    ctx, Pi = ctx_pi
    B, H, cap, L, d, hq = 2, 2, 704, 700, 128, 8
    seq = [700, 333]
    pcb = PQ.polar_codebooks(128, b1, b2)
    cbv = T.codebook(d, 3)
    K = synth.outlier_kv(76, (b1, b2, 1), synth.TAG_SCALES_K, (B, H, L, d))
    V = synth.outlier_kv(76, (b1, b2, 2), synth.TAG_SCALES_V, (B, H, L, d))
    Q = synth.gaussian(76, (b1, b2, 3), (B, hq, d), qdtype)
    cache = tq.PolarKVCache(B, H, cap, b1=b1, b2=b2)
    recs = {}
    for b in range(B):
        for h in range(H):
            s = b * H + h
            kr = PQ.pack_polar(PQ.polar_encode(K[b, h], Pi, pcb), pcb)
            vr = T.pack_values(T.encode(V[b, h], Pi, cbv), 3)
            cache.keys.words[s * cap:s * cap + L].copy_(torch.from_numpy(kr["bits"].view(np.int32)).to(DEV))
            cache.keys.norms[s * cap:s * cap + L].copy_(torch.from_numpy(kr["norms"]).to(DEV))
            nb = vr["bits"].shape[0]
            cache.values.v.words[s * cap // 32:s * cap // 32 + nb].copy_(torch.from_numpy(vr["bits"].view(np.int32)).to(DEV))
            cache.values.v.norms[s * cap:s * cap + L].copy_(torch.from_numpy(vr["norms"]).to(DEV))
            recs[s] = (kr, vr)
    cache.seq_len.copy_(torch.tensor(seq, dtype=torch.int32))
    cache.host_max_len = max(seq)
    scale = 1 / math.sqrt(d)
    out = cache.decode(ctx, _dev(Q, qdtype), scale).cpu().numpy()
    g = hq // H
    for b in range(B):
        for h in range(H):
            kr, vr = recs[b * H + h]
            n = seq[b]
            ref = PQ.polar_attention_decode(Q[b, h * g:(h + 1) * g], Pi, pcb, cbv,
                                            {"bits": kr["bits"][:n], "norms": kr["norms"][:n]},
                                            {"bits": vr["bits"], "norms": vr["norms"][:n]}, n, scale,
                                            T.unpack_values)
            assert np.max(np.abs(out[b, h * g:(h + 1) * g] - ref)) <= 2e-3, f"b={b} h={h}"


def test_polar_cache_prefill_and_decode(ctx_pi):
    """PolarKVCache.prefill encodes keys on the GPU (stream-strided records) and
    values with the fused quantize; decode over them matches the oracle over the
    records the GPU wrote."""
    ctx, Pi = ctx_pi
    B, H, cap, L, d, hq = 2, 2, 640, 600, 128, 8
    K = synth.outlier_kv(75, (1,), synth.TAG_SCALES_K, (B, H, L, d), "bf16")
    V = synth.outlier_kv(75, (2,), synth.TAG_SCALES_V, (B, H, L, d), "bf16")
    Q = synth.gaussian(75, (3,), (B, hq, d), "bf16")
    cache = tq.PolarKVCache(B, H, cap)
    cache.prefill(ctx, _dev(K, "bf16"), _dev(V, "bf16"))
    out = cache.decode(ctx, _dev(Q, "bf16")).cpu().numpy()
    kw, kn = cache.keys.host()
    vw, vn = cache.values.v.host()
    pcb = PQ.polar_codebooks(128, 4, 3)
    cbv = T.codebook(d, 3)
    for b in range(B):
        for h in range(H):
            s = b * H + h
            check_polar_records(kw[s * cap:s * cap + L], kn[s * cap:s * cap + L], K[b, h], Pi, pcb)
            ref = PQ.polar_attention_decode(Q[b, h * 4:h * 4 + 4], Pi, pcb, cbv,
                                            {"bits": kw[s * cap:s * cap + L], "norms": kn[s * cap:s * cap + L]},
                                            {"bits": vw[s * cap // 32:(s + 1) * cap // 32], "norms": vn[s * cap:s * cap + L]},
                                            L, 1 / math.sqrt(d), T.unpack_values)
            assert np.max(np.abs(out[b, h * 4:h * 4 + 4] - ref)) <= 2e-3
