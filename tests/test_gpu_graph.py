"""HIP graph capture of the serving hot path. A prefill (tq_quantize_kv of all
K/V into the cache) and a run of fused decode steps (tq_decode_step) are
captured once with torch.cuda.graph and replayed several times, with eager work
and synchronisation between replays; every replay reproduces the eager run bit
for bit (same kernels on the same inputs): the step outputs, the appended
records and the device lengths. The library's hot-path calls only launch
kernels (no allocation, memset or host synchronisation), so they capture; the
host-side length (host_max_len) advances once, during capture, and fixes each
captured launch's chunk count, so a replay starts from the captured state."""
import numpy as np
import pytest

import synth

torch = pytest.importorskip("torch")
tq = pytest.importorskip("kv_cache_vector_turboquant_amd")

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("key_bits,qjl", [(3, True), (2, False)], ids=["tq4", "mse2"])
def test_graph_replays_match_eager(key_bits, qjl):
    B, H, Hq, L0, NS, cap, d = 2, 2, 8, 200, 6, 256, 128
    ctx = tq.Context(d, 0)
    K = synth.torch_outlier_kv(31, (1,), synth.TAG_SCALES_K, (B, H, L0, d), torch.bfloat16, DEV)
    V = synth.torch_outlier_kv(31, (2,), synth.TAG_SCALES_V, (B, H, L0, d), torch.bfloat16, DEV)
    KA = synth.torch_outlier_kv(31, (3,), synth.TAG_SCALES_K, (NS, B, H, d), torch.bfloat16, DEV)
    VA = synth.torch_outlier_kv(31, (4,), synth.TAG_SCALES_V, (NS, B, H, d), torch.bfloat16, DEV)
    Q = synth.torch_gaussian(31, (5,), (NS, B, Hq, d), torch.bfloat16, DEV)
    cache = tq.KVCache(B, H, cap, d, key_bits, 3, key_qjl=qjl)
    kwork = torch.empty(max(tq.quantize_ws_bytes(ctx, B * H, L0, True), 4), dtype=torch.uint8, device=DEV)
    cache.host_max_len = cap
    ws = torch.empty(cache.decode_step_ws_bytes(ctx, Hq), dtype=torch.uint8, device=DEV)
    outs = torch.empty((NS, B, Hq, d), dtype=torch.float32, device=DEV)

    def run():
        tq.quantize_kv(ctx, K.view(B * H, L0, d), cache.k, out_stream_stride=cap, work=kwork)
        tq.quantize_kv(ctx, V.view(B * H, L0, d), cache.v, out_stream_stride=cap)
        cache.seq_len.fill_(L0)
        cache.host_max_len = L0
        for i in range(NS):
            cache.decode_step(ctx, KA[i], VA[i], Q[i], out=outs[i], ws=ws)

    run()
    torch.cuda.synchronize()
    ref_out, ref_k, ref_v = outs.clone(), cache.k.words.clone(), cache.v.words.clone()
    ref_len = cache.seq_len.clone()
    assert ref_len.tolist() == [L0 + NS] * B and cache.host_max_len == L0 + NS

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()  # warm-up on the capture stream's side, as torch recommends
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        # eager work between replays: clobber everything the graph writes
        outs.fill_(float(rep + 1))
        cache.seq_len.zero_()
        cache.k.words.zero_()
        cache.v.words.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(outs, ref_out), f"replay {rep}: outputs differ"
        assert torch.equal(cache.k.words, ref_k) and torch.equal(cache.v.words, ref_v), f"replay {rep}: records differ"
        assert torch.equal(cache.seq_len, ref_len), f"replay {rep}: lengths differ"
        assert np.isfinite(outs.cpu().numpy()).all()
