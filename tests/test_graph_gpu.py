"""Decode loops captured in a HIP graph (torch.cuda.CUDAGraph over the
library's launches) and replayed.

The library enqueues only kernel launches on the caller's stream (no memory
sets, no allocation, no synchronisation), so a loop of steps can be captured
once and replayed without host launch overhead. Each replay is checked bit
for bit against the same loop run eagerly, with the program's own eager work
(resetting the caches and lengths, reading results back) and
synchronisations between the replays; every replay is also held to the
oracle bar at its last step. Covered: the fused one-token step on both paths
and with the split merge by a second launch or by the parts themselves, the multi-token step (append +
attention, two launches per step) on contiguous and paged caches, and the
fused step over a block pool.
"""
import numpy as np
import pytest
import torch

from gpu_util import assert_parity, to_dev, to_host_bits
from gqa_kv_cache_decode_amd import api, inputs
from paged_util import make_paged

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,b,h,g,d,lens,path", [
    ("bf16", 4, 28, 4, 128, [100, 300, 511, 64], api.PATH_AUTO),     # matrix path
    ("f32", 2, 4, 2, 16, [37, 64], api.PATH_AUTO),                    # vector path (the tiny fp32 shape)
    ("bf16", 2, 32, 1, 128, [700, 1300], api.PATH_AUTO),              # matrix path, merged by a second launch
    # merged by the parts at the end of the launch: the generation advances on every replay
    ("bf16", 2, 32, 1, 128, [700, 1300], api.PATH_MATRIX | api.MERGE_SPREAD),
])
def test_graph_replay_of_a_decode_loop(gpu_lib, oracle_mod, dtype, b, h, g, d, lens, path):
    steps = 6
    cap = max(lens) + steps + 4
    bt = inputs.Batch(seed=1600 + h + g, b=b, h=h, g=g, d=d, cap=cap, lens=lens, dtype=dtype, poison=True)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    scale = float(np.float32(1.0 / np.sqrt(d)))
    kc0, vc0 = to_dev(bt.k_cache), to_dev(bt.v_cache)
    lens0 = torch.from_numpy(bt.lens.copy()).cuda()
    qs = [to_dev(bt.q(s)) for s in range(steps)]
    news = [tuple(to_dev(a) for a in bt.new_kv(s)) for s in range(steps)]
    ws = api.make_workspace(b, h, g, d, d, cap, tdt, "cuda")
    kc, vc, lens_d = kc0.clone(), vc0.clone(), lens0.clone()
    outs = [torch.empty(b, h, d, dtype=tdt, device="cuda") for _ in range(steps)]

    def loop():
        m = int(bt.lens.max())
        for s in range(steps):
            api.decode_step(outs[s], qs[s], news[s][0], news[s][1], kc, vc, lens_d, m + s, scale, ws, path=path)

    def reset():
        kc.copy_(kc0)
        vc.copy_(vc0)
        lens_d.copy_(lens0)

    # eager reference run (also fills the library's per-device caches before capture)
    loop()
    torch.cuda.synchronize()
    want = [to_host_bits(o) for o in outs]
    want_k, want_lens = to_host_bits(kc), lens_d.cpu().numpy()

    reset()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        loop()
    torch.cuda.synchronize()
    for replay in range(3):
        reset()
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for s in range(steps):
            assert np.array_equal(to_host_bits(outs[s]).view(np.uint16 if dtype == "bf16" else np.uint32),
                                  want[s].view(np.uint16 if dtype == "bf16" else np.uint32)), (replay, s)
        assert np.array_equal(to_host_bits(kc).view(np.uint8), want_k.view(np.uint8))
        assert np.array_equal(lens_d.cpu().numpy(), want_lens)
    # and the replayed loop is the decode loop: its last step against the oracle
    kh, vh, lh = bt.k_cache.copy(), bt.v_cache.copy(), bt.lens.copy()
    for s in range(steps):
        kn, vn = bt.new_kv(s)
        oracle_mod.kv_append(kh, vh, kn, vn, lh)
    assert_parity(outs[-1], oracle_mod.decode_attention(bt.q(steps - 1), kh, vh, lh, scale), dtype, "graph replay")


@pytest.mark.parametrize("form,dtype,b,h,g,d,n,lens,bs", [
    ("multi", "bf16", 3, 32, 4, 128, 4, [100, 300, 63], 32),          # append + causal attention, matrix path
    ("multi_paged", "bf16", 3, 16, 2, 128, 2, [40, 97, 200], 64),     # the same over a block pool
    ("paged", "f32", 2, 8, 4, 64, 1, [31, 150], 32),                  # fused one-token step over a pool, vector path
])
def test_graph_replay_of_paged_and_multi_token_loops(gpu_lib, oracle_mod, form, dtype, b, h, g, d, n, lens, bs):
    steps = 3
    cap = (max(lens) + n * steps + 4 + bs - 1) // bs * bs
    bt = inputs.Batch(seed=1700 + h + n, b=b, h=h, g=g, d=d, cap=cap, lens=lens, dtype=dtype, poison=True)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    scale = float(np.float32(1.0 / np.sqrt(d)))
    rng = np.random.default_rng(1800 + h)

    def draw(*shape):
        x = rng.standard_normal(shape).astype(np.float32)
        return inputs.f32_to_bf16_bits(x) if dtype == "bf16" else x
    paged = form != "multi"
    if paged:
        kp, table_h = make_paged(bt.k_cache, bt.lens, bs, np.random.default_rng(1900 + h), room=n * steps)
        vp, _ = make_paged(bt.v_cache, bt.lens, bs, np.random.default_rng(1900 + h), room=n * steps)
        kc0, vc0, table = to_dev(kp), to_dev(vp), torch.from_numpy(table_h).cuda()
    else:
        kc0, vc0 = to_dev(bt.k_cache), to_dev(bt.v_cache)
    lens0 = torch.from_numpy(bt.lens.copy()).cuda()
    if n > 1:
        q_h = [draw(b, n, h, d) for _ in range(steps)]
        new_h = [(draw(b, n, g, d), draw(b, n, g, d)) for _ in range(steps)]
        ws = api.make_multi_workspace(b, n, h, g, d, d, tdt, "cuda")
        outs = [torch.empty(b, n, h, d, dtype=tdt, device="cuda") for _ in range(steps)]
    else:
        q_h = [bt.q(s) for s in range(steps)]
        new_h = [bt.new_kv(s) for s in range(steps)]
        ws = api.make_workspace(b, h, g, d, d, cap, tdt, "cuda")
        outs = [torch.empty(b, h, d, dtype=tdt, device="cuda") for _ in range(steps)]
    qs = [to_dev(x) for x in q_h]
    news = [(to_dev(kn), to_dev(vn)) for kn, vn in new_h]
    kc, vc, lens_d = kc0.clone(), vc0.clone(), lens0.clone()

    def loop():
        m = int(bt.lens.max())
        for s in range(steps):
            if form == "multi":
                api.decode_step_multi(outs[s], qs[s], news[s][0], news[s][1], kc, vc, lens_d, m + n * s, scale, ws)
            elif form == "multi_paged":
                api.decode_step_multi_paged(outs[s], qs[s], news[s][0], news[s][1], kc, vc, lens_d, table, m + n * s,
                                            scale, ws)
            else:
                api.decode_step_paged(outs[s], qs[s], news[s][0], news[s][1], kc, vc, lens_d, table, m + s, scale, ws)

    def reset():
        kc.copy_(kc0)
        vc.copy_(vc0)
        lens_d.copy_(lens0)

    loop()
    torch.cuda.synchronize()
    bits = np.uint16 if dtype == "bf16" else np.uint32
    want = [to_host_bits(o).view(bits) for o in outs]
    want_k, want_lens = to_host_bits(kc).view(np.uint8), lens_d.cpu().numpy()
    reset()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        loop()
    torch.cuda.synchronize()
    for replay in range(3):
        reset()
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for s in range(steps):
            assert np.array_equal(to_host_bits(outs[s]).view(bits), want[s]), (replay, s)
        assert np.array_equal(to_host_bits(kc).view(np.uint8), want_k)
        assert np.array_equal(lens_d.cpu().numpy(), want_lens)
    # the loop against the oracle at its last step (a pool stands for its contiguous cache)
    kh, vh, lh = bt.k_cache.copy(), bt.v_cache.copy(), bt.lens.copy()
    for kn, vn in new_h:
        if n > 1:
            oracle_mod.kv_append_multi(kh, vh, kn, vn, lh)
        else:
            oracle_mod.kv_append(kh, vh, kn, vn, lh)
    ref = oracle_mod.decode_attention_multi(q_h[-1], kh, vh, lh, scale) if n > 1 else \
        oracle_mod.decode_attention(q_h[-1], kh, vh, lh, scale)
    assert_parity(outs[-1], ref, dtype, f"graph replay {form}")
