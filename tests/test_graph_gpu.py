"""The decode loop captured in a HIP graph (torch.cuda.CUDAGraph over the
library's launches) and replayed.

The library enqueues only kernel launches on the caller's stream (no memory
sets, no allocation, no synchronisation), so a loop of steps can be captured
once and replayed without host launch overhead. Each replay is checked bit
for bit against the same loop run eagerly, with the program's own eager work
(resetting the caches and lengths, reading results back) and
synchronisations between the replays; every replay is also held to the
oracle bar at its last step.
"""
import numpy as np
import pytest
import torch

from gpu_util import assert_parity, to_dev, to_host_bits
from gqa_kv_cache_decode_amd import api, inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,b,h,g,d,lens", [
    ("bf16", 4, 28, 4, 128, [100, 300, 511, 64]),     # matrix path
    ("f32", 2, 4, 2, 16, [37, 64]),                    # vector path (the tiny fp32 shape)
    ("bf16", 2, 32, 1, 128, [700, 1300]),              # matrix path, merged by a second launch
])
def test_graph_replay_of_a_decode_loop(gpu_lib, oracle_mod, dtype, b, h, g, d, lens):
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
            api.decode_step(outs[s], qs[s], news[s][0], news[s][1], kc, vc, lens_d, m + s, scale, ws)

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
