"""A decode step captured in a HIP graph and replayed gives the eager step's O and S
bit for bit on every replay (the launches take only by-value arguments and leave the
workspace ready for the next call: counters at zero, per-group call epochs advanced,
which changes no arithmetic)."""
import numpy as np
import pytest

import workloads as wl

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def test_step_graph_replays_match_eager():
    import hybrid_head_sparse_retrieval_amd as ld
    from hybrid_head_sparse_retrieval_amd.step import DecodeStep
    ld.load_library()
    dev = "cuda"
    B, Hq, Hkv, d, n = 1, 8, 2, 128, 5000
    masks = [0xFF, 0b00100001, 0, 0b00001100, 0b00010000]
    k = (3 * n) // 10
    layers = []
    for l in range(len(masks)):
        q, kc, vc = wl.random_qkv(B, Hq, Hkv, d, n, 300 + l)
        layers.append((q.to(dev), kc.to(dev), vc.to(dev)))
    step = DecodeStep(B, Hq, Hkv, d, [n], [k], masks, device=dev)
    step.run(layers)
    torch.cuda.synchronize()
    ref_o = [o.clone() for o in step.outs]
    ref_s = step.S.clone()

    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        step.run(layers)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=cap):
            step.run(layers)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    scratch = torch.zeros(1 << 20, device=dev)
    for rep in range(4):
        for o in step.outs:
            o.fill_(7.0)
        step.S.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        for l, o in enumerate(step.outs):
            assert torch.equal(o, ref_o[l]), f"replay {rep}: layer {l} output differs"
        assert torch.equal(step.S, ref_s), f"replay {rep}: S differs"
        scratch.add_(1.0)               # eager work between replays
        step.run(layers)                 # and an eager step on the same workspace
        torch.cuda.synchronize()
        assert torch.equal(step.S, ref_s)
