"""Token-block selection (HySparse form): every retrieval row keeps the k/64 blocks of
64 tokens with the largest block maxima of its logits. S equals the oracle's block
selection on the GPU's own fp32 logits bit for bit, the sparse layers that read it
match the oracle, and a HySparse stack (one full layer, sparse layers on its KV and
its blocks) gathers whole blocks."""
import numpy as np
import pytest

import workloads as wl
from oracle import lychee_oracle as orc
from tests import gpu_helpers as gh

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _ld():
    import hybrid_head_sparse_retrieval_amd as ld
    ld.load_library()
    return ld


@pytest.mark.parametrize("case", [
    # (Hq, Hkv, d, n, k, masks, shared_kv)
    (8, 2, 128, 4096, 1280, [0xFF, 0x12, 0x00], False),
    (4, 4, 64, 2048, 640, [0xF, 0x1], False),
    (8, 2, 128, 8192, 2048, [0xFF, 0x00, 0x00, 0x00], True),
])
def test_block_selection_matches_oracle(case):
    Hq, Hkv, d, n, k, masks, shared = case
    ld = _ld()
    dev = "cuda"
    B = 1
    S = torch.zeros((B, Hq, k), dtype=torch.int32, device=dev)
    scores = torch.full((B, Hq, n), float("nan"), dtype=torch.float32, device=dev)
    ws = None
    base = wl.random_qkv(B, Hq, Hkv, d, n, 950)
    for l, mask in enumerate(masks):
        q, kc, vc = wl.random_qkv(B, Hq, Hkv, d, n, 951 + l)
        if shared:
            kc, vc = base[1], base[2]
        qd, kd, vd = q.to(dev), kc.to(dev), vc.to(dev)
        if ws is None:
            ws = ld.Workspace(ld.make_shape(qd, kd), k, dev)
        S_before = S.cpu().numpy().copy()
        flags = ld.FLAG_BLOCK_SELECT | (ld.FLAG_S_CHAINED if l else 0)
        out = ld.hybrid_layer(qd, kd, vd, mask, k, S if l else None, s_out=S, scores_out=scores, flags=flags,
                              workspace=ws)
        torch.cuda.synchronize()
        S_now = S.cpu().numpy()
        sc = scores.cpu().numpy()
        ret = [bool(mask >> h & 1) for h in range(Hq)]
        for h in range(Hq):
            if ret[h]:
                exact = orc.select_topk_blocks(sc[0, h].astype(np.float32), k, 64)
                assert np.array_equal(S_now[0, h], exact), f"layer {l} head {h}"
            else:
                assert np.array_equal(S_now[0, h], S_before[0, h])
        S_in = None if l == 0 else {(0, h): S_before[0, h].astype(np.int64) for h in range(Hq)}
        O_ref, _, _ = orc.hybrid_layer_bf16(wl.bf16_bits(q), wl.bf16_bits(kc), wl.bf16_bits(vc), [0, n], ret,
                                            [k], S_in)
        gh.check_outputs(out, O_ref, [(0, h) for h in range(Hq)], f"block layer {l}")
    ws.check()


def test_block_selection_rejects_unsupported_shapes():
    ld = _ld()
    dev = "cuda"
    q, kc, vc = wl.random_qkv(1, 4, 4, 64, 2048, 960)
    qd, kd, vd = q.to(dev), kc.to(dev), vc.to(dev)
    ws = ld.Workspace(ld.make_shape(qd, kd), 700, dev)
    S = torch.zeros((1, 4, 700), dtype=torch.int32, device=dev)
    with pytest.raises(ld.LycheeDecodeError, match="invalid argument"):
        ld.hybrid_layer(qd, kd, vd, 0xF, 700, None, s_out=S, flags=ld.FLAG_BLOCK_SELECT, workspace=ws)
