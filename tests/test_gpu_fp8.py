"""Quantised KV (8-bit E4M3 codes with per-tensor scales): with unit scales the layers
give S bit for bit equal to the bf16 path on the decoded values (every E4M3 value is
exact in bf16, so the logits are the same), and O equal up to the order of its fp32
sums (the E4M3 path takes two 16-row tiles per online-softmax step, the bf16 path one,
so a running sum can round differently: O may differ in its last bf16 bit); with other
scales, paged or not, they match the oracle."""
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


def _codes(x):
    """E4M3 codes (uint8) of a float tensor, rounded to nearest even by torch."""
    return x.float().to(torch.float8_e4m3fn).view(torch.uint8)


def _decoded_bf16(codes):
    return torch.as_tensor(orc.fp8_e4m3_to_f64(codes.numpy()), dtype=torch.float32).to(torch.bfloat16)


@pytest.mark.parametrize("case", [
    # (B, Hq, Hkv, d, n, masks, waves flag)
    (1, 8, 2, 128, 5000, [0xFF, 0x11, 0x00], 0),
    (1, 8, 2, 128, 5000, [0xFF, 0x11, 0x00], 2),
    (1, 4, 4, 64, 2100, [0xF, 0x2], 0),
    (1, 16, 2, 128, 3000, [0xFFFF, 0x0101], 0),
    (1, 16, 2, 128, 3000, [0xFFFF, 0x0101], 2),
])
def test_fp8_unit_scales_equal_bf16_of_decoded(case):
    B, Hq, Hkv, d, n, masks, waves = case
    ld = _ld()
    dev = "cuda"
    k = int(0.3 * n)
    Sa = torch.zeros((B, Hq, k), dtype=torch.int32, device=dev)
    Sb = torch.zeros_like(Sa)
    wsa = wsb = None
    for l, mask in enumerate(masks):
        q, kc, vc = wl.random_qkv(B, Hq, Hkv, d, n, 800 + l)
        k8, v8 = _codes(kc), _codes(vc)
        kb, vb = _decoded_bf16(k8), _decoded_bf16(v8)
        qd = q.to(dev)
        if wsa is None:
            wsa = ld.Workspace(ld.make_shape(qd, k8.to(dev)), k, dev)
            wsb = ld.Workspace(ld.make_shape(qd, kb.to(dev)), k, dev)
        flags = (ld.FLAG_S_CHAINED if l else 0) | ld.flag_waves(waves)
        oa = ld.hybrid_layer(qd, k8.to(dev), v8.to(dev), mask, k, Sa if l else None, s_out=Sa, flags=flags,
                             workspace=wsa)
        ob = ld.hybrid_layer(qd, kb.to(dev), vb.to(dev), mask, k, Sb if l else None, s_out=Sb, flags=flags,
                             workspace=wsb)
        torch.cuda.synchronize()
        # at most one bf16 unit in the last place (2^-7 relative) apart, element by element
        oaf, obf = oa.float(), ob.float()
        assert torch.all((oaf - obf).abs() <= 2.0 ** -7 * obf.abs() + 1e-7), f"layer {l}: O differs"
        assert torch.equal(Sa, Sb), f"layer {l}: S differs"
    wsa.check()
    wsb.check()


@pytest.mark.parametrize("paged", [False, True])
def test_fp8_scaled_matches_oracle(paged):
    ld = _ld()
    dev = "cuda"
    B, Hq, Hkv, d, n, page = 1, 8, 2, 128, 4100, 64
    k = int(0.3 * n)
    k_scale, v_scale = 0.25, 3.0
    S = torch.zeros((B, Hq, k), dtype=torch.int32, device=dev)
    ws = None
    masks = [0xFF, 0x12, 0x00]
    for l, mask in enumerate(masks):
        q, kc, vc = wl.random_qkv(B, Hq, Hkv, d, n, 850 + l)
        k8, v8 = _codes(kc * 4.0), _codes(vc / 3.0)          # stored codes; values = scale * code
        qd = q.to(dev)
        if paged:
            npg = (n + page - 1) // page
            perm = torch.as_tensor(np.random.default_rng(l).permutation(npg + 3), dtype=torch.int64)
            kp = torch.zeros((Hkv, (npg + 3) * page, d), dtype=torch.uint8)
            vp = torch.zeros_like(kp)
            bt = torch.zeros((B, npg), dtype=torch.int32)
            for j in range(npg):
                pid = int(perm[j]); bt[0, j] = pid
                r0, r1 = j * page, min(n, (j + 1) * page)
                kp[:, pid * page: pid * page + r1 - r0] = k8[:, r0:r1]
                vp[:, pid * page: pid * page + r1 - r0] = v8[:, r0:r1]
            kk_, vv_, extra = kp.to(dev), vp.to(dev), dict(block_table=bt.to(dev), page_size=page, seq_len=n)
        else:
            kk_, vv_, extra = k8.to(dev), v8.to(dev), {}
        if ws is None:
            ws = ld.Workspace(ld.make_shape(qd, kk_, k_scale=k_scale, v_scale=v_scale, **extra), k, dev)
        S_before = S.cpu().numpy().copy()
        scores = torch.full((B, Hq, n), float("nan"), dtype=torch.float32, device=dev)
        out = ld.hybrid_layer(qd, kk_, vv_, mask, k, S if l else None, s_out=S, scores_out=scores,
                              flags=ld.FLAG_S_CHAINED if l else 0, workspace=ws, k_scale=k_scale,
                              v_scale=v_scale, **extra)
        torch.cuda.synchronize()
        ret = [bool(mask >> h & 1) for h in range(Hq)]
        S_in = None if l == 0 else {(0, h): S_before[0, h].astype(np.int64) for h in range(Hq)}
        O_ref, S_ref, sc_ref = orc.hybrid_layer_fp8(wl.bf16_bits(q), k8.numpy(), v8.numpy(), k_scale, v_scale,
                                                    [0, n], ret, [k], S_in)
        gh.check_outputs(out, O_ref, [(0, h) for h in range(Hq)], f"fp8 layer {l}")
        S_now = S.cpu().numpy()
        for h in range(Hq):
            if ret[h]:
                gh.check_selected_row(S_now[0, h], scores[0, h].cpu().numpy(), sc_ref[(0, h)], k,
                                      what=f"fp8 layer {l} head {h}: ")
            else:
                assert np.array_equal(S_now[0, h], S_before[0, h])
    ws.check()
