"""The hybrid-head layer over a causal prefill (ld_prefill_hybrid_layer) against the
oracle's prefill_hybrid_layer on the same bf16 bytes: every head's output rows, the
retrieval heads' column sums, and their selected sets (bit-exact on the launch's own
fp32 column sums; against the fp64 selection, differences only inside the tie zone).
Layers are chained with teacher forcing (the oracle takes the GPU's S)."""
import numpy as np
import pytest

import workloads as wl
from oracle import lychee_oracle as orc
from tests import gpu_helpers as gh

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

# Column sums: each term is a probability from fp32 scores of bf16 products and the
# row's fp32 log-sum-exp (a few ulp each), summed in fp32 over at most T/4 terms per
# lane; 2e-4 relative (plus 1e-7 absolute for tokens that receive almost nothing)
# bounds that for the prompt lengths tested here.
IMP_REL, IMP_ABS = 2e-4, 1e-7


def _ld():
    import hybrid_head_sparse_retrieval_amd as ld
    ld.load_library()
    return ld


def _qkv(B, Hq, Hkv, d, T, seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(wl.stream_seed("prefill", seed))
    q = torch.randn((Hq, B * T, d), generator=g).to(torch.bfloat16)
    k = torch.randn((Hkv, B * T, d), generator=g).to(torch.bfloat16)
    v = torch.randn((Hkv, B * T, d), generator=g).to(torch.bfloat16)
    return q, k, v


def _f64(t):
    return orc.bf16_bits_to_f64(wl.bf16_bits(t))


def _check_layer(l, B, Hq, T, k, mask, O_gpu, S_gpu, imp_gpu, O_ref, S_ref, imp_ref, S_before):
    Og = _f64(O_gpu)
    for h in range(Hq):
        for b in range(B):
            got, ref = Og[h, b * T:(b + 1) * T], O_ref[h, b * T:(b + 1) * T]
            assert np.all(np.isfinite(got)), (l, b, h)
            err = np.abs(got - ref).max()
            rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
            assert err <= gh.MAX_ABS and rel <= gh.REL_L2, (l, b, h, err, rel)
            if mask >> h & 1:
                ig, ir = imp_gpu[b, h], imp_ref[(b, h)]
                assert np.all(np.abs(ig - ir) <= IMP_REL * ir + IMP_ABS), (l, b, h, np.abs(ig - ir).max())
                # exact on the launch's own fp32 sums; tie zone against fp64
                assert np.array_equal(S_gpu[b, h], orc.select_topk_f32(ig, k)), (l, b, h)
                diff = np.setxor1d(S_gpu[b, h], S_ref[(b, h)])
                if diff.size:
                    kth = np.sort(ir)[::-1][k - 1]
                    assert np.all(np.abs(ir[diff] - kth) <= IMP_REL * kth + IMP_ABS), (l, b, h, diff[:8])
            else:
                assert np.array_equal(S_gpu[b, h], S_before[b, h]), "a sparse head's set changed"


def run_prefill(B, Hq, Hkv, d, T, k, masks, seed, separate_out=False):
    ld = _ld()
    dev = "cuda"
    S = torch.full((B, Hq, k), -1, dtype=torch.int32, device=dev)
    for l, mask in enumerate(masks):
        qc, kc, vc = _qkv(B, Hq, Hkv, d, T, seed * 10 + l)
        q, kk, vv = qc.to(dev), kc.to(dev), vc.to(dev)
        imp = torch.full((B, Hq, T), float("nan"), dtype=torch.float32, device=dev)
        S_before = S.cpu().numpy().copy()
        s_out = torch.full_like(S, -1) if separate_out else S
        out = ld.prefill_hybrid_layer(q, kk, vv, mask, k, S if l > 0 else None, batch=B, s_out=s_out,
                                      importance_out=imp)
        torch.cuda.synchronize()
        S_now = s_out.cpu().numpy()
        ret = [bool(mask >> h & 1) for h in range(Hq)]
        S_in = None if l == 0 else {(b, h): S_before[b, h].astype(np.int64) for b in range(B) for h in range(Hq)}
        O_ref, S_ref, imp_ref = orc.prefill_hybrid_layer(_f64(qc), _f64(kc), _f64(vc), B, ret, k, S_in)
        _check_layer(l, B, Hq, T, k, mask, out, S_now, imp.cpu().numpy(), O_ref, S_ref, imp_ref, S_before)
        S = s_out


@pytest.mark.parametrize("case", [
    # B, Hq, Hkv, d, T, k, masks (layer 0 all retrieval), seed
    (1, 4, 2, 64, 300, 90, [0xF, 0b0101, 0], 1),            # GQA 2:1, ragged tail (300 = 4 * 64 + 44)
    (2, 8, 2, 128, 200, 60, [0xFF, 0b00100001, 0b1000], 2),  # two sequences, GQA 4:1
    (1, 2, 2, 128, 64, 19, [0x3, 0b10], 3),                  # one query block
    (1, 2, 1, 64, 1, 1, [0x3, 0b01], 4),                     # a one-token prompt
    (1, 4, 4, 128, 2500, 1500, [0xF, 0b0010], 5),            # more than one 1024-key chunk
])
def test_prefill_layers_match_oracle(case):
    B, Hq, Hkv, d, T, k, masks, seed = case
    run_prefill(B, Hq, Hkv, d, T, k, masks, seed)


def test_separate_s_buffers_copy_sparse_rows():
    run_prefill(1, 4, 2, 64, 150, 40, [0xF, 0b1001], 6, separate_out=True)


def test_rows_before_a_sparse_set_are_zero_and_single_tokens_exact():
    """Sparse row t sees the set's tokens at or before t: rows before the first one are
    zero, and a row that sees exactly one token gets that token's V row exactly."""
    ld = _ld()
    dev = "cuda"
    B, Hq, Hkv, d, T, k = 1, 2, 1, 64, 257, 3
    qc, kc, vc = _qkv(B, Hq, Hkv, d, T, 7)
    S = torch.tensor([[[5, 100, 200], [130, 131, 256]]], dtype=torch.int32, device=dev)
    out = ld.prefill_hybrid_layer(qc.to(dev), kc.to(dev), vc.to(dev), 0, k, S)
    torch.cuda.synchronize()
    o = out.cpu()
    assert torch.all(o[0, :5] == 0) and torch.all(o[1, :130] == 0)
    assert torch.equal(o[0, 5:100], vc[0, 5].expand(95, d))      # weight exactly 1 on token 5
    assert torch.equal(o[1, 130], vc[0, 130])
    S_in = {(0, 0): np.array([5, 100, 200]), (0, 1): np.array([130, 131, 256])}
    O_ref, _, _ = orc.prefill_hybrid_layer(_f64(qc), _f64(kc), _f64(vc), B, [False, False], k, S_in)
    assert np.abs(_f64(out) - O_ref).max() <= gh.MAX_ABS


def test_skip_topk_leaves_sets_and_sums():
    ld = _ld()
    dev = "cuda"
    qc, kc, vc = _qkv(1, 4, 2, 128, 130, 8)
    S = torch.full((1, 4, 40), 7, dtype=torch.int32, device=dev)
    imp = torch.full((1, 4, 130), 3.0, dtype=torch.float32, device=dev)
    out = ld.prefill_hybrid_layer(qc.to(dev), kc.to(dev), vc.to(dev), 0xF, 40, None, s_out=S, importance_out=imp,
                                  flags=ld.FLAG_SKIP_TOPK)
    torch.cuda.synchronize()
    assert torch.all(S == 7) and torch.all(imp == 3.0)
    O_ref, _, _ = orc.prefill_hybrid_layer(_f64(qc), _f64(kc), _f64(vc), 1, [True] * 4, 40)
    assert np.abs(_f64(out) - O_ref).max() <= gh.MAX_ABS


def test_invalid_prefill_arguments_are_rejected():
    ld = _ld()
    dev = "cuda"
    q = torch.zeros((4, 100, 64), dtype=torch.bfloat16, device=dev)
    kv = torch.zeros((2, 100, 64), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ld.LycheeDecodeError):
        ld.prefill_hybrid_layer(q, kv, kv, 0b0011, 10, None)          # sparse heads without S
    with pytest.raises(ValueError):
        ld.prefill_hybrid_layer(q, kv, kv, 0xF, 10, None, batch=3)    # 100 rows are not 3 prompts


def test_llama_shape_32k_prompt_properties_and_sampled_rows():
    """A full-attention prefill layer at the Llama-3-8B head shape and a 32K prompt: the
    sums of every head add up to T (each attention row sums to one), the sets equal
    the selection on the launch's own sums, and sampled rows of every head match the
    decode oracle on their prefix."""
    ld = _ld()
    dev = "cuda"
    B, Hq, Hkv, d, T = 1, 32, 8, 128, 32768
    k = int(0.3 * T)
    g = torch.Generator(device=dev)
    g.manual_seed(wl.stream_seed("prefill-32k"))
    q = torch.randn((Hq, T, d), generator=g, device=dev).to(torch.bfloat16)
    kc = torch.randn((Hkv, T, d), generator=g, device=dev).to(torch.bfloat16)
    vc = torch.randn((Hkv, T, d), generator=g, device=dev).to(torch.bfloat16)
    S = torch.empty((B, Hq, k), dtype=torch.int32, device=dev)
    imp = torch.empty((B, Hq, T), dtype=torch.float32, device=dev)
    out = ld.prefill_hybrid_layer(q, kc, vc, (1 << Hq) - 1, k, None, s_out=S, importance_out=imp)
    torch.cuda.synchronize()
    impc, Sc = imp.cpu().numpy(), S.cpu().numpy()
    for h in range(Hq):
        assert abs(float(impc[0, h].astype(np.float64).sum()) - T) <= 1e-3 * T, h
        assert np.all(impc[0, h] >= 0)
        assert np.array_equal(Sc[0, h], orc.select_topk_f32(impc[0, h], k)), h
    rng = np.random.default_rng(9)
    Og = _f64(out)
    sc = orc.default_scale(d)
    for h in (0, 7, 13, 31):
        Kg, Vg = _f64(kc[h // 4]), _f64(vc[h // 4])
        qh = _f64(q[h])
        for t in sorted({0, 63, 64, T - 1} | set(int(x) for x in rng.integers(0, T, 3))):
            want, _ = orc.softmax_attention(qh[t], Kg[:t + 1], Vg[:t + 1], sc)
            err = np.abs(Og[h, t] - want).max()
            assert err <= gh.MAX_ABS, (h, t, err)
