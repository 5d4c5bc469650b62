"""Token Sparse Attention (compress -> dense -> scatter) through the C ABI: the selected
positions equal the oracle's selection on the same fp32 scores bit for bit, every
selected row of the output matches the oracle, and every other row is zero (zero fill)
or keeps what the caller wrote."""
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


def _inputs(B, Hq, Hkv, d, T, seed):
    g = torch.Generator().manual_seed(wl.stream_seed("tsa", seed))
    q = torch.randn((Hq, B * T, d), generator=g).to(torch.bfloat16)
    k = torch.randn((Hkv, B * T, d), generator=g).to(torch.bfloat16)
    v = torch.randn((Hkv, B * T, d), generator=g).to(torch.bfloat16)
    sc = torch.randn((B, Hq, T), generator=g)
    return q, k, v, sc


def _check(ld, B, Hq, Hkv, d, T, k, causal, seed, zero_fill=True):
    dev = "cuda"
    q, kc, vc, sc = _inputs(B, Hq, Hkv, d, T, seed)
    sentinel = torch.full_like(q, 7.0)
    out, idx = ld.tsa_attention(q.to(dev), kc.to(dev), vc.to(dev), sc.to(dev), k, out=sentinel.to(dev),
                                causal=causal, zero_fill=zero_fill)
    torch.cuda.synchronize()
    ref, ref_idx = orc.tsa_attention(gh.bf16_tensor_to_f64(q), gh.bf16_tensor_to_f64(kc),
                                     gh.bf16_tensor_to_f64(vc), sc.numpy(), k, causal=causal,
                                     zero_fill=zero_fill)
    idx = idx.cpu().numpy()
    got = gh.bf16_tensor_to_f64(out.cpu())
    kk = min(k, T)
    for b in range(B):
        for h in range(Hq):
            assert np.array_equal(idx[b, h], ref_idx[(b, h)]), f"selection (b={b}, h={h})"
            rows = b * T + ref_idx[(b, h)]
            # selected rows: the attention output, to the usual tolerances
            err = np.abs(got[h, rows] - ref[h, rows])
            rel = np.linalg.norm(got[h, rows] - ref[h, rows]) / np.linalg.norm(ref[h, rows])
            assert err.max() <= gh.MAX_ABS and rel <= gh.REL_L2, f"(b={b}, h={h}): {err.max():.3e} {rel:.3e}"
            others = np.setdiff1d(np.arange(b * T, (b + 1) * T), rows)
            want = 0.0 if zero_fill else 7.0
            assert np.all(got[h, others] == want), f"unselected rows (b={b}, h={h})"
    assert idx.shape == (B, Hq, kk)


@pytest.mark.parametrize("case", [
    # (B, Hq, Hkv, d, T, k, causal)
    (1, 4, 2, 128, 2000, 300, False),
    (1, 4, 2, 128, 2000, 300, True),
    (2, 8, 2, 64, 1000, 130, True),
    (2, 4, 4, 64, 1000, 130, False),
    (1, 2, 1, 128, 96, 96, True),        # every token kept
    (1, 2, 1, 128, 50, 80, False),       # budget above T: clamped
    (1, 2, 2, 128, 700, 1, True),        # one token
    (1, 8, 2, 128, 20000, 1024, True),   # the page's budget range, several tiles and query blocks
    (1, 4, 2, 64, 3000, 700, False),     # a small grid: key splits and their merge, d = 64
    (1, 4, 2, 64, 3000, 700, True),
])
def test_tsa_matches_oracle(case):
    B, Hq, Hkv, d, T, k, causal = case
    _check(_ld(), B, Hq, Hkv, d, T, k, causal, seed=B * 100000 + T * 7 + k + int(causal))


def test_tsa_keeps_unselected_rows_without_zero_fill():
    _check(_ld(), 1, 4, 2, 128, 1500, 200, True, seed=77, zero_fill=False)


def test_tsa_ties_go_to_lower_positions():
    """Constant scores: every head keeps the first k positions."""
    ld = _ld()
    dev = "cuda"
    q, kc, vc, _ = _inputs(1, 4, 2, 128, 1000, 5)
    sc = torch.zeros((1, 4, 1000))
    _, idx = ld.tsa_attention(q.to(dev), kc.to(dev), vc.to(dev), sc.to(dev), 100, causal=True)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy()[0], np.tile(np.arange(100), (4, 1)))


def test_tsa_given_sets_equal_selected_sets():
    """With the sets given (no selection launch) the output equals the call that
    selects the same sets."""
    ld = _ld()
    dev = "cuda"
    q, kc, vc, sc = _inputs(1, 4, 2, 128, 3000, 91)
    qd, kd, vd = q.to(dev), kc.to(dev), vc.to(dev)
    out1, idx = ld.tsa_attention(qd, kd, vd, sc.to(dev), 500, causal=True)
    out2, _ = ld.tsa_attention(qd, kd, vd, None, 500, idx_out=idx.clone(), causal=True, given_idx=True, batch=1)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))


def test_tsa_at_the_longest_sequence():
    """T = 2^21 tokens (the longest sequence the selection takes), two heads, small k."""
    _check(_ld(), 1, 2, 1, 64, 1 << 21, 100, True, seed=2024)


def test_tsa_at_the_bench_configuration():
    """The timed configuration: B = 1, 32 query and 8 KV heads, d = 128, T = 131072,
    k = 1024 per head, causal, residual scatter. Every head's selection equals the
    oracle's bit for bit; the dense stage of every head is checked against the oracle
    run on that head's selected rows alone (attention among the selected tokens is all
    the dense stage computes, and the ascending order keeps the causal order); a sample
    of unselected rows keeps what the caller wrote."""
    ld = _ld()
    dev = "cuda"
    B, Hq, Hkv, d, T, k = 1, 32, 8, 128, 131072, 1024
    g = torch.Generator(device=dev).manual_seed(wl.stream_seed("tsa-bench", T, k))
    q = torch.randn((Hq, B * T, d), generator=g, device=dev).to(torch.bfloat16)
    kc = torch.randn((Hkv, B * T, d), generator=g, device=dev).to(torch.bfloat16)
    vc = torch.randn((Hkv, B * T, d), generator=g, device=dev).to(torch.bfloat16)
    sc = torch.randn((B, Hq, T), generator=g, device=dev)
    out = torch.full_like(q, 7.0)
    out, idx = ld.tsa_attention(q, kc, vc, sc, k, out=out, causal=True, zero_fill=False)
    torch.cuda.synchronize()
    idx_h = idx.cpu().numpy()
    sc_h = sc.cpu().numpy()
    rng = np.random.default_rng(3)
    for h in range(Hq):
        want = orc.select_topk_f32(sc_h[0, h], k)
        assert np.array_equal(idx_h[0, h], want), f"selection of head {h}"
        sel = torch.as_tensor(want, device=dev)
        gk = h // (Hq // Hkv)
        qs = gh.bf16_tensor_to_f64(q[h, sel].cpu())[None]
        ks = gh.bf16_tensor_to_f64(kc[gk, sel].cpu())[None]
        vs = gh.bf16_tensor_to_f64(vc[gk, sel].cpu())[None]
        ref, _ = orc.tsa_attention(qs, ks, vs, np.zeros((1, 1, k)), k, causal=True)
        got = gh.bf16_tensor_to_f64(out[h, sel].cpu())
        err = np.abs(got - ref[0])
        rel = np.linalg.norm(got - ref[0]) / np.linalg.norm(ref[0])
        assert err.max() <= gh.MAX_ABS and rel <= gh.REL_L2, f"head {h}: {err.max():.3e} {rel:.3e}"
        others = np.setdiff1d(rng.integers(0, T, size=2048), want)
        assert torch.all(out[h, torch.as_tensor(others, device=dev)] == 7.0), f"unselected rows of head {h}"
