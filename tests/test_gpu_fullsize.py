"""Full-size parity: the whole decode step of each large workload, in the launch
configuration the benchmark times (automatic split size and waves, chained S
bitmaps), every layer checked against the fp64 oracle on sampled heads (and two
sampled sequences of a batch) with teacher forcing,
plus properties that hold for every S row at any size (ascending, distinct, in
range; sparse rows handed over unchanged, LycheeDecode summary page, method step 4).
"""
import numpy as np
import pytest

import workloads as wl
from oracle import lychee_oracle as orc
from tests import gpu_helpers as gh

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _head_sample(mask, Hq, rng, n=3):
    ret = [h for h in range(Hq) if mask >> h & 1]
    sp = [h for h in range(Hq) if not mask >> h & 1]
    pick = []
    if ret:
        pick += list(rng.choice(ret, size=min(n, len(ret)), replace=False))
    if sp:
        pick += list(rng.choice(sp, size=min(n, len(sp)), replace=False))
    return sorted(int(h) for h in pick)


def _check_rows(S_rows, lens, B, Hq):
    for b in range(B):
        for h in range(Hq):
            s = S_rows[(b, h)]
            assert s.size >= 1
            assert np.all(np.diff(s) > 0), f"S row {(b, h)} not strictly ascending"
            assert s[0] >= 0 and s[-1] < lens[b]


def _e4m3(x):
    """E4M3 codes (uint8) of the same draws, rounded to nearest even by torch."""
    return x.float().to(torch.float8_e4m3fn).view(torch.uint8)


def _paged(kc, vc, offs, page, seed):
    """K/V moved into pools of `page`-row pages in a seeded random order, with the
    block table that maps each sequence's pages."""
    B = len(offs) - 1
    npp = [(int(offs[b + 1] - offs[b]) + page - 1) // page for b in range(B)]
    perm = np.random.default_rng(seed).permutation(sum(npp))
    Hkv, _, d = kc.shape
    kp = torch.zeros((Hkv, sum(npp) * page, d), dtype=kc.dtype, device=kc.device)
    vp = torch.zeros_like(kp)
    bt = np.zeros((B, max(npp)), dtype=np.int32)
    j = 0
    for b in range(B):
        for i in range(npp[b]):
            pid = int(perm[j]); j += 1
            bt[b, i] = pid
            r0 = int(offs[b]) + i * page
            r1 = min(int(offs[b + 1]), r0 + page)
            kp[:, pid * page: pid * page + r1 - r0] = kc[:, r0:r1]
            vp[:, pid * page: pid * page + r1 - r0] = vc[:, r0:r1]
    return kp, vp, torch.as_tensor(bt, device=kc.device)


@pytest.mark.parametrize("name,layers,kv,page", [
    ("llama3_8b_32k", None, "bf16", 0),
    ("qwen3_8b_128k", None, "bf16", 0),   # all 36 layers
    ("ragged_b8", None, "bf16", 0),       # all 32 layers
    ("hysparse_7layer", None, "bf16", 0),
    ("llama3_8b_32k", 8, "e4m3", 0),      # 8-bit E4M3 KV codes with unit scales
    ("qwen3_8b_128k", 4, "e4m3", 64),     # E4M3 codes in 64-row pages of a shuffled pool
])
def test_fullsize_step(name, layers, kv, page):
    import hybrid_head_sparse_retrieval_amd as ld
    from hybrid_head_sparse_retrieval_amd.step import DecodeStep
    ld.load_library()
    w = wl.get_workload(name)
    if layers is not None and layers < w.layers:
        w = wl.get_workload(name, layers=layers, retrieval_masks=w.retrieval_masks[:layers])
    dev = "cuda"
    B, Hq, Hkv, d, L = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.layers
    G = Hq // Hkv
    inputs = []
    for l in range(L):
        x = wl.make_layer_inputs(w, l, device=dev)
        if x.k is not None and kv == "e4m3":
            x.k, x.v = _e4m3(x.k), _e4m3(x.v)
        inputs.append((x.q, x.k, x.v) if x.k is not None else (x.q, inputs[0][1], inputs[0][2]))
    step = DecodeStep(B, Hq, Hkv, d, w.seq_lens, w.k_per_seq, w.retrieval_masks,
                      csr=w.ragged_csr, device=dev)
    if kv == "e4m3":
        def kv_f64(t):
            return orc.fp8_e4m3_to_f64(t.cpu().numpy())
    else:
        def kv_f64(t):
            return orc.bf16_bits_to_f64(wl.bf16_bits(t))
    lens = list(w.seq_lens)
    offs = w.kv_offsets()
    scores = torch.full((B, Hq, w.max_seq), float("nan"), dtype=torch.float32, device=dev)
    rng = np.random.default_rng(w.index)
    sampled_layers = set(range(L))       # every layer, on sampled heads and sequences
    kb = [min(w.k_per_seq[b], lens[b]) for b in range(B)]
    checked = 0
    for l in range(L):
        q, kc, vc = inputs[l]
        S_before = step.s_rows() if l > 0 else None
        if page:
            kp, vp, bt = _paged(kc, vc, w.kv_offsets(), page, seed=l)
            step.layer(l, q, kp, vp, scores_out=scores, block_table=bt, page_size=page)
            del kp, vp
        else:
            step.layer(l, q, kc, vc, scores_out=scores)
        torch.cuda.synchronize()
        S_after = step.s_rows()
        _check_rows(S_after, lens, B, Hq)
        mask = w.retrieval_masks[l]
        for b in range(B):
            for h in range(Hq):
                if l > 0 and not (mask >> h & 1):
                    assert np.array_equal(S_after[(b, h)], S_before[(b, h)]), "sparse row changed"
        if l not in sampled_layers:
            continue
        heads = _head_sample(mask, Hq, rng)
        bs = range(B) if B <= 2 else sorted(int(x) for x in rng.choice(B, 2, replace=False))
        qb = wl.bf16_bits(q)
        Og = orc.bf16_bits_to_f64(wl.bf16_bits(step.outs[l]))
        sc = scores.cpu().numpy()
        kv_cache = {}
        for b in bs:
            for h in heads:
                g = h // G
                if (b, g) not in kv_cache:
                    lo, hi = int(offs[b]), int(offs[b + 1])
                    Kg = kv_f64(kc[g, lo:hi])
                    Vg = kv_f64(vc[g, lo:hi])
                    kv_cache[(b, g)] = (Kg, Vg)
                Kg, Vg = kv_cache[(b, g)]
                qh = orc.bf16_bits_to_f64(qb[b, h])
                scale = orc.default_scale(d)
                if mask >> h & 1:
                    O, S_ref, s_ref = orc.retrieval_head(qh, Kg, Vg, kb[b], scale)
                    gh.check_selected_row(S_after[(b, h)], sc[b, h, :lens[b]], s_ref, kb[b])
                else:
                    O, _ = orc.sparse_head(qh, Kg, Vg, S_before[(b, h)], scale)
                err = np.abs(Og[b, h] - O).max()
                rel = np.linalg.norm(Og[b, h] - O) / np.linalg.norm(O)
                assert err <= gh.MAX_ABS and rel <= gh.REL_L2, (name, l, b, h, err, rel)
                checked += 1
    assert checked >= 3 * len(sampled_layers), checked


def test_hysparse_block_with_block_selection_and_window():
    """The HySparse group as timed with block selection and a 128-token window branch
    (N = 131072, k = 4096, 1 full + 6 sparse layers on the full layer's cache): every
    head's S equals the oracle's block selection on the layer's own fp32 logits, sampled
    full-layer heads match the oracle's attention, every head of the first and the last
    sparse layer matches the oracle's gated layer, and S passes through the sparse
    layers unchanged."""
    import hybrid_head_sparse_retrieval_amd as ld
    from hybrid_head_sparse_retrieval_amd.step import DecodeStep
    ld.load_library()
    w = wl.get_workload("hysparse_7layer")
    dev = "cuda"
    B, Hq, Hkv, d, L, N, W = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.layers, w.max_seq, 128
    G = Hq // Hkv
    k = w.k_per_seq[0]
    x0 = wl.make_layer_inputs(w, 0, device=dev)
    kc, vc = x0.k, x0.v
    qs = [x0.q] + [wl.make_layer_inputs(w, l, device=dev).q for l in range(1, L)]
    windows = [None]
    gen = torch.Generator(device="cpu")
    for l in range(1, L):
        gen.manual_seed(wl.stream_seed("window", w.name, l))
        kw = torch.randn((Hkv, B * W, d), generator=gen).to(torch.bfloat16).to(dev)
        vw = torch.randn((Hkv, B * W, d), generator=gen).to(torch.bfloat16).to(dev)
        gate = torch.randn((B, Hq), generator=gen).to(dev)
        windows.append((kw, vw, gate))
    step = DecodeStep(B, Hq, Hkv, d, w.seq_lens, w.k_per_seq, w.retrieval_masks, device=dev,
                      split_flag=ld.FLAG_BLOCK_SELECT, window_len=W)
    scores = torch.full((B, Hq, N), float("nan"), dtype=torch.float32, device=dev)
    step.layer(0, qs[0], kc, vc, scores_out=scores)
    torch.cuda.synchronize()
    S0 = step.s_rows()
    sc = scores.cpu().numpy()
    for h in range(Hq):
        assert np.array_equal(S0[(0, h)], orc.select_topk_blocks(sc[0, h], k)), f"block selection of head {h}"
    K = orc.bf16_bits_to_f64(wl.bf16_bits(kc))
    V = orc.bf16_bits_to_f64(wl.bf16_bits(vc))
    scale = orc.default_scale(d)
    O0 = orc.bf16_bits_to_f64(wl.bf16_bits(step.outs[0]))
    q0 = orc.bf16_bits_to_f64(wl.bf16_bits(qs[0]))
    for h in (0, 13, 31):
        O, _, _ = orc.retrieval_head(q0[0, h], K[h // G], V[h // G], k, scale)
        err = np.abs(O0[0, h] - O).max()
        rel = np.linalg.norm(O0[0, h] - O) / np.linalg.norm(O)
        assert err <= gh.MAX_ABS and rel <= gh.REL_L2, ("full layer", h, err, rel)
    for l in range(1, L):
        step.layer(l, qs[l], kc, vc, window=windows[l])
        torch.cuda.synchronize()
        S = step.s_rows()
        for h in range(Hq):
            assert np.array_equal(S[(0, h)], S0[(0, h)]), f"layer {l} changed the S row of head {h}"
        if l not in (1, L - 1):
            continue
        kw, vw, gate = windows[l]
        ref = orc.hysparse_sparse_layer(orc.bf16_bits_to_f64(wl.bf16_bits(qs[l])), K, V, [0, N], S0,
                                        orc.bf16_bits_to_f64(wl.bf16_bits(kw)),
                                        orc.bf16_bits_to_f64(wl.bf16_bits(vw)), gate.cpu().numpy(), scale)
        got = orc.bf16_bits_to_f64(wl.bf16_bits(step.outs[l]))
        for h in range(Hq):
            err = np.abs(got[0, h] - ref[0, h]).max()
            rel = np.linalg.norm(got[0, h] - ref[0, h]) / np.linalg.norm(ref[0, h])
            assert err <= gh.MAX_ABS and rel <= gh.REL_L2, ("sparse layer", l, h, err, rel)
