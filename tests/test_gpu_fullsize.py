"""Full-size parity: the decode step of each large workload, in the launch
configuration the benchmark times (automatic split size and waves, chained S
bitmaps), checked against the fp64 oracle on sampled heads with teacher forcing,
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


@pytest.mark.parametrize("name,layers", [
    ("llama3_8b_32k", None),
    ("qwen3_8b_128k", 8),
    ("ragged_b8", 6),
    ("hysparse_7layer", None),
])
def test_fullsize_step(name, layers):
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
        inputs.append((x.q, x.k, x.v) if x.k is not None else (x.q, inputs[0][1], inputs[0][2]))
    step = DecodeStep(B, Hq, Hkv, d, w.seq_lens, w.k_per_seq, w.retrieval_masks,
                      csr=w.ragged_csr, device=dev)
    lens = list(w.seq_lens)
    offs = w.kv_offsets()
    scores = torch.full((B, Hq, w.max_seq), float("nan"), dtype=torch.float32, device=dev)
    rng = np.random.default_rng(w.index)
    sampled_layers = sorted({0, 1, L // 2, L - 1} | {l for l in range(1, L) if w.retrieval_masks[l]} if L <= 8
                            else {0, 1, L // 2, L - 1} | set(int(l) for l in rng.choice(range(1, L), 2, replace=False)))
    kb = [min(w.k_per_seq[b], lens[b]) for b in range(B)]
    checked = 0
    for l in range(L):
        q, kc, vc = inputs[l]
        S_before = step.s_rows() if l > 0 else None
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
                    Kg = orc.bf16_bits_to_f64(wl.bf16_bits(kc[g, lo:hi]))
                    Vg = orc.bf16_bits_to_f64(wl.bf16_bits(vc[g, lo:hi]))
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
