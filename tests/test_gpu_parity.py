"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle on the
same bf16 inputs, layer by layer with teacher forcing (the oracle consumes the S the
GPU handed to the layer), over shapes that span several splits, ragged tails, MHA and
grouped KV heads, mixed and sparse-only groups."""
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


def run_layers(B, Hq, Hkv, d, lens, masks, seed, k=None, csr=False, chain=True, split=0,
               check=True, frac=0.3, extra_flags=0):
    """Run len(masks) layers on the GPU and check every layer against the oracle."""
    ld = _ld()
    dev = "cuda"
    L = len(masks)
    lens = list(lens)
    N = max(lens)
    ragged = len(set(lens)) > 1 or csr
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(offs[-1])
    kb = [min(k, n) if k is not None else max(1, int(frac * n)) for n in lens]
    kv_indptr = torch.as_tensor(offs, device=dev) if ragged else None
    if csr:
        rows = [kb[b] for b in range(B) for _ in range(Hq)]
        s_indptr_h = np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)
        s_indptr = torch.as_tensor(s_indptr_h, device=dev)
        S = torch.zeros(int(s_indptr_h[-1]), dtype=torch.int32, device=dev)
        kmax = max(kb)
    else:
        assert len(set(kb)) == 1
        s_indptr_h, s_indptr = None, None
        S = torch.zeros((B, Hq, kb[0]), dtype=torch.int32, device=dev)
        kmax = kb[0]
    layers = [wl.random_qkv(B, Hq, Hkv, d, T, seed * 100 + l) for l in range(L)]
    shape = ld.make_shape(layers[0][0].to(dev), layers[0][1].to(dev), kv_indptr, N)
    ws = ld.Workspace(shape, kmax, dev)
    scores = torch.full((B, Hq, N), float("nan"), dtype=torch.float32, device=dev)
    results = []
    for l in range(L):
        qc, kc, vc = layers[l]
        q, kk, vv = qc.to(dev), kc.to(dev), vc.to(dev)
        S_before = S.cpu().numpy().copy()
        out = torch.empty_like(q)
        flags = (ld.FLAG_S_CHAINED if (chain and l > 0) else 0) | ld.flag_split_rows(split) | extra_flags
        ld.hybrid_layer(q, kk, vv, masks[l], kmax, S if l > 0 else None, s_out=S, s_indptr=s_indptr,
                        scores_out=scores, out=out, flags=flags, workspace=ws,
                        kv_indptr=kv_indptr, seq_len=N)
        torch.cuda.synchronize()
        S_after = S.cpu().numpy()
        sc = scores.cpu().numpy()
        results.append((out.clone(), S_after.copy()))
        if not check:
            continue
        ret = [bool(masks[l] >> h & 1) for h in range(Hq)]
        S_in = None if l == 0 else gh.s_rows_to_dict(S_before, B, Hq, s_indptr_h)
        O_ref, S_ref, sc_ref = orc.hybrid_layer_bf16(
            wl.bf16_bits(qc), wl.bf16_bits(kc), wl.bf16_bits(vc), offs, ret, kb, S_in)
        gh.check_outputs(out, O_ref, [(b, h) for b in range(B) for h in range(Hq)], f"layer {l}")
        S_dict = gh.s_rows_to_dict(S_after, B, Hq, s_indptr_h)
        for b in range(B):
            for h in range(Hq):
                if ret[h]:
                    gh.check_selected_row(S_dict[(b, h)], sc[b, h, :lens[b]], sc_ref[(b, h)], kb[b],
                                          what=f"layer {l} (b, h) = {(b, h)}: ")
                else:
                    assert np.array_equal(S_dict[(b, h)], S_in[(b, h)]), "sparse row changed"
    ws.check()    # no bounded wait between workgroups gave up
    return results


@pytest.mark.parametrize("case", [
    # B, Hq, Hkv, d, lens, masks (layer 0 all retrieval), seed
    (1, 8, 2, 128, [5000], [0xFF, 0b00100001, 0, 0b1000], 1),      # GQA 4:1, mixed + sparse-only groups
    (2, 4, 4, 64, [3000, 3000], [0xF, 0b0010, 0], 2),               # MHA d=64
    (1, 16, 2, 128, [1100], [0xFFFF, 0x0101, 0], 3),                 # GQA 8:1
    (1, 8, 4, 64, [2049], [0xFF, 0b01000010, 0], 4),                 # GQA 2:1, tail of 1 row
    (1, 32, 8, 128, [4096], wl.seeded_masks(5, 3, 32, 2), 5),        # Llama head shape
    (1, 64, 8, 128, [3000], [(1 << 64) - 1, (1 << 63) | 1, 0], 6),   # 64 query heads: every mask bit
    (1, 4, 4, 128, [3000], [0xF, 0b0100, 0], 8),                     # MHA d=128: 32 merge lanes per column
])
def test_layers_match_oracle(case):
    B, Hq, Hkv, d, lens, masks, seed = case
    run_layers(B, Hq, Hkv, d, lens, masks, seed)


def test_ragged_csr_batch():
    run_layers(3, 8, 2, 128, [777, 2100, 1500], [0xFF, 0b10000100, 0], 6, csr=True)


def test_unchained_equals_chained():
    a = run_layers(1, 8, 2, 128, [3000], [0xFF, 0b00010000, 0], 7, chain=True, check=False)
    b = run_layers(1, 8, 2, 128, [3000], [0xFF, 0b00010000, 0], 7, chain=False, check=True)
    for (oa, sa), (ob, sb) in zip(a, b):
        assert torch.equal(oa, ob) and np.array_equal(sa, sb)


@pytest.mark.parametrize("n", [1, 2, 5, 31, 257, 513])
def test_small_and_tail_lengths(n):
    k = max(1, (3 * n) // 10)
    run_layers(1, 4, 2, 128, [n], [0xF, 0b0001, 0], 10 + n, k=k)


@pytest.mark.parametrize("split", [1, 2, 3, 4, 5])
def test_split_size_invariance(split):
    run_layers(1, 8, 2, 128, [6000], [0xFF, 0b00000010, 0], 11, split=split)


def test_deterministic_and_batch_permutation():
    ld = _ld()
    dev = "cuda"
    Hq, Hkv, d = 8, 2, 128
    lens = [900, 2500, 1700]
    k = 250
    perm = [2, 0, 1]
    q, kc, vc = wl.random_qkv(3, Hq, Hkv, d, sum(lens), 12)
    offs = np.concatenate([[0], np.cumsum(lens)])

    def run(q, kc, vc, lens):
        offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
        kvi = torch.as_tensor(offs, device=dev)
        qd, kd, vd = q.to(dev), kc.to(dev), vc.to(dev)
        shape = ld.make_shape(qd, kd, kvi, max(lens))
        ws = ld.Workspace(shape, k, dev)
        S = torch.zeros((3, Hq, k), dtype=torch.int32, device=dev)
        out0 = ld.hybrid_layer(qd, kd, vd, 0xFF, k, None, s_out=S, workspace=ws, kv_indptr=kvi, seq_len=max(lens))
        out1 = ld.hybrid_layer(qd, kd, vd, 0b00100000, k, S, workspace=ws, kv_indptr=kvi, seq_len=max(lens),
                               flags=ld.FLAG_S_CHAINED)
        torch.cuda.synchronize()
        return out0.cpu(), out1.cpu(), S.cpu()

    r1 = run(q, kc, vc, lens)
    r2 = run(q, kc, vc, lens)
    for a, b in zip(r1, r2):
        assert torch.equal(a, b), "run-to-run results differ"
    kp = torch.cat([kc[:, offs[p]:offs[p + 1]] for p in perm], dim=1)
    vp = torch.cat([vc[:, offs[p]:offs[p + 1]] for p in perm], dim=1)
    rp = run(q[perm], kp, vp, [lens[p] for p in perm])
    for a, b in zip(r1, rp):
        assert torch.equal(a[perm], b), "batch permutation changed results"


def test_sparse_full_set_equals_retrieval_and_single_index():
    ld = _ld()
    dev = "cuda"
    Hq, Hkv, d, n = 8, 2, 128, 3333
    q, kc, vc = [t.to(dev) for t in wl.random_qkv(1, Hq, Hkv, d, n, 13)]
    shape = ld.make_shape(q, kc)
    ws = ld.Workspace(shape, n, dev)
    full = ld.retrieval_decode(q, kc, vc, 0xFF, n, workspace=ws)
    S = torch.arange(n, dtype=torch.int32, device=dev).repeat(1, Hq, 1).contiguous()
    sp = ld.sparse_decode(q, kc, vc, 0xFF, n, S, workspace=ws)
    torch.cuda.synchronize()
    O_ref, _, _ = orc.hybrid_layer_bf16(wl.bf16_bits(q), wl.bf16_bits(kc), wl.bf16_bits(vc),
                                        [0, n], [True] * Hq, [n], None)
    gh.check_outputs(full, O_ref, [(0, h) for h in range(Hq)])
    gh.check_outputs(sp, O_ref, [(0, h) for h in range(Hq)])
    # a single index: weight exactly 1, output is that value row bit for bit
    pos = torch.tensor([0, 17, 3332, 1666, 5, 900, 2048, 1], dtype=torch.int32, device=dev)
    S1 = pos.view(1, Hq, 1).contiguous()
    ws1 = ld.Workspace(shape, 1, dev)
    o1 = ld.sparse_decode(q, kc, vc, 0xFF, 1, S1, workspace=ws1)
    torch.cuda.synchronize()
    for h in range(Hq):
        assert torch.equal(o1[0, h].cpu(), vc[h // 4, int(pos[h])].cpu())


def test_retrieval_decode_subset_of_heads_leaves_others():
    ld = _ld()
    dev = "cuda"
    Hq, Hkv, d, n, k = 8, 2, 64, 2000, 600
    q, kc, vc = [t.to(dev) for t in wl.random_qkv(1, Hq, Hkv, d, n, 14)]
    shape = ld.make_shape(q, kc)
    ws = ld.Workspace(shape, k, dev)
    out = torch.full_like(q, 7.0)
    S = torch.full((1, Hq, k), -5, dtype=torch.int32, device=dev)
    mask = 0b01100100
    ld.retrieval_decode(q, kc, vc, mask, k, s_out=S, out=out, workspace=ws)
    torch.cuda.synchronize()
    O_ref, S_ref, _ = orc.hybrid_layer_bf16(wl.bf16_bits(q), wl.bf16_bits(kc), wl.bf16_bits(vc),
                                            [0, n], [True] * Hq, [k], None)
    for h in range(Hq):
        if mask >> h & 1:
            gh.check_outputs(out, O_ref, [(0, h)])
            assert np.all(np.diff(S[0, h].cpu().numpy()) > 0)
        else:
            assert torch.all(out[0, h] == 7.0) and torch.all(S[0, h] == -5)


@pytest.mark.parametrize("case", [
    (1, 8, 2, 128, [5000], [0xFF, 0b00100001, 0, 0b1000], 21, False),
    (2, 32, 8, 128, [3000, 4100], wl.seeded_masks(22, 3, 32, 2), 22, True),
])
def test_separate_merge_and_select_steps(case):
    # the same layers with the split merge and argsTopK run as their own launches
    ld = _ld()
    B, Hq, Hkv, d, lens, masks, seed, csr = case
    run_layers(B, Hq, Hkv, d, lens, masks, seed, csr=csr, extra_flags=ld.FLAG_SEPARATE_SELECT)


def test_in_launch_and_separate_select_agree():
    ld = _ld()
    args = (2, 8, 2, 128, [2600, 6100], [0xFF, 0b01000010, 0, 0b00010000], 23)
    a = run_layers(*args, csr=True, check=False)
    b = run_layers(*args, csr=True, check=False, extra_flags=ld.FLAG_SEPARATE_SELECT)
    for (oa, sa), (ob, sb) in zip(a, b):
        assert np.array_equal(sa, sb), "selected sets differ between the two launch modes"
        da = gh.bf16_tensor_to_f64(oa)
        db = gh.bf16_tensor_to_f64(ob)
        assert np.abs(da - db).max() <= gh.MAX_ABS


@pytest.mark.parametrize("entry,mask", [("layer", 0xFF), ("layer-separate", 0xFF),
                                        ("retrieval", 0x11), ("retrieval", 0x22)])
def test_ties_at_the_threshold_span_splits(entry, mask):
    # every third key row of a KV head is the same vector, aligned with the group's
    # queries: 2000 equal top scores per head, of which the k = 1800 lowest rows win
    ld = _ld()
    dev = "cuda"
    Hq, Hkv, d, n, k = 8, 2, 128, 6000, 1800
    q, kc, vc = wl.random_qkv(1, Hq, Hkv, d, n, 24)
    G = Hq // Hkv
    for g in range(Hkv):
        u = q[0, g * G:(g + 1) * G].float().mean(0)
        u = 10.0 * u / u.norm()
        kc[g, 0::3] = u.to(kc.dtype)
    qd, kd, vd = q.to(dev), kc.to(dev), vc.to(dev)
    shape = ld.make_shape(qd, kd)
    ws = ld.Workspace(shape, k, dev)
    S = torch.zeros((1, Hq, k), dtype=torch.int32, device=dev)
    scores = torch.empty((1, Hq, n), dtype=torch.float32, device=dev)
    # one retrieval head per KV group (0x11, 0x22) selects inside the attention launch
    out = torch.zeros_like(qd)
    if entry == "retrieval":
        ld.retrieval_decode(qd, kd, vd, mask, k, s_out=S, scores_out=scores, out=out, workspace=ws)
    else:
        flags = ld.FLAG_SEPARATE_SELECT if entry == "layer-separate" else 0
        ld.hybrid_layer(qd, kd, vd, mask, k, None, s_out=S, scores_out=scores, out=out, flags=flags,
                        workspace=ws)
    torch.cuda.synchronize()
    sc = scores.cpu().numpy()
    Sh = S.cpu().numpy()
    heads = [h for h in range(Hq) if mask >> h & 1]
    for h in heads:
        exact = orc.select_topk_f32(sc[0, h], k)
        assert np.array_equal(Sh[0, h], exact)
        assert np.array_equal(Sh[0, h], np.arange(0, 3 * k, 3)), "ties must go to the lowest rows"
    O_ref, _, _ = orc.hybrid_layer_bf16(wl.bf16_bits(q), wl.bf16_bits(kc), wl.bf16_bits(vc),
                                        [0, n], [True] * Hq, [k], None)
    gh.check_outputs(out, O_ref, [(0, h) for h in heads])


@pytest.mark.parametrize("stride", [1, 2])
def test_more_candidates_than_lds_holds(stride):
    # every stride-th key row of a KV head is the same vector: 20000 / stride equal top
    # scores per retrieval head share one digit-1 bin, more candidates than the
    # in-launch selection stages in LDS (8192), so it reads them from the sub-lists
    ld = _ld()
    dev = "cuda"
    Hq, Hkv, d, n, k = 8, 2, 128, 20000, 6000
    q, kc, vc = wl.random_qkv(1, Hq, Hkv, d, n, 25)
    G = Hq // Hkv
    for g in range(Hkv):
        u = q[0, g * G:(g + 1) * G].float().mean(0)
        u = 10.0 * u / u.norm()
        kc[g, 0::stride] = u.to(kc.dtype)
    qd, kd, vd = q.to(dev), kc.to(dev), vc.to(dev)
    ws = ld.Workspace(ld.make_shape(qd, kd), k, dev)
    S = torch.zeros((1, Hq, k), dtype=torch.int32, device=dev)
    scores = torch.empty((1, Hq, n), dtype=torch.float32, device=dev)
    out = torch.zeros_like(qd)
    ld.retrieval_decode(qd, kd, vd, 0x11, k, s_out=S, scores_out=scores, out=out, workspace=ws)
    torch.cuda.synchronize()
    sc = scores.cpu().numpy()
    Sh = S.cpu().numpy()
    for h in (0, 4):
        assert np.array_equal(Sh[0, h], orc.select_topk_f32(sc[0, h], k))
        assert np.array_equal(Sh[0, h], np.arange(0, stride * k, stride)), "ties must go to the lowest rows"
    O_ref, _, _ = orc.hybrid_layer_bf16(wl.bf16_bits(q), wl.bf16_bits(kc), wl.bf16_bits(vc),
                                        [0, n], [True] * Hq, [k], None)
    gh.check_outputs(out, O_ref, [(0, 0), (0, 4)])


def test_wait_flag_is_reported_and_cleared():
    # the flag that a kernel sets when a bounded wait gives up: set it from the host,
    # then the check reports it once and clears it
    ld = _ld()
    q, kc, vc = wl.random_qkv(1, 4, 4, 64, 1024, 26)
    shape = ld.make_shape(q.cuda(), kc.cuda())
    for ws in (ld.Workspace(shape, 307, "cuda"), ld.TopkWorkspace(2, 1024, "cuda")):
        ws.check()
        ws.buf[0:4] = torch.tensor([1, 0, 0, 0], dtype=torch.uint8, device="cuda")
        with pytest.raises(ld.LycheeDecodeError, match="bounded wait"):
            ws.check()
        ws.check()


def test_undersized_buffers_are_rejected_before_launch():
    import hybrid_head_sparse_retrieval_amd as ld
    ld.load_library()
    dev = "cuda"
    B, Hq, Hkv, d, n, k = 1, 8, 2, 128, 512, 100
    q = torch.zeros((B, Hq, d), dtype=torch.bfloat16, device=dev)
    kc = torch.zeros((Hkv, B * n, d), dtype=torch.bfloat16, device=dev)
    S = torch.zeros((B, Hq, k), dtype=torch.int32, device=dev)
    small = torch.zeros((B, Hq, k - 1), dtype=torch.int32, device=dev)
    with pytest.raises(ValueError, match="s_out"):
        ld.hybrid_layer(q, kc, kc, 0xFF, k, None, s_out=small)
    with pytest.raises(ValueError, match="s_in"):
        ld.sparse_decode(q, kc, kc, 0xFF, k, small)
    with pytest.raises(ValueError, match="scores_out"):
        ld.retrieval_decode(q, kc, kc, 0xFF, k, s_out=S,
                            scores_out=torch.zeros((B, Hq, n - 1), dtype=torch.float32, device=dev))
    with pytest.raises(ValueError, match="out must"):
        ld.hybrid_layer(q, kc, kc, 0xFF, k, None, s_out=S, out=torch.zeros((B, Hq - 1, d), dtype=torch.bfloat16,
                                                                           device=dev))
    with pytest.raises(ValueError, match="kv_indptr"):
        ld.hybrid_layer(q, kc, kc, 0xFF, k, None, s_out=S, seq_len=n,
                        kv_indptr=torch.zeros(3, dtype=torch.int64, device=dev))


def test_csr_rows_are_clipped_to_the_s_buffer():
    """CSR offsets that run past the S buffer: every kernel clips each row to the buffer
    (ld_shape.s_capacity), so nothing past it is read or written; rows inside it are
    the oracle's selection, a clipped row keeps as many of its row's best indices as fit."""
    ld = _ld()
    dev = "cuda"
    B, Hq, Hkv, d = 2, 4, 4, 64
    lens = [700, 900]
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    rows = [200] * (B * Hq)
    ind_h = np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)
    cap = int(ind_h[-1]) - 350                      # the last two rows run past the buffer
    guard = torch.full((int(ind_h[-1]) + 64,), -5, dtype=torch.int32, device=dev)
    S = guard[:cap]
    s_indptr = torch.as_tensor(ind_h, device=dev)
    kv_indptr = torch.as_tensor(offs, device=dev)
    masks = [0xF, 0b0100]
    for l, mask in enumerate(masks):
        qc, kc, vc = wl.random_qkv(B, Hq, Hkv, d, int(offs[-1]), 900 + l)
        out = torch.empty_like(qc, device=dev)
        scores = torch.full((B, Hq, max(lens)), float("nan"), dtype=torch.float32, device=dev)
        S_before = S.cpu().numpy().copy()
        ld.hybrid_layer(qc.to(dev), kc.to(dev), vc.to(dev), mask, 200, S if l else None, s_out=S,
                        s_indptr=s_indptr, scores_out=scores, out=out, kv_indptr=kv_indptr, seq_len=max(lens),
                        flags=ld.FLAG_S_CHAINED if l else 0)
        torch.cuda.synchronize()
        g = guard.cpu().numpy()
        assert np.all(g[cap:] == -5), f"layer {l}: entries past the S buffer were written"
        sc = scores.cpu().numpy()
        for b in range(B):
            for h in range(Hq):
                r = b * Hq + h
                a, e = min(ind_h[r], cap), min(ind_h[r + 1], cap)
                if not (mask >> h & 1):
                    assert np.array_equal(g[a:e], S_before[a:e])
                    continue
                if e > a:
                    want = orc.select_topk_f32(sc[b, h, :lens[b]], int(e - a))
                    assert np.array_equal(g[a:e], want), (l, b, h)


@pytest.mark.parametrize("flags", [0, 4])   # selection in the attention launch, or in launches of its own
def test_empty_csr_row_leaves_no_counts_behind(flags):
    """A retrieval row whose CSR S row is empty keeps nothing, yet the attention launch
    counts its scores into the first-digit histogram; those counts must be gone before
    the next call on the same workspace selects that row (LycheeDecode summary page,
    method step 3: each call's argsTopK sees only its own scores)."""
    ld = _ld()
    dev = "cuda"
    B, Hq, Hkv, d, N, k = 1, 4, 4, 64, 3000, 300
    shape = None
    ws = None
    for call, rows in enumerate([[k, 0, k, k], [k, k, k, k]]):
        ind_h = np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)
        s_indptr = torch.as_tensor(ind_h, device=dev)
        S = torch.full((int(ind_h[-1]),), -1, dtype=torch.int32, device=dev)
        qc, kc, vc = wl.random_qkv(B, Hq, Hkv, d, N, 1300 + call)
        q, kk, vv = qc.to(dev), kc.to(dev), vc.to(dev)
        if ws is None:
            shape = ld.make_shape(q, kk, None, N)
            ws = ld.Workspace(shape, k, dev)
        scores = torch.full((B, Hq, N), float("nan"), dtype=torch.float32, device=dev)
        out = torch.empty_like(q)
        ld.hybrid_layer(q, kk, vv, 0xF, k, None, s_out=S, s_indptr=s_indptr, scores_out=scores, out=out,
                        flags=flags, workspace=ws, seq_len=N)
        torch.cuda.synchronize()
        g = S.cpu().numpy()
        sc = scores.cpu().numpy()
        for h in range(Hq):
            a, e = int(ind_h[h]), int(ind_h[h + 1])
            if e > a:
                assert np.array_equal(g[a:e], orc.select_topk_f32(sc[0, h], e - a)), (call, h)
    ws.check()


def _plan_for(ld, Hq, Hkv, d, N, mask, s_in=True, flags=0):
    dev = "cuda"
    q = torch.empty((1, Hq, d), dtype=torch.bfloat16, device=dev)
    kv = torch.empty((Hkv, N, d), dtype=torch.bfloat16, device=dev)
    S = torch.empty((1, Hq, max(1, int(0.3 * N))), dtype=torch.int32, device=dev)
    return ld.hybrid_layer_plan(q, kv, kv, mask, S.shape[2], S if s_in else None, s_out=S,
                                flags=flags, seq_len=N)


def test_layer_plan_describes_the_launches():
    ld = _ld()
    full = (1 << 32) - 1
    # a sparse-only or one-retrieval-head layer on chained S: one attention launch that
    # also merges O and, with a retrieval head, selects its S
    p = _plan_for(ld, 32, 8, 128, 32768, 0, flags=ld.FLAG_S_CHAINED)
    assert p["launches"] == 1 and p["select_in_launch"] == 0 and p["split_rows_stream"] == 0
    p = _plan_for(ld, 32, 8, 128, 32768, 1 << 5, flags=ld.FLAG_S_CHAINED)
    assert p["launches"] == 1 and p["select_in_launch"] == 1 and p["selector_parts"] >= 2
    # unchained S adds the bitmap build
    assert _plan_for(ld, 32, 8, 128, 32768, 1 << 5)["launches"] == 2
    # the forced separate mode and a 32-head full layer at 32K select in launches of their own
    # (the attention launch fuses the first radix digit, so the selection adds one or two)
    p = _plan_for(ld, 32, 8, 128, 32768, 1 << 5, flags=ld.FLAG_S_CHAINED | ld.FLAG_SEPARATE_SELECT)
    assert p["launches"] >= 2 and p["select_in_launch"] == 0
    p = _plan_for(ld, 32, 8, 128, 32768, full, s_in=False)
    assert p["launches"] >= 2 and p["select_in_launch"] == 0
    assert p["attention_workgroups"] >= 8


def test_both_sides_of_the_in_launch_selection_rule():
    """A 32-head all-retrieval layer selects inside the launch up to some length and in
    launches of its own past it; the lengths on both sides of that boundary (found with
    the plan query) match the oracle."""
    ld = _ld()
    full = (1 << 32) - 1
    inl = lambda n: _plan_for(ld, 32, 8, 128, n, full, s_in=False)["select_in_launch"] == 1
    lo, hi = 1024, 65536
    assert inl(lo) and not inl(hi)
    while hi - lo > 1:
        mid = (lo + hi) // 2
        lo, hi = (mid, hi) if inl(mid) else (lo, mid)
    for n in (lo, hi):
        run_layers(1, 32, 8, 128, [n], [full, 1 << 7], 40 + n % 7)


@pytest.mark.parametrize("waves", [1, 2])
def test_both_wave_counts_match_oracle(waves):
    """The launch runs 4 waves per workgroup unless the caller asks for 8
    (LD_FLAG_WAVES(2)); both instances of the Llama head shape match the oracle."""
    ld = _ld()
    run_layers(1, 32, 8, 128, [4100], wl.seeded_masks(31, 3, 32, 2), 31, extra_flags=ld.flag_waves(waves))
