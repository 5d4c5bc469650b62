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


def test_block_hint_on_token_sets_gives_the_same_layer():
    """LD_FLAG_BLOCK_SELECT on a layer without retrieval heads only changes how the
    gather work is split among waves: token sets (not whole blocks) give the oracle's
    layer all the same, including ragged split tails."""
    ld = _ld()
    dev = "cuda"
    B, Hq, Hkv, d, n, k = 1, 8, 2, 128, 5000, 1500
    S = torch.zeros((B, Hq, k), dtype=torch.int32, device=dev)
    q0, k0, v0 = wl.random_qkv(B, Hq, Hkv, d, n, 970)
    ws = ld.Workspace(ld.make_shape(q0.to(dev), k0.to(dev)), k, dev)
    ld.hybrid_layer(q0.to(dev), k0.to(dev), v0.to(dev), 0xFF, k, None, s_out=S, workspace=ws)
    q1, k1, v1 = wl.random_qkv(B, Hq, Hkv, d, n, 971)
    out = ld.hybrid_layer(q1.to(dev), k1.to(dev), v1.to(dev), 0x00, k, S, s_out=S, workspace=ws,
                          flags=ld.FLAG_BLOCK_SELECT | ld.FLAG_S_CHAINED)
    torch.cuda.synchronize()
    Sh = S.cpu().numpy()
    S_in = {(0, h): Sh[0, h].astype(np.int64) for h in range(Hq)}
    O_ref, _, _ = orc.hybrid_layer_bf16(wl.bf16_bits(q1), wl.bf16_bits(k1), wl.bf16_bits(v1), [0, n],
                                        [False] * Hq, [k], S_in)
    gh.check_outputs(out, O_ref, [(0, h) for h in range(Hq)], "token sets with the block hint")
    ws.check()


def test_block_hint_on_a_ragged_batch():
    """The block hint over a ragged batch: each sequence's splits share out that
    sequence's union of 64-row blocks (lengths that end inside a block, sequences that
    start past row 0), with token sets and with whole-block sets."""
    ld = _ld()
    dev = "cuda"
    B, Hq, Hkv, d = 3, 8, 2, 128
    lens = [4100, 777, 6400]
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T, N = int(offs[-1]), max(lens)
    kv_indptr = torch.as_tensor(offs, device=dev)
    rng = np.random.default_rng(980)
    for blocks in (False, True):
        rows = {}
        for b in range(B):
            for h in range(Hq):
                n = lens[b]
                if blocks:
                    nblk = (n + 63) // 64
                    kb = rng.choice(nblk, size=max(1, nblk // 5), replace=False)
                    s = np.concatenate([np.arange(64 * j, min(64 * j + 64, n)) for j in sorted(kb)])
                else:
                    s = np.sort(rng.choice(n, size=max(1, n // 4), replace=False))
                rows[(b, h)] = s.astype(np.int64)
        ind_h = np.concatenate([[0], np.cumsum([rows[(b, h)].size for b in range(B) for h in range(Hq)])])
        s_indptr = torch.as_tensor(ind_h.astype(np.int64), device=dev)
        S = torch.as_tensor(np.concatenate([rows[(b, h)] for b in range(B) for h in range(Hq)]).astype(np.int32),
                            device=dev)
        q, kc, vc = wl.random_qkv(B, Hq, Hkv, d, T, 981 + int(blocks))
        qd, kd, vd = q.to(dev), kc.to(dev), vc.to(dev)
        out = ld.hybrid_layer(qd, kd, vd, 0x00, int(max(r.size for r in rows.values())), S, s_out=S,
                              s_indptr=s_indptr, kv_indptr=kv_indptr, seq_len=N, flags=ld.FLAG_BLOCK_SELECT)
        torch.cuda.synchronize()
        O_ref, _, _ = orc.hybrid_layer_bf16(wl.bf16_bits(q), wl.bf16_bits(kc), wl.bf16_bits(vc), offs,
                                            [False] * Hq, [int(max(r.size for r in rows.values()))] * B, rows)
        gh.check_outputs(out, O_ref, [(b, h) for b in range(B) for h in range(Hq)],
                         f"ragged batch, {'block' if blocks else 'token'} sets with the block hint")


@pytest.mark.parametrize("Hq,Hkv,d,n", [
    (4, 4, 64, 3000),       # one query head per KV head
    (16, 2, 128, 9000),     # eight query heads per KV head
    (4, 2, 64, 140000),     # past the rows that block shares cover: the splits keep row ranges
])
def test_block_hint_shapes(Hq, Hkv, d, n):
    """Whole-block sets with the block hint on a layer of sparse heads, for other group
    sizes and for a sequence longer than the block shares handle."""
    ld = _ld()
    dev = "cuda"
    rng = np.random.default_rng(990 + n)
    nblk = (n + 63) // 64
    rows = {}
    for h in range(Hq):
        kb = np.sort(rng.choice(nblk, size=max(1, nblk // 10), replace=False))
        rows[(0, h)] = np.concatenate([np.arange(64 * j, min(64 * j + 64, n)) for j in kb]).astype(np.int64)
    k = int(max(r.size for r in rows.values()))
    ind_h = np.concatenate([[0], np.cumsum([rows[(0, h)].size for h in range(Hq)])]).astype(np.int64)
    S = torch.as_tensor(np.concatenate([rows[(0, h)] for h in range(Hq)]).astype(np.int32), device=dev)
    q, kc, vc = wl.random_qkv(1, Hq, Hkv, d, n, 991)
    out = ld.hybrid_layer(q.to(dev), kc.to(dev), vc.to(dev), 0x00, k, S, s_out=S,
                          s_indptr=torch.as_tensor(ind_h, device=dev), flags=ld.FLAG_BLOCK_SELECT)
    torch.cuda.synchronize()
    O_ref, _, _ = orc.hybrid_layer_bf16(wl.bf16_bits(q), wl.bf16_bits(kc), wl.bf16_bits(vc), [0, n],
                                        [False] * Hq, [k], rows)
    gh.check_outputs(out, O_ref, [(0, h) for h in range(Hq)], f"block sets, G = {Hq // Hkv}, n = {n}")
