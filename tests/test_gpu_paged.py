"""Paged KV: the same layers with K/V scattered over a pool of pages (a random page order,
unused pool rows filled with NaN, so a wrong read shows up in O) give O and S bit for bit
equal to the contiguous layout, and match the oracle. Covers stream and gather groups,
GQA and MHA, a ragged CSR batch, and page sizes from 16 to 256 rows."""
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


def _paged_pool(kc, vc, offs, page, seed, extra_pages=7):
    """Scatter the rows of each sequence over pages of a shuffled pool. Returns the pool
    tensors [Hkv][pages*page][d] and the block table [B][pages_per_seq] (int32)."""
    rng = np.random.default_rng(seed)
    B = len(offs) - 1
    lens = np.diff(offs)
    npp = [(int(n) + page - 1) // page for n in lens]
    pps = max(npp) + 2
    total_pages = sum(npp) + extra_pages
    order = rng.permutation(total_pages)
    Hkv, _, d = kc.shape
    kp = torch.full((Hkv, total_pages * page, d), float("nan"), dtype=torch.bfloat16)
    vp = torch.full((Hkv, total_pages * page, d), float("nan"), dtype=torch.bfloat16)
    bt = np.asarray(rng.integers(0, total_pages, size=(B, pps)), dtype=np.int32)  # unused slots: any page
    nxt = 0
    for b in range(B):
        for j in range(npp[b]):
            pid = int(order[nxt]); nxt += 1
            bt[b, j] = pid
            r0 = int(offs[b]) + j * page
            r1 = min(int(offs[b + 1]), r0 + page)
            kp[:, pid * page: pid * page + (r1 - r0)] = kc[:, r0:r1]
            vp[:, pid * page: pid * page + (r1 - r0)] = vc[:, r0:r1]
    return kp, vp, torch.as_tensor(bt)


@pytest.mark.parametrize("case", [
    # (B, Hq, Hkv, d, lens, masks, page, csr)
    (1, 8, 2, 128, [5000], [0xFF, 0x11, 0x00], 64, False),
    (1, 8, 2, 128, [3000], [0xFF, 0x12], 16, False),
    (1, 4, 4, 64, [2100], [0xF, 0x1], 256, False),
    (3, 8, 2, 128, [1900, 4200, 777], [0xFF, 0x24], 128, True),
])
def test_paged_equals_contiguous_and_oracle(case):
    B, Hq, Hkv, d, lens, masks, page, csr = case
    ld = _ld()
    dev = "cuda"
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T, N = int(offs[-1]), max(lens)
    ragged = B > 1
    kb = [max(1, int(0.3 * n)) for n in lens]
    kv_indptr = torch.as_tensor(offs, device=dev) if ragged else None
    if csr:
        rows = [kb[b] for b in range(B) for _ in range(Hq)]
        s_indptr_h = np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)
        s_indptr = torch.as_tensor(s_indptr_h, device=dev)
        mkS = lambda: torch.zeros(int(s_indptr_h[-1]), dtype=torch.int32, device=dev)
        kmax = max(kb)
    else:
        s_indptr_h, s_indptr = None, None
        mkS = lambda: torch.zeros((B, Hq, kb[0]), dtype=torch.int32, device=dev)
        kmax = kb[0]
    layers = [wl.random_qkv(B, Hq, Hkv, d, T, 700 + l) for l in range(len(masks))]
    S_c, S_p = mkS(), mkS()
    ws_c = ws_p = None
    for l, mask in enumerate(masks):
        qc, kc, vc = layers[l]
        kp, vp, bt = _paged_pool(kc, vc, offs, page, 900 + l)
        q = qc.to(dev)
        shape_c = ld.make_shape(q, kc.to(dev), kv_indptr, N)
        shape_p = ld.make_shape(q, kp.to(dev), kv_indptr, N, None, bt.to(dev), page)
        if ws_c is None:
            ws_c, ws_p = ld.Workspace(shape_c, kmax, dev), ld.Workspace(shape_p, kmax, dev)
        flags = ld.FLAG_S_CHAINED if l > 0 else 0
        S_before = S_c.cpu().numpy().copy()
        out_c = ld.hybrid_layer(q, kc.to(dev), vc.to(dev), mask, kmax, S_c if l else None, s_out=S_c,
                                s_indptr=s_indptr, flags=flags, workspace=ws_c, kv_indptr=kv_indptr,
                                seq_len=N)
        out_p = ld.hybrid_layer(q, kp.to(dev), vp.to(dev), mask, kmax, S_p if l else None, s_out=S_p,
                                s_indptr=s_indptr, flags=flags, workspace=ws_p, kv_indptr=kv_indptr,
                                seq_len=N, block_table=bt.to(dev), page_size=page)
        torch.cuda.synchronize()
        assert torch.equal(out_c.view(torch.int16), out_p.view(torch.int16)), f"layer {l}: O differs"
        assert torch.equal(S_c, S_p), f"layer {l}: S differs"
        ret = [bool(mask >> h & 1) for h in range(Hq)]
        S_in = None if l == 0 else gh.s_rows_to_dict(S_before, B, Hq, s_indptr_h)
        O_ref, _, _ = orc.hybrid_layer_bf16(wl.bf16_bits(qc), wl.bf16_bits(kc), wl.bf16_bits(vc), offs,
                                            ret, kb, S_in)
        gh.check_outputs(out_p, O_ref, [(b, h) for b in range(B) for h in range(Hq)], f"paged layer {l}")
    ws_c.check()
    ws_p.check()
