"""ld_topk_select must equal the oracle's selection bit for bit on identical fp32
scores (LycheeDecode summary page, method step 3: S = argsTopK(scores, k); ties go
to the lower index, -0.0 equals +0.0, NaN ranks last)."""
import numpy as np
import pytest

from oracle import lychee_oracle as orc

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _ld():
    import hybrid_head_sparse_retrieval_amd as ld
    ld.load_library()
    return ld


def _check(rows_np, k, with_vals=True):
    ld = _ld()
    x = torch.as_tensor(np.ascontiguousarray(rows_np, dtype=np.float32), device="cuda")
    val = torch.empty((x.shape[0], k), dtype=torch.float32, device="cuda") if with_vals else None
    idx = ld.topk_select(x, k, val_out=val)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    for r in range(x.shape[0]):
        want = orc.select_topk_f32(rows_np[r].astype(np.float32), k)
        assert np.array_equal(got[r], want), f"row {r}: first mismatch at {np.nonzero(got[r] != want)[0][:5]}"
        if with_vals:
            v = val.cpu().numpy()[r]
            assert np.array_equal(v.view(np.uint32), rows_np[r].astype(np.float32)[want].view(np.uint32))


def _rng(s):
    return np.random.default_rng(s)


@pytest.mark.parametrize("n,k", [(1, 1), (7, 3), (64, 64), (511, 100), (512, 1), (513, 512),
                                 (5000, 1500), (32768, 9830), (131072, 39321)])
def test_random_normal(n, k):
    _check(_rng(n).normal(size=(3, n)).astype(np.float32), k)


def test_constant_rows_take_lowest_indices():
    for n, k in [(10, 4), (20000, 6000), (1025, 1025)]:
        _check(np.full((2, n), 0.5, dtype=np.float32), k)


def test_signed_zeros_infs_nans_and_duplicates():
    rng = _rng(1)
    pool = np.array([-1.0, -0.0, 0.0, 0.5, 2.0, np.inf, -np.inf, np.nan], dtype=np.float32)
    for n in (9, 300, 4097):
        rows = pool[rng.integers(0, len(pool), size=(4, n))]
        for k in sorted({1, 2, n // 3, n // 2, n - 1, n} - {0}):
            _check(rows, k)


def test_sorted_and_reverse_sorted():
    n = 10000
    inc = np.arange(n, dtype=np.float32)[None, :]
    _check(inc, 3000)
    _check(inc[:, ::-1].copy(), 3000)


def test_heavy_ties_at_threshold():
    # many keys equal to the k-th value: the kept ones are the lowest indices
    rng = _rng(2)
    n = 50000
    x = rng.integers(0, 4, size=(2, n)).astype(np.float32)
    for k in (1, 12345, 25000, 49999):
        _check(x, k)


@pytest.mark.parametrize("n", [4097, 30001, 32768])
def test_heavy_ties_within_two_spans(n):
    # one or two spans: many keys equal to the k-th value, NaN among them; only the lowest
    # indices among the ties are kept
    rng = _rng(n)
    x = rng.integers(0, 5, size=(3, n)).astype(np.float32)
    x[1, ::7] = np.nan
    for k in (1, n // 5, n // 2, n - 3):
        _check(x, k)


def test_near_ties_differ_in_last_bit():
    base = np.float32(0.7)
    n = 3000
    bits = (np.int64(base.view(np.uint32)) + np.arange(-5, 5)).astype(np.uint32)
    x = np.resize(bits.view(np.float32), n)[None, :]
    _check(x, 1000)


def test_many_rows_and_strided_input():
    ld = _ld()
    rng = _rng(3)
    full = rng.normal(size=(33, 1200)).astype(np.float32)
    x = torch.as_tensor(full, device="cuda")[:, :1000]     # row stride 1200
    idx = ld.topk_select(x, 250)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    for r in range(33):
        assert np.array_equal(got[r], orc.select_topk_f32(full[r, :1000], 250))


def test_repeated_calls_reuse_workspace():
    ld = _ld()
    rng = _rng(4)
    ws = ld.TopkWorkspace(2, 4000, "cuda")
    for it in range(5):
        x = rng.normal(size=(2, 4000)).astype(np.float32)
        idx = ld.topk_select(torch.as_tensor(x, device="cuda"), 1000 + it, workspace=ws)
        torch.cuda.synchronize()
        for r in range(2):
            assert np.array_equal(idx.cpu().numpy()[r], orc.select_topk_f32(x[r], 1000 + it))


def test_more_spans_than_resident_workgroups():
    # 300 rows of three 16384-score spans: more workgroups than the device holds at once
    # (the selection launches assume nothing about residency)
    rng = _rng(5)
    x = rng.normal(size=(300, 40000)).astype(np.float32)
    x[7, :] = 1.0                                   # a constant row: ties everywhere
    x[9, 100:200] = np.nan
    _check(x, 5100, with_vals=False)


@pytest.mark.parametrize("rows,n,k", [
    # digit-1 chunks are sized for about 256 workgroups; each case takes one load width
    (32, 131072, 1024),    # 16384-score chunks: two rounds of 8 float4 loads per thread
    (40, 40960, 12000),    # 8192-score chunks: one round of 8
    (8, 131072, 40000),    # 4096-score chunks: one round of 4
    (3, 131072, 39321),    # 2048-score chunks: one round of 2
    (50, 5000, 1500),      # 1024-score chunks: one float4 per thread, the ragged last chunk scalar
    (40, 16385, 5000),     # rows whose starts are not 16-byte aligned take the scalar loads
    (12, 40961, 12000),    # the same over three spans
    (6, 33000, 9000),      # a ragged last chunk over three spans
])
def test_digit1_chunk_sizes(rows, n, k):
    _check(_rng(7 + rows).normal(size=(rows, n)).astype(np.float32), k, with_vals=False)


def test_many_and_few_rows_agree_bitwise():
    ld = _ld()
    rng = _rng(6)
    x = rng.normal(size=(300, 20000)).astype(np.float32)
    x[:, 5000:5100] = 0.25                          # a block of ties near the threshold
    xt = torch.as_tensor(x, device="cuda")
    many = ld.topk_select(xt, 6000).cpu().numpy()   # 600 workgroups
    few = ld.topk_select(xt[:5], 6000).cpu().numpy()  # 10 workgroups
    assert np.array_equal(many[:5], few)
    for r in (0, 4, 299):
        assert np.array_equal(many[r], orc.select_topk_f32(x[r], 6000))


def test_in_launch_selection_repeated_fresh_workspaces():
    # selection inside the attention launch (one retrieval head per KV group): the S
    # rows equal the oracle's selection on the launch's own fp32 logits, call after
    # call with fresh workspaces (a regression test for a race between waves that
    # share the bin-search result)
    import workloads as wl
    ld = _ld()
    dev = "cuda"
    B, Hq, Hkv, d, n, k = 2, 4, 4, 64, 3000, 900
    q, kc, vc = wl.random_qkv(B, Hq, Hkv, d, B * n, 200)
    qd, kd, vd = q.to(dev), kc.to(dev), vc.to(dev)
    shape = ld.make_shape(qd, kd, None, n)
    for trial in range(4):
        ws = ld.Workspace(shape, k, dev)
        S = torch.zeros((B, Hq, k), dtype=torch.int32, device=dev)
        scores = torch.full((B, Hq, n), float("nan"), dtype=torch.float32, device=dev)
        ld.hybrid_layer(qd, kd, vd, 0xF, k, None, s_out=S, scores_out=scores, workspace=ws, seq_len=n,
                        flags=ld.flag_waves(1))
        torch.cuda.synchronize()
        sc, Sh = scores.cpu().numpy(), S.cpu().numpy()
        for b in range(B):
            for h in range(Hq):
                assert np.array_equal(Sh[b, h], orc.select_topk_f32(sc[b, h], k)), (trial, b, h)


def test_undersized_outputs_are_rejected_before_launch():
    ld = _ld()
    x = torch.zeros((3, 1000), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="idx_out"):
        ld.topk_select(x, 10, idx_out=torch.empty(29, dtype=torch.int32, device="cuda"))
    with pytest.raises(ValueError, match="val_out"):
        ld.topk_select(x, 10, val_out=torch.empty(29, dtype=torch.float32, device="cuda"))


def _check_ragged(rows_np, n_r, k_r, *, csr, k_default, sentinel=-7):
    """Rows of their own lengths n_r and budgets k_r (None: the default k), dense or CSR
    output: every row equals the oracle on its first n_r scores with min(k_r, n_r)
    indices (the pages' clamp), and entries past them keep the sentinel."""
    ld = _ld()
    rows, n = rows_np.shape
    x = torch.as_tensor(np.ascontiguousarray(rows_np, dtype=np.float32), device="cuda")
    nt = torch.as_tensor(np.asarray(n_r, dtype=np.int32), device="cuda")
    kt = None if k_r is None else torch.as_tensor(np.asarray(k_r, dtype=np.int32), device="cuda")
    want_k = [min(k_default if k_r is None else k_r[r], n_r[r]) for r in range(rows)]
    if csr:
        cap = [max(0, kk) + 3 for kk in want_k]            # room to spare: the tail stays
        off = np.concatenate([[0], np.cumsum(cap)]).astype(np.int64)
        ind = torch.as_tensor(off, device="cuda")
        out = torch.full((int(off[-1]),), sentinel, dtype=torch.int32, device="cuda")
        ld.topk_select(x, k_default, idx_out=out, n_per_row=nt, k_per_row=kt, idx_indptr=ind)
        got = out.cpu().numpy()
        rows_got = [got[off[r]:off[r + 1]] for r in range(rows)]
    else:
        out = torch.full((rows, k_default), sentinel, dtype=torch.int32, device="cuda")
        ld.topk_select(x, k_default, idx_out=out, n_per_row=nt, k_per_row=kt)
        rows_got = list(out.cpu().numpy())
    for r in range(rows):
        kk = max(0, min(want_k[r], len(rows_got[r])))
        if kk >= 1:
            want = orc.select_topk_f32(rows_np[r, :n_r[r]].astype(np.float32), kk)
            assert np.array_equal(rows_got[r][:kk], want), f"row {r} (n {n_r[r]}, k {kk})"
        assert np.all(rows_got[r][kk:] == sentinel), f"row {r}: entries past k_r were written"


@pytest.mark.parametrize("n", [3000, 40000])
def test_ragged_rows_with_their_own_k_dense_and_csr(n):
    rng = _rng(n + 5)
    rows = 9
    x = rng.normal(size=(rows, n)).astype(np.float32)
    n_r = [n, 1, n // 2, 777, n - 3, 64, 0, n // 3 + 1, 2]
    k_r = [int(0.3 * v) for v in n_r]
    k_r[1] = 5                                              # k above the row length: clamped to it
    k_r[3] = 777
    for csr in (False, True):
        _check_ragged(x, n_r, k_r, csr=csr, k_default=max(k_r))
        _check_ragged(x, n_r, None, csr=csr, k_default=n // 4)


def test_k_above_n_is_clamped():
    """k > n keeps every score (k = min(k, n), Token Sparse Attention skill page, Step 3)."""
    x = _rng(3).normal(size=(2, 50)).astype(np.float32)
    _check_ragged(x, [50, 50], None, csr=False, k_default=80)
