"""C-ABI contract checks that need no GPU: the library loads, exports every symbol the
header declares, sizes workspaces, and rejects invalid arguments on the host before
launching anything (no call here reaches a kernel)."""
import ctypes
import os
import re

import pytest

import hybrid_head_sparse_retrieval_amd as ld

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lychee_decode.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ld.library_path()):
        pytest.fail("liblychee_decode.so is not built (run __graft_entry__.build())")
    return ld.load_library()


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:ld_status|size_t|const char\*)\s+(ld_\w+)\s*\(", txt, re.M)))


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert set(names) == set(ld.EXPORTED_SYMBOLS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in range(7):
        assert lib.ld_status_string(code)
    assert lib.ld_status_string(99) == b"unknown status"


def _shape(**kw):
    s = ld.Shape()
    s.batch, s.num_q_heads, s.num_kv_heads, s.head_dim, s.seq_len = 1, 32, 8, 128, 32768
    for k, v in kw.items():
        setattr(s, k, v)
    return s


FAKE = 0x10000  # a 16-byte-aligned non-null address; never dereferenced (validation fails first)


def test_workspace_size(lib):
    s = _shape()
    n = lib.ld_workspace_size(ctypes.byref(s), 9830)
    assert n > 0 and n % 256 == 0
    # scales with the sequence length
    s2 = _shape(seq_len=65536)
    assert lib.ld_workspace_size(ctypes.byref(s2), 9830) > n
    # invalid shapes give 0
    for bad in (dict(head_dim=96), dict(num_kv_heads=5), dict(num_q_heads=65, num_kv_heads=65),
                dict(seq_len=0), dict(batch=0), dict(num_kv_heads=2),
                # paged KV: page size not a power of two in 16..4096, no table, a table that
                # does not cover seq_len, a pool of partial pages, table fields without paging
                dict(page_size=48, pages_per_seq=1024, block_table=FAKE, total_tokens=1 << 20),
                dict(page_size=8, pages_per_seq=4096, block_table=FAKE, total_tokens=1 << 20),
                dict(page_size=64, pages_per_seq=512, block_table=None, total_tokens=1 << 20),
                dict(page_size=64, pages_per_seq=511, block_table=FAKE, total_tokens=1 << 20),
                dict(page_size=64, pages_per_seq=512, block_table=FAKE, total_tokens=(1 << 20) + 32),
                dict(page_size=0, pages_per_seq=512), dict(page_size=0, block_table=FAKE),
                # quantised KV: unknown format, missing or bad scales, scales without it
                dict(kv_dtype=2), dict(kv_dtype=1), dict(kv_dtype=1, k_scale=1.0, v_scale=-1.0),
                dict(kv_dtype=1, k_scale=float("inf"), v_scale=1.0), dict(kv_dtype=0, k_scale=1.0),
                dict(reserved=1)):
        assert lib.ld_workspace_size(ctypes.byref(_shape(**bad)), 10) == 0, bad
    paged = _shape(page_size=64, pages_per_seq=512, block_table=FAKE, total_tokens=1 << 20)
    assert lib.ld_workspace_size(ctypes.byref(paged), 10) > 0
    fp8 = _shape(kv_dtype=1, k_scale=0.5, v_scale=2.0)
    assert lib.ld_workspace_size(ctypes.byref(fp8), 10) > 0
    assert lib.ld_workspace_size(ctypes.byref(s), 0) == 0
    assert lib.ld_workspace_size(ctypes.byref(s), 32769) == 0
    assert lib.ld_topk_workspace_size(4, 1000) > 0
    assert lib.ld_topk_workspace_size(0, 1000) == 0


def _hyb(lib, shape, **kw):
    a = dict(mask=1, q=FAKE, k=FAKE, v=FAKE, kk=10, s_in=FAKE, s_out=FAKE, s_indptr=None,
             scores=None, out=FAKE, flags=0, ws=FAKE, wsb=1 << 40)
    a.update(kw)
    return lib.ld_hybrid_layer(ctypes.byref(shape), a["mask"], a["q"], a["k"], a["v"], a["kk"],
                               a["s_in"], a["s_out"], a["s_indptr"], a["scores"], a["out"],
                               a["flags"], a["ws"], a["wsb"], None)


def test_invalid_arguments_are_rejected(lib):
    s = _shape()
    INV, UNS, WSE = 1, 2, 3
    assert _hyb(lib, s, q=None) == INV
    assert _hyb(lib, s, out=None) == INV
    assert _hyb(lib, s, k=FAKE + 2) == INV                  # misaligned K
    assert _hyb(lib, s, kk=0) == INV                        # k < 1
    assert _hyb(lib, s, kk=32769) == INV                    # k > N
    assert _hyb(lib, s, mask=1 << 40) == INV                # head beyond Hq
    assert _hyb(lib, s, s_in=None) == INV                   # sparse heads without S
    assert _hyb(lib, s, s_out=None) == INV                  # retrieval heads, top-k, no S out
    assert _hyb(lib, s, ws=None) == WSE
    assert _hyb(lib, s, wsb=1024) == WSE
    assert _hyb(lib, _shape(head_dim=80)) == UNS
    assert _hyb(lib, _shape(num_kv_heads=2)) == UNS         # group of 16
    assert _hyb(lib, _shape(num_kv_heads=3)) == INV         # does not divide
    assert _hyb(lib, _shape(seq_len=(1 << 21) + 1)) == UNS
    # scale must be finite
    assert _hyb(lib, _shape(softmax_scale=float("inf"))) == INV


def test_noalloc_rejects_before_any_device_call(lib):
    """The allocation-free layer validates the shape and its scratch size on the host
    first: a shape larger than the static buffer, or an invalid one, never reaches
    the device (no GPU here, so a call that passed validation would return LD_ERR_HIP)."""
    INV, UNS, LIMIT = 1, 2, 6

    def na(shape, mask=1):
        return lib.ld_hybrid_layer_noalloc(ctypes.byref(shape), mask, FAKE, FAKE, FAKE, 10, FAKE, FAKE,
                                           None, None, FAKE, 0, None)
    big = _shape(seq_len=1 << 20)
    assert lib.ld_workspace_size(ctypes.byref(big), 10) > ld.NOALLOC_SCRATCH_BYTES
    assert na(big) == LIMIT
    fits = _shape()
    assert lib.ld_workspace_size(ctypes.byref(fits), 9830) <= ld.NOALLOC_SCRATCH_BYTES
    assert na(_shape(head_dim=80)) == UNS
    assert na(fits, mask=1 << 40) == INV


def test_csr_s_needs_its_capacity(lib):
    """CSR S rows are clipped to ld_shape.s_capacity on the device; a call with CSR
    offsets and no capacity is rejected before any launch."""
    s = _shape()
    assert _hyb(lib, s, s_indptr=FAKE) == 1
    assert _hyb(lib, _shape(s_capacity=-1)) == 1


def test_binding_clamps_k_and_sets_the_s_capacity():
    class Buf:
        def __init__(self, n):
            self.n = n

        def numel(self):
            return self.n
    s = _shape(seq_len=100)
    assert ld._clamp_k(s, 250, None, [("s", Buf(10))]) == 100 and s.s_capacity == 0
    assert ld._clamp_k(s, 30, object(), [("s", Buf(500)), ("s_out", Buf(400))]) == 30
    assert s.s_capacity == 400
    with pytest.raises(ValueError):
        ld._clamp_k(s, 0, None, [])


def test_hysparse_workspace_and_arguments(lib):
    s = _shape()
    n = lib.ld_hysparse_workspace_size(ctypes.byref(s), 9830, 128)
    assert n > lib.ld_workspace_size(ctypes.byref(s), 9830) and n % 256 == 0
    for w in (0, -1, 4097):
        assert lib.ld_hysparse_workspace_size(ctypes.byref(s), 9830, w) == 0
    assert lib.ld_hysparse_workspace_size(ctypes.byref(_shape(head_dim=96)), 10, 128) == 0

    def hys(shape, **kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, kk=10, s_in=FAKE, s_indptr=None, kw=FAKE, vw=FAKE, w=128,
                 gate=FAKE, out=FAKE, flags=0, ws=FAKE, wsb=1 << 40)
        a.update(kw)
        return lib.ld_hysparse_layer(ctypes.byref(shape), a["q"], a["k"], a["v"], a["kk"], a["s_in"],
                                     a["s_indptr"], a["kw"], a["vw"], a["w"], a["gate"], a["out"],
                                     a["flags"], a["ws"], a["wsb"], None)
    INV, UNS, WSE = 1, 2, 3
    assert hys(s, w=0) == INV and hys(s, w=4097) == INV
    assert hys(s, kw=None) == INV and hys(s, gate=None) == INV and hys(s, s_in=None) == INV
    assert hys(s, vw=FAKE + 8) == INV                       # misaligned window cache
    assert hys(s, gate=FAKE + 2) == INV
    assert hys(s, flags=4) == INV                           # selection modes are the full layer's
    assert hys(s, flags=1) == INV
    assert hys(s, flags=2 | 8 | 16) == INV                  # an unknown bit beside the accepted ones
    assert hys(s, ws=None) == WSE and hys(s, wsb=1 << 20) == WSE
    assert hys(_shape(head_dim=80)) == UNS


def test_tsa_workspace_and_arguments(lib):
    s = _shape(seq_len=4096, total_tokens=4096)
    assert lib.ld_tsa_workspace_size(ctypes.byref(s), 1024) >= lib.ld_topk_workspace_size(32, 4096) > 0
    assert lib.ld_tsa_workspace_size(ctypes.byref(s), 0) == 0
    for bad in (dict(head_dim=96), dict(kv_dtype=1, k_scale=1.0, v_scale=1.0),
                dict(page_size=64, pages_per_seq=512, block_table=FAKE, total_tokens=1 << 20)):
        assert lib.ld_tsa_workspace_size(ctypes.byref(_shape(**bad)), 64) == 0, bad

    def tsa(shape, **kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, sc=FAKE, kk=64, idx=FAKE, out=FAKE, flags=0, ws=FAKE, wsb=1 << 40)
        a.update(kw)
        return lib.ld_tsa_attention(ctypes.byref(shape), a["q"], a["k"], a["v"], a["sc"], a["kk"], a["idx"],
                                    a["out"], a["flags"], a["ws"], a["wsb"], None)
    INV, UNS, WSE = 1, 2, 3
    assert tsa(s, q=None) == INV and tsa(s, sc=None) == INV and tsa(s, idx=None) == INV
    assert tsa(s, kk=0) == INV
    assert tsa(s, k=FAKE + 4) == INV and tsa(s, sc=FAKE + 2) == INV
    assert tsa(s, flags=8) == INV                           # unknown flag
    assert tsa(_shape(seq_len=4096, total_tokens=4095)) == INV
    assert tsa(s, ws=None) == WSE and tsa(s, wsb=1024) == WSE
    assert tsa(_shape(seq_len=4096, total_tokens=4096, head_dim=80)) == UNS
    assert tsa(_shape(kv_dtype=1, k_scale=1.0, v_scale=1.0)) == UNS


def test_topk_invalid_arguments(lib):
    f = lib.ld_topk_select

    def call(sc=FAKE, rows=1, n=10, stride=10, n_per_row=None, k=3, k_per_row=None, idx=FAKE, ind=None,
             val=None, ws=FAKE, wsb=1 << 30):
        return f(sc, rows, n, stride, n_per_row, k, k_per_row, idx, ind, val, ws, wsb, None)
    assert call(sc=None) == 1 and call(idx=None) == 1
    assert call(k=0) == 1                                   # k < 1
    assert call(stride=9) == 1                              # rows overlap
    assert call(n=0) == 1 and call(rows=0) == 1
    assert call(n_per_row=FAKE + 2) == 1                    # misaligned per-row arrays
    assert call(k_per_row=FAKE + 1) == 1
    assert call(ind=FAKE + 4) == 1                          # int64 offsets: 8-byte aligned
    assert call(ws=16, wsb=16) == 3
    assert call(wsb=16) == 3


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import importlib
    monkeypatch.setattr(ld, "_lib", None)
    monkeypatch.setattr(ld, "library_path", lambda: str(tmp_path / "missing.so"))
    with pytest.raises(ld.LycheeDecodeUnavailable):
        ld.load_library()


def test_layer_plan_validates_like_the_layer(lib):
    """ld_hybrid_layer_plan applies the layer's own argument checks before it asks the
    device anything; a missing plan pointer is rejected too."""
    INV, UNS = 1, 2
    plan = ld.LayerPlan()

    def pl(shape, mask=1, kk=10, s_in=FAKE, p=True):
        return lib.ld_hybrid_layer_plan(ctypes.byref(shape), mask, FAKE, FAKE, FAKE, kk, s_in, FAKE,
                                        None, None, FAKE, 0, ctypes.byref(plan) if p else None)
    assert pl(_shape(), p=False) == INV
    assert pl(_shape(), kk=0) == INV
    assert pl(_shape(), mask=1 << 40) == INV
    assert pl(_shape(), s_in=None) == INV                   # sparse heads without S
    assert pl(_shape(head_dim=80)) == UNS


def test_prefill_workspace_and_arguments(lib):
    """The prefill layer takes one contiguous bf16 prompt per sequence; invalid shapes
    and arguments are rejected on the host (no call here reaches a kernel)."""
    INV, UNS, WSE = 1, 2, 3
    s = _shape(seq_len=4096)
    n = lib.ld_prefill_workspace_size(ctypes.byref(s), 1000)
    assert n >= 2 * 32 * 4096 * 4                          # log-sum-exp and column sums
    assert lib.ld_prefill_workspace_size(ctypes.byref(s), 0) == 0
    assert lib.ld_prefill_workspace_size(ctypes.byref(s), 4097) == 0
    fp8 = _shape(seq_len=4096, kv_dtype=1, k_scale=1.0, v_scale=1.0)
    assert lib.ld_prefill_workspace_size(ctypes.byref(fp8), 10) == 0

    def pf(shape, mask=(1 << 32) - 1, kk=100, s_in=None, s_out=FAKE, flags=0, ws=FAKE, wsb=1 << 40):
        return lib.ld_prefill_hybrid_layer(ctypes.byref(shape), mask, FAKE, FAKE, FAKE, kk, s_in, s_out, None,
                                           FAKE, flags, ws, wsb, None)
    assert pf(s, mask=1) == INV                            # sparse heads without S
    assert pf(s, s_out=None) == INV                        # retrieval heads select into nothing
    assert pf(s, kk=0) == INV and pf(s, kk=4097) == INV
    assert pf(s, flags=ld.FLAG_S_CHAINED) == INV           # only LD_FLAG_SKIP_TOPK is taken
    assert pf(s, ws=None) == WSE and pf(s, wsb=16) == WSE
    assert pf(fp8) == UNS                                  # 8-bit codes: decode only
    assert pf(_shape(seq_len=4096, kv_indptr=FAKE)) == UNS   # ragged prompts
    assert pf(_shape(seq_len=4096, head_dim=80)) == UNS
