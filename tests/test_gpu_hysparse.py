"""HySparse sparse layer (HySparse, section 3 Methodology): a block-sparse branch over
rows S of the shared (full layer's) cache and a window branch over the layer's own
cache of the last W tokens, mixed per head by sigmoid(gate). Output vs the oracle on
the same bf16 bytes, uniform and ragged batches, one-token and full windows."""
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
    # (lens, Hq, Hkv, d, k, W, seed)
    ([4096], 8, 2, 128, 1280, 128, 970),
    ([8192, 8192], 32, 8, 128, 2048, 128, 971),
    ([3000, 777, 2048], 4, 4, 64, 300, 1, 972),
    ([5000, 1400], 8, 1, 128, 1000, 300, 973),
    ([6000], 8, 2, 128, 1500, 4096, 974),       # the largest window
    ([2500, 2500], 4, 2, 64, 800, 200, 975),
    ([2048], 64, 8, 64, 256, 16, 976),          # 64 query heads: every bit of the head masks
])
def test_hysparse_layer_matches_oracle(case):
    lens, Hq, Hkv, d, k, W, seed = case
    ld = _ld()
    dev = "cuda"
    B, N = len(lens), max(lens)
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(offs[-1])
    ragged = len(set(lens)) > 1
    q, kc, vc = wl.random_qkv(B, Hq, Hkv, d, T, seed)
    _, kw, vw = wl.random_qkv(B, Hq, Hkv, d, B * W, seed + 50)
    g = torch.Generator().manual_seed(wl.stream_seed("gate", seed))
    gate = torch.randn((B, Hq), generator=g) * 3.0
    gate[0, 0] = 40.0           # saturated: the sparse branch alone
    gate[-1, Hq - 1] = -40.0    # saturated: the window branch alone
    kb = [min(k, n) for n in lens]
    rows = [wl.random_sorted_sets(wl.stream_seed("S", seed, b), lens[b], kb[b], Hq) for b in range(B)]
    if ragged:
        s_indptr_h = np.concatenate([[0], np.cumsum([kb[b] for b in range(B) for _ in range(Hq)])]).astype(np.int64)
        S_h = np.concatenate([r.reshape(-1) for r in rows]).astype(np.int32)
        s_indptr = torch.as_tensor(s_indptr_h, device=dev)
        kv_indptr = torch.as_tensor(offs, device=dev)
    else:
        S_h = np.stack(rows).astype(np.int32)
        s_indptr_h = s_indptr = kv_indptr = None
    S = torch.as_tensor(S_h, device=dev)
    qd, kd, vd = q.to(dev), kc.to(dev), vc.to(dev)
    out = ld.hysparse_layer(qd, kd, vd, max(kb), S, kw.to(dev), vw.to(dev), gate.to(dev), s_indptr=s_indptr,
                            kv_indptr=kv_indptr, seq_len=N)
    torch.cuda.synchronize()
    S_in = gh.s_rows_to_dict(S_h, B, Hq, s_indptr_h)
    O_ref = orc.hysparse_sparse_layer(gh.bf16_tensor_to_f64(q), gh.bf16_tensor_to_f64(kc),
                                      gh.bf16_tensor_to_f64(vc), offs, S_in, gh.bf16_tensor_to_f64(kw),
                                      gh.bf16_tensor_to_f64(vw), gate.numpy().astype(np.float64))
    gh.check_outputs(out, O_ref, [(b, h) for b in range(B) for h in range(Hq)], f"hysparse {case}")


def test_hysparse_layer_chained_and_repeated():
    """Several sparse layers of one HySparse block share one S and one workspace
    (bitmaps built once, then chained); every layer matches the oracle."""
    ld = _ld()
    dev = "cuda"
    B, Hq, Hkv, d, N, k, W = 2, 16, 4, 128, 6144, 1536, 128
    q0, kc, vc = wl.random_qkv(B, Hq, Hkv, d, B * N, 980)
    kd, vd = kc.to(dev), vc.to(dev)
    S_h = np.stack([wl.random_sorted_sets(wl.stream_seed("S", 980, b), N, k, Hq) for b in range(B)])
    S = torch.as_tensor(S_h, device=dev)
    shape = ld.make_shape(q0.to(dev), kd)
    ws = ld.HySparseWorkspace(shape, k, W, dev)
    for layer in range(3):
        q, _, _ = wl.random_qkv(B, Hq, Hkv, d, 1, 981 + layer)
        _, kw, vw = wl.random_qkv(B, Hq, Hkv, d, B * W, 990 + layer)
        g = torch.Generator().manual_seed(wl.stream_seed("gate", 980, layer))
        gate = torch.randn((B, Hq), generator=g) * 2.0
        out = ld.hysparse_layer(q.to(dev), kd, vd, k, S, kw.to(dev), vw.to(dev), gate.to(dev),
                                flags=ld.FLAG_S_CHAINED if layer else 0, workspace=ws)
        torch.cuda.synchronize()
        O_ref = orc.hysparse_sparse_layer(gh.bf16_tensor_to_f64(q), gh.bf16_tensor_to_f64(kc),
                                          gh.bf16_tensor_to_f64(vc), [0, N, 2 * N],
                                          gh.s_rows_to_dict(S_h, B, Hq), gh.bf16_tensor_to_f64(kw),
                                          gh.bf16_tensor_to_f64(vw), gate.numpy().astype(np.float64))
        gh.check_outputs(out, O_ref, [(b, h) for b in range(B) for h in range(Hq)], f"hysparse layer {layer}")
    ws.check()


def test_hysparse_layer_rejects_bad_arguments():
    ld = _ld()
    dev = "cuda"
    q, kc, vc = wl.random_qkv(1, 4, 4, 64, 1024, 985)
    qd, kd, vd = q.to(dev), kc.to(dev), vc.to(dev)
    S = torch.as_tensor(wl.random_sorted_sets(985, 1024, 64, 4)[None], device=dev)
    gate = torch.zeros((1, 4), dtype=torch.float32, device=dev)
    kw = torch.zeros((4, 5000, 64), dtype=torch.bfloat16, device=dev)
    shape = ld.make_shape(qd, kd)
    with pytest.raises(ld.LycheeDecodeError, match="invalid argument"):
        ld.hysparse_workspace_bytes(shape, 64, 5000)       # window above 4096
    with pytest.raises(ld.LycheeDecodeError, match="invalid argument"):
        ld.hysparse_layer(qd, kd, vd, 64, S, kw, kw, gate)
    kw = torch.zeros((4, 16, 64), dtype=torch.bfloat16, device=dev)
    ws = ld.HySparseWorkspace(shape, 64, 16, dev)
    with pytest.raises(ld.LycheeDecodeError, match="invalid argument"):
        ld.hysparse_layer(qd, kd, vd, 64, S, kw, kw, gate, flags=ld.FLAG_SEPARATE_SELECT, workspace=ws)


def test_full_layer_then_hysparse_layers_share_one_workspace():
    """A HySparse block through the step runner: the full layer (all heads retrieval,
    64-token block selection) writes S and the bitmaps into the leading part of the
    HySparse workspace; the sparse layers chain from them and add their window
    branches. Every sparse layer matches the oracle on the full layer's S."""
    from hybrid_head_sparse_retrieval_amd.step import DecodeStep
    ld = _ld()
    dev = "cuda"
    B, Hq, Hkv, d, N, k, W, L = 1, 16, 4, 128, 8192, 2048, 128, 3
    step = DecodeStep(B, Hq, Hkv, d, [N], [k], [(1 << Hq) - 1] + [0] * (L - 1), device=dev,
                      split_flag=ld.FLAG_BLOCK_SELECT, window_len=W)
    q0, kc, vc = wl.random_qkv(B, Hq, Hkv, d, N, 1000)
    kd, vd = kc.to(dev), vc.to(dev)
    layers, windows, host = [(q0.to(dev), kd, vd)], [None], []
    for l in range(1, L):
        q, _, _ = wl.random_qkv(B, Hq, Hkv, d, 1, 1000 + l)
        _, kw, vw = wl.random_qkv(B, Hq, Hkv, d, B * W, 1100 + l)
        gate = torch.randn((B, Hq), generator=torch.Generator().manual_seed(wl.stream_seed("gate", 1000, l)))
        layers.append((q.to(dev), kd, vd))
        windows.append((kw.to(dev), vw.to(dev), gate.to(dev)))
        host.append((q, kw, vw, gate))
    outs = step.run(layers, windows=windows)
    torch.cuda.synchronize()
    S = step.s_rows()
    for l in range(1, L):
        q, kw, vw, gate = host[l - 1]
        O_ref = orc.hysparse_sparse_layer(gh.bf16_tensor_to_f64(q), gh.bf16_tensor_to_f64(kc),
                                          gh.bf16_tensor_to_f64(vc), [0, N], S, gh.bf16_tensor_to_f64(kw),
                                          gh.bf16_tensor_to_f64(vw), gate.numpy().astype(np.float64))
        gh.check_outputs(outs[l], O_ref, [(0, h) for h in range(Hq)], f"hysparse block layer {l}")
    for h in range(Hq):
        assert S[(0, h)].size == k and np.all(S[(0, h)] % 64 == np.arange(k) % 64)
    step.workspace.check()


def test_hysparse_layer_on_paged_e4m3_shared_cache():
    """The block-sparse branch reads a paged pool of E4M3 codes with per-tensor scales
    (the full layer's cache); the window cache stays bf16. Output vs the oracle on the
    decoded values."""
    ld = _ld()
    dev = "cuda"
    B, Hq, Hkv, d, N, k, W, page = 2, 8, 2, 128, 4096, 1200, 128, 64
    k_scale, v_scale = 0.75, 1.5
    q, kc, vc = wl.random_qkv(B, Hq, Hkv, d, B * N, 990)
    _, kw, vw = wl.random_qkv(B, Hq, Hkv, d, B * W, 991)
    k8 = kc.float().to(torch.float8_e4m3fn).view(torch.uint8)
    v8 = vc.float().to(torch.float8_e4m3fn).view(torch.uint8)
    # pool of pages in a seeded order; block_table[b][i] = pool page of page i of sequence b
    npp = N // page
    perm = np.random.default_rng(wl.stream_seed("pages", 990)).permutation(B * npp)
    table = perm.reshape(B, npp).astype(np.int32)
    kp = torch.empty_like(k8)
    vp = torch.empty_like(v8)
    for b in range(B):
        for i in range(npp):
            src = slice(b * N + i * page, b * N + (i + 1) * page)
            dst = slice(int(table[b, i]) * page, (int(table[b, i]) + 1) * page)
            kp[:, dst] = k8[:, src]
            vp[:, dst] = v8[:, src]
    S_h = np.stack([wl.random_sorted_sets(wl.stream_seed("S", 990, b), N, k, Hq) for b in range(B)])
    gate = torch.randn((B, Hq), generator=torch.Generator().manual_seed(wl.stream_seed("gate", 990))) * 2.0
    bt = torch.as_tensor(table, device=dev)
    out = ld.hysparse_layer(q.to(dev), kp.to(dev), vp.to(dev), k, torch.as_tensor(S_h, device=dev), kw.to(dev),
                            vw.to(dev), gate.to(dev), seq_len=N, block_table=bt, page_size=page,
                            k_scale=k_scale, v_scale=v_scale)
    torch.cuda.synchronize()
    K = k_scale * orc.fp8_e4m3_to_f64(k8.numpy())
    V = v_scale * orc.fp8_e4m3_to_f64(v8.numpy())
    O_ref = orc.hysparse_sparse_layer(gh.bf16_tensor_to_f64(q), K, V, [0, N, 2 * N], gh.s_rows_to_dict(S_h, B, Hq),
                                      gh.bf16_tensor_to_f64(kw), gh.bf16_tensor_to_f64(vw),
                                      gate.numpy().astype(np.float64))
    gh.check_outputs(out, O_ref, [(b, h) for b in range(B) for h in range(Hq)], "hysparse paged e4m3")
