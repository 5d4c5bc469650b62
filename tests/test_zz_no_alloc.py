"""The allocation-free layer entry point (ld_hybrid_layer_noalloc) against the
workspace entry point (ld_hybrid_layer) on the same inputs: two calls in a row on the
library's static scratch, the second with a smaller shape, each compared with the
workspace call (S bit for bit, O within the oracle tolerances) and with the oracle."""
import numpy as np
import pytest
import torch

import hybrid_head_sparse_retrieval_amd as ld
import workloads as wl
from oracle import lychee_oracle as orc
from gpu_helpers import MAX_ABS, REL_L2, check_outputs, HostLayer

pytestmark = pytest.mark.gpu


def _case(B, Hq, Hkv, d, N, k, mask, seed):
    dev = torch.device("cuda:0")
    q, kc, vc = wl.random_qkv(B, Hq, Hkv, d, B * N, seed)
    q = q.reshape(B, Hq, d)
    S_in = torch.as_tensor(wl.random_sorted_sets(seed + 1, N, k, B * Hq).reshape(B, Hq, k), dtype=torch.int32)
    return q.to(dev), kc.to(dev), vc.to(dev), S_in.to(dev)


def _run_pair(B, Hq, Hkv, d, N, k, mask, seed):
    q, kc, vc, S_in = _case(B, Hq, Hkv, d, N, k, mask, seed)
    out_ws = torch.empty_like(q)
    S_ws = S_in.clone()
    ws = ld.Workspace(ld.make_shape(q, kc), k, q.device)
    ld.hybrid_layer(q, kc, vc, mask, k, S_ws, out=out_ws, workspace=ws)
    out_na = torch.full_like(q, float("nan"))
    S_na = S_in.clone()
    print(f"[no-alloc] B={B} Hq={Hq} Hkv={Hkv} d={d} N={N} k={k} mask={mask:#x}", flush=True)
    ld.hybrid_layer_noalloc(q, kc, vc, mask, k, S_na, out=out_na)
    torch.cuda.synchronize()
    return q, kc, vc, S_in, out_ws, S_ws, out_na, S_na


@pytest.mark.parametrize("first,second", [
    ((1, 32, 8, 128, 32768, 9830, 0x00010002), (1, 4, 4, 64, 1024, 307, 0x1)),
    ((2, 8, 2, 128, 8192, 2457, 0x0F), (1, 8, 4, 64, 777, 233, 0x81)),
])
def test_noalloc_matches_workspace_entry(first, second):
    for i, cfg in enumerate((first, second)):
        B, Hq, Hkv, d, N, k, mask = cfg
        q, kc, vc, S_in, out_ws, S_ws, out_na, S_na = _run_pair(B, Hq, Hkv, d, N, k, mask, 1000 + 17 * i)
        # the static-scratch call equals the workspace call
        assert torch.equal(S_na, S_ws), f"call {i}: S differs from the workspace entry point"
        a = out_na.float().cpu().numpy()
        b = out_ws.float().cpu().numpy()
        assert np.all(np.isfinite(a)), f"call {i}: non-finite output"
        err = float(np.abs(a - b).max())
        rel = float(np.linalg.norm(a - b) / np.linalg.norm(b))
        assert err <= MAX_ABS and rel <= REL_L2, f"call {i}: O differs (max {err:.2e}, rel {rel:.2e})"
        # and the oracle (teacher forcing on S_in)
        h = HostLayer(q, kc, vc)
        ret = [bool(mask >> j & 1) for j in range(Hq)]
        S_dict = {(b_, j): S_in[b_, j].cpu().numpy().astype(np.int64) for b_ in range(B) for j in range(Hq)}
        offs = np.arange(B + 1, dtype=np.int64) * N
        O_ref, _, _ = orc.hybrid_layer_bf16(h.q, h.k, h.v, offs, ret, [k] * B, S_dict)
        check_outputs(out_na, O_ref, [(b_, j) for b_ in range(B) for j in range(Hq)], f"call {i}")
        # sparse rows untouched
        for b_ in range(B):
            for j in range(Hq):
                if not ret[j]:
                    assert torch.equal(S_na[b_, j], S_in[b_, j])


def test_noalloc_rejects_a_shape_beyond_its_scratch():
    dev = torch.device("cuda:0")
    q = torch.zeros((1, 32, 128), dtype=torch.bfloat16, device=dev)
    kc = torch.zeros((8, 1 << 20, 128), dtype=torch.bfloat16, device=dev)
    out = torch.empty_like(q)
    S = torch.zeros((1, 32, 16), dtype=torch.int32, device=dev)
    with pytest.raises(ld.LycheeDecodeError) as e:
        ld.hybrid_layer_noalloc(q, kc, kc, 0xffffffff, 16, None, s_out=S, out=out)
    assert e.value.status == 6
