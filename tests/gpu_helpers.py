"""Shared helpers of the GPU parity tests: run layers through the C ABI, run the
oracle on the same bf16 bytes, and compare with the stated tolerances."""
from __future__ import annotations

import numpy as np

import workloads as wl
from oracle import lychee_oracle as orc

# Output tolerances per head (oracle fp64 vs GPU bf16 output).
MAX_ABS = 1e-2
REL_L2 = 5e-3
# End-to-end selected sets may differ only at scores within this relative distance
# of the k-th score.
TIE_REL = 1e-5


def bf16_tensor_to_f64(t):
    return orc.bf16_bits_to_f64(wl.bf16_bits(t))


def check_outputs(O_gpu_bf16, O_ref, heads, what=""):
    """O_gpu_bf16: torch bf16 [B][Hq][d]; O_ref fp64 [B][Hq][d]; heads: iterable of (b,h)."""
    G = bf16_tensor_to_f64(O_gpu_bf16)
    worst = (0.0, 0.0, None)
    for (b, h) in heads:
        ref = O_ref[b, h]
        got = G[b, h]
        assert np.all(np.isfinite(got)), f"{what} non-finite output at {(b, h)}"
        err = np.abs(got - ref).max()
        rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
        assert err <= MAX_ABS, f"{what} head {(b, h)}: max abs err {err:.3e}"
        assert rel <= REL_L2, f"{what} head {(b, h)}: rel L2 {rel:.3e}"
        if rel > worst[1]:
            worst = (err, rel, (b, h))
    return worst


def check_selected_row(S_gpu_row, scores_gpu_row_f32, scores_ref_f64, k, what=""):
    """(a) bit-exact vs the oracle's selection on the GPU's own fp32 scores;
    (b) vs the oracle's fp64 selection, differences only inside the tie zone."""
    S_gpu_row = np.asarray(S_gpu_row, dtype=np.int64)
    exact = orc.select_topk_f32(np.asarray(scores_gpu_row_f32, dtype=np.float32), k)
    if not np.array_equal(S_gpu_row, exact):
        extra = np.setdiff1d(S_gpu_row, exact)[:6]
        missing = np.setdiff1d(exact, S_gpu_row)[:6]
        sc = np.asarray(scores_gpu_row_f32, dtype=np.float32)
        kth = np.sort(sc)[::-1][k - 1]
        raise AssertionError(
            f"{what}GPU selection differs from the oracle on identical fp32 scores: len {S_gpu_row.size} vs {k}, "
            f"extra {extra.tolist()} (scores {sc[extra].tolist()}), missing {missing.tolist()} "
            f"(scores {sc[missing].tolist()}), k-th score {kth!r}")
    ref = orc.select_topk(scores_ref_f64, k)
    diff = np.setxor1d(S_gpu_row, ref)
    if diff.size:
        kth = np.sort(scores_ref_f64)[::-1][k - 1]
        zone = np.abs(scores_ref_f64[diff] - kth) <= TIE_REL * abs(kth)
        assert np.all(zone), f"selected sets differ outside the tie zone at {diff[~zone][:8]}"
    return diff.size


class HostLayer:
    """Host copies (bf16 bits) of one layer's inputs."""

    def __init__(self, q, k, v):
        self.q = wl.bf16_bits(q)
        self.k = wl.bf16_bits(k)
        self.v = wl.bf16_bits(v)


def s_rows_to_dict(S_host, B, Hq, s_indptr_host=None, k=None):
    d = {}
    for b in range(B):
        for h in range(Hq):
            r = b * Hq + h
            if s_indptr_host is None:
                d[(b, h)] = S_host[b, h].astype(np.int64)
            else:
                d[(b, h)] = S_host[s_indptr_host[r]:s_indptr_host[r + 1]].astype(np.int64)
    return d
