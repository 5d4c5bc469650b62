"""Seeded synthetic workloads for the hybrid-head sparse decode step.

This module only *draws inputs*: shapes, seeds, bf16 tensors, head-type masks and
sorted index sets. It holds none of the method's arithmetic (no attention, no
softmax, no selection), so that the CPU oracle and the HIP path can both consume
the same bytes without sharing any computation.

Workload shapes follow the two models the LycheeDecode README names for its
latency results (Llama-3-8B-Instruct-1048k and Qwen3-8B: 32 query heads, 8 KV
heads, head dim 128), the key-token budget of 30 % of the sequence and the
retrieval-head budget of 32 from the LycheeDecode summary page (reproducibility
paragraph), contexts up to 128K from the LycheeDecode skill page (Practical
Guidance), and the HySparse block of one full layer followed by sparse layers
that reuse its KV cache (HySparse, section 3 Methodology).

Value recipe (the pages evaluate on long-context suites that are not available
here; these synthetic draws stand in for them):
  * Q, K, V elements ~ N(0, 1) in fp32, rounded to nearest-even bf16.
  * Planted heavy hitters: per (sequence b, KV head g) a position set P of
    floor(f * N_b) positions (f = 2 % for the tiny workload, 1 % otherwise), drawn
    without replacement and shared by all layers. In layer l, for p in P,
    K[g][p] = 4 * u + eps_p where u is the unit vector along the mean query of the
    group's query heads and eps_p is that row's own N(0, 1) draw.
  * Head-type masks: layer 0 all retrieval; 32 further retrieval heads at seeded
    distinct (layer >= 1, head) slots (or an explicit mask for the tiny workload).
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import List, Optional, Sequence

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "get_workload",
    "stream_seed",
    "LayerInputs",
    "make_layer_inputs",
    "heavy_hitter_positions",
    "bf16_bits",
    "random_sorted_sets",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    """Static description of one decode-step workload."""

    name: str
    index: int                 # base seed
    batch: int
    layers: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    seq_lens: tuple            # per-sequence context length N_b
    k_per_seq: tuple           # per-sequence token budget k_b
    retrieval_masks: tuple     # per layer: int bitmask, bit h set = retrieval head
    heavy_frac: float
    shared_kv_from_layer0: bool = False   # HySparse-style: layers >= 1 read layer 0's K/V
    ragged_csr: bool = False              # S stored in CSR (per-sequence k)

    @property
    def group_size(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def max_seq(self) -> int:
        return max(self.seq_lens)

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seq_lens))

    def kv_offsets(self) -> np.ndarray:
        """Token offsets [B+1]: sequence b occupies rows [off[b], off[b+1])."""
        return np.concatenate([[0], np.cumsum(self.seq_lens)]).astype(np.int64)

    def kv_layers(self) -> int:
        """Number of distinct per-layer KV caches that must be resident."""
        return 1 if self.shared_kv_from_layer0 else self.layers


def stream_seed(*parts) -> int:
    """Deterministic 63-bit seed from a tuple of ints/strings (blake2b)."""
    h = hashlib.blake2b(repr(tuple(parts)).encode(), digest_size=8).digest()
    return int.from_bytes(h, "little") & ((1 << 63) - 1)


def _seeded_mask(index: int, layers: int, hq: int, extra: int) -> tuple:
    rng = np.random.Generator(np.random.PCG64(stream_seed(index, "mask")))
    slots = rng.choice((layers - 1) * hq, size=extra, replace=False)
    masks = [(1 << hq) - 1] + [0] * (layers - 1)
    for s in slots:
        l, h = 1 + int(s) // hq, int(s) % hq
        masks[l] |= 1 << h
    return tuple(masks)


def _floor30(n: int) -> int:
    return (3 * n) // 10


def _build() -> dict:
    w = {}
    w["tiny"] = Workload(
        name="tiny", index=1, batch=1, layers=2, num_q_heads=4, num_kv_heads=4,
        head_dim=64, seq_lens=(1024,), k_per_seq=(307,),
        retrieval_masks=(0b1111, 0b0001), heavy_frac=0.02)
    w["llama3_8b_32k"] = Workload(
        name="llama3_8b_32k", index=2, batch=1, layers=32, num_q_heads=32,
        num_kv_heads=8, head_dim=128, seq_lens=(32768,), k_per_seq=(_floor30(32768),),
        retrieval_masks=_seeded_mask(2, 32, 32, 32), heavy_frac=0.01)
    w["qwen3_8b_128k"] = Workload(
        name="qwen3_8b_128k", index=3, batch=1, layers=36, num_q_heads=32,
        num_kv_heads=8, head_dim=128, seq_lens=(131072,), k_per_seq=(_floor30(131072),),
        retrieval_masks=_seeded_mask(3, 36, 32, 32), heavy_frac=0.01)
    rng = np.random.Generator(np.random.PCG64(stream_seed(4, "lens")))
    lens = tuple(int(x) for x in rng.integers(16384, 65536, size=8, endpoint=True))
    w["ragged_b8"] = Workload(
        name="ragged_b8", index=4, batch=8, layers=32, num_q_heads=32, num_kv_heads=8,
        head_dim=128, seq_lens=lens, k_per_seq=tuple(_floor30(n) for n in lens),
        retrieval_masks=_seeded_mask(2, 32, 32, 32), heavy_frac=0.01, ragged_csr=True)
    # between the two headline lengths: the Llama-3-8B layout at 64K (launch-shape checks)
    w["llama3_8b_64k"] = Workload(
        name="llama3_8b_64k", index=6, batch=1, layers=32, num_q_heads=32,
        num_kv_heads=8, head_dim=128, seq_lens=(65536,), k_per_seq=(_floor30(65536),),
        retrieval_masks=_seeded_mask(2, 32, 32, 32), heavy_frac=0.01)
    w["hysparse_7layer"] = Workload(
        name="hysparse_7layer", index=5, batch=1, layers=7, num_q_heads=32,
        num_kv_heads=8, head_dim=128, seq_lens=(131072,), k_per_seq=(4096,),
        retrieval_masks=((1 << 32) - 1,) + (0,) * 6, heavy_frac=0.01,
        shared_kv_from_layer0=True)
    return w


WORKLOADS = _build()


def get_workload(name: str, **overrides) -> Workload:
    """Return a named workload, optionally with fields replaced (e.g. layers=4)."""
    w = WORKLOADS[name]
    return dataclasses.replace(w, **overrides) if overrides else w


def heavy_hitter_positions(w: Workload, b: int, g: int) -> np.ndarray:
    """Planted positions for (sequence b, KV head g), sorted, shared across layers."""
    n = w.seq_lens[b]
    cnt = int(np.floor(w.heavy_frac * n))
    rng = np.random.Generator(np.random.PCG64(stream_seed(w.index, "plant", b, g)))
    return np.sort(rng.choice(n, size=cnt, replace=False)).astype(np.int64)


@dataclasses.dataclass
class LayerInputs:
    q: "torch.Tensor"          # bf16 [B][Hq][d]
    k: "torch.Tensor"          # bf16 [Hkv][T_total][d]
    v: "torch.Tensor"          # bf16 [Hkv][T_total][d]


def _randn(shape, seed: int, device) -> "torch.Tensor":
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def make_layer_inputs(w: Workload, layer: int, device="cpu", q_only: bool = False) -> LayerInputs:
    """Draw Q, K, V for one layer (bf16) with planted heavy hitters.

    For HySparse-style workloads, layers >= 1 draw only Q (their K/V is layer 0's).
    """
    import torch
    B, Hq, Hkv, d = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim
    q32 = _randn((B, Hq, d), stream_seed(w.index, layer, "q"), device)
    q = q32.to(torch.bfloat16)
    if q_only or (w.shared_kv_from_layer0 and layer > 0):
        return LayerInputs(q=q, k=None, v=None)
    T = w.total_tokens
    k32 = _randn((Hkv, T, d), stream_seed(w.index, layer, "k"), device)
    v = _randn((Hkv, T, d), stream_seed(w.index, layer, "v"), device).to(torch.bfloat16)
    offs = w.kv_offsets()
    G = w.group_size
    for b in range(B):
        for g in range(Hkv):
            pos = heavy_hitter_positions(w, b, g)
            if pos.size == 0:
                continue
            mean_q = q32[b, g * G:(g + 1) * G].mean(dim=0)
            u = mean_q / mean_q.norm()
            rows = torch.as_tensor(pos + offs[b], device=device)
            k32[g, rows] = 4.0 * u + k32[g, rows]
    k = k32.to(torch.bfloat16)
    del k32
    return LayerInputs(q=q, k=k, v=v)


def bf16_bits(t) -> np.ndarray:
    """Raw bf16 bit patterns of a torch bf16 tensor as a numpy uint16 array (host copy)."""
    import torch
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def random_sorted_sets(seed: int, n: int, k: int, rows: int) -> np.ndarray:
    """rows x k distinct indices in [0, n), each row sorted ascending (int32)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = np.empty((rows, k), dtype=np.int32)
    for r in range(rows):
        out[r] = np.sort(rng.choice(n, size=k, replace=False))
    return out


def random_qkv(B: int, Hq: int, Hkv: int, d: int, T: int, seed: int, scale_q: float = 1.0):
    """Unstructured N(0,1) draws in bf16 (CPU tensors): q [B][Hq][d], k, v [Hkv][T][d]."""
    import torch
    g = torch.Generator(device="cpu")
    g.manual_seed(stream_seed("qkv", seed))
    q = (torch.randn((B, Hq, d), generator=g) * scale_q).to(torch.bfloat16)
    k = torch.randn((Hkv, T, d), generator=g).to(torch.bfloat16)
    v = torch.randn((Hkv, T, d), generator=g).to(torch.bfloat16)
    return q, k, v


def seeded_masks(seed: int, layers: int, hq: int, per_layer: int) -> list:
    """Layer 0 all retrieval, then `per_layer` seeded retrieval heads in each later layer."""
    rng = np.random.Generator(np.random.PCG64(stream_seed("masks", seed)))
    out = [(1 << hq) - 1]
    for _ in range(1, layers):
        m = 0
        for h in rng.choice(hq, size=min(per_layer, hq), replace=False):
            m |= 1 << int(h)
        out.append(m)
    return out
