"""CPU oracle for the hybrid-head sparse decode step (LycheeDecode).

TEST INFRASTRUCTURE ONLY. This module is the slow, plain, fp64 statement of what
the decode step computes. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import it; the product path (the HIP library and its Python
binding) never does, and shares no code, headers, tables or helpers with it.

Sources (cited by page title and passage):
  [LD]  "LycheeDecode: Accelerating Long-Context LLM Inference via Hybrid-Head
        Sparse Decoding" (summary page of arXiv 2602.04541), method paragraph,
        steps (1), (3), (4) and (7); reproducibility paragraph (30 % key-token budget).
  [SK]  "LycheeDecode: Head-Level KV Cache Sharing" (skill page), Step 3
        "Implement Hybrid Attention Layer" (1/sqrt(head_dim) scaling, softmax, 0.5
        head-type threshold).
  [HS]  "HySparse: A Hybrid Sparse Attention Architecture with Oracle Token
        Selection and KV Cache Sharing", section 3 Methodology (sparse layers reuse
        the full layer's token selection and KV cache).
  [TSA] "Token Sparse Attention: Efficient Long-Context Inference" (skill page),
        Step 3 (the budget is clamped to the sequence length: k = min(k, seq_len)),
        "Core Concept" and Steps 2-3 (compress to the top-k tokens, dense attention
        among them, scatter back to the sequence).

Readings taken where the pages are silent (each is listed in the design notes):
  * Head type and the token set S are per *query* head; under grouped KV heads,
    query head h reads KV head g = h // (Hq // Hkv).
  * argsTopK ranks the logits q.k/sqrt(d) (softmax is strictly increasing per row,
    so the selected set equals that of the probabilities whenever they are untied).
    Total order: larger value first; equal values -> lower index first; -0.0 equals
    +0.0; NaN ranks below every number (NaNs among themselves by index).
  * S is a set; it is stored in ascending index order.
  * No causal mask at decode: the single query attends to all N cached rows.
  * A sparse head reads its own layer's K/V at S ([LD] step 4); for HySparse-style
    stacks the caller passes the full layer's K/V ([HS] section 3).
  * Prefill (the extension [LD]'s future-work paragraph names): see
    prefill_hybrid_layer for the readings of a multi-row attention matrix.

Parity pins: tests/test_oracle_pins.py checks every function here against closed
forms, hand-derived examples (tests/golden/), brute-force ranking and invariants.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "bf16_bits_to_f64",
    "fp8_e4m3_to_f64",
    "hybrid_layer_fp8",
    "select_topk_blocks",
    "hysparse_sparse_layer",
    "tsa_attention",
    "prefill_hybrid_layer",
    "softmax_attention",
    "select_topk",
    "select_topk_f32",
    "retrieval_head",
    "sparse_head",
    "hybrid_layer_f64",
    "hybrid_layer_bf16",
    "default_scale",
]


def default_scale(head_dim: int) -> float:
    """1/sqrt(d_k) ([LD] step 3; [SK] Step 3)."""
    return 1.0 / math.sqrt(head_dim)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64.

    A bf16 value is the upper half of an IEEE binary32 word, so shifting the 16 bits
    into the high half gives the identical float32, which widens exactly to float64.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def fp8_e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """Exact value of 8-bit E4M3 floating-point codes (uint8), the OCP 8-bit floating
    point format used for quantised KV caches: 1 sign bit, 4 exponent bits with bias 7,
    3 mantissa bits. Exponent field 0 encodes subnormals m/8 * 2^-6; the codes with all
    exponent and mantissa bits set (0x7F, 0xFF) are NaN; there are no infinities, so
    the largest magnitude is 1.75 * 2^8 = 448.

    The pages name quantised KV only as a combinable extension; the format is the
    reading taken here.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((e == 15) & (c & 0x7 == 7), np.nan, mag)
    return sign * mag


def softmax_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray,
                      scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """One query row against n cached rows, in fp64 ([LD] step 3).

    s_i = (q . K_i) * scale;  w_i = exp(s_i - max s);  O = sum_i w_i V_i / sum_i w_i.
    Returns (O [d], s [n]).
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    assert K.ndim == 2 and K.shape[0] >= 1, "softmax over an empty set is undefined"
    s = (K @ q) * scale
    m = np.max(s)
    w = np.exp(s - m)
    O = (w @ V) / np.sum(w)
    return O, s


def select_topk(scores: np.ndarray, k: int) -> np.ndarray:
    """argsTopK ([LD] step 3): the k best entries under the total order above,
    returned as ascending int64 indices."""
    s = np.asarray(scores)
    n = s.shape[0]
    assert 1 <= k <= n, "k must satisfy 1 <= k <= n"
    s = s.astype(np.float64)                     # exact for float32 inputs
    isnan = np.isnan(s)
    v = np.where(isnan, 0.0, s) + 0.0            # -0.0 + 0.0 == +0.0
    # lexsort: last key is primary -> non-NaN first, then value descending,
    # then index ascending.
    order = np.lexsort((np.arange(n), -v, isnan))
    return np.sort(order[:k]).astype(np.int64)


def select_topk_f32(scores_f32: np.ndarray, k: int) -> np.ndarray:
    """The same selection applied to float32 values exactly as given."""
    s = np.asarray(scores_f32)
    assert s.dtype == np.float32
    return select_topk(s, k)


def select_topk_blocks(scores: np.ndarray, k: int, block: int = 64) -> np.ndarray:
    """Token-block selection of HySparse (section 3 Methodology): the full layer's
    scores are reduced to one score per block of `block` consecutive tokens, the block
    maximum, and the k / block blocks with the largest block scores are kept; their
    tokens form the set handed to the sparse layers. Block scores are ranked like token
    scores (select_topk: larger first, lower block index first on ties, NaN lowest; a
    block's maximum ignores NaN unless every score in it is NaN). Returns the token
    indices of the kept blocks in ascending order (exactly k of them).

    Reading taken: the pages give the block maximum and k/B blocks (B = 64); this form
    requires n and k to be multiples of the block size.
    """
    s = np.asarray(scores, dtype=np.float64)
    n = s.size
    assert n % block == 0 and k % block == 0 and 0 < k <= n
    blocks = s.reshape(n // block, block)
    with np.errstate(invalid="ignore"):
        allnan = np.all(np.isnan(blocks), axis=1)
        bmax = np.where(allnan, np.nan, np.nanmax(np.where(np.isnan(blocks), -np.inf, blocks), axis=1))
    kept = select_topk(bmax, k // block)
    return (kept[:, None] * block + np.arange(block)[None, :]).reshape(-1)


def retrieval_head(q, K, V, k: int, scale: float):
    """Retrieval head ([LD] step 3): full attention over all n rows, then
    S_next = argsTopK(scores, k). Returns (O, S_next, scores)."""
    O, s = softmax_attention(q, K, V, scale)
    return O, select_topk(s, k), s


def sparse_head(q, K, V, S: np.ndarray, scale: float):
    """Sparse head ([LD] step 4): attention over rows S of its own layer's K/V;
    S is forwarded unchanged. Returns (O, S)."""
    S = np.asarray(S, dtype=np.int64)
    n = K.shape[0]
    assert S.ndim == 1 and S.size >= 1
    assert np.all((S >= 0) & (S < n)), "S entries must lie in [0, n)"
    assert np.unique(S).size == S.size, "S entries must be distinct"
    O, _ = softmax_attention(q, K[S], V[S], scale)
    return O, S


def hybrid_layer_f64(Q: np.ndarray, K: np.ndarray, V: np.ndarray,
                     kv_offsets: Sequence[int], retrieval: Sequence[bool],
                     k_per_seq: Sequence[int], S_in: Optional[Dict[Tuple[int, int], np.ndarray]],
                     scale: Optional[float] = None, active: Optional[Sequence[bool]] = None,
                     ):
    """One layer of the recurrence for every (sequence b, query head h).

    Q: [B][Hq][d]; K, V: [Hkv][T][d] (sequence b owns rows kv_offsets[b]:kv_offsets[b+1]).
    retrieval[h]: True for a retrieval head (the inference split E[z] > 0.5 of
    [LD] step 7 is given as this mask). S_in[(b, h)]: the set handed over by the
    previous layer (required for every active sparse head).
    active[h]: heads to compute (default all).

    Returns (O [B][Hq][d] with NaN rows for inactive heads,
             S_out {(b,h): indices}, scores {(b,h): fp64 scores of retrieval rows}).
    S_out[(b,h)] = argsTopK for retrieval heads ([LD] step 3), S_in[(b,h)] for sparse
    heads ([LD] step 4).
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    B, Hq, d = Q.shape
    Hkv = K.shape[0]
    assert Hq % Hkv == 0
    G = Hq // Hkv
    if scale is None:
        scale = default_scale(d)
    if active is None:
        active = [True] * Hq
    O = np.full((B, Hq, d), np.nan)
    S_out: Dict[Tuple[int, int], np.ndarray] = {}
    scores: Dict[Tuple[int, int], np.ndarray] = {}
    for b in range(B):
        lo, hi = int(kv_offsets[b]), int(kv_offsets[b + 1])
        n = hi - lo
        kb = min(int(k_per_seq[b]), n)           # [TSA] Step 3 clamp
        for h in range(Hq):
            if not active[h]:
                if S_in is not None and (b, h) in S_in:
                    S_out[(b, h)] = np.asarray(S_in[(b, h)], dtype=np.int64)
                continue
            g = h // G
            Kg, Vg = K[g, lo:hi], V[g, lo:hi]
            if retrieval[h]:
                O[b, h], S_out[(b, h)], scores[(b, h)] = retrieval_head(Q[b, h], Kg, Vg, kb, scale)
            else:
                assert S_in is not None and (b, h) in S_in, "sparse head needs S from the previous layer"
                O[b, h], S_out[(b, h)] = sparse_head(Q[b, h], Kg, Vg, S_in[(b, h)], scale)
    return O, S_out, scores


def hybrid_layer_bf16(q_bits, k_bits, v_bits, kv_offsets, retrieval, k_per_seq, S_in,
                      scale=None, active=None):
    """hybrid_layer_f64 on raw bf16 bit patterns (uint16), widened exactly."""
    return hybrid_layer_f64(bf16_bits_to_f64(q_bits), bf16_bits_to_f64(k_bits),
                            bf16_bits_to_f64(v_bits), kv_offsets, retrieval, k_per_seq,
                            S_in, scale=scale, active=active)


def hybrid_layer_fp8(q_bits, k_codes, v_codes, k_scale, v_scale, kv_offsets, retrieval, k_per_seq,
                     S_in, scale=None, active=None):
    """hybrid_layer_f64 with a quantised KV cache: K = k_scale * E4M3(k_codes) and
    V = v_scale * E4M3(v_codes) (one scale per tensor), Q from bf16 bits."""
    return hybrid_layer_f64(bf16_bits_to_f64(q_bits), float(k_scale) * fp8_e4m3_to_f64(k_codes),
                            float(v_scale) * fp8_e4m3_to_f64(v_codes), kv_offsets, retrieval,
                            k_per_seq, S_in, scale=scale, active=active)


def hysparse_sparse_layer(Q, K, V, kv_offsets, S_in, Kw, Vw, gate, scale=None):
    """A HySparse sparse layer ([HS] section 3 Methodology): each query head runs two
    branches and mixes them with a sigmoid gate.

    Block-sparse branch: sparse_head over rows S_in[(b, h)] of the shared cache K, V
    ([Hkv][T][d], sequence b at kv_offsets[b]:kv_offsets[b+1]), i.e. the KV cache and
    the selection of the preceding full layer.
    Window branch: softmax_attention over the layer's own cache Kw, Vw ([Hkv][B*W][d];
    rows b*W:(b+1)*W hold the last W tokens of sequence b).
    Output: O = w * O_sparse + (1 - w) * O_window with w = 1 / (1 + exp(-gate[b][h])).

    Readings taken: one scalar gate per (sequence, query head), given as an input (the
    pages fix the sigmoid, not the gate's producer); w multiplies the sparse branch and
    1 - w the window branch. Returns O [B][Hq][d].
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    Kw = np.asarray(Kw, dtype=np.float64)
    Vw = np.asarray(Vw, dtype=np.float64)
    gate = np.asarray(gate, dtype=np.float64)
    B, Hq, d = Q.shape
    Hkv = K.shape[0]
    G = Hq // Hkv
    W = Kw.shape[1] // B
    assert Kw.shape[1] == B * W and W >= 1
    if scale is None:
        scale = default_scale(d)
    O = np.empty((B, Hq, d))
    for b in range(B):
        lo, hi = int(kv_offsets[b]), int(kv_offsets[b + 1])
        for h in range(Hq):
            g = h // G
            o_s, _ = sparse_head(Q[b, h], K[g, lo:hi], V[g, lo:hi], S_in[(b, h)], scale)
            o_w, _ = softmax_attention(Q[b, h], Kw[g, b * W:(b + 1) * W], Vw[g, b * W:(b + 1) * W], scale)
            w = 1.0 / (1.0 + math.exp(-gate[b, h]))
            O[b, h] = w * o_s + (1.0 - w) * o_w
    return O


def tsa_attention(Q, K, V, scores, k: int, scale=None, causal: bool = False, zero_fill: bool = True):
    """Token Sparse Attention, compress -> dense -> scatter ([TSA] "Core Concept" and
    Steps 2-3), for every (sequence b, query head h) of a prefill of T tokens.

    Q: [Hq][B*T][d]; K, V: [Hkv][B*T][d] (query head h reads KV head h // (Hq // Hkv));
    scores: [B][Hq][T] per-token importance of each head.
    Compress: I = argsTopK(scores[b][h], min(k, T)) (select_topk order, ascending).
    Dense: among the selected tokens only, O_i = softmax_j(q_{I_i} . k_{I_j} * scale) v_{I_j};
    causal: only keys with I_j <= I_i.
    Scatter: row I_i of the output gets O_i; every other row is zero (zero_fill) or NaN
    (left to the caller).

    Readings taken: the scores are an input (the page's scoring formulas are not legible);
    no mask unless causal is asked for (the page's listing applies none).
    Returns (out [Hq][B*T][d], idx {(b, h): ascending int64 indices}).
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    sc = np.asarray(scores)
    Hq, BT, d = Q.shape
    Hkv = K.shape[0]
    G = Hq // Hkv
    B, _, T = sc.shape
    assert BT == B * T
    if scale is None:
        scale = default_scale(d)
    kk = min(int(k), T)                          # [TSA] Step 3 clamp
    out = np.zeros((Hq, BT, d)) if zero_fill else np.full((Hq, BT, d), np.nan)
    idx = {}
    for b in range(B):
        for h in range(Hq):
            g = h // G
            I = select_topk(sc[b, h], kk)
            idx[(b, h)] = I
            rows = b * T + I
            Ks, Vs = K[g, rows], V[g, rows]
            for i in range(kk):
                keys = np.arange(kk) if not causal else np.arange(i + 1)   # I ascending: I_j <= I_i iff j <= i
                out[h, rows[i]], _ = softmax_attention(Q[h, rows[i]], Ks[keys], Vs[keys], scale)
    return out, idx


def prefill_hybrid_layer(Q, K, V, batch: int, retrieval: Sequence[bool], k: int,
                         S_in: Optional[Dict[Tuple[int, int], np.ndarray]] = None, scale=None):
    """One layer of the hybrid-head recurrence ([LD] steps 3 and 4) applied to a prefill
    of T prompt tokens per sequence instead of one decode token.

    Q: [Hq][B*T][d]; K, V: [Hkv][B*T][d] (query head h reads KV head h // (Hq // Hkv));
    the rows of sequence b are b*T .. b*T + T - 1, and query row t sees key rows 0..t of
    its own sequence (the prompt is causal).
    Retrieval head h: A = softmax(Q_h K_h^T * scale) under that mask, O = A V, and
    S_next = argsTopK(A, k) read as the k tokens with the largest column sums of A
    (importance_j = sum over rows t >= j of A[t, j], the attention mass token j receives
    in the prompt), ranked like select_topk.
    Sparse head h: row t attends to the tokens of S_in[(b, h)] at positions <= t only;
    a row with none of them (t below the set's first token) outputs zeros. S is
    forwarded unchanged.

    Readings taken (the pages name the extension but give no formula for it): the
    token set stays one set per head and layer, as in decoding, so that S is the same
    object the decode recurrence hands on; with one query row (T = 1) every rule above
    is the decode layer's. Returns (O [Hq][B*T][d], S_out {(b, h): ascending int64},
    importance {(b, h): [T] fp64} for retrieval heads).
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    Hq, BT, d = Q.shape
    Hkv = K.shape[0]
    G = Hq // Hkv
    B = int(batch)
    assert BT % B == 0 and len(retrieval) == Hq
    T = BT // B
    assert 1 <= k <= T
    if scale is None:
        scale = default_scale(d)
    O = np.zeros((Hq, BT, d))
    S_out: Dict[Tuple[int, int], np.ndarray] = {}
    importance: Dict[Tuple[int, int], np.ndarray] = {}
    for b in range(B):
        r0 = b * T
        for h in range(Hq):
            g = h // G
            Kb, Vb = K[g, r0:r0 + T], V[g, r0:r0 + T]
            if retrieval[h]:
                col = np.zeros(T)
                for t in range(T):
                    O[h, r0 + t], s = softmax_attention(Q[h, r0 + t], Kb[:t + 1], Vb[:t + 1], scale)
                    w = np.exp(s - np.max(s))
                    col[:t + 1] += w / np.sum(w)       # row t of A (its entries past t are 0)
                importance[(b, h)] = col
                S_out[(b, h)] = select_topk(col, k)
            else:
                assert S_in is not None, "sparse heads need S from the previous layer"
                S = np.asarray(S_in[(b, h)], dtype=np.int64)
                assert np.all((S >= 0) & (S < T)) and np.unique(S).size == S.size
                for t in range(T):
                    vis = S[S <= t]
                    if vis.size:
                        O[h, r0 + t], _ = softmax_attention(Q[h, r0 + t], Kb[vis], Vb[vis], scale)
                S_out[(b, h)] = np.sort(S)
    return O, S_out, importance


def decode_step_f64(layers: List[Tuple[np.ndarray, np.ndarray, np.ndarray]],
                    kv_offsets, retrieval_masks: Sequence[Sequence[bool]], k_per_seq,
                    scale=None):
    """The whole recurrence over L layers ([LD] steps (1), (3), (4)).

    layers[l] = (Q, K, V) in fp64. Layer 0 must be all retrieval ([LD] step 1).
    Returns lists of per-layer O and S_out.
    """
    assert all(retrieval_masks[0]), "every head of layer 0 is a retrieval head"
    S = None
    outs, sets = [], []
    for l, (Q, K, V) in enumerate(layers):
        O, S, _ = hybrid_layer_f64(Q, K, V, kv_offsets, retrieval_masks[l], k_per_seq, S, scale)
        outs.append(O)
        sets.append(S)
    return outs, sets
