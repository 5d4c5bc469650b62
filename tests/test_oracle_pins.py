"""Pins for the CPU oracle against things other than itself: hand-derived golden
examples, closed forms, brute-force ranking and invariants of the recurrence on the
LycheeDecode summary page (method steps (1), (3), (4))."""
import json
import math
import os

import numpy as np
import pytest

from oracle import lychee_oracle as orc
from tests.conftest import GOLDEN


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f(x):
    return float(x)  # "nan", "inf", "-inf" strings parse too


# ----------------------------------------------------------------- bf16 widening

def test_bf16_widening_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x7F80, 0xFF80, 0x0000, 0x8000, 0x3E80, 0x4049, 0x0001],
                    dtype=np.uint16)
    got = orc.bf16_bits_to_f64(bits)
    want = [1.0, -2.0, math.inf, -math.inf, 0.0, -0.0, 0.25, 3.140625, 2.0 ** -133]
    for g, w in zip(got, want):
        assert g == w and math.copysign(1, g) == math.copysign(1, w)
    assert np.isnan(orc.bf16_bits_to_f64(np.array([0x7FC0], dtype=np.uint16)))[0]


# ------------------------------------------------------------ attention closed forms

def test_two_token_golden():
    g = _load("two_token_softmax.json")
    O, s = orc.softmax_attention(np.array(g["q"]), np.array(g["K"]), np.array(g["V"]),
                                 orc.default_scale(4))
    np.testing.assert_allclose(O, g["expected_O"], rtol=1e-14, atol=1e-13)
    np.testing.assert_allclose(s, g["expected_scores"], rtol=1e-14, atol=1e-15)


def test_single_row_returns_value_row():
    rng = np.random.default_rng(0)
    q, K, V = rng.normal(size=8), rng.normal(size=(1, 8)), rng.normal(size=(1, 8))
    O, _ = orc.softmax_attention(q, K, V, 0.3)
    assert np.array_equal(O, V[0])


@pytest.mark.parametrize("d", [4, 64, 128])
def test_identical_keys_give_mean_of_values(d):
    rng = np.random.default_rng(d)
    n = 37
    q = rng.normal(size=d)
    K = np.tile(rng.normal(size=d), (n, 1))
    V = rng.normal(size=(n, d))
    O, _ = orc.softmax_attention(q, K, V, orc.default_scale(d))
    np.testing.assert_allclose(O, V.mean(axis=0), rtol=1e-12, atol=1e-13)


def test_zero_query_gives_mean_of_values():
    rng = np.random.default_rng(1)
    K, V = rng.normal(size=(11, 16)), rng.normal(size=(11, 16))
    O, _ = orc.softmax_attention(np.zeros(16), K, V, 0.25)
    np.testing.assert_allclose(O, V.mean(axis=0), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("gap", [60.0, 1000.0])
def test_dominant_logit_selects_its_value_row(gap):
    # A logit `gap` above all others puts weight exp(-gap) (< 1e-26) elsewhere;
    # gap = 1000 also checks that the maximum is subtracted before exp.
    rng = np.random.default_rng(2)
    d, n, p = 8, 20, 13
    K = rng.normal(size=(n, d)) * 0.1
    q = np.zeros(d); q[0] = 1.0
    K[p, 0] = gap / orc.default_scale(d) + 1.0
    V = rng.normal(size=(n, d))
    O, _ = orc.softmax_attention(q, K, V, orc.default_scale(d))
    np.testing.assert_allclose(O, V[p], rtol=1e-15, atol=1e-15)


def test_row_permutation_invariance():
    rng = np.random.default_rng(3)
    q, K, V = rng.normal(size=32), rng.normal(size=(50, 32)), rng.normal(size=(50, 32))
    perm = rng.permutation(50)
    O1, _ = orc.softmax_attention(q, K, V, 0.2)
    O2, _ = orc.softmax_attention(q, K[perm], V[perm], 0.2)
    np.testing.assert_allclose(O1, O2, rtol=1e-13, atol=1e-14)


def test_key_shift_along_null_direction_is_invariant():
    # Adding c to every key with q.c = t shifts every logit by the same t*scale,
    # which softmax cancels.
    rng = np.random.default_rng(4)
    d = 16
    q, K, V = rng.normal(size=d), rng.normal(size=(25, d)), rng.normal(size=(25, d))
    c = rng.normal(size=d) * 3
    O1, _ = orc.softmax_attention(q, K, V, 0.25)
    O2, _ = orc.softmax_attention(q, K + c, V, 0.25)
    np.testing.assert_allclose(O1, O2, rtol=1e-12, atol=1e-13)


# -------------------------------------------------------------------- top-k

def _brute_force_topk(vals, k):
    """Rank by counting who beats whom (no sorting), then keep rank < k."""
    n = len(vals)
    v = [float(x) for x in vals]

    def beats(j, i):
        nj, ni = math.isnan(v[j]), math.isnan(v[i])
        if nj != ni:
            return ni                      # a number beats NaN
        if nj and ni:
            return j < i
        if v[j] != v[i]:                   # -0.0 == +0.0 here
            return v[j] > v[i]
        return j < i

    rank = [sum(beats(j, i) for j in range(n) if j != i) for i in range(n)]
    return sorted(i for i in range(n) if rank[i] < k)


def test_topk_golden_special_values():
    g = _load("topk_special_values.json")
    vals = np.array([_f(x) for x in g["values"]], dtype=np.float32)
    for k, want in g["expected"].items():
        assert orc.select_topk_f32(vals, int(k)).tolist() == want
    for case in g["signed_zero_cases"]:
        vals = np.array(case["values"], dtype=np.float32)
        assert orc.select_topk_f32(vals, case["k"]).tolist() == case["expected"]


@pytest.mark.parametrize("seed", range(30))
def test_topk_matches_brute_force_with_heavy_ties(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 41))
    pool = np.array([-1.0, -0.0, 0.0, 0.5, 2.0, np.inf, -np.inf, np.nan], dtype=np.float32)
    if seed % 3 == 0:
        vals = rng.normal(size=n).astype(np.float32)
    else:
        vals = pool[rng.integers(0, len(pool), size=n)]
    for k in range(1, n + 1):
        assert orc.select_topk_f32(vals, k).tolist() == _brute_force_topk(vals, k)


def test_topk_special_cases():
    n = 100
    const = np.full(n, 0.75, dtype=np.float32)
    assert orc.select_topk_f32(const, 17).tolist() == list(range(17))
    inc = np.arange(n, dtype=np.float32)
    assert orc.select_topk_f32(inc, 30).tolist() == list(range(70, 100))
    dec = inc[::-1].copy()
    assert orc.select_topk_f32(dec, 30).tolist() == list(range(30))
    assert orc.select_topk_f32(np.random.default_rng(0).normal(size=n).astype(np.float32), n).tolist() == list(range(n))


def test_topk_on_logits_equals_topk_on_probabilities():
    rng = np.random.default_rng(7)
    for _ in range(20):
        s = rng.normal(size=500) * 3
        p = np.exp(s - s.max())
        p /= p.sum()
        assert np.unique(p).size == p.size
        for k in (1, 50, 150, 499):
            assert np.array_equal(orc.select_topk(s, k), orc.select_topk(p, k))


def test_topk_rejects_bad_k():
    with pytest.raises(AssertionError):
        orc.select_topk(np.zeros(4), 0)
    with pytest.raises(AssertionError):
        orc.select_topk(np.zeros(4), 5)


# ------------------------------------------------------- sparse head and layer

def test_sparse_with_all_rows_equals_full():
    rng = np.random.default_rng(8)
    n, d = 64, 32
    q, K, V = rng.normal(size=d), rng.normal(size=(n, d)), rng.normal(size=(n, d))
    O_full, _ = orc.softmax_attention(q, K, V, 0.2)
    O_sp, S = orc.sparse_head(q, K, V, np.arange(n), 0.2)
    np.testing.assert_allclose(O_sp, O_full, rtol=1e-13, atol=1e-14)
    # S given in any order is the same set
    O_sp2, _ = orc.sparse_head(q, K, V, rng.permutation(n), 0.2)
    np.testing.assert_allclose(O_sp2, O_full, rtol=1e-13, atol=1e-14)


def test_sparse_single_index_returns_that_row():
    rng = np.random.default_rng(9)
    q, K, V = rng.normal(size=16), rng.normal(size=(40, 16)), rng.normal(size=(40, 16))
    for p in (0, 17, 39):
        O, S = orc.sparse_head(q, K, V, np.array([p]), 0.25)
        assert np.array_equal(O, V[p]) and S.tolist() == [p]


def test_sparse_ignores_rows_outside_set():
    rng = np.random.default_rng(10)
    n, d = 30, 8
    q, K, V = rng.normal(size=d), rng.normal(size=(n, d)), rng.normal(size=(n, d))
    S = np.array([2, 5, 11, 29])
    O1, _ = orc.sparse_head(q, K, V, S, 0.3)
    K2, V2 = K.copy(), V.copy()
    mask = np.ones(n, bool); mask[S] = False
    K2[mask] = 1e3; V2[mask] = -1e3
    O2, _ = orc.sparse_head(q, K2, V2, S, 0.3)
    assert np.array_equal(O1, O2)


def test_gqa_head_to_kv_mapping():
    # KV head g holds constant value rows equal to g+1; query head h must read
    # KV head h // (Hq/Hkv).
    B, Hq, Hkv, n, d = 1, 8, 2, 10, 4
    rng = np.random.default_rng(11)
    Q = rng.normal(size=(B, Hq, d))
    K = rng.normal(size=(Hkv, n, d))
    V = np.stack([np.full((n, d), g + 1.0) for g in range(Hkv)])
    O, S, _ = orc.hybrid_layer_f64(Q, K, V, [0, n], [True] * Hq, [3], None)
    for h in range(Hq):
        np.testing.assert_allclose(O[0, h], np.full(d, h // 4 + 1.0), rtol=1e-14)


def test_recurrence_golden_three_layers():
    g = _load("recurrence_3layer.json")
    N, d, k = g["N"], g["d"], g["k"]
    layers = []
    for l in range(3):
        Q = np.zeros((1, 2, d)); Q[0, :, 0] = math.sqrt(2.0)
        K = np.zeros((2, N, d)); V = np.zeros((2, N, d))
        for h in range(2):
            K[h, :, 0] = g["K_first_coord"][l][h]
            for i in range(N):
                V[h, i] = [i + 1 + 10 * h + 100 * l, (i + 1) ** 2]
        layers.append((Q, K, V))
    outs, sets = orc.decode_step_f64(layers, [0, N], g["retrieval_masks"], [k])
    for l in range(3):
        for h in range(2):
            assert sets[l][(0, h)].tolist() == g["expected_S"][l][h], (l, h)
    for e in g["expected_O_sparse"]:
        np.testing.assert_allclose(outs[e["layer"]][0, e["head"]], e["O"], rtol=1e-14)


def test_layer0_must_be_all_retrieval():
    Q = np.zeros((1, 2, 2)); K = np.zeros((2, 4, 2)); V = np.zeros((2, 4, 2))
    with pytest.raises(AssertionError):
        orc.decode_step_f64([(Q, K, V)], [0, 4], [[True, False]], [2])


def test_sparse_head_carries_layer0_set_through_all_sparse_layers():
    rng = np.random.default_rng(12)
    B, Hq, n, d, L = 1, 3, 40, 8, 5
    masks = [[True] * Hq] + [[h == 0 for h in range(Hq)] for _ in range(L - 1)]
    layers = [(rng.normal(size=(B, Hq, d)), rng.normal(size=(Hq, n, d)), rng.normal(size=(Hq, n, d)))
              for _ in range(L)]
    outs, sets = orc.decode_step_f64(layers, [0, n], masks, [12])
    for h in (1, 2):
        for l in range(1, L):
            assert np.array_equal(sets[l][(0, h)], sets[0][(0, h)])
    assert not np.array_equal(sets[L - 1][(0, 0)], sets[0][(0, 0)])


def test_batch_permutation_invariance_ragged():
    rng = np.random.default_rng(13)
    Hq, Hkv, d = 4, 2, 16
    lens = [23, 40, 17]
    offs = np.concatenate([[0], np.cumsum(lens)])
    T = offs[-1]
    Q = rng.normal(size=(3, Hq, d))
    K = rng.normal(size=(Hkv, T, d)); V = rng.normal(size=(Hkv, T, d))
    ks = [7, 12, 5]
    ret = [True, False, True, False]
    S_in = {(b, h): np.sort(rng.choice(lens[b], ks[b], replace=False)) for b in range(3) for h in range(Hq)}
    O, S, _ = orc.hybrid_layer_f64(Q, K, V, offs, ret, ks, S_in)
    perm = [2, 0, 1]
    lens_p = [lens[p] for p in perm]
    offs_p = np.concatenate([[0], np.cumsum(lens_p)])
    Kp = np.concatenate([K[:, offs[p]:offs[p + 1]] for p in perm], axis=1)
    Vp = np.concatenate([V[:, offs[p]:offs[p + 1]] for p in perm], axis=1)
    S_in_p = {(i, h): S_in[(p, h)] for i, p in enumerate(perm) for h in range(Hq)}
    Op, Sp, _ = orc.hybrid_layer_f64(Q[perm], Kp, Vp, offs_p, ret, [ks[p] for p in perm], S_in_p)
    for i, p in enumerate(perm):
        assert np.array_equal(Op[i], O[p])
        for h in range(Hq):
            assert np.array_equal(Sp[(i, h)], S[(p, h)])


def test_hybrid_layer_bf16_matches_widened_f64():
    rng = np.random.default_rng(14)
    Hq, Hkv, n, d = 4, 2, 33, 8
    qb = rng.integers(0x3000, 0x4000, size=(1, Hq, d)).astype(np.uint16)
    kb = rng.integers(0x3000, 0x4000, size=(Hkv, n, d)).astype(np.uint16)
    vb = rng.integers(0xB000, 0xC000, size=(Hkv, n, d)).astype(np.uint16)
    O1, S1, _ = orc.hybrid_layer_bf16(qb, kb, vb, [0, n], [True] * Hq, [9], None)
    O2, S2, _ = orc.hybrid_layer_f64(orc.bf16_bits_to_f64(qb), orc.bf16_bits_to_f64(kb),
                                     orc.bf16_bits_to_f64(vb), [0, n], [True] * Hq, [9], None)
    assert np.array_equal(O1, O2)


# ---- quantised KV: E4M3 decode and the fp8 layer

def test_fp8_e4m3_known_codes():
    # values fixed by the format's definition (bias 7, 3 mantissa bits, subnormals at
    # exponent 0, S.1111.111 NaN, no infinities)
    known = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x30: 0.5,
             0x38: 1.0, 0x39: 1.125, 0x3C: 1.5, 0x40: 2.0, 0x78: 256.0, 0x7E: 448.0,
             0xB8: -1.0, 0xFE: -448.0, 0xC0: -2.0}
    for c, v in known.items():
        assert orc.fp8_e4m3_to_f64(np.uint8(c)) == v, hex(c)
    assert np.signbit(orc.fp8_e4m3_to_f64(np.uint8(0x80)))
    assert np.isnan(orc.fp8_e4m3_to_f64(np.uint8(0x7F))) and np.isnan(orc.fp8_e4m3_to_f64(np.uint8(0xFF)))


def test_fp8_e4m3_order_symmetry_and_count():
    codes = np.arange(256, dtype=np.uint8)
    v = orc.fp8_e4m3_to_f64(codes)
    pos = v[:0x7F]                                # 0x00 .. 0x7E
    assert np.all(np.diff(pos) > 0), "positive codes increase strictly"
    assert np.array_equal(v[0x80:0xFF], -pos)     # sign-magnitude
    finite = v[np.isfinite(v)]
    assert finite.size == 254 and np.unique(finite).size == 253   # +0 and -0 are equal
    # every value is a multiple of the smallest subnormal and fits bf16 exactly
    assert np.all(np.mod(finite, 2.0 ** -9) == 0)
    f32 = finite.astype(np.float32)
    assert np.array_equal((f32.view(np.uint32) & np.uint32(0xFFFF)), np.zeros(254, np.uint32))


def test_fp8_layer_scales_are_exact_factors():
    # doubling k_scale doubles every logit exactly; doubling v_scale doubles every output
    rng = np.random.default_rng(3)
    B, Hq, Hkv, d, n = 1, 4, 2, 64, 300
    qb = (rng.standard_normal((B, Hq, d)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    kc = rng.integers(0, 256, size=(Hkv, n, d)).astype(np.uint8)
    vc = rng.integers(0, 256, size=(Hkv, n, d)).astype(np.uint8)
    kc[(kc & 0x7F) == 0x7F] = 0x38                # no NaN codes
    vc[(vc & 0x7F) == 0x7F] = 0x38
    args = ([0, n], [True] * Hq, [90], None)
    O1, S1, sc1 = orc.hybrid_layer_fp8(qb, kc, vc, 1.0, 1.0, *args)
    O2, S2, sc2 = orc.hybrid_layer_fp8(qb, kc, vc, 1.0, 2.0, *args)
    _, S3, sc3 = orc.hybrid_layer_fp8(qb, kc, vc, 2.0, 1.0, *args)
    assert np.array_equal(O2, 2.0 * O1)
    for key in sc1:
        assert np.array_equal(sc3[key], 2.0 * sc1[key])
        assert np.array_equal(S1[key], S3[key]) and np.array_equal(S1[key], S2[key])


# ---- HySparse token-block selection

def _blocks_brute(scores, k, block):
    n = len(scores)
    cand = []
    for j in range(n // block):
        vals = [float(x) for x in scores[j * block:(j + 1) * block] if not math.isnan(float(x))]
        best = max(vals) if vals else float("nan")
        cand.append((math.isnan(best), -(best if not math.isnan(best) else 0.0) + 0.0, j))
    kept = sorted(j for (_, _, j) in sorted(cand)[:k // block])
    return np.array([j * block + r for j in kept for r in range(block)], dtype=np.int64)


def test_block_selection_brute_force_with_ties_and_nans():
    rng = np.random.default_rng(11)
    for it in range(60):
        block = int(rng.choice([2, 4, 8]))
        nb = int(rng.integers(2, 12))
        n = nb * block
        k = block * int(rng.integers(1, nb + 1))
        s = rng.choice([-1.0, 0.0, -0.0, 0.5, 2.0, np.nan], size=n)
        assert np.array_equal(orc.select_topk_blocks(s, k, block), _blocks_brute(s, k, block)), it


def test_block_selection_reduces_to_token_selection_and_known_case():
    rng = np.random.default_rng(12)
    s = rng.standard_normal(40)
    assert np.array_equal(orc.select_topk_blocks(s, 7, 1), orc.select_topk(s, 7))
    ramp = np.arange(256, dtype=np.float64)
    assert np.array_equal(orc.select_topk_blocks(ramp, 128, 64), np.arange(128, 256))
    spike = np.zeros(256); spike[5] = 9.0          # one high token lifts its whole block
    assert np.array_equal(orc.select_topk_blocks(spike, 64, 64), np.arange(0, 64))


# ---- HySparse sparse layer: sigmoid-gated block-sparse and window branches

def test_hysparse_single_row_branches_closed_form():
    # |S| = 1 and W = 1: each branch's softmax has one term, so the branch outputs are
    # the selected V row and the window V row; w = sigmoid(+-ln 3) = 3/4 and 1/4.
    B, Hq, Hkv, d = 2, 4, 2, 4
    offs = [0, 5, 12]
    rng = np.random.default_rng(5)
    Q = rng.standard_normal((B, Hq, d))
    K = rng.standard_normal((Hkv, 12, d))
    V = np.zeros((Hkv, 12, d))
    V[0, 3] = [4, 0, -8, 2]          # sequence 0, KV head 0, local row 3
    V[1, 1] = [8, 4, 0, -4]          # sequence 0, KV head 1, local row 1
    V[0, 5 + 6] = [-4, 4, 4, 8]      # sequence 1, KV head 0, local row 6
    V[1, 5 + 0] = [0, 0, 12, 4]      # sequence 1, KV head 1, local row 0
    Kw = rng.standard_normal((Hkv, B, d))
    Vw = np.array([[[0, 8, 4, -2], [4, 0, 0, 0]], [[-8, 0, 4, 4], [0, -4, 0, 8]]], dtype=float)
    S = {(0, 0): [3], (0, 1): [3], (0, 2): [1], (0, 3): [1],
         (1, 0): [6], (1, 1): [6], (1, 2): [0], (1, 3): [0]}
    ln3 = math.log(3.0)
    gate = np.array([[ln3, -ln3, ln3, -ln3], [-ln3, ln3, ln3, -ln3]])
    O = orc.hysparse_sparse_layer(Q, K, V, offs, S, Kw, Vw, gate)
    want = np.array([
        [[3, 2, -5, 1], [1, 6, 1, -1], [4, 3, 1, -2], [-4, 1, 3, 2]],
        [[2, 1, 1, 2], [-2, 3, 3, 6], [0, -1, 9, 5], [0, -3, 3, 7]],
    ], dtype=float)
    np.testing.assert_allclose(O, want, atol=1e-12, rtol=0)


def test_hysparse_branches_agree_when_the_window_is_the_selection():
    # When the window cache holds the sequence's last W rows of the shared cache and S
    # selects exactly those rows, both branches are the same softmax, so the gate
    # cannot change the output; saturated gates pick one branch.
    B, Hq, Hkv, d, N, W = 2, 4, 2, 16, 40, 6
    rng = np.random.default_rng(8)
    Q = rng.standard_normal((B, Hq, d))
    K = rng.standard_normal((Hkv, B * N, d))
    V = rng.standard_normal((Hkv, B * N, d))
    offs = [0, N, 2 * N]
    Kw = np.concatenate([K[:, b * N + N - W:(b + 1) * N] for b in range(B)], axis=1)
    Vw = np.concatenate([V[:, b * N + N - W:(b + 1) * N] for b in range(B)], axis=1)
    S = {(b, h): np.arange(N - W, N) for b in range(B) for h in range(Hq)}
    ref = None
    for gate in (np.zeros((B, Hq)), rng.standard_normal((B, Hq)) * 4):
        O = orc.hysparse_sparse_layer(Q, K, V, offs, S, Kw, Vw, gate)
        if ref is None:
            ref = O
        np.testing.assert_allclose(O, ref, atol=1e-13, rtol=0)
    S2 = {(b, h): rng.choice(N, 9, replace=False) for b in range(B) for h in range(Hq)}
    hi = orc.hysparse_sparse_layer(Q, K, V, offs, S2, Kw, Vw, np.full((B, Hq), 60.0))
    lo = orc.hysparse_sparse_layer(Q, K, V, offs, S2, Kw, Vw, np.full((B, Hq), -60.0))
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            o_s, _ = orc.sparse_head(Q[b, h], K[g, b * N:(b + 1) * N], V[g, b * N:(b + 1) * N],
                                     S2[(b, h)], 1 / math.sqrt(d))
            o_w, _ = orc.softmax_attention(Q[b, h], K[g, b * N + N - W:(b + 1) * N],
                                           V[g, b * N + N - W:(b + 1) * N], 1 / math.sqrt(d))
            np.testing.assert_allclose(hi[b, h], o_s, atol=1e-12, rtol=0)
            np.testing.assert_allclose(lo[b, h], o_w, atol=1e-12, rtol=0)


# ---- Token Sparse Attention: compress -> dense -> scatter

def test_tsa_full_budget_reduces_to_library_attention():
    # k = T keeps every token, so the layer is plain attention of the sequence (with the
    # query head's KV head repeated), which torch's scaled_dot_product_attention computes
    torch = pytest.importorskip("torch")
    B, Hq, Hkv, T, d = 2, 4, 2, 9, 8
    rng = np.random.default_rng(31)
    Q = rng.standard_normal((Hq, B * T, d))
    K = rng.standard_normal((Hkv, B * T, d))
    V = rng.standard_normal((Hkv, B * T, d))
    sc = rng.standard_normal((B, Hq, T))
    for causal in (False, True):
        out, idx = orc.tsa_attention(Q, K, V, sc, T, causal=causal)
        q = torch.tensor(Q).reshape(Hq, B, T, d).permute(1, 0, 2, 3)
        kk = torch.tensor(K).reshape(Hkv, B, T, d).permute(1, 0, 2, 3).repeat_interleave(Hq // Hkv, dim=1)
        vv = torch.tensor(V).reshape(Hkv, B, T, d).permute(1, 0, 2, 3).repeat_interleave(Hq // Hkv, dim=1)
        ref = torch.nn.functional.scaled_dot_product_attention(q, kk, vv, is_causal=causal)
        ref = ref.permute(1, 0, 2, 3).reshape(Hq, B * T, d).numpy()
        np.testing.assert_allclose(out, ref, atol=1e-12, rtol=0)
        assert all(np.array_equal(i, np.arange(T)) for i in idx.values())


def test_tsa_scatter_and_equal_keys_closed_form():
    # equal keys make every softmax uniform: a selected row gets the mean of the V rows it
    # may attend to, placed at its own position; unselected rows stay zero (or NaN when
    # the caller keeps them)
    B, Hq, Hkv, T, d = 1, 2, 1, 6, 3
    Q = np.random.default_rng(2).standard_normal((Hq, T, d))
    K = np.ones((Hkv, T, d))
    V = np.arange(T * d, dtype=float).reshape(1, T, d) * np.array([1.0, -2.0, 0.5])
    sc = np.array([[[0.1, 5.0, -1.0, 5.0, 2.0, 0.0],        # head 0 keeps 1, 3, 4 (the tie 1/3 both in)
                    [9.0, 1.0, 1.0, 1.0, 1.0, 8.0]]])       # head 1 keeps 0, 5 and index 1 (ties -> lower)
    out, idx = orc.tsa_attention(Q, K, V, sc, 3)
    assert idx[(0, 0)].tolist() == [1, 3, 4] and idx[(0, 1)].tolist() == [0, 1, 5]
    for h, I in ((0, [1, 3, 4]), (1, [0, 1, 5])):
        for t in range(T):
            want = V[0, I].mean(axis=0) if t in I else np.zeros(d)
            np.testing.assert_allclose(out[h, t], want, atol=1e-12, rtol=0)
    out_c, _ = orc.tsa_attention(Q, K, V, sc, 3, causal=True)
    for h, I in ((0, [1, 3, 4]), (1, [0, 1, 5])):
        for i, t in enumerate(I):
            np.testing.assert_allclose(out_c[h, t], V[0, I[:i + 1]].mean(axis=0), atol=1e-12, rtol=0)
    kept, _ = orc.tsa_attention(Q, K, V, sc, 3, zero_fill=False)
    assert np.isnan(kept[0, [0, 2, 5]]).all() and not np.isnan(kept[0, [1, 3, 4]]).any()
    # a budget above T is clamped to T
    full, idx2 = orc.tsa_attention(Q, K, V, sc, 50)
    assert all(i.size == T for i in idx2.values())
