"""Pins for the oracle's prefill form of the hybrid-head layer (the extension the
LycheeDecode summary page's future-work paragraph names; the readings are stated in
prefill_hybrid_layer): a hand-derived golden, the decode oracle on each prompt prefix,
closed forms of the column sums, and invariants."""
import json
import os

import numpy as np

from oracle import lychee_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "prefill_three_tokens.json")


def _rand(seed, Hq, Hkv, B, T, d):
    rng = np.random.default_rng(seed)
    return (rng.normal(size=(Hq, B * T, d)), rng.normal(size=(Hkv, B * T, d)), rng.normal(size=(Hkv, B * T, d)))


def test_golden_three_tokens():
    g = json.load(open(GOLDEN))
    Q = np.array(g["Q"])[:, :, None]
    K = np.array(g["K"])[None, :, None]
    V = np.array(g["V"])[None, :, None]
    O, S, imp = orc.prefill_hybrid_layer(Q, K, V, 1, g["retrieval"], g["k"], {(0, 1): np.array(g["S_in_head1"])})
    assert np.allclose(O[:, :, 0], np.array(g["expected_O"]), rtol=0, atol=1e-12)
    assert np.allclose(imp[(0, 0)], g["expected_importance_head0"], rtol=0, atol=1e-12)
    for h in range(2):
        assert np.array_equal(S[(0, h)], g["expected_S"][h])
    assert (0, 1) not in imp


def test_every_prompt_row_is_the_decode_layer_on_its_prefix():
    # GQA 2:1, two sequences: row t of head h equals the (pinned) decode heads over the
    # rows 0..t of its own sequence and KV head
    Hq, Hkv, B, T, d, k = 4, 2, 2, 9, 8, 4
    Q, K, V = _rand(1, Hq, Hkv, B, T, d)
    ret = [True, False, False, True]
    S_in = {(b, h): np.sort(np.random.default_rng(10 + 4 * b + h).choice(T, k, replace=False))
            for b in range(B) for h in range(Hq)}
    O, S, _ = orc.prefill_hybrid_layer(Q, K, V, B, ret, k, S_in)
    sc = orc.default_scale(d)
    for b in range(B):
        for h in range(Hq):
            g = h // 2
            for t in range(T):
                r = b * T + t
                Kp, Vp = K[g, b * T:r + 1], V[g, b * T:r + 1]
                if ret[h]:
                    want, _, _ = orc.retrieval_head(Q[h, r], Kp, Vp, 1, sc)
                else:
                    vis = S_in[(b, h)][S_in[(b, h)] <= t]
                    want = orc.sparse_head(Q[h, r], Kp, Vp, vis, sc)[0] if vis.size else np.zeros(d)
                assert np.allclose(O[h, r], want, rtol=1e-12, atol=1e-12), (b, h, t)
            if not ret[h]:
                assert np.array_equal(S[(b, h)], S_in[(b, h)])


def test_equal_logits_give_the_harmonic_tail_and_the_first_tokens():
    # q = 0: every visible logit is 0, A[t, j] = 1 / (t + 1), so the column sum of token
    # j is H_T - H_j (harmonic numbers), strictly decreasing: S = {0 .. k-1}
    T, d, k = 17, 4, 6
    Q = np.zeros((1, T, d))
    _, K, V = _rand(2, 1, 1, 1, T, d)
    O, S, imp = orc.prefill_hybrid_layer(Q, K, V, 1, [True], k)
    H = np.concatenate([[0.0], np.cumsum(1.0 / np.arange(1, T + 1))])
    assert np.allclose(imp[(0, 0)], H[T] - H[:T], rtol=0, atol=1e-12)
    assert np.array_equal(S[(0, 0)], np.arange(k))
    # and O is the running mean of V
    assert np.allclose(O[0], np.cumsum(V[0], axis=0) / np.arange(1, T + 1)[:, None], atol=1e-12)


def test_column_sums_add_up_to_the_prompt_length():
    Hq, T, d = 3, 23, 16
    Q, K, V = _rand(3, Hq, 1, 1, T, d)
    _, _, imp = orc.prefill_hybrid_layer(Q * 3, K, V, 1, [True] * Hq, 5)
    for h in range(Hq):
        assert abs(imp[(0, h)].sum() - T) < 1e-10
        assert np.all(imp[(0, h)] >= 0)


def test_a_dominant_token_takes_every_row_and_ties_go_to_lower_indices():
    # every query is aligned with key 0 and its logit exceeds the others by ~1000, so
    # A[t, 0] = 1 (exp(-1000) is 0 in fp64): the column sums are [T, 0, 0, ...], and the
    # other k - 1 places go to the lowest indices among the tied zeros
    T, d, k = 12, 4, 5
    Q = np.zeros((1, T, d)); Q[0, :, 0] = 50.0
    K = np.zeros((1, T, d)); K[0, 0, 0] = 40.0
    K[0, 1:, 1] = np.linspace(-1, 1, T - 1)
    V = np.arange(T * d, dtype=np.float64).reshape(1, T, d)
    O, S, imp = orc.prefill_hybrid_layer(Q, K, V, 1, [True], k)
    assert imp[(0, 0)][0] == T and np.all(imp[(0, 0)][1:] == 0.0)
    assert np.array_equal(S[(0, 0)], np.arange(k))
    assert np.allclose(O[0], np.repeat(V[0, :1], T, axis=0))


def test_causality_later_rows_do_not_change_earlier_outputs():
    Hq, T, d, t = 2, 15, 8, 6
    Q, K, V = _rand(4, Hq, 1, 1, T, d)
    S_in = {(0, 1): np.array([2, 5, 9, 12])}
    O1, _, _ = orc.prefill_hybrid_layer(Q, K, V, 1, [True, False], 4, S_in)
    K2, V2 = K.copy(), V.copy()
    K2[:, t + 1:] += 3.0
    V2[:, t + 1:] -= 7.0
    O2, _, _ = orc.prefill_hybrid_layer(Q, K2, V2, 1, [True, False], 4, S_in)
    assert np.array_equal(O1[:, :t + 1], O2[:, :t + 1])
    assert not np.allclose(O1[:, t + 1:], O2[:, t + 1:])


def test_full_set_sparse_head_equals_the_retrieval_head():
    T, d = 13, 8
    Q, K, V = _rand(5, 2, 1, 1, T, d)
    Q[1] = Q[0]
    O, _, _ = orc.prefill_hybrid_layer(Q, K, V, 1, [True, False], T, {(0, 1): np.arange(T)})
    assert np.allclose(O[0], O[1], rtol=1e-13, atol=1e-13)


def test_one_prompt_token_is_the_decode_layer():
    Hq, Hkv, B, d = 4, 2, 3, 8
    Q, K, V = _rand(6, Hq, Hkv, B, 1, d)
    O, S, imp = orc.prefill_hybrid_layer(Q, K, V, B, [True] * Hq, 1)
    Od, Sd, _ = orc.hybrid_layer_f64(np.transpose(Q, (1, 0, 2)), K, V, list(range(B + 1)), [True] * Hq, [1] * B, None)
    assert np.allclose(np.transpose(O, (1, 0, 2)), Od, atol=1e-13)
    for b in range(B):
        for h in range(Hq):
            assert np.array_equal(S[(b, h)], Sd[(b, h)]) and imp[(b, h)][0] == 1.0
