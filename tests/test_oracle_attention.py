"""Pins of the attention oracle (and of the column-parallel projection with no
activation) to what the mathematics fixes, independent of the oracle's own
code: closed forms, a hand-computed example, invariants and reductions.

Sources: Vaswani et al., arXiv:1706.03762, section 3.2 (scaled dot-product
attention, multi-head attention, the decoder's causal mask); Ainslie et al.,
arXiv:2305.13245 (grouped key/value heads); "Tensor parallelism" guide,
"Walking through a transformer block" (heads, or GQA groups, sharded across
ranks; the KV cache sharded along heads).  Everything runs on the CPU.
"""
import math

import numpy as np
import pytest

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


def _qkv(seed, Bs=2, Sq=7, Lk=7, nh=4, nkv=4, d=8, scale=1.0):
    r = _rng(seed)
    Q = r.standard_normal((Bs, Sq, nh * d)) * scale
    K = r.standard_normal((Bs, Lk, nkv * d)) * scale
    V = r.standard_normal((Bs, Lk, nkv * d))
    return Q, K, V


def test_attn_first_query_returns_first_value():
    # causal: the first position sees only itself, whatever q and k hold
    Q, K, V = _qkv(1, nh=4, nkv=2)
    c = oracle.attention(Q, K, V, 4, 2, causal=True)
    d = 8
    for h in range(4):
        g = h // 2
        assert np.array_equal(c[:, 0, h * d:(h + 1) * d], V[:, 0, g * d:(g + 1) * d])
    # one valid key, non-causal decode: the same
    c1 = oracle.attention(Q[:, :1], K, V, 4, 2, causal=False, kv_len=[1, 1])
    assert np.array_equal(c1[:, 0, :d], V[:, 0, :d])


def test_attn_constant_values_pass_through():
    # the weights sum to one: equal value rows come out unchanged
    Q, K, V = _qkv(2, Lk=9, Sq=9)
    row = _rng(3).standard_normal(V.shape[2])
    V[:] = row
    for causal in (True, False):
        c = oracle.attention(Q, K, V, 4, 4, causal)
        assert np.allclose(c, np.broadcast_to(row, c.shape), rtol=1e-13, atol=1e-13)


def test_attn_zero_query_gives_mean_of_visible_values():
    # q = 0: every score is 0, the weights are uniform over the visible keys
    Bs, S, d = 3, 6, 4
    Q = np.zeros((Bs, S, d))
    _, K, V = _qkv(4, Bs=Bs, Sq=S, Lk=S, nh=1, nkv=1, d=d)
    c = oracle.attention(Q, K, V, 1, 1, causal=True)
    running = np.cumsum(V, axis=1) / np.arange(1, S + 1)[None, :, None]
    assert np.allclose(c, running, rtol=1e-13, atol=1e-14)
    lens = np.array([6, 2, 4])
    c = oracle.attention(Q[:, :1], K, V, 1, 1, causal=False, kv_len=lens)
    for b in range(Bs):
        assert np.allclose(c[b, 0], V[b, :lens[b]].mean(axis=0), rtol=1e-13, atol=1e-14)


def test_attn_hand_example_fixes_the_scale():
    # d = 4, two keys: q.k0 = 2, q.k1 = 0, so with the 1/sqrt(d) = 1/2 scale
    # the scores are 1 and 0 and the weights e/(1+e), 1/(1+e)
    Q = np.array([[[2.0, 0, 0, 0]]])
    K = np.array([[[1.0, 0, 0, 0], [0, 0, 0, 0]]])
    V = np.array([[[1.0, 0, 0, 0], [0, 1.0, 0, 0]]])
    c = oracle.attention(Q, K, V, 1, 1, causal=False)
    e = math.e
    assert np.allclose(c[0, 0], [e / (1 + e), 1 / (1 + e), 0, 0], rtol=0, atol=1e-15)
    # d = 16 (scale 1/4), q.k0 = 8: scores 2 and 0
    Q = np.zeros((1, 1, 16)); Q[0, 0, 0] = 8.0
    K = np.zeros((1, 2, 16)); K[0, 0, 0] = 1.0
    V = np.zeros((1, 2, 16)); V[0, 0, 3] = 1.0; V[0, 1, 5] = 1.0
    c = oracle.attention(Q, K, V, 1, 1, causal=False)
    w0 = e * e / (1 + e * e)
    assert abs(c[0, 0, 3] - w0) < 1e-15 and abs(c[0, 0, 5] - (1 - w0)) < 1e-15


def test_attn_key_order_does_not_matter_without_mask():
    Q, K, V = _qkv(5, Sq=3, Lk=11)
    c = oracle.attention(Q, K, V, 4, 4, causal=False)
    perm = _rng(6).permutation(11)
    assert np.allclose(oracle.attention(Q, K[:, perm], V[:, perm], 4, 4, causal=False), c, rtol=1e-12, atol=1e-14)
    # moving the values alone does change the result (the check above is not vacuous)
    assert not np.allclose(oracle.attention(Q, K, V[:, perm], 4, 4, causal=False), c, rtol=1e-6)


def test_attn_causal_mask_boundary():
    Q, K, V = _qkv(7, Bs=1, Sq=8, Lk=8)
    c = oracle.attention(Q, K, V, 4, 4, causal=True)
    for p in range(8):
        K2, V2 = K.copy(), V.copy()
        K2[:, p + 1:] += 5.0
        V2[:, p + 1:] -= 3.0
        c2 = oracle.attention(Q, K2, V2, 4, 4, causal=True)
        assert np.array_equal(c2[:, :p + 1], c[:, :p + 1])      # later keys are invisible
        V3 = V.copy()
        V3[:, p] += 1.0
        c3 = oracle.attention(Q, K, V3, 4, 4, causal=True)
        assert not np.allclose(c3[:, p], c[:, p], rtol=1e-9)   # the own position is visible


def test_attn_decode_rows_match_prefill_rows():
    # the queries of a call are the last Sq positions of each sequence
    Q, K, V = _qkv(8, Bs=2, Sq=10, Lk=10, nh=4, nkv=2)
    full = oracle.attention(Q, K, V, 4, 2, causal=True)
    for s in range(10):
        one = oracle.attention(Q[:, s:s + 1], K, V, 4, 2, causal=True, kv_len=[s + 1, s + 1])
        assert np.allclose(one[:, 0], full[:, s], rtol=1e-13, atol=1e-14)
    last3 = oracle.attention(Q[:, 7:], K, V, 4, 2, causal=True)
    assert np.allclose(last3, full[:, 7:], rtol=1e-13, atol=1e-14)
    # ragged lengths: sequence 1 has 6 valid keys, its last query is position 5
    r = oracle.attention(Q[:, 5:6], K, V, 4, 2, causal=True, kv_len=[10, 6])
    assert np.allclose(r[1, 0], full[1, 5], rtol=1e-13, atol=1e-14)


def test_attn_gqa_equals_heads_with_repeated_keys_and_values():
    nh, nkv, d = 8, 2, 4
    Q, K, V = _qkv(9, Sq=5, Lk=5, nh=nh, nkv=nkv, d=d)
    G = nh // nkv
    Kr = np.repeat(K.reshape(2, 5, nkv, d), G, axis=2).reshape(2, 5, nh * d)
    Vr = np.repeat(V.reshape(2, 5, nkv, d), G, axis=2).reshape(2, 5, nh * d)
    for causal in (True, False):
        assert np.allclose(oracle.attention(Q, K, V, nh, nkv, causal),
                           oracle.attention(Q, Kr, Vr, nh, nh, causal), rtol=1e-13, atol=1e-14)


def test_attn_common_key_shift_and_huge_scores():
    # adding one vector u to every key adds q.u/sqrt(d) to all of a query's
    # scores, which the softmax ignores; with u large the scores reach 1e4
    Q, K, V = _qkv(10, Sq=6, Lk=6)
    c = oracle.attention(Q, K, V, 4, 4, causal=True)
    u = _rng(11).standard_normal(K.shape[2]) * 3000.0
    c2 = oracle.attention(Q, K + u, V, 4, 4, causal=True)
    assert np.isfinite(c2).all()
    assert np.allclose(c2, c, rtol=1e-8, atol=1e-8)


def test_attn_peaked_scores_pick_one_value():
    # orthonormal keys, q a large multiple of key j: the weight of j tends to 1
    d = 8
    K = np.eye(d)[None]
    V = _rng(12).standard_normal((1, d, d))
    for j in range(d):
        Q = (200.0 * math.sqrt(d) * np.eye(d)[j])[None, None]
        c = oracle.attention(Q, K, V, 1, 1, causal=False)
        assert np.allclose(c[0, 0], V[0, j], rtol=0, atol=1e-12)


def test_attn_linear_in_values():
    Q, K, V = _qkv(13, Sq=4, Lk=9)
    V2 = _rng(14).standard_normal(V.shape)
    a = oracle.attention(Q, K, V, 4, 4, False, kv_len=[9, 5])
    b = oracle.attention(Q, K, V2, 4, 4, False, kv_len=[9, 5])
    s = oracle.attention(Q, K, V + 2.0 * V2, 4, 4, False, kv_len=[9, 5])
    assert np.allclose(s, a + 2.0 * b, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("T", [2, 4])
def test_attn_head_shards_are_the_unsharded_heads(T):
    # rank i's query heads and its key/value heads (GQA groups stay whole)
    nh, nkv, d = 8, 4, 4
    Q, K, V = _qkv(15, Sq=6, Lk=6, nh=nh, nkv=nkv, d=d)
    full = oracle.attention(Q, K, V, nh, nkv, True)
    qh, kh = nh // T * d, nkv // T * d
    for i in range(T):
        part = oracle.attention(Q[:, :, i * qh:(i + 1) * qh], K[:, :, i * kh:(i + 1) * kh],
                                V[:, :, i * kh:(i + 1) * kh], nh // T, nkv // T, True)
        assert np.array_equal(part, full[:, :, i * qh:(i + 1) * qh])


def test_colpar_linear_integer_exact_and_sharded():
    # small integers: every product and sum is exact in fp64
    r = _rng(16)
    X = r.integers(-4, 5, (5, 12)).astype(float)
    W = r.integers(-3, 4, (12, 16)).astype(float)
    b = r.integers(-9, 10, 16).astype(float)
    want = X.astype(np.int64) @ W.astype(np.int64) + b.astype(np.int64)
    for T in (1, 2, 4):
        got = np.concatenate([oracle.colpar_linear(X, W, b, T, i) for i in range(T)], axis=1)
        assert np.array_equal(got, want)
    assert np.array_equal(oracle.colpar_linear(np.zeros((3, 12)), W, b, 2, 1), np.tile(b[8:], (3, 1)))
    assert np.array_equal(oracle.colpar_linear(X, W, None, 1, 0), X.astype(np.int64) @ W.astype(np.int64))


def test_attn_rejects_bad_arguments():
    Q, K, V = _qkv(17, Sq=4, Lk=4, nh=4, nkv=4)
    with pytest.raises(ValueError):
        oracle.attention(Q, K, V, 4, 3, True)                      # nh not a multiple of nkv
    with pytest.raises(ValueError):
        oracle.attention(Q, K, V, 4, 4, True, kv_len=[4, 5])       # beyond the cache
    with pytest.raises(ValueError):
        oracle.attention(Q, K, V, 4, 4, True, kv_len=[4, 3])       # fewer keys than causal queries
    with pytest.raises(ValueError):
        oracle.attention(Q, K, V, 4, 4, False, kv_len=[4, 0])      # an empty sequence
    with pytest.raises(ValueError):
        oracle.attention(Q, K[:, :, :8], V[:, :, :8], 4, 4, True)  # head widths differ
    with pytest.raises(ValueError):
        oracle.colpar_gated(np.ones((2, 4)), np.ones((4, 4)), np.ones((4, 4)), None, None, 1, 0, oracle.ACT_NONE)
