"""Pins of the oracle's score and mask modifications (non-causal attention,
ALiBi-style distance bias, arbitrary elementwise masks) against what the
mathematics fixes: closed forms, identities that reduce a modification to the
plain causal path, and dense brute force on tiny inputs.

The semantics pinned (CPUAttn "Operator model" and "Parallel lowering"):
non-causal rows see every key of the history; an ALiBi slope m adds
-m |pos - j| to the logit after the softcap; a mask hides keys elementwise on
top of the causal / window rule; a row with nothing visible is NaN with
lse = -inf when allowed."""
import math

import numpy as np
import pytest

import oracle


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32)


def test_noncausal_identical_keys_give_the_mean_of_v():
    """All keys equal: every visible key has the same logit, so each row is
    the plain mean of V over the whole history, whatever its position."""
    L, D = 37, 16
    k = np.tile(rnd((1, 1, D), 1), (1, L, 1))
    v = rnd((1, L, D), 2)
    q = rnd((5, 2, D), 3)
    pos = np.array([0, 3, 17, 30, 36], np.int32)
    out, lse = oracle.attend(q, k, v, pos, [0, 0], 0.25, causal=False)
    want = v[0].astype(np.float64).mean(axis=0)
    assert np.allclose(out, want[None, None, :], rtol=0, atol=1e-12)
    s = 0.25 * (q.astype(np.float64) @ k[0, 0].astype(np.float64))
    assert np.allclose(lse, s + math.log(L), rtol=0, atol=1e-12)


def test_noncausal_row_equals_causal_last_row():
    """Without a mask a non-causal row sees the same keys as a causal row at
    the last position."""
    L, D, hq = 50, 32, 4
    q, k, v = rnd((6, hq, D), 4), rnd((2, L, D), 5), rnd((2, L, D), 6)
    hm = oracle.default_head_map(hq, 2)
    pos = np.array([0, 5, 9, 20, 41, 49], np.int32)
    o_nc, l_nc = oracle.attend(q, k, v, pos, hm, 0.2, causal=False)
    o_c, l_c = oracle.attend(q, k, v, np.full(6, L - 1, np.int32), hm, 0.2)
    assert np.array_equal(o_nc, o_c) and np.array_equal(l_nc, l_c)


def test_mask_identities():
    """An all-ones mask changes nothing; the lower-triangular mask j <= pos on
    a non-causal call is the causal call; a mask on a causal call only
    removes keys the causal rule already allows."""
    L, D, hq = 40, 16, 2
    q, k, v = rnd((7, hq, D), 7), rnd((1, L, D), 8), rnd((1, L, D), 9)
    pos = np.array([0, 1, 7, 16, 25, 38, 39], np.int32)
    hm = [0, 0]
    base = oracle.attend(q, k, v, pos, hm, 0.3)
    ones = oracle.attend(q, k, v, pos, hm, 0.3, mask=np.ones((7, L), bool))
    assert np.array_equal(base[0], ones[0]) and np.array_equal(base[1], ones[1])
    tril = np.arange(L)[None, :] <= pos[:, None]
    nc = oracle.attend(q, k, v, pos, hm, 0.3, causal=False, mask=tril)
    assert np.array_equal(base[0], nc[0]) and np.array_equal(base[1], nc[1])
    # With a window the same holds for the window's own mask.
    W, S = 9, 2
    wmask = tril & ((np.arange(L)[None, :] > pos[:, None] - W) | (np.arange(L)[None, :] < S))
    win = oracle.attend(q, k, v, pos, hm, 0.3, window=W, n_sinks=S)
    ncw = oracle.attend(q, k, v, pos, hm, 0.3, causal=False, mask=wmask)
    assert np.array_equal(win[0], ncw[0]) and np.array_equal(win[1], ncw[1])


def _geo0(r, n):
    """sum_{t=0}^{n} r^t."""
    return (1.0 - r ** (n + 1)) / (1.0 - r)


def _geo1(r, n):
    """sum_{t=0}^{n} t r^t."""
    return r * (1.0 - (n + 1) * r ** n + n * r ** (n + 1)) / (1.0 - r) ** 2


@pytest.mark.parametrize("causal", [True, False])
def test_alibi_on_zero_scores_is_a_geometric_average(causal):
    """q = 0 makes every raw score 0, so the weights are r^|pos - j| with
    r = e^-m; with V[j] = j the output is a ratio of finite geometric sums
    (closed forms), and lse is the log of the denominator."""
    L, D = 60, 8
    slopes = np.array([0.5, 0.125, 1.0 / 64], np.float64)
    q = np.zeros((4, 3, D), np.float32)
    k = rnd((1, L, D), 10)
    v = np.zeros((1, L, D), np.float32)
    v[0, :, 0] = np.arange(L)
    v[0, :, 1] = 1.0
    pos = np.array([0, 13, 40, 59], np.int32)
    out, lse = oracle.attend(q, k, v, pos, [0, 0, 0], 0.125, causal=causal, alibi=slopes)
    for i, p in enumerate(pos):
        for h, m in enumerate(slopes):
            r = math.exp(-m)
            num = p * _geo0(r, p) - _geo1(r, p)
            den = _geo0(r, p)
            if not causal:
                n2 = L - 1 - p
                num += p * (_geo0(r, n2) - 1.0) + _geo1(r, n2)
                den += _geo0(r, n2) - 1.0
            assert abs(out[i, h, 0] - num / den) <= 1e-10 * max(1.0, num / den)
            assert abs(out[i, h, 1] - 1.0) <= 1e-12
            assert abs(lse[i, h] - math.log(den)) <= 1e-12


def test_causal_alibi_equals_one_extra_key_dimension():
    """On a causal row, -m (pos - j) = m j - m pos; the row constant cancels
    in the softmax, and m j is the score of one extra dimension holding j in
    K and m / scale in Q.  So ALiBi equals the plain causal path on D + 1
    dimensions, with lse shifted by m pos (slopes and scale are powers of two,
    so the extra Q entry is exact)."""
    L, D, hq, hkv = 45, 16, 4, 2
    scale = 0.125
    slopes = np.array([2.0 ** -1, 2.0 ** -3, 2.0 ** -5, 2.0 ** -8])
    q, k, v = rnd((5, hq, D), 11), rnd((hkv, L, D), 12), rnd((hkv, L, D), 13)
    hm = oracle.default_head_map(hq, hkv)
    pos = np.array([0, 4, 22, 30, 44], np.int32)
    o_a, l_a = oracle.attend(q, k, v, pos, hm, scale, alibi=slopes)
    q2 = np.concatenate([q, np.broadcast_to((slopes / scale).astype(np.float32)[None, :, None], (5, hq, 1))], 2)
    k2 = np.concatenate([k, np.broadcast_to(np.arange(L, dtype=np.float32)[None, :, None], (hkv, L, 1))], 2)
    v2 = np.concatenate([v, np.zeros((hkv, L, 1), np.float32)], 2)
    o_p, l_p = oracle.attend(q2, k2, v2, pos, hm, scale)
    assert np.allclose(o_a, o_p[..., :D], rtol=1e-12, atol=1e-12)
    assert np.allclose(l_a, l_p - slopes[None, :] * pos[:, None], rtol=0, atol=1e-10)


def test_fully_masked_rows():
    L, D = 20, 8
    q, k, v = rnd((3, 1, D), 14), rnd((1, L, D), 15), rnd((1, L, D), 16)
    pos = np.array([5, 10, 19], np.int32)
    mask = np.ones((3, L), bool)
    mask[1] = False
    mask[2, :19] = False                      # only key 19 left on the last row
    with pytest.raises(ValueError):
        oracle.attend(q, k, v, pos, [0], 0.5, mask=mask)
    out, lse = oracle.attend(q, k, v, pos, [0], 0.5, mask=mask, allow_empty=True)
    assert np.isnan(out[1]).all() and lse[1, 0] == -np.inf
    assert np.allclose(out[2, 0], v[0, 19], rtol=0, atol=1e-12)     # one visible key returns its V row
    ref = oracle.attend(q[[0]], k, v, pos[[0]], [0], 0.5)
    assert np.array_equal(out[0], ref[0][0]) and lse[0, 0] == ref[1][0, 0]


@pytest.mark.parametrize("causal", [True, False])
def test_mods_against_dense_brute_force(causal):
    """Dense matrices on a tiny case: S = scale Q K^T, softcap, ALiBi bias,
    the causal rule and a random mask as -inf, row softmax, P V."""
    L, D, hq, hkv, nq = 23, 8, 4, 2, 6
    scale, cap = 0.4, 3.0
    slopes = np.array([0.3, 0.05, 0.0, 1.1])
    q, k, v = rnd((nq, hq, D), 17), rnd((hkv, L, D), 18), rnd((hkv, L, D), 19)
    hm = oracle.default_head_map(hq, hkv)
    pos = np.array([2, 7, 8, 15, 20, 22], np.int32)
    mask = np.random.default_rng(20).random((nq, L)) < 0.7
    mask[np.arange(nq), pos] = True          # keep each row non-empty
    out, lse = oracle.attend(q, k, v, pos, hm, scale, softcap=cap, causal=causal, alibi=slopes, mask=mask)
    j = np.arange(L)
    for h in range(hq):
        g = hm[h]
        s = scale * (q[:, h].astype(np.float64) @ k[g].astype(np.float64).T)     # [nq][L]
        s = cap * np.tanh(s / cap)
        s = s - slopes[h] * np.abs(pos[:, None] - j[None, :])
        vis = mask & ((j[None, :] <= pos[:, None]) if causal else True)
        s = np.where(vis, s, -np.inf)
        mx = s.max(axis=1, keepdims=True)
        w = np.exp(s - mx)
        o = (w @ v[g].astype(np.float64)) / w.sum(axis=1, keepdims=True)
        assert np.allclose(out[:, h], o, rtol=1e-12, atol=1e-12)
        assert np.allclose(lse[:, h], (mx[:, 0] + np.log(w.sum(axis=1))), rtol=0, atol=1e-12)
