"""Pins of the fp64 oracle to facts fixed by the pages and by mathematics.

None of these compares the oracle with itself: each check is a closed form, an
invariant, a special case, brute force in pure Python, or an independent
library routine (scipy's logsumexp).  The sources are the FA notes (§2.1
standard attention, §3.1 online softmax merge, §3.2 tiled forward) and the S12
course chapter (core-idea recurrence, paged loop, NaN box, exercises 1-2).
"""

import math

import numpy as np
import pytest
from scipy.special import logsumexp

import oracle
from oracle import (M_GUARD, attention_fwd, brute_fwd, kv_outer_tiled,
                    online_rows, split_merge)
from workloads import WORKLOADS

MASKS = [  # (causal, kv_valid)
    (False, None), (True, None), (False, 3), (True, 4), (False, 0)]


def _one_head(x):
    return np.asarray(x)[None, None]


def _fwd1(q, k, v, scale=None, causal=False, kv_valid=None, rows=None):
    kv_len = None if kv_valid is None else [kv_valid]
    o, m, l = attention_fwd(_one_head(q), _one_head(k), _one_head(v), scale,
                            causal, kv_len, rows)
    return o[0, 0], m[0, 0], l[0, 0]


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------- forward --

@pytest.mark.parametrize("causal,kv_valid", MASKS)
@pytest.mark.parametrize("N,d", [(1, 1), (3, 2), (5, 4), (8, 3)])
def test_brute_force_matches_definition(N, d, causal, kv_valid):
    """FA notes §2.1 in pure-Python scalars equals the NumPy definition."""
    rng = np.random.default_rng([100, N, d])
    q, k, v = _rand(rng, N, d), _rand(rng, N, d), _rand(rng, N, d + 1)
    scale = 0.7
    kvv = None if kv_valid is None else min(kv_valid, N)
    ob = np.array(brute_fwd(q.tolist(), k.tolist(), v.tolist(), scale, causal,
                            kvv))
    o, _, _ = _fwd1(q, k, v, scale, causal, kvv)
    assert np.max(np.abs(o - ob)) <= 1e-12


@pytest.mark.parametrize("causal,kv_valid", MASKS)
def test_identity_values_expose_P(causal, kv_valid):
    """With V = I the output is P itself: every visible row of P sums to 1,
    entries are in [0, 1], masked entries are exactly 0, and P is a softmax:
    log P_ij = s_ij - logsumexp_j(s_i.) on visible entries."""
    rng = np.random.default_rng(7)
    N, d = 9, 5
    q, k = _rand(rng, N, d), _rand(rng, N, d)
    P, m, l = _fwd1(q, k, np.eye(N), 0.9, causal, kv_valid)
    vis = oracle.visible_mask(np.arange(N), N, causal,
                              N if kv_valid is None else kv_valid)
    assert np.all(P[~vis] == 0.0)
    rows = vis.any(axis=1)
    assert np.allclose(P[rows].sum(axis=1), 1.0, atol=1e-12, rtol=0)
    assert np.all((P >= 0) & (P <= 1))
    s = 0.9 * q @ k.T
    for i in np.nonzero(rows)[0]:
        lse = logsumexp(s[i, vis[i]])
        assert np.allclose(np.log(P[i, vis[i]]), s[i, vis[i]] - lse,
                           atol=1e-12, rtol=0)
        # saved statistics: m is the max of the scaled visible scores and
        # m + ln l is the row's log-sum-exp
        assert m[i] == pytest.approx(s[i, vis[i]].max(), abs=1e-12)
        assert m[i] + math.log(l[i]) == pytest.approx(lse, abs=1e-12)
    if not rows.all():
        assert np.all(np.isneginf(m[~rows])) and np.all(l[~rows] == 0)


@pytest.mark.parametrize("causal,kv_valid", MASKS[:4])
def test_constant_values_give_constant_output(causal, kv_valid):
    rng = np.random.default_rng(8)
    N, d = 33, 8
    q, k = 3 * _rand(rng, N, d), 3 * _rand(rng, N, d)
    c = _rand(rng, d)
    o, _, _ = _fwd1(q, k, np.tile(c, (N, 1)), None, causal, kv_valid)
    assert np.max(np.abs(o - c)) <= 1e-12


@pytest.mark.parametrize("causal,kv_valid", MASKS[:4])
def test_zero_queries_average_visible_values(causal, kv_valid):
    """Q = 0 makes all visible scores equal, so O_i is the mean of the visible
    V_j: the prefix mean (1/(i+1)) sum_{j<=i} V_j under the causal mask."""
    rng = np.random.default_rng(9)
    N, d = 17, 6
    v = _rand(rng, N, d)
    o, _, _ = _fwd1(np.zeros((N, d)), _rand(rng, N, d), v, None, causal,
                    kv_valid)
    L = N if kv_valid is None else kv_valid
    for i in range(N):
        hi = min(L, i + 1) if causal else L
        assert np.allclose(o[i], v[:hi].mean(axis=0), atol=1e-12, rtol=0)


def test_special_cases_single_key_and_first_causal_row():
    rng = np.random.default_rng(10)
    q, k, v = _rand(rng, 1, 4), _rand(rng, 1, 4), _rand(rng, 1, 4)
    o, m, l = _fwd1(q, k, v)
    assert np.allclose(o, v, atol=1e-15) and l[0] == 1.0
    q, k, v = _rand(rng, 6, 4), _rand(rng, 6, 4), _rand(rng, 6, 4)
    o, _, _ = _fwd1(q, k, v, causal=True)
    assert np.allclose(o[0], v[0], atol=1e-15)


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(11)
    N, d = 12, 4
    q, k, v = _rand(rng, N, d) * 0.1, _rand(rng, N, d) * 0.1, _rand(rng, N, d)
    q[:, 0] = 1.0
    k[5, 0] = 400.0           # score of key 5 exceeds the rest by ~200
    o, _, _ = _fwd1(q, k, v, scale=1.0)
    assert np.max(np.abs(o - v[5])) <= 1e-12


def test_invariances():
    rng = np.random.default_rng(12)
    N, d = 20, 7
    q, k, v = _rand(rng, N, d), _rand(rng, N, d), _rand(rng, N, d)
    o, m, l = _fwd1(q, k, v)
    # K -> K + 1 u^T adds q_i.u to every score of row i: O and l unchanged,
    # m shifts by scale * q_i.u
    u = _rand(rng, d)
    o2, m2, l2 = _fwd1(q, k + u, v)
    assert np.max(np.abs(o2 - o)) <= 1e-12
    assert np.allclose(l2, l, rtol=1e-12, atol=0)
    assert np.allclose(m2 - m, (q @ u) / math.sqrt(d), atol=1e-12, rtol=0)
    # permuting keys together with values leaves O unchanged
    p = rng.permutation(N)
    o3, _, _ = _fwd1(q, k[p], v[p])
    assert np.max(np.abs(o3 - o)) <= 1e-12
    # permuting queries permutes the output rows
    o4, _, _ = _fwd1(q[p], k, v)
    assert np.max(np.abs(o4 - o[p])) <= 1e-12
    # the scale multiplies the scores: scale s on Q equals s folded into Q
    o5, _, _ = _fwd1(q * 0.3, k, v, scale=1.0)
    o6, _, _ = _fwd1(q, k, v, scale=0.3)
    assert np.max(np.abs(o5 - o6)) <= 1e-12


def test_rows_argument_and_chunking_are_pointwise():
    rng = np.random.default_rng(13)
    N, d = 50, 4
    q, k, v = _rand(rng, N, d), _rand(rng, N, d), _rand(rng, N, d)
    full, m, l = _fwd1(q, k, v, causal=True)
    rows = np.array([0, 7, 31, 49])
    part, mp, lp = _fwd1(q, k, v, causal=True, rows=rows)
    assert np.array_equal(part, full[rows])
    assert np.array_equal(mp, m[rows]) and np.array_equal(lp, l[rows])
    o_c, _, _ = attention_fwd(_one_head(q), _one_head(k), _one_head(v),
                              causal=True, row_chunk=7)
    assert np.max(np.abs(o_c[0, 0] - full)) <= 1e-14


def test_large_scores_do_not_overflow():
    rng = np.random.default_rng(14)
    N, d = 64, 16
    q, k, v = 30 * _rand(rng, N, d), 30 * _rand(rng, N, d), _rand(rng, N, d)
    P, m, l = _fwd1(q, k, np.eye(N))
    assert np.all(np.isfinite(P)) and np.allclose(P.sum(1), 1.0, atol=1e-12)
    assert np.all(l >= 1.0)     # the max term contributes exp(0) = 1


# ---------------------------------------------------- the method's loops --

def _tiny_f32():
    w = WORKLOADS["tiny_f32"]
    q, k, v = w.qkv()
    return q.exact[0, 0], k.exact[0, 0], v.exact[0, 0]


@pytest.mark.parametrize("tile", [1, 16, 64, 256])
@pytest.mark.parametrize("causal,kv_valid", [(False, None), (True, None),
                                             (False, 200), (True, 130)])
def test_online_recurrence_equals_definition(tile, causal, kv_valid):
    """S12 core-idea recurrence at tile sizes 1/16/64/N equals the plain
    softmax to rounding (S12 states ~1e-15; tolerance 1e-13)."""
    q, k, v = _tiny_f32()
    o_ref, m_ref, l_ref = _fwd1(q, k, v, None, causal, kv_valid)
    m, l, o = online_rows(q, k, v, tile, None, causal, kv_valid)
    assert np.max(np.abs(o / l[:, None] - o_ref)) <= 1e-13
    assert np.max(np.abs(m - m_ref)) <= 1e-13
    assert np.max(np.abs(l / l_ref - 1)) <= 1e-13


@pytest.mark.parametrize("br,bc", [(1, 1), (16, 16), (64, 64), (1, 16),
                                   (64, 16), (256, 256)])
@pytest.mark.parametrize("causal,kv_valid", [(False, None), (True, None),
                                             (True, 100)])
def test_kv_outer_tiled_equals_definition(br, bc, causal, kv_valid):
    """FA notes §3.2 KV-outer tiled forward, normalised every step."""
    q, k, v = _tiny_f32()
    o_ref, m_ref, l_ref = _fwd1(q, k, v, None, causal, kv_valid)
    o, m, l = kv_outer_tiled(q, k, v, br, bc, None, causal, kv_valid)
    assert np.max(np.abs(o - o_ref)) <= 1e-13
    assert np.max(np.abs(m - m_ref)) <= 1e-13
    assert np.max(np.abs(l / l_ref - 1)) <= 1e-13


def test_nan_guard_reproduced_and_fixed():
    """S12's NaN box / exercise 2: a fully masked tile gives exp(-inf - -inf)
    = NaN when the running max starts at -inf; a finite negative start
    (masked scores kept at -inf) gives the right answer."""
    q, k, v = _tiny_f32()
    with np.errstate(invalid="ignore"):
        o_bad, _, _ = kv_outer_tiled(q, k, v, 16, 16, causal=True,
                                     guard=False)
        m_bad, l_bad, o2_bad = online_rows(q, k, v, 16, kv_valid=0,
                                           guard=False)
    assert np.isnan(o_bad).any()
    assert np.isnan(o2_bad).all()
    o_ref, _, _ = _fwd1(q, k, v, causal=True)
    o_ok, _, _ = kv_outer_tiled(q, k, v, 16, 16, causal=True, guard=True)
    assert np.max(np.abs(o_ok - o_ref)) <= 1e-13
    m, l, o = online_rows(q, k, v, 16, kv_valid=0, guard=True)
    assert np.all(l == 0) and np.all(o == 0) and np.all(m == M_GUARD)


@pytest.mark.parametrize("splits", [4, 8])
@pytest.mark.parametrize("kv_valid", [None, 100, 30])
def test_split_merge_equals_single_pass(splits, kv_valid):
    """S12 exercise 1: keys split over workers, (m, l, o) triples merged with
    the FA notes §3.1 rule, equals one pass.  kv_valid=30 leaves workers with
    no visible key at all."""
    q, k, v = _tiny_f32()
    o_ref, _, _ = _fwd1(q, k, v, None, False, kv_valid)
    o = split_merge(q, k, v, splits, tile=16, kv_valid=kv_valid)
    assert np.max(np.abs(o - o_ref)) <= 1e-13


def test_merge_rule_two_blocks_closed_form():
    """FA notes §3.1: for x = [x1, x2], m(x) = max(m1, m2) and
    l(x) = e^{m1-m} l1 + e^{m2-m} l2 equals sum exp(x - m(x))."""
    rng = np.random.default_rng(15)
    x1, x2 = 5 * rng.standard_normal(9), 5 * rng.standard_normal(4) + 3
    m1, m2 = x1.max(), x2.max()
    l1, l2 = np.exp(x1 - m1).sum(), np.exp(x2 - m2).sum()
    m, l, _ = oracle.merge_triples(np.array([[m1], [m2]]),
                                   np.array([[l1], [l2]]),
                                   np.zeros((2, 1, 1)))
    x = np.concatenate([x1, x2])
    assert m[0] == x.max()
    assert l[0] == pytest.approx(np.exp(x - x.max()).sum(), rel=1e-14)
