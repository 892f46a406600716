"""Pins of the packed variable-length oracle (oracle/varlen.py).

Each pin reaches the expected value by another route than the varlen code:
pure-Python brute force on each sequence, the (separately pinned) dense
definitions on each sequence's slice, permutation of the packing, sequence
isolation, and central finite differences for the backward."""

import numpy as np
import pytest

from oracle import (attention_bwd, attention_bwd_varlen, attention_fwd,
                    attention_fwd_varlen, brute_fwd, varlen_visible)


def _packed(lens, H, d, rng):
    total = int(sum(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    q, k, v, do = (rng.standard_normal((H, total, d)) for _ in range(4))
    return cu, q, k, v, do


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_matches_brute_force_per_sequence(causal):
    rng = np.random.default_rng([31, int(causal)])
    lens = [3, 0, 5, 1, 4]
    cu, q, k, v, _ = _packed(lens, 1, 4, rng)
    o, _, _ = attention_fwd_varlen(q, k, v, cu, 0.7, causal)
    for b in range(len(lens)):
        s, e = cu[b], cu[b + 1]
        if s == e:
            continue
        ref = brute_fwd(q[0, s:e].tolist(), k[0, s:e].tolist(),
                        v[0, s:e].tolist(), 0.7, causal)
        assert np.max(np.abs(o[0, s:e] - np.array(ref))) <= 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_equals_dense_on_each_slice(causal):
    rng = np.random.default_rng([32, int(causal)])
    lens = [17, 1, 40, 0, 9]
    cu, q, k, v, _ = _packed(lens, 2, 8, rng)
    o, m, l = attention_fwd_varlen(q, k, v, cu, None, causal)
    for b in range(len(lens)):
        s, e = cu[b], cu[b + 1]
        if s == e:
            continue
        od, md, ld = attention_fwd(q[None, :, s:e], k[None, :, s:e],
                                   v[None, :, s:e], None, causal)
        assert np.max(np.abs(o[:, s:e] - od[0])) <= 1e-13
        assert np.max(np.abs(m[:, s:e] - md[0])) <= 1e-13
        assert np.max(np.abs(l[:, s:e] - ld[0])) <= 1e-12 * np.max(ld)


def test_varlen_reordering_sequences_permutes_rows():
    rng = np.random.default_rng(33)
    lens = [6, 11, 2, 7]
    cu, q, k, v, _ = _packed(lens, 2, 5, rng)
    o, _, _ = attention_fwd_varlen(q, k, v, cu, None, True)
    order = [2, 0, 3, 1]
    idx = np.concatenate([np.arange(cu[b], cu[b + 1]) for b in order])
    lens2 = [lens[b] for b in order]
    cu2 = np.concatenate([[0], np.cumsum(lens2)])
    o2, _, _ = attention_fwd_varlen(q[:, idx], k[:, idx], v[:, idx], cu2,
                                    None, True)
    # the products sum over the packed key axis in another order: equal up to
    # rounding
    assert np.max(np.abs(o2 - o[:, idx])) <= 1e-13


def test_varlen_sequences_are_isolated():
    rng = np.random.default_rng(34)
    lens = [5, 8]
    cu, q, k, v, do = _packed(lens, 1, 4, rng)
    o, _, _ = attention_fwd_varlen(q, k, v, cu, None, False)
    g = attention_bwd_varlen(q, k, v, do, cu, None, False)
    k2, v2 = k.copy(), v.copy()
    k2[:, :5] += 3.0
    v2[:, :5] -= 2.0
    o2, _, _ = attention_fwd_varlen(q, k2, v2, cu, None, False)
    g2 = attention_bwd_varlen(q, k2, v2, do, cu, None, False)
    assert np.array_equal(o2[:, 5:], o[:, 5:])
    for a, b in zip(g, g2):
        assert np.array_equal(a[:, 5:], b[:, 5:])


def test_varlen_visibility_rule():
    vis = varlen_visible([0, 2, 2, 5], np.arange(5), 5, True)
    want = np.array([[1, 0, 0, 0, 0],
                     [1, 1, 0, 0, 0],
                     [0, 0, 1, 0, 0],
                     [0, 0, 1, 1, 0],
                     [0, 0, 1, 1, 1]], dtype=bool)
    assert np.array_equal(vis, want)
    with pytest.raises(ValueError):
        varlen_visible([1, 5], np.arange(4), 5, False)


def _loss(q, k, v, do, cu, scale, causal):
    o, _, _ = attention_fwd_varlen(q, k, v, cu, scale, causal)
    return float((o * do).sum())


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_backward_matches_finite_differences(causal):
    rng = np.random.default_rng([35, int(causal)])
    lens = [2, 3, 0, 2]
    cu, q, k, v, do = _packed(lens, 1, 3, rng)
    scale = 0.9
    dq, dk, dv, _ = attention_bwd_varlen(q, k, v, do, cu, scale, causal)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            args = {"q": q, "k": k, "v": v}
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args[name] = xp
            lp = _loss(args["q"], args["k"], args["v"], do, cu, scale, causal)
            args[name] = xm
            lm = _loss(args["q"], args["k"], args["v"], do, cu, scale, causal)
            num[idx] = (lp - lm) / (2 * h)
        err = np.max(np.abs(num - g)) / max(1e-12, np.max(np.abs(g)))
        assert err <= 1e-6, (name, err)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_backward_equals_dense_on_each_slice(causal):
    rng = np.random.default_rng([36, int(causal)])
    lens = [13, 0, 30, 1]
    cu, q, k, v, do = _packed(lens, 2, 6, rng)
    dq, dk, dv, D = attention_bwd_varlen(q, k, v, do, cu, None, causal)
    for b in range(len(lens)):
        s, e = cu[b], cu[b + 1]
        if s == e:
            continue
        ref = attention_bwd(q[None, :, s:e], k[None, :, s:e], v[None, :, s:e],
                            do[None, :, s:e], None, causal)
        for got, want in zip((dq, dk, dv, D), ref):
            assert np.max(np.abs(got[:, s:e] - want[0])) <= 1e-12
