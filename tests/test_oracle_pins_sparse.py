"""Pins of the block-sparse oracle (oracle/sparse.py), each against another
route: the dense definitions (all-ones mask, block-triangular mask with the
causal rule), the varlen oracle (block-diagonal mask = equal-length packed
sequences), pure-Python brute force over each row's visible keys, and
central finite differences for the backward."""

import math

import numpy as np
import pytest

from oracle import (attention_bwd, attention_bwd_block_sparse,
                    attention_bwd_varlen, attention_fwd,
                    attention_fwd_block_sparse, attention_fwd_varlen,
                    brute_fwd)


def _inputs(shape, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal(shape) for _ in range(4)]


def test_all_ones_mask_is_dense_attention():
    q, k, v, _ = _inputs((2, 2, 37, 8), 51)
    mask = np.ones((2, 5, 5), np.uint8)
    for causal in (False, True):
        o, m, l = attention_fwd_block_sparse(q, k, v, mask, 8, None, causal)
        od, md, ld = attention_fwd(q, k, v, None, causal)
        assert np.max(np.abs(o - od)) <= 1e-13
        assert np.max(np.abs(m - md)) <= 1e-13


def test_lower_block_triangle_with_causal_is_causal_attention():
    q, k, v, _ = _inputs((1, 1, 40, 8), 52)
    nb = 5
    mask = np.tril(np.ones((1, nb, nb), np.uint8))
    o, _, _ = attention_fwd_block_sparse(q, k, v, mask, 8, None, True)
    od, _, _ = attention_fwd(q, k, v, None, True)
    assert np.max(np.abs(o - od)) <= 1e-13


def test_block_diagonal_mask_is_varlen_attention():
    q, k, v, do = _inputs((1, 2, 48, 8), 53)
    mask = np.stack([np.eye(4, dtype=np.uint8)] * 2)
    cu = [0, 12, 24, 36, 48]
    o, _, _ = attention_fwd_block_sparse(q, k, v, mask, 12, None, False)
    ov, _, _ = attention_fwd_varlen(q[0], k[0], v[0], cu, None, False)
    assert np.max(np.abs(o[0] - ov)) <= 1e-13
    g = attention_bwd_block_sparse(q, k, v, do, mask, 12, None, True)
    gv = attention_bwd_varlen(q[0], k[0], v[0], do[0], cu, None, True)
    for a, b in zip(g, gv):
        assert np.max(np.abs(a[0] - b)) <= 1e-12


def test_matches_brute_force_on_each_rows_visible_keys():
    rng = np.random.default_rng(54)
    q, k, v, _ = _inputs((1, 1, 10, 3), 55)
    mask = (rng.random((1, 4, 4)) < 0.5).astype(np.uint8)
    mask[0, 0, 0] = 1
    mask[0, 2, :] = 0                          # rows 6..8 see nothing
    for causal in (False, True):
        o, m, l = attention_fwd_block_sparse(q, k, v, mask, 3, 0.7, causal)
        for i in range(10):
            keys = [j for j in range(10) if mask[0, i // 3, j // 3]
                    and (not causal or j <= i)]
            if not keys:
                assert np.all(o[0, 0, i] == 0) and l[0, 0, i] == 0
                assert m[0, 0, i] == -math.inf
                continue
            ref = brute_fwd([q[0, 0, i].tolist()],
                            [k[0, 0, j].tolist() for j in keys],
                            [v[0, 0, j].tolist() for j in keys], 0.7)
            assert np.max(np.abs(o[0, 0, i] - np.array(ref[0]))) <= 1e-13


def _loss(q, k, v, do, mask, block, scale, causal):
    o, _, _ = attention_fwd_block_sparse(q, k, v, mask, block, scale, causal)
    return float((o * do).sum())


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_finite_differences(causal):
    q, k, v, do = _inputs((1, 1, 7, 3), [56, int(causal)])
    mask = np.array([[[1, 0, 1, 0], [0, 1, 1, 0], [0, 0, 0, 0],
                      [1, 1, 0, 1]]], np.uint8)
    scale, block = 0.8, 2
    dq, dk, dv, _ = attention_bwd_block_sparse(q, k, v, do, mask, block,
                                               scale, causal)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            args = {"q": q, "k": k, "v": v}
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args[name] = xp
            lp = _loss(args["q"], args["k"], args["v"], do, mask, block,
                       scale, causal)
            args[name] = xm
            lm = _loss(args["q"], args["k"], args["v"], do, mask, block,
                       scale, causal)
            num[idx] = (lp - lm) / (2 * h)
        err = np.max(np.abs(num - g)) / max(1e-12, np.max(np.abs(g)))
        assert err <= 1e-6, (name, err)


def test_backward_all_ones_is_dense():
    q, k, v, do = _inputs((2, 1, 30, 4), 57)
    mask = np.ones((1, 4, 4), np.uint8)
    g = attention_bwd_block_sparse(q, k, v, do, mask, 8, None, True)
    gd = attention_bwd(q, k, v, do, None, True)
    for a, b in zip(g, gd):
        assert np.max(np.abs(a - b)) <= 1e-12
