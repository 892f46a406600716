"""Pins of the backward oracles' stored-output option (o=...).

The pages keep the output O and the statistics (m, l) in HBM for the
backward pass (FA notes §3.3); a backward that reads O forms the row term
D = rowsum(dO * O) from it.  With the exact O the option must change
nothing.  With one visible key per row the softmax is one-hot, so the exact
dS = P (dP - D) is 0; a stored O = O + delta leaves dS = -(dO . delta) on
that key, i.e. dQ_i = -scale (dO_i . delta_i) K_key(i), dK_j = -scale sum
over the rows i whose key is j of (dO_i . delta_i) Q_i, and dV unchanged.
"""

import numpy as np

from oracle import (attention_bwd, attention_bwd_block_sparse,
                    attention_bwd_dropout, attention_bwd_varlen,
                    attention_fwd, attention_fwd_dropout,
                    attention_fwd_varlen)


def _close(a, b, tol=1e-12):
    for x, y in zip(a, b):
        assert np.max(np.abs(np.asarray(x) - np.asarray(y))) <= tol


def _inputs(shape, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal(shape) for _ in range(4)]


def test_dense_exact_output_changes_nothing():
    q, k, v, do = _inputs((2, 2, 37, 16), 1)
    for causal, kv in [(False, None), (True, None), (False, [20, 37])]:
        o, _, _ = attention_fwd(q, k, v, None, causal, kv)
        _close(attention_bwd(q, k, v, do, None, causal, kv),
               attention_bwd(q, k, v, do, None, causal, kv, o=o))


def test_dense_one_hot_rows_give_the_closed_form():
    q, k, v, do = _inputs((1, 2, 9, 8), 2)
    sc = 1 / np.sqrt(8)
    o, _, _ = attention_fwd(q, k, v, None, False, [1])
    delta = np.random.default_rng(3).standard_normal(o.shape) * 1e-2
    ref = attention_bwd(q, k, v, do, None, False, [1])
    dq, dk, dv, _ = attention_bwd(q, k, v, do, None, False, [1], o=o + delta)
    r = -np.sum(do * delta, axis=-1)                    # dS on key 0
    assert np.max(np.abs(ref[0])) <= 1e-12              # exact dQ is 0
    assert np.max(np.abs(dq - sc * r[..., None] * k[:, :, :1])) <= 1e-12
    dk0 = sc * np.einsum("bhi,bhid->bhd", r, q)
    assert np.max(np.abs(dk[:, :, 0] - dk0)) <= 1e-12
    assert np.all(dk[:, :, 1:] == 0)
    assert np.max(np.abs(dv - ref[2])) <= 1e-12


def test_dropout_option_matches_closed_form_and_exact_case():
    q, k, v, do = _inputs((1, 2, 9, 8), 4)
    p, seed, off = 0.3, 77, 5
    o, _, _ = attention_fwd_dropout(q, k, v, p, seed, off)
    _close(attention_bwd_dropout(q, k, v, do, p, seed, off),
           attention_bwd_dropout(q, k, v, do, p, seed, off, o=o))
    o1, _, _ = attention_fwd_dropout(q, k, v, p, seed, off, kv_len=[1])
    delta = np.random.default_rng(5).standard_normal(o1.shape) * 1e-2
    dq, _, _, _ = attention_bwd_dropout(q, k, v, do, p, seed, off,
                                        kv_len=[1], o=o1 + delta)
    r = -np.sum(do * delta, axis=-1)
    assert np.max(np.abs(dq - r[..., None] * k[:, :, :1] / np.sqrt(8))) \
        <= 1e-12


def test_varlen_option_on_single_token_sequences():
    rng = np.random.default_rng(6)
    H, d = 2, 8
    cu = np.array([0, 1, 2, 9, 10])        # three one-token sequences
    q, k, v, do = (rng.standard_normal((H, 10, d)) for _ in range(4))
    o, _, _ = attention_fwd_varlen(q, k, v, cu, None, True)
    _close(attention_bwd_varlen(q, k, v, do, cu, None, True),
           attention_bwd_varlen(q, k, v, do, cu, None, True, o=o))
    delta = rng.standard_normal(o.shape) * 1e-2
    dq, _, _, _ = attention_bwd_varlen(q, k, v, do, cu, None, True,
                                       o=o + delta)
    r = -np.sum(do * delta, axis=-1)
    for t in (0, 1, 9):                    # one-hot on their own key
        assert np.max(np.abs(dq[:, t] - r[:, t, None] * k[:, t] /
                             np.sqrt(d))) <= 1e-12


def test_block_sparse_option_reduces_to_dense():
    q, k, v, do = _inputs((1, 2, 200, 8), 7)
    ones = np.ones((2, 2, 2), np.uint8)
    o, _, _ = attention_fwd(q, k, v, None, True)
    delta = np.random.default_rng(8).standard_normal(o.shape) * 1e-2
    _close(attention_bwd_block_sparse(q, k, v, do, ones, 128, None, True,
                                      o=o + delta),
           attention_bwd(q, k, v, do, None, True, o=o + delta))
