"""Pins of the dropout oracle (oracle/dropout.py).

The generator is pinned to the published known-answer vectors of Philox4x32-10
(tests/golden/philox4x32_10_kat.json, with its citation); the stream layout to
a scalar route that packs the output words into bytes with ``struct``; the
keep rule to its exact rate and to byte uniformity; the forward to pure-Python
loops and to plain attention at p = 0; the backward to torch autograd (float64,
CPU) of the forward definition and to central finite differences."""

import json
import math
import os
import struct

import numpy as np
import pytest
import torch

from oracle import (attention_bwd_dropout, attention_fwd,
                    attention_fwd_dropout, dropout_keep, dropout_threshold,
                    philox4x32_10)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden",
                      "philox4x32_10_kat.json")


def _kat():
    with open(GOLDEN) as f:
        vecs = json.load(f)["vectors"]
    h = lambda xs: [int(x, 16) for x in xs]  # noqa: E731
    return [(h(v["counter"]), h(v["key"]), h(v["output"])) for v in vecs]


def test_philox_known_answer_vectors():
    kat = _kat()
    for ctr, key, out in kat:
        got = philox4x32_10(np.array(ctr), np.array(key))
        assert [int(x) for x in got] == out
    # batched, with a different key per counter
    ctrs = np.array([c for c, _, _ in kat])
    keys = np.array([k for _, k, _ in kat])
    got = philox4x32_10(ctrs, keys)
    assert got.tolist() == [o for _, _, o in kat]


def test_philox_is_injective_on_a_counter_range():
    # For a fixed key each round is a bijection of the 128-bit state.
    ctr = np.zeros((1 << 16, 4), np.uint64)
    ctr[:, 0] = np.arange(1 << 16)
    ctr[:, 2] = 7
    out = philox4x32_10(ctr, np.array([11, 13]))
    assert len({tuple(r) for r in out.tolist()}) == 1 << 16


@pytest.mark.parametrize("p,t", [(0.0, 0), (0.1, 26), (0.5, 128),
                                 (0.5 / 256, 1), (0.25 / 256, 0),
                                 (0.998, 255), (254.5 / 256, 255)])
def test_threshold_rounds_half_up(p, t):
    T, s = dropout_threshold(p)
    assert T == t
    assert s == 256.0 / (256 - t)


@pytest.mark.parametrize("p", [-0.01, 0.999, 1.0, 255.5 / 256])
def test_threshold_rejects_out_of_range(p):
    with pytest.raises(ValueError):
        dropout_threshold(p)


def _keep_scalar(bh, i, j, seed, offset, T):
    """Keep decision of one element through a separate route: the four output
    words are packed little-endian with struct and byte t is indexed."""
    block, within = divmod(j, 32)
    half = (within // 8) % 2          # which 8-key run of a 16-key half
    g = 2 * block + half
    t = 8 * (within // 16) + within % 8
    words = philox4x32_10(np.array([i, g, bh, offset]),
                          np.array([seed % (1 << 32), seed >> 32]))
    raw = struct.pack("<4I", *[int(w) for w in words])
    return raw[t] >= T


def test_keep_matches_scalar_route():
    rng = np.random.default_rng(61)
    seed, offset, T = 0x1234_5678_9ABC_DEF0, 77, 90
    rows = np.array([0, 1, 31, 32, 100, 4095])
    z = dropout_keep(5, rows, 200, seed, offset, T)
    for ri, i in enumerate(rows):
        for j in list(range(40)) + list(rng.integers(40, 200, 20)):
            assert z[ri, j] == _keep_scalar(5, int(i), int(j), seed, offset, T)


def test_each_call_serves_sixteen_keys_once():
    # Every (group, byte) pair is used by exactly one key of the row.
    n = 160
    seen = {}
    for j in range(n):
        within = j % 32
        key = (2 * (j // 32) + (within // 8) % 2, 8 * (within // 16) + within % 8)
        assert key not in seen
        seen[key] = j
    assert all(0 <= t < 16 for _, t in seen)
    assert len({g for g, _ in seen}) == 2 * (n // 32)


@pytest.mark.parametrize("T", [0, 26, 128, 255])
def test_keep_rate_is_the_quantised_probability(T):
    z = dropout_keep(3, np.arange(512), 2048, 99, 0, T)
    rate = z.mean()
    expect = (256 - T) / 256
    if T == 0:
        assert z.all()
        return
    sigma = math.sqrt(expect * (1 - expect) / z.size)
    assert abs(rate - expect) < 6 * sigma


def test_bytes_are_uniform():
    ctr = np.zeros((1 << 16, 4), np.uint64)
    ctr[:, 0] = np.arange(1 << 16) % 257
    ctr[:, 1] = np.arange(1 << 16) // 257
    words = philox4x32_10(ctr, np.array([5, 6]))
    byts = np.concatenate([(words >> np.uint64(8 * s)) & np.uint64(255)
                           for s in range(4)]).ravel()
    hist = np.bincount(byts.astype(np.int64), minlength=256)
    e = byts.size / 256
    chi2 = ((hist - e) ** 2 / e).sum()
    assert chi2 < 255 + 6 * math.sqrt(2 * 255)   # 255 degrees of freedom


def test_streams_depend_on_every_coordinate():
    base = dropout_keep(2, np.arange(64), 64, 42, 0, 128)
    assert np.array_equal(base, dropout_keep(2, np.arange(64), 64, 42, 0, 128))
    for other in (dropout_keep(3, np.arange(64), 64, 42, 0, 128),
                  dropout_keep(2, np.arange(64), 64, 43, 0, 128),
                  dropout_keep(2, np.arange(64), 64, 42 + (1 << 32), 0, 128),
                  dropout_keep(2, np.arange(64), 64, 42, 1, 128),
                  dropout_keep(2, np.arange(64, 128), 64, 42, 0, 128)):
        assert not np.array_equal(base, other)
        assert 0.4 < (base == other).mean() < 0.6


@pytest.mark.parametrize("causal", [False, True])
def test_zero_drop_is_plain_attention(causal):
    rng = np.random.default_rng(62)
    q, k, v = (rng.standard_normal((2, 2, 45, 8)) for _ in range(3))
    o, m, l = attention_fwd_dropout(q, k, v, 0.0, 1, 0, None, causal, [45, 30])
    od, md, ld = attention_fwd(q, k, v, None, causal, [45, 30])
    assert np.max(np.abs(o - od)) <= 1e-13
    assert np.array_equal(m, md) and np.max(np.abs(l - ld)) <= 1e-13


@pytest.mark.parametrize("causal,valid", [(False, 11), (True, 11), (False, 7)])
def test_forward_matches_brute_force(causal, valid):
    rng = np.random.default_rng([63, valid, int(causal)])
    B, H, N, d = 1, 2, 11, 3
    q, k, v = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    p, seed, off = 0.3, 2024, 5
    T = math.floor(0.3 * 256 + 0.5)
    s = 256 / (256 - T)
    o, _, _ = attention_fwd_dropout(q, k, v, p, seed, off, 0.6, causal, [valid])
    for h in range(H):
        for i in range(N):
            keys = [j for j in range(N) if j < valid and (not causal or j <= i)]
            sc = [0.6 * sum(q[0, h, i, c] * k[0, h, j, c] for c in range(d))
                  for j in keys]
            mx = max(sc)
            e = [math.exp(x - mx) for x in sc]
            tot = sum(e)
            for c in range(d):
                acc = 0.0
                for jj, j in enumerate(keys):
                    if _keep_scalar(h, i, j, seed, off, T):
                        acc += e[jj] / tot * s * v[0, h, j, c]
                assert abs(o[0, h, i, c] - acc) <= 1e-13


def _torch_loss(q, k, v, do, z, scale, causal, valid):
    s = scale * q @ k.transpose(-1, -2)
    N = q.shape[-2]
    j = torch.arange(N)
    vis = j[None, :] < valid
    if causal:
        vis = vis & (j[None, :] <= j[:, None])
    s = s.masked_fill(~vis, float("-inf"))
    p = torch.softmax(s, dim=-1)
    o = (p * z) @ v
    return (o * do).sum(), o


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_autograd(causal):
    rng = np.random.default_rng([64, int(causal)])
    B, H, N, d = 1, 2, 40, 8
    q, k, v, do = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    p, seed, off = 0.2, 31337, 2
    T, ks = dropout_threshold(p)
    dq, dk, dv, D = attention_bwd_dropout(q, k, v, do, p, seed, off, None,
                                          causal)
    o, _, _ = attention_fwd_dropout(q, k, v, p, seed, off, None, causal)
    for h in range(H):
        z = torch.tensor(dropout_keep(h, np.arange(N), N, seed, off, T) * ks)
        tq, tk, tv = (torch.tensor(x[0, h], requires_grad=True)
                      for x in (q, k, v))
        loss, to = _torch_loss(tq, tk, tv, torch.tensor(do[0, h]), z,
                               1 / math.sqrt(d), causal, N)
        loss.backward()
        assert np.max(np.abs(to.detach().numpy() - o[0, h])) <= 1e-12
        assert np.max(np.abs(tq.grad.numpy() - dq[0, h])) <= 1e-11
        assert np.max(np.abs(tk.grad.numpy() - dk[0, h])) <= 1e-11
        assert np.max(np.abs(tv.grad.numpy() - dv[0, h])) <= 1e-11
    # D is the identity rowsum(dO * O) the kernels use
    assert np.max(np.abs(D - (do * o).sum(-1))) <= 1e-12


def test_backward_finite_differences():
    rng = np.random.default_rng(65)
    B, H, N, d = 1, 1, 9, 4
    q, k, v, do = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    args = (0.4, 8, 0, 0.5, True, [8])
    dq, dk, dv, _ = attention_bwd_dropout(q, k, v, do, *args)

    def loss(q_, k_, v_):
        o, _, _ = attention_fwd_dropout(q_, k_, v_, *args)
        return (o * do).sum()

    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in [(0, 0, 3, 1), (0, 0, 7, 2), (0, 0, 0, 0), (0, 0, 8, 3)]:
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            pick = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            pickm = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            fd = (loss(*pick) - loss(*pickm)) / (2 * eps)
            assert abs(fd - g[idx]) <= 1e-7, (name, idx)


def test_row_subset_equals_full_rows():
    rng = np.random.default_rng(66)
    q, k, v = (rng.standard_normal((1, 2, 70, 8)) for _ in range(3))
    rows = np.array([69, 0, 33, 34])
    o, m, l = attention_fwd_dropout(q, k, v, 0.3, 5, 1, None, True)
    os_, ms, ls = attention_fwd_dropout(q, k, v, 0.3, 5, 1, None, True,
                                        rows=rows)
    assert np.array_equal(os_, o[:, :, rows])
    assert np.array_equal(ms, m[:, :, rows]) and np.array_equal(ls, l[:, :, rows])
