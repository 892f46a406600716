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


# ----------------------------------------------------------- paged prefill --

from oracle import decode_paged, prefill_paged  # noqa: E402
from workloads import paged_cache  # noqa: E402


def _cache_from_packed(kp, vp, lens, bs, rng):
    """Scatter packed per-sequence K/V [Hkv, total, d] into a shuffled
    head-major cache (V [num_blocks, Hkv, bs, d], K in the grouped cache
    order [num_blocks, Hkv, d/32, bs, 32]); returns (kc, vc, table)."""
    Hkv, _, d = kp.shape
    nblk = [-(-L // bs) for L in lens]
    total_blocks = max(1, sum(nblk))
    perm = rng.permutation(total_blocks)
    kc = np.full((total_blocks, Hkv, bs, d), np.nan)
    vc = np.full((total_blocks, Hkv, bs, d), np.nan)
    table = np.full((len(lens), max(1, max(nblk))), -1)
    off = tok = 0
    for b, L in enumerate(lens):
        for t in range(nblk[b]):
            phys = perm[off + t]
            table[b, t] = phys
            n = min(bs, L - t * bs)
            kc[phys, :, :n] = kp[:, tok + t * bs:tok + t * bs + n]
            vc[phys, :, :n] = vp[:, tok + t * bs:tok + t * bs + n]
        off += nblk[b]
        tok += L
    grouped = np.empty((total_blocks, Hkv, d // 32, bs, 32))
    for g in range(d // 32):
        grouped[:, :, g] = kc[:, :, :, 32 * g:32 * g + 32]
    return grouped, vc, table


@pytest.mark.parametrize("causal", [False, True])
def test_prefill_from_empty_context_equals_varlen(causal):
    rng = np.random.default_rng([41, int(causal)])
    lens = [20, 1, 37, 16]
    Hkv, G, d = 2, 2, 32
    cu = np.concatenate([[0], np.cumsum(lens)])
    kp = rng.standard_normal((Hkv, cu[-1], d))
    vp = rng.standard_normal((Hkv, cu[-1], d))
    q = rng.standard_normal((Hkv * G, cu[-1], d))
    kc, vc, table = _cache_from_packed(kp, vp, lens, 16, rng)
    o, m, l = prefill_paged(q, kc, vc, table, lens, cu, None, causal)
    ko, mo, lo = attention_fwd_varlen(q, np.repeat(kp, G, axis=0),
                                      np.repeat(vp, G, axis=0), cu, None,
                                      causal)
    assert np.max(np.abs(o - ko)) <= 1e-13
    assert np.max(np.abs(m - mo)) <= 1e-13
    assert np.max(np.abs(l / lo - 1)) <= 1e-13


def test_prefill_of_one_token_equals_paged_decode():
    rng = np.random.default_rng(42)
    lens = np.array([1, 17, 40, 100])
    cache = paged_cache(lens, 2, 32, 16, 8, cfg_seed=43)
    q = rng.standard_normal((4, 8, 32))         # [B, Hq, d] one token each
    ref = decode_paged(q, cache.k_cache.exact, cache.v_cache.exact,
                       cache.block_table, lens)
    cu = np.arange(5)
    o, _, _ = prefill_paged(q.transpose(1, 0, 2), cache.k_cache.exact,
                            cache.v_cache.exact, cache.block_table, lens, cu,
                            None, True)
    assert np.max(np.abs(o.transpose(1, 0, 2) - ref)) <= 1e-13


def test_prefill_matches_brute_force_with_context():
    rng = np.random.default_rng(44)
    L, qlen, d = 23, 6, 32
    kp = rng.standard_normal((1, L, d))
    vp = rng.standard_normal((1, L, d))
    qfull = rng.standard_normal((L, d))
    kc, vc, table = _cache_from_packed(kp, vp, [L], 4, rng)
    o, _, _ = prefill_paged(qfull[None, L - qlen:], kc, vc, table, [L],
                            [0, qlen], 0.6, True)
    # brute force over every position; the new tokens are the last qlen rows
    ref = brute_fwd(qfull.tolist(), kp[0].tolist(), vp[0].tolist(), 0.6, True)
    assert np.max(np.abs(o[0] - np.array(ref[L - qlen:]))) <= 1e-13


def test_prefill_is_invariant_to_moving_blocks():
    rng = np.random.default_rng(45)
    lens = np.array([33, 70])
    cache = paged_cache(lens, 1, 32, 16, 5, cfg_seed=46)
    cu = np.array([0, 9, 29])
    q = rng.standard_normal((2, 29, 32))
    kc, vc = cache.k_cache.exact, cache.v_cache.exact
    o, _, _ = prefill_paged(q, kc, vc, cache.block_table, lens, cu)
    perm = rng.permutation(kc.shape[0])
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[perm], vc2[perm] = kc, vc
    table2 = np.where(cache.block_table >= 0, perm[cache.block_table], -1)
    o2, _, _ = prefill_paged(q, kc2, vc2, table2, lens, cu)
    assert np.array_equal(o, o2)
