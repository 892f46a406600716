"""Pins of the oracle's paged decode and backward pass.

Paged decode: S12 ("implement it") says the paged kernel is the same loop
with a block-table lookup, so it must equal contiguous attention on the
gathered sequence and must not care where blocks physically live; the S12
production-practice paragraph adds the GQA head sharing.

Backward: the pages give no gradient formulas (FA notes §3.3 only says S and
P are recomputed), so the oracle's chain rule is pinned by central finite
differences of L = sum(dO * O) and by identities the gradients must satisfy.
"""

import numpy as np
import pytest

from oracle import (attention_bwd, attention_fwd, decode_paged, k_cache_rows,
                    paged_online)
from workloads import TID_KC, TID_VC, bf16_bits, paged_cache, rng as wl_rng


def _grouped(kc):
    """[nb, Hkv, bs, d] token rows -> the K cache order [nb, Hkv, d/32, bs,
    32] (element 32g + j of token u at [.., g, u, j]), by explicit loops."""
    nb, hkv, bs, d = kc.shape
    out = np.empty((nb, hkv, d // 32, bs, 32), dtype=kc.dtype)
    for g in range(d // 32):
        for u in range(bs):
            out[:, :, g, u, :] = kc[:, :, u, 32 * g:32 * g + 32]
    return out


def test_k_cache_rows_follows_the_documented_index():
    """Entry [p, h, g, u, j] of the K cache is element 32g + j of token u of
    head h in block p; k_cache_rows must put it at rows[p, h, u, 32g + j]."""
    rng = np.random.default_rng(23)
    k = rng.standard_normal((3, 2, 2, 5, 32))     # d = 64, block of 5
    rows = k_cache_rows(k)
    assert rows.shape == (3, 2, 5, 64)
    for p in range(3):
        for h in range(2):
            for g in range(2):
                for u in range(5):
                    for j in range(32):
                        assert rows[p, h, u, 32 * g + j] == k[p, h, g, u, j]
    assert np.array_equal(k_cache_rows(_grouped(rows)), rows)
    with pytest.raises(ValueError):
        k_cache_rows(np.zeros((1, 1, 2, 4, 16)))


def test_paged_cache_stores_k_grouped():
    """The generator draws K and V as [nb, Hkv, bs, d] from their seeded
    streams; V is stored as drawn, K at [.., g, u, j] = draw[.., u, 32g + j]."""
    lens = np.array([20, 35])
    cache = paged_cache(lens, 2, 64, 16, 3, cfg_seed=95, poison_tails=False)
    nb = cache.v_cache.store.shape[0]
    kd = wl_rng(95, TID_KC).standard_normal(size=(nb, 2, 16, 64),
                                            dtype=np.float32)
    vd = wl_rng(95, TID_VC).standard_normal(size=(nb, 2, 16, 64),
                                            dtype=np.float32)
    kbits, vbits = bf16_bits(kd), bf16_bits(vd)
    assert cache.k_cache.store.shape == (nb, 2, 2, 16, 32)
    assert np.array_equal(cache.v_cache.store, vbits)
    for g in range(2):
        for u in range(16):
            assert np.array_equal(cache.k_cache.store[:, :, g, u, :],
                                  kbits[:, :, u, 32 * g:32 * g + 32])


def _contiguous_to_paged(Kc, Vc, block_size, rng):
    """Scatter contiguous per-sequence K/V [L, Hkv, d] into a shuffled cache
    (V by token, K in the grouped cache order)."""
    lens = [x.shape[0] for x in Kc]
    nblk = [-(-L // block_size) for L in lens]
    total = sum(nblk)
    perm = rng.permutation(total)
    Hkv, d = Kc[0].shape[1:]
    kc = np.full((total, Hkv, block_size, d), np.nan)
    vc = np.full((total, Hkv, block_size, d), np.nan)
    table = np.full((len(lens), max(nblk)), -1)
    off = 0
    for b, L in enumerate(lens):
        for t in range(nblk[b]):
            phys = perm[off + t]
            table[b, t] = phys
            n = min(block_size, L - t * block_size)
            rows = slice(t * block_size, t * block_size + n)
            kc[phys, :, :n] = Kc[b][rows].transpose(1, 0, 2)
            vc[phys, :, :n] = Vc[b][rows].transpose(1, 0, 2)
        off += nblk[b]
    return _grouped(kc), vc, table


def test_paged_decode_equals_contiguous_attention():
    rng = np.random.default_rng(20)
    B, Hq, Hkv, d, bs = 3, 8, 2, 32, 4
    lens = [1, 13, 40]
    Kc = [rng.standard_normal((L, Hkv, d)) for L in lens]
    Vc = [rng.standard_normal((L, Hkv, d)) for L in lens]
    q = rng.standard_normal((B, Hq, d))
    kc, vc, table = _contiguous_to_paged(Kc, Vc, bs, rng)
    out = decode_paged(q, kc, vc, table, np.array(lens))
    G = Hq // Hkv
    for b in range(B):
        for hq in range(Hq):
            hk = hq // G      # consecutive query heads share one KV head
            o, _, _ = attention_fwd(q[b, hq][None, None, None],
                                    Kc[b][:, hk][None, None],
                                    Vc[b][:, hk][None, None])
            assert np.max(np.abs(out[b, hq] - o[0, 0, 0])) <= 1e-12
    assert np.all(np.isfinite(out))   # NaN tail slots never read


def test_paged_decode_invariant_to_block_placement():
    rng = np.random.default_rng(21)
    lens = np.array([37, 64, 5])
    cache = paged_cache(lens, 2, 32, 16, 4, cfg_seed=99)
    q = rng.standard_normal((3, 4, 32))
    out = decode_paged(q, cache.k_cache.exact, cache.v_cache.exact,
                       cache.block_table, lens)
    # move every physical block to a new slot and rewrite the table to match
    nb = cache.k_cache.exact.shape[0]
    perm = rng.permutation(nb)
    kc2 = np.empty_like(cache.k_cache.exact)
    vc2 = np.empty_like(cache.v_cache.exact)
    kc2[perm] = cache.k_cache.exact
    vc2[perm] = cache.v_cache.exact
    table2 = np.where(cache.block_table >= 0,
                      perm[np.maximum(cache.block_table, 0)], -1)
    out2 = decode_paged(q, kc2, vc2, table2, lens)
    assert np.array_equal(out, out2)


def test_paged_online_loop_equals_paged_definition():
    """The paged recurrence (one query, one KV head; table resolved to token
    rows, one block per tile) equals gather + softmax (the plain definition
    in ``decode_paged``)."""
    rng = np.random.default_rng(22)
    lens = np.array([1, 16, 17, 100])
    cache = paged_cache(lens, 1, 32, 16, 7, cfg_seed=98)
    q = rng.standard_normal((4, 1, 32))
    ref = decode_paged(q, cache.k_cache.exact, cache.v_cache.exact,
                       cache.block_table, lens)
    for b in range(4):
        o = paged_online(q[b, 0], k_cache_rows(cache.k_cache.exact)[:, 0],
                         cache.v_cache.exact[:, 0], cache.block_table[b],
                         int(lens[b]))
        assert np.max(np.abs(o - ref[b, 0])) <= 1e-13


def test_paged_decode_empty_sequence_is_zero():
    cache = paged_cache(np.array([0, 3]), 1, 32, 16, 2, cfg_seed=97)
    out = decode_paged(np.ones((2, 2, 32)), cache.k_cache.exact,
                       cache.v_cache.exact, cache.block_table, np.array([0, 3]))
    assert np.all(out[0] == 0) and np.all(np.isfinite(out[1]))


# --------------------------------------------------------------- backward --

def _loss(q, k, v, do, scale, causal, kv_len):
    o, _, _ = attention_fwd(q, k, v, scale, causal, kv_len)
    return float((o * do).sum())


@pytest.mark.parametrize("causal,kv_len", [(False, None), (True, None),
                                           (False, [3, 5]), (True, [4, 2])])
def test_backward_matches_finite_differences(causal, kv_len):
    rng = np.random.default_rng([23, int(causal)])
    B, H, N, d = 2, 1, 6, 3
    q, k, v, do = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    scale = 0.8
    dq, dk, dv, _ = attention_bwd(q, k, v, do, scale, causal, kv_len)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = _loss(args["q"], args["k"], args["v"], do, scale, causal,
                       kv_len)
            args[name] = xm
            lm = _loss(args["q"], args["k"], args["v"], do, scale, causal,
                       kv_len)
            num[idx] = (lp - lm) / (2 * h)
        err = np.max(np.abs(num - g)) / max(1e-12, np.max(np.abs(g)))
        assert err <= 1e-6, (name, err)


def test_backward_identities():
    rng = np.random.default_rng(24)
    B, H, N, d = 2, 2, 24, 5
    q, k, v, do = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    kv_len = [11, 24]
    o, _, _ = attention_fwd(q, k, v, None, True, kv_len)
    dq, dk, dv, D = attention_bwd(q, k, v, do, None, True, kv_len)
    # D = rowsum(P * dP) equals rowsum(dO * O)
    assert np.max(np.abs(D - (do * o).sum(-1))) <= 1e-12
    # keys beyond the valid length receive exactly zero gradient
    assert np.all(dk[0, :, 11:] == 0) and np.all(dv[0, :, 11:] == 0)
    # rows of dS sum to zero, so sum over keys of dK vanishes ...
    assert np.max(np.abs(dk.sum(axis=2))) <= 1e-12
    # ... and dQ is unchanged when every key is shifted by the same vector
    dq2, _, _, _ = attention_bwd(q, k + rng.standard_normal(d), v, do, None,
                                 True, kv_len)
    assert np.max(np.abs(dq2 - dq)) <= 1e-11
    # dV = P^T dO, so the sum over keys of dV is the sum of dO over the rows
    # that see at least one key (rows of P sum to 1)
    assert np.allclose(dv.sum(axis=2), do.sum(axis=2), atol=1e-12)


def test_backward_chunking_is_exact():
    rng = np.random.default_rng(25)
    q, k, v, do = (rng.standard_normal((1, 1, 40, 4)) for _ in range(4))
    a = attention_bwd(q, k, v, do, None, True, None, row_chunk=1024)
    b = attention_bwd(q, k, v, do, None, True, None, row_chunk=9)
    for x, y in zip(a, b):
        assert np.max(np.abs(x - y)) <= 1e-13
