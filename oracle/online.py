"""The method's own loops, in float64, written from the pages' descriptions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

These are a second, independent CPU path: they follow the order of operations
the pages give for the tiled computation, so the tests can show that every
variant reaches the plain definition of ``reference`` to rounding.

* ``kv_outer_tiled`` -- FA notes §3.2: key/value tiles in the outer loop,
  query tiles in the inner loop, O, l and m kept in "HBM" arrays, every step
  renormalised by diag(l_new)^-1.
* ``online_rows``    -- S12 "core idea": one pass over key tiles per query,
  running max m, running sum l, unnormalised accumulator o, rescale
  alpha = exp(m_old - m_new), one division at the end.
* ``merge_triples`` / ``split_merge`` -- S12 exercise 1 (flash-decoding): keys
  split over workers, each keeps its own (m, l, o), and the triples merge with
  the FA notes §3.1 rule m = max(m1, m2), l = e^{m1-m} l1 + e^{m2-m} l2.
* ``paged_online``   -- S12 "implement it" (paged addressing): the block
  table resolved to token rows, then ``online_rows`` with one cache block
  per tile.

The NaN guard (S12's box on exp(-inf - -inf)): with ``guard=False`` the running
max starts at -inf, so a first tile that is entirely masked gives NaN; with
``guard=True`` it starts at the large finite negative ``M_GUARD`` and masked
scores stay -inf, so their exponentials are exactly 0.
"""

import math

import numpy as np

from .reference import visible_mask

__all__ = ["M_GUARD", "kv_outer_tiled", "online_rows", "merge_triples",
           "split_merge", "paged_online"]

# Finite stand-in for -inf in the running max.  It must be a number that no
# visible score reaches and must differ from the masked value (-inf), or a
# fully masked tile would give exp(0) = 1 for its masked entries.
M_GUARD = -1.0e30


def _scale(d, scale):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def kv_outer_tiled(q, k, v, br, bc, scale=None, causal=False, kv_valid=None,
                   guard=True):
    """FA notes §3.2 tiled forward for one head: q [N,d], k/v [Nk,d].

    Outer loop over key/value tiles j (size bc), inner loop over query tiles i
    (size br).  For each pair: S_ij, tile row max m~, P~ = exp(S - m~), tile
    row sum l~; m_new = max(m_i, m~);
    l_new = e^{m_i - m_new} l_i + e^{m~ - m_new} l~;
    O_i = diag(l_new)^-1 (diag(l_i) e^{m_i - m_new} O_i + e^{m~ - m_new} P~ V_j).

    Masks (not in the §3.2 listing; added as §3.4's "optional masking") set
    masked scores to -inf.  With guard=True the tile max is floored at M_GUARD
    (so P~ of a fully masked tile row is exactly 0) and rows whose l is still 0
    keep O = 0.  Returns (o, m, l); m is M_GUARD (guard) for rows with nothing
    visible.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    N, d = q.shape
    Nk = k.shape[0]
    sc = _scale(d, scale)
    valid = Nk if kv_valid is None else int(kv_valid)
    init = M_GUARD if guard else -np.inf
    O = np.zeros((N, v.shape[1]))
    l = np.zeros(N)
    m = np.full(N, init)
    for j0 in range(0, Nk, bc):
        Kj, Vj = k[j0:j0 + bc], v[j0:j0 + bc]
        cols = np.arange(j0, j0 + Kj.shape[0])
        for i0 in range(0, N, br):
            rows = np.arange(i0, min(N, i0 + br))
            Qi, Oi, li, mi = q[rows], O[rows], l[rows], m[rows]
            S = sc * (Qi @ Kj.T)
            vis = visible_mask(rows, Nk, causal, valid)[:, cols]
            S = np.where(vis, S, -np.inf)
            mt = S.max(axis=1)
            if guard:
                mt = np.maximum(mt, M_GUARD)
            Pt = np.exp(S - mt[:, None])
            lt = Pt.sum(axis=1)
            m_new = np.maximum(mi, mt)
            a_old = np.exp(mi - m_new)
            a_new = np.exp(mt - m_new)
            l_new = a_old * li + a_new * lt
            num = (li * a_old)[:, None] * Oi + a_new[:, None] * (Pt @ Vj)
            if guard:
                Oi = np.divide(num, l_new[:, None], out=np.zeros_like(num),
                               where=l_new[:, None] > 0)
            else:
                Oi = num / l_new[:, None]
            O[rows], l[rows], m[rows] = Oi, l_new, m_new
    return O, m, l


def online_rows(q, k, v, tile, scale=None, causal=False, kv_valid=None,
                guard=True, key_range=None):
    """S12 "core idea" recurrence, run for every query row of one head.

    q [N,d], k/v [Nk,d].  For each key tile: s = scale * q k^T (masked -> -inf),
    m_new = max(m, max s), alpha = exp(m - m_new), p = exp(s - m_new),
    l = alpha l + sum p, o = alpha o + p V, m = m_new.  Returns the
    *unnormalised* triple (m, l, o); the output is o / l.

    key_range=(lo, hi) restricts the loop to keys lo..hi-1 (one worker's share
    in flash-decoding).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    N, d = q.shape
    Nk = k.shape[0]
    sc = _scale(d, scale)
    valid = Nk if kv_valid is None else int(kv_valid)
    lo, hi = (0, Nk) if key_range is None else key_range
    rows = np.arange(N)
    m = np.full(N, M_GUARD if guard else -np.inf)
    l = np.zeros(N)
    o = np.zeros((N, v.shape[1]))
    for j0 in range(lo, hi, tile):
        j1 = min(hi, j0 + tile)
        s = sc * (q @ k[j0:j1].T)
        vis = visible_mask(rows, Nk, causal, valid)[:, j0:j1]
        s = np.where(vis, s, -np.inf)
        m_new = np.maximum(m, s.max(axis=1))
        alpha = np.exp(m - m_new)
        p = np.exp(s - m_new[:, None])
        l = alpha * l + p.sum(axis=1)
        o = alpha[:, None] * o + p @ v[j0:j1]
        m = m_new
    return m, l, o


def merge_triples(ms, ls, os_):
    """Merge per-worker (m, l, o) triples (FA notes §3.1 rule; S12 ex. 1).

    ms, ls: [P, N]; os_: [P, N, d].  m = max_p m_p, w_p = exp(m_p - m),
    l = sum_p w_p l_p, o = sum_p w_p o_p.  Returns (m, l, o), unnormalised.
    A worker that saw no visible key has (M_GUARD, 0, 0) and weight
    exp(M_GUARD - m) = 0 whenever any worker saw one.
    """
    ms = np.asarray(ms, np.float64)
    m = ms.max(axis=0)
    w = np.exp(ms - m[None])
    l = (w * ls).sum(axis=0)
    o = (w[..., None] * os_).sum(axis=0)
    return m, l, o


def split_merge(q, k, v, n_splits, tile=64, scale=None, causal=False,
                kv_valid=None):
    """Flash-decoding on one head: split keys into n_splits contiguous ranges
    of ceil(Nk / n_splits) keys, run ``online_rows`` on each, merge.

    Returns the normalised output [N, d] (0 for rows with l = 0).
    """
    Nk = k.shape[0]
    per = -(-Nk // n_splits)
    ms, ls, os_ = [], [], []
    for p in range(n_splits):
        lo, hi = min(Nk, p * per), min(Nk, (p + 1) * per)
        mp, lp, op = online_rows(q, k, v, tile, scale, causal, kv_valid,
                                 guard=True, key_range=(lo, hi))
        ms.append(mp)
        ls.append(lp)
        os_.append(op)
    m, l, o = merge_triples(ms, ls, os_)
    return np.divide(o, l[:, None], out=np.zeros_like(o), where=l[:, None] > 0)


def paged_online(q, k_cache, v_cache, table, length, scale=None):
    """Decode of one query vector q [d] against one KV head's paged cache.

    Definition followed: S12 "implement it" (paged addressing): token p of
    the sequence is slot p mod bs of physical block table[p // bs], with bs
    the block size, so the last block is only partly filled.  Here the table
    is first resolved into the flat cache row of each of the ``length``
    tokens, and ``online_rows`` (the S12 recurrence, pinned on its own) then
    runs over the gathered rows with tile = bs, i.e. one cache block per step
    of the recurrence.

    k_cache, v_cache: [num_blocks, bs, d] (one KV head).  Returns o / l
    (zeros for length 0).
    """
    n_blocks, bs, dv = v_cache.shape
    q = np.asarray(q, np.float64)
    if length <= 0:
        return np.zeros(dv)
    pos = np.arange(int(length))
    flat = np.asarray(table, np.int64)[pos // bs] * bs + pos % bs
    keys = np.asarray(k_cache, np.float64).reshape(n_blocks * bs, -1)[flat]
    vals = np.asarray(v_cache, np.float64).reshape(n_blocks * bs, dv)[flat]
    _, l, o = online_rows(q[None, :], keys, vals, bs, scale)
    return o[0] / l[0] if l[0] > 0 else np.zeros(dv)
