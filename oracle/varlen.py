"""Packed variable-length ("varlen") attention: the plain fp64 definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

S12's NaN box notes that under a causal mask on a ragged batch whole tiles are
routinely masked out.  Ragged batches are packed: the B sequences of a batch
lie back to back along one token axis, sequence b occupying tokens
cu_seqlens[b] .. cu_seqlens[b+1]-1 (cu_seqlens[0] = 0, non-decreasing).
Readings (listed in the design notes):

* Self-attention: queries and keys share the packing.  Token i attends token j
  iff both belong to the same sequence and, when causal, j <= i (within one
  sequence, packed order is position order).
* Layout: head-major packed, q, k, v, o [H, total, d]; m, l [H, total].
* A sequence of length 0 holds no tokens; there is nothing to compute for it.

The definition is the masked softmax of FA notes §2.1 applied on the packed
token axis with that block-diagonal (and causal) visibility; rows are done in
chunks only to bound memory.
"""

import math

import numpy as np

from .reference import k_cache_rows

__all__ = ["varlen_visible", "attention_fwd_varlen", "attention_bwd_varlen",
           "prefill_paged"]


def _scale(d, scale):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def _seq_of(cu_seqlens, total):
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if cu[0] != 0 or cu[-1] != total or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must start at 0, end at total and not "
                         "decrease")
    seq = np.empty(total, dtype=np.int64)
    for b in range(cu.size - 1):
        seq[cu[b]:cu[b + 1]] = b
    return seq


def varlen_visible(cu_seqlens, rows, total, causal):
    """Boolean [len(rows), total]: key token j visible to query token i."""
    seq = _seq_of(cu_seqlens, total)
    rows = np.asarray(rows, dtype=np.int64)
    vis = seq[rows][:, None] == seq[None, :]
    if causal:
        vis &= np.arange(total)[None, :] <= rows[:, None]
    return vis


def _softmax_rows(s, vis):
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1, initial=-np.inf)
    m0 = np.where(np.isfinite(m), m, 0.0)
    e = np.where(vis, np.exp(s - m0[:, None]), 0.0)
    l = e.sum(axis=1)
    p = np.divide(e, l[:, None], out=np.zeros_like(e), where=l[:, None] > 0)
    return p, m, l


def attention_fwd_varlen(q, k, v, cu_seqlens, scale=None, causal=False,
                         rows=None, row_chunk=512):
    """q, k, v: [H, total, d].  Returns (o [H,R,d], m [H,R], l [H,R]) for the
    rows asked for (all when rows is None): S = scale * Q K^T over the visible
    keys, m its row max, l = sum exp(S - m), O = softmax(S) V."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    H, total, d = q.shape
    sc = _scale(d, scale)
    rows = np.arange(total) if rows is None else np.asarray(rows, np.int64)
    o = np.zeros((H, rows.size, v.shape[2]))
    m = np.full((H, rows.size), -np.inf)
    l = np.zeros((H, rows.size))
    for r0 in range(0, rows.size, row_chunk):
        rr = rows[r0:r0 + row_chunk]
        vis = varlen_visible(cu_seqlens, rr, total, causal)
        for h in range(H):
            p, mm, ll = _softmax_rows(sc * (q[h, rr] @ k[h].T), vis)
            o[h, r0:r0 + rr.size] = p @ v[h]
            m[h, r0:r0 + rr.size] = mm
            l[h, r0:r0 + rr.size] = ll
    return o, m, l


def attention_bwd_varlen(q, k, v, do, cu_seqlens, scale=None, causal=False,
                         row_chunk=512, o=None):
    """Gradients of sum(dO * O) for O = attention_fwd_varlen(...), by the same
    chain rule as the dense backward (dV = P^T dO, dP = dO V^T,
    D = rowsum(P * dP), dS = P * (dP - D), dQ = scale dS K,
    dK = scale dS^T Q).

    o: None, or the stored forward output that the backward reads (FA notes
    §3.3 keeps O and (m, l) in HBM for the backward): then D is the row sum of
    dO * o.  With the exact O that is the same D; with O as stored in a
    narrower format it is the D such a backward forms, and the gradients are
    those of the recomputation given that O.

    Returns (dq, dk, dv, D [H, total])."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    H, total, d = q.shape
    sc = _scale(d, scale)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    D = np.zeros((H, total))
    for r0 in range(0, total, row_chunk):
        rr = np.arange(r0, min(total, r0 + row_chunk))
        vis = varlen_visible(cu_seqlens, rr, total, causal)
        for h in range(H):
            p, _, _ = _softmax_rows(sc * (q[h, rr] @ k[h].T), vis)
            dv[h] += p.T @ do[h, rr]
            dp = do[h, rr] @ v[h].T
            if o is None:
                Di = (p * dp).sum(axis=1)
            else:
                Di = (do[h, rr] * np.asarray(o[h, rr], np.float64)).sum(axis=1)
            ds = p * (dp - Di[:, None])
            dq[h, rr] = sc * (ds @ k[h])
            dk[h] += sc * (ds.T @ q[h, rr])
            D[h, rr] = Di
    return dq, dk, dv, D


def prefill_paged(q, k_cache, v_cache, block_table, seq_lens, cu_seqlens_q,
                  scale=None, causal=True):
    """Prefill of packed new tokens against a paged KV cache, by gather +
    masked softmax (fp64).

    S12's paged loop reads logical block t of a sequence from physical block
    block_table[t], the last block holding n = min(block_size, seq_len -
    t*block_size) tokens; GQA (S12 production paragraph): query head hq reads
    KV head hq // (Hq/Hkv).  Readings: the cache already holds the K/V of
    every one of the seq_lens[b] tokens of sequence b, including its new
    ones; the new tokens are the last qlen_b = cu[b+1] - cu[b] positions, so
    new token i sits at position seq_lens[b] - qlen_b + i and, when causal,
    sees cached positions <= that one.

    q: [Hq, total_q, d]; v_cache: [num_blocks, Hkv, block_size, d]; k_cache:
    the same blocks of K in the library's grouped order
    (``reference.k_cache_rows``);
    block_table: [B, max_blocks]; seq_lens: [B].  Returns (o, m, l) with
    o [Hq, total_q, d] and m, l [Hq, total_q] as in the dense definition.
    """
    q = np.asarray(q, dtype=np.float64)
    Hq, total_q, d = q.shape
    k_cache = k_cache_rows(k_cache)
    Hkv, bs = k_cache.shape[1], k_cache.shape[2]
    G = Hq // Hkv
    sc = _scale(d, scale)
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    o = np.zeros((Hq, total_q, v_cache.shape[3]))
    m = np.full((Hq, total_q), -np.inf)
    l = np.zeros((Hq, total_q))
    for b in range(cu.size - 1):
        qs, qe = int(cu[b]), int(cu[b + 1])
        L = int(seq_lens[b])
        if qe == qs:
            continue
        kk, vv = [], []
        for t in range(-(-L // bs)):
            n = min(bs, L - t * bs)
            phys = int(block_table[b, t])
            kk.append(np.asarray(k_cache[phys, :, :n], dtype=np.float64))
            vv.append(np.asarray(v_cache[phys, :, :n], dtype=np.float64))
        Kb = np.concatenate(kk, axis=1) if kk else np.zeros((Hkv, 0, d))
        Vb = np.concatenate(vv, axis=1) if vv else np.zeros((Hkv, 0, d))
        pos = L - (qe - qs) + np.arange(qe - qs)
        vis = np.ones((qe - qs, L), dtype=bool)
        if causal:
            vis &= np.arange(L)[None, :] <= pos[:, None]
        for hq in range(Hq):
            hk = hq // G
            p, mm, ll = _softmax_rows(sc * (q[hq, qs:qe] @ Kb[hk].T), vis)
            o[hq, qs:qe] = p @ Vb[hk]
            m[hq, qs:qe] = mm
            l[hq, qs:qe] = ll
    return o, m, l
