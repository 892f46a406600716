"""Block-sparse attention: the plain fp64 definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

FA notes §4.4 extends the method to block-sparse attention: the score matrix
is cut into blocks and most of them are skipped, which approximates full
attention (it is exact attention under the block mask).  The notes give no
mask format.  Readings (listed in the design notes): the mask is
block_mask[h, i, j] over blocks of `block` queries x `block` keys (nonzero:
query block i attends key block j), combined with the causal rule when
asked; a query row with no visible key has o = 0, l = 0, m = -inf and
contributes no gradient.  Layout as for dense attention: [B, H, N, d].
"""

import math

import numpy as np

__all__ = ["block_sparse_visible", "attention_fwd_block_sparse",
           "attention_bwd_block_sparse"]


def block_sparse_visible(block_mask_h, rows, n_keys, block, causal):
    """Boolean [len(rows), n_keys]: key j visible to query row i."""
    rows = np.asarray(rows, dtype=np.int64)
    keys = np.arange(n_keys)
    vis = np.asarray(block_mask_h)[rows[:, None] // block,
                                   keys[None, :] // block] != 0
    if causal:
        vis &= keys[None, :] <= rows[:, None]
    return vis


def _softmax_rows(s, vis):
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1, initial=-np.inf)
    m0 = np.where(np.isfinite(m), m, 0.0)
    e = np.where(vis, np.exp(s - m0[:, None]), 0.0)
    l = e.sum(axis=1)
    p = np.divide(e, l[:, None], out=np.zeros_like(e), where=l[:, None] > 0)
    return p, m, l


def attention_fwd_block_sparse(q, k, v, block_mask, block=128, scale=None,
                               causal=False, rows=None, row_chunk=512):
    """q, k, v: [B,H,N,d]; block_mask: [H, ceil(N/block), ceil(N/block)].
    Returns (o [B,H,R,d], m, l [B,H,R]) for the rows asked for."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, H, N, d = q.shape
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    rows = np.arange(N) if rows is None else np.asarray(rows, np.int64)
    o = np.zeros((B, H, rows.size, v.shape[3]))
    m = np.full((B, H, rows.size), -np.inf)
    l = np.zeros((B, H, rows.size))
    for h in range(H):
        for r0 in range(0, rows.size, row_chunk):
            rr = rows[r0:r0 + row_chunk]
            vis = block_sparse_visible(block_mask[h], rr, N, block, causal)
            for b in range(B):
                p, mm, ll = _softmax_rows(sc * (q[b, h, rr] @ k[b, h].T), vis)
                o[b, h, r0:r0 + rr.size] = p @ v[b, h]
                m[b, h, r0:r0 + rr.size] = mm
                l[b, h, r0:r0 + rr.size] = ll
    return o, m, l


def attention_bwd_block_sparse(q, k, v, do, block_mask, block=128, scale=None,
                               causal=False, row_chunk=512, o=None):
    """Gradients of sum(dO * O) under the block mask (the chain rule of the
    dense backward).

    o: None, or the stored forward output that the backward reads (FA notes
    §3.3 keeps O and (m, l) in HBM for the backward): then D is the row sum of
    dO * o.  With the exact O that is the same D; with O as stored in a
    narrower format it is the D such a backward forms, and the gradients are
    those of the recomputation given that O.

    Returns (dq, dk, dv, D [B,H,N])."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    B, H, N, d = q.shape
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    D = np.zeros((B, H, N))
    for h in range(H):
        for r0 in range(0, N, row_chunk):
            rr = np.arange(r0, min(N, r0 + row_chunk))
            vis = block_sparse_visible(block_mask[h], rr, N, block, causal)
            for b in range(B):
                p, _, _ = _softmax_rows(sc * (q[b, h, rr] @ k[b, h].T), vis)
                dv[b, h] += p.T @ do[b, h, rr]
                dp = do[b, h, rr] @ v[b, h].T
                if o is None:
                    Di = (p * dp).sum(axis=1)
                else:
                    Di = (do[b, h, rr] *
                          np.asarray(o[b, h, rr], np.float64)).sum(axis=1)
                ds = p * (dp - Di[:, None])
                dq[b, h, rr] = sc * (ds @ k[b, h])
                dk[b, h] += sc * (ds.T @ q[b, h, rr])
                D[b, h, rr] = Di
    return dq, dk, dv, D
