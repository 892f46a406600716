"""Plain fp64 definitions of attention forward, backward and paged decode.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Everything here is the textbook definition written out with NumPy in float64.
There is no tiling, no online recurrence and no fusion: each query row sees all
of its visible keys at once.  Rows may be processed in chunks purely to bound
memory (a row's result does not depend on other rows), so N = 65536 never holds
an N x N array.

Readings of points the pages leave open (each is listed in the design notes):

* Scale: the FA notes §2.1 statement has no scale; S12's recurrence divides the
  scores by sqrt(d).  Here S = scale * Q K^T with scale defaulting to
  1/sqrt(d), applied before the max, so the stored max m is in scaled units.
* Masks are applied by excluding keys (the score is -inf), never by adding a
  finite penalty.  Key j is visible to query i iff j < kv_len[b] and, when
  causal, j <= i (square problems, top-left alignment).
* A row with no visible key (only reachable through kv_len = 0) has O = 0,
  l = 0 and m = -inf, and contributes nothing to any gradient.
"""

import math

import numpy as np

__all__ = ["visible_mask", "attention_fwd", "attention_bwd", "decode_paged",
           "k_cache_rows"]


def _default_scale(d, scale):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def visible_mask(rows, n_keys, causal, kv_valid):
    """Boolean [len(rows), n_keys]: True where key j is visible to query row i.

    The causal rule (key j visible iff j <= i) is S12 exercise 2's causal
    tiled variant; the key-padding rule (keys j >= valid length excluded) is
    the "optional masking" of FA notes §3.4's fused op list.
    """
    rows = np.asarray(rows)
    j = np.arange(n_keys)
    vis = np.broadcast_to(j[None, :] < kv_valid, (rows.size, n_keys)).copy()
    if causal:
        vis &= j[None, :] <= rows[:, None]
    return vis


def _row_softmax(s, vis):
    """Safe softmax of the visible entries of each row of s (FA notes §3.1).

    Returns (p, m, l): m is the row max over visible entries, l the sum of
    exp(s - m) over them, p = exp(s - m) / l with zeros where not visible.
    Rows with nothing visible give p = 0, m = -inf, l = 0.
    """
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1, initial=-np.inf)
    any_vis = vis.any(axis=1)
    m_safe = np.where(any_vis, m, 0.0)
    e = np.where(vis, np.exp(s - m_safe[:, None]), 0.0)
    l = e.sum(axis=1)
    p = np.divide(e, l[:, None], out=np.zeros_like(e), where=l[:, None] > 0)
    return p, m, l


def attention_fwd(q, k, v, scale=None, causal=False, kv_len=None, rows=None,
                  row_chunk=1024):
    """Exact attention forward, FA notes §2.1 (Algorithm 0) in float64.

    q: [B,H,N,d]; k, v: [B,H,Nk,d] (any real dtype, computed in float64).
    kv_len: None or int sequence [B] of valid key counts.
    rows: None for every query row, or a 1-D array of row indices to compute
    (the result for a row depends on that row alone).

    Returns (o [B,H,R,d], m [B,H,R], l [B,H,R]) where R = N or len(rows):
    S = scale * Q K^T, m = rowmax of visible S, l = sum exp(S - m),
    P = exp(S - m) / l, O = P V.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, d = q.shape
    Nk = k.shape[2]
    dv = v.shape[3]
    sc = _default_scale(d, scale)
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.size
    o = np.zeros((B, H, R, dv))
    m = np.full((B, H, R), -np.inf)
    l = np.zeros((B, H, R))
    for b in range(B):
        valid = Nk if kv_len is None else int(kv_len[b])
        for r0 in range(0, R, row_chunk):
            rr = rows[r0:r0 + row_chunk]
            kend = valid
            if causal and rr.size:
                kend = min(kend, int(rr.max()) + 1)
            kend = max(kend, 0)
            vis = visible_mask(rr, kend, causal, valid)
            for h in range(H):
                s = sc * (q[b, h, rr] @ k[b, h, :kend].T)
                p, mm, ll = _row_softmax(s, vis)
                o[b, h, r0:r0 + rr.size] = p @ v[b, h, :kend]
                m[b, h, r0:r0 + rr.size] = mm
                l[b, h, r0:r0 + rr.size] = ll
    return o, m, l


def attention_bwd(q, k, v, do, scale=None, causal=False, kv_len=None,
                  row_chunk=1024, o=None):
    """Gradients of L = sum(dO * O) for O = attention_fwd(q, k, v), float64.

    The pages only say that the backward pass recomputes S and P from the
    saved statistics (FA notes §3.3); the gradient formulas are the textbook
    softmax chain rule, written out here:

        dV = P^T dO
        dP = dO V^T
        D_i = sum_j P_ij dP_ij            (equals sum_c dO_ic O_ic)
        dS = P * (dP - D)
        dQ = scale * dS K
        dK = scale * dS^T Q

    o: None, or the stored forward output that the backward reads (FA notes
    §3.3 keeps O and (m, l) in HBM for the backward): then D is the row sum of
    dO * o.  With the exact O that is the same D; with O as stored in a
    narrower format it is the D such a backward forms, and the gradients are
    those of the recomputation given that O.

    Returns (dq, dk, dv, D) with D of shape [B,H,N].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, H, N, d = q.shape
    Nk = k.shape[2]
    sc = _default_scale(d, scale)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    D = np.zeros((B, H, N))
    for b in range(B):
        valid = Nk if kv_len is None else int(kv_len[b])
        for r0 in range(0, N, row_chunk):
            rr = np.arange(r0, min(N, r0 + row_chunk))
            kend = valid
            if causal:
                kend = min(kend, int(rr[-1]) + 1)
            kend = max(kend, 0)
            vis = visible_mask(rr, kend, causal, valid)
            for h in range(H):
                qi = q[b, h, rr]
                kj = k[b, h, :kend]
                vj = v[b, h, :kend]
                doi = do[b, h, rr]
                p, _, _ = _row_softmax(sc * (qi @ kj.T), vis)
                dv[b, h, :kend] += p.T @ doi
                dp = doi @ vj.T
                if o is None:
                    Di = (p * dp).sum(axis=1)
                else:
                    Di = (doi * np.asarray(o[b, h, rr], np.float64)).sum(axis=1)
                ds = p * (dp - Di[:, None])
                dq[b, h, rr] = sc * (ds @ kj)
                dk[b, h, :kend] += sc * (ds.T @ qi)
                D[b, h, rr] = Di
    return dq, dk, dv, D


def k_cache_rows(k_cache):
    """The paged K cache as token rows.

    The library stores each KV head's block of K in groups of 32 head-dim
    elements: entry [physical, head, g, u, j] is element 32*g + j of the
    block's token u (shape [num_blocks, Hkv, d/32, block_size, 32]).  This is
    a storage order of the library, not of the pages, which index a head's
    block by token: the returned array is [num_blocks, Hkv, block_size, d]
    with rows[physical, head, u, 32*g + j] = k_cache[physical, head, g, u, j].
    The V cache is stored by token already.
    """
    k = np.asarray(k_cache)
    nb, hkv, groups, bs, width = k.shape
    if width != 32:
        raise ValueError("K cache groups hold 32 elements")
    return k.transpose(0, 1, 3, 2, 4).reshape(nb, hkv, bs, groups * 32)


def decode_paged(q, k_cache, v_cache, block_table, seq_lens, scale=None):
    """Single-token GQA decode over a paged KV cache, by gather + softmax.

    S12 ("implement it") gives the paged loop: logical block t of a sequence
    lives in physical block block_table[t], and the last block holds only
    n = min(block_size, seq_len - t * block_size) valid slots.  S12's
    production-practice paragraph adds GQA: every query head of a group reads
    the group's shared KV head.  Reading: query head hq uses KV head
    hq // (Hq / Hkv) (consecutive query heads share a KV head).

    q: [B,Hq,d]; v_cache: [num_blocks, Hkv, block_size, d] (the pages index
    one KV head's cache as cache[physical, :n]; with several heads, each
    block keeps its heads one after another); k_cache: the same blocks of K
    in the library's grouped order (``k_cache_rows``);
    block_table: int [B, max_blocks]; seq_lens: int [B].
    The plain definition is applied to the gathered keys: the method's loop is
    in ``online.paged_online``.  A sequence of length 0 gives out = 0.
    Returns out [B,Hq,d] float64.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    k_cache = k_cache_rows(k_cache)
    Hkv = k_cache.shape[1]
    bs = k_cache.shape[2]
    G = Hq // Hkv
    sc = _default_scale(d, scale)
    out = np.zeros((B, Hq, v_cache.shape[3]))
    for b in range(B):
        L = int(seq_lens[b])
        if L <= 0:
            continue
        nblk = -(-L // bs)
        kk, vv = [], []
        for t in range(nblk):
            n = min(bs, L - t * bs)
            phys = int(block_table[b, t])
            kk.append(np.asarray(k_cache[phys, :, :n], dtype=np.float64))
            vv.append(np.asarray(v_cache[phys, :, :n], dtype=np.float64))
        Kb = np.concatenate(kk, axis=1)  # [Hkv, L, d]
        Vb = np.concatenate(vv, axis=1)
        for hq in range(Hq):
            hk = hq // G
            s = sc * (Kb[hk] @ q[b, hq])
            s = s - s.max()
            e = np.exp(s)
            out[b, hq] = (e / e.sum()) @ Vb[hk]
    return out
