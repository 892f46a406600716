"""Attention with dropout on the probability matrix, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

FA notes §2.1 names dropout on the probabilities as one of the memory-bound
element-wise steps of standard attention, and FA notes §3.4 lists it among
the operations the fused kernel performs on chip (matmul, mask, softmax,
dropout, matmul), so the dropped matrix never reaches HBM.  The pages fix
neither the random generator nor how the backward pass sees the same mask.
Readings (each is listed in the design notes):

* Generator: Philox4x32-10, the counter-based generator of Salmon, Moraes,
  Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC 2011),
  written here from that definition.  A counter-based generator lets any
  pass regenerate the keep decision of element (i, j) from its coordinates
  alone, which is what recomputation in the backward pass (FA notes §3.3)
  needs.
* Stream layout: one Philox call per (query row, group of 16 keys) yields 16
  random bytes.  For head bh = b*H + h, query i and key j:
      group  g(j) = 2*(j // 32) + (j // 8) % 2
      byte   t(j) = 8*((j // 16) % 2) + j % 8
      counter = (i, g(j), bh, offset),  key = (seed mod 2^32, seed >> 32)
  byte t is bits 8*(t%4) .. 8*(t%4)+7 of output word t // 4.
* Keep rule: with T = round(256 p) (halves up), element (i, j) is kept iff
  its byte >= T, so the keep probability is exactly (256 - T)/256; kept
  probabilities are multiplied by 256/(256 - T) (inverted dropout, so the
  expectation of the output is the attention output).  T must be <= 255.
* The statistics m, l are those of the softmax before dropout; dropout
  multiplies P element-wise after normalisation:
      O = (P * Z * s) V,  Z = keep mask,  s = 256/(256 - T).
"""

from fractions import Fraction

import numpy as np

from .reference import _default_scale, _row_softmax, visible_mask

__all__ = [
    "philox4x32_10",
    "dropout_threshold",
    "dropout_keep",
    "attention_fwd_dropout",
    "attention_bwd_dropout",
]

# Philox4x32 constants (Salmon et al., SC 2011, the Philox section): the two
# round multipliers and the two Weyl key increments.
_M0, _M1 = 0xD2511F53, 0xCD9E8D57
_W0, _W1 = 0x9E3779B9, 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(counter, key):
    """Philox4x32 with 10 rounds on arrays of 32-bit words.

    counter: uint-like array [..., 4]; key: array [..., 2] broadcastable to
    it.  Each round multiplies words 0 and 2 by the two constants, splits each
    64-bit product into (hi, lo), and forms the new state
        (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0));
    the key is advanced by the Weyl increments between rounds.  Returns the
    four output words as uint64 values below 2^32, shape [..., 4].
    """
    c = np.asarray(counter, dtype=np.uint64) & _MASK32
    k = np.asarray(key, dtype=np.uint64) & _MASK32
    c0, c1, c2, c3 = (c[..., n] for n in range(4))
    k0 = np.broadcast_to(k[..., 0], c0.shape).copy()
    k1 = np.broadcast_to(k[..., 1], c0.shape).copy()
    m0, m1 = np.uint64(_M0), np.uint64(_M1)
    for _ in range(10):
        p0 = m0 * c0            # < 2^64: exact in uint64
        p1 = m1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
        k0 = (k0 + np.uint64(_W0)) & _MASK32
        k1 = (k1 + np.uint64(_W1)) & _MASK32
    return np.stack([c0, c1, c2, c3], axis=-1)


def dropout_threshold(p_drop):
    """Byte threshold T = floor(256 p + 1/2) of a float32 drop probability.

    Computed exactly (the float32 value of p as a rational), so it does not
    depend on any rounding.  Raises ValueError unless 0 <= p and T <= 255.
    Returns (T, keep_scale) with keep_scale = 256 / (256 - T).
    """
    pf = Fraction(float(np.float32(p_drop)))
    if pf < 0:
        raise ValueError("drop probability must be >= 0")
    t = int((pf * 256 + Fraction(1, 2)).__floor__())
    if t > 255:
        raise ValueError("drop probability rounds to 256/256")
    return t, 256.0 / (256 - t)


def _group_byte(j):
    j = np.asarray(j, dtype=np.int64)
    g = 2 * (j // 32) + (j // 8) % 2
    t = 8 * ((j // 16) % 2) + j % 8
    return g, t


def dropout_keep(bh, rows, n_keys, seed, offset, threshold):
    """Boolean [len(rows), n_keys]: keep decision of (row i, key j) of head bh.

    bh = b*H + h; seed is a 64-bit integer, offset a 32-bit one.  Follows the
    stream layout and keep rule stated in the module docstring.
    """
    rows = np.asarray(rows, dtype=np.int64)
    j = np.arange(n_keys)
    g, t = _group_byte(j)
    ng = int(g.max()) + 1 if n_keys else 0
    seed = int(seed)
    key = np.array([seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], np.uint64)
    ctr = np.zeros((rows.size, ng, 4), np.uint64)
    ctr[..., 0] = rows[:, None]
    ctr[..., 1] = np.arange(ng)[None, :]
    ctr[..., 2] = int(bh)
    ctr[..., 3] = int(offset) & 0xFFFFFFFF
    words = philox4x32_10(ctr, key)                      # [R, ng, 4]
    shifts = np.uint64(8) * (np.arange(16, dtype=np.uint64) % np.uint64(4))
    byts = (words[..., np.arange(16) // 4] >> shifts) & np.uint64(0xFF)
    return byts[:, g, t] >= np.uint64(threshold)         # [R, n_keys]


def attention_fwd_dropout(q, k, v, p_drop, seed, offset=0, scale=None,
                          causal=False, kv_len=None, rows=None,
                          row_chunk=512):
    """Attention forward with dropout on P (FA notes §2.1 / §3.4), float64.

    q, k, v: [B,H,N,d]; masking as in reference.attention_fwd.  rows: None
    for every query row, or the row indices to compute (a row's result
    depends on that row alone).  Returns (o, m, l) over those rows:
    o = (P * Z * s) V with the mask Z of dropout_keep, and the pre-dropout
    softmax statistics m, l.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, d = q.shape
    sc = _default_scale(d, scale)
    T, ks = dropout_threshold(p_drop)
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.size
    o = np.zeros((B, H, R, v.shape[3]))
    m = np.full((B, H, R), -np.inf)
    l = np.zeros((B, H, R))
    for b in range(B):
        valid = N if kv_len is None else int(kv_len[b])
        for r0 in range(0, R, row_chunk):
            rr = rows[r0:r0 + row_chunk]
            out = slice(r0, r0 + rr.size)
            vis = visible_mask(rr, N, causal, valid)
            for h in range(H):
                p, mm, ll = _row_softmax(sc * (q[b, h, rr] @ k[b, h].T), vis)
                z = dropout_keep(b * H + h, rr, N, seed, offset, T)
                o[b, h, out] = (p * z * ks) @ v[b, h]
                m[b, h, out] = mm
                l[b, h, out] = ll
    return o, m, l


def attention_bwd_dropout(q, k, v, do, p_drop, seed, offset=0, scale=None,
                          causal=False, kv_len=None, row_chunk=512, o=None):
    """Gradients of L = sum(dO * O) for O = attention_fwd_dropout(...).

    The chain rule with the mask Z held fixed (the pages print no backward
    formulas; the mask is regenerated, not stored, per FA notes §3.3):

        A  = P * Z * s                   (dropped probabilities)
        dV = A^T dO
        dA = dO V^T
        dP = dA * Z * s
        D_i = sum_j P_ij dP_ij           (equals sum_c dO_ic O_ic)
        dS = P * (dP - D)
        dQ = scale * dS K,   dK = scale * dS^T Q

    o: None, or the stored forward output [B,H,N,d] that the backward reads
    (FA notes §3.3 keeps O and (m, l) in HBM for the backward): then
    D_i = sum_c dO_ic o_ic from it.  With the exact O this is the same D;
    with O as stored in a narrower format it is the D such a backward forms,
    and the gradients are those of the recomputation given that O.

    Returns (dq, dk, dv, D).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, H, N, d = q.shape
    sc = _default_scale(d, scale)
    T, ks = dropout_threshold(p_drop)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    D = np.zeros((B, H, N))
    for b in range(B):
        valid = N if kv_len is None else int(kv_len[b])
        for r0 in range(0, N, row_chunk):
            rr = np.arange(r0, min(N, r0 + row_chunk))
            vis = visible_mask(rr, N, causal, valid)
            for h in range(H):
                qi, doi = q[b, h, rr], do[b, h, rr]
                p, _, _ = _row_softmax(sc * (qi @ k[b, h].T), vis)
                z = dropout_keep(b * H + h, rr, N, seed, offset, T) * ks
                dv[b, h] += (p * z).T @ doi
                dp = (doi @ v[b, h].T) * z
                if o is None:
                    Di = (p * dp).sum(axis=1)
                else:
                    Di = (doi * np.asarray(o[b, h, rr], np.float64)).sum(axis=1)
                ds = p * (dp - Di[:, None])
                dq[b, h, rr] = sc * (ds @ k[b, h])
                dk[b, h] += sc * (ds.T @ qi)
                D[b, h, rr] = Di
    return dq, dk, dv, D
