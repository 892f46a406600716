"""Pure-Python scalar attention for tiny inputs (no NumPy arithmetic).

TEST INFRASTRUCTURE ONLY (see the package docstring).

FA notes §2.1 (Algorithm 0) for one head, spelled out with Python floats and
``math.exp`` so that it shares nothing with the vectorised definition it pins:
s_ij = scale * sum_c q_ic k_jc over visible keys, p_ij = exp(s_ij - max_j s_ij)
/ sum_j exp(s_ij - max_j s_ij), o_ic = sum_j p_ij v_jc.  A row with no visible
key gives o = 0.
"""

import math

__all__ = ["brute_fwd"]


def brute_fwd(q, k, v, scale, causal=False, kv_valid=None):
    """q: list of N rows (lists of d floats); k, v: lists of Nk rows.

    Returns o as a list of N rows (lists of floats).
    """
    n_keys = len(k)
    valid = n_keys if kv_valid is None else kv_valid
    out = []
    for i, qi in enumerate(q):
        keys = [j for j in range(n_keys)
                if j < valid and (not causal or j <= i)]
        if not keys:
            out.append([0.0] * len(v[0]))
            continue
        s = {}
        for j in keys:
            acc = 0.0
            for c in range(len(qi)):
                acc += qi[c] * k[j][c]
            s[j] = scale * acc
        mx = max(s.values())
        e = {j: math.exp(s[j] - mx) for j in keys}
        tot = sum(e.values())
        row = []
        for c in range(len(v[0])):
            acc = 0.0
            for j in keys:
                acc += e[j] / tot * v[j][c]
            row.append(acc)
        out.append(row)
    return out
