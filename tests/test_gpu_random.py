"""GPU parity on randomly drawn shapes (a fixed seed, so every run checks the
same cases): dense forward + backward with causal masks and key padding,
packed varlen forward + backward, block-sparse and dropout forward +
backward, the FP8 forward (within its derived rounding bound), paged GQA
decode over group sizes 1-16 and 1-64 splits, and paged prefill.  Lengths are drawn so that tails are ragged, sequences are empty or
a single token, and some keys collect the dO of many queries.  Each case goes
through the same checks and tolerances as the dedicated tests.

Every backward is also checked on its own: fed the oracle's forward outputs
as they would sit in HBM (O rounded to bf16, m and l in fp32) and compared
with the oracle's backward given that same stored O.  The row term
D = rowsum(dO * O) is formed from the stored O, so against the exact
gradient a backward carries O's rounding through D; when dS = P (dP - D)
nearly cancels (one or two visible keys, or dropout's keep scale magnifying
O) that term is all that is left of dQ and dK.  The end-to-end comparison
(the GPU forward's outputs into the GPU backward, against the exact
gradient) is kept for the dense and varlen kinds.
"""

import numpy as np
import pytest

import oracle
from tests import test_gpu_bwd as tb
from tests import test_gpu_decode as tdec
from tests import test_gpu_fwd as tf
from tests import test_gpu_prefill as tpre
from tests import test_gpu_varlen as tv
from tests import test_gpu_fp8 as t8
from tests import test_gpu_sparse as tsp
from tests.helpers import BF16_TOL, assert_close, stored_forward, to_device
from tests.helpers import to_numpy64
from workloads import TID_DO, normal, normal_fp8, paged_cache

pytestmark = pytest.mark.gpu

KINDS = ("dense", "varlen", "decode", "prefill", "sparse", "dropout", "fp8")
PER_KIND = 10


def _draw(case):
    """The parameters of case `case` (its own generator: cases are
    independent of each other and of the order they run in)."""
    rng = np.random.default_rng([20261202, case])
    kind = KINDS[case % len(KINDS)]
    seed = int(rng.integers(1, 1 << 30))
    d = int(rng.choice([64, 128]))
    causal = bool(rng.integers(0, 2))
    if kind == "dense":
        B, H = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        N = int(rng.integers(1, 700))
        kv = ([int(x) for x in rng.integers(0, N + 1, size=B)]
              if rng.integers(0, 2) else None)
        return kind, dict(B=B, H=H, N=N, d=d, causal=causal, kv=kv, seed=seed)
    if kind == "varlen":
        lens = [int(x) for x in rng.integers(0, 450, size=rng.integers(1, 7))]
        lens[0] = max(lens[0], 1)
        return kind, dict(lens=lens, H=int(rng.integers(1, 4)), d=d,
                          causal=causal, seed=seed)
    if kind == "decode":
        B = int(rng.integers(1, 21))
        return kind, dict(lens=[int(x) for x in rng.integers(0, 1500, size=B)],
                          Hkv=int(rng.choice([1, 2, 4])),
                          G=int(rng.integers(1, 17)), d=d,
                          splits=int(rng.choice([1, 2, 3, 5, 8, 16, 64])),
                          spare=int(rng.integers(0, 3)), seed=seed)
    if kind == "sparse":
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        return kind, dict(B=B, H=H, N=int(rng.integers(1, 900)), d=d,
                          causal=causal, density=float(rng.uniform(0.1, 1)),
                          seed=seed)
    if kind == "dropout":
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        N = int(rng.integers(1, 600))
        kv = ([int(x) for x in rng.integers(0, N + 1, size=B)]
              if rng.integers(0, 2) else None)
        return kind, dict(B=B, H=H, N=N, d=d, causal=causal, kv=kv,
                          p=float(rng.choice([0.05, 0.1, 0.3, 0.5, 0.8])),
                          dseed=int(rng.integers(0, 1 << 63)),
                          off=int(rng.integers(0, 1 << 20)), seed=seed)
    if kind == "fp8":
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        N = int(rng.integers(1, 700))
        kv = ([int(x) for x in rng.integers(1, N + 1, size=B)]
              if rng.integers(0, 2) else None)
        return kind, dict(B=B, H=H, N=N, d=d, causal=causal, kv=kv, seed=seed)
    ctx = [int(x) for x in rng.integers(1, 900, size=rng.integers(1, 5))]
    qlen = [int(rng.integers(0, c + 1)) for c in ctx]
    qlen[0] = max(qlen[0], 1)
    return kind, dict(ctx=ctx, qlen=qlen, Hkv=int(rng.choice([1, 2, 4])),
                      G=int(rng.choice([1, 2, 4])), d=d, causal=causal,
                      seed=seed)


def _grads(name, got, ref):
    for g, r, n in zip(got, ref, ("dq", "dk", "dv")):
        assert_close(f"{name}.{n}", to_numpy64(g), r, BF16_TOL)


def _kv(kv):
    import torch
    return None if kv is None else torch.tensor(kv, dtype=torch.int32,
                                                device="cuda")


def _dense(B, H, N, d, causal, kv, seed):
    import exact_io_aware_15_amd as fa
    q, k, v = (normal((B, H, N, d), seed, t, "bf16") for t in range(3))
    do = normal((B, H, N, d), seed, TID_DO, "bf16")
    tf._check("fwd", q, k, v, causal, kv, BF16_TOL)
    tb._check("bwd", q, k, v, do, causal, kv)
    ro, rm, rl = oracle.attention_fwd(q.exact, k.exact, v.exact, None, causal,
                                      kv)
    o_dev, o_st, m_dev, l_dev = stored_forward(ro, rm, rl)
    g = fa.bwd(to_device(q), to_device(k), to_device(v), o_dev, to_device(do),
               m_dev, l_dev, causal=causal, kv_len=_kv(kv))
    _grads("bwd-stored", g, oracle.attention_bwd(q.exact, k.exact, v.exact,
                                                 do.exact, None, causal, kv,
                                                 o=o_st))


def _varlen(lens, H, d, causal, seed):
    import torch
    import exact_io_aware_15_amd as fa
    cu = tv._cu(lens)
    q, k, v = (normal((H, int(cu[-1]), d), seed, t, "bf16") for t in range(3))
    do = normal((H, int(cu[-1]), d), seed, TID_DO, "bf16")
    tv._check_fwd("varlen", q, k, v, cu, causal, BF16_TOL)
    tv._bwd_case(lens, H, d, causal, seed)
    ro, rm, rl = oracle.attention_fwd_varlen(q.exact, k.exact, v.exact, cu,
                                             None, causal)
    o_dev, o_st, m_dev, l_dev = stored_forward(ro, rm, rl)
    g = fa.bwd_varlen(to_device(q), to_device(k), to_device(v), o_dev,
                      to_device(do), m_dev, l_dev,
                      torch.from_numpy(cu).cuda(), max(1, max(lens)),
                      causal=causal)
    _grads("varlen-stored", g, oracle.attention_bwd_varlen(
        q.exact, k.exact, v.exact, do.exact, cu, None, causal, o=o_st))


def _sparse(B, H, N, d, causal, density, seed):
    import torch
    import exact_io_aware_15_amd as fa
    q, k, v = (normal((B, H, N, d), seed, t, "bf16") for t in range(3))
    do = normal((B, H, N, d), seed, TID_DO, "bf16")
    mask = tsp._mask(H, N, density, seed)
    (o, m, l), _ = tsp._run(q, k, v, mask, causal)
    ro, rm, rl = oracle.attention_fwd_block_sparse(q.exact, k.exact, v.exact,
                                                   mask, 128, None, causal)
    assert_close("sparse.o", o, ro, BF16_TOL)
    vis = np.isfinite(rm)
    assert np.array_equal(np.isfinite(m), vis)
    if vis.any():
        assert np.max(np.abs(m[vis] - rm[vis]) /
                      np.maximum(1, np.abs(rm[vis]))) <= 1e-5
        assert np.max(np.abs(l[vis] / rl[vis] - 1)) <= 2.0 ** -8 + 1e-5
    o_dev, o_st, m_dev, l_dev = stored_forward(ro, rm, rl)
    g = fa.bwd_block_sparse(to_device(q), to_device(k), to_device(v), o_dev,
                            to_device(do), m_dev, l_dev,
                            torch.from_numpy(mask).cuda(), causal=causal)
    _grads("sparse-stored", g, oracle.attention_bwd_block_sparse(
        q.exact, k.exact, v.exact, do.exact, mask, 128, None, causal,
        o=o_st))


def _dropout(B, H, N, d, causal, kv, p, dseed, off, seed):
    import exact_io_aware_15_amd as fa
    q, k, v = (normal((B, H, N, d), seed, t, "bf16") for t in range(3))
    do = normal((B, H, N, d), seed, TID_DO, "bf16")
    qd, kd, vd, dod = (to_device(x) for x in (q, k, v, do))
    o, m, l = fa.fwd_dropout(qd, kd, vd, p, dseed, off, causal=causal,
                             kv_len=_kv(kv))
    o, m, l = (to_numpy64(x) for x in (o, m, l))
    ro, rm, rl = oracle.attention_fwd_dropout(q.exact, k.exact, v.exact, p,
                                              dseed, off, None, causal, kv)
    assert_close("dropout.o", o, ro, BF16_TOL)
    vis = np.isfinite(rm)
    assert np.array_equal(np.isfinite(m), vis)
    if vis.any():
        assert np.max(np.abs(m[vis] - rm[vis]) /
                      np.maximum(1, np.abs(rm[vis]))) <= 1e-5
    o_dev, o_st, m_dev, l_dev = stored_forward(ro, rm, rl)
    g = fa.bwd_dropout(qd, kd, vd, o_dev, dod, m_dev, l_dev, p, dseed, off,
                       causal=causal, kv_len=_kv(kv))
    _grads("dropout-stored", g, oracle.attention_bwd_dropout(
        q.exact, k.exact, v.exact, do.exact, p, dseed, off, None, causal, kv,
        o=o_st))


def _decode(lens, Hkv, G, d, splits, spare, seed):
    mb = max(1, max(-(-L // 16) for L in lens) + spare)
    cache = paged_cache(lens, Hkv, d, 16, mb, seed, poison_tails=True)
    q = normal((len(lens), G * Hkv, d), seed, 0, "bf16")
    assert_close("decode", tdec._run(q, cache, splits), tdec._ref(q, cache),
                 BF16_TOL)


def _prefill(ctx, qlen, Hkv, G, d, causal, seed):
    cu = np.concatenate([[0], np.cumsum(qlen)]).astype(np.int32)
    cache = paged_cache(ctx, Hkv, d, 16, max(-(-c // 16) for c in ctx) + 1,
                        seed, poison_tails=True)
    q = normal((G * Hkv, int(cu[-1]), d), seed, 9, "bf16")
    o, m, l = tpre._gpu(q, cache, cu, causal)
    ro, rm, rl = oracle.prefill_paged(q.exact, cache.k_cache.exact,
                                      cache.v_cache.exact, cache.block_table,
                                      cache.seq_lens, cu, None, causal)
    assert_close("prefill.o", o, ro, BF16_TOL)
    vis = np.isfinite(rm)
    assert np.max(np.abs(m[vis] - rm[vis]) /
                  np.maximum(1, np.abs(rm[vis]))) <= 1e-5
    # l sums bf16-rounded p: at most 2^-8 relative error per term
    assert np.max(np.abs(l[vis] / rl[vis] - 1)) <= 2.0 ** -8 + 1e-5


def _fp8(B, H, N, d, causal, kv, seed):
    shape = (B, H, N, d)
    q, qd = normal_fp8(shape, seed, 0)
    k, kd = normal_fp8(shape, seed, 1)
    v, vd = normal_fp8(shape, seed, 2, transpose=True)
    scale = 1 / np.sqrt(d)
    o, m, l = t8._run(q.store, k.store, v.store, qd, kd, vd, causal, kv,
                      scale)
    ro, rm, rl = oracle.attention_fwd(q.exact, k.exact, v.exact, scale, causal,
                                      kv)
    A = t8._score_mass(q.exact, k.exact, scale, causal, kv, np.arange(N))
    t8._check_stats_model(m, l, rm, rl, A)
    bound, var = t8._fp8_bound(q.exact, k.exact, v.exact, scale, causal, kv,
                               np.arange(N), rm, rl, ro, A)
    err = np.abs(o - ro)
    assert np.all(err <= bound), float(np.max(err / bound))
    assert np.sqrt(np.mean(err ** 2)) <= np.sqrt(np.mean(var))


RUN = {"dense": _dense, "varlen": _varlen, "decode": _decode,
       "prefill": _prefill, "sparse": _sparse, "dropout": _dropout,
       "fp8": _fp8}


@pytest.mark.parametrize("case", range(PER_KIND * len(KINDS)))
def test_random_case(case):
    kind, p = _draw(case)
    print(f"random case {case}: {kind} {p}", flush=True)
    RUN[kind](**p)
