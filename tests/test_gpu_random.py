"""GPU parity on randomly drawn shapes (a fixed seed, so every run checks the
same cases): dense forward + backward with causal masks and key padding,
packed varlen forward + backward, paged GQA decode over group sizes 1-16 and
1-64 splits, and paged prefill.  Lengths are drawn so that tails are ragged,
sequences are empty or a single token, and some keys collect the dO of many
queries.  Each case goes through the same checks and tolerances as the
dedicated tests.
"""

import numpy as np
import pytest

import oracle
from tests import test_gpu_bwd as tb
from tests import test_gpu_decode as tdec
from tests import test_gpu_fwd as tf
from tests import test_gpu_prefill as tpre
from tests import test_gpu_varlen as tv
from tests.helpers import BF16_TOL, assert_close
from workloads import TID_DO, normal, paged_cache

pytestmark = pytest.mark.gpu

KINDS = ("dense", "varlen", "decode", "prefill")
PER_KIND = 12


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
    ctx = [int(x) for x in rng.integers(1, 900, size=rng.integers(1, 5))]
    qlen = [int(rng.integers(0, c + 1)) for c in ctx]
    qlen[0] = max(qlen[0], 1)
    return kind, dict(ctx=ctx, qlen=qlen, Hkv=int(rng.choice([1, 2, 4])),
                      G=int(rng.choice([1, 2, 4])), d=d, causal=causal,
                      seed=seed)


def _dense(B, H, N, d, causal, kv, seed):
    q, k, v = (normal((B, H, N, d), seed, t, "bf16") for t in range(3))
    do = normal((B, H, N, d), seed, TID_DO, "bf16")
    tf._check("fwd", q, k, v, causal, kv, BF16_TOL)
    tb._check("bwd", q, k, v, do, causal, kv)


def _varlen(lens, H, d, causal, seed):
    cu = tv._cu(lens)
    q, k, v = (normal((H, int(cu[-1]), d), seed, t, "bf16") for t in range(3))
    tv._check_fwd("varlen", q, k, v, cu, causal, BF16_TOL)
    tv._bwd_case(lens, H, d, causal, seed)


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


RUN = {"dense": _dense, "varlen": _varlen, "decode": _decode,
       "prefill": _prefill}


@pytest.mark.parametrize("case", range(PER_KIND * len(KINDS)))
def test_random_case(case):
    kind, p = _draw(case)
    print(f"random case {case}: {kind} {p}", flush=True)
    RUN[kind](**p)
