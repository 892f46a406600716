"""GPU parity of fa_fwd_dropout / fa_bwd_dropout against the fp64 dropout
oracle.

Three structured problems expose the keep mask of every kernel exactly.
With zero scores each row's probabilities are uniform, and one-hot rows of
weight 2^(index // d) in V, dO, K or Q turn the outputs into sums of distinct
powers of two of the keep bits:

* O and dV read the mask of the forward kernel and of the key-stationary
  kernel's P path;
* dQ reads it in the query-stationary backward kernel's dS path;
* dK reads it in the key-stationary kernel's dS path.

Each element is compared with the oracle to a quarter of its smallest bit
weight, so a single wrong keep decision fails.  Random inputs are then
compared at the bf16 tolerance: ragged lengths, causal, key padding with an
empty row, d = 64 and 128.  p = 0 must give fa_fwd / fa_bwd bit for bit, and
the 4K workload is compared on sampled rows."""

import math

import numpy as np
import pytest

import oracle
from tests.helpers import BF16_TOL, assert_close, to_device, to_numpy64
from workloads import TID_DO, WORKLOADS, normal

pytestmark = pytest.mark.gpu

SEED = 0x9E37_79B9_7F4A_7C15     # both 32-bit halves in use
P_DROP = 0.3


def _bf16(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).cuda()


def _weighted_one_hot(B, H, N, d):
    """Row i = 2^(i // d) e_(i % d): distinct powers of two per column."""
    x = np.zeros((B, H, N, d))
    i = np.arange(N)
    x[:, :, i, i % d] = 2.0 ** (i // d)
    return x


def _e0(B, H, N, d):
    x = np.zeros((B, H, N, d))
    x[..., 0] = 1.0
    return x


def _run(q, k, v, do, causal, kv_len=None, p=P_DROP, seed=SEED, offset=5):
    import torch
    import exact_io_aware_15_amd as fa
    qd, kd, vd, dod = (_bf16(x) for x in (q, k, v, do))
    o, m, l = fa.fwd_dropout(qd, kd, vd, p, seed, offset, causal=causal,
                             kv_len=kv_len)
    g = fa.bwd_dropout(qd, kd, vd, o, dod, m, l, p, seed, offset,
                       causal=causal, kv_len=kv_len)
    torch.cuda.synchronize()
    return [to_numpy64(x) for x in (o, m, l)], [to_numpy64(x) for x in g]


def _keep_scale(p=P_DROP):
    return oracle.dropout_threshold(p)[1]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_mask_exposed_in_o_and_dv(d, causal):
    B, H, N = 2, 3, 4 * d
    print(f"dropout mask via O/dV d={d} causal={causal}", flush=True)
    q = k = np.zeros((B, H, N, d))
    v = _weighted_one_hot(B, H, N, d)
    do = _weighted_one_hot(B, H, N, d)
    (o, _, _), (dq, dk, dv) = _run(q, k, v, do, causal)
    ro, _, _ = oracle.attention_fwd_dropout(q, k, v, P_DROP, SEED, 5, None,
                                            causal)
    s = _keep_scale()
    n_i = (np.arange(N) + 1.0) if causal else np.full(N, float(N))
    unit = (s / n_i)[None, None, :, None]          # weight of one keep bit
    assert np.all(np.abs(o - ro) <= 0.25 * unit)
    assert np.all(dq == 0) and np.all(dk == 0)     # q = k = 0
    if not causal:  # uniform P: each dV element is a sum of distinct bits
        _, _, rv, _ = oracle.attention_bwd_dropout(q, k, v, do, P_DROP, SEED,
                                                   5, None, causal)
        assert np.all(np.abs(dv - rv) <= 0.25 * s / N)


@pytest.mark.parametrize("d", [64, 128])
def test_mask_exposed_in_dq(d):
    # Q = 0 (uniform P), K one-hot weighted, V = dO = e_0 (dO V^T = 1).
    B, H, N = 1, 2, 4 * d
    print(f"dropout mask via dQ d={d}", flush=True)
    q = np.zeros((B, H, N, d))
    k = _weighted_one_hot(B, H, N, d)
    v = do = _e0(B, H, N, d)
    _, (dq, dk, dv) = _run(q, k, v, do, False)
    rq, _, rv, _ = oracle.attention_bwd_dropout(q, k, v, do, P_DROP, SEED, 5,
                                                None, False)
    sc = 1 / math.sqrt(d)
    assert np.all(np.abs(dq - rq) <= 0.25 * sc * _keep_scale() / N)
    assert np.all(dk == 0)
    assert_close("dv", dv, rv, BF16_TOL)


@pytest.mark.parametrize("d", [64, 128])
def test_mask_exposed_in_dk(d):
    # K = 0 (uniform P), Q one-hot weighted, V = dO = e_0.
    B, H, N = 1, 2, 4 * d
    print(f"dropout mask via dK d={d}", flush=True)
    q = _weighted_one_hot(B, H, N, d)
    k = np.zeros((B, H, N, d))
    v = do = _e0(B, H, N, d)
    _, (dq, dk, dv) = _run(q, k, v, do, False)
    _, rk, _, _ = oracle.attention_bwd_dropout(q, k, v, do, P_DROP, SEED, 5,
                                               None, False)
    sc = 1 / math.sqrt(d)
    assert np.all(np.abs(dk - rk) <= 0.25 * sc * _keep_scale() / N)
    assert np.all(dq == 0)


CASES = [  # (B, H, N, d, causal, kv_len, p)
    (2, 3, 300, 64, False, None, 0.1),
    (1, 2, 517, 64, True, None, 0.25),
    (2, 2, 384, 128, True, [384, 200], 0.5),
    (2, 2, 250, 128, False, [250, 0], 0.1),
    (1, 1, 77, 64, True, [60], 0.5),
    (1, 2, 1, 64, False, None, 0.5),      # one query, one key
    (1, 1, 17, 128, True, None, 0.3),     # shorter than one tile
]


@pytest.mark.parametrize("B,H,N,d,causal,kv_len,p", CASES)
def test_dropout_fwd_bwd_random(B, H, N, d, causal, kv_len, p):
    seed = 7000 + N + d
    q, k, v = (normal((B, H, N, d), seed, t, "bf16") for t in range(3))
    do = normal((B, H, N, d), seed, TID_DO, "bf16")
    print(f"dropout B={B} H={H} N={N} d={d} causal={causal} kv_len={kv_len} "
          f"p={p}", flush=True)
    import torch
    import exact_io_aware_15_amd as fa
    kvl = None if kv_len is None else torch.tensor(kv_len, dtype=torch.int32,
                                                   device="cuda")
    qd, kd, vd, dod = (to_device(x) for x in (q, k, v, do))
    o, m, l = fa.fwd_dropout(qd, kd, vd, p, seed, 3, causal=causal,
                             kv_len=kvl)
    dq, dk, dv = fa.bwd_dropout(qd, kd, vd, o, dod, m, l, p, seed, 3,
                                causal=causal, kv_len=kvl)
    torch.cuda.synchronize()
    o, m, l, dq, dk, dv = (to_numpy64(x) for x in (o, m, l, dq, dk, dv))
    ro, rm, rl = oracle.attention_fwd_dropout(q.exact, k.exact, v.exact, p,
                                              seed, 3, None, causal, kv_len)
    assert_close("o", o, ro, BF16_TOL)
    vis = np.isfinite(rm)
    assert np.array_equal(np.isfinite(m), vis)
    assert np.max(np.abs(m[vis] - rm[vis]) / np.maximum(1, np.abs(rm[vis]))) \
        <= 1e-5
    assert np.max(np.abs(l[vis] - rl[vis]) / rl[vis]) <= 1e-2
    assert np.all(o[~vis] == 0)
    rq, rk, rv, _ = oracle.attention_bwd_dropout(
        q.exact, k.exact, v.exact, do.exact, p, seed, 3, None, causal, kv_len)
    assert_close("dq", dq, rq, BF16_TOL)
    assert_close("dk", dk, rk, BF16_TOL)
    assert_close("dv", dv, rv, BF16_TOL)


def test_zero_drop_matches_plain_kernels_bitwise():
    import torch
    import exact_io_aware_15_amd as fa
    q, k, v, do = (to_device(normal((2, 2, 333, 64), 7100, t, "bf16"))
                   for t in (0, 1, 2, TID_DO))
    for causal in (False, True):
        o, m, l = fa.fwd(q, k, v, causal=causal)
        od, md, ld = fa.fwd_dropout(q, k, v, 0.0, 123, 0, causal=causal)
        g = fa.bwd(q, k, v, o, do, m, l, causal=causal)
        gd = fa.bwd_dropout(q, k, v, o, do, m, l, 0.0, 123, 0, causal=causal)
        torch.cuda.synchronize()
        for a, b in zip((o, m, l) + tuple(g), (od, md, ld) + tuple(gd)):
            assert torch.equal(a, b)


def test_mask_is_deterministic_and_keyed():
    import torch
    import exact_io_aware_15_amd as fa
    q, k, v = (to_device(normal((1, 2, 256, 64), 7200, t, "bf16"))
               for t in range(3))
    a = fa.fwd_dropout(q, k, v, 0.2, 99, 0)[0]
    b = fa.fwd_dropout(q, k, v, 0.2, 99, 0)[0]
    c = fa.fwd_dropout(q, k, v, 0.2, 99, 1)[0]
    d = fa.fwd_dropout(q, k, v, 0.2, 99 + (1 << 32), 0)[0]
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert not torch.equal(a, c) and not torch.equal(a, d)


def test_gpt2_medium_4k_sampled_rows():
    """The 4K causal GPT-2-medium workload with p = 0.1, forward compared on
    sampled rows of every head (first, last, tile edges, random)."""
    import torch
    import exact_io_aware_15_amd as fa
    w = WORKLOADS["gpt2_medium_causal_4k"]
    q, k, v = w.qkv()
    print(f"dropout {w.name} sampled rows", flush=True)
    qd, kd, vd = (to_device(x) for x in (q, k, v))
    o, m, l = fa.fwd_dropout(qd, kd, vd, 0.1, 2024, 1, causal=w.causal)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7300)
    N = w.N
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, N - 1],
                                     rng.integers(0, N, 9)]))
    ro, rm, rl = oracle.attention_fwd_dropout(q.exact, k.exact, v.exact, 0.1,
                                              2024, 1, None, w.causal,
                                              rows=rows)
    assert_close("o rows", to_numpy64(o)[:, :, rows], ro, BF16_TOL)
    assert np.max(np.abs(to_numpy64(m)[:, :, rows] - rm)) <= 1e-4
