"""GPU parity of fa_bwd against the fp64 oracle's gradients (through the C ABI).

The GPU backward consumes the GPU forward's O, m and l (as a training step
would); the oracle computes dQ, dK, dV from the exact inputs.  dO is iid
N(0,1) rounded to bf16 for every case.
"""

import numpy as np
import pytest

import oracle
from tests.helpers import BF16_TOL, assert_close, to_device, to_numpy64
from workloads import TID_DO, WORKLOADS, normal

pytestmark = pytest.mark.gpu


def _gpu_grads(q, k, v, do, causal, kv_len):
    import torch
    import exact_io_aware_15_amd as fa
    qd, kd, vd, dod = (to_device(t) for t in (q, k, v, do))
    kl = None if kv_len is None else torch.tensor(kv_len, dtype=torch.int32,
                                                   device="cuda")
    o, m, l = fa.fwd(qd, kd, vd, causal=causal, kv_len=kl)
    dq, dk, dv = fa.bwd(qd, kd, vd, o, dod, m, l, causal=causal, kv_len=kl)
    torch.cuda.synchronize()
    return [to_numpy64(x) for x in (dq, dk, dv)]


def _check(name, q, k, v, do, causal, kv_len, heads=None):
    dq, dk, dv = _gpu_grads(q, k, v, do, causal, kv_len)
    ex = [t.exact for t in (q, k, v, do)]
    if heads is not None:   # the oracle on a subset of heads
        ex = [x[:, heads] for x in ex]
        dq, dk, dv = dq[:, heads], dk[:, heads], dv[:, heads]
    rq, rk, rv, _ = oracle.attention_bwd(*ex, None, causal, kv_len)
    assert_close(name + ".dq", dq, rq, BF16_TOL)
    assert_close(name + ".dk", dk, rk, BF16_TOL)
    assert_close(name + ".dv", dv, rv, BF16_TOL)
    if kv_len is not None:
        for b, L in enumerate(kv_len):
            assert np.all(dk[b, :, L:] == 0) and np.all(dv[b, :, L:] == 0)


SMALL = [  # (B, H, N, d, causal, padded)
    (1, 1, 1, 64, False, False),
    (1, 2, 32, 64, True, False),
    (2, 2, 200, 64, False, False),
    (2, 2, 200, 64, True, False),
    (3, 2, 333, 64, False, True),
    (3, 2, 333, 64, True, True),
    (2, 1, 160, 128, False, False),
    (2, 1, 161, 128, True, True),
]


@pytest.mark.parametrize("B,H,N,d,causal,padded", SMALL)
def test_bwd_small(B, H, N, d, causal, padded):
    seed = 2000 + N + d + 7 * causal + 3 * padded
    q, k, v = (normal((B, H, N, d), seed, t, "bf16") for t in range(3))
    do = normal((B, H, N, d), seed, TID_DO, "bf16")
    kv_len = None
    if padded:
        kv_len = [int(x) for x in
                  np.random.default_rng(seed).integers(1, N + 1, size=B)]
        kv_len[0] = N
    print(f"bwd B={B} H={H} N={N} d={d} causal={causal} kv={kv_len}",
          flush=True)
    _check("small", q, k, v, do, causal, kv_len)


# Few valid keys under many queries: each such key collects the dO of
# hundreds of queries, so dK and dV reach magnitudes of 5-10, where bf16
# rounding (of P, dS and the outputs) alone exceeds 2e-2 absolute; the
# tolerance floor of one unit in the last place of the largest value
# applies (see tests/helpers.py).  Shapes found by a randomized sweep.
LARGE = [  # (B, H, N, d, causal, kv_len, seed)
    (3, 1, 508, 64, False, [6, 379, 317], 550717758),
    (3, 1, 99, 128, True, [2, 41, 80], 794539958),
    (1, 1, 558, 64, True, [16], 764689141),
    (3, 2, 188, 128, True, [62, 38, 5], 512586306),
]


@pytest.mark.parametrize("B,H,N,d,causal,kv_len,seed", LARGE)
def test_bwd_large_gradients(B, H, N, d, causal, kv_len, seed):
    q, k, v = (normal((B, H, N, d), seed, t, "bf16") for t in range(3))
    do = normal((B, H, N, d), seed, TID_DO, "bf16")
    print(f"bwd large B={B} H={H} N={N} d={d} causal={causal} kv={kv_len}",
          flush=True)
    _check("large", q, k, v, do, causal, kv_len)


def test_bwd_zero_length_sequence():
    q, k, v = (normal((2, 1, 96, 64), 81, t, "bf16") for t in range(3))
    do = normal((2, 1, 96, 64), 81, TID_DO, "bf16")
    print("bwd kv_len=0", flush=True)
    dq, dk, dv = _gpu_grads(q, k, v, do, False, [0, 96])
    assert np.all(dq[0] == 0) and np.all(dk[0] == 0) and np.all(dv[0] == 0)


@pytest.mark.parametrize("name", ["bert_large_padded", "gpt2_medium_causal_1k"])
def test_bwd_workload_full(name):
    w = WORKLOADS[name]
    q, k, v = w.qkv()
    do = w.dout()
    kv_len = w.kv_len()
    kv_len = None if kv_len is None else [int(x) for x in kv_len]
    print(f"bwd workload {name} (full)", flush=True)
    _check(name, q, k, v, do, w.causal, kv_len)


def test_bwd_workload_4k_sampled_heads():
    w = WORKLOADS["gpt2_medium_causal_4k"]
    q, k, v = w.qkv()
    do = w.dout()
    print("bwd workload gpt2_medium_causal_4k (heads 0, 9)", flush=True)
    _check(w.name, q, k, v, do, True, None, heads=[0, 9])


def test_bwd_is_bitwise_deterministic():
    """No atomics anywhere in the backward: two runs agree bit for bit."""
    import torch
    import exact_io_aware_15_amd as fa
    q, k, v = (to_device(normal((2, 3, 300, 64), 82, t, "bf16"))
               for t in range(3))
    do = to_device(normal((2, 3, 300, 64), 82, TID_DO, "bf16"))
    o, m, l = fa.fwd(q, k, v, causal=True)
    a = fa.bwd(q, k, v, o, do, m, l, causal=True)
    b = fa.bwd(q, k, v, o, do, m, l, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_masked_keys_never_read_into_arithmetic():
    """Keys past kv_len hold NaN in K and V: dq equals the clean run's, and
    dk, dv are exactly zero there."""
    import torch
    import exact_io_aware_15_amd as fa
    q, k, v = (to_device(normal((2, 2, 260, 64), 83, t, "bf16"))
               for t in range(3))
    do = to_device(normal((2, 2, 260, 64), 83, TID_DO, "bf16"))
    kl = torch.tensor([130, 211], dtype=torch.int32, device="cuda")
    o, m, l = fa.fwd(q, k, v, kv_len=kl)
    g1 = fa.bwd(q, k, v, o, do, m, l, kv_len=kl)
    kp, vp = k.clone(), v.clone()
    for b, L in enumerate([130, 211]):
        kp[b, :, L:] = float("nan")
        vp[b, :, L:] = float("nan")
    g2 = fa.bwd(q, kp, vp, o, do, m, l, kv_len=kl)
    torch.cuda.synchronize()
    assert torch.equal(g1[0], g2[0])
    for b, L in enumerate([130, 211]):
        assert torch.all(g2[1][b, :, L:] == 0) and torch.all(g2[2][b, :, L:] == 0)
        assert torch.equal(g1[1][b, :, :L], g2[1][b, :, :L])
        assert torch.equal(g1[2][b, :, :L], g2[2][b, :, :L])
