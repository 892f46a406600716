"""GPU parity of fa_fwd against the fp64 oracle (through the C ABI).

Sizes: small shapes that span several 128-query / 64-key tiles with ragged
tails (full comparison), the BERT-large-shaped and GPT-2-medium-shaped
workloads in full, and the long-context workloads on sampled query rows (the
oracle computes a row from that row alone).
"""

import numpy as np
import pytest

import oracle
from tests.helpers import BF16_TOL, F32_TOL, assert_close, to_device, to_numpy64
from workloads import WORKLOADS, Workload, normal

pytestmark = pytest.mark.gpu


def _run(q, k, v, causal, kv_len):
    import torch
    import exact_io_aware_15_amd as fa
    kl = None if kv_len is None else torch.tensor(kv_len, dtype=torch.int32,
                                                   device="cuda")
    o, m, l = fa.fwd(to_device(q), to_device(k), to_device(v), causal=causal,
                     kv_len=kl)
    torch.cuda.synchronize()
    return to_numpy64(o), to_numpy64(m), to_numpy64(l)


def _check(name, q, k, v, causal, kv_len, tol, rows=None, l_rel=None):
    o, m, l = _run(q, k, v, causal, kv_len)
    ro, rm, rl = oracle.attention_fwd(q.exact, k.exact, v.exact, None, causal,
                                      kv_len, rows=rows)
    if rows is not None:
        o, m, l = o[:, :, rows], m[:, :, rows], l[:, :, rows]
    assert_close(name + ".o", o, ro, tol)
    vis = np.isfinite(rm)
    assert np.array_equal(np.isfinite(m), vis), name + ".m finiteness"
    if not vis.any():   # every key masked: nothing but zeros to check
        assert np.all(l == 0) and np.all(o == 0)
        return o
    assert np.max(np.abs(m[vis] - rm[vis]) / np.maximum(1, np.abs(rm[vis]))) \
        <= 1e-5, name + ".m"
    # l is summed from the bf16-rounded p that feeds the P V product.  bf16
    # keeps 8 significant bits, so round-to-nearest changes a term by at most
    # half a unit in its last place, 2^-8 of the term: |l_gpu / l - 1| <=
    # 2^-8, plus fp32 accumulation.
    lr = l_rel if l_rel is not None else 2.0 ** -8 + 1e-5
    assert np.max(np.abs(l[vis] / rl[vis] - 1)) <= lr, name + ".l"
    assert np.all(l[~vis] == 0) and np.all(o[~vis] == 0)
    return o


SMALL = [  # (B, H, N, d, causal, padded)
    (1, 1, 1, 64, False, False),
    (1, 2, 64, 64, True, False),
    (2, 3, 333, 64, False, False),
    (2, 3, 333, 64, True, False),
    (3, 2, 333, 64, False, True),
    (3, 2, 333, 64, True, True),
    (2, 2, 200, 128, False, False),
    (2, 2, 257, 128, True, True),
    # causal d = 64 edge shapes: one query (one tile, one key), a ragged
    # second query tile, an odd number of query tiles, padding
    (1, 1, 1, 64, True, False),
    (1, 2, 129, 64, True, False),
    (2, 1, 640, 64, True, True),
    (1, 3, 1000, 64, True, False),
]


@pytest.mark.parametrize("B,H,N,d,causal,padded", SMALL)
def test_fwd_bf16_small(B, H, N, d, causal, padded):
    seed = 1000 + N + d + 7 * causal + 3 * padded
    q, k, v = (normal((B, H, N, d), seed, t, "bf16") for t in range(3))
    kv_len = None
    if padded:
        kv_len = list(np.random.default_rng(seed).integers(1, N + 1, size=B))
        kv_len[0] = N
    print(f"fwd bf16 B={B} H={H} N={N} d={d} causal={causal} kv={kv_len}",
          flush=True)
    _check("small", q, k, v, causal, kv_len, BF16_TOL)


@pytest.mark.parametrize("causal,kv_len", [(False, None), (True, None),
                                           (False, [100]), (True, [7])])
def test_fwd_f32_tiny_workload(causal, kv_len):
    w = WORKLOADS["tiny_f32"]
    q, k, v = w.qkv()
    print(f"fwd f32 tiny causal={causal} kv={kv_len}", flush=True)
    _check("tiny_f32", q, k, v, causal, kv_len, F32_TOL, l_rel=1e-5)


def test_fwd_zero_length_rows_are_zero():
    q, k, v = (normal((2, 1, 70, 64), 77, t, "bf16") for t in range(3))
    print("fwd kv_len=0", flush=True)
    o, m, l = _run(q, k, v, False, [0, 70])
    assert np.all(o[0] == 0) and np.all(l[0] == 0) and np.all(np.isneginf(m[0]))
    ro, _, _ = oracle.attention_fwd(q.exact[1:], k.exact[1:], v.exact[1:])
    assert_close("kv0.o", o[1:], ro, BF16_TOL)


def test_fwd_every_key_masked():
    """kv_len = 0 for every sequence: all rows are empty (o = 0, l = 0)."""
    q, k, v = (normal((2, 2, 130, 128), 79, t, "bf16") for t in range(3))
    print("fwd kv_len all 0", flush=True)
    _check("allmasked", q, k, v, True, [0, 0], BF16_TOL)


def test_fwd_masked_keys_never_read_into_arithmetic():
    """Keys past kv_len hold NaN: the output must equal the clean run."""
    import torch
    import exact_io_aware_15_amd as fa
    q, k, v = (normal((2, 2, 300, 64), 78, t, "bf16") for t in range(3))
    kv_len = [150, 211]
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    kl = torch.tensor(kv_len, dtype=torch.int32, device="cuda")
    o1, _, _ = fa.fwd(qd, kd, vd, kv_len=kl)
    kp, vp = kd.clone(), vd.clone()
    for b, L in enumerate(kv_len):
        kp[b, :, L:] = float("nan")
        vp[b, :, L:] = float("nan")
    o2, _, _ = fa.fwd(qd, kp, vp, kv_len=kl)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_fwd_constant_values_and_determinism():
    import torch
    import exact_io_aware_15_amd as fa
    q, k = (normal((1, 4, 500, 64), 79, t, "bf16", 3.0) for t in range(2))
    qd, kd = to_device(q), to_device(k)
    vd = torch.full((1, 4, 500, 64), 0.375, dtype=torch.bfloat16,
                    device="cuda")
    for causal in (False, True):
        o, _, _ = fa.fwd(qd, kd, vd, causal=causal)
        # rows of bf16-rounded P are summed from the same rounded values, so
        # a constant V comes back to fp32 rounding, then bf16 rounding
        assert torch.all(o == 0.375), causal
    v = to_device(normal((1, 4, 500, 64), 80, 2, "bf16"))
    a, ma, la = fa.fwd(qd, kd, v, causal=True)
    b, mb, lb = fa.fwd(qd, kd, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(ma, mb) and torch.equal(la, lb)


@pytest.mark.parametrize("name", ["bert_large_padded", "gpt2_medium_causal_1k"])
def test_fwd_workload_full(name):
    w = WORKLOADS[name]
    q, k, v = w.qkv()
    kv_len = w.kv_len()
    kv_len = None if kv_len is None else [int(x) for x in kv_len]
    print(f"fwd workload {name} (full)", flush=True)
    _check(name, q, k, v, w.causal, kv_len, BF16_TOL)


@pytest.mark.parametrize("name", ["gpt2_medium_causal_4k",
                                  "long_causal_16k_d128",
                                  "long_causal_64k_d64"])
def test_fwd_workload_sampled_rows(name):
    w = WORKLOADS[name]
    q, k, v = w.qkv()
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([
        [0, 1, 63, 64, 127, 128, w.N - 129, w.N - 128, w.N - 2, w.N - 1],
        rng.integers(0, w.N, size=22)]))
    print(f"fwd workload {name} (rows {rows.size})", flush=True)
    _check(name, q, k, v, w.causal, None, BF16_TOL, rows=rows)


# Long d = 64 rows with ragged tails (N not a multiple of the 128-query or
# 64-key tile), padded and not, causal and not, on sampled rows: a partial
# last query tile, a partial last key tile, and key padding that ends inside
# a tile, all at lengths where the causal deal order reverses whole rounds.
@pytest.mark.parametrize("N,causal,kv_len", [
    (8192, True, [8192, 5000]),
    (8193, True, None),
    (8257, False, [8257, 7000]),
    (8257, True, [3000, 8200]),
])
def test_fwd_d64_long_rows_ragged_tails_and_padding(N, causal, kv_len):
    B, H, d = 2, 1, 64
    q, k, v = (normal((B, H, N, d), 9600 + N, t, "bf16") for t in range(3))
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 2999, 3000, 4999, 5000,
                                      N - 65, N - 64, N - 1],
                                     np.random.default_rng(N).integers(
                                         0, N, size=12)]))
    print(f"fwd d=64 N={N} causal={causal} kv_len={kv_len}", flush=True)
    _check(f"occ N={N}", q, k, v, causal, kv_len, BF16_TOL, rows=rows)
