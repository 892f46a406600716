"""GPU parity of fa_fwd_fp8 against the fp64 oracle on the dequantised
inputs (code * descale): the oracle is plain attention (FA notes §2.1) on
exactly the values the kernel multiplies.

The kernel rounds each probability to E4M3 before the P V product, so the
tolerance is derived from that rounding rather than fixed:

* Exact case.  With integer raw scores and the score scale chosen so that
  c = scale * q_descale * k_descale * log2(e) = 1, every probability the
  kernel forms is a power of two inside E4M3's range, so rounding is exact and
  O must equal the oracle up to the bf16 output rounding (2^-8 relative).
  This pins every index: tile layout, key order, both operand layouts, masks,
  descales.
* Random case.  Probability j of row i carries an absolute error of at most
  max(2^-4 P_ij, 2^-10 / (2^6 l_i)) (half an E4M3 step: relative 2^-4 for
  normal values, 2^-10 in the kernel's 2^6-shifted units for subnormals,
  with l_i = sum_j exp(S_ij - m_i) >= 1), so
      |O_ic - ref_ic| <= sum_j max(2^-4 P_ij, 2^-16 / l_i) |V_jc|
                         + 2^-8 |ref_ic| (bf16 output) + 1e-6,
  and, the roundings being independent and at most that size, the RMS error
  over all elements stays within that of uniform errors of the same bounds.
* The FP8 matrix instruction does not accumulate its 64-term dot products
  exactly in fp32: measured, the raw scores come out within about 1e-5 of
  their magnitude (the exact case, whose sums are small integers, is not
  affected).  m is therefore compared at 2^-10 relative, l too (it carries
  the score error through exp), and the O bound gets a 2^-10 P_ij term per
  key for the score error's effect on p.  In the exact case m and l match
  to fp32 accuracy (1e-5)."""

import math

import numpy as np
import pytest

import oracle
from tests.helpers import to_device, to_numpy64
from workloads import (WORKLOADS, e4m3_codes, e4m3_value, normal_fp8,
                       uniform_int)

pytestmark = pytest.mark.gpu


def _dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _run(q8, k8, vt8, qd, kd, vd, causal, kv_len, scale):
    import torch
    import exact_io_aware_15_amd as fa
    kvl = None if kv_len is None else torch.tensor(kv_len, dtype=torch.int32,
                                                   device="cuda")
    ds = [None if x is None else _dev(np.asarray(x, np.float32))
          for x in (qd, kd, vd)]
    o, m, l = fa.fwd_fp8(_dev(q8), _dev(k8), _dev(vt8), *ds, causal=causal,
                         kv_len=kvl, scale=scale)
    torch.cuda.synchronize()
    return [to_numpy64(x) for x in (o, m, l)]


def _transpose_pad(v8):
    B, H, N, d = v8.shape
    ldv = -(-N // 16) * 16
    vt = np.zeros((B, H, d, ldv), np.uint8)
    vt[..., :N] = np.swapaxes(v8, 2, 3)
    return vt


def _check_stats(m, l, rm, rl, tol=2.0 ** -10):
    vis = np.isfinite(rm)
    assert np.array_equal(np.isfinite(m), vis)
    assert np.all(l[~vis] == 0)
    if vis.any():
        assert np.max(np.abs(m[vis] - rm[vis]) /
                      np.maximum(1, np.abs(rm[vis]))) <= tol
        assert np.max(np.abs(l[vis] - rl[vis]) / rl[vis]) <= tol


EXACT = [  # (B, H, N, d, causal, kv_len)
    (1, 2, 200, 64, False, None),
    (2, 2, 333, 64, True, None),
    (1, 3, 256, 128, False, [256]),
    (2, 1, 190, 128, True, [190, 77]),
    (1, 1, 64, 128, False, [0]),
    (1, 2, 1, 64, True, None),            # one query, one key
]


@pytest.mark.parametrize("B,H,N,d,causal,kv_len", EXACT)
def test_exact_when_probabilities_are_powers_of_two(B, H, N, d, causal,
                                                    kv_len):
    print(f"fp8 exact B={B} H={H} N={N} d={d} causal={causal} "
          f"kv_len={kv_len}", flush=True)
    rng = np.random.default_rng([9100, N, d])
    # Q and K rows: two entries of +-1 at random positions (raw scores are
    # integers in [-2, 2]); V: integers in [-8, 8]; all exact in E4M3.
    def two_hot(shape):
        x = np.zeros(shape)
        idx = np.argsort(rng.random(shape), axis=-1)[..., :2]
        np.put_along_axis(x, idx, rng.choice([-1.0, 1.0], idx.shape), -1)
        return x
    q, k = two_hot((B, H, N, d)), two_hot((B, H, N, d))
    v = rng.integers(-8, 9, (B, H, N, d)).astype(np.float64)
    q8, k8, v8 = e4m3_codes(q), e4m3_codes(k), e4m3_codes(v)
    assert np.array_equal(e4m3_value(v8), v)
    qd = np.full(B * H, 2.0, np.float32)
    kd = np.full(B * H, 0.5, np.float32)
    vd = np.full(B * H, 0.25, np.float32)
    scale = math.log(2.0)              # c = scale * 2 * 0.5 * log2(e) = 1
    o, m, l = _run(q8, k8, _transpose_pad(v8), qd, kd, vd, causal, kv_len,
                   scale)
    ro, rm, rl = oracle.attention_fwd(2.0 * q, 0.5 * k, 0.25 * v, scale,
                                      causal, kv_len)
    assert np.all(np.abs(o - ro) <= 2.0 ** -8 * np.abs(ro) + 1e-6)
    _check_stats(m, l, rm, rl, 1e-5)


def _fp8_bound(q, k, v, scale, causal, kv_len, rows, rm, rl, ro):
    """Per-element bound and per-element standard deviation of the error that
    rounding P to E4M3 (and O to bf16) can cause; see the module docstring."""
    B, H, N, d = q.shape
    bound = np.zeros(ro.shape)
    var = np.zeros(ro.shape)
    for b in range(B):
        valid = N if kv_len is None else kv_len[b]
        vis = oracle.visible_mask(rows, N, causal, valid)
        for h in range(H):
            s = scale * (q[b, h, rows] @ k[b, h].T)
            mm, ll = rm[b, h][:, None], rl[b, h][:, None]
            with np.errstate(invalid="ignore", over="ignore"):
                p = np.where(vis, np.exp(s - mm) / ll, 0.0)
                e = np.where(vis, np.maximum(2.0 ** -4 * p,
                                             2.0 ** -16 / ll) +
                             2.0 ** -10 * p, 0.0)
            e = np.nan_to_num(e)
            bound[b, h] = e @ np.abs(v[b, h]) + \
                2.0 ** -8 * np.abs(ro[b, h]) + 1e-6
            var[b, h] = (e ** 2) @ (v[b, h] ** 2) / 3 + \
                (2.0 ** -9 * ro[b, h]) ** 2 / 3
    return bound, var


RANDOM = [  # (B, H, N, d, causal, kv_len)
    (2, 2, 300, 64, False, None),
    (1, 3, 517, 64, True, None),
    (2, 2, 384, 128, True, [384, 130]),
    (1, 2, 250, 128, False, [200]),
    (2, 1, 17, 128, True, None),          # shorter than one tile
]


@pytest.mark.parametrize("B,H,N,d,causal,kv_len", RANDOM)
def test_random_inputs_within_the_rounding_bound(B, H, N, d, causal, kv_len):
    print(f"fp8 random B={B} H={H} N={N} d={d} causal={causal} "
          f"kv_len={kv_len}", flush=True)
    seed = 9200 + N + d
    shape = (B, H, N, d)
    q, qd = normal_fp8(shape, seed, 0)
    k, kd = normal_fp8(shape, seed, 1)
    v, vd = normal_fp8(shape, seed, 2, transpose=True)
    scale = 1 / math.sqrt(d)
    o, m, l = _run(q.store, k.store, v.store, qd, kd, vd, causal, kv_len,
                   scale)
    ro, rm, rl = oracle.attention_fwd(q.exact, k.exact, v.exact, scale,
                                      causal, kv_len)
    _check_stats(m, l, rm, rl)
    bound, var = _fp8_bound(q.exact, k.exact, v.exact, scale, causal,
                            kv_len, np.arange(N), rm, rl, ro)
    err = np.abs(o - ro)
    assert np.all(err <= bound), float(np.max(err / bound))
    rms, rms_bound = math.sqrt(np.mean(err ** 2)), math.sqrt(np.mean(var))
    assert rms <= rms_bound, (rms, rms_bound)


def test_null_descales_mean_one():
    import torch
    import exact_io_aware_15_amd as fa
    shape = (1, 2, 200, 64)
    q, _ = normal_fp8(shape, 9300, 0)
    k, _ = normal_fp8(shape, 9300, 1)
    v, _ = normal_fp8(shape, 9300, 2, transpose=True)
    qq, kk, vv = (to_device(x) for x in (q, k, v))
    ones = torch.ones(2, dtype=torch.float32, device="cuda")
    a = fa.fwd_fp8(qq, kk, vv, causal=True)
    b = fa.fwd_fp8(qq, kk, vv, ones, ones, ones, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_long_causal_16k_d128_sampled_rows():
    """The 16K causal d = 128 FP8 workload: sampled rows of every head
    against the oracle with the derived bound."""
    import torch
    import exact_io_aware_15_amd as fa
    w = WORKLOADS["long_causal_16k_d128_fp8"]
    q, k, v, qd, kd, vd = w.fp8_inputs()
    print(f"fp8 {w.name} sampled rows", flush=True)
    o, m, l = fa.fwd_fp8(to_device(q), to_device(k), to_device(v), _dev(qd),
                         _dev(kd), _dev(vd), causal=True)
    torch.cuda.synchronize()
    N = w.N
    rows = np.unique(np.concatenate(
        [[0, 1, 63, 64, 127, 128, N - 1],
         uniform_int(9, 0, N - 1, 9400, 0)]))
    scale = 1 / math.sqrt(w.d)
    ro, rm, rl = oracle.attention_fwd(q.exact, k.exact, v.exact, scale, True,
                                      None, rows=rows)
    o, m, l = (to_numpy64(x)[:, :, rows] for x in (o, m, l))
    _check_stats(m, l, rm, rl)
    bound, var = _fp8_bound(q.exact, k.exact, v.exact, scale, True, None,
                            rows, rm, rl, ro)
    err = np.abs(o - ro)
    assert np.all(err <= bound), float(np.max(err / bound))
    assert math.sqrt(np.mean(err ** 2)) <= math.sqrt(np.mean(var))
