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
* Score accumulation.  The FP8 matrix instruction does not sum its 64-term
  dot products exactly in fp32.  Modelled as |S'_ij - S_ij| <= EPS_ACC *
  scale * sum_k |q_ik k_jk| (dequantised values), with EPS_ACC = 2^-13.
  Measured on the random E4M3 inputs below (N(0,1) draws): the largest
  observed ratio |m' - m| / A_i, with A_i = scale * max_j sum_k |q_ik k_jk|
  over the row's visible keys, was 2^-15.15 at d = 64 and 2^-16.3 at
  d = 128 (every random-input test prints it), so EPS_ACC carries a factor
  4.4 over the largest one.  From the model: m is held to EPS_ACC * A_i;
  each term of l = sum_j exp(S_ij - m_i) moves by at most 2 EPS_ACC A_i in
  the log, so l to expm1(2 EPS_ACC A_i) relative (plus 2^-17 for fp32
  summation; measured at most 1.8e-4 against a bound near 1.5e-3); and each
  P_ij, the ratio of such a term to l, by at most expm1(4 EPS_ACC A_i)
  relative, which is the score term of the O bound.  In the exact case
  (small-integer sums) m and l match to 1e-5."""

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


# Relative accumulation error of the FP8 score products (see above).
EPS_ACC = 2.0 ** -13


def _check_stats(m, l, rm, rl, tol=1e-5):
    """Exact case: m and l to fp32 accuracy."""
    vis = np.isfinite(rm)
    assert np.array_equal(np.isfinite(m), vis)
    assert np.all(l[~vis] == 0)
    if vis.any():
        assert np.max(np.abs(m[vis] - rm[vis]) /
                      np.maximum(1, np.abs(rm[vis]))) <= tol
        assert np.max(np.abs(l[vis] - rl[vis]) / rl[vis]) <= tol


def _score_mass(q, k, scale, causal, kv_len, rows):
    """A_i = scale * max over visible keys j of sum_k |q_ik k_jk|, [B,H,R]."""
    B, H, N, d = q.shape
    A = np.zeros((B, H, len(rows)))
    for b in range(B):
        valid = N if kv_len is None else kv_len[b]
        vis = oracle.visible_mask(rows, N, causal, valid)
        for h in range(H):
            a = scale * (np.abs(q[b, h, rows]) @ np.abs(k[b, h]).T)
            A[b, h] = np.where(vis, a, 0.0).max(axis=1, initial=0.0)
    return A


def _check_stats_model(m, l, rm, rl, A):
    """Random case: m within EPS_ACC * A_i, l within expm1(2 EPS_ACC A_i)
    relative (+ 2^-17 for its fp32 sum); prints the observed ratios."""
    vis = np.isfinite(rm)
    assert np.array_equal(np.isfinite(m), vis)
    assert np.all(l[~vis] == 0)
    if not vis.any():
        return
    em = np.abs(m[vis] - rm[vis])
    el = np.abs(l[vis] - rl[vis]) / rl[vis]
    Av = A[vis]
    ratio = float(np.max(em / Av))
    print(f"  fp8 score error: max |m' - m| / A = {ratio:.3e} "
          f"(= 2^{math.log2(max(ratio, 1e-30)):.2f}; EPS_ACC = 2^-13); "
          f"max l rel err {float(np.max(el)):.3e}", flush=True)
    assert np.all(em <= EPS_ACC * Av + 1e-6 * np.abs(rm[vis]))
    assert np.all(el <= np.expm1(2 * EPS_ACC * Av) + 2.0 ** -17)


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
    _check_stats(m, l, rm, rl)


def _fp8_bound(q, k, v, scale, causal, kv_len, rows, rm, rl, ro, A):
    """Per-element bound and per-element standard deviation of the error that
    rounding P to E4M3 (and O to bf16) and the score accumulation error can
    cause; see the module docstring."""
    B, H, N, d = q.shape
    bound = np.zeros(ro.shape)
    var = np.zeros(ro.shape)
    for b in range(B):
        valid = N if kv_len is None else kv_len[b]
        vis = oracle.visible_mask(rows, N, causal, valid)
        for h in range(H):
            s = scale * (q[b, h, rows] @ k[b, h].T)
            mm, ll = rm[b, h][:, None], rl[b, h][:, None]
            es = np.expm1(4 * EPS_ACC * A[b, h])[:, None]
            with np.errstate(invalid="ignore", over="ignore"):
                p = np.where(vis, np.exp(s - mm) / ll, 0.0)
                e = np.where(vis, np.maximum(2.0 ** -4 * p,
                                             2.0 ** -16 / ll) +
                             es * p, 0.0)
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
    A = _score_mass(q.exact, k.exact, scale, causal, kv_len, np.arange(N))
    _check_stats_model(m, l, rm, rl, A)
    bound, var = _fp8_bound(q.exact, k.exact, v.exact, scale, causal,
                            kv_len, np.arange(N), rm, rl, ro, A)
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
    A = _score_mass(q.exact, k.exact, scale, True, None, rows)
    _check_stats_model(m, l, rm, rl, A)
    bound, var = _fp8_bound(q.exact, k.exact, v.exact, scale, True, None,
                            rows, rm, rl, ro, A)
    err = np.abs(o - ro)
    assert np.all(err <= bound), float(np.max(err / bound))
    assert math.sqrt(np.mean(err ** 2)) <= math.sqrt(np.mean(var))
