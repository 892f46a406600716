"""CPU pins of the FP8 (E4M3) input codec in workloads/: every code's value
against the OCP format's definition and against torch's float8_e4m3fn, and
the round-to-nearest-even encoder against torch's conversion, including
exact ties and saturation."""

import numpy as np
import pytest
import torch

from workloads import E4M3_MAX, e4m3_codes, e4m3_value, normal_fp8


def test_named_codes():
    # 0x38 = 1.0, 0x7E = 448 (max), 0x01 = 2^-9 (min subnormal),
    # 0x08 = 2^-6 (min normal), 0x80 = -0, 0xB8 = -1
    v = e4m3_value(np.array([0x38, 0x7E, 0x01, 0x08, 0x80, 0xB8, 0x00],
                            np.uint8))
    assert v.tolist()[:4] == [1.0, 448.0, 2.0 ** -9, 2.0 ** -6]
    assert v[4] == 0 and v[5] == -1.0 and v[6] == 0
    assert np.isnan(e4m3_value(np.array([0x7F, 0xFF], np.uint8))).all()
    assert E4M3_MAX == 448.0


def test_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3_value(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_encode_matches_torch_including_ties():
    pos = e4m3_value(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[1:] + pos[:-1]) / 2              # exact ties
    rng = np.random.default_rng(81)
    x = np.concatenate([mids, -mids, pos, rng.standard_normal(20000) * 30,
                        rng.standard_normal(2000) * 1e-3])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8)
    assert np.array_equal(e4m3_codes(x), ref.numpy())
    # ties go to the even code
    assert np.all(e4m3_codes(mids) % 2 == 0)


def test_encode_saturates():
    assert e4m3_codes(np.array([500.0, -1e9, 448.0])).tolist() == [
        0x7E, 0xFE, 0x7E]


@pytest.mark.parametrize("transpose", [False, True])
def test_quantised_tensor_layout(transpose):
    t, ds = normal_fp8((2, 3, 37, 64), 5, 1, 0.5, transpose=transpose)
    assert ds.dtype == np.float32 and ds.shape == (6,)
    codes = t.store
    if transpose:
        assert codes.shape == (2, 3, 64, 48)
        assert np.all(codes[..., 37:] == 0)
        codes = np.swapaxes(codes[..., :37], 2, 3)
    exact = e4m3_value(codes) * ds.astype(np.float64).reshape(2, 3, 1, 1)
    assert np.array_equal(exact, t.exact)
    # the largest magnitude of each head maps to 448
    amax = np.abs(codes.astype(np.int64) & 0x7F).reshape(6, -1).max(axis=1)
    assert np.all(amax == 0x7E)
