"""The debug build (libfa355_debug.so): device-side checks of the arrays whose
contents are the caller's contract (kv_len, cu_seqlens, seq_lens, block
tables; S12's paged loop reads logical block t of a sequence from physical
block block_table[t]).

Every entry point that reads such an array is called with valid contents
(no bit set, and outputs bitwise equal to the ordinary build's, the kernels
being the same) and with each kind of violation (exactly the expected bits).
The kernels clamp malformed values, so these calls stay inside the buffers;
their outputs are unspecified and not compared."""

import numpy as np
import pytest

import exact_io_aware_15_amd as fa
from exact_io_aware_15_amd import _lib
from tests.helpers import to_device
from workloads import TID_DO, normal, normal_fp8, paged_cache

pytestmark = pytest.mark.gpu

KV, CU, SEQ, TAB = (fa.CHECK_KV_LEN, fa.CHECK_CU_SEQLENS, fa.CHECK_SEQ_LENS,
                    fa.CHECK_BLOCK_TABLE)


@pytest.fixture(scope="module")
def builds():
    return _lib.load(_lib.RELEASE_LIB_PATH), _lib.load(_lib.DEBUG_LIB_PATH)


def _run(handle, fn):
    """fn() with `handle` as the library every wrapper calls."""
    old = _lib._lib
    _lib._lib = handle
    try:
        return fn()
    finally:
        _lib._lib = old


def _flags(debug):
    return _run(debug, lambda: fa.debug_flags(clear=True))


def _i32(x):
    import torch
    return torch.tensor(np.asarray(x, np.int32), device="cuda")


def _f32(x):
    import torch
    return torch.from_numpy(np.asarray(x, np.float32)).cuda()


def _same(a, b):
    import torch
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def _expect(builds, fn, bits, compare=False):
    """Run fn under the debug build: the contract word must read `bits`;
    when compare, its outputs must equal the ordinary build's bit for bit."""
    release, debug = builds
    _flags(debug)
    out = _run(debug, fn)
    assert _flags(debug) == bits
    if compare:
        _same(out, _run(release, fn))


def test_ordinary_build_reports_unsupported(builds):
    release, _ = builds
    with pytest.raises(fa.FaError) as e:
        _run(release, lambda: fa.debug_flags())
    assert e.value.status == -3


def _dense(seed, B=2, H=2, N=200, d=64):
    q, k, v, do = (to_device(normal((B, H, N, d), seed, t, "bf16"))
                   for t in (0, 1, 2, TID_DO))
    return q, k, v, do


@pytest.mark.parametrize("kv_len,bits", [
    ([200, 77], 0), ([0, 200], 0), ([201, 77], KV), ([200, -1], KV)])
def test_kv_len(builds, kv_len, bits):
    print(f"debug kv_len={kv_len}", flush=True)
    q, k, v, do = _dense(9500)
    kl = _i32(kv_len)
    fwd = lambda: fa.fwd(q, k, v, causal=True, kv_len=kl)
    _expect(builds, fwd, bits, compare=bits == 0)
    o, m, l = _run(builds[0], fwd)
    _expect(builds, lambda: fa.bwd(q, k, v, o, do, m, l, causal=True,
                                   kv_len=kl), bits, compare=bits == 0)
    _expect(builds, lambda: fa.fwd_dropout(q, k, v, 0.1, 7, kv_len=kl),
            bits, compare=bits == 0)
    _expect(builds, lambda: fa.bwd_dropout(q, k, v, o, do, m, l, 0.1, 7,
                                           causal=True, kv_len=kl),
            bits, compare=bits == 0)


@pytest.mark.parametrize("kv_len,bits", [([200, 130], 0), ([-5, 130], KV)])
def test_kv_len_fp8(builds, kv_len, bits):
    shape = (2, 2, 200, 64)
    q, qd = normal_fp8(shape, 9501, 0)
    k, kd = normal_fp8(shape, 9501, 1)
    v, vd = normal_fp8(shape, 9501, 2, transpose=True)
    qq, kk, vv = (to_device(x) for x in (q, k, v))
    ds = [_f32(x) for x in (qd, kd, vd)]
    kl = _i32(kv_len)
    _expect(builds, lambda: fa.fwd_fp8(qq, kk, vv, *ds, causal=True,
                                       kv_len=kl), bits, compare=bits == 0)


@pytest.mark.parametrize("cu,max_seqlen,bits", [
    ([0, 50, 80, 100], 50, 0),
    ([0, 0, 100, 100], 100, 0),           # empty sequences are allowed
    ([0, 50, 30, 100], 70, CU),           # decreasing
    ([3, 50, 80, 100], 50, CU),           # does not start at 0
    ([0, 50, 80, 90], 50, CU),            # does not end at total
    ([0, 60, 80, 100], 50, CU),           # a sequence above max_seqlen
])
def test_cu_seqlens(builds, cu, max_seqlen, bits):
    print(f"debug cu_seqlens={cu} max_seqlen={max_seqlen}", flush=True)
    H, total, d = 2, 100, 64
    q, k, v, do = (to_device(normal((H, total, d), 9502, t, "bf16"))
                   for t in (0, 1, 2, TID_DO))
    c = _i32(cu)
    fwd = lambda: fa.fwd_varlen(q, k, v, c, max_seqlen, causal=True)
    _expect(builds, fwd, bits, compare=bits == 0)
    o, m, l = _run(builds[0], fwd)
    _expect(builds, lambda: fa.bwd_varlen(q, k, v, o, do, m, l, c,
                                          max_seqlen, causal=True),
            bits, compare=bits == 0)


def _cache(lens, max_blocks, Hkv=2, d=64, seed=9503):
    # ordinary N(0,1) tails: a malformed length may bring them into the
    # arithmetic, and only the flags are compared then
    return paged_cache(lens, Hkv, d, 16, max_blocks, seed, poison_tails=False)


def _decode(cache, table, seq_lens, Hq=4):
    q = to_device(normal((len(seq_lens), Hq, cache.v_cache.exact.shape[-1]),
                         9504, 0, "bf16"))
    kc, vc = to_device(cache.k_cache), to_device(cache.v_cache)
    t, s = _i32(table), _i32(seq_lens)
    return lambda: (fa.decode_paged(q, kc, vc, t, s, num_splits=3),)


def test_decode_valid_and_unused_entries(builds):
    """Entries past a sequence's blocks (-1 here) are never read and so
    never flagged."""
    cache = _cache([37, 300, 0], 22)
    assert np.any(cache.block_table < 0)
    _expect(builds, _decode(cache, cache.block_table, cache.seq_lens), 0,
            compare=True)


def test_decode_bad_entries_and_lengths(builds):
    cache = _cache([37, 300, 16], 22)
    nb = cache.k_cache.exact.shape[0]
    for row, t, val in [(0, 2, nb), (1, 18, -1), (2, 0, -7)]:
        print(f"debug decode table[{row},{t}]={val}", flush=True)
        table = cache.block_table.copy()
        table[row, t] = val
        _expect(builds, _decode(cache, table, cache.seq_lens), TAB)
    # a length past the table's capacity: flagged, and (clamped to the
    # capacity) it reaches row 2's -1 entries too
    lens = cache.seq_lens.copy()
    lens[2] = 22 * 16 + 1
    _expect(builds, _decode(cache, cache.block_table, lens), SEQ | TAB)
    table = np.where(cache.block_table < 0, 0, cache.block_table)
    _expect(builds, _decode(cache, table, lens), SEQ)
    lens[2] = -1
    _expect(builds, _decode(cache, cache.block_table, lens), SEQ)


def _prefill(cache, table, seq_lens, cu, Hq=4):
    total = int(cu[-1])
    d = cache.v_cache.exact.shape[-1]
    q = to_device(normal((Hq, total, d), 9505, 0, "bf16"))
    kc, vc = to_device(cache.k_cache), to_device(cache.v_cache)
    t, s, c = _i32(table), _i32(seq_lens), _i32(cu)
    max_q = max(1, int(np.max(np.diff(cu))))
    return lambda: fa.prefill_paged(q, kc, vc, t, s, c, max_q, causal=True)


def test_prefill(builds):
    cache = _cache([300, 40, 129], 22)
    cu = np.array([0, 100, 140, 141], np.int32)
    _expect(builds, _prefill(cache, cache.block_table, cache.seq_lens, cu), 0,
            compare=True)
    nb = cache.k_cache.exact.shape[0]
    table = cache.block_table.copy()
    table[1, 2] = nb
    _expect(builds, _prefill(cache, table, cache.seq_lens, cu), TAB)
    lens = cache.seq_lens.copy()
    lens[1] = 30                          # fewer positions than new tokens
    _expect(builds, _prefill(cache, cache.block_table, lens, cu), SEQ)
    bad_cu = np.array([0, 100, 90, 141], np.int32)   # decreasing
    _expect(builds, _prefill(cache, cache.block_table, cache.seq_lens,
                             bad_cu), CU)


def test_word_is_sticky_until_cleared(builds):
    _, debug = builds
    q, k, v, _ = _dense(9506)
    _flags(debug)
    _run(debug, lambda: fa.fwd(q, k, v, kv_len=_i32([300, 5])))
    cache = _cache([37], 4)
    table = cache.block_table.copy()
    table[0, 1] = -2
    _run(debug, _decode(cache, table, cache.seq_lens))
    assert _run(debug, lambda: fa.debug_flags()) == KV | TAB
    assert _run(debug, lambda: fa.debug_flags(clear=True)) == KV | TAB
    assert _run(debug, lambda: fa.debug_flags()) == 0
