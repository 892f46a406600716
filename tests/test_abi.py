"""CPU checks of the C ABI: the library loads, exports every function that
include/fa355.h declares, and rejects invalid arguments before launching
anything.  No call here reaches a kernel launch (every call is invalid by
construction, or has no rows to compute), so these run without a GPU."""

import ctypes
import os
import re

import pytest

from exact_io_aware_15_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa355.h")

FAKE = ctypes.c_void_p(0x1000)   # non-null, never dereferenced by validation
NULL = None


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libfa355.so not built")
    return _lib.lib()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(_lib.SIGNATURES), names
    for n in names:
        assert hasattr(lib, n), n


def test_both_builds_export_every_symbol():
    for path in (_lib.RELEASE_LIB_PATH, _lib.DEBUG_LIB_PATH):
        if not os.path.exists(path):
            pytest.skip(f"{path} not built")
        handle = _lib.load(path)
        for n in declared_functions():
            assert hasattr(handle, n), (path, n)


def test_debug_flags_without_device():
    """The ordinary build checks nothing and says so; the debug build rejects
    a NULL destination before touching the device."""
    for path in (_lib.RELEASE_LIB_PATH, _lib.DEBUG_LIB_PATH):
        if not os.path.exists(path):
            pytest.skip(f"{path} not built")
    release = _lib.load(_lib.RELEASE_LIB_PATH)
    word = ctypes.c_uint32(7)
    assert release.fa_debug_flags(ctypes.byref(word), 1) == -3
    assert release.fa_debug_flags(NULL, 0) == -3
    assert word.value == 7
    debug = _lib.load(_lib.DEBUG_LIB_PATH)
    assert debug.fa_debug_flags(NULL, 0) == -1
    assert debug.fa_debug_flags(NULL, 1) == -1


def test_status_strings(lib):
    for code in range(-5, 1):
        s = lib.fa_status_str(code).decode()
        assert s.startswith(_lib.STATUS[code])
    assert b"unknown" in lib.fa_status_str(42)


def _fwd(lib, dtype=1, B=1, H=1, N=16, d=64, q=FAKE, m=NULL, l=NULL,
         scale=0.125):
    return lib.fa_fwd(dtype, B, H, N, d, q, FAKE, FAKE, FAKE, m, l, NULL, 0,
                      scale, NULL)


def test_fwd_validation(lib):
    assert _fwd(lib, q=NULL) == -1
    assert _fwd(lib, m=FAKE) == -1            # m without l
    assert _fwd(lib, N=0) == -2
    assert _fwd(lib, B=0) == -2
    assert _fwd(lib, N=(1 << 20) + 1) == -2
    assert _fwd(lib, B=1 << 16, H=1 << 10, N=1 << 10) == -2   # > 2^31 rows
    assert _fwd(lib, scale=0.0) == -2
    assert _fwd(lib, scale=float("nan")) == -2
    assert _fwd(lib, scale=float("inf")) == -2
    assert _fwd(lib, d=96) == -3
    assert _fwd(lib, dtype=7) == -3


def test_bwd_workspace_and_validation(lib):
    ws = lib.fa_bwd_workspace_bytes(2, 3, 100, 64)
    rows = 2 * 3 * 100
    up = lambda x: (x + 255) // 256 * 256   # noqa: E731
    assert ws == 2 * up(rows * 4)
    assert lib.fa_bwd_workspace_bytes(2, 3, 100, 80) == 0
    assert lib.fa_bwd_workspace_bytes(0, 3, 100, 64) == 0
    # block-sparse: the dense workspace plus [2][H * ceil(N/128)] int32 work
    # counts and orders, each padded to 256 bytes
    sp = lib.fa_bwd_block_sparse_workspace_bytes(2, 3, 300, 64)
    dense = lib.fa_bwd_workspace_bytes(2, 3, 300, 64)
    assert sp == dense + 2 * 256                # 2 * 3 * 3 * 4 = 72 bytes
    assert lib.fa_bwd_block_sparse_workspace_bytes(2, 3, 100, 80) == 0
    assert lib.fa_bwd_block_sparse_workspace_bytes(0, 3, 100, 64) == 0

    def call(ws_ptr=FAKE, ws_bytes=ws, d=64, q=FAKE, N=100, scale=0.125):
        return lib.fa_bwd(2, 3, N, d, q, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                          NULL, 1, scale, FAKE, FAKE, FAKE, ws_ptr, ws_bytes,
                          NULL)
    assert call(q=NULL) == -1
    assert call(N=0) == -2
    assert call(scale=-1.0) == -2
    assert call(d=32) == -3
    assert call(ws_ptr=NULL) == -4
    assert call(ws_bytes=ws - 1) == -4
    assert call(ws_ptr=ctypes.c_void_p(0x1008)) == -4   # not 256-aligned


def test_decode_workspace_and_validation(lib):
    ws = lib.fa_decode_workspace_bytes(16, 32, 128, 8)
    parts = 16 * 32 * 8
    up = lambda x: (x + 255) // 256 * 256   # noqa: E731
    assert ws == 2 * up(parts * 4) + up(parts * 128 * 4)
    assert lib.fa_decode_workspace_bytes(16, 32, 128, 0) == 0
    assert lib.fa_decode_workspace_bytes(16, 32, 128, 65) == 0

    def call(Hq=32, Hkv=8, d=128, bs=16, splits=8, ws_bytes=ws, q=FAKE,
             nb=100, scale=0.1):
        return lib.fa_decode_paged(16, Hq, Hkv, d, q, FAKE, FAKE, nb, bs,
                                   FAKE, 512, FAKE, splits, scale, FAKE,
                                   FAKE, ws_bytes, NULL)
    assert call(q=NULL) == -1
    assert call(Hkv=7) == -2             # 32 % 7 != 0
    assert call(nb=0) == -2
    assert call(splits=0) == -2
    assert call(scale=0.0) == -2
    assert call(Hq=64, Hkv=2) == -3      # group of 32 > 16
    assert call(Hq=34, Hkv=2) == -3      # group of 17 > 16
    # Groups that are not a power of two pass the group check: with a short
    # workspace they stop at the workspace check (-4), not at -3.
    for Hq, Hkv in ((24, 8), (40, 8), (48, 8), (30, 2), (15, 1)):
        short = lib.fa_decode_workspace_bytes(16, Hq, 128, 8) - 4
        assert call(Hq=Hq, Hkv=Hkv, ws_bytes=short) == -4, (Hq, Hkv)
    assert call(d=96) == -3
    assert call(bs=32) == -3
    assert call(ws_bytes=ws - 4) == -4
    # the no-allocation variant validates the same way, and rejects a
    # request its fixed scratch cannot hold before touching the device
    def call_na(Hq=32, Hkv=8, d=128, splits=8, B=16, q=FAKE):
        return lib.fa_decode_paged_noalloc(B, Hq, Hkv, d, q, FAKE, FAKE, 100,
                                           16, FAKE, 512, FAKE, splits, 0.1,
                                           FAKE, NULL)
    assert call_na(q=NULL) == -1
    assert call_na(Hkv=7) == -2
    assert call_na(Hq=64, Hkv=2) == -3
    assert lib.fa_decode_workspace_bytes(64, 64, 128, 8) > \
        _lib.FA_DECODE_SCRATCH_BYTES
    assert call_na(B=64, Hq=64) == -6
    # a capacity of max_blocks_per_seq * 16 tokens must fit an int
    assert lib.fa_decode_paged(1, 32, 8, 128, FAKE, FAKE, FAKE, 100, 16, FAKE,
                               1 << 27, FAKE, 8, 0.1, FAKE, FAKE, ws,
                               NULL) == -2
    # one workgroup per (partition slot, head): B * num_splits * Hq must fit
    # an int
    B = (1 << 31) // (64 * 32) + 1
    assert lib.fa_decode_paged(B, 32, 8, 128, FAKE, FAKE, FAKE, 100, 16, FAKE,
                               1, FAKE, 64, 0.1, FAKE, FAKE, 1 << 62,
                               NULL) == -2


def test_last_hip_error_starts_clear(lib):
    # Validation failures are not HIP errors and leave the record untouched.
    assert _fwd(lib, q=NULL) == -1
    assert lib.fa_last_hip_error() == 0
    assert lib.fa_last_hip_error_str()


def _fwd_varlen(lib, dtype=1, B=2, H=1, total=10, max_seqlen=8, d=64,
                cu=FAKE, q=FAKE, m=NULL, l=NULL, scale=0.125):
    return lib.fa_fwd_varlen(dtype, B, H, total, max_seqlen, d, cu, q, FAKE,
                             FAKE, FAKE, m, l, 1, scale, NULL)


def test_fwd_varlen_validation(lib):
    assert _fwd_varlen(lib, cu=NULL) == -1
    assert _fwd_varlen(lib, q=NULL) == -1
    assert _fwd_varlen(lib, m=FAKE) == -1
    assert _fwd_varlen(lib, B=0) == -2
    assert _fwd_varlen(lib, total=-1) == -2
    assert _fwd_varlen(lib, max_seqlen=0) == -2
    assert _fwd_varlen(lib, max_seqlen=(1 << 20) + 1) == -2
    assert _fwd_varlen(lib, H=1 << 12, total=1 << 20) == -2  # > 2^31 rows
    assert _fwd_varlen(lib, scale=0.0) == -2
    assert _fwd_varlen(lib, d=96) == -3
    assert _fwd_varlen(lib, dtype=7) == -3
    # no tokens: nothing to launch (no device is touched), NULL buffers fine
    assert _fwd_varlen(lib, total=0) == 0
    assert _fwd_varlen(lib, total=0, cu=NULL, q=NULL) == 0


def test_bwd_varlen_workspace_and_validation(lib):
    assert lib.fa_bwd_varlen_workspace_bytes(3, 1000, 64) == 2 * 12032
    assert lib.fa_bwd_varlen_workspace_bytes(3, 0, 64) == 0
    assert lib.fa_bwd_varlen_workspace_bytes(0, 10, 64) == 0
    assert lib.fa_bwd_varlen_workspace_bytes(3, 10, 80) == 0

    def call(cu=FAKE, total=1000, ws=FAKE, ws_bytes=1 << 20, d=64):
        return lib.fa_bwd_varlen(2, 3, total, 600, d, cu, FAKE, FAKE, FAKE,
                                 FAKE, FAKE, FAKE, FAKE, 1, 0.125, FAKE, FAKE,
                                 FAKE, ws, ws_bytes, NULL)
    assert call(cu=NULL) == -1
    assert call(d=80) == -3
    assert call(ws=NULL) == -4
    assert call(ws_bytes=2 * 12032 - 1) == -4
    assert call(ws=ctypes.c_void_p(0x1008)) == -4
    assert call(total=0, ws=NULL, ws_bytes=0) == 0


def test_block_sparse_validation(lib):
    def fwd(q=FAKE, mask=FAKE, N=300, d=64, m=NULL):
        return lib.fa_fwd_block_sparse(1, 2, N, d, q, FAKE, FAKE, FAKE, m,
                                       NULL, mask, 0, 0.125, NULL)
    assert fwd(mask=NULL) == -1
    assert fwd(q=NULL) == -1
    assert fwd(m=FAKE) == -1
    assert fwd(N=0) == -2
    assert fwd(d=96) == -3

    def bwd(mask=FAKE, ws=FAKE, ws_bytes=1 << 20):
        return lib.fa_bwd_block_sparse(1, 2, 300, 64, FAKE, FAKE, FAKE, FAKE,
                                       FAKE, FAKE, FAKE, mask, 1, 0.125, FAKE,
                                       FAKE, FAKE, ws, ws_bytes, NULL)
    assert bwd(mask=NULL) == -1
    assert bwd(ws=NULL) == -4
    assert bwd(ws_bytes=16) == -4
    # the dense backward's workspace lacks the items' work and order arrays
    assert bwd(ws_bytes=lib.fa_bwd_workspace_bytes(1, 2, 300, 64)) == -4


def test_dropout_validation(lib):
    def fwd(q=FAKE, N=64, d=64, p=0.1, m=NULL, scale=0.125):
        return lib.fa_fwd_dropout(1, 2, N, d, q, FAKE, FAKE, FAKE, m, NULL,
                                  NULL, 0, scale, p, 1, 0, NULL)
    assert fwd(q=NULL) == -1
    assert fwd(m=FAKE) == -1
    assert fwd(N=0) == -2
    assert fwd(scale=0.0) == -2
    assert fwd(p=-0.01) == -2
    assert fwd(p=float("nan")) == -2
    assert fwd(p=255.5 / 256) == -2           # rounds to 256/256
    assert fwd(p=1.0) == -2
    assert fwd(d=96) == -3
    assert fwd(d=96, p=0.5) == -3             # a valid p does not hide d

    def bwd(ws=FAKE, ws_bytes=1 << 20, p=0.1, l=FAKE):
        return lib.fa_bwd_dropout(1, 2, 64, 64, FAKE, FAKE, FAKE, FAKE, FAKE,
                                  FAKE, l, NULL, 1, 0.125, p, 7, 3, FAKE,
                                  FAKE, FAKE, ws, ws_bytes, NULL)
    assert bwd(l=NULL) == -1
    assert bwd(p=2.0) == -2
    assert bwd(ws=NULL) == -4
    assert bwd(ws_bytes=16) == -4


def test_fp8_validation(lib):
    def call(q=FAKE, vt=FAKE, N=100, ldv=112, d=128, m=NULL, scale=0.1):
        return lib.fa_fwd_fp8(1, 2, N, d, q, FAKE, vt, ldv, NULL, NULL, NULL,
                              FAKE, m, NULL, NULL, 1, scale, NULL)
    assert call(q=NULL) == -1
    assert call(vt=NULL) == -1
    assert call(m=FAKE) == -1
    assert call(N=0) == -2
    assert call(ldv=96) == -2                 # < N
    assert call(ldv=104) == -2                # not a multiple of 16
    assert call(vt=ctypes.c_void_p(0x1008)) == -2   # not 16-byte aligned
    assert call(scale=-1.0) == -2
    assert call(d=96) == -3


PROBE_HEADER = os.path.join(ROOT, "include", "fa355_probe.h")


def test_probe_library_exports_and_validates():
    """The measurement library exports what its header declares and rejects
    invalid arguments before touching a device."""
    from exact_io_aware_15_amd import probe
    if not os.path.exists(probe.PROBE_LIB_PATH):
        pytest.skip("libfa355_probe.so not built")
    text = re.sub(r"/\*.*?\*/", "", open(PROBE_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(fa_probe_[a-z0-9_]+)\s*\(", text)))
    assert set(names) == set(probe.SIGNATURES)
    h = probe.lib()
    d = ctypes.c_double()
    assert h.fa_probe_mfma_bf16(0, 2, None, None, None) == -1
    assert h.fa_probe_mfma_bf16(10, 0, None, None, None) == -1
    assert h.fa_probe_mfma_bf16(10, 5, None, None, None) == -1
    assert h.fa_probe_read_bw(1000, 1, ctypes.byref(d)) == -1
    assert h.fa_probe_read_bw(1 << 20, 0, ctypes.byref(d)) == -1


def test_pack_k_cache_gives_the_generator_layout():
    """pack_k_cache turns token-ordered K into the grouped cache order;
    on the generator's own draw it must give the stored K bit for bit."""
    import numpy as np
    import torch

    from exact_io_aware_15_amd import pack_k_cache
    from workloads import TID_KC, bf16_bits, paged_cache, rng

    cache = paged_cache([40, 9], 2, 64, 16, 3, cfg_seed=77, poison_tails=False)
    nb = cache.v_cache.store.shape[0]
    draw = rng(77, TID_KC).standard_normal(size=(nb, 2, 16, 64),
                                           dtype=np.float32)
    bits = torch.from_numpy(bf16_bits(draw).view(np.int16))
    packed = pack_k_cache(bits)
    assert packed.is_contiguous()
    assert np.array_equal(packed.numpy().view(np.uint16), cache.k_cache.store)
    with pytest.raises(ValueError):
        pack_k_cache(torch.zeros(1, 1, 16, 48))
