"""fa_decode_paged_noalloc (the decode entry point that allocates nothing,
for callers under graph capture or in tight serving loops) against
fa_decode_paged, both called through the C ABI: the same kernels, so the
outputs must agree bit for bit.  Two calls in a row on one GPU's fixed
scratch, the second smaller than the first, so a stale partial of the first
call that leaked into the second would show; then the first shape again."""

import ctypes

import numpy as np
import pytest

from exact_io_aware_15_amd import _lib
from workloads import normal, paged_cache

pytestmark = pytest.mark.gpu


def _inputs(lens, Hq, Hkv, d, seed):
    import torch
    from workloads import to_device
    max_blocks = -(-max(lens) // 16) + 1
    cache = paged_cache(lens, Hkv, d, 16, max_blocks, seed, poison_tails=True)
    q = normal((len(lens), Hq, d), seed, 0, "bf16")
    return (to_device(q), to_device(cache.k_cache), to_device(cache.v_cache),
            torch.from_numpy(cache.block_table).cuda(),
            torch.from_numpy(cache.seq_lens).cuda())


def _call_both(lib, inp, splits):
    import torch
    q, kc, vc, table, lens = inp
    B, Hq, d = q.shape
    nb, Hkv, bs, _ = vc.shape
    scale = 1.0 / d ** 0.5
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    need = lib.fa_decode_workspace_bytes(B, Hq, d, splits)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    ref = torch.empty_like(q)
    got = torch.full_like(q, float("nan"))
    st = lib.fa_decode_paged(B, Hq, Hkv, d, q.data_ptr(), kc.data_ptr(),
                             vc.data_ptr(), nb, bs, table.data_ptr(),
                             table.shape[1], lens.data_ptr(), splits, scale,
                             ref.data_ptr(), ws.data_ptr(), need, stream)
    assert st == 0, st
    st = lib.fa_decode_paged_noalloc(B, Hq, Hkv, d, q.data_ptr(),
                                     kc.data_ptr(), vc.data_ptr(), nb, bs,
                                     table.data_ptr(), table.shape[1],
                                     lens.data_ptr(), splits, scale,
                                     got.data_ptr(), stream)
    assert st == 0, st
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_decode_matches_workspace_decode_twice():
    import torch
    lib = _lib.lib()
    big = _inputs([700, 33, 1, 4100, 160], 32, 8, 128, 8800)
    small = _inputs([17, 300], 12, 4, 64, 8801)
    for name, inp, splits in (("big", big, 8), ("small", small, 3),
                              ("big again", big, 8)):
        print(f"noalloc decode {name}: B={inp[0].shape[0]} "
              f"Hq={inp[0].shape[1]} d={inp[0].shape[2]} splits={splits}",
              flush=True)
        ref, got = _call_both(lib, inp, splits)
        assert torch.isfinite(got).all()
        assert torch.equal(ref, got), name


def test_noalloc_decode_rejects_more_than_its_scratch():
    lib = _lib.lib()
    fake = ctypes.c_void_p(0x1000)
    # B * Hq * splits * (d + 2) * 4 bytes > 8 MiB
    B, Hq, d, splits = 64, 64, 128, 8
    assert lib.fa_decode_workspace_bytes(B, Hq, d, splits) > \
        _lib.FA_DECODE_SCRATCH_BYTES
    st = lib.fa_decode_paged_noalloc(B, Hq, 8, d, fake, fake, fake, 100, 16,
                                     fake, 512, fake, splits, 0.1, fake, None)
    assert st == -6
    assert b"scratch" in lib.fa_status_str(-6)
