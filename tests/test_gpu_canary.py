"""Out-of-bounds write checks: every output and workspace buffer is placed
between canary regions and called directly through the C ABI; after the call
the canaries must be untouched.  Shapes have ragged tails."""

import ctypes

import numpy as np
import pytest

from exact_io_aware_15_amd import _lib
from workloads import TID_DO, normal, paged_cache, to_device

pytestmark = pytest.mark.gpu

PAD = 4096
FILL = 0xA5


class Guarded:
    """A device buffer of `nbytes` with PAD canary bytes on each side."""

    def __init__(self, nbytes):
        import torch
        self.n = nbytes
        self.buf = torch.full((nbytes + 2 * PAD,), FILL, dtype=torch.uint8,
                              device="cuda")

    @property
    def ptr(self):
        return ctypes.c_void_p(self.buf.data_ptr() + PAD)

    def intact(self):
        import torch
        torch.cuda.synchronize()
        h = self.buf.cpu().numpy()
        return bool(np.all(h[:PAD] == FILL) and np.all(h[PAD + self.n:] == FILL))


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("dtype,d,causal,padded", [
    ("bf16", 64, True, False), ("bf16", 128, False, True),
    ("f32", 64, True, True)])
def test_fwd_writes_stay_in_bounds(dtype, d, causal, padded):
    import torch
    B, H, N = 2, 3, 333
    q, k, v = (to_device(normal((B, H, N, d), 84, t, dtype)) for t in range(3))
    es = 2 if dtype == "bf16" else 4
    o = Guarded(B * H * N * d * es)
    m = Guarded(B * H * N * 4)
    l = Guarded(B * H * N * 4)
    kl = torch.tensor([N, 100], dtype=torch.int32, device="cuda")
    st = _lib.lib().fa_fwd(1 if dtype == "bf16" else 0, B, H, N, d, _p(q),
                           _p(k), _p(v), o.ptr, m.ptr, l.ptr,
                           _p(kl) if padded else None, int(causal),
                           1.0 / np.sqrt(d), _stream())
    assert st == 0
    assert o.intact() and m.intact() and l.intact()


def test_bwd_writes_stay_in_bounds():
    import torch
    import exact_io_aware_15_amd as fa
    B, H, N, d = 2, 2, 333, 64
    q, k, v = (to_device(normal((B, H, N, d), 85, t, "bf16")) for t in range(3))
    do = to_device(normal((B, H, N, d), 85, TID_DO, "bf16"))
    kl = torch.tensor([N, 150], dtype=torch.int32, device="cuda")
    o, m, l = fa.fwd(q, k, v, causal=True, kv_len=kl)
    grads = [Guarded(B * H * N * d * 2) for _ in range(3)]
    wsb = _lib.lib().fa_bwd_workspace_bytes(B, H, N, d)
    ws = Guarded(wsb)
    # the workspace pointer must be 256-byte aligned: PAD keeps it so
    st = _lib.lib().fa_bwd(B, H, N, d, _p(q), _p(k), _p(v), _p(o), _p(do),
                           _p(m), _p(l), _p(kl), 1, 0.125, grads[0].ptr,
                           grads[1].ptr, grads[2].ptr, ws.ptr, wsb, _stream())
    assert st == 0
    assert all(g.intact() for g in grads) and ws.intact()


def test_decode_writes_stay_in_bounds():
    import torch
    lens = [37, 300, 1, 0]
    cache = paged_cache(lens, 2, 128, 16, 20, 86, poison_tails=True)
    q = to_device(normal((4, 8, 128), 86, 0, "bf16"))
    kc, vc = to_device(cache.k_cache), to_device(cache.v_cache)
    table = torch.from_numpy(cache.block_table).cuda()
    sl = torch.from_numpy(cache.seq_lens).cuda()
    out = Guarded(4 * 8 * 128 * 2)
    wsb = _lib.lib().fa_decode_workspace_bytes(4, 8, 128, 3)
    ws = Guarded(wsb)
    st = _lib.lib().fa_decode_paged(4, 8, 2, 128, _p(q), _p(kc), _p(vc),
                                    kc.shape[0], 16, _p(table), 20, _p(sl), 3,
                                    1.0 / np.sqrt(128), out.ptr, ws.ptr, wsb,
                                    _stream())
    assert st == 0
    assert out.intact() and ws.intact()


def test_varlen_malformed_boundaries_stay_in_bounds():
    """cu_seqlens that decreases and overruns total: the kernels clamp each
    sequence into [0, total], so every write stays inside the buffers (the
    results themselves are unspecified)."""
    import torch
    H, total, d = 2, 100, 64
    q, k, v = (to_device(normal((H, total, d), 87, t, "bf16"))
               for t in range(3))
    do = to_device(normal((H, total, d), 87, TID_DO, "bf16"))
    cu = torch.tensor([0, 50, 30, 400], dtype=torch.int32, device="cuda")
    o = Guarded(H * total * d * 2)
    m = Guarded(H * total * 4)
    l = Guarded(H * total * 4)
    st = _lib.lib().fa_fwd_varlen(1, 3, H, total, 128, d, _p(cu), _p(q),
                                  _p(k), _p(v), o.ptr, m.ptr, l.ptr, 1, 0.125,
                                  _stream())
    assert st == 0
    assert o.intact() and m.intact() and l.intact()
    grads = [Guarded(H * total * d * 2) for _ in range(3)]
    wsb = _lib.lib().fa_bwd_varlen_workspace_bytes(H, total, d)
    ws = Guarded(wsb)
    st = _lib.lib().fa_bwd_varlen(3, H, total, 128, d, _p(cu), _p(q), _p(k),
                                  _p(v), o.ptr, _p(do), m.ptr, l.ptr, 1, 0.125,
                                  grads[0].ptr, grads[1].ptr, grads[2].ptr,
                                  ws.ptr, wsb, _stream())
    assert st == 0
    assert all(g.intact() for g in grads) and ws.intact()


def test_dropout_writes_stay_in_bounds():
    import torch
    B, H, N, d = 2, 2, 333, 64
    q, k, v = (to_device(normal((B, H, N, d), 87, t, "bf16")) for t in range(3))
    do = to_device(normal((B, H, N, d), 87, TID_DO, "bf16"))
    kl = torch.tensor([N, 120], dtype=torch.int32, device="cuda")
    o = Guarded(B * H * N * d * 2)
    m, l = Guarded(B * H * N * 4), Guarded(B * H * N * 4)
    lib = _lib.lib()
    st = lib.fa_fwd_dropout(B, H, N, d, _p(q), _p(k), _p(v), o.ptr, m.ptr,
                            l.ptr, _p(kl), 1, 0.125, 0.2, 77, 3, _stream())
    assert st == 0
    assert o.intact() and m.intact() and l.intact()
    grads = [Guarded(B * H * N * d * 2) for _ in range(3)]
    wsb = lib.fa_bwd_workspace_bytes(B, H, N, d)
    ws = Guarded(wsb)
    st = lib.fa_bwd_dropout(B, H, N, d, _p(q), _p(k), _p(v), o.ptr, _p(do),
                            m.ptr, l.ptr, _p(kl), 1, 0.125, 0.2, 77, 3,
                            grads[0].ptr, grads[1].ptr, grads[2].ptr, ws.ptr,
                            wsb, _stream())
    assert st == 0
    assert all(g.intact() for g in grads) and ws.intact()


@pytest.mark.parametrize("d,causal", [(64, True), (128, False)])
def test_fp8_writes_stay_in_bounds(d, causal):
    import torch
    from workloads import normal_fp8
    B, H, N = 2, 2, 333
    q, qd = normal_fp8((B, H, N, d), 88, 0)
    k, kd = normal_fp8((B, H, N, d), 88, 1)
    v, vd = normal_fp8((B, H, N, d), 88, 2, transpose=True)
    qq, kk, vv = (to_device(x) for x in (q, k, v))
    ds = [torch.from_numpy(x).cuda() for x in (qd, kd, vd)]
    kl = torch.tensor([N, 91], dtype=torch.int32, device="cuda")
    o = Guarded(B * H * N * d * 2)
    m, l = Guarded(B * H * N * 4), Guarded(B * H * N * 4)
    st = _lib.lib().fa_fwd_fp8(B, H, N, d, _p(qq), _p(kk), _p(vv),
                               vv.shape[3], _p(ds[0]), _p(ds[1]), _p(ds[2]),
                               o.ptr, m.ptr, l.ptr, _p(kl), int(causal),
                               1.0 / np.sqrt(d), _stream())
    assert st == 0
    assert o.intact() and m.intact() and l.intact()


def test_block_sparse_writes_stay_in_bounds():
    import torch
    B, H, N, d = 1, 2, 333, 128
    q, k, v = (to_device(normal((B, H, N, d), 89, t, "bf16")) for t in range(3))
    do = to_device(normal((B, H, N, d), 89, TID_DO, "bf16"))
    mask = torch.tensor([[[1, 0, 1], [0, 1, 0], [1, 1, 1]]] * H,
                        dtype=torch.uint8, device="cuda")
    lib = _lib.lib()
    o = Guarded(B * H * N * d * 2)
    m, l = Guarded(B * H * N * 4), Guarded(B * H * N * 4)
    st = lib.fa_fwd_block_sparse(B, H, N, d, _p(q), _p(k), _p(v), o.ptr,
                                 m.ptr, l.ptr, _p(mask), 1, 0.1, _stream())
    assert st == 0
    assert o.intact() and m.intact() and l.intact()
    grads = [Guarded(B * H * N * d * 2) for _ in range(3)]
    wsb = lib.fa_bwd_block_sparse_workspace_bytes(B, H, N, d)
    ws = Guarded(wsb)
    st = lib.fa_bwd_block_sparse(B, H, N, d, _p(q), _p(k), _p(v), o.ptr,
                                 _p(do), m.ptr, l.ptr, _p(mask), 1, 0.1,
                                 grads[0].ptr, grads[1].ptr, grads[2].ptr,
                                 ws.ptr, wsb, _stream())
    assert st == 0
    assert all(g.intact() for g in grads) and ws.intact()


def test_prefill_writes_stay_in_bounds():
    import torch
    ctx = [40, 300, 17]
    qlen = [5, 130, 17]
    Hq, Hkv, d = 4, 2, 64
    cache = paged_cache(ctx, Hkv, d, 16, 24, 90, poison_tails=True)
    cu = np.concatenate([[0], np.cumsum(qlen)]).astype(np.int32)
    total = int(cu[-1])
    q = to_device(normal((Hq, total, d), 90, 0, "bf16"))
    kc, vc = to_device(cache.k_cache), to_device(cache.v_cache)
    table = torch.from_numpy(cache.block_table).cuda()
    sl = torch.from_numpy(cache.seq_lens).cuda()
    cud = torch.from_numpy(cu).cuda()
    o = Guarded(Hq * total * d * 2)
    m, l = Guarded(Hq * total * 4), Guarded(Hq * total * 4)
    st = _lib.lib().fa_prefill_paged(3, Hq, Hkv, d, total, 130, _p(cud), _p(q),
                                     _p(kc), _p(vc), kc.shape[0], 16,
                                     _p(table), 24, _p(sl), 1, 0.125, o.ptr,
                                     m.ptr, l.ptr, _stream())
    assert st == 0
    assert o.intact() and m.intact() and l.intact()
