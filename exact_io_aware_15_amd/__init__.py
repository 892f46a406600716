"""fa355: exact, IO-aware attention on AMD MI355X (gfx950).

A thin binding over libfa355's C ABI (include/fa355.h).  It checks tensor
dtypes, shapes and devices, allocates outputs and workspaces with PyTorch, and
passes raw device pointers plus the current HIP stream; every step of the
computation runs in the library's HIP kernels.  There is no fallback path: if
the library is missing, the calls raise.

    o, m, l = fwd(q, k, v, causal=False, kv_len=None, scale=None)
    dq, dk, dv = bwd(q, k, v, o, do, m, l, causal=False, kv_len=None)
    o, m, l = fwd_varlen(q, k, v, cu_seqlens, max_seqlen, causal=False)
    dq, dk, dv = bwd_varlen(q, k, v, o, do, m, l, cu_seqlens, max_seqlen)
    k_cache = pack_k_cache(k_rows)      # [nb, Hkv, 16, d] -> K cache order
    out = decode_paged(q, k_cache, v_cache, block_table, seq_lens, num_splits=8)
    o, m, l = prefill_paged(q, k_cache, v_cache, block_table, seq_lens,
                            cu_seqlens_q, max_q, causal=True)
    bits = debug_flags(clear=False)     # debug build (FA355_DEBUG=1) only
"""

import ctypes
import math

from ._lib import FA_BF16, FA_F32, FaError, LibraryMissing, check, lib

__all__ = ["fwd", "bwd", "fwd_dropout", "bwd_dropout", "fwd_fp8",
           "fwd_varlen", "bwd_varlen", "fwd_block_sparse",
           "bwd_block_sparse", "decode_paged", "decode_paged_noalloc",
           "prefill_paged", "pack_k_cache",
           "bwd_workspace_bytes", "bwd_varlen_workspace_bytes",
           "bwd_block_sparse_workspace_bytes",
           "decode_workspace_bytes", "debug_flags", "CHECK_KV_LEN",
           "CHECK_CU_SEQLENS", "CHECK_SEQ_LENS", "CHECK_BLOCK_TABLE",
           "FaError", "LibraryMissing"]

# Bits of the debug build's contract word (FA_CHECK_* in fa355.h).
CHECK_KV_LEN, CHECK_CU_SEQLENS, CHECK_SEQ_LENS, CHECK_BLOCK_TABLE = 1, 2, 4, 8


def debug_flags(clear=False):
    """The debug build's record of contract violations on the current device
    (an OR of CHECK_* bits since the last clear); waits for the device.
    Raises FaError (FA_E_UNSUPPORTED) when the ordinary build is loaded."""
    word = ctypes.c_uint32(0)
    check("fa_debug_flags", lib().fa_debug_flags(ctypes.byref(word),
                                                 int(bool(clear))))
    return word.value


def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float32:
        return FA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _check_dev(name, t, dtype=None, shape=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, "
                         f"got {tuple(t.shape)}")


def _workspace(workspace, need, device):
    """The caller's workspace (a contiguous uint8 GPU tensor on the inputs'
    device; its byte count is passed on, and the library rejects one that is
    too small) or a new one of the size the library asks for."""
    torch = _torch()
    if workspace is None:
        return torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    _check_dev("workspace", workspace, torch.uint8)
    if workspace.device != device:
        raise ValueError("workspace must be on the inputs' device")
    return workspace


def _stream(t):
    torch = _torch()
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _kv_len(kv_len, B, device):
    torch = _torch()
    if kv_len is None:
        return None
    if not torch.is_tensor(kv_len):
        kv_len = torch.tensor(list(kv_len), dtype=torch.int32, device=device)
    _check_dev("kv_len", kv_len, torch.int32, (B,))
    return kv_len


def fwd(q, k, v, causal=False, kv_len=None, scale=None, return_stats=True):
    """Exact attention forward.  q, k, v: [B,H,N,d] bf16 or fp32 on the GPU.

    Returns (o, m, l): o like q; m, l fp32 [B,H,N] (None if not requested).
    """
    torch = _torch()
    B, H, N, d = q.shape
    _check_dev("q", q)
    _check_dev("k", k, q.dtype, q.shape)
    _check_dev("v", v, q.dtype, q.shape)
    kv_len = _kv_len(kv_len, B, q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q)
    m = l = None
    if return_stats:
        m = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        l = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):
        st = lib().fa_fwd(_dtype_code(q), B, H, N, d, _ptr(q), _ptr(k),
                          _ptr(v), _ptr(o), _ptr(m), _ptr(l), _ptr(kv_len),
                          int(bool(causal)), scale, _stream(q))
    check("fa_fwd", st)
    return o, m, l


def fwd_fp8(q, k, v_t, q_descale=None, k_descale=None, v_descale=None,
            causal=False, kv_len=None, scale=None, return_stats=True):
    """Attention forward on FP8 (E4M3) operands.

    q, k: [B,H,N,d] uint8 E4M3 codes; v_t: V transposed, [B,H,d,ldv] uint8
    codes with ldv >= N a multiple of 16; descales: fp32 [B*H] (or [B,H])
    tensors or None for 1.  The real inputs are code * descale.  Returns
    (o, m, l): o bf16 [B,H,N,d], m, l fp32 [B,H,N] (None if not requested).
    """
    torch = _torch()
    B, H, N, d = q.shape
    _check_dev("q", q, torch.uint8)
    _check_dev("k", k, torch.uint8, q.shape)
    _check_dev("v_t", v_t, torch.uint8)
    if v_t.dim() != 4 or tuple(v_t.shape[:3]) != (B, H, d):
        raise ValueError(f"v_t must be [B,H,d,ldv], got {tuple(v_t.shape)}")
    ds = []
    for name, t in (("q_descale", q_descale), ("k_descale", k_descale),
                    ("v_descale", v_descale)):
        if t is not None:
            _check_dev(name, t, torch.float32)
            if t.numel() != B * H:
                raise ValueError(f"{name} must hold B*H values")
        ds.append(t)
    kv_len = _kv_len(kv_len, B, q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q.device)
    m = l = None
    if return_stats:
        m = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        l = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):
        st = lib().fa_fwd_fp8(B, H, N, d, _ptr(q), _ptr(k), _ptr(v_t),
                              v_t.shape[3], _ptr(ds[0]), _ptr(ds[1]),
                              _ptr(ds[2]), _ptr(o), _ptr(m), _ptr(l),
                              _ptr(kv_len), int(bool(causal)), scale,
                              _stream(q))
    check("fa_fwd_fp8", st)
    return o, m, l


def bwd_workspace_bytes(B, H, N, d):
    return int(lib().fa_bwd_workspace_bytes(B, H, N, d))


def bwd_block_sparse_workspace_bytes(B, H, N, d):
    return int(lib().fa_bwd_block_sparse_workspace_bytes(B, H, N, d))


def bwd(q, k, v, o, do, m, l, causal=False, kv_len=None, scale=None,
        workspace=None):
    """Gradients (dq, dk, dv) of exact attention; all bf16 [B,H,N,d]."""
    torch = _torch()
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check_dev(name, t, torch.bfloat16, (B, H, N, d))
    _check_dev("m", m, torch.float32, (B, H, N))
    _check_dev("l", l, torch.float32, (B, H, N))
    kv_len = _kv_len(kv_len, B, q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    workspace = _workspace(workspace, bwd_workspace_bytes(B, H, N, d),
                           q.device)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    with torch.cuda.device(q.device):
        st = lib().fa_bwd(B, H, N, d, _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                          _ptr(do), _ptr(m), _ptr(l), _ptr(kv_len),
                          int(bool(causal)), scale, _ptr(dq), _ptr(dk),
                          _ptr(dv), _ptr(workspace), workspace.numel(),
                          _stream(q))
    check("fa_bwd", st)
    return dq, dk, dv


def fwd_dropout(q, k, v, p_drop, seed, offset=0, causal=False, kv_len=None,
                scale=None, return_stats=True):
    """Attention forward with dropout on P fused in: q, k, v [B,H,N,d] bf16.

    Element (i, j) of head b*H + h is kept iff its Philox4x32-10 byte (counter
    (i, group(j), b*H + h, offset), key = seed) is >= round(256 p_drop); kept
    probabilities are scaled by 256 / (256 - round(256 p_drop)).  Returns
    (o, m, l) with the pre-dropout softmax statistics m, l.
    """
    torch = _torch()
    B, H, N, d = q.shape
    _check_dev("q", q, torch.bfloat16)
    _check_dev("k", k, q.dtype, q.shape)
    _check_dev("v", v, q.dtype, q.shape)
    kv_len = _kv_len(kv_len, B, q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q)
    m = l = None
    if return_stats:
        m = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        l = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):
        st = lib().fa_fwd_dropout(B, H, N, d, _ptr(q), _ptr(k), _ptr(v),
                                  _ptr(o), _ptr(m), _ptr(l), _ptr(kv_len),
                                  int(bool(causal)), scale, float(p_drop),
                                  int(seed), int(offset), _stream(q))
    check("fa_fwd_dropout", st)
    return o, m, l


def bwd_dropout(q, k, v, o, do, m, l, p_drop, seed, offset=0, causal=False,
                kv_len=None, scale=None, workspace=None):
    """Gradients (dq, dk, dv) of fwd_dropout with the same p_drop, seed and
    offset (the mask is regenerated on chip); all bf16 [B,H,N,d]."""
    torch = _torch()
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check_dev(name, t, torch.bfloat16, (B, H, N, d))
    _check_dev("m", m, torch.float32, (B, H, N))
    _check_dev("l", l, torch.float32, (B, H, N))
    kv_len = _kv_len(kv_len, B, q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    workspace = _workspace(workspace, bwd_workspace_bytes(B, H, N, d),
                           q.device)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    with torch.cuda.device(q.device):
        st = lib().fa_bwd_dropout(B, H, N, d, _ptr(q), _ptr(k), _ptr(v),
                                  _ptr(o), _ptr(do), _ptr(m), _ptr(l),
                                  _ptr(kv_len), int(bool(causal)), scale,
                                  float(p_drop), int(seed), int(offset),
                                  _ptr(dq), _ptr(dk), _ptr(dv),
                                  _ptr(workspace), workspace.numel(),
                                  _stream(q))
    check("fa_bwd_dropout", st)
    return dq, dk, dv


def _block_mask(mask, H, N, device):
    torch = _torch()
    nb = (N + 127) // 128
    _check_dev("block_mask", mask, torch.uint8, (H, nb, nb))
    return mask


def fwd_block_sparse(q, k, v, block_mask, causal=False, scale=None,
                     return_stats=True):
    """Block-sparse attention: q, k, v [B,H,N,d] bf16; block_mask uint8
    [H, ceil(N/128), ceil(N/128)] (nonzero: the 128-query block attends the
    128-key block).  Returns (o, m, l)."""
    torch = _torch()
    B, H, N, d = q.shape
    _check_dev("q", q, torch.bfloat16)
    _check_dev("k", k, q.dtype, q.shape)
    _check_dev("v", v, q.dtype, q.shape)
    block_mask = _block_mask(block_mask, H, N, q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q)
    m = l = None
    if return_stats:
        m = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        l = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):
        st = lib().fa_fwd_block_sparse(B, H, N, d, _ptr(q), _ptr(k), _ptr(v),
                                       _ptr(o), _ptr(m), _ptr(l),
                                       _ptr(block_mask), int(bool(causal)),
                                       scale, _stream(q))
    check("fa_fwd_block_sparse", st)
    return o, m, l


def bwd_block_sparse(q, k, v, o, do, m, l, block_mask, causal=False,
                     scale=None, workspace=None):
    """Gradients (dq, dk, dv) of fwd_block_sparse; bf16 [B,H,N,d]."""
    torch = _torch()
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check_dev(name, t, torch.bfloat16, (B, H, N, d))
    _check_dev("m", m, torch.float32, (B, H, N))
    _check_dev("l", l, torch.float32, (B, H, N))
    block_mask = _block_mask(block_mask, H, N, q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    workspace = _workspace(
        workspace, bwd_block_sparse_workspace_bytes(B, H, N, d), q.device)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    with torch.cuda.device(q.device):
        st = lib().fa_bwd_block_sparse(B, H, N, d, _ptr(q), _ptr(k), _ptr(v),
                                       _ptr(o), _ptr(do), _ptr(m), _ptr(l),
                                       _ptr(block_mask), int(bool(causal)),
                                       scale, _ptr(dq), _ptr(dk), _ptr(dv),
                                       _ptr(workspace), workspace.numel(),
                                       _stream(q))
    check("fa_bwd_block_sparse", st)
    return dq, dk, dv


def _cu_seqlens(cu, device):
    torch = _torch()
    if not torch.is_tensor(cu):
        cu = torch.tensor(list(cu), dtype=torch.int32, device=device)
    _check_dev("cu_seqlens", cu, torch.int32)
    if cu.dim() != 1 or cu.numel() < 2:
        raise ValueError("cu_seqlens must be [B+1] with B >= 1")
    return cu


def fwd_varlen(q, k, v, cu_seqlens, max_seqlen, causal=False, scale=None,
               return_stats=True):
    """Exact attention on a packed ragged batch.  q, k, v: [H,total,d] bf16 or
    fp32 (head-major packed); sequence b is tokens cu_seqlens[b] ..
    cu_seqlens[b+1]-1 and attends only itself.  max_seqlen: at least every
    sequence's length.  Returns (o, m, l) with m, l fp32 [H,total]."""
    torch = _torch()
    H, total, d = q.shape
    _check_dev("q", q)
    _check_dev("k", k, q.dtype, q.shape)
    _check_dev("v", v, q.dtype, q.shape)
    cu = _cu_seqlens(cu_seqlens, q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q)
    m = l = None
    if return_stats:
        m = torch.empty((H, total), dtype=torch.float32, device=q.device)
        l = torch.empty((H, total), dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):
        st = lib().fa_fwd_varlen(_dtype_code(q), cu.numel() - 1, H, total,
                                 int(max_seqlen), d, _ptr(cu), _ptr(q),
                                 _ptr(k), _ptr(v), _ptr(o), _ptr(m), _ptr(l),
                                 int(bool(causal)), scale, _stream(q))
    check("fa_fwd_varlen", st)
    return o, m, l


def bwd_varlen_workspace_bytes(H, total, d):
    return int(lib().fa_bwd_varlen_workspace_bytes(H, total, d))


def bwd_varlen(q, k, v, o, do, m, l, cu_seqlens, max_seqlen, causal=False,
               scale=None, workspace=None):
    """Gradients (dq, dk, dv) for fwd_varlen; bf16 [H,total,d]."""
    torch = _torch()
    H, total, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check_dev(name, t, torch.bfloat16, (H, total, d))
    _check_dev("m", m, torch.float32, (H, total))
    _check_dev("l", l, torch.float32, (H, total))
    cu = _cu_seqlens(cu_seqlens, q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    workspace = _workspace(workspace, bwd_varlen_workspace_bytes(H, total, d),
                           q.device)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    with torch.cuda.device(q.device):
        st = lib().fa_bwd_varlen(cu.numel() - 1, H, total, int(max_seqlen), d,
                                 _ptr(cu), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                 _ptr(do), _ptr(m), _ptr(l),
                                 int(bool(causal)), scale, _ptr(dq), _ptr(dk),
                                 _ptr(dv), _ptr(workspace), workspace.numel(),
                                 _stream(q))
    check("fa_bwd_varlen", st)
    return dq, dk, dv


def _paged_cache_shape(k_cache, v_cache, d):
    """Checks a paged cache pair against head dim d: v_cache [num_blocks,
    Hkv, block_size, d], k_cache [num_blocks, Hkv, d/32, block_size, 32]
    (grouped).  Returns (num_blocks, Hkv, block_size)."""
    torch = _torch()
    _check_dev("v_cache", v_cache, torch.bfloat16)
    if v_cache.dim() != 4 or v_cache.shape[3] != d:
        raise ValueError("v_cache must be [num_blocks, Hkv, block_size, d]")
    nb, Hkv, bs, _ = v_cache.shape
    _check_dev("k_cache", k_cache, torch.bfloat16,
               (nb, Hkv, d // 32, bs, 32))
    return nb, Hkv, bs


def pack_k_cache(k_rows):
    """A K cache held by token ([num_blocks, Hkv, block_size, d]) in the
    library's grouped order [num_blocks, Hkv, d/32, block_size, 32]: entry
    [.., g, u, j] is element 32g + j of token u.  A layout change for callers
    that fill their cache by token; the paged calls read K in this order."""
    nb, Hkv, bs, d = k_rows.shape
    if d % 32:
        raise ValueError("d must be divisible by 32")
    return k_rows.reshape(nb, Hkv, bs, d // 32, 32).permute(
        0, 1, 3, 2, 4).contiguous()


def prefill_paged(q, k_cache, v_cache, block_table, seq_lens, cu_seqlens_q,
                  max_q, causal=True, scale=None, return_stats=True):
    """New tokens of each sequence (packed [Hq, total_q, d] bf16) against a
    paged cache (v_cache [num_blocks, Hkv, 16, d], k_cache grouped
    [num_blocks, Hkv, d/32, 16, 32], see pack_k_cache) that already holds
    them;
    sequence
    b's new tokens are its last cu[b+1]-cu[b] of seq_lens[b] positions.
    Returns (o, m, l) with m, l fp32 [Hq, total_q]."""
    torch = _torch()
    Hq, total_q, d = q.shape
    _check_dev("q", q, torch.bfloat16)
    nb, Hkv, bs = _paged_cache_shape(k_cache, v_cache, d)
    _check_dev("block_table", block_table, torch.int32)
    if block_table.dim() != 2:
        raise ValueError("block_table must be [B, max_blocks]")
    B = block_table.shape[0]
    _check_dev("seq_lens", seq_lens, torch.int32, (B,))
    cu = _cu_seqlens(cu_seqlens_q, q.device)
    if cu.numel() != B + 1:
        raise ValueError("cu_seqlens_q must be [B+1]")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q)
    m = l = None
    if return_stats:
        m = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device)
        l = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):
        st = lib().fa_prefill_paged(B, Hq, Hkv, d, total_q, int(max_q),
                                    _ptr(cu), _ptr(q), _ptr(k_cache),
                                    _ptr(v_cache), nb, bs, _ptr(block_table),
                                    block_table.shape[1], _ptr(seq_lens),
                                    int(bool(causal)), scale, _ptr(o),
                                    _ptr(m), _ptr(l), _stream(q))
    check("fa_prefill_paged", st)
    return o, m, l


def decode_workspace_bytes(B, Hq, d, num_splits):
    return int(lib().fa_decode_workspace_bytes(B, Hq, d, num_splits))


def decode_paged(q, k_cache, v_cache, block_table, seq_lens, num_splits=8,
                 scale=None, workspace=None):
    """Single-token GQA decode over a paged cache.

    q: [B,Hq,d] bf16; v_cache: [num_blocks, Hkv, block_size, d] bf16;
    k_cache: [num_blocks, Hkv, d/32, block_size, 32] bf16 (grouped, see
    pack_k_cache);
    block_table: int32 [B, max_blocks]; seq_lens: int32 [B].  Returns out
    [B,Hq,d] bf16.
    """
    torch = _torch()
    B, Hq, d = q.shape
    _check_dev("q", q, torch.bfloat16)
    nb, Hkv, bs = _paged_cache_shape(k_cache, v_cache, d)
    _check_dev("block_table", block_table, torch.int32)
    _check_dev("seq_lens", seq_lens, torch.int32, (B,))
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_blocks]")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    workspace = _workspace(workspace,
                           decode_workspace_bytes(B, Hq, d, num_splits),
                           q.device)
    out = torch.empty_like(q)
    with torch.cuda.device(q.device):
        st = lib().fa_decode_paged(B, Hq, Hkv, d, _ptr(q), _ptr(k_cache),
                                   _ptr(v_cache), nb, bs, _ptr(block_table),
                                   block_table.shape[1], _ptr(seq_lens),
                                   num_splits, scale, _ptr(out),
                                   _ptr(workspace), workspace.numel(),
                                   _stream(q))
    check("fa_decode_paged", st)
    return out


def decode_paged_noalloc(q, k_cache, v_cache, block_table, seq_lens,
                         num_splits=8, scale=None, out=None):
    """decode_paged through fa_decode_paged_noalloc: no workspace; the
    partials live in the library's fixed per-GPU scratch (calls on one GPU
    must not overlap).  `out` ([B,Hq,d] bf16) may be passed in, so that the
    call allocates nothing."""
    torch = _torch()
    B, Hq, d = q.shape
    _check_dev("q", q, torch.bfloat16)
    nb, Hkv, bs = _paged_cache_shape(k_cache, v_cache, d)
    _check_dev("block_table", block_table, torch.int32)
    _check_dev("seq_lens", seq_lens, torch.int32, (B,))
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_blocks]")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_dev("out", out, torch.bfloat16, q.shape)
    with torch.cuda.device(q.device):
        st = lib().fa_decode_paged_noalloc(
            B, Hq, Hkv, d, _ptr(q), _ptr(k_cache), _ptr(v_cache), nb, bs,
            _ptr(block_table), block_table.shape[1], _ptr(seq_lens),
            num_splits, scale, _ptr(out), _stream(q))
    check("fa_decode_paged_noalloc", st)
    return out
