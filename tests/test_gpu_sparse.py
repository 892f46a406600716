"""GPU parity of fa_fwd_block_sparse / fa_bwd_block_sparse against the fp64
block-sparse oracle: random masks with ragged last blocks, fully masked
rows, causal and not, d = 64 and 128, masks wider than the kernels' 64-block
ballot window (forward and full gradients); an all-ones mask must reproduce
the dense kernel bit for bit; the 16K workload is compared on sampled
rows."""

import numpy as np
import pytest

import oracle
from tests.helpers import BF16_TOL, assert_close, to_device, to_numpy64
from workloads import TID_DO, WORKLOADS, block_sparse_mask, normal

pytestmark = pytest.mark.gpu


def _mask(H, N, density, seed, empty_row=None):
    nb = -(-N // 128)
    rng = np.random.default_rng(seed)
    m = (rng.random((H, nb, nb)) < density).astype(np.uint8)
    if empty_row is not None:
        m[:, empty_row, :] = 0
    return m


def _run(q, k, v, mask, causal, do=None):
    import torch
    import exact_io_aware_15_amd as fa
    qd, kd, vd = (to_device(x) for x in (q, k, v))
    md = torch.from_numpy(mask).cuda()
    o, m, l = fa.fwd_block_sparse(qd, kd, vd, md, causal=causal)
    g = None
    if do is not None:
        g = fa.bwd_block_sparse(qd, kd, vd, o, to_device(do), m, l, md,
                                causal=causal)
    torch.cuda.synchronize()
    out = [to_numpy64(x) for x in (o, m, l)]
    return out, (None if g is None else [to_numpy64(x) for x in g])


CASES = [  # (B, H, N, d, causal, density, empty_row)
    (1, 2, 600, 64, False, 0.4, 2),
    (2, 2, 600, 64, True, 0.6, 1),
    (1, 2, 384, 128, False, 0.5, None),
    (1, 1, 521, 128, True, 0.5, 0),
]


@pytest.mark.parametrize("B,H,N,d,causal,density,empty_row", CASES)
def test_block_sparse_fwd_bwd(B, H, N, d, causal, density, empty_row):
    seed = 5000 + N + d + causal
    q, k, v = (normal((B, H, N, d), seed, t, "bf16") for t in range(3))
    do = normal((B, H, N, d), seed, TID_DO, "bf16")
    mask = _mask(H, N, density, seed, empty_row)
    print(f"block-sparse B={B} H={H} N={N} d={d} causal={causal} "
          f"density={mask.mean():.2f}", flush=True)
    (o, m, l), (dq, dk, dv) = _run(q, k, v, mask, causal, do)
    ro, rm, rl = oracle.attention_fwd_block_sparse(q.exact, k.exact, v.exact,
                                                   mask, 128, None, causal)
    assert_close("o", o, ro, BF16_TOL)
    vis = np.isfinite(rm)
    assert np.array_equal(np.isfinite(m), vis)
    assert np.max(np.abs(m[vis] - rm[vis]) / np.maximum(1, np.abs(rm[vis]))) \
        <= 1e-5
    assert np.all(o[~vis] == 0) and np.all(l[~vis] == 0)
    rq, rk, rv, _ = oracle.attention_bwd_block_sparse(
        q.exact, k.exact, v.exact, do.exact, mask, 128, None, causal)
    assert_close("dq", dq, rq, BF16_TOL)
    assert_close("dk", dk, rk, BF16_TOL)
    assert_close("dv", dv, rv, BF16_TOL)


# More than 64 mask blocks per row and column (N > 64 * 128): the mask walks
# of the forward and dQ kernels (along a mask row) and of the dK/dV kernel
# (down a mask column, stride nb) re-ballot when they cross from the first
# 64-block window into the second.  Some rows and columns allow only blocks
# of the second window, so a walk must skip the whole first window; one row
# and one column allow nothing at all.
WIDE = [  # (N, d, causal, density)
    (8448, 64, False, 0.25),
    (8448 + 37, 64, True, 0.5),
    (8448, 128, True, 0.3),
]


def _wide_mask(N, density, seed):
    nb = -(-N // 128)
    assert nb > 64
    m = _mask(1, N, density, seed)
    m[0, 3, :] = 0
    m[0, 3, 65] = 1            # row 3: only a block of the second window
    m[0, :, 2] = 0
    m[0, 64, 2] = m[0, 65, 2] = 1  # column 2: only second-window blocks
    m[0, 10, :] = 0            # a row with no allowed block
    m[0, :, 11] = 0            # a column with no allowed block
    m[0, nb - 1, 0] = 1        # the last row reaches back to block 0
    return m


@pytest.mark.parametrize("N,d,causal,density", WIDE)
def test_block_sparse_wider_than_one_ballot_window(N, d, causal, density):
    seed = 5200 + N + d + causal
    q, k, v = (normal((1, 1, N, d), seed, t, "bf16") for t in range(3))
    do = normal((1, 1, N, d), seed, TID_DO, "bf16")
    mask = _wide_mask(N, density, seed)
    print(f"block-sparse wide N={N} d={d} causal={causal} "
          f"blocks={mask.shape[1]} density={mask.mean():.2f}", flush=True)
    (o, m, l), (dq, dk, dv) = _run(q, k, v, mask, causal, do)
    ro, rm, rl = oracle.attention_fwd_block_sparse(q.exact, k.exact, v.exact,
                                                   mask, 128, None, causal)
    assert_close("wide.o", o, ro, BF16_TOL)
    vis = np.isfinite(rm)
    assert np.array_equal(np.isfinite(m), vis)
    assert np.all(o[~vis] == 0) and np.all(l[~vis] == 0)
    rq, rk, rv, _ = oracle.attention_bwd_block_sparse(
        q.exact, k.exact, v.exact, do.exact, mask, 128, None, causal)
    assert_close("wide.dq", dq, rq, BF16_TOL)
    assert_close("wide.dk", dk, rk, BF16_TOL)
    assert_close("wide.dv", dv, rv, BF16_TOL)
    # keys of a column with no allowed block get exactly zero gradients
    assert np.all(dk[0, 0, 11 * 128:12 * 128] == 0)
    assert np.all(dv[0, 0, 11 * 128:12 * 128] == 0)


def test_all_ones_mask_matches_dense_kernel_bitwise():
    import torch
    import exact_io_aware_15_amd as fa
    q, k, v = (to_device(normal((2, 2, 500, 64), 5101, t, "bf16"))
               for t in range(3))
    mask = torch.ones((2, 4, 4), dtype=torch.uint8, device="cuda")
    for causal in (False, True):
        od, md, ld = fa.fwd(q, k, v, causal=causal)
        os_, ms, ls = fa.fwd_block_sparse(q, k, v, mask, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(od, os_) and torch.equal(md, ms)


def test_block_sparse_workload_sampled_rows():
    w = WORKLOADS["block_sparse_16k"]
    q, k, v = w.qkv()
    mask = block_sparse_mask(w.H, w.N)
    rng = np.random.default_rng(5102)
    rows = np.unique(np.concatenate([[0, 127, 128, w.N - 1],
                                     rng.integers(0, w.N, 60)]))
    print(f"block-sparse workload rows={rows.size}", flush=True)
    (o, _, _), _ = _run(q, k, v, mask, False)
    ro, _, _ = oracle.attention_fwd_block_sparse(
        q.exact[:, :2], k.exact[:, :2], v.exact[:, :2], mask[:2], 128, None,
        False, rows=rows)
    assert_close("workload.o", o[:, :2, rows], ro, BF16_TOL)
