"""GPU parity of fa_fwd_varlen / fa_bwd_varlen (packed ragged batches)
against the fp64 varlen oracle.

Small packings with ragged tails, empty sequences and sequences shorter than
one tile are compared in full; the 16-prompt prefill workload is compared on
sampled rows (every sequence's first and last token and random ones) for the
forward and on a reduced packing for the backward.  A packing with malformed
boundaries must stay inside its buffers.
"""

import numpy as np
import pytest

import oracle
from tests.helpers import BF16_TOL, F32_TOL, assert_close, to_device, to_numpy64
from workloads import TID_DO, WORKLOADS, normal

pytestmark = pytest.mark.gpu


def _cu(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def _fwd(q, k, v, cu, max_seqlen, causal):
    import torch
    import exact_io_aware_15_amd as fa
    cud = torch.from_numpy(cu).cuda()
    o, m, l = fa.fwd_varlen(to_device(q), to_device(k), to_device(v), cud,
                            max_seqlen, causal=causal)
    torch.cuda.synchronize()
    return to_numpy64(o), to_numpy64(m), to_numpy64(l)


def _check_fwd(name, q, k, v, cu, causal, tol, rows=None):
    max_seqlen = max(1, int(np.max(np.diff(cu))))
    o, m, l = _fwd(q, k, v, cu, max_seqlen, causal)
    ro, rm, rl = oracle.attention_fwd_varlen(q.exact, k.exact, v.exact, cu,
                                             None, causal, rows=rows)
    if rows is not None:
        o, m, l = o[:, rows], m[:, rows], l[:, rows]
    assert_close(name + ".o", o, ro, tol)
    assert np.max(np.abs(m - rm) / np.maximum(1, np.abs(rm))) <= 1e-5
    # l sums the bf16-rounded p (8 significant bits: relative error <= 2^-8
    # per term)
    lr = 2.0 ** -8 + 1e-5 if tol is BF16_TOL else 1e-5
    assert np.max(np.abs(l / rl - 1)) <= lr, name + ".l"


SMALL = [  # (lens, H, d, causal)
    ([1], 1, 64, False),
    ([130, 0, 64, 1, 200, 7], 2, 64, True),
    ([130, 0, 64, 1, 200, 7], 2, 64, False),
    ([333, 129, 5], 3, 64, True),
    ([100, 257, 0, 31], 2, 128, True),
    ([100, 257, 0, 31], 2, 128, False),
]


@pytest.mark.parametrize("lens,H,d,causal", SMALL)
def test_varlen_fwd_small(lens, H, d, causal):
    cu = _cu(lens)
    seed = 3000 + int(cu[-1]) + d + 7 * causal
    shape = (H, int(cu[-1]), d)
    q, k, v = (normal(shape, seed, t, "bf16") for t in range(3))
    print(f"varlen fwd lens={lens} H={H} d={d} causal={causal}", flush=True)
    _check_fwd("small", q, k, v, cu, causal, BF16_TOL)


def test_varlen_fwd_f32():
    lens = [70, 0, 129, 1]
    cu = _cu(lens)
    q, k, v = (normal((2, int(cu[-1]), 64), 3101, t, "f32") for t in range(3))
    print("varlen fwd f32", flush=True)
    _check_fwd("f32", q, k, v, cu, True, F32_TOL)


def test_varlen_single_sequence_equals_dense():
    import torch
    import exact_io_aware_15_amd as fa
    q, k, v = (normal((1, 2, 300, 64), 3102, t, "bf16") for t in range(3))
    qd, kd, vd = (to_device(x) for x in (q, k, v))
    od, md, ld = fa.fwd(qd, kd, vd, causal=True)
    cu = torch.tensor([0, 300], dtype=torch.int32, device="cuda")
    ov, mv, lv = fa.fwd_varlen(qd[0], kd[0], vd[0], cu, 300, causal=True)
    torch.cuda.synchronize()
    # same kernel, same tiles: identical bits
    assert torch.equal(od[0], ov) and torch.equal(md[0], mv)
    assert torch.equal(ld[0], lv)


def test_varlen_prefill_workload_sampled_rows():
    w = WORKLOADS["varlen_causal_prefill"]
    cu, q, k, v = w.varlen_inputs()
    rng = np.random.default_rng(3103)
    edges = np.concatenate([cu[:-1], cu[1:] - 1])
    rows = np.unique(np.concatenate(
        [edges[edges >= 0], rng.integers(0, int(cu[-1]), 200)]))
    print(f"varlen workload {w.name} rows={rows.size}", flush=True)
    o, m, l = _fwd(q, k, v, cu, w.N, True)
    ro, rm, _ = oracle.attention_fwd_varlen(q.exact, k.exact, v.exact, cu,
                                            None, True, rows=rows)
    assert_close("prefill.o", o[:, rows], ro, BF16_TOL)
    assert np.max(np.abs(m[:, rows] - rm) / np.maximum(1, np.abs(rm))) <= 1e-5


def _bwd_case(lens, H, d, causal, seed):
    import torch
    import exact_io_aware_15_amd as fa
    cu = _cu(lens)
    total = int(cu[-1])
    q, k, v = (normal((H, total, d), seed, t, "bf16") for t in range(3))
    do = normal((H, total, d), seed, TID_DO, "bf16")
    max_seqlen = max(1, int(np.max(np.diff(cu))))
    qd, kd, vd, dod = (to_device(x) for x in (q, k, v, do))
    cud = torch.from_numpy(cu).cuda()
    o, m, l = fa.fwd_varlen(qd, kd, vd, cud, max_seqlen, causal=causal)
    g = fa.bwd_varlen(qd, kd, vd, o, dod, m, l, cud, max_seqlen,
                      causal=causal)
    torch.cuda.synchronize()
    dq, dk, dv = (to_numpy64(x) for x in g)
    rq, rk, rv, _ = oracle.attention_bwd_varlen(q.exact, k.exact, v.exact,
                                                do.exact, cu, None, causal)
    assert_close("dq", dq, rq, BF16_TOL)
    assert_close("dk", dk, rk, BF16_TOL)
    assert_close("dv", dv, rv, BF16_TOL)


BWD = [  # (lens, H, d, causal)
    ([130, 0, 64, 1, 200, 7], 2, 64, True),
    ([130, 0, 64, 1, 200, 7], 2, 64, False),
    ([100, 257, 0, 31], 1, 128, True),
    ([700, 1500, 33, 2100, 900], 2, 64, True),
]


@pytest.mark.parametrize("lens,H,d,causal", BWD)
def test_varlen_bwd(lens, H, d, causal):
    print(f"varlen bwd lens={lens} H={H} d={d} causal={causal}", flush=True)
    _bwd_case(lens, H, d, causal, 3200 + sum(lens) + d + causal)


def test_varlen_empty_batch_is_a_no_op():
    import torch
    import exact_io_aware_15_amd as fa
    z = torch.empty((2, 0, 64), dtype=torch.bfloat16, device="cuda")
    cu = torch.zeros(3, dtype=torch.int32, device="cuda")
    o, m, l = fa.fwd_varlen(z, z, z, cu, 1)
    assert o.shape == (2, 0, 64)
