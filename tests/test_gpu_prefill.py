"""GPU parity of fa_prefill_paged (packed new tokens against a paged KV cache)
against the fp64 oracle.

Small cases cover GQA, chunks longer than one 128-query tile, contexts that
end mid-block, no earlier context, one new token, sequences with no new token
and NaN in every cache slot past a sequence's length; the chunked-prefill
workload is compared on sampled rows.
"""

import numpy as np
import pytest

import oracle
from tests.helpers import BF16_TOL, assert_close, to_device, to_numpy64
from workloads import WORKLOADS, normal, paged_cache

pytestmark = pytest.mark.gpu


def _gpu(q, cache, cu, causal, max_q=None):
    import torch
    import exact_io_aware_15_amd as fa
    max_q = max(1, int(np.max(np.diff(cu)))) if max_q is None else max_q
    o, m, l = fa.prefill_paged(
        to_device(q), to_device(cache.k_cache), to_device(cache.v_cache),
        torch.from_numpy(cache.block_table).cuda(),
        torch.from_numpy(cache.seq_lens).cuda(),
        torch.from_numpy(np.asarray(cu, np.int32)).cuda(), max_q,
        causal=causal)
    torch.cuda.synchronize()
    return to_numpy64(o), to_numpy64(m), to_numpy64(l)


CASES = [  # (ctx lens, new-token counts, Hq, Hkv, d, causal)
    ([300], [300], 2, 2, 64, True),                  # no earlier context
    ([1, 17, 200], [1, 1, 1], 4, 1, 64, True),        # one new token each
    ([517, 40, 1000, 33], [200, 40, 7, 0], 8, 2, 64, True),
    ([517, 40, 1000, 33], [200, 40, 7, 0], 8, 2, 64, False),
    ([700, 129], [300, 100], 8, 8, 128, True),
    ([700, 129], [300, 100], 4, 2, 128, False),
    # contexts of whole 64-key tiles: the last tile is whole too
    ([256, 640], [64, 640], 4, 2, 64, True),
    ([640, 256], [100, 256], 8, 2, 128, False),
    # workgroups take sequences longest first: equal lengths (ties keep
    # index order), and more than 64 sequences (taken in their own order)
    ([300, 300, 300], [120, 7, 300], 4, 2, 128, True),
    ([17 + (37 * i) % 200 for i in range(70)],
     [1 + (11 * i) % (17 + (37 * i) % 200) for i in range(70)], 2, 1, 64,
     True),
]


@pytest.mark.parametrize("ctx,qlen,Hq,Hkv,d,causal", CASES)
def test_prefill_small(ctx, qlen, Hq, Hkv, d, causal):
    seed = 4000 + sum(ctx) + sum(qlen) + d + causal
    cu = np.concatenate([[0], np.cumsum(qlen)]).astype(np.int32)
    max_blocks = max(-(-c // 16) for c in ctx) + 2
    cache = paged_cache(ctx, Hkv, d, 16, max_blocks, seed, poison_tails=True)
    q = normal((Hq, int(cu[-1]), d), seed, 9, "bf16")
    print(f"prefill ctx={ctx} qlen={qlen} Hq={Hq} Hkv={Hkv} d={d} "
          f"causal={causal}", flush=True)
    o, m, l = _gpu(q, cache, cu, causal)
    ro, rm, rl = oracle.prefill_paged(q.exact, cache.k_cache.exact,
                                      cache.v_cache.exact, cache.block_table,
                                      cache.seq_lens, cu, None, causal)
    assert_close("prefill.o", o, ro, BF16_TOL)
    assert np.max(np.abs(m - rm) / np.maximum(1, np.abs(rm))) <= 1e-5
    # l sums bf16-rounded p: at most 2^-8 relative error per term
    assert np.max(np.abs(l / rl - 1)) <= 2.0 ** -8 + 1e-5


def test_prefill_workload_sampled_rows():
    w = WORKLOADS["paged_chunked_prefill"]
    cu, q, cache = w.prefill_inputs(poison_tails=True)
    rng = np.random.default_rng(4101)
    edges = np.concatenate([cu[:-1], cu[1:] - 1])
    rows = np.unique(np.concatenate([edges, rng.integers(0, int(cu[-1]), 60)]))
    print(f"prefill workload rows={rows.size}", flush=True)
    o, _, _ = _gpu(q, cache, cu, True, max_q=w.seq_range[1])
    # the oracle on the sampled rows only: rebuild a packing of those rows
    # as one-token chunks at their own positions
    seq = np.searchsorted(cu, rows, side="right") - 1
    ref = []
    for r, b in zip(rows, seq):
        L = int(cache.seq_lens[b])
        pos = L - int(cu[b + 1] - cu[b]) + int(r - cu[b])
        # new token at position pos sees the first pos + 1 cached tokens:
        # a one-token chunk of a sequence cut to pos + 1 tokens
        table = cache.block_table[b:b + 1]
        o1, _, _ = oracle.prefill_paged(q.exact[:, r:r + 1],
                                        cache.k_cache.exact,
                                        cache.v_cache.exact, table,
                                        [pos + 1], [0, 1], None, True)
        ref.append(o1[:, 0])
    ref = np.stack(ref, axis=1)
    assert_close("prefill_workload.o", o[:, rows], ref, BF16_TOL)
