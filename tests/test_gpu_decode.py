"""GPU parity of fa_decode_paged against the fp64 oracle (through the C ABI).

Slots past each sequence's length hold NaN in the cache (``paged_cache``
poisons them), so any kernel that multiplies them fails the finiteness check.
"""

import numpy as np
import pytest

import oracle
from tests.helpers import BF16_TOL, assert_close, to_device, to_numpy64
from workloads import WORKLOADS, normal, paged_cache

pytestmark = pytest.mark.gpu


def _run(q, cache, splits, table=None):
    import torch
    import exact_io_aware_15_amd as fa
    table = cache.block_table if table is None else table
    out = fa.decode_paged(
        to_device(q), to_device(cache.k_cache), to_device(cache.v_cache),
        torch.from_numpy(table).cuda(), torch.from_numpy(cache.seq_lens).cuda(),
        num_splits=splits)
    torch.cuda.synchronize()
    return to_numpy64(out)


def _ref(q, cache):
    return oracle.decode_paged(q.exact, cache.k_cache.exact,
                               cache.v_cache.exact, cache.block_table,
                               cache.seq_lens)


@pytest.mark.parametrize("splits", [1, 3, 8, 64])
def test_decode_workload(splits):
    w = WORKLOADS["paged_gqa_decode"]
    q, cache = w.decode_inputs(poison_tails=True)
    print(f"decode workload splits={splits}", flush=True)
    assert_close("decode.out", _run(q, cache, splits), _ref(q, cache),
                 BF16_TOL)


CASES = [  # (B, Hq, Hkv, d, lens)
    (4, 8, 8, 128, [1, 15, 16, 17]),
    (3, 8, 4, 128, [0, 33, 200]),
    (2, 16, 2, 128, [100, 257]),
    (3, 32, 2, 64, [5, 64, 1000]),
    (2, 4, 1, 64, [16, 31]),
    # group sizes that are not a power of two (run on the next one's kernel)
    (3, 12, 4, 128, [1, 40, 333]),     # G = 3
    (2, 10, 2, 128, [17, 250]),        # G = 5
    (2, 12, 2, 64, [64, 129]),         # G = 6
    (2, 12, 1, 128, [7, 300]),         # G = 12
]


@pytest.mark.parametrize("B,Hq,Hkv,d,lens", CASES)
@pytest.mark.parametrize("splits", [1, 4])
def test_decode_shapes(B, Hq, Hkv, d, lens, splits):
    seed = 3000 + Hq * 7 + Hkv + d + sum(lens)
    max_blocks = -(-max(lens) // 16) + 2
    cache = paged_cache(lens, Hkv, d, 16, max_blocks, seed, poison_tails=True)
    q = normal((B, Hq, d), seed, 0, "bf16")
    print(f"decode B={B} Hq={Hq} Hkv={Hkv} d={d} lens={lens} splits={splits}",
          flush=True)
    out = _run(q, cache, splits)
    assert_close("decode.out", out, _ref(q, cache), BF16_TOL)
    for b, L in enumerate(lens):
        if L == 0:
            assert np.all(out[b] == 0)


def test_decode_invariant_to_block_placement():
    """Moving the blocks to other physical slots (and rewriting the table)
    must not change a single output bit."""
    import torch
    lens = [300, 17, 64]
    cache = paged_cache(lens, 2, 128, 16, 24, 3100, poison_tails=True)
    q = normal((3, 8, 128), 3100, 0, "bf16")
    out1 = _run(q, cache, 4)
    nb = cache.k_cache.store.shape[0]
    perm = np.random.default_rng(1).permutation(nb)
    kc = np.empty_like(cache.k_cache.store)
    vc = np.empty_like(cache.v_cache.store)
    kc[perm] = cache.k_cache.store
    vc[perm] = cache.v_cache.store
    cache.k_cache.store, cache.v_cache.store = kc, vc
    table = np.where(cache.block_table >= 0,
                     perm[np.maximum(cache.block_table, 0)], -1).astype(np.int32)
    out2 = _run(q, cache, 4, table=table)
    assert np.array_equal(out1, out2)
    del torch


@pytest.mark.parametrize("lens,splits", [
    # more than 64 sequences: every sequence is split into equal parts
    ([17 + (37 * i) % 400 for i in range(70)], 4),
    # exactly 64 sequences: the largest batch that gets the split plan
    ([1 + (53 * i) % 700 for i in range(64)], 3),
    # tied lengths: slots go longest first, ties by sequence index
    ([300, 300, 17, 300, 17, 1, 300, 0, 300], 3),
    # one split per sequence
    ([5, 1000, 0, 160], 1),
    # a single sequence over 63 partitions of a few blocks each
    ([4000], 64),
    # one long sequence among short ones: most partitions go to it
    ([3000, 1, 2, 16, 17], 2),
    # every sequence empty: no partition runs, every output is 0
    ([0, 0, 0], 4),
    # 300 sequences x 64 splits x 2 KV heads: 38,400 workgroups in the
    # one-dimensional grid, dealt over many rounds with a partial last one
    ([1 + (7919 * i) % 100 for i in range(300)], 64),
])
def test_decode_split_plan_cases(lens, splits):
    B, Hq, Hkv, d = len(lens), 8, 2, 128
    seed = 3200 + B
    max_blocks = -(-max(lens) // 16) + 1
    cache = paged_cache(lens, Hkv, d, 16, max_blocks, seed, poison_tails=True)
    q = normal((B, Hq, d), seed, 0, "bf16")
    print(f"decode split plan B={B} splits={splits}", flush=True)
    out = _run(q, cache, splits)
    assert_close("decode.out", out, _ref(q, cache), BF16_TOL)
    for b, L in enumerate(lens):
        if L == 0:
            assert np.all(out[b] == 0)
