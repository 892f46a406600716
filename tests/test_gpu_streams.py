"""Calls on several streams at once.

The library keeps no state between calls (apart from the no-allocation
decode's per-GPU scratch, which is documented as not shared between
concurrent calls and is not used here): a dense forward + backward, a varlen
forward + backward and a paged decode, enqueued on three streams of default
priority without waiting for each other, must give exactly the outputs of
the same calls made one after another on the default stream."""

import numpy as np
import pytest

from workloads import TID_DO, normal, paged_cache, to_device

pytestmark = pytest.mark.gpu


def test_concurrent_streams_match_sequential():
    import torch
    import exact_io_aware_15_amd as fa

    B, H, N, d = 1, 4, 1000, 64
    dense = [to_device(normal((B, H, N, d), 41, t, "bf16"))
             for t in (0, 1, 2, TID_DO)]
    lens = [300, 1, 512]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32),
                      device="cuda")
    total = int(sum(lens))
    packed = [to_device(normal((2, total, 128), 42, t, "bf16"))
              for t in (0, 1, 2, TID_DO)]
    dlens = [700, 33, 2000, 64]
    cache = paged_cache(dlens, 2, 128, 16, -(-max(dlens) // 16) + 1, 43,
                        poison_tails=True)
    qdec = to_device(normal((len(dlens), 8, 128), 43, 0, "bf16"))
    kc, vc = to_device(cache.k_cache), to_device(cache.v_cache)
    table = torch.from_numpy(cache.block_table).cuda()
    seq = torch.from_numpy(cache.seq_lens).cuda()

    def run_dense():
        q, k, v, do = dense
        o, m, l = fa.fwd(q, k, v, causal=True)
        return (o, m, l) + tuple(fa.bwd(q, k, v, o, do, m, l, causal=True))

    def run_varlen():
        q, k, v, do = packed
        o, m, l = fa.fwd_varlen(q, k, v, cu, max(lens), causal=True)
        return (o, m, l) + tuple(fa.bwd_varlen(q, k, v, o, do, m, l, cu,
                                               max(lens), causal=True))

    def run_decode():
        return (fa.decode_paged(qdec, kc, vc, table, seq, num_splits=8),)

    jobs = (run_dense, run_varlen, run_decode)
    want = [[x.clone() for x in job()] for job in jobs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in jobs]
    for rep in range(3):
        print(f"streams replay {rep}", flush=True)
        start = torch.cuda.current_stream()
        got = []
        for job, st in zip(jobs, streams):
            st.wait_stream(start)
            with torch.cuda.stream(st):
                got.append(job())
        for st in streams:
            torch.cuda.current_stream().wait_stream(st)
        torch.cuda.synchronize()
        for j, (outs, refs) in enumerate(zip(got, want)):
            for i, (x, y) in enumerate(zip(outs, refs)):
                assert torch.equal(x, y), f"rep {rep}: job {j} output {i}"
