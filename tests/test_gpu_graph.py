"""The hot path under HIP graph capture.

Every entry point is captured once and replayed several times: fa_fwd +
fa_bwd, the paged decode (with a workspace and without one), varlen,
block-sparse and dropout forward + backward, the FP8 forward and the paged
prefill.  Between replays the inputs
are rewritten in place by eager work, with a synchronisation before each
replay.  Every replay must equal, bit for bit, an eager call on the same
inputs.  The kernels are deterministic, and the calls allocate nothing,
wait for nothing on the host and clear no memory with hipMemsetAsync, so
a captured call behaves like an eager one."""

import os

import pytest

from workloads import TID_DO, normal, paged_cache, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _release_build_only():
    if os.environ.get("FA355_DEBUG", "0") not in ("", "0"):
        pytest.skip("the debug build reads its contract checks back on the "
                    "host, which a captured stream cannot do")


def _capture(step, args):
    """Warm up on a side stream, then capture step(*args) into a graph."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(*args)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = step(*args)
    return graph, outs


@pytest.mark.parametrize("causal,padded", [(True, False), (False, True)])
def test_fwd_bwd_graph_replays_match_eager(causal, padded):
    import torch
    import exact_io_aware_15_amd as fa
    B, H, N, d = 2, 3, 333, 64

    def inputs(seed):
        x = [to_device(normal((B, H, N, d), seed, t, "bf16")) for t in range(3)]
        return x + [to_device(normal((B, H, N, d), seed, TID_DO, "bf16"))]

    kv = (torch.tensor([N, 200], dtype=torch.int32, device="cuda")
          if padded else None)

    def step(q, k, v, do):
        o, m, l = fa.fwd(q, k, v, causal=causal, kv_len=kv)
        dq, dk, dv = fa.bwd(q, k, v, o, do, m, l, causal=causal, kv_len=kv)
        return o, m, l, dq, dk, dv

    static = inputs(11)
    graph, outs = _capture(step, static)
    for rep in range(4):
        print(f"graph fwd+bwd causal={causal} padded={padded} replay {rep}",
              flush=True)
        fresh = inputs(300 + rep)
        for s, f in zip(static, fresh):
            s.copy_(f)
        want = [x.clone() for x in step(*fresh)]
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, ref in zip(("o", "m", "l", "dq", "dk", "dv"), outs,
                                  want):
            assert torch.equal(got, ref), f"replay {rep}: {name}"


def test_decode_graph_replays_match_eager():
    import torch
    import exact_io_aware_15_amd as fa
    lens, Hkv, G, d, splits = [37, 300, 1000, 5], 2, 4, 128, 8
    B, Hq = len(lens), Hkv * G
    max_blocks = -(-max(lens) // 16) + 1
    cache = paged_cache(lens, Hkv, d, 16, max_blocks, 21, poison_tails=True)
    q = to_device(normal((B, Hq, d), 21, 0, "bf16"))
    kc, vc = to_device(cache.k_cache), to_device(cache.v_cache)
    table = torch.from_numpy(cache.block_table).cuda()
    seq = torch.from_numpy(cache.seq_lens).cuda()
    ws = torch.empty(fa.decode_workspace_bytes(B, Hq, d, splits),
                     dtype=torch.uint8, device="cuda")
    out_na = torch.empty_like(q)
    # The no-allocation call finds its scratch array on its first call on
    # a device; make that call before the capture.
    fa.decode_paged_noalloc(q, kc, vc, table, seq, splits, out=out_na)

    def step():
        out = fa.decode_paged(q, kc, vc, table, seq, splits, workspace=ws)
        fa.decode_paged_noalloc(q, kc, vc, table, seq, splits, out=out_na)
        return out

    graph, out = _capture(step, ())
    for rep in range(4):
        print(f"graph decode replay {rep}", flush=True)
        q.copy_(to_device(normal((B, Hq, d), 500 + rep, 0, "bf16")))
        vc.mul_(-1.0)
        want = fa.decode_paged(q, kc, vc, table, seq, splits)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"replay {rep}: decode"
        assert torch.equal(out_na, want), f"replay {rep}: decode (no alloc)"


def _replays_match_eager(name, make, step, reps=3):
    """make(seed) -> list of device tensors; step(*tensors) -> outputs.  The
    graph is captured on the tensors of make(1); each replay first rewrites
    them in place with make(seed) for a new seed."""
    import torch
    static = make(1)
    graph, outs = _capture(step, static)
    for rep in range(reps):
        print(f"graph {name} replay {rep}", flush=True)
        fresh = make(700 + rep)
        for s, f in zip(static, fresh):
            s.copy_(f)
        want = [x.clone() for x in step(*fresh)]
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (got, ref) in enumerate(zip(outs, want)):
            assert torch.equal(got, ref), f"{name} replay {rep}: output {i}"


def test_varlen_graph_replays_match_eager():
    import numpy as np
    import torch
    import exact_io_aware_15_amd as fa
    lens, H, d = [130, 1, 77, 256], 2, 64
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32),
                      device="cuda")
    total = int(sum(lens))

    def make(seed):
        return [to_device(normal((H, total, d), seed, t, "bf16"))
                for t in (0, 1, 2, TID_DO)]

    def step(q, k, v, do):
        o, m, l = fa.fwd_varlen(q, k, v, cu, max(lens), causal=True)
        return (o, m, l) + tuple(fa.bwd_varlen(q, k, v, o, do, m, l, cu,
                                               max(lens), causal=True))

    _replays_match_eager("varlen", make, step)


def test_block_sparse_graph_replays_match_eager():
    import numpy as np
    import torch
    import exact_io_aware_15_amd as fa
    B, H, N, d = 1, 2, 300, 64
    nb = -(-N // 128)
    mask = torch.from_numpy(
        (np.random.default_rng(5).random((H, nb, nb)) < 0.6).astype(
            np.uint8)).cuda()

    def make(seed):
        return [to_device(normal((B, H, N, d), seed, t, "bf16"))
                for t in (0, 1, 2, TID_DO)]

    def step(q, k, v, do):
        o, m, l = fa.fwd_block_sparse(q, k, v, mask, causal=True)
        return (o, m, l) + tuple(fa.bwd_block_sparse(q, k, v, o, do, m, l,
                                                     mask, causal=True))

    _replays_match_eager("block-sparse", make, step)


def test_dropout_graph_replays_match_eager():
    import exact_io_aware_15_amd as fa
    B, H, N, d = 1, 2, 200, 64

    def make(seed):
        return [to_device(normal((B, H, N, d), seed, t, "bf16"))
                for t in (0, 1, 2, TID_DO)]

    def step(q, k, v, do):
        o, m, l = fa.fwd_dropout(q, k, v, 0.2, 1234, 7, causal=True)
        return (o, m, l) + tuple(fa.bwd_dropout(q, k, v, o, do, m, l, 0.2,
                                                1234, 7, causal=True))

    _replays_match_eager("dropout", make, step)


def test_fp8_graph_replays_match_eager():
    import numpy as np
    import torch
    import exact_io_aware_15_amd as fa
    from workloads import normal_fp8
    shape = (1, 2, 333, 128)

    def dev(x):
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()

    def make(seed):
        (q, qd), (k, kd), (v, vd) = (normal_fp8(shape, seed, t, transpose=t == 2)
                                     for t in range(3))
        return [dev(q.store), dev(k.store), dev(v.store),
                dev(np.asarray(qd, np.float32)), dev(np.asarray(kd, np.float32)),
                dev(np.asarray(vd, np.float32))]

    def step(q8, k8, v8, qd, kd, vd):
        return fa.fwd_fp8(q8, k8, v8, qd, kd, vd, causal=True)

    _replays_match_eager("fp8", make, step)


def test_prefill_graph_replays_match_eager():
    import numpy as np
    import torch
    import exact_io_aware_15_amd as fa
    ctx, new, Hkv, G, d = [300, 40, 129], [64, 1, 129], 2, 2, 128
    lens = [c + n for c, n in zip(ctx, new)]
    max_blocks = -(-max(lens) // 16) + 1
    cache = paged_cache(lens, Hkv, d, 16, max_blocks, 31, poison_tails=True)
    kc, vc = to_device(cache.k_cache), to_device(cache.v_cache)
    table = torch.from_numpy(cache.block_table).cuda()
    seq = torch.from_numpy(cache.seq_lens).cuda()
    cu = torch.tensor(np.concatenate([[0], np.cumsum(new)]).astype(np.int32),
                      device="cuda")
    total = int(sum(new))

    def make(seed):
        return [to_device(normal((Hkv * G, total, d), seed, 0, "bf16"))]

    def step(q):
        return fa.prefill_paged(q, kc, vc, table, seq, cu, max(new),
                                causal=True)

    _replays_match_eager("prefill", make, step)
