"""The Python binding rejects malformed tensors before anything reaches the
library: host tensors, non-contiguous views, wrong dtypes or shapes, and a
caller's workspace that is not a uint8 tensor on the inputs' device (the
library itself rejects a workspace that is too small)."""

import pytest


def _host(shape, dtype):
    import torch
    return torch.zeros(shape, dtype=dtype)


def test_host_tensors_are_rejected():
    import torch
    import exact_io_aware_15_amd as fa
    bf = torch.bfloat16
    q = _host((1, 1, 8, 64), bf)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.fwd(q, q, q)
    m = _host((1, 1, 8), torch.float32)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.bwd(q, q, q, q, q, m, m)
    qd = _host((2, 4, 128), bf)
    vc = _host((3, 1, 16, 128), bf)
    kc = _host((3, 1, 4, 16, 32), bf)
    table = _host((2, 3), torch.int32)
    lens = _host((2,), torch.int32)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.decode_paged(qd, kc, vc, table, lens)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.fwd_varlen(_host((1, 8, 64), bf), _host((1, 8, 64), bf),
                      _host((1, 8, 64), bf), [0, 8], 8)


@pytest.mark.gpu
def test_malformed_gpu_tensors_are_rejected():
    import torch
    import exact_io_aware_15_amd as fa
    from exact_io_aware_15_amd._lib import FaError
    bf = torch.bfloat16
    B, H, N, d = 1, 2, 64, 64
    q, k, v, do = (torch.zeros(B, H, N, d, dtype=bf, device="cuda")
                   for _ in range(4))
    with pytest.raises(ValueError, match="contiguous"):
        fa.fwd(q.transpose(2, 3).contiguous().transpose(2, 3), k, v)
    with pytest.raises(TypeError):
        fa.fwd(q, k.float(), v)
    with pytest.raises(ValueError, match="shape"):
        fa.fwd(q, k, v[:, :, :32].contiguous())
    o, m, l = fa.fwd(q, k, v)
    need = fa.bwd_workspace_bytes(B, H, N, d)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.bwd(q, k, v, o, do, m, l,
               workspace=torch.empty(need, dtype=torch.uint8))
    with pytest.raises(TypeError):
        fa.bwd(q, k, v, o, do, m, l,
               workspace=torch.empty(need, dtype=torch.float32,
                                     device="cuda"))
    with pytest.raises(FaError):
        fa.bwd(q, k, v, o, do, m, l,
               workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    # a workspace of exactly the asked size is accepted
    g = fa.bwd(q, k, v, o, do, m, l,
               workspace=torch.empty(need, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert all(torch.isfinite(x.float()).all() for x in g)
