"""The entry points under HIP graph capture.

The library queues kernels only (no allocation, no memset, no host
synchronisation), so a captured forward + backward must replay to the same
bits as the eager calls.  The graph is replayed several times with eager work
and synchronisations in between, and every replay is compared with the eager
result.
"""
import pytest
import torch

import exact_io_aware_51_amd as fa
from exact_io_aware_51_amd import workloads as W
from gpu_util import announce, device, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_captured_step_replays_bit_identically(dtype):
    dev = device()
    announce("graph capture", dtype)
    B, H, N, d = 2, 4, 700, 128
    code = {"f32": fa.FA_F32, "f16": fa.FA_F16, "bf16": fa.FA_BF16}[dtype]
    q, k, v, do = to_dev(W.kv_inputs(B, H, N, N, d, dtype, 51000), dev)
    scale = 0.0883883
    o, lse = torch.empty_like(q), torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    wsb = fa.fa_bwd_workspace_bytes(B, H, N, d, code)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)

    def step():
        st = torch.cuda.current_stream(dev).cuda_stream
        assert fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, d, scale,
                         1, code, st) == 0
        assert fa.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                         dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), wsb, B, H, N, d, scale, 1, code,
                         st) == 0

    step()
    torch.cuda.synchronize()
    want = [t.clone() for t in (o, lse, dq, dk, dv)]

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s):
        for t in (o, lse, dq, dk, dv):  # the replays must rewrite these
            t.zero_()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream(dev).wait_stream(s)
    torch.cuda.synchronize()

    for rep in range(4):
        for t in (o, lse, dq, dk, dv):
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for name, got, ref in zip(("o", "lse", "dq", "dk", "dv"), (o, lse, dq, dk, dv), want):
            assert torch.equal(got, ref), f"replay {rep}: {name} differs from the eager call"
        step()  # eager work between replays
        torch.cuda.synchronize()
