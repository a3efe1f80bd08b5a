"""The decode path captured in a HIP graph (torch.cuda.CUDAGraph, which records the launches
made on its capture stream) and replayed.  The library's launches make no allocation, memset,
copy or host synchronisation, so its kernels are recorded as they are; every replay must give
the eager call's cache, out and lse bit for bit.  Before each replay the outputs are cleared,
the appended rows are taken out of the cache again and other work runs on the device, so a
replay that skipped a kernel, or read state left by the previous one, would show.  Covers
mla_decode_step (the append's partial products, the absorbed queries and the plan, the
append's rows, the attention, the merge) and mla_decode alone."""
import pytest

from mla_rank_latent_amd import synth
from tests import harness as H

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _check_replays(graph, c, ref, pool0):
    import torch
    for i in range(REPLAYS):
        c.out.zero_()
        c.lse.zero_()
        if pool0 is not None:
            c.pool.copy_(pool0)
        other = torch.randn(1 << 20, device="cuda")
        (other * other).sum().item()
        graph.replay()
        torch.cuda.synchronize()
        H.log(f"replay {i}: status {int(c.status.item())}")
        assert int(c.status.item()) == 0
        assert torch.equal(c.out.view(torch.int16), ref.out.view(torch.int16)), f"replay {i}: out"
        assert torch.equal(c.lse, ref.lse), f"replay {i}: lse"
        assert torch.equal(c.pool.view(torch.int16), ref.pool.view(torch.int16)), f"replay {i}: cache"


def _capture(launch):
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        launch()   # a first call off the default stream, outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launch()
    torch.cuda.synchronize()
    return g


def test_decode_step_replays_from_a_graph():
    import torch
    from mla_rank_latent_amd import mla
    lens = [130, 64, 700, 2]
    spec = H.small_spec("graph_step", len(lens), 1, lens, append=True, seed=171)
    x = synth.make_inputs(spec)
    H.log(f"graph step lens={lens}")
    ref = H.GpuCase(x)
    n = mla.mla_decode_step_workspace_bytes(ref.d, spec.batch, spec.sq, 0)
    ws_ref = torch.empty(n, dtype=torch.uint8, device="cuda")

    def step_args(c, ws):
        return (c.d, c.h, c.w_dkv, c.w_kr, c.positions, c.q_nope, c.q_rope, c.w_uk, c.w_uv, c.pool, c.block_table,
                c.seq_lens, x["scale"], ws, c.out)

    mla.mla_decode_step(*step_args(ref, ws_ref), lse=ref.lse, status=ref.status)
    torch.cuda.synchronize()
    assert int(ref.status.item()) == 0

    c = H.GpuCase(x)
    pool0 = c.pool.clone()
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    g = _capture(lambda: mla.mla_decode_step(*step_args(c, ws), lse=c.lse, status=c.status))
    _check_replays(g, c, ref, pool0)


def test_decode_replays_from_a_graph():
    import torch
    lens = [1000, 3, 257]
    spec = H.small_spec("graph_decode", len(lens), 2, lens, seed=172)
    x = synth.make_inputs(spec)
    H.log(f"graph decode lens={lens} sq=2")
    ref = H.GpuCase(x)
    ref.decode()
    torch.cuda.synchronize()
    assert int(ref.status.item()) == 0
    c = H.GpuCase(x)
    g = _capture(c.decode)
    _check_replays(g, c, ref, None)
