"""The decode path captured in a HIP graph (torch.cuda.CUDAGraph, which records the launches
made on its capture stream) and replayed.  The library's launches make no allocation, memset,
copy or host synchronisation, so its kernels are recorded as they are; every replay must give
the eager call's cache, out and lse bit for bit.  Before each replay the outputs are cleared,
the appended rows are taken out of the cache again and other work runs on the device, so a
replay that skipped a kernel, or read state left by the previous one, would show.  Covers
mla_decode_step (the append's partial products, the absorbed queries and the plan, the
append's rows, the attention, the merge), mla_decode alone (also replayed with new lengths
and queries in the same buffers), the FP8-cache decode, the decode that allocates nothing,
and prefill run in groups of sequences."""
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


def test_decode_graph_follows_new_lengths_and_queries():
    """A serving loop captures once and replays with new contents in the same buffers: the plan
    is rebuilt on the device from seq_lens at every replay, so shorter lengths and other queries
    give what an eager call on those contents gives."""
    import torch
    lens, new_lens = [1000, 3, 257], [500, 2, 64]
    spec = H.small_spec("graph_contents", len(lens), 2, lens, seed=173)
    x = synth.make_inputs(spec)
    H.log(f"graph decode lens={lens} -> {new_lens} sq=2")
    c = H.GpuCase(x)
    g = _capture(c.decode)
    ref = H.GpuCase(x)
    for case in (c, ref):
        case.seq_lens.copy_(torch.tensor(new_lens, dtype=torch.int32))
        case.q_nope.neg_()
        case.q_rope.mul_(0.5)
    ref.decode()
    torch.cuda.synchronize()
    assert int(ref.status.item()) == 0
    c.out.zero_()
    c.lse.zero_()
    g.replay()
    torch.cuda.synchronize()
    assert int(c.status.item()) == 0
    assert torch.equal(c.out.view(torch.int16), ref.out.view(torch.int16))
    assert torch.equal(c.lse, ref.lse)


def test_fp8_decode_replays_from_a_graph():
    """The FP8-cache decode (pages made by mla_cache_quantize) captured and replayed."""
    import torch
    lens = [700, 1, 130]
    spec = H.small_spec("graph_fp8", len(lens), 1, lens, seed=174)
    x = H.with_fp8_cache(synth.make_inputs(spec))
    H.log(f"graph fp8 decode lens={lens}")
    ref = H.GpuCase(x, cache="fp8")
    ref.decode()
    torch.cuda.synchronize()
    assert int(ref.status.item()) == 0
    c = H.GpuCase(x, cache="fp8")
    g = _capture(c.decode)
    _check_replays(g, c, ref, None)


def test_prefill_in_groups_replays_from_a_graph():
    """mla_prefill with a workspace for two of five sequences (expand, then attend, per group,
    all on the capture stream) captured and replayed."""
    import torch
    from mla_rank_latent_amd import mla
    spec = synth.Spec("graph_prefill", batch=5, sq=96, seq_lens=[700, 300, 1000, 129, 512], paged=True, seed=175,
                      n_heads=16)
    x = synth.make_inputs(spec)
    H.log("graph prefill, 5 sequences in groups of 2")
    ref = H.PrefillCase(x)
    ref.run()
    torch.cuda.synchronize()
    assert int(ref.status.item()) == 0
    c = H.PrefillCase(x)
    per_seq = mla.mla_prefill_workspace_bytes(c.d, 1, int(x["block_table"].shape[1]))
    c.ws = torch.empty(2 * per_seq, dtype=torch.uint8, device="cuda")
    g = _capture(c.run)
    _check_replays(g, c, ref, None)


def test_noalloc_decode_replays_from_a_graph():
    """mla_decode_noalloc, the entry point for callers that cannot allocate (code under graph
    capture among them), captured and replayed: each replay equals mla_decode with a caller
    workspace, bit for bit."""
    import torch
    from mla_rank_latent_amd import mla
    lens = [900, 5, 320, 64]
    spec = H.small_spec("graph_noalloc", len(lens), 1, lens, seed=176)
    x = synth.make_inputs(spec)
    H.log(f"graph noalloc decode lens={lens}")
    ref = H.GpuCase(x)
    ref.decode()
    torch.cuda.synchronize()
    assert int(ref.status.item()) == 0
    c = H.GpuCase(x)
    g = _capture(lambda: mla.mla_decode_noalloc(c.d, c.q_nope, c.q_rope, c.w_uk, c.w_uv, c.pool, c.block_table,
                                                c.seq_lens, x["scale"], c.out, lse=c.lse, status=c.status))
    _check_replays(g, c, ref, None)
