"""mla_decode_step (a decode step that appends its own tokens, the append's partial
products, the absorbed queries and the split plan in one launch) against
mla_cache_append followed by mla_decode, through the C ABI: the written cache, out and
lse must be equal bit for bit (the same kernels' code computes them), and the outputs
match the oracle.  Covers one and two new tokens per sequence, ragged paged batches,
the phases called one by one, two new tokens that fall in two token ranges, new
positions inside the context rather than at its end and outside every table row
(reported, not written), model widths with 7, 8 and 23 append slices, the batch-64
context-8192 benchmark step, and a step of 2048 new tokens (mla_cache_append's many-row
GEMM path)."""
import numpy as np
import pytest

from mla_rank_latent_amd import synth
from tests import harness as H

pytestmark = pytest.mark.gpu


def _pair(x, phases_one_by_one=False, num_splits=0, status=0):
    import torch
    from mla_rank_latent_amd import mla
    spec = x["spec"]
    # reference: mla_cache_append (with its workspace) then mla_decode
    r = H.GpuCase(x, num_splits=num_splits)
    r.step()
    # the fused step on a fresh copy of the same inputs
    c = H.GpuCase(x, num_splits=num_splits)
    n = mla.mla_decode_step_workspace_bytes(c.d, spec.batch, spec.sq, num_splits)
    assert n > 0
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    args = (c.d, c.h, c.w_dkv, c.w_kr, c.positions, c.q_nope, c.q_rope, c.w_uk, c.w_uv, c.pool, c.block_table,
            c.seq_lens, x["scale"], ws, c.out)
    if phases_one_by_one:
        for ph in (mla.MLA_PHASE_PREPARE, mla.MLA_PHASE_ATTEND, mla.MLA_PHASE_FINISH):
            mla.mla_decode_step(*args, lse=c.lse, status=c.status, phases=ph, num_splits=num_splits)
    else:
        mla.mla_decode_step(*args, lse=c.lse, status=c.status, num_splits=num_splits)
    torch.cuda.synchronize()
    assert int(r.status.item()) == status and int(c.status.item()) == status
    assert torch.equal(c.pool.view(torch.int16), r.pool.view(torch.int16))
    assert torch.equal(c.out.view(torch.int16), r.out.view(torch.int16))
    assert torch.equal(c.lse, r.lse)
    return c


@pytest.mark.parametrize("name,lens,sq,one_by_one", [
    ("step_b3_sq1", [130, 64, 700], 1, False),
    ("step_b4_sq2", [2, 65, 513, 1000], 2, False),
    ("step_b3_phases", [200, 77, 1500], 1, True),
    # 300 sequences: five 64-token append groups, the planner's scans over two chunks
    ("step_b300_sq1", [1 + (41 * b + 5) % 300 for b in range(300)], 1, False),
])
def test_step_equals_append_then_decode(name, lens, sq, one_by_one):
    spec = H.small_spec(name, len(lens), sq, lens, append=True, seed=91 + sq)
    x = synth.make_inputs(spec)
    H.log(f"{name} lens={lens} sq={sq} phases one by one={one_by_one}")
    c = _pair(x, one_by_one)
    rows = H.oracle_append_rows(x)
    ref, lse = H.oracle_decode(x, appended_rows=rows)
    H.assert_close(H.host(c.out), ref, "bf16", name)
    assert np.max(np.abs(H.host(c.lse) - lse)) <= 2e-2


@pytest.mark.parametrize("d_model", [2048, 2560, 7168])
def test_step_other_model_widths(d_model):
    """Model widths whose append splits d_model into 7, 8 and 23 slices: with 18 column
    tiles per 64-token group, 8 slices give a tile count that is a multiple of 8 (tiles
    that read one block of h grouped per XCD), 7 and 23 do not (tiles in plain slice
    order); both paths write the same rows as mla_cache_append and match the oracle."""
    spec = H.small_spec(f"step_dmodel{d_model}", 3, 1, [130, 64, 300], append=True, seed=99, d_model=d_model)
    x = synth.make_inputs(spec)
    H.log(f"step d_model={d_model}")
    c = _pair(x)
    rows = H.oracle_append_rows(x)
    ref, lse = H.oracle_decode(x, appended_rows=rows)
    H.assert_close(H.host(c.out), ref, "bf16", spec.name)
    assert np.max(np.abs(H.host(c.lse) - lse)) <= 2e-2
    pool = H.host(c.pool)
    for b in range(3):
        p = int(x["positions"][b, 0])
        g = pool[x["block_table"][b, p // 64], p % 64]
        # every element of the written row within one bf16 ulp of the oracle's rounded row
        assert np.all(np.abs(g - rows[b, 0]) <= H.bf16_ulp(rows[b, 0]) + 1e-30)


def test_step_new_tokens_in_two_ranges():
    """Two new tokens at positions 127 and 128 of a 129-token sequence, with token ranges of
    128: the two new rows are read by two ranges, each with two head groups (sq = 2)."""
    spec = H.small_spec("step_two_ranges", 2, 2, [129, 300], append=True, seed=97)
    x = synth.make_inputs(spec)
    H.log("step_two_ranges: new rows 127 | 128 split between ranges")
    c = _pair(x, num_splits=4)     # 512 rounded tokens: ranges of 128
    rows = H.oracle_append_rows(x)
    ref, _ = H.oracle_decode(x, appended_rows=rows)
    H.assert_close(H.host(c.out), ref, "bf16", "step_two_ranges")


def test_step_positions_inside_and_outside_the_context():
    """Sequence 0 appends at position 100 of 300 (a row inside the context, read by a range
    that does not hold the context's end), sequence 1 at position -1 (outside every table
    row: reported, not written, by both paths), sequence 2 at its end."""
    from mla_rank_latent_amd import mla
    spec = H.small_spec("step_positions", 3, 1, [300, 200, 150], append=True, seed=98)
    x = synth.make_inputs(spec)
    x["positions"] = x["positions"].copy()
    x["positions"][0, 0] = 100          # ranges of 192 tokens: range 0 of sequence 0
    x["positions"][1, 0] = -1
    H.log(f"step_positions: positions {x['positions'][:, 0].tolist()}")
    _pair(x, num_splits=4, status=mla.MLA_STATUS_BAD_POS)


@pytest.mark.timeout(600)
def test_step_benchmark_shape():
    x = synth.make_inputs(synth.presets()["v2_b64_ctx8192_paged_append"])
    H.log("step at batch 64 x context 8192 (the benchmark step)")
    c = _pair(x)
    rows = H.oracle_append_rows(x)
    ref, _ = H.oracle_decode(x, batches=[0, 31, 63], appended_rows=rows)
    H.assert_close(H.host(c.out)[[0, 31, 63]], ref[[0, 31, 63]], "bf16", "step benchmark shape, 3 sequences")


def test_step_many_new_tokens():
    """256 sequences x 8 new tokens = 2048 appended rows: the many-row GEMM append, then decode."""
    rng = np.random.default_rng(95)
    lens = [int(v) for v in rng.integers(8, 200, size=256)]
    spec = H.small_spec("step_b256_sq8", 256, 8, lens, append=True, seed=96, n_heads=16)
    x = synth.make_inputs(spec)
    H.log("step_b256_sq8: 2048 new rows")
    c = _pair(x)
    rows = H.oracle_append_rows(x)
    ref, _ = H.oracle_decode(x, batches=list(range(0, 256, 37)), appended_rows=rows)
    got = H.host(c.out)
    sel = list(range(0, 256, 37))
    H.assert_close(got[sel], ref[sel], "bf16", "step_b256_sq8 sampled sequences")
