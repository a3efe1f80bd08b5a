"""Edge cases of the bf16 path on the GPU, through the C ABI: head counts other
than 128 (partial and several head groups), the largest query group, contexts
that hold only the query tokens, more splits than there is work, and the data
problems the status word reports (block id outside the pool, length outside the
table row, append position outside the table row), which must be clamped or
skipped, never turned into out-of-bounds accesses."""
import numpy as np
import pytest

from mla_rank_latent_amd import synth
from tests import harness as H

pytestmark = pytest.mark.gpu

BAD_BLOCK, BAD_LENGTH, BAD_POS = 0x1, 0x2, 0x4


def _run(spec, num_splits=0, mutate=None):
    import torch
    x = synth.make_inputs(spec)
    if mutate is not None:
        mutate(x)
    H.log(f"{spec.name} H={spec.n_heads} B={spec.batch} sq={spec.sq} lens={list(x['seq_lens'])[:6]} "
          f"splits={num_splits}")
    c = H.GpuCase(x, num_splits)
    c.step()
    torch.cuda.synchronize()
    return x, c


@pytest.mark.parametrize("n_heads,sq,lens", [
    (16, 1, [70, 300]),          # one partial head group
    (200, 1, [129, 64]),         # two head groups, the second ragged
    (72, 3, [3, 190]),           # 42 heads per group at sq = 3
    (128, 8, [8, 65, 300]),      # the largest query group
])
def test_head_counts_and_query_groups(n_heads, sq, lens):
    spec = H.small_spec(f"heads{n_heads}_sq{sq}", len(lens), sq, lens, seed=31 + n_heads + sq, n_heads=n_heads)
    x, c = _run(spec)
    assert int(c.status.item()) == 0
    ref, lse = H.oracle_decode(x)
    H.assert_close(H.host(c.out), ref, "bf16", spec.name)
    assert np.max(np.abs(H.host(c.lse) - lse)) <= 2e-2


def test_context_of_query_tokens_only():
    """seq_len == sq: each query sees the tokens of its own group up to itself."""
    spec = H.small_spec("query_only", 3, 2, [2, 2, 40], seed=41)
    x, c = _run(spec)
    assert int(c.status.item()) == 0
    ref, lse = H.oracle_decode(x)
    H.assert_close(H.host(c.out), ref, "bf16", spec.name)
    assert np.max(np.abs(H.host(c.lse) - lse)) <= 2e-2


def test_more_splits_than_work():
    """1024 ranges for 3 short sequences: most ranges are empty."""
    spec = H.small_spec("splits1024", 3, 1, [1, 65, 130], seed=43)
    x, c = _run(spec, num_splits=1024)
    assert int(c.status.item()) == 0
    ref, _ = H.oracle_decode(x)
    H.assert_close(H.host(c.out), ref, "bf16", spec.name)


def test_bad_block_id_is_reported_and_clamped():
    def mutate(x):
        x["block_table"] = x["block_table"].copy()
        x["block_table"][1, 0] = 1 << 20          # far outside the pool
    spec = H.small_spec("bad_block", 2, 1, [100, 100], seed=45)
    x, c = _run(spec, mutate=mutate)
    assert int(c.status.item()) & BAD_BLOCK
    out = H.host(c.out)
    assert np.all(np.isfinite(out))
    ref, _ = H.oracle_decode(x, batches=[0])       # the untouched sequence is still right
    H.assert_close(out[:1], ref, "bf16", "bad_block seq 0")


def test_bad_lengths_are_reported_and_clamped():
    def mutate(x):
        x["seq_lens"] = x["seq_lens"].copy()
        x["seq_lens"][0] = x["block_table"].shape[1] * 64 + 5    # longer than its table row
        x["seq_lens"][2] = 0                                     # shorter than the query group
    spec = H.small_spec("bad_len", 3, 1, [64, 77, 50], seed=47)
    x, c = _run(spec, mutate=mutate)
    assert int(c.status.item()) & BAD_LENGTH
    out = H.host(c.out)
    assert np.all(np.isfinite(out))
    assert np.all(H.host(c.lse)[2] == -np.inf) and np.all(out[2] == 0.0)   # sees no token
    ref, _ = H.oracle_decode(x, batches=[1])
    H.assert_close(out[1:2], ref, "bf16", "bad_len seq 1")


@pytest.mark.parametrize("split", [True, False])
def test_bad_append_position_is_reported_and_skipped(split):
    import torch
    spec = H.small_spec("bad_pos", 2, 1, [70, 90], append=True, seed=49)
    x = synth.make_inputs(spec)
    x["positions"] = x["positions"].copy()
    x["positions"][1, 0] = x["block_table"].shape[1] * 64      # one past the table row
    H.log(f"bad_pos split={split}")
    c = H.GpuCase(x)
    before = x["pool"].copy()
    c.append(split)
    torch.cuda.synchronize()
    assert int(c.status.item()) & BAD_POS
    after = c.pool.view(torch.int16).cpu().numpy().view(np.uint16)
    p0 = int(x["positions"][0, 0])
    blk0 = x["block_table"][0, p0 // 64]
    changed = np.argwhere(np.any(after != before, axis=-1))
    assert [tuple(r) for r in changed] == [(blk0, p0 % 64)]     # only sequence 0's row was written


@pytest.mark.parametrize("num_splits", [1, 4])
def test_late_dominant_token_restarts_the_range(num_splits):
    """One token, late in its range, whose rotary key is scaled 60x: for most heads
    its score beats the range's first-stage maximum by far more than 2^16, which
    makes the kernel re-run the range against the larger reference.  The latent
    values are untouched, so the output keeps its usual magnitude."""
    spec = H.small_spec("late_spike", 2, 1, [500, 300], seed=51)

    def mutate(x):
        pool = synth.bf16_bits_to_f32(x["pool"]).copy()
        t = 400                                    # past the first stage of its range in both split counts
        blk = x["block_table"][0, t // 64]
        pool[blk, t % 64, 512:] *= 60.0
        x["pool"] = synth.f32_to_bf16_bits(pool.astype(np.float32))

    x, c = _run(spec, num_splits=num_splits, mutate=mutate)
    assert int(c.status.item()) == 0
    ref, lse = H.oracle_decode(x)
    H.assert_close(H.host(c.out), ref, "bf16", f"late_spike splits={num_splits}")
    assert np.max(np.abs(H.host(c.lse) - lse) / np.maximum(np.abs(lse), 1.0)) <= 2e-2


@pytest.mark.parametrize("scale", [0.0, -0.0721687836, 0.0721687836 * 3.0, 1e-3])
def test_softmax_scale_extremes(scale):
    """The softmax scale reaches the kernels as a power of two applied to the absorbed query
    and a factor in [0.71, 1.42] applied to the logits.  Zero gives uniform weights, a negative
    scale flips the logits' order, three times the usual scale makes the softmax sharp (a few
    tokens carry each row), a tiny one makes every weight nearly equal; each must still match
    the oracle.  (A sharper softmax amplifies the logits' rounding, which comes from the bf16
    absorbed query at any scale: at five times the usual scale the absolute error reaches the
    2e-2 bar.)"""
    spec = H.small_spec("scales", 2, 2, [700, 129], seed=61)
    x = synth.make_inputs(spec)
    x["scale"] = float(scale)
    c = H.GpuCase(x)
    c.decode()
    import torch
    torch.cuda.synchronize()
    assert int(c.status.item()) == 0
    ref, lse = H.oracle_decode(x)
    out = H.host(c.out).astype(np.float64)
    r = H.rel_l2(out, ref)
    # A sharp softmax puts single cache values, up to ~4 in size, into the output, whose own
    # bf16 rounding is then up to 2^-8 of it: the absolute bar counts beyond that rounding.
    excess = np.max(np.abs(out - ref) - 2.0 ** -8 * np.abs(ref))
    H.log(f"  scale={scale}: rel_l2={r:.3e} max_abs={np.max(np.abs(out - ref)):.3e} beyond rounding={excess:.3e}")
    assert r <= 1e-2 and excess <= 2e-2, (scale, r, excess)
    assert np.max(np.abs(H.host(c.lse) - lse) / np.maximum(np.abs(lse), 1.0)) <= 2e-2
