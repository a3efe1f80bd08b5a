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
    (64, 1, [100, 257]),         # 64 heads: the absorb tiles' XCD grouping, half-filled rows
    (192, 2, [5, 130]),          # 192 heads at sq = 2: three head groups, the grouping again
    (1, 1, [50, 300]),           # one head: 127 of a workgroup's 128 rows are padding
    (8, 2, [2, 700]),            # 8 heads at two query tokens
    (1024, 1, [130, 64]),        # the most heads the kernels take: eight head groups
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


@pytest.mark.parametrize("num_splits", [1, 3, 5])
def test_every_stage_count_before_the_epilogue(num_splits):
    """A range's last iterations issue copies into ring slots (nsub + 1) % 4 and
    (nsub + 2) % 4 (nsub: the range's 32-token stages), and its partial state then goes out
    through ring slots 0 and 1.  Lengths 33 .. 225 in steps of 32 give every nsub % 4, on
    whole ranges (one split: a range per sequence) and on ranges cut inside sequences;
    every head of every sequence is compared with the oracle."""
    lens = [33, 65, 97, 129, 161, 193, 225, 64, 96]
    spec = H.small_spec(f"nsub_mod4_s{num_splits}", len(lens), 1, lens, seed=47 + num_splits)
    x, c = _run(spec, num_splits=num_splits)
    assert int(c.status.item()) == 0
    ref, lse = H.oracle_decode(x)
    H.assert_close(H.host(c.out), ref, "bf16", spec.name)
    assert np.max(np.abs(H.host(c.lse) - lse)) <= 2e-2


@pytest.mark.parametrize("name,sq,lens,num_splits", [
    ("skewed5", 1, [6000, 64, 1500, 130, 3000], 256),    # one row holds most of the pieces
    ("one_long16", 1, [2000] + [64 + 7 * i for i in range(15)], 256),   # 16 rows: half the slots spare
    ("second_block8", 1, [70 + 5 * i for i in range(32)] + [4000, 65, 900, 64, 2500, 130, 64, 1200], 512),
    ("sq2_skewed3", 2, [3000, 66, 700], 128),            # rows of one sequence share its count
])
def test_merge_slots_follow_piece_counts(name, sq, lens, num_splits):
    """A row block with at most 16 valid rows shares its 32 thread slots out by the rows'
    piece counts: lengths far apart put many pieces on one row and one or two on the
    others, and a block of 8 rows after a full block of 32; every head of every row is
    compared with the oracle."""
    spec = H.small_spec(name, len(lens), sq, lens, seed=53 + len(lens))
    x, c = _run(spec, num_splits=num_splits)
    assert int(c.status.item()) == 0
    ref, lse = H.oracle_decode(x)
    H.assert_close(H.host(c.out), ref, "bf16", spec.name)
    assert np.max(np.abs(H.host(c.lse) - lse)) <= 2e-2


def test_planner_keeps_sequences_out_of_shared_ranges():
    """With the range count left to the library, the planner weighs a few range lengths by
    the extra pieces that ranges holding a sequence boundary cost.  Lengths 20480, 10240,
    5120 and 3200 on 256 ranges would cut ranges of 192 tokens, two of which hold a
    boundary; ranges of 256 tokens hold one sequence each, so the plan (the workspace's
    header: total tokens, tokens per range, pieces) has as many pieces as ranges.  Every
    head of every sequence is compared with the oracle."""
    import torch
    lens = [20480, 10240, 5120, 3200]
    spec = H.small_spec("planner_aligned", len(lens), 1, lens, seed=59)
    x, c = _run(spec)
    assert int(c.status.item()) == 0
    total, quota, pieces = (int(v) for v in c.ws[:12].view(torch.int32).cpu())
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    q0 = max(128, -(-(-(-total // cus)) // 64) * 64)
    H.log(f"  plan: total {total}, quota {quota} (even split {q0}), pieces {pieces}")
    assert total == sum(lens) and quota % 64 == 0 and q0 <= quota <= q0 + 7 * 64
    assert pieces == -(-total // quota)   # no range holds two sequences
    ref, lse = H.oracle_decode(x)
    H.assert_close(H.host(c.out), ref, "bf16", spec.name)
    assert np.max(np.abs(H.host(c.lse) - lse)) <= 2e-2


@pytest.mark.parametrize("name,sq,lens", [
    ("ragged24_sq1", 1, [5132, 4555, 9064, 9286, 5703, 8086, 8933, 8538, 2163, 5261, 9917, 11967, 8511, 11977, 3584,
                         11378, 10241, 2388, 2190, 8256, 9248, 8050, 6976, 7295]),
    ("ragged40_sq2", 2, [1833, 1732, 528, 1977, 2971, 739, 2166, 1411, 938, 261, 269, 2522, 2804, 88, 2005, 96, 2107,
                         2811, 2295, 2911, 748, 2580, 295, 2080, 2156, 497, 2860, 2725, 904, 1529, 424, 2110, 1047,
                         99, 2576, 379, 1073, 2094, 1266, 2847]),
    # short batches whose cost targets step less than one boundary's piece cost: several
    # targets fall inside one boundary's step, so the plan has empty ranges at boundaries,
    # which no sequence may count as a piece
    ("tiny5_sq2", 2, [34, 131, 137, 188, 3]),
    ("tiny6_sq1", 1, [192, 7, 182, 62, 168, 90]),
])
def test_planner_balances_ragged_batches(name, sq, lens):
    """Ragged batches whose even ranges would hold several sequence boundaries each get
    cost-balanced ranges (the plan header's quota 0): ranges are shorter where they hold
    boundaries.  The pieces stay within the workspace's bound, and every head of every
    sequence (and query token) matches the oracle."""
    import torch
    spec = H.small_spec(name, len(lens), sq, lens, seed=61 + sq)
    x, c = _run(spec)
    assert int(c.status.item()) == 0
    total, quota, pieces = (int(v) for v in c.ws[:12].view(torch.int32).cpu())
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    H.log(f"  plan: total {total}, quota {quota}, pieces {pieces}")
    assert total == sum(-(-v // 64) * 64 for v in lens)
    assert quota == 0 and len(lens) <= pieces <= cus // (1 if sq == 1 else 2) + len(lens)
    ref, lse = H.oracle_decode(x)
    H.assert_close(H.host(c.out), ref, "bf16", spec.name)
    assert np.max(np.abs(H.host(c.lse) - lse)) <= 2e-2


@pytest.mark.parametrize("name,batch,sq,num_splits", [
    ("b300_sq1", 300, 1, 0),      # two 256-sequence chunks in the planner's scans
    ("b520_sq1", 520, 1, 0),      # three chunks; 17 row blocks of 32 in the absorb and the merge
    ("b300_sq2", 300, 2, 0),      # two head groups, 600 query rows per head
    ("b300_sq1_s64", 300, 1, 64),  # a forced range count: ranges holding many sequence boundaries
])
def test_batches_beyond_256_sequences(name, batch, sq, num_splits):
    """More than 256 sequences: the split planner's prefix sums run over several 256-sequence
    chunks and read the segment starts back from the workspace (no cost-balanced plan), and
    the absorb and merge kernels see more than eight 32-row blocks.  Every sequence, query
    token and head is compared with the oracle."""
    lens = [sq + (37 * b + 11) % 250 for b in range(batch)]
    spec = H.small_spec(name, batch, sq, lens, seed=71 + batch + sq)
    x, c = _run(spec, num_splits)
    assert int(c.status.item()) == 0
    ref, lse = H.oracle_decode(x)
    H.assert_close(H.host(c.out), ref, "bf16", spec.name)
    assert np.max(np.abs(H.host(c.lse) - lse)) <= 2e-2


@pytest.mark.parametrize("name,lens,num_splits", [
    ("one_row_300", [300], 0),
    ("one_row_5000_s7", [5000], 7),
    ("rows33", [100 + 37 * i for i in range(33)], 0),   # the second block of 32 rows holds one
])
def test_blocks_of_one_row(name, lens, num_splits):
    """A merge row block that holds a single query row (batch 1 at one query token, or the
    33rd row) multiplies it with the W^UV slice on the vector units instead of the
    32-row MFMA product; with one and several pieces, compared with the oracle."""
    spec = H.small_spec(name, len(lens), 1, lens, seed=67 + len(lens))
    x, c = _run(spec, num_splits=num_splits)
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
    a = np.max(np.abs(out - ref))
    # A sharp softmax puts single cache values, up to ~4 in size, into the output, whose own
    # bf16 rounding is then up to 2^-8 of it: beyond the workloads' scale (1/sqrt(192)) the
    # absolute bar counts what exceeds that rounding; up to it, the plain bar holds.
    excess = np.max(np.abs(out - ref) - 2.0 ** -8 * np.abs(ref))
    H.log(f"  scale={scale}: rel_l2={r:.3e} max_abs={a:.3e} beyond rounding={excess:.3e}")
    assert r <= 1e-2 and excess <= 2e-2, (scale, r, excess)
    if abs(scale) <= 1.0 / np.sqrt(192.0) + 1e-9:
        assert a <= 2e-2, (scale, a)
    assert np.max(np.abs(H.host(c.lse) - lse) / np.maximum(np.abs(lse), 1.0)) <= 2e-2
