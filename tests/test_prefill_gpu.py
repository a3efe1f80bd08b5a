"""Prefill (mla_prefill) on the GPU against the fp64 oracle, through the C ABI.

Prefill's queries are the last t tokens of each sequence, and the oracle's
definition for them is its decode with a query group of t: query s at position
L - t + s sees tokens 0 .. L - t + s.  Cases span several 256-row query tiles
with a ragged tail, prior context or none, head counts that fill and do not
fill the 8-way workgroup grouping, t = 1, sequences shorter than their query
group, bad block ids, paging, and the full-size workload on sampled rows."""
import numpy as np
import pytest

from mla_rank_latent_amd import synth
from tests import harness as H

pytestmark = pytest.mark.gpu

BAD_BLOCK, BAD_LENGTH = 0x1, 0x2


def _spec(name, lens, t, n_heads=128, seed=61, paged=True):
    return synth.Spec(name, batch=len(lens), sq=t, seq_lens=list(lens), paged=paged, seed=seed, n_heads=n_heads)


def _run(x):
    import torch
    spec = x["spec"]
    H.log(f"{spec.name} H={spec.n_heads} B={spec.batch} t={spec.sq} lens={[int(v) for v in x['seq_lens']][:6]}")
    c = H.PrefillCase(x)
    c.run()
    torch.cuda.synchronize()
    return c


@pytest.mark.parametrize("lens,t,n_heads", [
    ([600, 333], 300, 128),        # two query tiles (the second partial), prior context
    ([320], 320, 128),             # the whole sequence is the query group
    ([64, 130, 900], 64, 16),      # 48 (sequence, head) groups, short and long contexts
    ([1, 77], 1, 128),             # t = 1: a decode step through the prefill path
    ([1000], 257, 8),              # one row past a query tile; 8 heads
])
def test_prefill_matches_oracle(lens, t, n_heads):
    x = synth.make_inputs(_spec(f"prefill_t{t}_h{n_heads}", lens, t, n_heads, seed=61 + t + n_heads))
    c = _run(x)
    assert int(c.status.item()) == 0
    ref, lse = H.oracle_decode(x)
    H.assert_close(H.host(c.out), ref, "bf16", x["spec"].name)
    assert np.max(np.abs(H.host(c.lse) - lse)) <= 2e-2


def test_prefill_probabilities_sum_to_one():
    """sum_j exp(z_j - lse) = 1 with the GPU's lse and the oracle's logits."""
    x = synth.make_inputs(_spec("prefill_lse", [700], 300, seed=71))
    c = _run(x)
    lse = H.host(c.lse)
    for s, h in [(0, 0), (1, 5), (150, 77), (255, 127), (256, 3), (299, 64)]:
        tot = H.lse_probability_sum(x, 0, s, h, float(lse[0, s, h]))
        assert abs(tot - 1.0) <= 1e-2, (s, h, tot)


def test_prefill_sequence_shorter_than_its_queries():
    """seq_lens[b] < t is reported; the first queries of that group see no token
    (out = 0, lse = -inf) and the rest are still right."""
    x = synth.make_inputs(_spec("prefill_short", [500, 300], 300, seed=73))
    x["seq_lens"] = x["seq_lens"].copy()
    x["seq_lens"][1] = 290
    c = _run(x)
    assert int(c.status.item()) & BAD_LENGTH
    out, lse = H.host(c.out), H.host(c.lse)
    assert np.all(out[1, :10] == 0.0) and np.all(lse[1, :10] == -np.inf)
    ref, rlse = H.oracle_decode(x)
    H.assert_close(out, ref, "bf16", "prefill_short")
    m = np.isfinite(rlse)
    assert np.max(np.abs(lse[m] - rlse[m])) <= 2e-2


def test_prefill_bad_block_is_reported_and_clamped():
    x = synth.make_inputs(_spec("prefill_bad_block", [200, 260], 100, seed=75))
    x["block_table"] = x["block_table"].copy()
    x["block_table"][1, 1] = 1 << 20
    c = _run(x)
    assert int(c.status.item()) & BAD_BLOCK
    out = H.host(c.out)
    assert np.all(np.isfinite(out))
    ref, _ = H.oracle_decode(x, batches=[0])
    H.assert_close(out[:1], ref[:1], "bf16", "prefill_bad_block seq 0")


def test_prefill_paging_is_bitwise_invariant():
    """A permuted block table gives the same bits as the identity table."""
    xp = synth.make_inputs(_spec("prefill_paged", [520, 300], 260, seed=77, paged=True))
    xc = dict(xp)
    # rebuild the contiguous layout: logical block i of sequence b at physical b * nblk + i
    bt = xp["block_table"]
    nb = bt.shape[1]
    pool = np.zeros((bt.shape[0] * nb,) + xp["pool"].shape[1:], dtype=xp["pool"].dtype)
    ident = np.full_like(bt, -1)
    for b in range(bt.shape[0]):
        for i in range(nb):
            if bt[b, i] >= 0:
                pool[b * nb + i] = xp["pool"][bt[b, i]]
                ident[b, i] = b * nb + i
    xc["pool"], xc["block_table"] = pool, ident
    cp, cc = _run(xp), _run(xc)
    assert np.array_equal(H.host(cp.out), H.host(cc.out))
    assert np.array_equal(H.host(cp.lse), H.host(cc.lse))


@pytest.mark.timeout(900)
def test_prefill_full_size_every_tile_every_head():
    """The benchmarked prefill (one 8192-token sequence, every token a query, 128 heads):
    two queries of every 256-row query tile (one at a varying offset inside the tile, and
    the tile's last row), every head, against the oracle (a query of the group is a single
    query over its visible prefix), plus the first and last queries of the sequence."""
    x = synth.make_inputs(_spec("prefill_b1_ctx8192", [8192], 8192, seed=79))
    c = _run(x)
    assert int(c.status.item()) == 0
    out, lse = H.host(c.out), H.host(c.lse)
    queries = sorted({0, 1, 8191} | {256 * k + (37 * k + 5) % 256 for k in range(32)} |
                     {256 * k + 255 for k in range(32)})
    want, want_lse = H.oracle_single_queries(x, 0, queries)
    got = out[0, queries]
    H.assert_close(got, want, "bf16", f"prefill_b1_ctx8192: {len(queries)} queries x 128 heads")
    d = np.max(np.abs(lse[0, queries] - want_lse))
    H.log(f"  lse max-abs {d:.3e}")
    assert d <= 2e-2
    assert np.all(np.isfinite(out))


@pytest.mark.parametrize("group", [1, 3])
def test_prefill_in_groups_of_sequences(group):
    """mla_prefill with a workspace for `group` sequences (fewer than the batch) expands and
    attends the sequences group by group: the output equals the one-workspace run bit for bit
    and matches the oracle."""
    import torch
    from mla_rank_latent_amd import mla
    x = synth.make_inputs(_spec("prefill_groups", [700, 300, 1000, 129, 512], 128, n_heads=16, seed=81))
    full = _run(x)
    out_full, lse_full = full.out.clone(), full.lse.clone()
    c = H.PrefillCase(x)
    per_seq = mla.mla_prefill_workspace_bytes(c.d, 1, int(x["block_table"].shape[1]))
    c.ws = torch.empty(group * per_seq, dtype=torch.uint8, device="cuda")
    H.log(f"prefill_groups: workspace for {group} of {x['spec'].batch} sequences")
    c.run()
    torch.cuda.synchronize()
    assert int(c.status.item()) == 0
    assert torch.equal(c.out.view(torch.int16), out_full.view(torch.int16))
    assert torch.equal(c.lse, lse_full)
    ref, lse = H.oracle_decode(x)
    H.assert_close(H.host(c.out), ref, "bf16", f"prefill in groups of {group}")
    assert np.max(np.abs(H.host(c.lse) - lse)) <= 2e-2


@pytest.mark.timeout(900)
def test_prefill_batch8_ctx8192_in_one_sequence_workspace():
    """Eight 8192-token sequences, the last 1024 tokens of each a query (a chunked-prefill
    step over a batch), with a workspace that holds one sequence's expanded keys and values
    (537 MB at 128 heads, an eighth of the batch's): every sequence is checked against the
    oracle on four queries spread over its group, every head."""
    import torch
    from mla_rank_latent_amd import mla
    x = synth.make_inputs(_spec("prefill_b8_ctx8192", [8192] * 8, 1024, seed=83))
    c = H.PrefillCase(x)
    per_seq = mla.mla_prefill_workspace_bytes(c.d, 1, int(x["block_table"].shape[1]))
    c.ws = torch.empty(per_seq, dtype=torch.uint8, device="cuda")
    H.log(f"prefill_b8_ctx8192: workspace {per_seq} bytes (one of 8 sequences)")
    c.run()
    torch.cuda.synchronize()
    assert int(c.status.item()) == 0
    out, lse = H.host(c.out), H.host(c.lse)
    assert np.all(np.isfinite(out))
    for b in range(8):
        queries = [0, 300 + 50 * b, 700, 1023]
        want, want_lse = H.oracle_single_queries(x, b, queries)
        H.assert_close(out[b, queries], want, "bf16", f"prefill_b8 sequence {b}")
        assert np.max(np.abs(lse[b, queries] - want_lse)) <= 2e-2
