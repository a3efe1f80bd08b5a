"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle on the
same seeded inputs.  Tolerances: bf16 rel-L2 <= 1e-2 and max-abs <= 2e-2 over
the whole output; fp32 rel-L2 <= 1e-4."""
import numpy as np
import pytest

from mla_rank_latent_amd import synth
from oracle import mla_oracle
from tests import harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _torch_cuda():
    import torch
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def test_tiny_f32_end_to_end():
    spec = synth.presets()["tiny_f32_ctx65"]
    x = synth.make_inputs(spec)
    H.log(f"tiny_f32 seed={spec.seed}: append 65 + q_project + decode")
    c = H.GpuCase(x)
    c.step()
    import torch
    torch.cuda.synchronize()
    assert int(c.status.item()) == 0
    rows = H.oracle_append_rows(x)
    gpu_rows = H.host(c.pool)[0:2].reshape(-1, spec.row)[:65]
    assert np.max(np.abs(gpu_rows - rows[0])) <= 1e-5 * np.max(np.abs(rows))
    qn, qr = mla_oracle.q_project(synth.as_float(x["h"][:, -1:], "f32"), synth.as_float(x["w_q"], "f32"),
                                  synth.as_float(x["w_qr"], "f32"), x["q_positions"], spec.n_heads, spec.rope_base)
    assert H.rel_l2(H.host(c.q_nope), qn) <= 1e-6 and H.rel_l2(H.host(c.q_rope), qr) <= 1e-6
    ref, lse = H.oracle_decode(x, appended_rows=rows, q=(qn, qr))
    H.assert_close(H.host(c.out), ref, "f32", "tiny_f32 out")
    assert np.max(np.abs(H.host(c.lse) - lse)) <= 1e-5


def _bf16_case(spec, num_splits=0, heads=None, split_append=True):
    x = synth.make_inputs(spec)
    H.log(f"{spec.name} seed={spec.seed} B={spec.batch} sq={spec.sq} lens={list(x['seq_lens'])[:8]} splits={num_splits}"
          f" split_append={split_append}")
    c = H.GpuCase(x, num_splits)
    c.split_append = split_append
    c.step()
    import torch
    torch.cuda.synchronize()
    return x, c


@pytest.mark.parametrize("name,batch,sq,lens,paged", [
    ("contig_b1_l300", 1, 1, [300], False),
    ("paged_b3_ragged", 3, 1, [1, 100, 700], True),
    ("paged_b4_sq2", 4, 2, [2, 65, 130, 513], True),
    ("paged_b2_sq3", 2, 3, [3, 200], True),
])
def test_bf16_small(name, batch, sq, lens, paged):
    spec = H.small_spec(name, batch, sq, lens, paged=paged)
    x, c = _bf16_case(spec)
    assert int(c.status.item()) == 0
    ref, lse = H.oracle_decode(x)
    H.assert_close(H.host(c.out), ref, "bf16", name)
    assert np.max(np.abs(H.host(c.lse) - lse)) <= 2e-2


@pytest.mark.parametrize("split_append", [True, False])
def test_bf16_append_then_decode(split_append):
    spec = H.small_spec("append_b2", 2, 1, [130, 64], append=True)
    x, c = _bf16_case(spec, split_append=split_append)
    assert int(c.status.item()) == 0
    rows = H.oracle_append_rows(x)
    pool = H.host(c.pool)
    ndiff = 0
    for b in range(2):
        p = int(x["positions"][b, 0])
        g = pool[x["block_table"][b, p // 64], p % 64]
        # every element within one bf16 ulp of the oracle's rounded row
        assert np.all(np.abs(g - rows[b, 0]) <= H.bf16_ulp(rows[b, 0]) + 1e-30)
        ndiff += int(np.count_nonzero(g != rows[b, 0]))
    H.log(f"  append split={split_append}: {ndiff} of {2 * spec.row} elements one bf16 ulp from the oracle")
    ref, _ = H.oracle_decode(x, appended_rows=rows)
    H.assert_close(H.host(c.out), ref, "bf16", "append_b2 out")


def test_split_count_invariance():
    spec = H.small_spec("splits_b3", 3, 1, [1, 900, 2000], seed=12)
    x = synth.make_inputs(spec)
    ref, _ = H.oracle_decode(x)
    outs = []
    import torch
    for ns in (1, 3, 7, 64, 256):
        H.log(f"splits_b3 num_splits={ns}")
        c = H.GpuCase(x, ns)
        c.decode()
        torch.cuda.synchronize()
        o = H.host(c.out)
        H.assert_close(o, ref, "bf16", f"splits={ns}")
        outs.append(o)
    for o in outs[1:]:
        assert H.rel_l2(o, outs[0]) <= 4e-3


def test_paging_is_bitwise_invisible():
    spec = H.small_spec("paging_b3", 3, 2, [70, 500, 129], seed=13)
    x = synth.make_inputs(spec)
    # the same data laid out contiguously
    bt = x["block_table"]
    order = np.concatenate([bt[b, :(int(x["seq_lens"][b]) + 63) // 64] for b in range(3)])
    y = dict(x)
    y["pool"] = x["pool"][order]
    ident = np.full_like(bt, -1)
    o = 0
    for b in range(3):
        n = (int(x["seq_lens"][b]) + 63) // 64
        ident[b, :n] = np.arange(o, o + n)
        o += n
    y["block_table"] = ident
    import torch
    outs = []
    for z in (x, y):
        H.log(f"paging_b3 table={'permuted' if z is x else 'identity'}")
        c = H.GpuCase(z)
        c.decode()
        torch.cuda.synchronize()
        outs.append(c.out.view(torch.int16).cpu().numpy())
    assert np.array_equal(outs[0], outs[1])


def test_deterministic_and_lse_normalised():
    spec = H.small_spec("det_b2", 2, 1, [333, 1000], seed=14)
    x = synth.make_inputs(spec)
    import torch
    H.log("det_b2 two decode calls")
    c = H.GpuCase(x)
    c.decode()
    a = c.out.clone()
    c.decode()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), c.out.view(torch.int16))
    lse = H.host(c.lse)
    for b, s, h in [(0, 0, 0), (1, 0, 77), (1, 0, 127)]:
        assert abs(H.lse_probability_sum(x, b, s, h, lse[b, s, h]) - 1.0) <= 1e-2


@pytest.mark.parametrize("split", [True, False])
def test_append_dyadic_is_bit_exact(split):
    """On dyadic inputs every partial sum is exact in fp32, so the latent part of
    the appended row equals the oracle's rounded row bit for bit; nothing
    outside the appended rows changes."""
    spec = H.small_spec("dyadic_b3", 3, 1, [64, 130, 7], append=True, seed=15)
    x = synth.make_inputs(spec)
    rng = np.random.default_rng(99)
    x["h"] = synth.f32_to_bf16_bits(rng.integers(-2, 3, size=x["h"].shape).astype(np.float32))
    x["w_dkv"] = synth.f32_to_bf16_bits((rng.integers(-64, 65, size=x["w_dkv"].shape) / 64.0).astype(np.float32))
    x["w_kr"] = synth.f32_to_bf16_bits((rng.integers(-64, 65, size=x["w_kr"].shape) / 64.0).astype(np.float32))
    H.log(f"dyadic_b3 append split={split}")
    c = H.GpuCase(x)
    before = x["pool"].copy()
    c.append(split)
    import torch
    torch.cuda.synchronize()
    assert int(c.status.item()) == 0
    after = c.pool.view(torch.int16).cpu().numpy().view(np.uint16)
    rows = H.oracle_append_rows(x)
    touched = np.zeros(after.shape[:2], dtype=bool)
    for b in range(3):
        p = int(x["positions"][b, 0])
        blk = x["block_table"][b, p // 64]
        touched[blk, p % 64] = True
        want = synth.f32_to_bf16_bits(rows[b, 0].astype(np.float32))   # oracle values are bf16-exact
        assert np.array_equal(after[blk, p % 64, :512], want[:512])
        kr = synth.bf16_bits_to_f32(after[blk, p % 64, 512:]).astype(np.float64)
        assert np.all(np.abs(kr - rows[b, 0, 512:]) <= H.bf16_ulp(rows[b, 0, 512:]) + 1e-30)
    assert np.array_equal(after[~touched], before[~touched])


def test_append_paths_agree():
    """The split and single-kernel append paths sum in different orders: on N(0,1)
    data they agree to within one bf16 ulp, and the rest of the pool is untouched
    by either (65 tokens: a ragged 64-token group)."""
    import torch
    spec = H.small_spec("append_paths_b65", 65, 1, [1 + (7 * b) % 200 for b in range(65)], append=True, seed=21)
    x = synth.make_inputs(spec)
    pools = []
    for split in (True, False):
        H.log(f"append_paths_b65 split={split}")
        c = H.GpuCase(x)
        c.append(split)
        torch.cuda.synchronize()
        assert int(c.status.item()) == 0
        pools.append(c.pool.view(torch.int16).cpu().numpy().view(np.uint16))
    changed = np.any(pools[0] != x["pool"], axis=-1) | np.any(pools[1] != x["pool"], axis=-1)
    assert changed.sum() <= spec.batch                 # only the appended rows
    a, b = (synth.bf16_bits_to_f32(p[changed]).astype(np.float64) for p in pools)
    # latent part: one bf16 ulp of the value, plus what two fp32 summation orders of a
    # 5120-term dot product can differ by (a few 1e-7 at unit scale; 2^-18 of the
    # row's rms bounds it), which matters only for values that cancel to near zero
    d = np.abs(a[:, :512] - b[:, :512])
    rms = np.sqrt(np.mean(a[:, :512] ** 2, axis=1, keepdims=True))
    lim = 2.0 ** -7 * np.maximum(np.abs(a[:, :512]), np.abs(b[:, :512])) + 2.0 ** -18 * rms
    bad = np.argwhere(d > lim)
    H.log(f"append_paths_b65 latent: {len(bad)} elements over one ulp; worst rel "
          f"{float(np.max(d / np.maximum(lim * 2.0 ** 7, 1e-30))):.3e}; first {[(int(r), int(k), a[r, k], b[r, k]) for r, k in bad[:4]]}")
    assert len(bad) == 0
    # rotary part: a rotation can cancel, so one ulp of the rotated pair's length (plus rounding of each side)
    pair = np.sqrt(a[:, 512::2] ** 2 + a[:, 513::2] ** 2).repeat(2, axis=1)
    assert np.all(np.abs(a[:, 512:] - b[:, 512:]) <= 2.0 ** -6 * pair + 1e-30)


def _many_token_append_case(seed, dyadic):
    """2 sequences x 1100 appended tokens = 2200 rows: the single-GEMM append path
    (2048 rows or more), with a ragged last 128-token tile."""
    spec = synth.Spec("append_many", batch=2, sq=1100, seq_lens=[1100, 1300], paged=True, append=True, seed=seed,
                      n_heads=8)
    x = synth.make_inputs(spec)
    if dyadic:
        rng = np.random.default_rng(seed + 1)
        x["h"] = synth.f32_to_bf16_bits(rng.integers(-2, 3, size=x["h"].shape).astype(np.float32))
        x["w_dkv"] = synth.f32_to_bf16_bits((rng.integers(-64, 65, size=x["w_dkv"].shape) / 64.0).astype(np.float32))
        x["w_kr"] = synth.f32_to_bf16_bits((rng.integers(-64, 65, size=x["w_kr"].shape) / 64.0).astype(np.float32))
    return x


def _append_many(x):
    import torch
    H.log(f"append_many rows={x['h'].shape[0] * x['h'].shape[1]}")
    c = H.GpuCase(x)
    c.append(True)   # the workspace query returns 0 here: the GEMM path needs none
    torch.cuda.synchronize()
    return c, c.pool.view(torch.int16).cpu().numpy().view(np.uint16)


def test_append_many_tokens_dyadic_is_bit_exact():
    x = _many_token_append_case(31, dyadic=True)
    before = x["pool"].copy()
    c, after = _append_many(x)
    assert int(c.status.item()) == 0
    rows = H.oracle_append_rows(x)
    touched = np.zeros(after.shape[:2], dtype=bool)
    for b in range(2):
        for t, p in enumerate(x["positions"][b]):
            blk = x["block_table"][b, p // 64]
            touched[blk, p % 64] = True
            want = synth.f32_to_bf16_bits(rows[b, t].astype(np.float32))
            assert np.array_equal(after[blk, p % 64, :512], want[:512]), (b, t)
            kr = synth.bf16_bits_to_f32(after[blk, p % 64, 512:]).astype(np.float64)
            assert np.all(np.abs(kr - rows[b, t, 512:]) <= H.bf16_ulp(rows[b, t, 512:]) + 1e-30), (b, t)
    assert np.array_equal(after[~touched], before[~touched])


def test_append_many_tokens_within_one_ulp():
    x = _many_token_append_case(33, dyadic=False)
    c, after = _append_many(x)
    assert int(c.status.item()) == 0
    rows = H.oracle_append_rows(x)
    got = np.stack([[synth.bf16_bits_to_f32(after[x["block_table"][b, p // 64], p % 64]).astype(np.float64)
                     for p in x["positions"][b]] for b in range(2)])
    want = rows.astype(np.float64)
    d = np.abs(got[..., :512] - want[..., :512])
    rms = np.sqrt(np.mean(want[..., :512] ** 2, axis=-1, keepdims=True))
    H.log(f"  append_many: {int(np.count_nonzero(d))} of {d.size} latent elements differ from the oracle's "
          f"rounded rows, {int(np.count_nonzero(d > H.bf16_ulp(want[..., :512])))} by more than one bf16 ulp "
          f"of the value (within the fp32 accumulation term)")
    assert np.all(d <= 2.0 ** -7 * np.abs(want[..., :512]) + 2.0 ** -18 * rms)
    pair = np.sqrt(want[..., 512::2] ** 2 + want[..., 513::2] ** 2).repeat(2, axis=-1)
    assert np.all(np.abs(got[..., 512:] - want[..., 512:]) <= 2.0 ** -6 * pair + 1e-30)


def test_append_many_tokens_bad_position_is_skipped():
    x = _many_token_append_case(35, dyadic=False)
    x["positions"] = x["positions"].copy()
    x["positions"][1, 5] = x["block_table"].shape[1] * 64          # one past the table row
    before = x["pool"].copy()
    c, after = _append_many(x)
    assert int(c.status.item()) & 0x4
    changed = np.any(after != before, axis=-1)
    assert changed.sum() == 2200 - 1


@pytest.mark.parametrize("num_splits", [1, 7, 0])
def test_weights_sum_to_one_through_the_whole_path(num_splits):
    """Every cached latent's first feature set to 1 and every head's first W^UV row set to
    e_0: the first output feature of every row is then sum_j p_j = 1, whatever the scores,
    the paging, the split count and the merge.  The weights are rounded to bf16 once and the
    weight sum adds the same rounded values; the partial latent sums carry one bf16 rounding
    (at most 2^-9 relative), which the output's own rounding to bf16 absorbs, so the first
    feature must come out within one bf16 step below 1."""
    spec = H.small_spec("sum_one", 3, 2, [65, 700, 2049], seed=15)
    x = synth.make_inputs(spec)
    pool = x["pool"].copy()
    pool[..., 0] = 0x3F80                                    # bf16 1.0
    x["pool"] = pool
    w_uv = synth.bf16_bits_to_f32(x["w_uv"]).copy()
    rows0 = np.arange(spec.n_heads) * spec.d_nope            # row 0 of each head's W^UV_i
    w_uv[rows0, :] = 0.0
    w_uv[rows0, 0] = 1.0
    x["w_uv"] = synth.f32_to_bf16_bits(w_uv.astype(np.float32))
    import torch
    c = H.GpuCase(x, num_splits)
    c.decode()
    torch.cuda.synchronize()
    o0 = H.host(c.out)[..., 0].astype(np.float64)
    H.log(f"  sum_one splits={num_splits}: first feature in [{o0.min():.6f}, {o0.max():.6f}]")
    assert np.all(np.abs(o0 - 1.0) <= 2.0 ** -8), (o0.min(), o0.max())
