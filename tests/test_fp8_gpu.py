"""The FP8 latent cache on the GPU, through the C ABI, against the fp64 oracle.

The GPU side runs the product chain: the library's quantiser (mla_cache_quantize)
turns the bf16 pool into pages, then decode reads them.  The oracle's side: its
own quantisation of the bf16 blocks and the float64 values those stand for
(what it decodes).  Quantisation is integer work and is compared bit for bit;
decode over the FP8 cache computes on exactly those values, so it is held to the
bf16 tolerance (rel-L2 <= 1e-2, max-abs <= 2e-2).  Tests that craft page bytes
hand the GPU the oracle's pages instead."""
import numpy as np
import pytest

from mla_rank_latent_amd import synth
from oracle import mla_oracle
from tests import harness as H

pytestmark = pytest.mark.gpu

PAGE = mla_oracle.fp8_page_bytes(64, 512, 64)


@pytest.fixture(scope="module", autouse=True)
def _torch_cuda():
    import torch
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def _pages_host(t) -> np.ndarray:
    return t.cpu().numpy().astype(np.uint8)


def _special_block(rng) -> np.ndarray:
    """64 bf16 rows (bit patterns) that reach the quantiser's corners: an all-zero row,
    negative zeros, amax exactly 448 * 2^k, every midpoint between neighbouring codes
    (ties), values that land in the subnormal codes, a huge dynamic range, tiny rows
    below the scale floor, sentinel-sized values."""
    E = mla_oracle.e4m3_values()[:0x7F]
    rows = np.zeros((64, 576))
    rows[1, :] = -0.0
    rows[2, :] = rng.standard_normal(576)
    rows[2, 17] = 448.0 * 2.0 ** -3
    mids = (E[:-1] + E[1:]) / 2
    for r in range(3, 8):   # midpoints at scale 2^(r - 5), with a 448 to pin the scale
        s = 2.0 ** (r - 5)
        sel = mids[(r - 3) * 100 // 4:][:511]
        rows[r, :len(sel)] = sel * s * np.where(np.arange(len(sel)) % 2, -1, 1)
        rows[r, 511] = 448.0 * s
    rows[8, :] = rng.standard_normal(576) * 1e-3
    rows[8, 5] = 300.0                      # the rest lands in small and subnormal codes
    rows[9, :] = rng.standard_normal(576)
    rows[9, 0], rows[9, 1] = 1e30, -1e-30   # huge dynamic range
    rows[10, :] = rng.standard_normal(576) * 1e-37   # below the scale floor 448 * 2^-124
    rows[11, :] = 1.33e7
    rows[12:, :] = rng.standard_normal((52, 576)) * np.exp(rng.uniform(-8, 8, (52, 1)))
    bits = synth.f32_to_bf16_bits(rows.astype(np.float32))
    bits[1, :] = 0x8000
    return bits


def test_quantize_matches_oracle_bit_for_bit():
    """mla_cache_quantize over a generated pool plus a block of corner-case rows: every byte of
    every page equals the oracle's quantisation (codes, k^R, scales)."""
    import torch
    from mla_rank_latent_amd import mla
    spec = H.small_spec("fp8_quant_b3", 3, 1, [300, 64, 901], seed=41)
    x = synth.make_inputs(spec)
    pool = np.concatenate([x["pool"], _special_block(np.random.default_rng(42))[None]], axis=0)
    H.log(f"fp8 quantize: {pool.shape[0]} blocks")
    src = H.dev(pool, "bf16")
    pages = torch.full((pool.shape[0], PAGE), 0xA5, dtype=torch.uint8, device="cuda")
    mla.mla_cache_quantize(H.mla_dims(spec, "fp8"), src, pages)
    torch.cuda.synchronize()
    got = _pages_host(pages)
    want = H.fp8_pages(pool, 512)
    bad = np.nonzero(got != want)
    assert bad[0].size == 0, f"{bad[0].size} bytes differ, first at page {bad[0][0]} byte {bad[1][0]}"


def _fp8_case(spec, num_splits=0):
    x = H.with_fp8_cache(synth.make_inputs(spec))
    H.log(f"{spec.name} seed={spec.seed} B={spec.batch} sq={spec.sq} H={spec.n_heads} "
          f"lens={list(x['seq_lens'])[:8]} splits={num_splits}")
    c = H.GpuCase(x, num_splits, cache="fp8")
    c.decode()
    import torch
    torch.cuda.synchronize()
    return x, c


@pytest.mark.parametrize("name,batch,sq,lens,paged,n_heads", [
    ("fp8_contig_b1_l300", 1, 1, [300], False, 128),
    ("fp8_paged_b3_ragged", 3, 1, [1, 100, 700], True, 128),
    ("fp8_paged_b4_sq2", 4, 2, [2, 65, 130, 513], True, 128),
    ("fp8_paged_b2_sq3", 2, 3, [3, 200], True, 128),
    ("fp8_paged_b2_sq8", 2, 8, [8, 1000], True, 128),
    ("fp8_h16_b3", 3, 1, [64, 130, 900], True, 16),
    ("fp8_h72_b2_sq2", 2, 2, [33, 2000], True, 72),
    ("fp8_h200_b2", 2, 1, [97, 640], True, 200),
    # 300 sequences: the planner's scans over two 256-sequence chunks, ten row blocks of 32
    ("fp8_paged_b300", 300, 1, [1 + (37 * b + 11) % 250 for b in range(300)], True, 128),
])
def test_fp8_decode_matches_oracle(name, batch, sq, lens, paged, n_heads):
    spec = synth.Spec(name, batch=batch, sq=sq, seq_lens=list(lens), paged=paged, seed=43 + batch + sq,
                      n_heads=n_heads)
    x, c = _fp8_case(spec)
    assert int(c.status.item()) == 0
    ref, lse = H.oracle_decode(x)
    H.assert_close(H.host(c.out), ref, "bf16", name)
    assert np.max(np.abs(H.host(c.lse) - lse)) <= 2e-2


def test_fp8_split_counts_agree():
    spec = H.small_spec("fp8_splits_b3", 3, 1, [1, 900, 2000], seed=44)
    x = H.with_fp8_cache(synth.make_inputs(spec))
    ref, _ = H.oracle_decode(x)
    import torch
    outs = []
    for ns in (1, 5, 64, 256):
        H.log(f"fp8_splits_b3 num_splits={ns}")
        c = H.GpuCase(x, ns, cache="fp8")
        c.decode()
        torch.cuda.synchronize()
        o = H.host(c.out)
        H.assert_close(o, ref, "bf16", f"fp8 splits={ns}")
        outs.append(o)
    for o in outs[1:]:
        assert H.rel_l2(o, outs[0]) <= 4e-3


def test_fp8_decode_tracks_bf16_decode_of_the_same_values():
    """The FP8 kernel on the pages and the bf16 kernel on a bf16 pool holding the values the
    pages stand for (exact in bf16) see the same operands; they differ only in summation
    order and in rounding p s instead of p to bf16."""
    import torch
    spec = H.small_spec("fp8_vs_bf16_b3", 3, 2, [70, 513, 1500], seed=45)
    x = H.with_fp8_cache(synth.make_inputs(spec), pages=True)
    x["pages_given"] = False          # the GPU quantises the pool itself
    vals = mla_oracle.dequantize_pages(x["pages"], 64, 512, 64)
    y = dict(x)
    del y["fp8"]
    y["pool"] = synth.f32_to_bf16_bits(vals.astype(np.float32))
    assert np.array_equal(synth.as_float(y["pool"], "bf16"), vals)   # exact in bf16
    H.log("fp8_vs_bf16_b3")
    c8 = H.GpuCase(x, cache="fp8")
    c8.decode()
    cb = H.GpuCase(y)
    cb.decode()
    torch.cuda.synchronize()
    assert H.rel_l2(H.host(c8.out), H.host(cb.out)) <= 3e-3
    assert np.max(np.abs(H.host(c8.lse) - H.host(cb.lse))) <= 5e-3


def test_fp8_garbage_past_sequence_end_is_invisible():
    """Slots past a sequence's end may hold any bytes: NaN scales and NaN codes there change no
    output bit."""
    import torch
    spec = H.small_spec("fp8_garbage_b3", 3, 2, [70, 300, 33], seed=46)
    x = H.with_fp8_cache(synth.make_inputs(spec), pages=True)   # page bytes crafted below
    dirty = dict(x)
    pages = x["pages"].copy()
    for b in range(3):
        L = int(x["seq_lens"][b])
        for p in range(L, (L + 63) // 64 * 64):
            blk = x["block_table"][b, p // 64]
            pages[blk, (p % 64) * 512:(p % 64 + 1) * 512] = 0x7F                    # NaN codes
            pages[blk, 40960 + 4 * (p % 64):40960 + 4 * (p % 64) + 4] = [0, 0, 0xC0, 0x7F]   # NaN scale
    dirty["pages"] = pages
    outs = []
    for z in (x, dirty):
        H.log(f"fp8_garbage_b3 {'dirty' if z is dirty else 'clean'}")
        c = H.GpuCase(z, cache="fp8")
        c.decode()
        torch.cuda.synchronize()
        assert int(c.status.item()) == 0
        outs.append((c.out.view(torch.int16).cpu().numpy(), c.lse.cpu().numpy(), H.host(c.out)))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    ref, _ = H.oracle_decode(x)
    H.assert_close(outs[1][2], ref, "bf16", "fp8_garbage_b3")


def test_fp8_bad_block_is_reported_and_clamped():
    import torch
    spec = H.small_spec("fp8_badblk_b2", 2, 1, [200, 260], seed=47)
    x = H.with_fp8_cache(synth.make_inputs(spec))
    x["block_table"] = x["block_table"].copy()
    x["block_table"][1, 2] = 1 << 20
    H.log("fp8_badblk_b2")
    c = H.GpuCase(x, cache="fp8")
    c.decode()
    torch.cuda.synchronize()
    assert int(c.status.item()) & 0x1
    out = H.host(c.out)
    assert np.all(np.isfinite(out))
    ref, _ = H.oracle_decode(x, batches=[0])
    H.assert_close(out[:1], ref[:1], "bf16", "fp8_badblk_b2 seq 0")


def _dyadic(x, seed):
    rng = np.random.default_rng(seed)
    x["h"] = synth.f32_to_bf16_bits(rng.integers(-2, 3, size=x["h"].shape).astype(np.float32))
    x["w_dkv"] = synth.f32_to_bf16_bits((rng.integers(-64, 65, size=x["w_dkv"].shape) / 64.0).astype(np.float32))
    x["w_kr"] = synth.f32_to_bf16_bits((rng.integers(-64, 65, size=x["w_kr"].shape) / 64.0).astype(np.float32))
    return x


@pytest.mark.parametrize("many", [False, True])
def test_fp8_append_dyadic_is_bit_exact(many):
    """On dyadic inputs the latent row is exact, so the appended codes and scales equal the
    oracle's quantisation of its own row bit for bit; k^R is within one bf16 ulp; no other
    byte of the pool changes.  many: 2200 rows (the single-GEMM append path)."""
    import torch
    if many:
        spec = synth.Spec("fp8_append_many", batch=2, sq=1100, seq_lens=[1100, 1300], paged=True, append=True,
                          seed=48, n_heads=8)
    else:
        spec = H.small_spec("fp8_append_b3", 3, 1, [64, 130, 7], append=True, seed=49)
    x = H.with_fp8_cache(_dyadic(synth.make_inputs(spec), 50))
    H.log(f"{spec.name} fp8 append rows={spec.batch * x['h'].shape[1]}")
    c = H.GpuCase(x, cache="fp8")
    before = _pages_host(c.pool)
    assert np.array_equal(before, H.fp8_pages(x["pool"], 512))   # the library's quantiser, bit for bit
    c.append(True)
    torch.cuda.synchronize()
    assert int(c.status.item()) == 0
    after = _pages_host(c.pool)
    rows = H.oracle_append_rows(x)                       # bf16-exact latent part
    codes, scales, _ = mla_oracle.quantize_rows(rows, 512)
    touched = np.zeros((after.shape[0], 64), dtype=bool)
    rc, rr, rs = mla_oracle.unpack_fp8_pages(after, 64, 512, 64)
    for b in range(spec.batch):
        for t, p in enumerate(x["positions"][b]):
            blk, slot = x["block_table"][b, p // 64], p % 64
            touched[blk, slot] = True
            assert np.array_equal(rc[blk, slot], codes[b, t]), (b, t)
            assert rs[blk, slot] == scales[b, t], (b, t)
            kr = synth.bf16_bits_to_f32(rr[blk, slot]).astype(np.float64)
            assert np.all(np.abs(kr - rows[b, t, 512:]) <= H.bf16_ulp(rows[b, t, 512:]) + 1e-30)
    bc, br, bsc = mla_oracle.unpack_fp8_pages(before, 64, 512, 64)
    assert np.array_equal(rc[~touched], bc[~touched]) and np.array_equal(rr[~touched], br[~touched])
    assert np.array_equal(rs[~touched].view(np.uint32), bsc[~touched].view(np.uint32))


def test_fp8_append_is_quantize_of_bf16_append():
    """On N(0,1) data: appending into the FP8 cache writes exactly the pages that
    mla_cache_quantize makes from the bf16 cache after a bf16 append of the same rows."""
    import torch
    from mla_rank_latent_amd import mla
    spec = H.small_spec("fp8_append_vs_bf16_b5", 5, 1, [1, 64, 65, 300, 1000], append=True, seed=51)
    x = synth.make_inputs(spec)
    x8 = H.with_fp8_cache(x)
    H.log("fp8_append_vs_bf16_b5")
    cb = H.GpuCase(x)
    cb.append(True)
    c8 = H.GpuCase(x8, cache="fp8")
    c8.append(True)
    q = torch.empty_like(c8.pool)
    mla.mla_cache_quantize(c8.d, cb.pool, q)
    torch.cuda.synchronize()
    assert int(cb.status.item()) == 0 and int(c8.status.item()) == 0
    assert torch.equal(q, c8.pool)


def test_fp8_append_then_decode():
    import torch
    spec = H.small_spec("fp8_append_decode_b2", 2, 1, [130, 64], append=True, seed=52)
    x = H.with_fp8_cache(synth.make_inputs(spec))
    H.log("fp8_append_decode_b2")
    c = H.GpuCase(x, cache="fp8")
    c.step()
    torch.cuda.synchronize()
    assert int(c.status.item()) == 0
    rows = H.oracle_append_rows(x)
    codes, scales, rope = mla_oracle.quantize_rows(rows, 512)
    ref, _ = H.oracle_decode(x, appended_rows=mla_oracle.dequantize_rows(codes, scales, rope))
    H.assert_close(H.host(c.out), ref, "bf16", "fp8_append_decode_b2 out")


def test_fp8_append_bad_position_is_skipped():
    import torch
    spec = H.small_spec("fp8_badpos_b2", 2, 1, [64, 100], append=True, seed=53)
    x = H.with_fp8_cache(synth.make_inputs(spec))
    x["positions"] = x["positions"].copy()
    x["positions"][0, 0] = 1 << 20
    H.log("fp8_badpos_b2")
    c = H.GpuCase(x, cache="fp8")
    before = _pages_host(c.pool)
    c.append(True)
    torch.cuda.synchronize()
    assert int(c.status.item()) & 0x4
    after = _pages_host(c.pool)
    p = int(x["positions"][1, 0])
    blk = x["block_table"][1, p // 64]
    changed = np.nonzero(np.any(after != before, axis=1))[0]
    assert set(changed.tolist()) <= {int(blk)}
