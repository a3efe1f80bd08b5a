"""GPU parity at full size, in the launch configuration bench.py times (one
attention workgroup per compute unit), against the fp64 oracle over the whole
output:

* every (sequence, query token, head) of the batch-1 context-4096, the batch-64
  context-8192 (with its append) and the batch-4 long-context workloads, bf16
  and, for the batch-64 step, the FP8 cache made by the library's quantiser;
* the ragged batch-128 two-query workload: every sequence and both query
  tokens on 32 of the 128 heads, a different set per sequence (heads
  b, b + 4, ..., b + 124 mod 128), so each head is compared on 32 sequences
  and both head groups of a workgroup are covered.

Tolerance (rel-L2 <= 1e-2 and plain max-abs <= 2e-2 over the whole compared
set, lse within 2e-2) is checked on everything compared; the logs name the
whole-set figures."""
import numpy as np
import pytest

from mla_rank_latent_amd import synth
from oracle import mla_oracle
from tests import harness as H

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]


def _run(x, cache=""):
    import torch
    spec = x["spec"]
    H.log(f"{spec.name}{' fp8' if cache else ''} seed={spec.seed} B={spec.batch} sq={spec.sq} "
          f"max_len={int(x['seq_lens'].max())} tokens={int(x['seq_lens'].sum())}: append={spec.append} + decode")
    c = H.GpuCase(x, cache=cache)
    c.step()
    torch.cuda.synchronize()
    assert int(c.status.item()) == 0
    return c


def _check(c, ref, lse, what):
    got = H.host(c.out)
    H.assert_close(got, ref, "bf16", what)
    m = ~np.isnan(lse)
    d = np.max(np.abs(H.host(c.lse)[m] - lse[m]))
    H.log(f"  {what}: lse max-abs {d:.3e} over {int(m.sum())} rows")
    assert d <= 2e-2
    assert np.isfinite(got).all()


def _appended_rows_check(c, x, rows):
    """The appended rows in the pool against the oracle's rounded rows: within one bf16 ulp
    (plus the fp32 accumulation term of a 5120-term dot product, 2^-18 of the row's rms, for
    values that cancel to near zero); the number of elements that differ by one ulp is logged."""
    import torch
    pool = c.pool.view(torch.int16).cpu().numpy().view(np.uint16)
    got = np.stack([[synth.bf16_bits_to_f32(pool[x["block_table"][b, p // 64], p % 64]).astype(np.float64)
                     for p in x["positions"][b]] for b in range(x["spec"].batch)])
    d = np.abs(got - rows)
    rms = np.sqrt(np.mean(rows[..., :512] ** 2, axis=-1, keepdims=True))
    lat_ok = d[..., :512] <= 2.0 ** -7 * np.abs(rows[..., :512]) + 2.0 ** -18 * rms
    pair = np.sqrt(rows[..., 512::2] ** 2 + rows[..., 513::2] ** 2).repeat(2, axis=-1)
    rope_ok = d[..., 512:] <= 2.0 ** -6 * pair + 1e-30
    H.log(f"  appended rows: {int(np.count_nonzero(d))} of {d.size} elements differ from the oracle's rounded "
          f"row; {int(np.count_nonzero(d[..., :512] > H.bf16_ulp(rows[..., :512])))} latent elements by more than "
          f"one bf16 ulp of the value (allowed only within the fp32 accumulation term)")
    assert lat_ok.all() and rope_ok.all()


@pytest.mark.parametrize("name", ["v2_b1_ctx4096", "v2_b64_ctx8192_paged_append", "v2_b4_longctx_128k"])
def test_full_size_whole_output(name):
    spec = synth.presets()[name]
    x = synth.make_inputs(spec)
    c = _run(x)
    rows = None
    if spec.append:
        rows = H.oracle_append_rows(x)
        _appended_rows_check(c, x, rows)
    ref, lse = H.oracle_decode(x, appended_rows=rows)
    assert not np.isnan(ref).any()
    _check(c, ref, lse, f"{name} whole output")


def test_ragged_sq2_every_sequence():
    name = "v2_b128_ragged_sq2"
    x = synth.make_inputs(synth.presets()[name])
    c = _run(x)
    heads_of = lambda b: [(b + 4 * k) % 128 for k in range(32)]
    ref, lse = H.oracle_decode(x, heads_of=heads_of)
    assert int(np.count_nonzero(~np.isnan(lse))) == 128 * 2 * 32
    _check(c, ref, lse, f"{name} every sequence, both queries, 32 heads each")


def test_fp8_full_size_whole_output():
    """The benchmarked FP8-cache step: the library quantises the bf16 pool into pages, appends
    one token per sequence and decodes; every (sequence, head) against the oracle's decode of
    its own quantisation of the same blocks and of its own appended rows."""
    spec = synth.presets()["v2_b64_ctx8192_paged_append"]
    x = H.with_fp8_cache(synth.make_inputs(spec))
    c = _run(x, cache="fp8")
    rows = H.oracle_append_rows(x)
    app = mla_oracle.dequantize_rows(*mla_oracle.quantize_rows(rows, 512))
    ref, lse = H.oracle_decode(x, appended_rows=app)
    assert not np.isnan(ref).any()
    _check(c, ref, lse, "fp8 v2_b64_ctx8192_paged_append whole output")


def test_one_sequence_of_a_million_tokens():
    """One sequence of 2^20 cached tokens (an eighth of the 2^23 tokens a table row may
    address), paged over 16384 permuted blocks: 256 token ranges of 4096 tokens each, the
    largest token and block offsets any test reaches.  Three heads (the first, one in the
    middle, the last) against the oracle."""
    spec = synth.Spec("v2_b1_ctx1m", batch=1, sq=1, seed=7, seq_lens=[1 << 20], paged=True)
    x = synth.make_inputs(spec)
    c = _run(x)
    ref, lse = H.oracle_decode(x, heads=[0, 77, 127])
    assert int(np.count_nonzero(~np.isnan(lse))) == 3
    _check(c, ref, lse, "v2_b1_ctx1m heads 0, 77, 127")
