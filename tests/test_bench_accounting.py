"""The benchmark's accounting, on the CPU: the algorithmic bytes and flops bench.py divides by
(written out here from the per-token figures, not from bench.py's code), the HBM/MFMA bound it
picks from the arithmetic intensity, the number of input copies it rotates over, and that the
counter profile of the benchmarked workload was taken from the attention sources as they stand
(otherwise bench.py reports its traffic as null).

Per-token figures ("DeepSeek-V2: Multi-Head Latent Attention (MLA) 原理与工程实现" §3.3 and
§2.2): a cached token is d_c + d_h^R = 576 elements (1152 B in bf16), read once per step; a
visible token costs 2 n_h (576 + 512) flop per query row (scores over [c ‖ k^R], then the
latent weighted sum)."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
from mla_rank_latent_amd import synth  # noqa: E402

H, DN, DR, DC, D = 128, 128, 64, 512, 5120


def test_benchmark_step_bytes_and_flops():
    """Batch 64 x context 8192 with one appended token per sequence."""
    spec = synth.presets()["v2_b64_ctx8192_paged_append"]
    wl = bench.workload_bytes_flops(spec, spec.seq_lens)
    tokens = 64 * 8192
    cache = tokens * 1152
    weights = 2 * H * DN * DC * 2                               # W^UK, W^UV
    queries = 64 * H * (DN + DR) * 2
    out = 64 * H * DN * 2
    append = ((DC + DR) * D + 64 * D) * 2 + 64 * 1152            # W^DKV, W^KR, h, the new rows
    assert wl["cache_bytes"] == cache == 603_979_776
    assert wl["bytes"] == cache + weights + queries + out + append == 649_404_416
    attn = tokens * 2 * H * (576 + 512)
    proj = 2 * 2 * 64 * H * DN * DC                             # absorb and up-projection
    app = 2 * 64 * (DC + DR) * D
    assert wl["attn_flops"] == attn == 146_028_888_064
    assert wl["flops"] == attn + proj + app == 148_553_859_072
    # intensity 241.8 flop/B, under the 312.5 flop/B ridge of 2.5 PFLOP/s over 8 TB/s: HBM-bound
    assert wl["attn_flops"] / wl["cache_bytes"] < bench.MFMA_BF16_PEAK_TFLOPS / bench.HBM_PEAK_GBS * 1e3


def test_two_query_tokens_count_the_causal_pair():
    """At two query tokens per sequence the first sees one token fewer than the second; the
    doubled intensity (483 flop/B) puts the attention over the ridge: MFMA-bound."""
    spec = synth.Spec("acct_sq2", batch=3, sq=2, seq_lens=[512, 1000, 32768])
    wl = bench.workload_bytes_flops(spec, spec.seq_lens)
    vis = sum(2 * L - 1 for L in spec.seq_lens)
    assert wl["attn_flops"] == vis * 2 * H * (576 + 512)
    assert wl["cache_bytes"] == sum(spec.seq_lens) * 1152
    assert wl["attn_flops"] / wl["cache_bytes"] > bench.MFMA_BF16_PEAK_TFLOPS / bench.HBM_PEAK_GBS * 1e3


def test_fp8_row_bytes():
    """The FP8 page format per token: 512 E4M3 codes, the bf16 rotary key, one fp32 scale."""
    spec = synth.presets()["v2_b64_ctx8192_paged_append"]
    wl = bench.workload_bytes_flops(spec, spec.seq_lens, fp8=True)
    assert wl["row_bytes"] == 512 + 64 * 2 + 4 == 644
    assert wl["cache_bytes"] == 64 * 8192 * 644


def test_rotation_keeps_every_step_out_of_the_last_level_cache():
    """Between two uses of one input copy the others move at least twice the 256 MB cache."""
    for step_bytes in (649_404_416, 38_400_000, 5_000_000, 300_000_000):
        k = bench.rotation_copies(0, step_bytes)
        assert k >= 2 and (k - 1) * step_bytes >= 2 * bench.MALL_BYTES
        assert k == 2 or (k - 2) * step_bytes < 2 * bench.MALL_BYTES   # the fewest that do
    assert bench.rotation_copies(0, 649_404_416) == 2
    assert bench.rotation_copies(5, 1) == 5


def test_benchmark_counter_profile_matches_the_sources():
    """bench.py reports the attention kernel's counted HBM traffic and MFMA busy fraction only
    while the committed profile's source hash matches the attention sources; for the
    benchmarked workload it must (retake the profile after changing those sources)."""
    got = bench.measured_counters("v2_b64_ctx8192_paged_append")
    assert "traffic" in got and "mfma_busy" in got
    # counted traffic: the cache bytes plus the partial states, queries and block table
    assert 603_979_776 <= got["traffic"] <= 1.2 * 603_979_776
    assert 0.0 < got["mfma_busy"] < 1.0
