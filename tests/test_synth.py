"""The seeded input generator (CPU only)."""
import numpy as np
import torch

from mla_rank_latent_amd import synth


def _small(**kw):
    base = dict(name="small", batch=3, sq=1, seed=7, seq_lens=[100, 64, 1], paged=True)
    base.update(kw)
    return synth.Spec(**base)


def test_deterministic():
    a = synth.make_inputs(_small())
    b = synth.make_inputs(_small())
    for k in ("pool", "block_table", "q_nope", "q_rope", "w_uk", "w_uv"):
        assert np.array_equal(a[k], b[k])
    c = synth.make_inputs(_small(seed=8))
    assert not np.array_equal(a["pool"], c["pool"])


def test_block_table_is_a_permutation():
    x = synth.make_inputs(_small())
    bt, lens = x["block_table"], x["seq_lens"]
    used = np.concatenate([bt[b, :(lens[b] + 63) // 64] for b in range(3)])
    assert sorted(used.tolist()) == list(range(x["num_blocks"]))
    assert np.all(bt[2, 1:] == -1)
    y = synth.make_inputs(_small(paged=False))
    assert y["block_table"][0, 1] == 1 and y["block_table"][1, 0] == 2


def test_shapes_dtypes_and_sentinels():
    x = synth.make_inputs(_small(append=True))
    assert x["pool"].dtype == np.uint16 and x["pool"].shape == (x["num_blocks"], 64, 576)
    assert x["q_nope"].shape == (3, 1, 128, 128) and x["q_rope"].shape == (3, 1, 128, 64)
    assert x["w_uk"].shape == (128 * 128, 512) and x["h"].shape == (3, 1, 5120)
    assert np.array_equal(x["positions"][:, 0], [99, 63, 0])
    bt = x["block_table"]
    # the append slot and everything past the end hold the sentinel
    assert np.all(x["pool"][bt[0, 1], 99 - 64] == synth.SENTINEL_BF16)
    assert np.all(x["pool"][bt[0, 1], 40:] == synth.SENTINEL_BF16)
    assert not np.any(x["pool"][bt[0, 0], :] == synth.SENTINEL_BF16)


def test_ragged_lengths_in_range():
    x = synth.make_inputs(synth.Spec("r", batch=50, sq=2, seed=4, ragged=(512, 600), d_model=64))
    assert x["seq_lens"].min() >= 512 and x["seq_lens"].max() <= 600


def test_bf16_cast_matches_torch():
    rng = np.random.default_rng(0)
    v = (rng.standard_normal(100000) * np.exp(rng.uniform(-30, 30, 100000))).astype(np.float32)
    mine = synth.f32_to_bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    assert np.array_equal(synth.bf16_bits_to_f32(mine), torch.from_numpy(v).to(torch.bfloat16).float().numpy())


def test_weight_variance_is_one_over_fan_in():
    x = synth.make_inputs(_small())
    w = synth.as_float(x["w_uk"], "bf16")
    assert abs(w.var() * 512 - 1.0) < 0.01


def test_presets_cover_the_five_workloads():
    p = synth.presets()
    assert len(p) == 5
    t = p["tiny_f32_ctx65"]
    assert (t.n_heads, t.d_nope, t.d_rope, t.d_latent, t.d_model, t.dtype) == (8, 16, 8, 32, 64, "f32")
    assert abs(t.softmax_scale() - 1 / np.sqrt(24)) < 1e-15
    assert abs(p["v2_b1_ctx4096"].softmax_scale() - 1 / np.sqrt(192)) < 1e-15
    x = synth.make_inputs(t)
    assert x["h"].shape == (1, 65, 64) and np.array_equal(x["positions"][0], np.arange(65))
    assert np.array_equal(x["q_positions"], [[64]])
