"""The oracle against what the pages and mathematics fix (CPU only)."""
import json
import math
import os
import types

import numpy as np
import pytest

from oracle import mla_oracle
from tests import oracle_pins as pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "cache_accounting.json")


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    assert pin(mla_oracle) < pins.PIN_TOL


def test_cache_accounting_matches_pages():
    g = json.load(open(GOLDEN))
    mla = mla_oracle.latent_elements_per_token(g["v2_mla_elements_per_token"]["d_latent"],
                                               g["v2_mla_elements_per_token"]["d_rope"])
    mha = mla_oracle.mha_elements_per_token(g["v2_mha_elements_per_token"]["n_heads"],
                                            g["v2_mha_elements_per_token"]["d_head"])
    assert mla == g["v2_mla_elements_per_token"]["value"]
    assert mha == g["v2_mha_elements_per_token"]["value"]
    assert mha * g["v2_mha_elements_per_token_60_layers"]["layers"] == g["v2_mha_elements_per_token_60_layers"]["value"]
    assert round(mha / mla, 1) == g["v2_compression_ratio"]["value"]
    # MLA's cache expressed as a number of GQA groups: 2 n_g d_h = d_c + d_R
    assert mla / mla_oracle.gqa_elements_per_token(1, g["v2_equivalent_gqa_groups"]["d_head"]) == g["v2_equivalent_gqa_groups"]["value"]
    assert round(100 * 64 / mla, 1) == g["v2_rope_key_share_percent"]["value"]


def test_demo_element_counts():
    g = json.load(open(GOLDEN))["demo_counts"]
    B, L, H, D = g["batch"], g["seq_len"], g["heads"], g["head_dim"]
    tokens = B * L
    assert mla_oracle.mha_elements_per_token(H, D) * tokens == g["mha"]
    assert mla_oracle.mqa_elements_per_token(D) * tokens == g["mqa"]
    assert mla_oracle.gqa_elements_per_token(g["gqa_groups"], D) * tokens == g["gqa"]
    # that demo caches two separate latents of width D_c and no rotary key
    assert mla_oracle.latent_elements_per_token(2 * g["latent_dim"], 0) * tokens == g["mla_separate_latents"]


# Planted mistakes: each is a plausible slip in the oracle; at least one pin must catch it.
MUTANTS = {
    "rope_sign": ("out[..., 0::2] = even * c - odd * s", "out[..., 0::2] = even * c + odd * s"),
    "rope_freq": ("theta = np.power(float(base), -2.0 * i / d)", "theta = np.power(float(base), -1.0 * i / d)"),
    "rope_half_split": ("even, odd = x[..., 0::2], x[..., 1::2]", "even, odd = x[..., :d // 2], x[..., d // 2:]"),
    "wrong_head_slice": ("            wk = w_uk[i * dn:(i + 1) * dn]            # d_h x d_c",
                         "            wk = w_uk[((i + 1) % H) * dn:((i + 1) % H + 1) * dn]"),
    "value_from_wk": ("            v = c @ wv.T                                # L x d_h", "            v = c @ wk.T"),
    "rope_key_dropped": ("k = np.concatenate([c @ wk.T, kr], axis=1)", "k = np.concatenate([c @ wk.T, 0 * kr], axis=1)"),
    "causal_off_by_one": ("                n = L - Sq + s + 1\n                if n <= 0:\n                    out[b, s, i], lse[b, s, i] = 0.0, -np.inf\n                    continue\n                q = np.concatenate",
                          "                n = L - Sq + s + (s == 0)\n                if n <= 0:\n                    out[b, s, i], lse[b, s, i] = 0.0, -np.inf\n                    continue\n                q = np.concatenate"),
    "causal_group_sees_all": ("                n = L - Sq + s + 1\n                if n <= 0:",
                              "                n = L\n                if n <= 0:"),
    "out_project_transposed": ("return o.reshape(B, S, -1) @ np.asarray(w_o, dtype=np.float64).T",
                               "return o.reshape(B, S, -1) @ np.asarray(w_o, dtype=np.float64)"),
    "layer_queries_uncompressed": ("return q_project(q_compress(h, w_dq), w_uq, w_qr, positions, n_heads, rope_base)",
                                   "return q_project(h, w_uq, w_qr, positions, n_heads, rope_base)"),
    "scale_dropped": ("_softmax_attend(scale * (k[:n] @ q), v[:n])", "_softmax_attend((k[:n] @ q), v[:n])"),
    "softmax_unnormalised": ("return (e / den) @ v, m + math.log(den)", "return (e / len(e)) @ v, m + math.log(den)"),
    "bf16_nine_bits": ("return _round_significand(x, 8, -126, 127)", "return _round_significand(x, 9, -126, 127)"),
    "gather_slot": ("np.asarray(pool[np.asarray(block_table)[j // block_size], j % block_size]",
                    "np.asarray(pool[np.asarray(block_table)[j // block_size], (j * 3) % block_size]"),
    "write_slot": ("p % block_size, :] = rows[b, t]", "(p + 1) % block_size, :] = rows[b, t]"),
    "q_rope_position": ("return qn, rope(qr, np.asarray(positions)[..., None], rope_base)",
                        "return qn, rope(qr, np.asarray(positions)[..., None] + 1, rope_base)"),
    "append_without_rope": ("kr = rope(h @ np.asarray(w_kr, dtype=np.float64).T, positions, rope_base)",
                            "kr = h @ np.asarray(w_kr, dtype=np.float64).T"),
    "e4m3_bias_8": ("vals[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)",
                    "vals[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 8)"),
    "e4m3_subnormal_as_normal": ("vals[code] = sign * (m / 8.0) * 2.0 ** -6",
                                 "vals[code] = sign * (1.0 + m / 8.0) * 2.0 ** -7"),
    "e4m3_ties_up": ("pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))",
                     "pick_hi = (d_hi <= d_lo)"),
    "e4m3_sign_dropped": ("return (mag_code | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)",
                          "return (mag_code | np.where(y < 0, 0x80, 0)).astype(np.uint8)"),
    "fp8_scale_one_binade_low": ("k = np.where(512.0 * m <= E4M3_MAX, e - 9, e - 8)",
                                 "k = np.where(512.0 * m <= E4M3_MAX, e - 10, e - 9)"),
    "fp8_scale_boundary": ("k = np.where(512.0 * m <= E4M3_MAX, e - 9, e - 8)",
                           "k = np.where(512.0 * m < E4M3_MAX, e - 9, e - 8)"),
    "fp8_scale_no_floor": ("    k = np.maximum(k, -124)\n", "    k = np.maximum(k, -200)\n"),
    "fp8_scale_not_applied": ("lat = e4m3_values()[np.asarray(codes, dtype=np.int64)] * np.asarray(scales, dtype=np.float64)[..., None]",
                              "lat = e4m3_values()[np.asarray(codes, dtype=np.int64)] * 1.0"),
    "fp8_page_rope_after_scales": ("    return np.concatenate([codes.reshape(nb, -1), rope_b.view(np.uint8).reshape(nb, -1),\n"
                                   "                           sc.view(np.uint8).reshape(nb, -1)], axis=1)",
                                   "    return np.concatenate([codes.reshape(nb, -1), sc.view(np.uint8).reshape(nb, -1),\n"
                                   "                           rope_b.view(np.uint8).reshape(nb, -1)], axis=1)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    src = open(mla_oracle.__file__, encoding="utf-8").read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    worst = 0.0
    for pin in pins.ALL_PINS:
        try:
            e = pin(mod)
        except Exception:
            e = math.inf
        if not e < pins.PIN_TOL:
            worst = math.inf
            break
    assert worst == math.inf, f"no pin caught the planted mistake {name}"
