"""The full layer's projections (mla_q_compress, mla_out_project) and the whole
layer decode step on the GPU, through the C ABI, against the fp64 oracle: the
compressed query c^Q = W^DQ h and its up-projections q^C = W^UQ c^Q and
q^R = RoPE(W^QR c^Q), the output u = W^O [o_1; ...], and append -> queries ->
decode -> u end to end, at small sizes and on one whole sequence of the
benchmarked batch-64, context-8192 step."""
import numpy as np
import pytest

from mla_rank_latent_amd import synth
from oracle import mla_oracle
from tests import harness as H

pytestmark = pytest.mark.gpu


def _spec(name, lens, sq=1, n_heads=128, seed=81):
    return synth.Spec(name, batch=len(lens), sq=sq, seq_lens=list(lens), paged=True, append=True, layer=True,
                      seed=seed, n_heads=n_heads)


def test_q_compress_matches_oracle():
    import torch
    from mla_rank_latent_amd import mla
    x = synth.make_inputs(_spec("layer_q", [40, 70, 9], sq=2, n_heads=16, seed=83))
    H.log("layer_q B=3 sq=2 H=16")
    c = H.LayerCase(x)
    mla.mla_q_compress(c.d, c.spec.d_qlat, c.h_q, c.w_dq, c.w_uq, c.w_qr_c, c.q_positions, c.q_nope, c.q_rope, c.lws)
    torch.cuda.synchronize()
    spec = x["spec"]
    f = lambda k: synth.as_float(x[k], spec.dtype)
    qn, qr = mla_oracle.layer_queries(f("h")[:, -2:], f("w_dq"), f("w_uq"), f("w_qr_c"), x["q_positions"],
                                      spec.n_heads, spec.rope_base)
    H.assert_close(H.host(c.q_nope), qn, "bf16", "q_nope")
    H.assert_close(H.host(c.q_rope), qr, "bf16", "q_rope")


def test_out_project_matches_oracle():
    import torch
    from mla_rank_latent_amd import mla
    x = synth.make_inputs(_spec("layer_o", [40, 70, 9], sq=3, n_heads=24, seed=85))
    H.log("layer_o B=3 sq=3 H=24")
    c = H.LayerCase(x)
    rng = np.random.default_rng(86)
    o = synth.f32_to_bf16_bits(rng.standard_normal(c.out.shape).astype(np.float32))
    c.out.copy_(H.dev(o, "bf16"))
    mla.mla_out_project(c.d, c.out, c.w_o, c.u, c.lws)
    torch.cuda.synchronize()
    want = mla_oracle.out_project(synth.as_float(o, "bf16"), synth.as_float(x["w_o"], "bf16"))
    H.assert_close(H.host(c.u), want, "bf16", "u")


@pytest.mark.parametrize("lens,sq", [([130, 64], 1), ([300, 3, 77], 2)])
def test_layer_step_matches_oracle(lens, sq):
    import torch
    x = synth.make_inputs(_spec(f"layer_step_sq{sq}", lens, sq=sq, seed=87 + sq))
    H.log(f"layer_step lens={lens} sq={sq}")
    c = H.LayerCase(x)
    c.layer_step()
    torch.cuda.synchronize()
    assert int(c.status.item()) == 0
    u, _, _ = H.oracle_layer(x)
    H.assert_close(H.host(c.u), u, "bf16", "layer u")


def test_layer_full_size_one_sequence():
    """The benchmarked full-layer step (64 sequences at context 8192, 128 heads):
    u of one whole sequence (every head contributes to it) against the oracle."""
    import torch
    x = synth.make_inputs(synth.layer_presets()["layer_b64_ctx8192"])
    H.log("layer_b64_ctx8192")
    c = H.LayerCase(x)
    c.layer_step()
    torch.cuda.synchronize()
    assert int(c.status.item()) == 0
    b = 37
    u, _, _ = H.oracle_layer(x, batches=[b])
    H.assert_close(H.host(c.u)[b:b + 1], u[b:b + 1], "bf16", "layer u, sequence 37")
    assert np.all(np.isfinite(H.host(c.u)))
