"""mla_decode_noalloc, the decode entry point that allocates nothing (its workspace is the
library's own per-GPU scratch array), against mla_decode with a caller workspace, through
the C ABI: two calls in a row, the first at the decode benchmark's shape (batch 64,
context 8192, 128 heads), the second smaller (batch 3, two query tokens), each output and
lse bit for bit equal to mla_decode's with the same split count; the smaller one is also
compared with the oracle over its whole output (rel-L2 <= 1e-2, max-abs <= 2e-2)."""
import numpy as np
import pytest

from mla_rank_latent_amd import synth
from tests import harness as H

pytestmark = pytest.mark.gpu


def _both(x):
    import torch
    from mla_rank_latent_amd import mla
    c = H.GpuCase(x)
    c.decode()
    torch.cuda.synchronize()
    out_ref = c.out.view(torch.int16).cpu().numpy().copy()
    lse_ref = c.lse.cpu().numpy().copy()
    out = torch.full_like(c.out, float("nan"))
    lse = torch.full_like(c.lse, float("nan"))
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    mla.mla_decode_noalloc(c.d, c.q_nope, c.q_rope, c.w_uk, c.w_uv, c.pool, c.block_table, c.seq_lens, x["scale"],
                           out, lse=lse, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0 and int(c.status.item()) == 0
    got = out.view(torch.int16).cpu().numpy()
    assert np.array_equal(got, out_ref)
    assert np.array_equal(lse.cpu().numpy(), lse_ref)
    return H.host(out), lse.cpu().numpy()


def test_noalloc_decode_equals_decode_twice_then_smaller():
    from mla_rank_latent_amd import mla
    big = synth.presets()["v2_b64_ctx8192_paged_append"]
    x = synth.make_inputs(big)
    need = mla.mla_decode_workspace_bytes(H.mla_dims(big), big.batch, big.sq)
    H.log(f"noalloc 1: {big.name} workspace {need} of {mla.MLA_NOALLOC_SCRATCH_BYTES} bytes")
    assert 0 < need <= mla.MLA_NOALLOC_SCRATCH_BYTES
    _both(x)
    del x
    small = H.small_spec("noalloc_b3_sq2", 3, 2, [700, 2000, 129], seed=71)
    x = synth.make_inputs(small)
    H.log(f"noalloc 2: {small.name} lens={list(x['seq_lens'])}")
    out, lse = _both(x)
    ref, ref_lse = H.oracle_decode(x)
    H.assert_close(out, ref, "bf16", small.name)
    assert np.max(np.abs(lse - ref_lse)) <= 2e-2
