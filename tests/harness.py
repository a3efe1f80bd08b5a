"""Shared helpers for the GPU tests: move generated inputs to the device, run the
library through its binding, and evaluate the oracle on the same inputs."""
from __future__ import annotations

import math
import sys

import numpy as np

from mla_rank_latent_amd import synth
from oracle import mla_oracle


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev(x, dtype: str):
    """numpy array -> torch device tensor; bf16 bit patterns become torch.bfloat16."""
    import torch
    if x.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to("cuda")


def host(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def mla_dims(spec: synth.Spec, cache: str = ""):
    """Library dims for a generated workload; cache="fp8" selects the FP8 page cache."""
    from mla_rank_latent_amd import mla
    dtype = "bf16_fp8" if cache == "fp8" else spec.dtype
    return mla.dims(spec.n_heads, spec.d_nope, spec.d_rope, spec.d_latent, spec.d_model, spec.block_size, dtype,
                    spec.rope_base)


def fp8_pages(pool_bits: np.ndarray, d_latent: int) -> np.ndarray:
    """The oracle's FP8 pages [nb, page bytes] for a bf16 pool (bit patterns [nb, 64, R])."""
    codes, scales, _ = mla_oracle.quantize_rows(synth.as_float(pool_bits, "bf16"), d_latent)
    return mla_oracle.pack_fp8_pages(codes, pool_bits[..., d_latent:], scales)


def with_fp8_cache(x: dict, pages: bool = False) -> dict:
    """A copy of generated inputs whose cache is FP8.  The oracle then reads every block as
    its own quantisation of the bf16 block, dequantised.  The GPU makes its pages from the
    bf16 pool with the library's own quantiser (mla_cache_quantize), unless ``pages``: then
    ``x["pages"]`` holds the oracle's quantisation of the whole pool and the GPU is handed
    those bytes (for tests that craft or inspect page bytes)."""
    x8 = dict(x)
    x8["fp8"] = True
    if pages:
        x8["pages"] = fp8_pages(x["pool"], x["spec"].d_latent)
        x8["pages_given"] = True
    return x8


def pool_blocks(x: dict, blocks) -> np.ndarray:
    """float64 values the oracle reads for the given cache blocks (for an FP8 cache: the
    oracle's quantisation of those bf16 blocks, dequantised)."""
    spec = x["spec"]
    blk = x["pool"][np.asarray(blocks)]
    if x.get("fp8"):
        return mla_oracle.dequantize_pages(fp8_pages(blk, spec.d_latent), spec.block_size, spec.d_latent,
                                           spec.d_rope)
    return synth.as_float(blk, spec.dtype)


class GpuCase:
    """Device copies of one generated workload, plus the calls of one decode step."""
    split_append = True    # append through the workspace (split) path

    def __init__(self, x: dict, num_splits: int = 0, cache: str = ""):
        import torch
        from mla_rank_latent_amd import mla
        self.x = x
        self.spec = spec = x["spec"]
        self.cache = cache
        self.d = mla_dims(spec, cache)
        self.num_splits = num_splits
        if cache == "fp8" and not x.get("pages_given", False):
            # the product chain: the library quantises the bf16 pool into its FP8 pages
            from mla_rank_latent_amd import mla as _mla
            src = dev(x["pool"], spec.dtype)
            self.pool = torch.empty(int(x["pool"].shape[0]), _mla.MLA_FP8_PAGE_BYTES, dtype=torch.uint8,
                                    device="cuda")
            _mla.mla_cache_quantize(self.d, src, self.pool)
            torch.cuda.synchronize()
            del src
        else:
            self.pool = dev(x["pages"] if cache == "fp8" else x["pool"], spec.dtype)
        self.block_table = dev(x["block_table"], spec.dtype)
        self.seq_lens = dev(x["seq_lens"], spec.dtype)
        self.w_uk = dev(x["w_uk"], spec.dtype)
        self.w_uv = dev(x["w_uv"], spec.dtype)
        B, S, H = spec.batch, spec.sq, spec.n_heads
        tdt = torch.bfloat16 if spec.dtype == "bf16" else torch.float32
        if spec.q_from_hidden:
            self.q_nope = torch.empty(B, S, H, spec.d_nope, dtype=tdt, device="cuda")
            self.q_rope = torch.empty(B, S, H, spec.d_rope, dtype=tdt, device="cuda")
        else:
            self.q_nope = dev(x["q_nope"], spec.dtype)
            self.q_rope = dev(x["q_rope"], spec.dtype)
        if "h" in x:
            self.h = dev(x["h"], spec.dtype)
            self.w_dkv = dev(x["w_dkv"], spec.dtype)
            self.w_kr = dev(x["w_kr"], spec.dtype)
            self.positions = dev(x["positions"], spec.dtype)
        if spec.q_from_hidden:
            self.w_q = dev(x["w_q"], spec.dtype)
            self.w_qr = dev(x["w_qr"], spec.dtype)
            self.q_positions = dev(x["q_positions"], spec.dtype)
            self.h_q = self.h[:, -S:].contiguous()
        self.out = torch.empty(B, S, H, spec.d_nope, dtype=tdt, device="cuda")
        self.lse = torch.empty(B, S, H, dtype=torch.float32, device="cuda")
        self.status = torch.zeros(1, dtype=torch.int32, device="cuda")
        # decode's workspace (none for query groups decode does not take, e.g. a
        # many-token append case that only appends)
        nbytes = mla.mla_decode_workspace_bytes(self.d, B, S, num_splits)
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda") if nbytes > 0 else None

    def append(self, split=True):
        """split: use the workspace (split over d_model) path; False: the single-kernel path."""
        import torch
        from mla_rank_latent_amd import mla
        ws = None
        if split:
            n = mla.mla_cache_append_workspace_bytes(self.d, int(self.h.shape[0]), int(self.h.shape[1]))
            ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda") if n else None
        mla.mla_cache_append(self.d, self.h, self.w_dkv, self.w_kr, self.positions, self.block_table, self.pool,
                             workspace=ws, status=self.status)

    def q_project(self):
        from mla_rank_latent_amd import mla
        mla.mla_q_project(self.d, self.h_q, self.w_q, self.w_qr, self.q_positions, self.q_nope, self.q_rope)

    def decode(self, num_splits=None):
        from mla_rank_latent_amd import mla
        assert self.ws is not None, "no decode workspace for this query group"
        mla.mla_decode(self.d, self.q_nope, self.q_rope, self.w_uk, self.w_uv, self.pool, self.block_table,
                       self.seq_lens, self.x["scale"], self.ws, self.out, lse=self.lse, status=self.status,
                       num_splits=self.num_splits if num_splits is None else num_splits)

    def step(self):
        """One pass of the hot path: append (if the workload has one), project (tiny case), decode."""
        if self.spec.append or self.spec.q_from_hidden:
            self.append(self.split_append)
        if self.spec.q_from_hidden:
            self.q_project()
        self.decode()


class LayerCase(GpuCase):
    """A GpuCase whose queries come from the full layer's compressed query path
    and whose output goes through W^O."""

    def __init__(self, x: dict, num_splits: int = 0):
        import torch
        from mla_rank_latent_amd import mla
        super().__init__(x, num_splits)
        spec = self.spec
        B, S = spec.batch, spec.sq
        self.w_dq, self.w_uq = dev(x["w_dq"], spec.dtype), dev(x["w_uq"], spec.dtype)
        self.w_qr_c, self.w_o = dev(x["w_qr_c"], spec.dtype), dev(x["w_o"], spec.dtype)
        self.q_positions = dev(x["q_positions"], spec.dtype)
        self.h_q = self.h[:, -S:].contiguous()
        self.u = torch.empty(B, S, spec.d_model, dtype=torch.bfloat16, device="cuda")
        n = mla.mla_layer_workspace_bytes(self.d, spec.d_qlat, B, S)
        assert n > 0
        self.lws = torch.empty(n, dtype=torch.uint8, device="cuda")

    def layer_step(self):
        from mla_rank_latent_amd import mla
        self.append(self.split_append)
        mla.mla_q_compress(self.d, self.spec.d_qlat, self.h_q, self.w_dq, self.w_uq, self.w_qr_c, self.q_positions,
                           self.q_nope, self.q_rope, self.lws)
        self.decode()
        mla.mla_out_project(self.d, self.out, self.w_o, self.u, self.lws)


class PrefillCase:
    """Device copies of a generated workload whose sq query tokens are a prefill chunk."""

    def __init__(self, x: dict):
        import torch
        from mla_rank_latent_amd import mla
        self.x = x
        self.spec = spec = x["spec"]
        self.d = mla_dims(spec)
        self.pool = dev(x["pool"], spec.dtype)
        self.block_table = dev(x["block_table"], spec.dtype)
        self.seq_lens = dev(x["seq_lens"], spec.dtype)
        self.w_uk = dev(x["w_uk"], spec.dtype)
        self.w_uv = dev(x["w_uv"], spec.dtype)
        self.q_nope = dev(x["q_nope"], spec.dtype)
        self.q_rope = dev(x["q_rope"], spec.dtype)
        B, T, H = spec.batch, spec.sq, spec.n_heads
        self.out = torch.empty(B, T, H, spec.d_nope, dtype=torch.bfloat16, device="cuda")
        self.lse = torch.empty(B, T, H, dtype=torch.float32, device="cuda")
        self.status = torch.zeros(1, dtype=torch.int32, device="cuda")
        nbytes = mla.mla_prefill_workspace_bytes(self.d, B, int(x["block_table"].shape[1]))
        assert nbytes > 0
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

    def run(self):
        from mla_rank_latent_amd import mla
        mla.mla_prefill(self.d, self.q_nope, self.q_rope, self.w_uk, self.w_uv, self.pool, self.block_table,
                        self.seq_lens, self.x["scale"], self.ws, self.out, lse=self.lse, status=self.status)


# ---------------------------------------------------------------------------
# oracle side
# ---------------------------------------------------------------------------
def oracle_append_rows(x: dict) -> np.ndarray:
    spec = x["spec"]
    return mla_oracle.cache_rows(synth.as_float(x["h"], spec.dtype), synth.as_float(x["w_dkv"], spec.dtype),
                                 synth.as_float(x["w_kr"], spec.dtype), x["positions"], spec.rope_base, spec.dtype)


def oracle_decode(x: dict, batches=None, heads=None, appended_rows=None, q=None, heads_of=None):
    """Oracle output for the sampled sequences/heads.  ``appended_rows`` [B, T, R]
    are the oracle's own rows for the append positions (so the oracle never
    reads a value the GPU wrote); ``q`` overrides (q_nope, q_rope) as float64;
    ``heads_of(b)``, if given, names the heads evaluated for sequence b."""
    spec = x["spec"]
    B, bs = spec.batch, spec.block_size
    batches = list(range(B)) if batches is None else list(batches)
    if q is None:
        qn, qr = synth.as_float(x["q_nope"], spec.dtype), synth.as_float(x["q_rope"], spec.dtype)
    else:
        qn, qr = q
    w_uk, w_uv = synth.as_float(x["w_uk"], spec.dtype), synth.as_float(x["w_uv"], spec.dtype)
    out = np.full(qn.shape, np.nan)
    lse = np.full(qn.shape[:3], np.nan)
    for b in batches:
        L = int(x["seq_lens"][b])
        nblk = (L + bs - 1) // bs
        sub = pool_blocks(x, x["block_table"][b, :nblk])   # this sequence's blocks, in order
        if appended_rows is not None:
            for t, p in enumerate(x["positions"][b]):
                sub[p // bs, p % bs] = appended_rows[b, t]
        o, l = mla_oracle.decode(qn[b:b + 1], qr[b:b + 1], w_uk, w_uv, sub, np.arange(nblk)[None, :], [L],
                                 x["scale"], bs, heads=heads if heads_of is None else heads_of(b))
        out[b], lse[b] = o[0], l[0]
    return out, lse


def oracle_single_queries(x: dict, b: int, queries):
    """Oracle out [len(queries), H, d_h] and lse [len(queries), H] for chosen queries s of
    sequence b's group, every head: query s is a single query over the first
    L - Sq + s + 1 tokens (the causal rule of a query group)."""
    spec = x["spec"]
    bs = spec.block_size
    qn, qr = synth.as_float(x["q_nope"][b], spec.dtype), synth.as_float(x["q_rope"][b], spec.dtype)
    w_uk, w_uv = synth.as_float(x["w_uk"], spec.dtype), synth.as_float(x["w_uv"], spec.dtype)
    L = int(x["seq_lens"][b])
    nblk = (L + bs - 1) // bs
    sub = pool_blocks(x, x["block_table"][b, :nblk])
    outs, lses = [], []
    for s in queries:
        n = L - spec.sq + int(s) + 1
        o, l = mla_oracle.decode(qn[None, s:s + 1], qr[None, s:s + 1], w_uk, w_uv, sub, np.arange(nblk)[None, :],
                                 [n], x["scale"], bs)
        outs.append(o[0, 0])
        lses.append(l[0, 0])
    return np.stack(outs), np.stack(lses)


def oracle_query_samples(x: dict, samples):
    """Oracle out [d_h] and lse for sampled (b, s, h): query s of sequence b's group is a single
    query over the first L - Sq + s + 1 tokens (the causal rule of a query group)."""
    spec = x["spec"]
    bs = spec.block_size
    qn, qr = synth.as_float(x["q_nope"], spec.dtype), synth.as_float(x["q_rope"], spec.dtype)
    w_uk, w_uv = synth.as_float(x["w_uk"], spec.dtype), synth.as_float(x["w_uv"], spec.dtype)
    res = []
    for b, s, h in samples:
        n = int(x["seq_lens"][b]) - spec.sq + s + 1
        nblk = (n + bs - 1) // bs
        sub = pool_blocks(x, x["block_table"][b, :nblk])
        o, l = mla_oracle.decode(qn[b:b + 1, s:s + 1], qr[b:b + 1, s:s + 1], w_uk, w_uv, sub, np.arange(nblk)[None, :],
                                 [n], x["scale"], bs, heads=[h])
        res.append((o[0, 0, h], l[0, 0, h]))
    return res


def oracle_layer(x: dict, batches=None):
    """Oracle u [B, S, d] (rows not in ``batches`` NaN) for a layer workload: the
    appended rows as the cache stores them, the compressed-query path, decode and
    W^O, in fp64 with no other rounding."""
    spec = x["spec"]
    f = lambda k: synth.as_float(x[k], spec.dtype)
    rows = oracle_append_rows(x)
    h_q = f("h")[:, -spec.sq:]
    qn, qr = mla_oracle.layer_queries(h_q, f("w_dq"), f("w_uq"), f("w_qr_c"), x["q_positions"], spec.n_heads,
                                      spec.rope_base)
    out, _ = oracle_decode(x, batches=batches, appended_rows=rows, q=(qn, qr))
    return mla_oracle.out_project(np.nan_to_num(out, nan=0.0), f("w_o")), qn, qr


def rel_l2(a: np.ndarray, ref: np.ndarray) -> float:
    m = ~np.isnan(ref)
    return float(np.linalg.norm((a - ref)[m]) / max(np.linalg.norm(ref[m]), 1e-300))


def max_abs(a: np.ndarray, ref: np.ndarray) -> float:
    m = ~np.isnan(ref)
    return float(np.max(np.abs((a - ref)[m]))) if m.any() else 0.0


# spec tolerances: bf16 rel-L2 <= 1e-2 and max-abs <= 2e-2; fp32 rel-L2 <= 1e-4
def assert_close(gpu: np.ndarray, ref: np.ndarray, dtype: str, what: str = "") -> None:
    r = rel_l2(gpu, ref)
    a = max_abs(gpu, ref)
    log(f"  {what}: rel_l2={r:.3e} max_abs={a:.3e}")
    if dtype == "bf16":
        assert r <= 1e-2 and a <= 2e-2, (what, r, a)
    else:
        assert r <= 1e-4, (what, r, a)


def small_spec(name, batch, sq, lens, paged=True, append=False, seed=11, n_heads=128, d_model=5120):
    return synth.Spec(name, batch=batch, sq=sq, seq_lens=list(lens), paged=paged, append=append, seed=seed,
                      n_heads=n_heads, d_model=d_model)


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |x| (for 1-ulp comparisons)."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - 7)


def lse_probability_sum(x: dict, b: int, s: int, h: int, lse: float) -> float:
    """sum_j exp(z_j - lse) over the visible tokens, with z from the oracle's decompressed logits."""
    spec = x["spec"]
    bs = spec.block_size
    L = int(x["seq_lens"][b])
    rows = mla_oracle.gather_rows(synth.as_float(x["pool"], spec.dtype), x["block_table"][b], L, bs)
    dc, dn = spec.d_latent, spec.d_nope
    wk = synth.as_float(x["w_uk"], spec.dtype)[h * dn:(h + 1) * dn]
    k = np.concatenate([rows[:, :dc] @ wk.T, rows[:, dc:]], axis=1)
    q = np.concatenate([synth.as_float(x["q_nope"], spec.dtype)[b, s, h], synth.as_float(x["q_rope"], spec.dtype)[b, s, h]])
    n = L - spec.sq + s + 1
    z = x["scale"] * (k[:n] @ q)
    return float(np.sum(np.exp(z - lse)))
