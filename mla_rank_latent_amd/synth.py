"""Seeded synthetic inputs for MLA decode over a paged latent KV cache.

This module only draws random numbers and lays them out: it holds none of the
attention arithmetic. The HIP library and the fp64 oracle both consume the
arrays it returns (as data), and it imports neither of them.

Shapes follow DeepSeek-V2's MLA dimensions as given in "DeepSeek-V2:
Multi-Head Latent Attention (MLA) 原理与工程实现" §1.1 (n_h = d_h = 128) and
§3.3 (d_c = 512, d_h^R = 64).  Weights are stored out x in, as that page
writes W in R^{out x in} (§1.1, §2.1).

Value recipe (all draws from ``numpy.random.default_rng(seed)``, PCG64):
  * activations, queries and cache rows ~ N(0, 1) drawn as float32;
  * every weight matrix ~ N(0, 1/fan_in) (variance 1/in_features), drawn as
    a float32 standard normal and multiplied by 1/sqrt(fan_in) in float32;
  * bf16 workloads store every array as bf16, rounded to nearest-even from
    the float32 draw (bit arithmetic below); fp32 workloads keep float32.
Draw order inside one workload is fixed:
  1. ragged lengths (ragged workload only): integers(lo, hi, endpoint=True)
  2. block permutation (paged workloads): permutation(total_blocks)
  3. the cache pool: one standard_normal stream over the whole pool, in
     (block, row, column) order, drawn in chunks
  4. q_nope then q_rope (workloads that hand queries in directly)
  5. W_UK then W_UV
  6. append inputs: h_new, W_DKV, W_KR
  7. query-projection inputs: W_Q, W_QR (their hidden state is the appended h)
  8. full-layer inputs (layer workloads): W_DQ, W_UQ, W_QR, W_O; the queries'
     hidden state is the appended h
Cache rows that hold no token (past a sequence's end, or the slot the append
will fill) are set to a finite sentinel, so a kernel that reads them by
mistake produces visibly wrong numbers.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np

SENTINEL_BF16 = np.uint16(0x4B4B)          # ~1.33e7 as bf16
SENTINEL_F32 = np.uint32(0x4B4B4B4B)       # ~1.33e7 as float32
_CHUNK = 1 << 24                           # normals drawn per chunk


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 values (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Spec:
    """One decode workload.  ``seq_lens`` include the query tokens."""
    name: str
    batch: int
    sq: int                      # query tokens per sequence
    n_heads: int = 128
    d_nope: int = 128
    d_rope: int = 64
    d_latent: int = 512
    d_model: int = 5120
    block_size: int = 64
    dtype: str = "bf16"          # "bf16" or "f32"
    rope_base: float = 10000.0
    seed: int = 0
    seq_lens: Optional[List[int]] = None
    ragged: Optional[tuple] = None   # (lo, hi) inclusive: lengths drawn per sequence
    paged: bool = True               # False: identity block table (contiguous cache)
    append: bool = False             # append the last sq tokens from hidden states
    q_from_hidden: bool = False      # queries come from projecting the appended hidden states
    layer: bool = False              # the full layer: compressed queries from h, output projection W^O
    d_qlat: int = 1536               # d'_c, the query latent width (layer workloads)
    scale: Optional[float] = None    # default 1/sqrt(d_nope + d_rope)

    @property
    def row(self) -> int:
        return self.d_latent + self.d_rope

    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.d_nope + self.d_rope)


def presets() -> Dict[str, Spec]:
    """The five decode workloads: one tiny fp32 case and four DeepSeek-V2-shaped bf16 ones."""
    return {
        # tiny fp32: 64 cached tokens + 1 query token, everything projected from hidden states
        "tiny_f32_ctx65": Spec("tiny_f32_ctx65", batch=1, sq=1, n_heads=8, d_nope=16, d_rope=8, d_latent=32,
                               d_model=64, dtype="f32", seed=0, seq_lens=[65], paged=False, append=True,
                               q_from_hidden=True),
        "v2_b1_ctx4096": Spec("v2_b1_ctx4096", batch=1, sq=1, seed=1, seq_lens=[4096], paged=False),
        "v2_b64_ctx8192_paged_append": Spec("v2_b64_ctx8192_paged_append", batch=64, sq=1, seed=2,
                                            seq_lens=[8192] * 64, paged=True, append=True),
        "v2_b4_longctx_128k": Spec("v2_b4_longctx_128k", batch=4, sq=1, seed=3,
                                   seq_lens=[131072, 65536, 32768, 16384], paged=True),
        "v2_b128_ragged_sq2": Spec("v2_b128_ragged_sq2", batch=128, sq=2, seed=4, ragged=(512, 32768), paged=True),
    }


def _normals(rng: np.random.Generator, n: int, scale: float, dtype: str) -> np.ndarray:
    """n values ~ N(0, scale^2), stored as bf16 bits (uint16) or float32."""
    out = np.empty(n, dtype=np.uint16 if dtype == "bf16" else np.float32)
    s = np.float32(scale)
    for lo in range(0, n, _CHUNK):
        hi = min(n, lo + _CHUNK)
        x = rng.standard_normal(hi - lo, dtype=np.float32)
        if scale != 1.0:
            x *= s
        out[lo:hi] = f32_to_bf16_bits(x) if dtype == "bf16" else x
    return out


def _weight(rng, out_f: int, in_f: int, dtype: str) -> np.ndarray:
    return _normals(rng, out_f * in_f, 1.0 / math.sqrt(in_f), dtype).reshape(out_f, in_f)


def layer_presets() -> Dict[str, Spec]:
    """Full-layer decode workloads: the batch-64 context-8192 step with query compression and W^O."""
    return {
        "layer_b64_ctx8192": Spec("layer_b64_ctx8192", batch=64, sq=1, seed=7, seq_lens=[8192] * 64, paged=True,
                                  append=True, layer=True),
    }


def prefill_presets() -> Dict[str, Spec]:
    """Prefill workloads: every one of the sequence's tokens is appended from hidden states and is a query."""
    return {
        "prefill_b1_ctx8192": Spec("prefill_b1_ctx8192", batch=1, sq=8192, seed=6, seq_lens=[8192], paged=True,
                                   append=True),
    }


def make_inputs(spec: Spec) -> Dict[str, object]:
    """Draw every input of ``spec``.  bf16 arrays are uint16 bit patterns."""
    rng = np.random.default_rng(spec.seed)
    B, bs, R = spec.batch, spec.block_size, spec.row
    if spec.ragged is not None:
        lo, hi = spec.ragged
        seq_lens = rng.integers(lo, hi, size=B, endpoint=True).astype(np.int32)
    else:
        assert spec.seq_lens is not None and len(spec.seq_lens) == B
        seq_lens = np.asarray(spec.seq_lens, dtype=np.int32)
    if np.any(seq_lens < spec.sq):
        raise ValueError("every sequence must hold at least its query tokens")
    nblk = (seq_lens + bs - 1) // bs
    total = int(nblk.sum())
    max_blocks = int(nblk.max())
    phys = rng.permutation(total).astype(np.int32) if spec.paged else np.arange(total, dtype=np.int32)
    block_table = np.full((B, max_blocks), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        block_table[b, :nblk[b]] = phys[off:off + nblk[b]]
        off += int(nblk[b])

    pool = _normals(rng, total * bs * R, 1.0, spec.dtype).reshape(total, bs, R)
    sentinel = SENTINEL_BF16 if spec.dtype == "bf16" else SENTINEL_F32.view(np.float32)
    # rows past each sequence's end, and the slots the append will fill, hold the sentinel
    n_append = spec.sq if spec.append else 0
    if spec.q_from_hidden:
        n_append = int(seq_lens.max())      # tiny case: every token comes from hidden states
    for b in range(B):
        L = int(seq_lens[b])
        first_empty = L - n_append if not spec.q_from_hidden else 0
        for p in range(first_empty, nblk[b] * bs):
            pool[block_table[b, p // bs], p % bs, :] = sentinel

    out: Dict[str, object] = dict(spec=spec, seq_lens=seq_lens, block_table=block_table, pool=pool,
                                  num_blocks=total, max_blocks=max_blocks, scale=spec.softmax_scale())
    H, dn, dr, dc, d = spec.n_heads, spec.d_nope, spec.d_rope, spec.d_latent, spec.d_model
    if not spec.q_from_hidden:
        out["q_nope"] = _normals(rng, B * spec.sq * H * dn, 1.0, spec.dtype).reshape(B, spec.sq, H, dn)
        out["q_rope"] = _normals(rng, B * spec.sq * H * dr, 1.0, spec.dtype).reshape(B, spec.sq, H, dr)
    out["w_uk"] = _weight(rng, H * dn, dc, spec.dtype)
    out["w_uv"] = _weight(rng, H * dn, dc, spec.dtype)
    if spec.append or spec.q_from_hidden:
        T = int(seq_lens.max()) if spec.q_from_hidden else spec.sq
        if spec.q_from_hidden and np.any(seq_lens != seq_lens[0]):
            raise ValueError("hidden-state workloads need equal lengths")
        out["h"] = _normals(rng, B * T * d, 1.0, spec.dtype).reshape(B, T, d)
        out["w_dkv"] = _weight(rng, dc, d, spec.dtype)
        out["w_kr"] = _weight(rng, dr, d, spec.dtype)
        out["positions"] = (seq_lens[:, None] - T + np.arange(T, dtype=np.int32)[None, :]).astype(np.int32)
    if spec.q_from_hidden:
        out["w_q"] = _weight(rng, H * dn, d, spec.dtype)
        out["w_qr"] = _weight(rng, H * dr, d, spec.dtype)
        # the last sq appended tokens are the queries
        out["q_positions"] = out["positions"][:, -spec.sq:].copy()
    if spec.layer:
        if not spec.append:
            raise ValueError("layer workloads append the query tokens' hidden states")
        dq = spec.d_qlat
        out["w_dq"] = _weight(rng, dq, d, spec.dtype)
        out["w_uq"] = _weight(rng, H * dn, dq, spec.dtype)
        out["w_qr_c"] = _weight(rng, H * dr, dq, spec.dtype)
        out["w_o"] = _weight(rng, d, H * dn, spec.dtype)
        out["q_positions"] = out["positions"][:, -spec.sq:].copy()
    return out


def as_float(x: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values as float64 (bf16 bits are widened exactly)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)
