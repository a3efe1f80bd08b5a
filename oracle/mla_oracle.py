"""fp64 CPU oracle for Multi-head Latent Attention (MLA) decode over a latent KV cache.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The HIP library
never calls it, and the two share no code: no kernels, headers, helpers,
tables or constants.  Inputs reach both sides as plain arrays.

It computes the plain definition, slowly and visibly, in float64:
  * the cache row of a token is the joint latent c = W^DKV h followed by the
    decoupled key k^R = RoPE_pos(W^KR h), rounded once to the storage type;
  * every head's key and value are decompressed from the latent
    (k^C = W^UK_i c, v = W^UV_i c): no matrix absorption;
  * the rotary key k^R is concatenated to each head's key, the rotary query
    q^R to each head's query, and standard softmax attention runs per head.
Matrix absorption is written separately (``decode_absorbed``) only so that a
test can check the two agree.

Pages (title, section) that fix what is computed:
  [V2]  "DeepSeek-V2: Multi-Head Latent Attention (MLA) 原理与工程实现"
        §1.1 (MHA and its per-token cache), §1.2 (MQA/GQA cache),
        §2.1 (joint low-rank compression, up-projections), §2.2 (absorption),
        §3.2 (decoupled RoPE: multi-head q^R, one shared k^R, concatenation),
        §3.3 (cache = d_c + d_h^R per token per layer).
  [QD]  "【深度学习】DeepSeek焦点架构-MLA：分析低秩联合压缩优化KV缓存、提升推理 ..."
        02 (2)-(5) (joint K/V compression, decoupled RoPE, per-head concat),
        04 (cache comparison).
  [R1]  "R1的 MLA是如何节约 KV cache的?" §2.2 (weight fusion identity).
  [KV]  "kv-cache 的优化学习" (the MHA demo: softmax(QK^T/sqrt(D))V per head).

Readings where the pages are silent (each listed in the design notes):
  * RoPE pairs are interleaved, (x_{2i}, x_{2i+1}) rotated by pos*theta_i with
    theta_i = base^(-2i/d); positions are 0-based.
  * k^R is cached after rotation; q^R handed to decode is already rotated.
  * query s of a group of Sq attends cached tokens 0 .. L-Sq+s (itself included).
  * cache rows are rounded to the storage type (bf16: nearest-even).
  * a query that sees no token returns zeros and lse = -inf.
  * the low-precision latent cache (the pages name quantisation only as a risk,
    [V2] §5.1 item 3, and fix no format): c^KV is stored as FP8 E4M3 codes
    (4 exponent bits, bias 7, 3 mantissa bits, no infinities, 0x7F/0xFF NaN,
    largest finite 448) with one power-of-two scale per token (the OCP
    microscaling convention), s = 2^k for the smallest k >= -124 with
    amax|c| <= 448 s (s = 1 for an all-zero row), code =
    round-to-nearest-even(c / s), which is exact division; k^R stays bf16.
    The row quantised is the bf16 row a bf16 cache would hold.  A 64-token
    page stores the 64 latent code rows, then the 64 bf16 rotary rows, then
    the 64 scales as fp32.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "round_to_storage", "rope", "cache_rows", "write_rows", "q_project", "gather_rows",
    "q_compress", "layer_queries", "out_project",
    "decode", "decode_absorbed", "latent_elements_per_token", "mha_elements_per_token",
    "mqa_elements_per_token", "gqa_elements_per_token",
    "e4m3_values", "round_e4m3", "fp8_scale_exponent", "quantize_rows", "dequantize_rows", "fp8_page_bytes",
    "pack_fp8_pages", "unpack_fp8_pages", "dequantize_pages",
]


# ---------------------------------------------------------------------------
# storage rounding (part of what a bf16 / fp32 cache *is*)
# ---------------------------------------------------------------------------
def _round_significand(x: np.ndarray, sig_bits: int, min_exp: int, max_exp: int) -> np.ndarray:
    """Round float64 values to a binary format with ``sig_bits`` significant bits
    (implicit bit included), round-to-nearest-even, gradual underflow below
    2^min_exp, overflow to +-inf above the largest finite value."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                        # x = m * 2^e, 0.5 <= |m| < 1
    q = np.maximum(e - sig_bits, min_exp - sig_bits + 1).astype(np.float64)
    quantum = np.ldexp(1.0, q.astype(np.int64))
    r = np.rint(x / quantum) * quantum        # rint: ties to even
    largest = (2.0 - 2.0 ** (1 - sig_bits)) * 2.0 ** max_exp
    return np.where(np.abs(r) > largest, np.copysign(np.inf, x), r)


def round_to_storage(x: np.ndarray, storage: str) -> np.ndarray:
    """Values of ``x`` after storing them as ``storage`` ('bf16', 'f32' or 'f64')."""
    if storage == "bf16":
        return _round_significand(x, 8, -126, 127)
    if storage == "f32":
        return _round_significand(x, 24, -126, 127)
    if storage == "f64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(storage)


# ---------------------------------------------------------------------------
# decoupled RoPE  ([V2] §3.2; RoPE itself is RoFormer's rotation)
# ---------------------------------------------------------------------------
def rope(x: np.ndarray, pos, base: float) -> np.ndarray:
    """Rotate consecutive pairs (x_{2i}, x_{2i+1}) by angle pos * base^(-2i/d).

    ``x`` has the rotary dimension last; ``pos`` broadcasts against x[..., 0]."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    i = np.arange(d // 2, dtype=np.float64)
    theta = np.power(float(base), -2.0 * i / d)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * theta
    c, s = np.cos(ang), np.sin(ang)
    even, odd = x[..., 0::2], x[..., 1::2]
    out = np.empty(np.broadcast_shapes(x.shape, ang.shape[:-1] + (d,)), dtype=np.float64)
    out[..., 0::2] = even * c - odd * s
    out[..., 1::2] = even * s + odd * c
    return out


# ---------------------------------------------------------------------------
# append: what one token leaves in the cache  ([V2] §2.1, §3.2, §3.3; [QD] 02 (2), 04 (2))
# ---------------------------------------------------------------------------
def cache_rows(h, w_dkv, w_kr, positions, rope_base: float, storage: str) -> np.ndarray:
    """Cache rows [c^KV ‖ k^R] for hidden states ``h`` [B, T, d].

    c^KV = W^DKV h (W^DKV is d_c x d); k^R = RoPE_pos(W^KR h) (W^KR is d_R x d);
    the concatenation is rounded once to ``storage``."""
    h = np.asarray(h, dtype=np.float64)
    c = h @ np.asarray(w_dkv, dtype=np.float64).T
    kr = rope(h @ np.asarray(w_kr, dtype=np.float64).T, positions, rope_base)
    return round_to_storage(np.concatenate([c, kr], axis=-1), storage)


def write_rows(pool: np.ndarray, block_table, positions, rows, block_size: int) -> None:
    """Paged write: the row of sequence b at position p goes to
    pool[block_table[b, p // block_size], p % block_size]."""
    positions = np.asarray(positions)
    for b in range(positions.shape[0]):
        for t in range(positions.shape[1]):
            p = int(positions[b, t])
            pool[int(block_table[b, p // block_size]), p % block_size, :] = rows[b, t]


def gather_rows(pool, block_table, seq_len: int, block_size: int) -> np.ndarray:
    """The L cached rows of one sequence, in logical order, as float64 [L, R]."""
    j = np.arange(seq_len)
    return np.asarray(pool[np.asarray(block_table)[j // block_size], j % block_size], dtype=np.float64)


# ---------------------------------------------------------------------------
# query path  ([V2] §1.1 W^Q applied to h, §3.2 q^R = RoPE(W^QR h) per head)
# ---------------------------------------------------------------------------
def q_project(h, w_q, w_qr, positions, n_heads: int, rope_base: float):
    """q^C_i = W^Q_i h and q^R_i = RoPE_pos(W^QR_i h) for each head i.

    ``h`` [B, S, d]; returns float64 q_nope [B, S, H, d_nope], q_rope [B, S, H, d_R]."""
    h = np.asarray(h, dtype=np.float64)
    B, S, _ = h.shape
    qn = (h @ np.asarray(w_q, dtype=np.float64).T).reshape(B, S, n_heads, -1)
    qr = (h @ np.asarray(w_qr, dtype=np.float64).T).reshape(B, S, n_heads, -1)
    return qn, rope(qr, np.asarray(positions)[..., None], rope_base)


# ---------------------------------------------------------------------------
# the full layer's query compression and output projection
# ([V2] §2.3 and [QD] 02 (3): the query is compressed to c^Q = W^DQ h; [QD]
# 02 (5): up-projections of c^Q give each head's q^C and its rotary q^R, and
# the heads' outputs, concatenated, pass through one linear map W^O)
# ---------------------------------------------------------------------------
def q_compress(h, w_dq):
    """c^Q = W^DQ h.  ``h`` [B, S, d], ``w_dq`` [d'_c, d]; returns float64 [B, S, d'_c]."""
    return np.asarray(h, dtype=np.float64) @ np.asarray(w_dq, dtype=np.float64).T


def layer_queries(h, w_dq, w_uq, w_qr, positions, n_heads: int, rope_base: float):
    """q^C_i = W^UQ_i c^Q and q^R_i = RoPE_pos(W^QR_i c^Q) with c^Q = W^DQ h: the
    query projection of q_project applied to the compressed query."""
    return q_project(q_compress(h, w_dq), w_uq, w_qr, positions, n_heads, rope_base)


def out_project(o, w_o):
    """u = W^O [o_1; ...; o_{n_h}].  ``o`` [B, S, H, d_h], ``w_o`` [d, H*d_h]; returns [B, S, d]."""
    o = np.asarray(o, dtype=np.float64)
    B, S = o.shape[:2]
    return o.reshape(B, S, -1) @ np.asarray(w_o, dtype=np.float64).T


# ---------------------------------------------------------------------------
# decode, non-absorbed: the oracle proper
# ---------------------------------------------------------------------------
def _softmax_attend(z: np.ndarray, v: np.ndarray):
    """Stable softmax over the last axis of the logits z [n], then weights @ v [n, d]."""
    m = z.max()
    e = np.exp(z - m)
    den = e.sum()
    return (e / den) @ v, m + math.log(den)


def decode(q_nope, q_rope, w_uk, w_uv, pool, block_table, seq_lens, scale: float,
           block_size: int, heads=None, batches=None):
    """MLA decode by decompression.

    For sequence b with L cached tokens (the Sq query tokens included) and head i:
      K^C_j = W^UK_i c_j, V_j = W^UV_i c_j, with W^UK_i, W^UV_i the rows
      i*d_h .. (i+1)*d_h - 1 of W^UK, W^UV  ([V2] §2.1);
      k_j = [K^C_j ; k^R_j], q_s = [q^C_s ; q^R_s]  ([V2] §3.2);
      z_j = scale * q_s . k_j for j <= L - Sq + s; o = softmax(z) V ([KV] demo_mha).
    Returns float64 out [B, Sq, H, d_h] and lse [B, Sq, H] (natural log of the
    sum of exp(z)); rows not in ``heads`` / ``batches`` are left NaN."""
    q_nope = np.asarray(q_nope, dtype=np.float64)
    q_rope = np.asarray(q_rope, dtype=np.float64)
    w_uk = np.asarray(w_uk, dtype=np.float64)
    w_uv = np.asarray(w_uv, dtype=np.float64)
    B, Sq, H, dn = q_nope.shape
    dc = w_uk.shape[1]
    out = np.full((B, Sq, H, dn), np.nan)
    lse = np.full((B, Sq, H), np.nan)
    for b in (range(B) if batches is None else batches):
        L = int(seq_lens[b])
        rows = gather_rows(pool, block_table[b], L, block_size) if L > 0 else np.zeros((0, w_uk.shape[1] + q_rope.shape[-1]))
        c, kr = rows[:, :dc], rows[:, dc:]
        for i in (range(H) if heads is None else heads):
            wk = w_uk[i * dn:(i + 1) * dn]            # d_h x d_c
            wv = w_uv[i * dn:(i + 1) * dn]
            k = np.concatenate([c @ wk.T, kr], axis=1)  # L x (d_h + d_R)
            v = c @ wv.T                                # L x d_h
            for s in range(Sq):
                n = L - Sq + s + 1
                if n <= 0:
                    out[b, s, i], lse[b, s, i] = 0.0, -np.inf
                    continue
                q = np.concatenate([q_nope[b, s, i], q_rope[b, s, i]])
                out[b, s, i], lse[b, s, i] = _softmax_attend(scale * (k[:n] @ q), v[:n])
    return out, lse


def decode_absorbed(q_nope, q_rope, w_uk, w_uv, pool, block_table, seq_lens, scale: float,
                    block_size: int, heads=None, batches=None):
    """The same decode with W^UK absorbed into the query and W^UV applied after the
    weighted sum ([V2] §2.2; [R1] §2.2): q~ = W^UK_i^T q^C,
    z_j = scale * (q~ . c_j + q^R . k^R_j), o = W^UV_i (sum_j p_j c_j).
    Exists only so a test can check that absorption is exact."""
    q_nope = np.asarray(q_nope, dtype=np.float64)
    q_rope = np.asarray(q_rope, dtype=np.float64)
    w_uk = np.asarray(w_uk, dtype=np.float64)
    w_uv = np.asarray(w_uv, dtype=np.float64)
    B, Sq, H, dn = q_nope.shape
    dc = w_uk.shape[1]
    out = np.full((B, Sq, H, dn), np.nan)
    lse = np.full((B, Sq, H), np.nan)
    for b in (range(B) if batches is None else batches):
        L = int(seq_lens[b])
        rows = gather_rows(pool, block_table[b], L, block_size)
        c, kr = rows[:, :dc], rows[:, dc:]
        for i in (range(H) if heads is None else heads):
            wk = w_uk[i * dn:(i + 1) * dn]
            wv = w_uv[i * dn:(i + 1) * dn]
            for s in range(Sq):
                n = L - Sq + s + 1
                if n <= 0:
                    out[b, s, i], lse[b, s, i] = 0.0, -np.inf
                    continue
                q_lat = wk.T @ q_nope[b, s, i]                  # d_c
                z = scale * (c[:n] @ q_lat + kr[:n] @ q_rope[b, s, i])
                o_lat, lse[b, s, i] = _softmax_attend(z, c[:n])  # latent weighted sum
                out[b, s, i] = wv @ o_lat
    return out, lse


# ---------------------------------------------------------------------------
# cache accounting, elements per token per layer
# ---------------------------------------------------------------------------
def latent_elements_per_token(d_latent: int, d_rope: int) -> int:
    """MLA caches c^KV and k^R: d_c + d_h^R elements ([V2] §3.3; [QD] 04 (2))."""
    return d_latent + d_rope


def mha_elements_per_token(n_heads: int, d_head: int) -> int:
    """MHA caches every head's key and value: 2 n_h d_h elements ([V2] §1.1; [QD] 04 (1))."""
    return 2 * n_heads * d_head


def mqa_elements_per_token(d_head: int) -> int:
    """One shared key/value head: 2 d_h elements ([V2] §1.2)."""
    return 2 * d_head


def gqa_elements_per_token(n_groups: int, d_head: int) -> int:
    """n_g shared key/value heads: 2 n_g d_h elements ([V2] §1.2)."""
    return 2 * n_groups * d_head


# ---------------------------------------------------------------------------
# FP8 latent cache (a reading: the pages fix no low-precision format; [V2] §5.1
# item 3 names quantisation error as the risk).  Everything here is the format's
# definition written out; decode over such a cache is ``decode`` applied to the
# dequantised rows.
# ---------------------------------------------------------------------------
E4M3_MAX = 448.0


def e4m3_values() -> np.ndarray:
    """The value of each of the 256 E4M3 codes, from the format's fields: sign
    bit, 4-bit exponent e (bias 7), 3-bit mantissa m; e = 0 is subnormal
    (m/8 * 2^-6), e = 15 with m = 7 is NaN (no infinities)."""
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e, m = (code >> 3) & 0xF, code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = sign * (m / 8.0) * 2.0 ** -6
        else:
            vals[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


def round_e4m3(y) -> np.ndarray:
    """E4M3 code of the value nearest to each finite y with |y| <= 448, ties to the
    code with an even mantissa; the sign bit is y's (so -0.0 and negative values
    that round to zero give 0x80)."""
    y = np.asarray(y, dtype=np.float64)
    if np.any(~np.isfinite(y)) or np.any(np.abs(y) > E4M3_MAX):
        raise ValueError("round_e4m3 takes finite values of magnitude <= 448")
    mags = e4m3_values()[:0x7F]                      # codes 0x00 .. 0x7E, increasing
    a = np.abs(y)
    hi = np.clip(np.searchsorted(mags, a, side="left"), 0, 0x7E)   # first magnitude >= a
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - mags[lo], mags[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    mag_code = np.where(pick_hi, hi, lo)
    return (mag_code | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)


def fp8_scale_exponent(amax) -> np.ndarray:
    """k of the per-token scale s = 2^k: the smallest integer k >= -124 with
    amax <= 448 * 2^k (0 where amax == 0).  amax = m 2^e (frexp, 1/2 <= m < 1)
    gives amax 2^-(e-9) = 512 m in [256, 512), so k is e - 9 or e - 8."""
    amax = np.asarray(amax, dtype=np.float64)
    m, e = np.frexp(amax)
    k = np.where(512.0 * m <= E4M3_MAX, e - 9, e - 8)
    k = np.maximum(k, -124)
    return np.where(amax > 0, k, 0).astype(np.int64)


def quantize_rows(rows, d_latent: int):
    """Quantise cache rows [..., d_latent + d_rope] (values a bf16 cache holds).

    Returns (codes uint8 [..., d_latent], scales float32 [...], rope float64
    [..., d_rope]): s = 2^k with k from fp8_scale_exponent(amax) over the row's
    latent part, code = round_e4m3(c / s) (c / s is exact and |c / s| <= 448)."""
    rows = np.asarray(rows, dtype=np.float64)
    lat = rows[..., :d_latent]
    k = fp8_scale_exponent(np.max(np.abs(lat), axis=-1))
    y = np.ldexp(lat, -k[..., None])
    return round_e4m3(y), np.ldexp(1.0, k).astype(np.float32), rows[..., d_latent:].copy()


def dequantize_rows(codes, scales, rope) -> np.ndarray:
    """Rows [s * value(code) ‖ k^R] in float64 (the products are exact)."""
    lat = e4m3_values()[np.asarray(codes, dtype=np.int64)] * np.asarray(scales, dtype=np.float64)[..., None]
    return np.concatenate([lat, np.asarray(rope, dtype=np.float64)], axis=-1)


def fp8_page_bytes(block_size: int, d_latent: int, d_rope: int) -> int:
    """Bytes of one page: block_size x (d_latent code bytes + 2 d_rope bf16 bytes + 4 scale bytes)."""
    return block_size * (d_latent + 2 * d_rope + 4)


def pack_fp8_pages(codes, rope_bf16_bits, scales) -> np.ndarray:
    """Pages uint8 [num_blocks, page bytes] from codes [nb, bs, d_c] (uint8),
    rotary rows [nb, bs, d_R] (bf16 bit patterns, uint16) and scales [nb, bs]
    (float32): the code rows, then the rotary rows, then the scales, each
    block_size rows long, little-endian."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    rope_b = np.ascontiguousarray(rope_bf16_bits, dtype="<u2")
    sc = np.ascontiguousarray(scales, dtype="<f4")
    nb = codes.shape[0]
    return np.concatenate([codes.reshape(nb, -1), rope_b.view(np.uint8).reshape(nb, -1),
                           sc.view(np.uint8).reshape(nb, -1)], axis=1)


def unpack_fp8_pages(pages, block_size: int, d_latent: int, d_rope: int):
    """Inverse of pack_fp8_pages: (codes, rope bf16 bit patterns, scales)."""
    pages = np.ascontiguousarray(pages, dtype=np.uint8)
    nb = pages.shape[0]
    a = block_size * d_latent
    b = a + block_size * d_rope * 2
    codes = pages[:, :a].reshape(nb, block_size, d_latent)
    rope_bits = pages[:, a:b].copy().view("<u2").reshape(nb, block_size, d_rope)
    scales = pages[:, b:b + 4 * block_size].copy().view("<f4").reshape(nb, block_size)
    return codes, rope_bits, scales


def dequantize_pages(pages, block_size: int, d_latent: int, d_rope: int) -> np.ndarray:
    """The float64 pool [nb, block_size, d_latent + d_rope] an FP8 page pool stands for."""
    codes, rope_bits, scales = unpack_fp8_pages(pages, block_size, d_latent, d_rope)
    rope = (rope_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return dequantize_rows(codes, scales, rope)
