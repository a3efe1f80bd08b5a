"""Pins for the fp64 oracle: checks against what the pages and plain mathematics fix.

Each ``pin_*`` function takes the oracle module (so a test can hand in a copy
with a planted mistake) and returns the worst error it saw; the pin passes when
that error is below ``PIN_TOL``.  None of these re-types the oracle's own
formula: each compares with a textbook special case written as explicit
loops, a closed form, an invariant, exact rational arithmetic, or a library
routine.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

PIN_TOL = 1e-10


def _rng(seed):
    return np.random.default_rng(1000 + seed)


def _paged_case(rng, B, H, dn, dr, dc, lens, bs, Sq):
    """Random fp64 decode inputs with a permuted block table."""
    nblk = [(L + bs - 1) // bs for L in lens]
    total = sum(nblk)
    perm = rng.permutation(total)
    bt = np.full((B, max(nblk)), -1, dtype=np.int64)
    o = 0
    for b in range(B):
        bt[b, :nblk[b]] = perm[o:o + nblk[b]]
        o += nblk[b]
    pool = rng.standard_normal((total, bs, dc + dr))
    qn = rng.standard_normal((B, Sq, H, dn))
    qr = rng.standard_normal((B, Sq, H, dr))
    wuk = rng.standard_normal((H * dn, dc)) / math.sqrt(dc)
    wuv = rng.standard_normal((H * dn, dc)) / math.sqrt(dc)
    return qn, qr, wuk, wuv, pool, bt


# ---------------------------------------------------------------- storage
def pin_bf16_rounding(orc) -> float:
    """bf16 rounding equals torch's float32 -> bfloat16 cast (nearest-even) on
    float32-exact inputs, plus hand-worked ties."""
    import torch
    rng = _rng(1)
    x32 = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    lib = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    err = float(np.max(np.abs(orc.round_to_storage(x32.astype(np.float64), "bf16") - lib) / np.maximum(np.abs(lib), 1e-300)))
    # ties: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> even (1);
    #       1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6 -> even (1 + 2^-6)
    ties = orc.round_to_storage(np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8)]), "bf16")
    want = np.array([1.0, 1 + 2.0 ** -6, -1.0])
    return max(err, float(np.max(np.abs(ties - want))))


def pin_f32_rounding(orc) -> float:
    """fp32 rounding equals numpy's float64 -> float32 cast, subnormals and overflow included."""
    rng = _rng(2)
    x = rng.standard_normal(20000) * np.exp(rng.uniform(-110, 90, 20000))
    x = np.concatenate([x, [3.5e38, -3.5e38, 1e-45, 7e-46, 0.0]])
    with np.errstate(over="ignore"):
        lib = x.astype(np.float32).astype(np.float64)
    mine = orc.round_to_storage(x, "f32")
    same = (mine == lib) | (np.isinf(mine) & np.isinf(lib) & (np.sign(mine) == np.sign(lib)))
    return 0.0 if bool(np.all(same)) else 1.0


# ---------------------------------------------------------------- RoPE
def pin_rope_rotation(orc) -> float:
    """RoPE as RoFormer's complex form: pair (x_{2i}, x_{2i+1}) read as the complex
    number x_{2i} + i x_{2i+1}, multiplied by exp(i p base^(-2i/d)).  Also: norm
    kept, identity at p = 0, and the score depends only on m - n."""
    rng = _rng(3)
    d, base = 8, 10000.0
    x = rng.standard_normal((5, d))
    pos = np.array([0, 1, 17, 4095, 8191])
    got = orc.rope(x, pos, base)
    err = 0.0
    for r in range(5):
        for i in range(d // 2):
            z = complex(x[r, 2 * i], x[r, 2 * i + 1]) * complex(math.cos(pos[r] * base ** (-2 * i / d)),
                                                                  math.sin(pos[r] * base ** (-2 * i / d)))
            err = max(err, abs(got[r, 2 * i] - z.real), abs(got[r, 2 * i + 1] - z.imag))
    err = max(err, float(np.max(np.abs(np.linalg.norm(got, axis=1) - np.linalg.norm(x, axis=1)))))
    err = max(err, float(np.max(np.abs(got[0] - x[0]))))
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    for m, n in [(5, 2), (103, 100), (9000, 8997)]:
        a = orc.rope(q, np.array(m), base) @ orc.rope(k, np.array(n), base)
        b = orc.rope(q, np.array(m - n), base) @ k
        err = max(err, abs(a - b))
    return err


# ---------------------------------------------------------------- absorption
def pin_absorption(orc) -> float:
    """Decompress-then-attend equals the absorbed latent-space form (associativity)."""
    rng = _rng(4)
    B, H, dn, dr, dc, bs, Sq = 2, 4, 8, 4, 16, 16, 2
    lens = [37, 16]
    qn, qr, wuk, wuv, pool, bt = _paged_case(rng, B, H, dn, dr, dc, lens, bs, Sq)
    o1, l1 = orc.decode(qn, qr, wuk, wuv, pool, bt, lens, 0.3, bs)
    o2, l2 = orc.decode_absorbed(qn, qr, wuk, wuv, pool, bt, lens, 0.3, bs)
    return float(max(np.max(np.abs(o1 - o2)) / np.max(np.abs(o1)), np.max(np.abs(l1 - l2))))


# ---------------------------------------------------------------- textbook MHA
def _mha_loops(x, wq, wk, wv, H, D):
    """softmax(q k^T / sqrt(D)) v per head for the last position, as explicit loops."""
    L, d = x.shape
    def proj(w, t, row):
        return sum(w[row][c] * x[t][c] for c in range(d))
    out = [[0.0] * D for _ in range(H)]
    for hh in range(H):
        q = [proj(wq, L - 1, hh * D + e) for e in range(D)]
        z = []
        for t in range(L):
            k = [proj(wk, t, hh * D + e) for e in range(D)]
            z.append(sum(q[e] * k[e] for e in range(D)) / math.sqrt(D))
        mx = max(z)
        w = [math.exp(zz - mx) for zz in z]
        s = sum(w)
        for t in range(L):
            v = [proj(wv, t, hh * D + e) for e in range(D)]
            for e in range(D):
                out[hh][e] += w[t] / s * v[e]
    return np.array(out)


def pin_mha_special_case(orc) -> float:
    """With d_c = 2 n_h d_h, W^DKV = [W_K; W_V], W^UK = [I 0], W^UV = [0 I] and zero
    rotary weights, the whole MLA path (append, query projection, decode) is
    plain MHA, checked against explicit loops."""
    rng = _rng(5)
    H, D, d, L, dr, bs = 2, 4, 6, 5, 2, 4
    x = rng.standard_normal((L, d))
    wq, wk, wv = (rng.standard_normal((H * D, d)) for _ in range(3))
    dc = 2 * H * D
    w_dkv = np.concatenate([wk, wv], axis=0)
    eye = np.eye(H * D)
    w_uk = np.concatenate([eye, np.zeros((H * D, H * D))], axis=1)
    w_uv = np.concatenate([np.zeros((H * D, H * D)), eye], axis=1)
    w_kr = np.zeros((dr, d))
    w_qr = np.zeros((H * dr, d))
    pos = np.arange(L)[None, :]
    rows = orc.cache_rows(x[None], w_dkv, w_kr, pos, 10000.0, "f64")
    nblk = (L + bs - 1) // bs
    pool = np.full((nblk, bs, dc + dr), 7.0)
    bt = np.arange(nblk)[None, :]
    orc.write_rows(pool, bt, pos, rows, bs)
    qn, qr = orc.q_project(x[None, L - 1:L], wq, w_qr, pos[:, L - 1:], H, 10000.0)
    out, _ = orc.decode(qn, qr, w_uk, w_uv, pool, bt, [L], 1.0 / math.sqrt(D), bs)
    ref = _mha_loops(x, wq, wk, wv, H, D)
    return float(np.max(np.abs(out[0, 0] - ref)))


# ---------------------------------------------------------------- MQA on the rotary key
def pin_mqa_special_case(orc) -> float:
    """With q^C = 0 and one W^UV shared by every head, every head attends the one
    shared key k^R with one shared value: MQA, checked against explicit loops."""
    rng = _rng(6)
    H, dn, dr, dc, bs, L = 3, 4, 4, 6, 8, 11
    qn, qr, wuk, _, pool, bt = _paged_case(rng, 1, H, dn, dr, dc, [L], bs, 1)
    qn[:] = 0.0
    w1 = rng.standard_normal((dn, dc))
    wuv = np.concatenate([w1] * H, axis=0)
    scale = 0.7
    out, _ = orc.decode(qn, qr, wuk, wuv, pool, bt, [L], scale, bs)
    err = 0.0
    rows = [pool[bt[0, t // bs], t % bs] for t in range(L)]
    for hh in range(H):
        z = [scale * sum(qr[0, 0, hh, e] * rows[t][dc + e] for e in range(dr)) for t in range(L)]
        mx = max(z)
        w = [math.exp(v - mx) for v in z]
        s = sum(w)
        for e in range(dn):
            ref = sum(w[t] / s * sum(w1[e][c] * rows[t][c] for c in range(dc)) for t in range(L))
            err = max(err, abs(out[0, 0, hh, e] - ref))
    return err


# ---------------------------------------------------------------- closed forms / invariants
def pin_softmax_normalised(orc) -> float:
    """If every cached latent has c_0 = 1 and row 0 of each W^UV_i is e_0, output
    element 0 is the sum of the attention weights: exactly 1."""
    rng = _rng(7)
    H, dn, dr, dc, bs = 3, 4, 2, 8, 8
    lens = [1, 9, 30]
    qn, qr, wuk, wuv, pool, bt = _paged_case(rng, 3, H, dn, dr, dc, lens, bs, 1)
    qn *= 5.0
    pool[:, :, 0] = 1.0
    for hh in range(H):
        wuv[hh * dn] = 0.0
        wuv[hh * dn, 0] = 1.0
    out, _ = orc.decode(qn, qr, wuk, wuv, pool, bt, lens, 0.5, bs)
    return float(np.max(np.abs(out[:, :, :, 0] - 1.0)))


def pin_closed_forms(orc) -> float:
    """One visible token: o = W^UV_i c_0.  Zero query: o = mean_j W^UV_i c_j and
    lse = ln(n).  With Sq = 2 and L = 2 the first query sees only token 0."""
    rng = _rng(8)
    H, dn, dr, dc, bs = 2, 4, 2, 6, 4
    err = 0.0
    qn, qr, wuk, wuv, pool, bt = _paged_case(rng, 1, H, dn, dr, dc, [1], bs, 1)
    out, lse = orc.decode(qn, qr, wuk, wuv, pool, bt, [1], 0.9, bs)
    c0 = pool[bt[0, 0], 0, :dc]
    for hh in range(H):
        err = max(err, float(np.max(np.abs(out[0, 0, hh] - wuv[hh * dn:(hh + 1) * dn] @ c0))))
    L = 13
    qn, qr, wuk, wuv, pool, bt = _paged_case(rng, 1, H, dn, dr, dc, [L], bs, 1)
    qn[:] = 0.0
    qr[:] = 0.0
    out, lse = orc.decode(qn, qr, wuk, wuv, pool, bt, [L], 0.9, bs)
    cs = np.array([pool[bt[0, t // bs], t % bs, :dc] for t in range(L)])
    for hh in range(H):
        err = max(err, float(np.max(np.abs(out[0, 0, hh] - wuv[hh * dn:(hh + 1) * dn] @ cs.mean(0)))))
        err = max(err, abs(lse[0, 0, hh] - math.log(L)))
    qn, qr, wuk, wuv, pool, bt = _paged_case(rng, 1, H, dn, dr, dc, [2], bs, 2)
    out, _ = orc.decode(qn, qr, wuk, wuv, pool, bt, [2], 0.9, bs)
    c0 = pool[bt[0, 0], 0, :dc]
    for hh in range(H):
        err = max(err, float(np.max(np.abs(out[0, 0, hh] - wuv[hh * dn:(hh + 1) * dn] @ c0))))
    return err


def pin_causal_group(orc) -> float:
    """Query s of an Sq-group over L tokens equals a single query over the first
    L - Sq + s + 1 tokens."""
    rng = _rng(9)
    H, dn, dr, dc, bs, L, Sq = 2, 4, 2, 6, 4, 10, 3
    qn, qr, wuk, wuv, pool, bt = _paged_case(rng, 1, H, dn, dr, dc, [L], bs, Sq)
    out, lse = orc.decode(qn, qr, wuk, wuv, pool, bt, [L], 0.8, bs)
    err = 0.0
    for s in range(Sq):
        o1, l1 = orc.decode(qn[:, s:s + 1], qr[:, s:s + 1], wuk, wuv, pool, bt, [L - Sq + s + 1], 0.8, bs)
        err = max(err, float(np.max(np.abs(out[:, s] - o1[:, 0]))), float(np.max(np.abs(lse[:, s] - l1[:, 0]))))
    return err


def pin_paging(orc) -> float:
    """A permuted block table over a permuted pool gives the same result as the
    identity table over the contiguous pool."""
    rng = _rng(10)
    H, dn, dr, dc, bs = 2, 4, 2, 6, 4
    lens = [9, 14]
    qn, qr, wuk, wuv, pool, bt = _paged_case(rng, 2, H, dn, dr, dc, lens, bs, 1)
    o1, _ = orc.decode(qn, qr, wuk, wuv, pool, bt, lens, 0.8, bs)
    contiguous = np.zeros((2, 4, bs, dc + dr))
    for b in range(2):
        for i in range((lens[b] + bs - 1) // bs):
            contiguous[b, i] = pool[bt[b, i]]
    bt2 = np.arange(8).reshape(2, 4)
    o2, _ = orc.decode(qn, qr, wuk, wuv, contiguous.reshape(8, bs, dc + dr), bt2, lens, 0.8, bs)
    return float(np.max(np.abs(o1 - o2)))


# ---------------------------------------------------------------- append
def pin_append_exact(orc) -> float:
    """On dyadic inputs the latent row c = W^DKV h is exact rational arithmetic;
    the rotary part at position 0 is the unrotated W^KR h; rows land in the slot
    the block table names and nowhere else."""
    rng = _rng(11)
    d, dc, dr, bs = 12, 6, 4, 4
    h = rng.integers(-2, 3, size=(2, 3, d)).astype(np.float64)
    w_dkv = rng.integers(-64, 65, size=(dc, d)) / 64.0
    w_kr = rng.integers(-64, 65, size=(dr, d)) / 64.0
    pos = np.array([[0, 5, 6], [0, 1, 9]])
    import torch
    rows = orc.cache_rows(h, w_dkv, w_kr, pos, 10000.0, "bf16")
    err = 0.0
    for b in range(2):
        for t in range(3):
            exact = [float(sum(Fraction(int(h[b, t, c])) * Fraction(int(round(w_dkv[r, c] * 64)), 64) for c in range(d)))
                     for r in range(dc)]
            # the exact sums fit float32; torch's cast rounds them to bf16 (nearest-even)
            lib = torch.tensor(exact, dtype=torch.float32).to(torch.bfloat16).double().numpy()
            err = max(err, float(np.max(np.abs(rows[b, t, :dc] - lib))))
            if pos[b, t] == 0:
                kr = [float(sum(Fraction(int(h[b, t, c])) * Fraction(int(round(w_kr[r, c] * 64)), 64) for c in range(d)))
                      for r in range(dr)]
                lib = torch.tensor(kr, dtype=torch.float32).to(torch.bfloat16).double().numpy()
                err = max(err, float(np.max(np.abs(rows[b, t, dc:] - lib))))
    pool = np.full((6, bs, dc + dr), -3.0)
    bt = np.array([[4, 1, 5], [0, 3, 2]])
    orc.write_rows(pool, bt, pos, rows, bs)
    expect = np.full_like(pool, -3.0)
    for b in range(2):
        for t in range(3):
            p = pos[b, t]
            expect[bt[b, p // bs], p % bs] = rows[b, t]
    err = max(err, float(np.max(np.abs(pool - expect))))
    return err


ALL_PINS = [
    pin_bf16_rounding, pin_f32_rounding, pin_rope_rotation, pin_absorption, pin_mha_special_case,
    pin_mqa_special_case, pin_softmax_normalised, pin_closed_forms, pin_causal_group, pin_paging,
    pin_append_exact,
]


def pin_query_key_rotation_alignment(orc) -> float:
    """The query projection and the append rotate by the same position: with
    W^QR = W^KR (one head) and the same hidden state at position p, the rotary
    score q^R . k^R equals |W^KR h|^2 (a rotation applied to both sides)."""
    rng = _rng(12)
    d, dr, dc = 10, 6, 4
    w_kr = rng.standard_normal((dr, d))
    w_dkv = rng.standard_normal((dc, d))
    w_q = rng.standard_normal((3, d))
    err = 0.0
    for p in [0, 1, 7, 300, 8191]:
        h = rng.standard_normal((1, 1, d))
        pos = np.array([[p]])
        row = orc.cache_rows(h, w_dkv, w_kr, pos, 10000.0, "f64")
        _, qr = orc.q_project(h, w_q, w_kr, pos, 1, 10000.0)
        want = float(np.sum((w_kr @ h[0, 0]) ** 2))
        err = max(err, abs(float(qr[0, 0, 0] @ row[0, 0, dc:]) - want) / want)
    return err


ALL_PINS.append(pin_query_key_rotation_alignment)


def _causal_mha_loops(x, wq, wk, wv, H, D):
    """Causal self-attention over every position t of x [L, d]: position t
    attends positions 0..t, softmax(q k^T / sqrt(D)) v per head, as loops."""
    L, d = x.shape

    def proj(w, t, row):
        return sum(w[row][c] * x[t][c] for c in range(d))
    out = np.zeros((L, H, D))
    for t in range(L):
        for hh in range(H):
            q = [proj(wq, t, hh * D + e) for e in range(D)]
            z = []
            for u in range(t + 1):
                k = [proj(wk, u, hh * D + e) for e in range(D)]
                z.append(sum(q[e] * k[e] for e in range(D)) / math.sqrt(D))
            mx = max(z)
            w = [math.exp(zz - mx) for zz in z]
            s = sum(w)
            for u in range(t + 1):
                v = [proj(wv, u, hh * D + e) for e in range(D)]
                for e in range(D):
                    out[t, hh, e] += w[u] / s * v[e]
    return out


def pin_prefill_causal_mha(orc) -> float:
    """Prefill: every token of a sequence is a query (a query group of the whole
    length).  With the MHA special case of the append and decompression weights
    (W^DKV = [W_K; W_V], W^UK = [I 0], W^UV = [0 I], no rotary part), position t
    must equal textbook causal self-attention over positions 0..t, checked
    against explicit loops for every position, in two sequences of different
    lengths sharing one permuted pool."""
    rng = _rng(13)
    H, D, d, dr, bs = 2, 3, 5, 2, 4
    lens = [7, 10]
    dc = 2 * H * D
    wq, wk, wv = (rng.standard_normal((H * D, d)) for _ in range(3))
    w_dkv = np.concatenate([wk, wv], axis=0)
    eye = np.eye(H * D)
    w_uk = np.concatenate([eye, np.zeros((H * D, H * D))], axis=1)
    w_uv = np.concatenate([np.zeros((H * D, H * D)), eye], axis=1)
    w_kr = np.zeros((dr, d))
    w_qr = np.zeros((H * dr, d))
    nblk = [(L + bs - 1) // bs for L in lens]
    perm = rng.permutation(sum(nblk))
    bt = np.full((2, max(nblk)), -1, dtype=np.int64)
    bt[0, :nblk[0]] = perm[:nblk[0]]
    bt[1, :nblk[1]] = perm[nblk[0]:]
    pool = np.full((sum(nblk), bs, dc + dr), 7.0)
    Lm = max(lens)
    xs = [rng.standard_normal((L, d)) for L in lens]
    qn = np.zeros((2, Lm, H, D))
    qr = np.zeros((2, Lm, H, dr))
    err = 0.0
    for b, (L, x) in enumerate(zip(lens, xs)):
        pos = np.arange(L)[None, :]
        rows = orc.cache_rows(x[None], w_dkv, w_kr, pos, 10000.0, "f64")
        orc.write_rows(pool, bt[b:b + 1], pos, rows, bs)
    for b, (L, x) in enumerate(zip(lens, xs)):
        pos = np.arange(L)[None, :]
        qn_b, qr_b = orc.q_project(x[None], wq, w_qr, pos, H, 10000.0)
        out, lse = orc.decode(qn_b, qr_b, w_uk, w_uv, pool, bt[b:b + 1], [L], 1.0 / math.sqrt(D), bs)
        ref = _causal_mha_loops(x, wq, wk, wv, H, D)
        err = max(err, float(np.max(np.abs(out[0] - ref))))
    return err


ALL_PINS.append(pin_prefill_causal_mha)


def _mha_layer_loops(x, wq, wk, wv, wo, H, D):
    """Textbook MHA layer output at the last position, as loops: per head
    softmax(q k^T / sqrt(D)) v, heads concatenated, then u = W_O [o_1; ...]."""
    o = _mha_loops(x, wq, wk, wv, H, D).reshape(-1)
    d = wo.shape[0]
    return np.array([sum(wo[r][c] * o[c] for c in range(H * D)) for r in range(d)])


def pin_layer_mha_special_case(orc) -> float:
    """The full layer (query compression, up-projections, attention, output
    projection) in the MHA special case: W^DQ a random invertible d x d map,
    W^UQ = W_Q (W^DQ)^-1 so that q^C = W_Q h, no rotary part, W^DKV = [W_K; W_V],
    W^UK = [I 0], W^UV = [0 I], and W^O = W_O: u must equal the textbook MHA
    layer output written as loops."""
    rng = _rng(14)
    H, D, d, L, dr, bs = 2, 3, 6, 5, 2, 4
    x = rng.standard_normal((L, d))
    wq, wk, wv = (rng.standard_normal((H * D, d)) for _ in range(3))
    wo = rng.standard_normal((d, H * D))
    w_dq = rng.standard_normal((d, d)) + 3.0 * np.eye(d)
    w_uq = wq @ np.linalg.inv(w_dq)
    w_qr = np.zeros((H * dr, d))
    dc = 2 * H * D
    w_dkv = np.concatenate([wk, wv], axis=0)
    eye = np.eye(H * D)
    w_uk = np.concatenate([eye, np.zeros((H * D, H * D))], axis=1)
    w_uv = np.concatenate([np.zeros((H * D, H * D)), eye], axis=1)
    pos = np.arange(L)[None, :]
    rows = orc.cache_rows(x[None], w_dkv, np.zeros((dr, d)), pos, 10000.0, "f64")
    nblk = (L + bs - 1) // bs
    pool = np.full((nblk, bs, dc + dr), 7.0)
    bt = np.arange(nblk)[None, :]
    orc.write_rows(pool, bt, pos, rows, bs)
    qn, qr = orc.layer_queries(x[None, L - 1:L], w_dq, w_uq, w_qr, pos[:, L - 1:], H, 10000.0)
    out, _ = orc.decode(qn, qr, w_uk, w_uv, pool, bt, [L], 1.0 / math.sqrt(D), bs)
    u = orc.out_project(out, wo)
    ref = _mha_layer_loops(x, wq, wk, wv, wo, H, D)
    return float(np.max(np.abs(u[0, 0] - ref)))


def pin_layer_queries_rotary(orc) -> float:
    """The compressed query's rotary part: with one head, W^DQ = I (a d-wide
    query latent) and W^QR = W^KR, q^R . k^R at the same position equals
    |W^KR h|^2 (both sides turned by the same rotation); and q^C equals
    W^UQ (W^DQ h) summed by hand."""
    rng = _rng(15)
    d, dr, dc = 8, 4, 3
    w_kr = rng.standard_normal((dr, d))
    w_dkv = rng.standard_normal((dc, d))
    w_dq = np.eye(d)
    w_uq = rng.standard_normal((5, d))
    err = 0.0
    for p in [0, 3, 4096]:
        h = rng.standard_normal((1, 1, d))
        pos = np.array([[p]])
        row = orc.cache_rows(h, w_dkv, w_kr, pos, 10000.0, "f64")
        qn, qr = orc.layer_queries(h, w_dq, w_uq, w_kr, pos, 1, 10000.0)
        want = float(np.sum((w_kr @ h[0, 0]) ** 2))
        err = max(err, abs(float(qr[0, 0, 0] @ row[0, 0, dc:]) - want) / want)
        hand = [sum(w_uq[r][c] * h[0, 0, c] for c in range(d)) for r in range(5)]
        err = max(err, float(np.max(np.abs(qn[0, 0, 0] - hand))))
    return err


ALL_PINS.append(pin_layer_mha_special_case)
ALL_PINS.append(pin_layer_queries_rotary)


# ---------------------------------------------------------------- FP8 latent cache
def pin_e4m3_table(orc) -> float:
    """The 256 E4M3 code values equal torch's float8_e4m3fn decoding, and the
    hand-worked ones: 0x01 = 2^-9 (smallest subnormal), 0x08 = 2^-6 (smallest
    normal), 0x38 = 1, 0x7E = 448, 0x7F NaN, 0x80 = -0, 0xFE = -448."""
    import torch
    mine = orc.e4m3_values()
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    if not np.array_equal(mine, lib, equal_nan=True):
        return math.inf
    hand = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x39: 1.125,
            0x7E: 448.0, 0xFE: -448.0}
    if any(mine[c] != v for c, v in hand.items()):
        return math.inf
    if not (np.isnan(mine[0x7F]) and np.isnan(mine[0xFF]) and mine[0x80] == 0 and np.signbit(mine[0x80])):
        return math.inf
    return 0.0


def pin_e4m3_rounding(orc) -> float:
    """Rounding to E4M3 equals torch's float32 -> float8_e4m3fn cast (nearest,
    ties to even) on log-uniform values from 2^-14 to 448 of both signs and on
    every midpoint between neighbouring codes; plus hand-worked cases."""
    import torch
    rng = _rng(16)
    mags = orc.e4m3_values()[:0x7F]
    y = np.exp(rng.uniform(math.log(2.0 ** -14), math.log(448.0), 20000)) * rng.choice([-1.0, 1.0], 20000)
    mids = (mags[:-1] + mags[1:]) / 2
    y = np.concatenate([y, mids, -mids, mags, -mags, [0.0, -0.0]]).astype(np.float32)
    lib = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    if not np.array_equal(orc.round_e4m3(y.astype(np.float64)), lib):
        return math.inf
    # 2^-10 sits halfway between 0 and 2^-9 -> 0; 3 * 2^-10 between codes 1 and 2 -> 2;
    # 1 + 1/16 between 1 (0x38) and 1.125 (0x39) -> 0x38; 1.1875 between 0x39 and 0x3A -> 0x3A;
    # a tiny negative value rounds to -0 (0x80)
    hand = orc.round_e4m3(np.array([2.0 ** -10, 3 * 2.0 ** -10, 1.0625, 1.1875, -1e-5, 447.0, -0.3]))
    want = np.array([0x00, 0x02, 0x38, 0x3A, 0x80, 0x7E, 0x80 | 0x2A], dtype=np.uint8)   # 0.3 -> 0.3125 = 1.25 * 2^-2
    return 0.0 if np.array_equal(hand, want) else math.inf


def _nearest_code_brute(y: float, vals) -> int:
    """Code of the finite E4M3 value nearest to y by trying all of them; a tie goes
    to the code with an even mantissa; the sign follows y."""
    best, best_d = None, None
    for code in range(0x7F):
        d = abs(abs(y) - vals[code])
        if best is None or d < best_d or (d == best_d and code % 2 == 0):
            best, best_d = code, d
    return best | (0x80 if math.copysign(1.0, y) < 0 else 0)


def pin_fp8_quantize(orc) -> float:
    """Row quantisation: (a) a row that is s0 times E4M3 values with a 448 in it
    (s0 a power of two) comes back exactly, with scale s0; (b) on small random
    bf16 rows the scale is the smallest power of two 2^k (k >= -124) with
    amax <= 448 * 2^k, found by trying every k, every code equals a brute-force
    nearest-code search on c / s, and |dequantised - c| stays within half a
    code step (relative 2^-4, absolute 2^-10 s below 2^-6 s); (c) an all-zero
    row gets scale 1 and zero codes, a row below the scale floor gets 2^-124;
    (d) k^R passes unchanged."""
    rng = _rng(17)
    vals = orc.e4m3_values()
    err = 0.0
    # (a), (d)
    for s0 in [2.0 ** -7, 1.0, 2.0 ** 5]:
        codes = rng.integers(0, 0x7F, 40) | (rng.integers(0, 2, 40) << 7)
        codes[7] = 0x7E
        lat = vals[codes] * s0
        row = np.concatenate([lat, [0.5, -2.0]])[None]
        c2, sc, rope = orc.quantize_rows(row, 40)
        deq = orc.dequantize_rows(c2, sc, rope)
        if sc[0] != np.float32(s0) or not np.array_equal(deq[0, :40], lat) or not np.array_equal(rope[0], [0.5, -2.0]):
            return math.inf
    # (b)
    import torch
    for trial in range(8):
        x = torch.from_numpy(rng.standard_normal(12) * np.exp(rng.uniform(-6, 6, 12))).to(torch.bfloat16)
        x = x.to(torch.float64).numpy()
        if trial == 0:
            x[3] = 448.0 * 2.0 ** -3          # amax exactly at a boundary: s = 2^-3
            x[:3] = x[4:] = 0.01
        codes, sc, _ = orc.quantize_rows(np.concatenate([x, [1.0]])[None], 12)
        amax = float(np.max(np.abs(x)))
        k = next(k for k in range(-124, 200) if amax <= 448.0 * 2.0 ** k)
        s = 2.0 ** k
        if float(sc[0]) != s:
            return math.inf
        for q in range(12):
            if int(codes[0, q]) != _nearest_code_brute(x[q] / s, vals):
                return math.inf
        deq = vals[codes[0]] * s
        step = np.where(np.abs(x) >= 2.0 ** -6 * s, np.abs(x) * 2.0 ** -4, 2.0 ** -10 * s)
        err = max(err, float(np.max(np.abs(deq - x) / step)) - 1.0)
    # (c)
    codes, sc, _ = orc.quantize_rows(np.zeros((1, 9)), 8)
    if sc[0] != 1.0 or np.any(codes & 0x7F):
        return math.inf
    codes, sc, _ = orc.quantize_rows(np.array([[1e-37, -3e-38, 0.0]]), 2)
    if float(sc[0]) != 2.0 ** -124 or int(codes[0, 0]) != _nearest_code_brute(1e-37 / 2.0 ** -124, vals):
        return math.inf
    return max(err, 0.0)


def pin_fp8_page_layout(orc) -> float:
    """A hand-built page (2 tokens, d_c = 2, d_R = 2): code rows, then bf16 rotary
    rows, then fp32 scales, little-endian; and what it dequantises to."""
    codes = np.array([[[1, 2], [3, 4]]], dtype=np.uint8)
    rope_bits = np.array([[[0x3F80, 0x4000], [0xBF80, 0x0000]]], dtype=np.uint16)   # 1, 2, -1, 0
    scales = np.array([[2.0, 0.5]], dtype=np.float32)
    want = bytes([1, 2, 3, 4, 0x80, 0x3F, 0x00, 0x40, 0x80, 0xBF, 0x00, 0x00,
                  0x00, 0x00, 0x00, 0x40, 0x00, 0x00, 0x00, 0x3F])
    page = orc.pack_fp8_pages(codes, rope_bits, scales)
    if page.shape != (1, 20) or bytes(page[0]) != want or orc.fp8_page_bytes(2, 2, 2) != 20:
        return math.inf
    c2, r2, s2 = orc.unpack_fp8_pages(page, 2, 2, 2)
    if not (np.array_equal(c2, codes) and np.array_equal(r2, rope_bits) and np.array_equal(s2, scales)):
        return math.inf
    # codes 1..4 are the subnormals k * 2^-9
    rows = orc.dequantize_pages(page, 2, 2, 2)
    hand = np.array([[[2.0 ** -8, 2.0 ** -7, 1.0, 2.0], [3 * 2.0 ** -10, 2.0 ** -8, -1.0, 0.0]]])
    return float(np.max(np.abs(rows - hand)))


ALL_PINS += [pin_e4m3_table, pin_e4m3_rounding, pin_fp8_quantize, pin_fp8_page_layout]
