// Tiles of a decode step's preparation, shared by the kernels that run them alone
// (the split append's partial products, the absorbed queries) and by the kernel that
// runs them side by side in one launch (a decode step that appends its own tokens).
// What they compute is described at the kernels in append_bf16.hip and absorb_bf16.hip.
#pragma once

#include "device_util.h"

namespace mla {
namespace prep {

__device__ __forceinline__ bf16x8 as_bf8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// ---- split append: K slices of at most kSliceSteps k-steps (32 elements) of d_model
constexpr int kSliceSteps = 10;
constexpr int kSliceChunks = 4 * kSliceSteps + 1;  // 16-byte chunks per padded LDS row
constexpr int kAppendPartialLds = (32 * kSliceChunks + 63) / 64 * 1024;   // 32 weight rows

// One [64 tokens x 32 columns] partial product over K slice sl of the split append:
// ct = 32-column tile of the 576-wide row, tg = 64-token group; lds holds
// kAppendPartialLds bytes (whole 1 KB copies: the lanes of the last copy past the tile
// still write their 16 bytes).  The 32 weight rows of the tile, read by all four waves,
// go through LDS; each wave's 16 token rows go straight into its operand registers
// (lane: token 16 wave + lane % 16, features 32 ks + 8 (lane / 16) .. +7 of the slice,
// the MFMA 16x16x32 A layout), issued together with the weight copies.
__device__ __forceinline__ void append_partial_tile(const uint16_t* __restrict__ h, const uint16_t* __restrict__ w_dkv,
                                                    const uint16_t* __restrict__ w_kr, int tokens, int d_model,
                                                    int nslice, float* __restrict__ part, MLA_LDS uint8_t* lds, int ct,
                                                    int tg, int sl) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int nks = d_model / 32;
  const int k0 = (int)((long long)sl * nks / nslice), k1 = (int)((long long)(sl + 1) * nks / nslice);
  const int nsteps = k1 - k0;                       // 1 .. kSliceSteps
  const int rch = 4 * nsteps + 1;                   // chunks per padded LDS row (odd)

  const int tok = tg * 64 + wave * 16 + (lane & 15);
  const bool tok_ok = tok < tokens;
  const uint16_t* hrow = h + (size_t)(tok_ok ? tok : 0) * d_model + 32 * k0 + 8 * (lane >> 4);
  u32x4 a[kSliceSteps];
#pragma unroll
  for (int ks = 0; ks < kSliceSteps; ++ks)
    if (ks < nsteps) a[ks] = *(const u32x4*)(hrow + 32 * ks);

  // copy: LDS chunk P = 64 q + lane holds weight row P / rch, chunk P % rch (the last chunk
  // of a row is padding: it re-reads the row's first chunk)
  const int nchunks = 32 * rch;
  for (int q = wave; q * 64 < nchunks; q += 4) {
    int P = q * 64 + lane;
    if (P >= nchunks) P = nchunks - 1;              // the tail lanes repeat the last chunk
    const int row = P / rch;
    int ch = P - row * rch;
    if (ch == rch - 1) ch = 0;
    const int col = ct * 32 + row;
    const uint16_t* src = col < kLat ? w_dkv + (size_t)col * d_model : w_kr + (size_t)(col - kLat) * d_model;
    src += 32 * k0 + 8 * ch;
    const uint32_t dst = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds + q * 1024));
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(dst) : "memory");
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();

  // wave w: tokens 16 w .. +15 (A rows) against the 32 columns (two 16-wide B blocks)
  const MLA_LDS uint8_t* brow0 = lds + (lane & 15) * rch * 16 + 16 * (lane >> 4);
  const MLA_LDS uint8_t* brow1 = brow0 + 16 * rch * 16;
  f32x4 acc[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
  for (int ks = 0; ks < kSliceSteps; ++ks) {
    if (ks < nsteps) {
      const u32x4 b0 = *(const MLA_LDS u32x4*)(brow0 + 64 * ks);
      const u32x4 b1 = *(const MLA_LDS u32x4*)(brow1 + 64 * ks);
      const u32x4 av = tok_ok ? a[ks] : u32x4{0u, 0u, 0u, 0u};
      acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(av), as_bf8(b0), acc[0], 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(av), as_bf8(b1), acc[1], 0, 0, 0);
    }
  }
  // D: lane holds column lane % 16 of its 16-column block, tokens 4 (lane / 16) + r of the wave's 16
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = tg * 64 + wave * 16 + 4 * (lane >> 4) + r;
      if (t < tokens) part[((size_t)t * nslice + sl) * kRow + ct * 32 + nb * 16 + (lane & 15)] = acc[nb][r];
    }
}

// Tile of the split append for linear index a = 0 .. T - 1, T = n_ct * n_tg * nslice.  The
// n_ct column tiles of one (token group, slice) read the same 64 x 32 k-step block of h,
// so they should share an XCD (and its L2): block ids equal modulo 8 share one, and with
// T a multiple of 8 the ids a with a % 8 = r take the r-th eighth of the tiles in
// (slice, token group, column tile) order.  Otherwise a is that order itself.
__device__ __forceinline__ void append_tile_of(int a, int n_ct, int n_tg, int nslice, int* ct, int* tg, int* sl) {
  const int T = n_ct * n_tg * nslice;
  const int s = T % 8 == 0 ? (a % 8) * (T / 8) + a / 8 : a;
  *ct = s % n_ct;
  *tg = (s / n_ct) % n_tg;
  *sl = s / (n_ct * n_tg);
}

// ---- absorbed queries
constexpr int kAbsorbLds = kNope * 256;   // the 128 x 128 W^UK slice
__device__ __forceinline__ int swz(int t) { return ((t & 3) << 1) | ((t >> 2) & 1); }

// One (head, 128 latent columns) block of the absorbed queries; bid = 0 .. 4 n_heads - 1;
// lds holds kAbsorbLds bytes, 1 KB aligned.  The weight slice goes through LDS (its
// contraction index runs along strided rows, which the transposing LDS read turns into
// the MFMA operand); the query rows, contiguous along the contraction, go straight into
// operand registers.
__device__ __forceinline__ void absorb_tile(const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_rope,
                                            const uint16_t* __restrict__ w_uk, int batch, int sq, int n_heads,
                                            float qscale, uint8_t* __restrict__ ws, const WsLayout& Lw,
                                            MLA_LDS uint8_t* lds, int bid) {
  uint8_t* q_lat = ws + Lw.off_qlat;   // operand order: qlat_byte()

  // (head, 128-column block of the latent).  Consecutive block ids go to the XCDs in turn,
  // so ids equal modulo 8 share an XCD and its L2.  With n_heads a multiple of 64, XCD x
  // takes heads 8 x .. 8 x + 7 (+ 64 k), all four column blocks of each: a head's blocks
  // share its query rows in L2, and the 128-byte lines of the operand-order layout (16
  // bytes of eight consecutive heads each) are written from one L2 only.  Otherwise the
  // four blocks of a head take ids 8 apart.
  int h, cb;
  if (n_heads % 64 == 0) {
    const int x = bid % 8, j = bid / 8;
    const int lh = j / 4;
    cb = j % 4;
    h = 8 * x + lh % 8 + 64 * (lh / 8);
  } else {
    const int full = (n_heads / 8) * 32;
    if (bid < full) {
      h = 8 * (bid / 32) + bid % 8;
      cb = (bid / 8) % 4;
    } else {
      h = (n_heads / 8) * 8 + (bid - full) / 4;
      cb = (bid - full) % 4;
    }
  }
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int M = batch * sq;
  const int nmb = (M + 31) / 32;      // 32-row blocks of query rows
  const int hh = lane >> 5;
  const int n = lane & 31;

  // query operand of row block mb (MFMA 32x32x16 layout, the query rows on the N side):
  // lane (hh, n) holds row 32 mb + n, features 16 ks + 8 hh .. +7; rows past M re-read row M - 1
  auto load_q = [&](int mb, u32x4 (&qa)[8]) {
    int m = mb * 32 + n;
    m = m < M ? m : M - 1;
    const uint16_t* src = q_nope + ((size_t)m * n_heads + h) * kNope + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qa[ks] = *(const u32x4*)(src + 16 * ks);
  };
  u32x4 qa[2][8];
  load_q(0, qa[0]);
  if (nmb > 1) load_q(1, qa[1]);

  // stage the slice: LDS row d holds columns cb*128 .. +127 of W^UK row 128 h + d,
  // its 16-byte chunk k at chunk k ^ swz(d)
  {
    const uint8_t* gbase = (const uint8_t*)w_uk + ((size_t)h * kNope * kLat + cb * 128) * 2;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      int P = 64 * (wave + 4 * k) + lane;   // 16-byte chunk index inside the 32 KB slice
      int d = P >> 4;
      int c = (P & 15) ^ swz(d);
      const uint8_t* src = gbase + (size_t)d * (kLat * 2) + c * 16;
      uint32_t dst = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds + (wave + 4 * k) * 1024));
      asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(dst) : "memory");
    }
  }
  // the rotary half of the latent query: q^R times a power of two (exact)
  if (cb == 0) {
    for (int i = tid; i < M * (kRope / 8); i += 256) {
      int m = i / (kRope / 8), j = i % (kRope / 8);
      const u32x4 v = *(const u32x4*)(q_rope + ((size_t)m * n_heads + h) * kRope + 8 * j);
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o[e] = pack_bf2(bf2f((uint16_t)(v[e] & 0xffffu)) * qscale, bf2f((uint16_t)(v[e] >> 16)) * qscale);
      const size_t r = ((size_t)(m / sq) * n_heads + h) * sq + m % sq;
      *(u32x4*)(q_lat + qlat_byte(r, kLat + 8 * j)) = o;
    }
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();

  // B operand (K = d, N = column): lane 16 g + 4 e + q reads row d = 16 ks + 8 hh + 4 r + e,
  // columns 32 wave + 16 (g % 2) + 4 q .. +3, which the transpose hands out as
  // 4 consecutive d of column 32 wave + (lane % 32).
  const int g16 = lane >> 4;
  const int e_ = (lane >> 2) & 3;
  const int q_ = lane & 3;
  const int chunk = 4 * wave + 2 * (g16 & 1) + (q_ >> 1);
  u32x4 bop[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    u32x2 part[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      int d = 16 * ks + 8 * hh + 4 * r + e_;
      int phys = (chunk & ~7) | ((chunk & 7) ^ (2 * e_ + r));
      const MLA_LDS uint8_t* p = lds + d * 256 + phys * 16 + 8 * (q_ & 1);
      s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS s16x4*)p);
      part[r] = __builtin_bit_cast(u32x2, v);
    }
    bop[ks] = u32x4{part[0][0], part[0][1], part[1][0], part[1][1]};
  }

  // row blocks two at a time in flight: block mb multiplies while block mb + 1 lands
  auto do_block = [&](int mb, u32x4(&cur)[8]) {
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      // operands in swapped roles: the product is D^T, [column x query row]
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(bop[ks]), as_bf8(cur[ks]), acc, 0, 0, 0);
    if (mb + 2 < nmb) load_q(mb + 2, cur);
    // D^T: lane holds query row 32 mb + n, columns 32 wave + 8 (i/4) + 4 hh + i % 4, so
    // each group of four registers is four adjacent columns: one 8-byte store
    const int mm = mb * 32 + n;
    if (mm < M) {
      // features cb*128 + 32 wave + 8 g + 4 hh .. +3: half of one 16-byte operand unit
      const size_t r = ((size_t)(mm / sq) * n_heads + h) * sq + mm % sq;
      // f0 % 16 = 4 hh, so feature f0 + 8 g sits (g / 2) k-steps and (g % 2) lane halves on
      uint8_t* dst = q_lat + qlat_byte(r, cb * 128 + 32 * wave + 4 * hh);
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *(u32x2*)(dst + 1024 * (g >> 1) + 16 * kQBlockRows * (g & 1)) =
            u32x2{pack_bf2(acc[4 * g] * qscale, acc[4 * g + 1] * qscale),
                  pack_bf2(acc[4 * g + 2] * qscale, acc[4 * g + 3] * qscale)};
    }
  };
  for (int mb = 0; mb < nmb; mb += 2) {
    do_block(mb, qa[0]);
    if (mb + 1 < nmb) do_block(mb + 1, qa[1]);
  }
}

}  // namespace prep
}  // namespace mla
