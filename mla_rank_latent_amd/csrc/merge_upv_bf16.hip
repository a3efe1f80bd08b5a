// Log-sum-exp merge of the split partial states and the W^UV up-projection,
// gfx950 bf16 MFMA with fp32 accumulate.
//
// Each range of cached tokens left, per query row, an un-normalised latent
// sum O_k = sum_j 2^(z_j - m_k) c_j (bf16) with its reference m_k and weight
// sum l_k (log2 units).  The exact merge is
//   M = max_k m_k,  w_k = 2^(m_k - M),
//   o_lat = sum_k w_k O_k / sum_k w_k l_k,   lse = ln 2 * (M + log2 sum_k w_k l_k).
// Then the value side of matrix absorption ("DeepSeek-V2: Multi-Head Latent
// Attention (MLA) 原理与工程实现" §2.2: sum_j p_j W^UV_i c_j = W^UV_i sum_j p_j c_j)
// restores the head's output, out_i = W^UV_i o_lat (W^UV_i = rows 128 i ..
// 128 i + 127 of W^UV, §2.1).
//
// One workgroup of eight waves per (head, 32 query rows).
//  - Merge: sixteen threads per row, each owning 32 of its 512 columns
//    (8 bytes at 128-byte strides, so the sixteen lanes of a row read whole
//    128-byte blocks).  Two pieces' loads are in flight per thread and the
//    piece weights are applied branch-free, so the partial states stream at
//    memory rate instead of one round trip per piece.
//  - The merged latent goes to LDS as a bf16 high part and a bf16 remainder
//    (two MFMAs per step keep the product close to fp32 accuracy).
//  - Up-projection [32 x 512] . [512 x 128] on MFMA 32x32x16, computed
//    transposed so that each lane ends with four adjacent output columns per
//    register group (8-byte stores): wave (kh, wc) takes output columns
//    32 wc .. 32 wc + 31 over latent half kh, with its W^UV slice loaded into
//    registers before the merge starts; the two latent halves are summed
//    through LDS.
#include "device_util.h"

namespace mla {

namespace {
__device__ __forceinline__ bf16x8 as_bf8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
constexpr int kMergeRows = 32;
}  // namespace

__global__ __launch_bounds__(512) void merge_upv_bf16_kernel(const uint16_t* __restrict__ w_uv, int batch, int sq,
                                                             int n_heads, int hg, int P,
                                                             const uint8_t* __restrict__ ws, WsLayout Lw,
                                                             uint16_t* __restrict__ out, float* __restrict__ lse) {
  // hi and lo parts of the merged latent (32 rows x 512, swizzled 16-byte
  // chunks), the upper latent half's partial products (32 x 128 fp32), and the
  // slots' partial sums when rows are shared by several slots (32 x 512 fp32)
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kMergeRows * kLat * 2 + kMergeRows * kNope * 4 +
                                                         kMergeRows * kLat * 4];
  __shared__ float s_mx[kMergeRows], s_den[kMergeRows];
  MLA_LDS uint8_t* s_hi = (MLA_LDS uint8_t*)smem;
  MLA_LDS uint8_t* s_lo = s_hi + kMergeRows * kLat * 2;
  MLA_LDS float* s_red = (MLA_LDS float*)(s_lo + kMergeRows * kLat * 2);
  MLA_LDS uint8_t* s_comb = (MLA_LDS uint8_t*)(s_red + kMergeRows * kNope);

  const int M = batch * sq;
  const int h = blockIdx.x % n_heads;
  const int mb = blockIdx.x / n_heads;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int hh = lane >> 5;
  const int n = lane & 31;
  const int kh = wave >> 2;    // latent half of the up-projection
  const int wc = wave & 3;     // output column block

  // B operand (K = latent, N = output column): lane holds
  // W^UV[128 h + 32 wc + n][256 kh + 16 ks + 8 hh .. +7], ks = 0..15.
  u32x4 bop[16];
  {
    const uint16_t* wp = w_uv + ((size_t)h * kNope + 32 * wc + n) * kLat + 256 * kh + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) bop[ks] = *(const u32x4*)(wp + 16 * ks);
  }

  // ---- merge.  Sixteen threads (a slot) own one row's 512 columns: thread c16 of a slot
  // holds columns 64 j + 4 c16 .. +3, j = 0..7.  With rv < 32 valid rows (small batches,
  // whose sequences are split into many pieces) a row gets pl_n = 32 / rp slots (rp = rv
  // rounded up to a power of two) that take every pl_n-th piece; their maxima and then
  // their weighted sums are combined through LDS in slot order.
  {
    const int rv = M - mb * kMergeRows < kMergeRows ? M - mb * kMergeRows : kMergeRows;
    int rp = 1;
    while (rp < rv) rp <<= 1;
    const int pl_n = kMergeRows / rp;
    const int slot = tid >> 4;
    const int c16 = tid & 15;
    const int i = slot % rp;          // row within the block
    const int pl = slot / rp;         // piece lane of the row
    const int m = mb * kMergeRows + i;
    const bool row_ok = i < rv;
    if (rv < kMergeRows) {
      // rows without a slot (or past M) must still hold finite values for the MFMAs
      for (int k = tid; k < kMergeRows * kLat / 4; k += 512) {
        ((MLA_LDS u32x2*)s_hi)[k] = u32x2{0u, 0u};
        ((MLA_LDS u32x2*)s_lo)[k] = u32x2{0u, 0u};
      }
      __syncthreads();   // the rows' own values land after the fill
    }
    f32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float den = 0.0f, Mx = -__builtin_inff();
    int p0 = 0, p1 = 0, r = 0;
    const float2* part_ml = (const float2*)(ws + Lw.off_lse);
    const uint16_t* part_o = (const uint16_t*)(ws + Lw.off_o);   // bf16
    if (row_ok) {
      const int b = m / sq;
      const int s = m - b * sq;
      const int g = h / hg;
      r = (h - g * hg) * sq + s;
      const int32_t* piece_base = (const int32_t*)(ws + Lw.off_piece);
      p0 = g * P + piece_base[b];
      p1 = g * P + piece_base[b + 1];
      // online merge: the running maximum rises as pieces arrive and the sums so far are
      // rescaled, so each pair's loads (states and weights together) need one round trip
      for (int p = p0 + pl; p < p1; p += 2 * pl_n) {
        // the second piece of the pair; past the end it re-reads piece p with weight 0
        const int q = p + pl_n < p1 ? p + pl_n : p;
        const float2 ml0 = part_ml[(size_t)p * Lw.rows + r];
        const float2 ml1 = part_ml[(size_t)q * Lw.rows + r];
        const u32x2* o0 = (const u32x2*)(part_o + ((size_t)p * Lw.rows + r) * kLat) + c16;
        const u32x2* o1 = (const u32x2*)(part_o + ((size_t)q * Lw.rows + r) * kLat) + c16;
        u32x2 b0[8], b1[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) b0[j] = o0[16 * j];
#pragma unroll
        for (int j = 0; j < 8; ++j) b1[j] = o1[16 * j];
        // an empty piece has l = 0 (m = -inf, O = 0): weight 0
        const float m0 = ml0.y > 0.0f ? ml0.x : -__builtin_inff();
        const float m1 = (q != p && ml1.y > 0.0f) ? ml1.x : -__builtin_inff();
        const float mn = fmaxf(Mx, fmaxf(m0, m1));
        if (mn == -__builtin_inff()) continue;   // nothing seen yet
        const float sc = Mx == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(Mx - mn);
        const float w0 = m0 == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m0 - mn);
        const float w1 = m1 == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m1 - mn);
        auto widen = [](u32x2 v) {
          return f32x4{__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xffff0000u), __uint_as_float(v[1] << 16),
                       __uint_as_float(v[1] & 0xffff0000u)};
        };
        den = den * sc + w0 * ml0.y + w1 * ml1.y;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = acc[j] * sc + w0 * widen(b0[j]) + w1 * widen(b1[j]);
        Mx = mn;
      }
    }
    if (pl_n > 1) {   // bring the row's slots to the row's maximum
      if (c16 == 0) s_mx[slot] = Mx;
      __syncthreads();
      float Mg = Mx;
      for (int q = 0; q < pl_n; ++q) Mg = fmaxf(Mg, s_mx[q * rp + i]);
      const float sc = Mx == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(Mx - Mg);
      den *= sc;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] *= sc;
      Mx = Mg;
    }
    if (pl_n > 1) {   // sum the row's slots in slot order
      MLA_LDS f32x4* comb = (MLA_LDS f32x4*)s_comb;
#pragma unroll
      for (int j = 0; j < 8; ++j) comb[(slot * 16 + c16) * 8 + j] = acc[j];
      if (c16 == 0) s_den[slot] = den;
      __syncthreads();
      if (pl == 0) {
        for (int q = 1; q < pl_n; ++q) {
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[j] += comb[((q * rp + i) * 16 + c16) * 8 + j];
          den += s_den[q * rp + i];
        }
      }
    }
    if (row_ok && pl == 0) {
      if (c16 == 0 && lse != nullptr)
        lse[(size_t)m * n_heads + h] =
            den > 0.0f ? (Mx + __builtin_amdgcn_logf(den)) * 0.69314718055994531f : -__builtin_inff();
      const float inv = den > 0.0f ? 1.0f / den : 0.0f;
      // columns 64 j + 4 c16 .. +3 are half (c16 & 1) of logical chunk 8 j + c16 / 2,
      // stored at chunk 8 j + ((c16 / 2) ^ (i % 8))
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        u32x2 vh, vl;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float x0 = acc[j][2 * e] * inv, x1 = acc[j][2 * e + 1] * inv;
          const uint32_t hp = pack_bf2(x0, x1);
          vh[e] = hp;
          vl[e] = pack_bf2(x0 - bf2f((uint16_t)(hp & 0xffffu)), x1 - bf2f((uint16_t)(hp >> 16)));
        }
        const int off = i * (kLat * 2) + (8 * j + ((c16 >> 1) ^ (i & 7))) * 16 + 8 * (c16 & 1);
        *(MLA_LDS u32x2*)(s_hi + off) = vh;
        *(MLA_LDS u32x2*)(s_lo + off) = vl;
      }
    }
  }
  __syncthreads();

  // ---- out[32 rows x 32 cols of this wave] over latent half kh
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) {
    const int chunk = 32 * kh + 2 * ks + hh;
    const int off = n * (kLat * 2) + ((chunk & ~7) | ((chunk & 7) ^ (n & 7))) * 16;
    const u32x4 ah = *(const MLA_LDS u32x4*)(s_hi + off);
    const u32x4 al = *(const MLA_LDS u32x4*)(s_lo + off);
    // operands in swapped roles: the product is out^T, [output column x row]
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(bop[ks]), as_bf8(ah), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(bop[ks]), as_bf8(al), acc, 0, 0, 0);
  }
  // out^T layout: lane holds row n, register r column 32 wc + 8 (r / 4) + 4 hh + r % 4, so each
  // group of four registers is four adjacent columns
  if (kh == 1) {
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *(MLA_LDS f32x4*)(s_red + n * kNope + 32 * wc + 8 * g + 4 * hh) =
          f32x4{acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
  }
  __syncthreads();
  if (kh == 0) {
    const int m = mb * kMergeRows + n;
    if (m < M) {
      uint16_t* dst = out + ((size_t)m * n_heads + h) * kNope + 32 * wc + 4 * hh;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 o = *(const MLA_LDS f32x4*)(s_red + n * kNope + 32 * wc + 8 * g + 4 * hh);
        *(u32x2*)(dst + 8 * g) = u32x2{pack_bf2(acc[4 * g] + o[0], acc[4 * g + 1] + o[1]),
                                        pack_bf2(acc[4 * g + 2] + o[2], acc[4 * g + 3] + o[3])};
      }
    }
  }
}

hipError_t launch_merge_upv_bf16(const WsLayout& L, const uint16_t* w_uv, int batch, int sq, int n_heads, uint8_t* ws,
                                 uint16_t* out, float* lse, hipStream_t st) {
  const int M = batch * sq;
  dim3 grid(n_heads * ((M + kMergeRows - 1) / kMergeRows));
  hipLaunchKernelGGL(merge_upv_bf16_kernel, grid, dim3(512), 0, st, w_uv, batch, sq, n_heads, L.hg, L.P,
                     (const uint8_t*)ws, L, out, lse);
  return hipGetLastError();
}

}  // namespace mla
