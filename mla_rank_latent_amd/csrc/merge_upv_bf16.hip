// Log-sum-exp merge of the split partial states and the W^UV up-projection,
// gfx950 bf16 MFMA with fp32 accumulate.
//
// Each range of cached tokens left, per query row, an un-normalised latent
// sum O_k = sum_j 2^(z_j - m_k) c_j with its reference m_k and weight sum
// l_k (log2 units).  The exact merge is
//   M = max_k m_k,  w_k = 2^(m_k - M),
//   o_lat = sum_k w_k O_k / sum_k w_k l_k,   lse = ln 2 * (M + log2 sum_k w_k l_k).
// Then the value side of matrix absorption ("DeepSeek-V2: Multi-Head Latent
// Attention (MLA) 原理与工程实现" §2.2: sum_j p_j W^UV_i c_j = W^UV_i sum_j p_j c_j)
// restores the head's output, out_i = W^UV_i o_lat (W^UV_i = rows 128 i ..
// 128 i + 127 of W^UV, §2.1).
// One workgroup per (head, 32 query rows): it merges its rows into LDS and
// runs [32 x 512] . [512 x 128] on MFMA 32x32x16.  The merged latent is split
// into a bf16 high part and a bf16 remainder (two MFMAs per step), which keeps
// the product close to fp32 accuracy.
#include "device_util.h"

namespace mla {

namespace {
__device__ __forceinline__ bf16x8 as_bf8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
}  // namespace

__global__ __launch_bounds__(256) void merge_upv_bf16_kernel(const uint16_t* __restrict__ w_uv, int batch, int sq,
                                                             int n_heads, int hg, int P,
                                                             const uint8_t* __restrict__ ws, WsLayout Lw,
                                                             uint16_t* __restrict__ out, float* __restrict__ lse) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * 32 * kLat * 2];   // hi and lo parts, 32 rows each
  MLA_LDS uint8_t* s_hi = (MLA_LDS uint8_t*)smem;
  MLA_LDS uint8_t* s_lo = s_hi + 32 * kLat * 2;

  const int M = batch * sq;
  const int h = blockIdx.x % n_heads;
  const int mb = blockIdx.x / n_heads;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int hh = lane >> 5;
  const int n = lane & 31;

  // Issue the W^UV_i loads first; they overlap with the merge.
  // B operand (K = latent c, N = output column d): lane holds W^UV[128 h + 32 wave + n][16 ks + 8 hh .. +7].
  u32x4 bop[32];
  {
    const uint16_t* wp = w_uv + ((size_t)h * kNope + 32 * wave + n) * kLat + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) bop[ks] = *(const u32x4*)(wp + 16 * ks);
  }

  // ---- merge: thread = (row i, 64-column part)
  {
    const int i = tid >> 3;
    const int cpart = tid & 7;
    const int m = mb * 32 + i;
    float acc[64];
#pragma unroll
    for (int c = 0; c < 64; ++c) acc[c] = 0.0f;
    float den = 0.0f, Mx = -__builtin_inff();
    if (m < M) {
      const int b = m / sq;
      const int s = m - b * sq;
      const int g = h / hg;
      const int r = (h - g * hg) * sq + s;
      const int32_t* piece_base = (const int32_t*)(ws + Lw.off_piece);
      const float2* part_ml = (const float2*)(ws + Lw.off_lse);
      const float* part_o = (const float*)(ws + Lw.off_o);
      const int p0 = g * P + piece_base[b];
      const int p1 = g * P + piece_base[b + 1];
      for (int p = p0; p < p1; ++p) {
        float2 ml = part_ml[(size_t)p * Lw.rows + r];
        if (ml.y > 0.0f) Mx = fmaxf(Mx, ml.x);
      }
      for (int p = p0; p < p1; ++p) {
        float2 ml = part_ml[(size_t)p * Lw.rows + r];
        if (!(ml.y > 0.0f)) continue;
        const float wk = __builtin_amdgcn_exp2f(ml.x - Mx);
        den += wk * ml.y;
        const f32x4* op = (const f32x4*)(part_o + ((size_t)p * Lw.rows + r) * kLat + cpart * 64);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          f32x4 v = op[j];
          acc[4 * j] += wk * v[0];
          acc[4 * j + 1] += wk * v[1];
          acc[4 * j + 2] += wk * v[2];
          acc[4 * j + 3] += wk * v[3];
        }
      }
      if (cpart == 0 && lse != nullptr)
        lse[(size_t)m * n_heads + h] =
            den > 0.0f ? (Mx + __builtin_amdgcn_logf(den)) * 0.69314718055994531f : -__builtin_inff();
    }
    const float inv = den > 0.0f ? 1.0f / den : 0.0f;
    // write 8 chunks of 8 columns, chunk k of row i at k ^ (i % 8); start at a
    // lane-dependent chunk so the 8 threads of a row hit different banks
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int j = (jj + cpart) & 7;
      u32x4 vh, vl;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x0 = acc[8 * j + 2 * e] * inv, x1 = acc[8 * j + 2 * e + 1] * inv;
        uint16_t h0 = f2bf(x0), h1 = f2bf(x1);
        vh[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        vl[e] = pack_bf2(x0 - bf2f(h0), x1 - bf2f(h1));
      }
      const int chunk = cpart * 8 + j;
      const int off = i * (kLat * 2) + ((chunk & ~7) | ((chunk & 7) ^ (i & 7))) * 16;
      *(MLA_LDS u32x4*)(s_hi + off) = vh;
      *(MLA_LDS u32x4*)(s_lo + off) = vl;
    }
  }
  __syncthreads();

  // ---- out[32 rows x 32 cols of this wave] = o_lat . W^UV_i^T
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
  for (int ks = 0; ks < 32; ++ks) {
    const int chunk = 2 * ks + hh;
    const int off = n * (kLat * 2) + ((chunk & ~7) | ((chunk & 7) ^ (n & 7))) * 16;
    u32x4 ah = *(const MLA_LDS u32x4*)(s_hi + off);
    u32x4 al = *(const MLA_LDS u32x4*)(s_lo + off);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(ah), as_bf8(bop[ks]), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(al), as_bf8(bop[ks]), acc, 0, 0, 0);
  }
  const int d = 32 * wave + n;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = mb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
    if (m < M) out[((size_t)m * n_heads + h) * kNope + d] = f2bf(acc[r]);
  }
}

hipError_t launch_merge_upv_bf16(const WsLayout& L, const uint16_t* w_uv, int batch, int sq, int n_heads, uint8_t* ws,
                                 uint16_t* out, float* lse, hipStream_t st) {
  const int M = batch * sq;
  dim3 grid(n_heads * ((M + 31) / 32));
  hipLaunchKernelGGL(merge_upv_bf16_kernel, grid, dim3(256), 0, st, w_uv, batch, sq, n_heads, L.hg, L.P,
                     (const uint8_t*)ws, L, out, lse);
  return hipGetLastError();
}

}  // namespace mla
