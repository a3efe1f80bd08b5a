// Cache append for MLA on gfx950: down-projection, decoupled RoPE, paged write.
//
// "DeepSeek-V2: Multi-Head Latent Attention (MLA) 原理与工程实现" §2.1 (joint
// compression c = W^DKV h), §3.2 (shared rotary key k^R = RoPE(W^KR h), applied
// directly and never compressed) and §3.3 (only [c ‖ k^R] is cached):
//   row = [W^DKV h ‖ RoPE_p(W^KR h)],  written to slot block_table[p / 64] * 64 + p % 64.
// The 576 output columns and the new tokens form a GEMM [tokens x d] . [d x 576]
// run on MFMA 16x16x32: one workgroup per (16 tokens, 16 columns), its sixteen
// waves splitting d (each issues all of its loads before its MFMAs, so the
// weights stream at memory rate) and summing their partial tiles in a fixed
// order (so the result does not depend on timing).  Both operands are
// K-contiguous in memory (h rows and W rows), so they stream straight from
// global memory.
// RoPE pairs (x_{2i}, x_{2i+1}) turn by angle p * base^(-2i/64), with the angle,
// its sine and cosine and the rotation in fp64; each value is then rounded
// once to bf16.
#include "device_util.h"

namespace mla {

namespace {
__device__ __forceinline__ bf16x8 as_bf8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
constexpr int kAppendWaves = 16;
}  // namespace

__global__ __launch_bounds__(64 * kAppendWaves) void append_bf16_kernel(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ w_dkv, const uint16_t* __restrict__ w_kr,
    const int32_t* __restrict__ positions, const int32_t* __restrict__ block_table, int max_blocks,
    uint16_t* __restrict__ cache, int num_blocks, int tokens, int t_per_seq, int d_model, double rope_base,
    int32_t* status) {
  __shared__ float part[kAppendWaves][16][17];
  const int cb = blockIdx.x % (kRow / 16);   // 16-column block of the 576-wide row
  const int tb = blockIdx.x / (kRow / 16);   // 16-token block
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;

  // A: h[token 16 tb + lane%16][k], B: W[col][k] with k = 32 ks + 8 (lane/16) .. +7
  const int tok_a = tb * 16 + (lane & 15);
  const int col_b = cb * 16 + (lane & 15);
  const uint16_t* wrow = col_b < kLat ? w_dkv + (size_t)col_b * d_model : w_kr + (size_t)(col_b - kLat) * d_model;
  const uint16_t* hrow = h + (size_t)(tok_a < tokens ? tok_a : 0) * d_model;
  const int koff = 8 * (lane >> 4);
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  const int nks = d_model / 32;   // k-steps of 32; wave w takes steps w, w + 16, ...
  const int nmine = (nks - wave + kAppendWaves - 1) / kAppendWaves;
  const bool tok_ok = tok_a < tokens;
  for (int i0 = 0; i0 < nmine; i0 += 8) {
    u32x4 a[8], b[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int ks = wave + kAppendWaves * (i0 + u < nmine ? i0 + u : i0);
      a[u] = *(const u32x4*)(hrow + 32 * ks + koff);
      b[u] = *(const u32x4*)(wrow + 32 * ks + koff);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      // steps past this wave's share repeat an earlier step with a zero operand
      const u32x4 av = (tok_ok && i0 + u < nmine) ? a[u] : u32x4{0u, 0u, 0u, 0u};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(av), as_bf8(b[u]), acc, 0, 0, 0);
    }
  }
  // D: lane holds column lane%16, rows 4 (lane/16) + r
#pragma unroll
  for (int r = 0; r < 4; ++r) part[wave][4 * (lane >> 4) + r][lane & 15] = acc[r];
  __syncthreads();

  if (tid < 256) {
    const int row = tid >> 4;   // token within the block
    const int cl = tid & 15;    // column within the block
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < kAppendWaves; ++w) v += part[w][row][cl];
    const int tok = tb * 16 + row;
    const int col = cb * 16 + cl;
    if (tok < tokens) {
      const int b = tok / t_per_seq;
      const int pos = positions[tok];
      if (pos < 0 || pos >= max_blocks * kBlk) {
        if (status) atomicOr(status, MLA_STATUS_BAD_POS);
        return;
      }
      const int blk = block_table[(size_t)b * max_blocks + pos / kBlk];
      if (blk < 0 || blk >= num_blocks) {
        if (status) atomicOr(status, MLA_STATUS_BAD_BLOCK);
        return;
      }
      uint16_t outv;
      if (col < kLat) {
        outv = f2bf(v);
      } else {
        // partner of the RoPE pair sits in the neighbouring column of the same block
        float vp = 0.0f;
#pragma unroll
        for (int w = 0; w < kAppendWaves; ++w) vp += part[w][row][cl ^ 1];
        const int j = col - kLat;
        const double x0 = (j & 1) ? vp : v;
        const double x1 = (j & 1) ? v : vp;
        double y0, y1;
        rope_pair(x0, x1, pos, j >> 1, kRope, rope_base, &y0, &y1);
        outv = d2bf((j & 1) ? y1 : y0);
      }
      cache[((size_t)blk * kBlk + pos % kBlk) * kRow + col] = outv;
    }
  }
}

hipError_t launch_append_bf16(const uint16_t* h, const uint16_t* w_dkv, const uint16_t* w_kr, const int32_t* positions,
                              const int32_t* block_table, int max_blocks, uint16_t* cache, int num_blocks, int tokens,
                              int t_per_seq, int d_model, float rope_base, int32_t* status, hipStream_t st) {
  dim3 grid((kRow / 16) * ((tokens + 15) / 16));
  hipLaunchKernelGGL(append_bf16_kernel, grid, dim3(64 * kAppendWaves), 0, st, h, w_dkv, w_kr, positions, block_table,
                     max_blocks, cache, num_blocks, tokens, t_per_seq, d_model, (double)rope_base, status);
  return hipGetLastError();
}

}  // namespace mla
