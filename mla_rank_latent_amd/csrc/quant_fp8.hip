// FP8 latent cache rows on gfx950: one fp32 scale and 512 E4M3 codes per token.
//
// The cache keeps [c^KV ‖ k^R] per token ("DeepSeek-V2: Multi-Head Latent
// Attention (MLA) 原理与工程实现" §3.3); that page's §5.1 (item 3) names
// quantisation error as the risk of a low-precision form and fixes none.  The
// format here: c^KV as E4M3 codes with one power-of-two scale per token (the
// OCP microscaling convention), s = 2^k for the smallest k >= -124 with
// amax|c| <= 448 s (s = 1 for an all-zero row), code = nearest-even(c / s);
// c / s is exact, and so is s * value(code) in bf16 for |c| < 2^127.  k^R stays
// bf16.  A 64-token page holds the 64 code rows (512 B each), then the 64 k^R
// rows (128 B each), then the 64 scales (fp32, 4 B each).
//
// One wave per row: lane l loads latent features 8 l .. 8 l + 7 (16 bytes of
// the bf16 row); the wave's maximum of |c| gives k (amax = m 2^e with
// 1/2 <= m < 1 makes 512 m in [256, 512), so k is e - 9 when 512 m <= 448 and
// e - 8 otherwise); each lane multiplies its eight values by 2^-k (exact) and
// converts pairs with the hardware's round-to-nearest-even conversion
// (v_cvt_pk_fp8_f32, which keeps the sign of zero); lanes 0..7 copy the 64
// bf16 k^R values.
#include "device_util.h"

namespace mla {

namespace {
constexpr float kE4m3Max = 448.0f;
constexpr int kMinScaleExp = -124;   // keeps s * value(code) representable in bf16
constexpr int kRowsPerWg = 4;   // one wave per row
}  // namespace

__global__ __launch_bounds__(64 * kRowsPerWg) void quant_rows_fp8_kernel(
    const uint16_t* __restrict__ src, long long n_rows, const int32_t* __restrict__ positions,
    const int32_t* __restrict__ block_table, int max_blocks, int t_per_seq, int num_blocks,
    uint8_t* __restrict__ pages, int32_t* status) {
  const long long row = (long long)blockIdx.x * kRowsPerWg + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= n_rows) return;
  // destination page and slot: row r of a whole pool, or token r's position in its table row
  long long blk;
  int slot;
  if (positions == nullptr) {
    blk = row / kBlk;
    slot = (int)(row % kBlk);
  } else {
    const int pos = positions[row];
    if (pos < 0 || pos >= max_blocks * kBlk) {
      if (lane == 0 && status) atomicOr(status, MLA_STATUS_BAD_POS);
      return;
    }
    const int b = (int)(row / t_per_seq);
    const int bi = block_table[(size_t)b * max_blocks + pos / kBlk];
    if (bi < 0 || bi >= num_blocks) {
      if (lane == 0 && status) atomicOr(status, MLA_STATUS_BAD_BLOCK);
      return;
    }
    blk = bi;
    slot = pos % kBlk;
  }
  const uint16_t* r = src + (size_t)row * kRow;
  uint8_t* page = pages + (size_t)blk * kFp8PageBytes;

  const u32x4 v = *(const u32x4*)(r + 8 * lane);
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(v[i] << 16);
    x[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
  }
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(x[i]));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) am = fmaxf(am, __shfl_xor(am, off));
  int k = 0;
  if (am > 0.0f) {
    int e;
    const float m = frexpf(am, &e);
    k = 512.0f * m <= kE4m3Max ? e - 9 : e - 8;
    k = k < kMinScaleExp ? kMinScaleExp : k;
  }
  const float s = ldexpf(1.0f, k);
  const float inv = ldexpf(1.0f, -k);

  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = fminf(fmaxf(x[i] * inv, -kE4m3Max), kE4m3Max);   // |c / s| <= 448
  uint32_t w[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    int word = __builtin_amdgcn_cvt_pk_fp8_f32(y[4 * h], y[4 * h + 1], 0, false);        // bytes 0, 1
    word = __builtin_amdgcn_cvt_pk_fp8_f32(y[4 * h + 2], y[4 * h + 3], word, true);      // bytes 2, 3
    w[h] = (uint32_t)word;
  }
  *(u32x2*)(page + (size_t)slot * kLat + 8 * lane) = u32x2{w[0], w[1]};
  if (lane < 8) {
    const u32x4 kr = *(const u32x4*)(r + kLat + 8 * lane);
    *(u32x4*)(page + kFp8RopeOff + (size_t)slot * (kRope * 2) + 16 * lane) = kr;
  }
  if (lane == 0) *(float*)(page + kFp8ScaleOff + 4 * slot) = s;
}

hipError_t launch_quant_rows_fp8(const uint16_t* src, long long n_rows, const int32_t* positions,
                                 const int32_t* block_table, int max_blocks, int t_per_seq, int num_blocks,
                                 uint8_t* pages, int32_t* status, hipStream_t st) {
  if (n_rows <= 0) return hipSuccess;
  dim3 grid((unsigned)((n_rows + kRowsPerWg - 1) / kRowsPerWg));
  hipLaunchKernelGGL(quant_rows_fp8_kernel, grid, dim3(64 * kRowsPerWg), 0, st, src, n_rows, positions, block_table,
                     max_blocks, t_per_seq, num_blocks, pages, status);
  return hipGetLastError();
}

}  // namespace mla
