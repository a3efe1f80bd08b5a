// Absorbed latent query for MLA decode on gfx950 (bf16 MFMA, fp32 accumulate).
//
// "DeepSeek-V2: Multi-Head Latent Attention (MLA) 原理与工程实现" §2.2: the query-key
// product through the up-projection, q^C . (W^UK_i c), equals (W^UK_i^T q^C) . c,
// so each head's query is moved into the d_c-wide latent space once per step:
//   q_lat[m, i, 0:512]   = s2 W^UK_i^T q^C[m, i]     (W^UK_i = rows 128 i .. 128 i + 127 of W^UK)
//   q_lat[m, i, 512:576] = s2 q^R[m, i]               (already rotated, §3.2)
// with s2 the power of two nearest to softmax scale * log2(e): the scaling is
// exact (q^R stays the caller's bf16 values up to the exponent) and the
// attention kernels apply the remaining factor, within [0.71, 1.42], in fp32.
// One workgroup per (head, 128 latent columns): the 128 x 128 slice of W^UK_i
// is staged in LDS once and used for every query row m, as a batched GEMM
// [M x 128] . [128 x 128] on MFMA 32x32x16.  The contraction runs along the
// rows of W^UK (d_h), which are strided in memory; the LDS transpose read
// (ds_read_b64_tr_b16) turns the row-major slice into the K-contiguous
// operand the MFMA needs.  The query rows of the head (256 bytes each, one
// row per n_heads * 256 bytes in memory) are contiguous along the contraction,
// so each lane loads its operand's eight features straight into registers,
// two 32-row blocks in flight at a time.  The slice (32 KB) is the only LDS:
// four workgroups fit on a CU.
//
// The first workgroup of the grid builds the split plan for the attention
// kernel (the two are independent, so the plan costs no extra launch).
#include "prep_tiles.h"

namespace mla {

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void absorb_bf16_kernel(const uint16_t* __restrict__ q_nope,
                                                          const uint16_t* __restrict__ q_rope,
                                                          const uint16_t* __restrict__ w_uk,
                                                          const int32_t* __restrict__ seq_lens, int max_blocks,
                                                          int batch, int sq, int n_heads, float qscale,
                                                          uint8_t* __restrict__ ws, WsLayout Lw, int32_t* status) {
  // block 0 builds the split plan: dispatched first, it overlaps the rest of the grid
  if (blockIdx.x == 0) {
    plan_build(seq_lens, batch, sq, max_blocks, kBlk, Lw.align, Lw.W, ws, Lw, status);
    return;
  }
  __shared__ __attribute__((aligned(1024))) uint8_t smem[prep::kAbsorbLds];
  prep::absorb_tile(q_nope, q_rope, w_uk, batch, sq, n_heads, qscale, ws, Lw, (MLA_LDS uint8_t*)smem, blockIdx.x - 1);
}

hipError_t launch_absorb_bf16(const WsLayout& L, const uint16_t* q_nope, const uint16_t* q_rope, const uint16_t* w_uk,
                              const int32_t* seq_lens, int max_blocks, int batch, int sq, int n_heads, float qscale,
                              uint8_t* ws, int32_t* status, hipStream_t st) {
  dim3 grid(n_heads * 4 + 1);
  hipLaunchKernelGGL(absorb_bf16_kernel, grid, dim3(256), 0, st, q_nope, q_rope, w_uk, seq_lens, max_blocks, batch,
                     sq, n_heads, qscale, ws, L, status);
  return hipGetLastError();
}

}  // namespace mla
