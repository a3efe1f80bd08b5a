// Absorbed latent query for MLA decode on gfx950 (bf16 MFMA, fp32 accumulate).
//
// "DeepSeek-V2: Multi-Head Latent Attention (MLA) 原理与工程实现" §2.2: the query-key
// product through the up-projection, q^C . (W^UK_i c), equals (W^UK_i^T q^C) . c,
// so each head's query is moved into the d_c-wide latent space once per step:
//   q_lat[m, i, 0:512]   = W^UK_i^T q^C[m, i]     (W^UK_i = rows 128 i .. 128 i + 127 of W^UK)
//   q_lat[m, i, 512:576] = q^R[m, i]               (already rotated, §3.2)
// One workgroup per (head, 128 latent columns): the 128 x 128 slice of W^UK_i
// is staged in LDS once and used for every query row m, as a batched GEMM
// [M x 128] . [128 x 128] on MFMA 32x32x16.  The contraction runs along the
// rows of W^UK (d_h), which are strided in memory; the LDS transpose read
// (ds_read_b64_tr_b16) turns the row-major slice into the K-contiguous
// operand the MFMA needs.
//
// The last workgroup of the grid builds the split plan for the attention
// kernel (the two are independent, so the plan costs no extra launch).
#include "device_util.h"

namespace mla {

namespace {
__device__ __forceinline__ int swz(int t) { return ((t & 3) << 1) | ((t >> 2) & 1); }
__device__ __forceinline__ bf16x8 as_bf8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
}  // namespace

__global__ __launch_bounds__(256) void absorb_bf16_kernel(const uint16_t* __restrict__ q_nope,
                                                          const uint16_t* __restrict__ q_rope,
                                                          const uint16_t* __restrict__ w_uk,
                                                          const int32_t* __restrict__ seq_lens, int max_blocks,
                                                          int batch, int sq, int n_heads, uint8_t* __restrict__ ws,
                                                          WsLayout Lw, int32_t* status) {
  if (blockIdx.x == gridDim.x - 1) {
    plan_build(seq_lens, batch, sq, max_blocks, kBlk, Lw.align, Lw.W, ws, Lw, status);
    return;
  }
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kNope * 256];   // W^UK_i slice: 128 rows x 128 cols bf16
  MLA_LDS uint8_t* lds = (MLA_LDS uint8_t*)smem;
  uint16_t* q_lat = (uint16_t*)(ws + Lw.off_qlat);

  const int h = blockIdx.x >> 2;
  const int cb = blockIdx.x & 3;      // 128-column block of the latent
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int M = batch * sq;

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
  // the rotary half of the latent query is a copy
  if (cb == 0) {
    for (int i = tid; i < M * (kRope / 8); i += 256) {
      int m = i / (kRope / 8), j = i % (kRope / 8);
      *(u32x4*)(q_lat + ((size_t)m * n_heads + h) * kRow + kLat + 8 * j) =
          *(const u32x4*)(q_rope + ((size_t)m * n_heads + h) * kRope + 8 * j);
    }
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();

  // B operand (K = d, N = column): lane 16 g + 4 e + q reads row d = 16 ks + 8 hh + 4 r + e,
  // columns 32 wave + 16 (g % 2) + 4 q .. +3, which the transpose hands out as
  // 4 consecutive d of column 32 wave + (lane % 32).
  const int hh = lane >> 5;
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

  const int n = lane & 31;
  for (int mb = 0; mb * 32 < M; ++mb) {
    const int m = mb * 32 + n;
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    const uint16_t* qp = q_nope + ((size_t)m * n_heads + h) * kNope + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      u32x4 a = {0u, 0u, 0u, 0u};
      if (m < M) a = *(const u32x4*)(qp + 16 * ks);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(a), as_bf8(bop[ks]), acc, 0, 0, 0);
    }
    // D[m][col]: lane holds column 32 wave + n, rows 8 (r/4) + 4 hh + r % 4
    const int col = cb * 128 + 32 * wave + n;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      int mm = mb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
      if (mm < M) q_lat[((size_t)mm * n_heads + h) * kRow + col] = f2bf(acc[r]);
    }
  }
}

hipError_t launch_absorb_bf16(const WsLayout& L, const uint16_t* q_nope, const uint16_t* q_rope, const uint16_t* w_uk,
                              const int32_t* seq_lens, int max_blocks, int batch, int sq, int n_heads, uint8_t* ws,
                              int32_t* status, hipStream_t st) {
  dim3 grid(n_heads * 4 + 1);
  hipLaunchKernelGGL(absorb_bf16_kernel, grid, dim3(256), 0, st, q_nope, q_rope, w_uk, seq_lens, max_blocks, batch,
                     sq, n_heads, ws, L, status);
  return hipGetLastError();
}

}  // namespace mla
