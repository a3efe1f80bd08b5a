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
// row per n_heads * 256 bytes in memory) reach LDS in double-buffered blocks
// of 64 by direct-to-LDS copies that read four whole rows each; their 16-byte
// chunks are XOR-swizzled by row so the operand reads are free of bank
// conflicts.
//
// The first workgroup of the grid builds the split plan for the attention
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
                                                          int batch, int sq, int n_heads, float qscale,
                                                          uint8_t* __restrict__ ws, WsLayout Lw, int32_t* status) {
  // block 0 builds the split plan: dispatched first, it overlaps the rest of the grid
  if (blockIdx.x == 0) {
    plan_build(seq_lens, batch, sq, max_blocks, kBlk, Lw.align, Lw.W, ws, Lw, status);
    return;
  }
  // W^UK_i slice (128 rows x 128 cols bf16), then two 64-row blocks of query rows
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kNope * 256 + 2 * 64 * kNope * 2];
  MLA_LDS uint8_t* lds = (MLA_LDS uint8_t*)smem;
  MLA_LDS uint8_t* qbuf = lds + kNope * 256;
  uint16_t* q_lat = (uint16_t*)(ws + Lw.off_qlat);

  // (head, 128-column block of the latent): the four blocks of a head take ids 8 apart, so
  // they run on one XCD and share its L2 for the head's query rows
  const int bid = blockIdx.x - 1;
  const int full = (n_heads / 8) * 32;
  int h, cb;
  if (bid < full) {
    h = 8 * (bid / 32) + bid % 8;
    cb = (bid / 8) % 4;
  } else {
    h = (n_heads / 8) * 8 + (bid - full) / 4;
    cb = (bid - full) % 4;
  }
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int M = batch * sq;
  const int nmb = (M + 63) / 64;      // 64-row blocks of query rows

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
  // copy query-row block mb into buffer (mb & 1): LDS chunk P = 64 (wave + 4 k) + lane holds
  // row P / 16 of the block, physical chunk P % 16 = logical chunk ^ (row % 16); rows past
  // M re-read row M - 1
  auto stage_q = [&](int mb) {
    MLA_LDS uint8_t* qb = qbuf + (mb & 1) * (64 * kNope * 2);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int P = 64 * (wave + 4 * k) + lane;
      const int r = P >> 4;
      int m = mb * 64 + r;
      m = m < M ? m : M - 1;
      const int c = (P & 15) ^ (r & 15);
      const uint16_t* src = q_nope + ((size_t)m * n_heads + h) * kNope + 8 * c;
      const uint32_t dst = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(qb + (wave + 4 * k) * 1024));
      asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(dst) : "memory");
    }
  };
  stage_q(0);
  // the rotary half of the latent query: q^R times a power of two (exact)
  if (cb == 0) {
    for (int i = tid; i < M * (kRope / 8); i += 256) {
      int m = i / (kRope / 8), j = i % (kRope / 8);
      const u32x4 v = *(const u32x4*)(q_rope + ((size_t)m * n_heads + h) * kRope + 8 * j);
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o[e] = pack_bf2(bf2f((uint16_t)(v[e] & 0xffffu)) * qscale, bf2f((uint16_t)(v[e] >> 16)) * qscale);
      *(u32x4*)(q_lat + ((size_t)m * n_heads + h) * kRow + kLat + 8 * j) = o;
    }
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();

  // B operand (K = d, N = column): lane 16 g + 4 e + q reads row d = 16 ks + 8 hh + 4 r + e,
  // columns 32 wave + 16 (g % 2) + 4 q .. +3, which the transpose hands out as
  // 4 consecutive d of column 32 wave + (lane % 32).
  const int hh = lane >> 5;
  const int n = lane & 31;
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

  for (int mb = 0; mb < nmb; ++mb) {
    if (mb + 1 < nmb) stage_q(mb + 1);   // the next block lands while this one is multiplied
    const MLA_LDS uint8_t* qb = qbuf + (mb & 1) * (64 * kNope * 2);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      // A operand: lane reads query row 32 half + n of the block, d = 16 ks + 8 hh .. +7
      const int r = 32 * half + n;
      f32x16 acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const u32x4 a = *(const MLA_LDS u32x4*)(qb + r * (kNope * 2) + (((2 * ks + hh) ^ (r & 15)) * 16));
        // operands in swapped roles: the product is D^T, [column x query row]
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(bop[ks]), as_bf8(a), acc, 0, 0, 0);
      }
      // D^T: lane holds query row 32 half + n, columns 32 wave + 8 (i/4) + 4 hh + i % 4, so
      // each group of four registers is four adjacent columns: one 8-byte store
      const int mm = mb * 64 + 32 * half + n;
      if (mm < M) {
        uint16_t* dst = q_lat + ((size_t)mm * n_heads + h) * kRow + cb * 128 + 32 * wave + 4 * hh;
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *(u32x2*)(dst + 8 * g) = u32x2{pack_bf2(acc[4 * g] * qscale, acc[4 * g + 1] * qscale),
                                          pack_bf2(acc[4 * g + 2] * qscale, acc[4 * g + 3] * qscale)};
      }
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));   // next block landed (and this block's stores issued)
    __syncthreads();                              // ... for every wave; this block's buffer is free
  }
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
