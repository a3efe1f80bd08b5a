// Projections of the full MLA layer for a few query rows, gfx950 bf16 MFMA with
// fp32 accumulation: y = x W^T with x [M, K] (M = batch * query tokens, small)
// and W [N, K] (out x in), the layout the weights are given in.
//   c^Q = W^DQ h                         ("DeepSeek-V2: Multi-Head Latent Attention
//                                          (MLA) 原理与工程实现" §2.3, query compression)
//   q^C = W^UQ c^Q, q^R = RoPE(W^QR c^Q) ("【深度学习】DeepSeek焦点架构-MLA" 02 (5))
//   u   = W^O [o_1; ...; o_{n_h}]        (same, 02 (5): the heads' outputs, concatenated,
//                                          through one linear map)
// With so few rows the weights dominate the bytes: the kernel streams them once.
// W may be two stacked matrices (q^C and q^R come from [W^UQ; W^QR] in one pass).
// proj_partial_bf16_kernel: workgroup (64-row tile, 64-column tile, K split);
//   the x rows and W rows of the split stream through a 3-slot LDS ring in
//   64-feature chunks (direct-to-LDS copies of 1 KB, 16-byte chunk c of a
//   128-byte LDS row r at c ^ ((r >> 1) & 7)); wave (mh, nh) accumulates rows
//   32 mh .. +31 x columns 32 nh .. +31 on MFMA 32x32x16.  Split over K, it
//   stores its fp32 partial; unsplit (enough column tiles to fill the chip),
//   it writes bf16 itself, taking a rotary pair's partner from the next lane.
// proj_finish_bf16_kernel: sums the splits of each element in split order (so
//   the result does not depend on timing) and writes bf16.
// Columns at or past `rope_from` are the rotary query: pairs (2j, 2j + 1) of
// each 64-wide head turn by angle pos * base^(-2j/64) in fp64 before rounding.
#include "device_util.h"

namespace mla {

namespace {
__device__ __forceinline__ bf16x8 as_bf8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
constexpr int kPT = 64;                       // rows and columns per tile
constexpr int kPK = 64;                       // features per chunk
constexpr int kPChunk = 2 * kPT * kPK * 2;    // 16 KB: x rows then W rows
constexpr int kPCopies = kPChunk / 1024 / 4;  // 4 copies of 1 KB per wave and chunk
constexpr int kPStages = 3;

__device__ __forceinline__ void dma16_at(uint64_t addr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(addr), "s"(lds_addr) : "memory");
}
__device__ __forceinline__ int pswz(int r) { return (r >> 1) & 7; }
}  // namespace

struct ProjOut {               // direct bf16 output (one split): columns < rope_from -> y0, the rest -> y1
  uint16_t* y0;
  int ld0;
  uint16_t* y1;
  int ld1;
  int rope_from, rope_width;
  const int32_t* positions;
  double rope_base;
};

__global__ __launch_bounds__(256) void proj_partial_bf16_kernel(const uint16_t* __restrict__ x,
                                                                const uint16_t* __restrict__ w0,
                                                                const uint16_t* __restrict__ w1, int n_w0, int M,
                                                                int N, int K, int splits, int chunks_per_split,
                                                                float* __restrict__ part, ProjOut po) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kPStages * kPChunk];
  MLA_LDS uint8_t* lds = (MLA_LDS uint8_t*)smem;
  const int n_tiles = N / kPT;
  // column tiles fastest, then splits: consecutive workgroups read different weight rows
  const int nt = blockIdx.x % n_tiles;
  const int sp = (blockIdx.x / n_tiles) % splits;
  const int mt = blockIdx.x / (n_tiles * splits);
  const int m0 = mt * kPT, n0 = nt * kPT;
  const int ch0 = sp * chunks_per_split;
  const int nch = min(chunks_per_split, K / kPK - ch0);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 5, n = lane & 31;

  // copy q (0..15) of a chunk: rows 8 q .. 8 q + 7 of the (x rows, W rows) stack;
  // wave w issues copies w + 4 k.  Rows of x past M repeat row M - 1.
  uint64_t src[kPCopies];
#pragma unroll
  for (int k = 0; k < kPCopies; ++k) {
    const int r = 8 * (wave + 4 * k) + lane / 8;
    const int lc = (lane % 8) ^ pswz(r);
    const uint16_t* rowp;
    if (r < kPT) {
      const int m = m0 + r < M ? m0 + r : M - 1;
      rowp = x + (size_t)m * K;
    } else {
      // weight row n: rows of w0 below n_w0, of w1 from there (a 64-column tile never straddles)
      const int nn = n0 + r - kPT;
      rowp = nn < n_w0 ? w0 + (size_t)nn * K : w1 + (size_t)(nn - n_w0) * K;
    }
    src[k] = (uint64_t)(uintptr_t)(rowp + (size_t)ch0 * kPK + 8 * lc);
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
  auto issue = [&](int c) {
    const uint32_t dst = lds0 + (c % kPStages) * kPChunk;
#pragma unroll
    for (int k = 0; k < kPCopies; ++k)
      dma16_at(src[k] + (uint64_t)c * (kPK * 2), __builtin_amdgcn_readfirstlane(dst + (wave + 4 * k) * 1024));
  };

  const int mh = wave >> 1, nh = wave & 1;
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
  if (nch > 0) issue(0);
  if (nch > 1) issue(1);
  for (int c = 0; c < nch; ++c) {
    if (c + 1 < nch) __builtin_amdgcn_s_waitcnt(waitcnt_vm(kPCopies));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();   // chunk c visible to every wave; chunk c - 1's slot free
    if (c + 2 < nch) issue(c + 2);
    const MLA_LDS uint8_t* buf = lds + (c % kPStages) * kPChunk;
#pragma unroll
    for (int ks = 0; ks < kPK / 16; ++ks) {
      const int lc = 2 * ks + g;
      const int ra = 32 * mh + n, rb = kPT + 32 * nh + n;
      const u32x4 a = *(const MLA_LDS u32x4*)(buf + ra * 128 + ((lc ^ pswz(ra)) << 4));
      const u32x4 b = *(const MLA_LDS u32x4*)(buf + rb * 128 + ((lc ^ pswz(rb)) << 4));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(a), as_bf8(b), acc, 0, 0, 0);
    }
  }
  // D layout: register r holds row 8 (r / 4) + 4 g + r % 4, column n
  const int col = n0 + 32 * nh + n;
  if (splits > 1) {   // fp32 partial [split][M][N], summed by proj_finish_bf16_kernel
    float* pp = part + ((size_t)sp * M) * N;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + 32 * mh + 8 * (r >> 2) + 4 * g + (r & 3);
      if (m < M) pp[(size_t)m * N + col] = acc[r];
    }
    return;
  }
  if (n0 < po.rope_from) {   // a plain tile (tiles never straddle rope_from: both are multiples of 64)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + 32 * mh + 8 * (r >> 2) + 4 * g + (r & 3);
      if (m < M) po.y0[(size_t)m * po.ld0 + col] = f2bf(acc[r]);
    }
    return;
  }
  // a rotary tile: the partner of column n's pair sits in lane n ^ 1 (DPP quad_perm [1, 0, 3, 2])
  const int c = col - po.rope_from;
  const int j = (c % po.rope_width) >> 1;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float mine = acc[r];
    const float other = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(mine), 0xB1, 0xF, 0xF, false));
    const int m = m0 + 32 * mh + 8 * (r >> 2) + 4 * g + (r & 3);
    if (m < M) {
      const double x0 = (c & 1) ? other : mine, x1 = (c & 1) ? mine : other;
      double y0, y1;
      rope_pair(x0, x1, po.positions[m], j, po.rope_width, po.rope_base, &y0, &y1);
      po.y1[(size_t)m * po.ld1 + c] = d2bf((c & 1) ? y1 : y0);
    }
  }
}

__global__ __launch_bounds__(256) void proj_finish_bf16_kernel(const float* __restrict__ part, int M, int N,
                                                               int splits, int rope_from, int rope_width,
                                                               const int32_t* __restrict__ positions,
                                                               double rope_base, uint16_t* __restrict__ y0,
                                                               int ld0, uint16_t* __restrict__ y1, int ld1) {
  // thread = (row, pair of adjacent columns); columns < rope_from go to y0 (row stride ld0),
  // the rest to y1 (row stride ld1) with their pairs turned
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)M * (N / 2)) return;
  const int m = (int)(idx / (N / 2));
  const int col = 2 * (int)(idx % (N / 2));
  const size_t stride = (size_t)M * N;
  const float* p = part + (size_t)m * N + col;
  float v0 = 0.0f, v1 = 0.0f;
  for (int s = 0; s < splits; ++s) {
    const float2 t = *(const float2*)(p + s * stride);
    v0 += t.x;
    v1 += t.y;
  }
  if (col < rope_from) {
    *(uint32_t*)(y0 + (size_t)m * ld0 + col) = (uint32_t)f2bf(v0) | ((uint32_t)f2bf(v1) << 16);
  } else {
    const int c = col - rope_from;
    double r0, r1;
    rope_pair((double)v0, (double)v1, positions[m], (c % rope_width) >> 1, rope_width, rope_base, &r0, &r1);
    *(uint32_t*)(y1 + (size_t)m * ld1 + c) = (uint32_t)d2bf(r0) | ((uint32_t)d2bf(r1) << 16);
  }
}

// splits of K (in 64-feature chunks) so that about 256 workgroups run, each with at least 4 chunks;
// with 256 tiles or more a projection runs unsplit and writes bf16 directly
int proj_splits(int M, int N, int K) {
  const long long tiles = (long long)((M + kPT - 1) / kPT) * (N / kPT);
  const int chunks = K / kPK;
  long long s = (256 + tiles - 1) / tiles;
  const int max_s = chunks / 4 > 0 ? chunks / 4 : 1;
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  return (int)s;
}

size_t proj_ws_bytes(int M, int N, int K) {
  const int s = proj_splits(M, N, K);
  return s > 1 ? (size_t)s * M * N * sizeof(float) : 0;
}

// y = x W^T with W = [w0 (n_w0 rows); w1] (+ RoPE on columns >= rope_from, written to y1);
// N, n_w0, rope_from and K multiples of 64
hipError_t launch_proj_bf16(const uint16_t* x, const uint16_t* w0, const uint16_t* w1, int n_w0, int M, int N, int K,
                            float* part, int rope_from, int rope_width, const int32_t* positions, float rope_base,
                            uint16_t* y0, int ld0, uint16_t* y1, int ld1, hipStream_t st) {
  const int splits = proj_splits(M, N, K);
  const int chunks = K / kPK;
  const int cps = (chunks + splits - 1) / splits;
  const long long tiles = (long long)((M + kPT - 1) / kPT) * (N / kPT);
  const ProjOut po{y0, ld0, y1, ld1, rope_from, rope_width, positions, (double)rope_base};
  hipLaunchKernelGGL(proj_partial_bf16_kernel, dim3((unsigned)(tiles * splits)), dim3(256), 0, st, x, w0, w1, n_w0, M,
                     N, K, splits, cps, part, po);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  const long long items = (long long)M * (N / 2);
  hipLaunchKernelGGL(proj_finish_bf16_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, st,
                     (const float*)part, M, N, splits, rope_from, rope_width, positions, (double)rope_base, y0, ld0,
                     y1, ld1);
  return hipGetLastError();
}

}  // namespace mla
