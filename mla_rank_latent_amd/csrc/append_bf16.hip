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
#include "prep_tiles.h"

namespace mla {

namespace {
__device__ __forceinline__ bf16x8 as_bf8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
constexpr int kAppendWaves = 16;

// Where token tok's row goes: its paged slot (block_table[b][pos / 64], pos % 64),
// or, with no block table, row tok of a dense [tokens][576] array (the staging
// rows the FP8 cache path quantises, which checks positions and blocks itself).
// Null, after reporting, for a position or block outside its table row.
__device__ __forceinline__ uint16_t* append_dst(uint16_t* cache, const int32_t* block_table, int max_blocks,
                                                int num_blocks, int tok, int t_per_seq, int pos, int32_t* status) {
  if (block_table == nullptr) return cache + (size_t)tok * kRow;
  if (pos < 0 || pos >= max_blocks * kBlk) {
    if (status) atomicOr(status, MLA_STATUS_BAD_POS);
    return nullptr;
  }
  const int blk = block_table[(size_t)(tok / t_per_seq) * max_blocks + pos / kBlk];
  if (blk < 0 || blk >= num_blocks) {
    if (status) atomicOr(status, MLA_STATUS_BAD_BLOCK);
    return nullptr;
  }
  return cache + ((size_t)blk * kBlk + pos % kBlk) * kRow;
}
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
      const int pos = positions[tok];
      uint16_t* dst = append_dst(cache, block_table, max_blocks, num_blocks, tok, t_per_seq, pos, status);
      if (dst == nullptr) return;
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
      dst[col] = outv;
    }
  }
}

// ---------------------------------------------------------------------------
// Split path (a caller workspace is given).  Every weight row is fetched once
// per 64 tokens: workgroup (32-column tile, 64-token group, K slice) computes
// its [64 x 32] partial product over a slice of at most kSliceSteps k-steps of
// d_model and stores it in fp32.  The slice's 96 row pieces (64 tokens of h,
// 32 weight rows) are first copied to LDS with direct-to-LDS loads, each of
// which reads 1 KB of contiguous memory (reading the MFMA operands straight
// from global memory touches 16 rows 10 KB apart per instruction, which the L1
// serves poorly).  LDS rows are padded to an odd number of 16-byte chunks, so
// the 16 rows of an operand read fall in distinct banks.  A second kernel sums
// the slices of each element in slice order (so the result does not depend on
// timing), applies RoPE to the k^R pairs and writes the bf16 rows.
// Workspace layout: [token][slice][576] fp32.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void append_partial_bf16_kernel(const uint16_t* __restrict__ h,
                                                                  const uint16_t* __restrict__ w_dkv,
                                                                  const uint16_t* __restrict__ w_kr, int tokens,
                                                                  int d_model, int nslice, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[prep::kAppendPartialLds];
  int ct, tg, sl;
  prep::append_tile_of(blockIdx.x, kRow / 32, (tokens + 63) / 64, nslice, &ct, &tg, &sl);
  prep::append_partial_tile(h, w_dkv, w_kr, tokens, d_model, nslice, part, (MLA_LDS uint8_t*)smem, ct, tg, sl);
}

__global__ __launch_bounds__(256) void append_finish_bf16_kernel(const float* __restrict__ part, int nslice,
                                                                 const int32_t* __restrict__ positions,
                                                                 const int32_t* __restrict__ block_table,
                                                                 int max_blocks, uint16_t* __restrict__ cache,
                                                                 int num_blocks, int tokens, int t_per_seq,
                                                                 double rope_base, int32_t* status) {
  // thread = (token, pair of adjacent columns): a RoPE pair for the k^R part.  The
  // position, then the first sixteen slices, are loaded first; the block-table lookup
  // (which needs the position) and the rotation angle are worked out while the slices land.
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)tokens * (kRow / 2)) return;
  const int tok = (int)(idx / (kRow / 2));
  const int col = 2 * (int)(idx % (kRow / 2));
  const float* pp = part + (size_t)tok * nslice * kRow + col;
  const int pos = positions[tok];
  float2 p[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) p[u] = *(const float2*)(pp + (size_t)(u < nslice ? u : 0) * kRow);
  uint16_t* dst = append_dst(cache, block_table, max_blocks, num_blocks, tok, t_per_seq, pos, status);
  double sn = 0.0, cs = 1.0;
  if (col >= kLat) rope_angle(pos, (col - kLat) >> 1, kRope, rope_base, &sn, &cs);
  float v0 = 0.0f, v1 = 0.0f;
#pragma unroll
  for (int u = 0; u < 16; ++u)
    if (u < nslice) {
      v0 += p[u].x;
      v1 += p[u].y;
    }
  for (int s0 = 16; s0 < nslice; s0 += 16) {
#pragma unroll
    for (int u = 0; u < 16; ++u) p[u] = *(const float2*)(pp + (size_t)(s0 + u < nslice ? s0 + u : s0) * kRow);
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (s0 + u < nslice) {
        v0 += p[u].x;
        v1 += p[u].y;
      }
  }
  if (dst == nullptr) return;
  uint32_t outv;
  if (col < kLat) {
    outv = (uint32_t)f2bf(v0) | ((uint32_t)f2bf(v1) << 16);
  } else {
    const double y0 = (double)v0 * cs - (double)v1 * sn, y1 = (double)v0 * sn + (double)v1 * cs;
    outv = (uint32_t)d2bf(y0) | ((uint32_t)d2bf(y1) << 16);
  }
  *(uint32_t*)(dst + col) = outv;
}

// ---------------------------------------------------------------------------
// Many-token path (prefill chunks): a plain GEMM [tokens x d] . [d x 576] over
// the whole d_model per workgroup, no scratch.  Workgroup = (128 tokens, 192
// columns); the h rows and weight rows stream through a 3-slot LDS ring in
// 64-feature chunks (direct-to-LDS copies, 1 KB each; 16-byte chunk c of a
// 128-byte LDS row r at c ^ ((r >> 1) & 7)).  Wave (tm, tn) accumulates tokens
// 64 tm .. +63 x columns 96 tn .. +95 on MFMA 32x32x16.  The fp32 tile is then
// staged in LDS and written as bf16 rows, the k^R pairs turned in fp64 first.
// ---------------------------------------------------------------------------
namespace {
constexpr int kGM = 128;                      // tokens per workgroup
constexpr int kGN = 192;                      // columns per workgroup (576 = 3 x 192)
constexpr int kGK = 64;                       // d_model features per chunk
constexpr int kGChunk = (kGM + kGN) * kGK * 2;   // 40 KB
constexpr int kGCopies = kGChunk / 1024 / 4;     // 10 copies of 1 KB per wave and chunk
constexpr int kGStages = 3;

__device__ __forceinline__ void dma16_row(uint64_t addr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(addr), "s"(lds_addr) : "memory");
}
__device__ __forceinline__ int gswz(int r) { return (r >> 1) & 7; }
}  // namespace

__global__ __launch_bounds__(256) void append_gemm_bf16_kernel(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ w_dkv, const uint16_t* __restrict__ w_kr,
    const int32_t* __restrict__ positions, const int32_t* __restrict__ block_table, int max_blocks,
    uint16_t* __restrict__ cache, int num_blocks, int tokens, int t_per_seq, int d_model, double rope_base,
    int32_t* status) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kGStages * kGChunk];
  MLA_LDS uint8_t* lds = (MLA_LDS uint8_t*)smem;
  const int tn = blockIdx.x % (kRow / kGN);   // the 3 column tiles of a token tile run side by side
  const int m0 = (blockIdx.x / (kRow / kGN)) * kGM;
  const int n0 = tn * kGN;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 5;
  const int n = lane & 31;

  // copy q (0..39) of a chunk: rows 8 q .. 8 q + 7 of the (h rows, weight rows)
  // stack; wave w issues copies w + 4 k.  Lane i: row 8 q + i / 8, physical chunk
  // i % 8, logical chunk (i % 8) ^ gswz(row).
  uint64_t src[kGCopies];
#pragma unroll
  for (int k = 0; k < kGCopies; ++k) {
    const int r = 8 * (wave + 4 * k) + lane / 8;
    const int lc = (lane % 8) ^ gswz(r);
    const uint16_t* rowp;
    if (r < kGM) {
      const int t = m0 + r < tokens ? m0 + r : tokens - 1;
      rowp = h + (size_t)t * d_model;
    } else {
      const int c = n0 + r - kGM;
      rowp = c < kLat ? w_dkv + (size_t)c * d_model : w_kr + (size_t)(c - kLat) * d_model;
    }
    src[k] = (uint64_t)(uintptr_t)(rowp + 8 * lc);
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
  auto issue = [&](int ch) {
    const uint32_t dst = lds0 + (ch % kGStages) * kGChunk;
#pragma unroll
    for (int k = 0; k < kGCopies; ++k)
      dma16_row(src[k] + (uint64_t)ch * (kGK * 2), __builtin_amdgcn_readfirstlane(dst + (wave + 4 * k) * 1024));
  };

  const int tm = wave >> 1, tw = wave & 1;
  f32x16 acc[2][3];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 3; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nch = d_model / kGK;
  issue(0);
  if (nch > 1) issue(1);
  for (int ch = 0; ch < nch; ++ch) {
    if (ch + 1 < nch) __builtin_amdgcn_s_waitcnt(waitcnt_vm(kGCopies));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();   // chunk ch visible to every wave; chunk ch - 1's slot free
    if (ch + 2 < nch) issue(ch + 2);
    const MLA_LDS uint8_t* buf = lds + (ch % kGStages) * kGChunk;
#pragma unroll
    for (int ks = 0; ks < kGK / 16; ++ks) {
      const int lc = 2 * ks + g;
      u32x4 a[2], b[3];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = 64 * tm + 32 * i + n;
        a[i] = *(const MLA_LDS u32x4*)(buf + r * 128 + ((lc ^ gswz(r)) << 4));
      }
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const int r = kGM + 96 * tw + 32 * j + n;
        b[j] = *(const MLA_LDS u32x4*)(buf + r * 128 + ((lc ^ gswz(r)) << 4));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(a[i]), as_bf8(b[j]), acc[i][j], 0, 0, 0);
    }
  }

  // ---- stage the fp32 tile [128 tokens][192 columns] (96 KB) and write the rows
  __syncthreads();   // every wave done with the last chunk
  MLA_LDS float* tile = (MLA_LDS float*)lds;
  // D layout: register r holds token row 8 (r / 4) + 4 g + r % 4, column n
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 3; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        tile[(64 * tm + 32 * i + 8 * (r >> 2) + 4 * g + (r & 3)) * kGN + 96 * tw + 32 * j + n] = acc[i][j][r];
  __syncthreads();
  // thread = (token, pair of adjacent columns): 128 x 96 pairs; a k^R pair is one RoPE pair
  for (int idx = tid; idx < kGM * (kGN / 2); idx += 256) {
    const int row = idx / (kGN / 2);
    const int cp = 2 * (idx % (kGN / 2));
    const int tok = m0 + row;
    if (tok >= tokens) continue;
    const float v0 = tile[row * kGN + cp], v1 = tile[row * kGN + cp + 1];
    const int col = n0 + cp;
    const int pos = positions[tok];
    uint16_t* dst = append_dst(cache, block_table, max_blocks, num_blocks, tok, t_per_seq, pos, status);
    if (dst == nullptr) continue;
    uint32_t outv;
    if (col < kLat) {
      outv = (uint32_t)f2bf(v0) | ((uint32_t)f2bf(v1) << 16);
    } else {
      double y0, y1;
      rope_pair((double)v0, (double)v1, pos, (col - kLat) >> 1, kRope, rope_base, &y0, &y1);
      outv = (uint32_t)d2bf(y0) | ((uint32_t)d2bf(y1) << 16);
    }
    *(uint32_t*)(dst + col) = outv;
  }
}

hipError_t launch_append_gemm_bf16(const uint16_t* h, const uint16_t* w_dkv, const uint16_t* w_kr,
                                   const int32_t* positions, const int32_t* block_table, int max_blocks,
                                   uint16_t* cache, int num_blocks, int tokens, int t_per_seq, int d_model,
                                   float rope_base, int32_t* status, hipStream_t st) {
  dim3 grid((unsigned)(((long long)tokens + kGM - 1) / kGM * (kRow / kGN)));
  hipLaunchKernelGGL(append_gemm_bf16_kernel, grid, dim3(256), 0, st, h, w_dkv, w_kr, positions, block_table,
                     max_blocks, cache, num_blocks, tokens, t_per_seq, d_model, (double)rope_base, status);
  return hipGetLastError();
}

int append_split_slices(int d_model) {
  const int nks = d_model / 32;
  return (nks + prep::kSliceSteps - 1) / prep::kSliceSteps;
}

size_t append_split_ws_bytes(int d_model, long long tokens) {
  return (size_t)append_split_slices(d_model) * (size_t)tokens * kRow * sizeof(float);
}

hipError_t launch_append_split_bf16(const uint16_t* h, const uint16_t* w_dkv, const uint16_t* w_kr,
                                    const int32_t* positions, const int32_t* block_table, int max_blocks,
                                    uint16_t* cache, int num_blocks, int tokens, int t_per_seq, int d_model,
                                    float rope_base, float* ws, int32_t* status, hipStream_t st) {
  const int nslice = append_split_slices(d_model);
  dim3 grid1((kRow / 32) * ((tokens + 63) / 64) * nslice);
  hipLaunchKernelGGL(append_partial_bf16_kernel, grid1, dim3(256), 0, st, h, w_dkv, w_kr, tokens, d_model, nslice,
                     ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_append_finish_bf16(ws, nslice, positions, block_table, max_blocks, cache, num_blocks, tokens,
                                   t_per_seq, rope_base, status, st);
}

hipError_t launch_append_finish_bf16(const float* part, int nslice, const int32_t* positions,
                                     const int32_t* block_table, int max_blocks, uint16_t* cache, int num_blocks,
                                     int tokens, int t_per_seq, float rope_base, int32_t* status, hipStream_t st) {
  const long long items = (long long)tokens * (kRow / 2);
  dim3 grid2((unsigned)((items + 255) / 256));
  hipLaunchKernelGGL(append_finish_bf16_kernel, grid2, dim3(256), 0, st, part, nslice, positions, block_table,
                     max_blocks, cache, num_blocks, tokens, t_per_seq, (double)rope_base, status);
  return hipGetLastError();
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
