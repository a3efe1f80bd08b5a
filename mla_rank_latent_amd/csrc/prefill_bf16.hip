// Prefill in expanded form on gfx950: decompress every context token's per-head
// key and value, then causal flash attention over them, bf16 MFMA with fp32
// accumulation.
//
// Prefill is the attention of decode for a query group of T tokens: the last T
// tokens of each sequence, query s at position L - T + s seeing tokens
// 0 .. L - T + s.  With many queries per cached token the expanded form is the
// cheaper one ("DeepSeek-V2: Multi-Head Latent Attention (MLA) 原理与工程实现"
// §2.1: per head i, k^C_{j,i} = W^UK_i c_j and v_{j,i} = W^UV_i c_j; §3.2:
// k_{j,i} = [k^C_{j,i} ‖ k^R_j], q_{s,i} = [q^C_{s,i} ‖ q^R_{s,i}]): scores over
// 192 features and values of 128 per head, instead of 576 and 512 in the
// absorbed form, for one decompression GEMM per token and head.
//
// Workspace (per sequence b and head h, t_ctx = max_blocks * 64 token slots):
//   kc [B][H][t_ctx][128] bf16   K^C, token-major;
//   vt [B][H][128][t_ctx] bf16   V transposed, dimension-major, with the token
//                                order inside every group of 16 permuted by
//                                swapping index bits 2 and 3.
// The permutation matches the order in which a 32x32x16 MFMA leaves the scores
// of 16 consecutive tokens in a lane (4 at offset 4g, 4 at offset 8 + 4g for
// lane half g), so the softmax weights feed the value product straight from
// the score registers and its operand is one contiguous 16-byte read.
//
// expand_kv_bf16_kernel: one workgroup (4 waves) per (sequence, 128-token
//   tile, head).  The tile's latent rows and the head's W^UK and W^UV rows go
//   to LDS in 64-feature chunks (direct-to-LDS copies, double-buffered); wave
//   w computes a 64 x 64 quadrant of K^C^T = W^UK_h c^T and of V = c W^UV_h^T,
//   whose MFMA result layout gives each lane 4 consecutive elements of the
//   stored row.  Rows past the sequence end repeat its last token (finite
//   values for the attention's last, partly masked key tile).
// prefill_attn_bf16_kernel: one workgroup (8 waves, two per SIMD) per
//   (sequence, head, 256 query rows); wave w owns 32 rows.  Key tiles of 64
//   tokens (one cache block: K^C rows, k^R rows from the cache, V^T rows)
//   stream through a 3-slot LDS ring, two tiles in flight.  Online softmax in
//   log2 units with a lazy reference: O and l are rescaled only when a row's
//   maximum grows by more than 2^8, so weights stay below 2^8 and the result
//   is exact either way.
#include "device_util.h"

namespace mla {

namespace {

__device__ __forceinline__ bf16x8 as_bf8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// a wave-uniform 64-bit address, made visibly uniform (scalar registers)
__device__ __forceinline__ uint64_t uniform_addr64(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// 16 bytes per lane from base + voff into LDS at lds_addr + 16 * lane
__device__ __forceinline__ void dma16(uint64_t base, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(lds_addr)
               : "memory");
}

// 16 bytes per lane from a per-lane 64-bit address into LDS at lds_addr + 16 * lane
__device__ __forceinline__ void dma16_v(uint64_t addr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(addr), "s"(lds_addr) : "memory");
}

__device__ __forceinline__ u32x4 lds16(const MLA_LDS uint8_t* p) { return *(const MLA_LDS u32x4*)p; }

// read-only tables through the constant address space: wave-uniform lookups
// become scalar loads, counted by lgkmcnt rather than with the tile copies
template <typename T>
__device__ __forceinline__ const __attribute__((address_space(4))) T* scalar_ptr(const T* p) {
  return (const __attribute__((address_space(4))) T*)p;
}

__device__ __forceinline__ int valid_block(int blk, int num_blocks, int32_t* status) {
  if (blk < 0 || blk >= num_blocks) {
    if (status) atomicOr(status, MLA_STATUS_BAD_BLOCK);
    return 0;
  }
  return blk;
}

// stored position of token t in a V^T row: bits 2 and 3 swapped
__device__ __forceinline__ int vt_pos(int t) { return (t & ~12) | ((t & 4) << 1) | ((t & 8) >> 1); }

// ---- expansion ---------------------------------------------------------------
constexpr int kXTok = 128;                        // tokens per workgroup
constexpr int kXK = 32;                           // latent features per chunk
constexpr int kXRow = kXK * 2;                    // 64 B per row and chunk
constexpr int kXRegion = 128 * kXRow;             // 8 KB: 128 rows
constexpr int kXChunk = 3 * kXRegion;             // latent rows, W^UK_h rows, W^UV_h rows
constexpr int kXCopies = kXChunk / 1024 / 4;      // 1 KB copies per wave per chunk (6)
constexpr int kXChunks = kLat / kXK;              // 16
constexpr int kXStages = 3;                       // LDS ring depth: two chunks in flight (72 KB,
                                                  // so two workgroups fit on a CU)

// LDS rows of 128 B: 16-byte chunk c of row r sits at c ^ ((r >> 1) & 7), so the
// 16 rows read by 16 lanes at one logical chunk cover all banks
__device__ __forceinline__ int swz128(int r) { return (r >> 1) & 7; }
// LDS rows of 64 B: chunk c of row r at c ^ ((r >> 2) & 3), for the same reason
__device__ __forceinline__ int swz64(int r) { return (r >> 2) & 3; }

// ---- attention -----------------------------------------------------------------
constexpr int kFWaves = 8;
constexpr int kFQ = 32 * kFWaves;                 // query rows per workgroup
constexpr int kFKT = 64;                          // key tokens per stage
constexpr int kFKc = kFKT * kNope * 2;            // 16 KB: K^C rows of 256 B
constexpr int kFKr = kFKT * kRope * 2;            // 8 KB: k^R rows of 128 B
constexpr int kFVt = kNope * kFKT * 2;            // 16 KB: V^T rows of 128 B
constexpr int kFStage = kFKc + kFKr + kFVt;       // 40 KB
constexpr int kFSlots = 3;
constexpr int kFCopies = kFStage / 1024 / kFWaves;   // 5
constexpr float kFTau = 8.0f;                     // lazy-rescale threshold (log2 units)

}  // namespace

__global__ __launch_bounds__(256, 2) void expand_kv_bf16_kernel(
    const uint16_t* __restrict__ cache, int num_blocks, const int32_t* __restrict__ block_table, int max_blocks,
    const int32_t* __restrict__ seq_lens, int batch, int n_heads, int t_ctx, int n_tiles,
    const uint16_t* __restrict__ w_uk,
    const uint16_t* __restrict__ w_uv, uint16_t* __restrict__ kc, uint16_t* __restrict__ vt,
    int32_t* __restrict__ status) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kXStages * kXChunk];
  MLA_LDS uint8_t* lds = (MLA_LDS uint8_t*)smem;

  // Workgroup i runs on XCD x = i % 8 (the i / 8-th there).  Each XCD takes the
  // heads h = x mod 8 and works through sets of 4 of its heads x 8 token tiles,
  // so that the 32 workgroups it holds at a time share 4 heads' weights and 8
  // latent tiles (about 2 MB) in its L2.
  const int x = blockIdx.x & 7;
  const int jx = blockIdx.x >> 3;
  const int n_bt = batch * n_tiles;
  const int n_tg = (n_bt + 7) / 8;
  const int inner = jx & 31, outer = jx >> 5;
  const int h = x + 8 * (4 * (outer / n_tg) + (inner >> 3));
  const int bt = 8 * (outer % n_tg) + (inner & 7);
  if (h >= n_heads || bt >= n_bt) return;
  const int tile = bt % n_tiles;
  const int b = bt / n_tiles;
  int L = seq_lens[b];
  L = L < 0 ? 0 : (L > t_ctx ? t_ctx : L);
  const int t0 = tile * kXTok;
  if (t0 >= L) return;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 5;
  const int n = lane & 31;

  // copy plan: copy q (0..23) of a chunk moves region q / 8, rows 16 (q % 8) .. +15;
  // lane i lands at row 16 (q % 8) + i / 4, physical chunk i % 4, and fetches the
  // logical chunk (i % 4) ^ swz64(row).  Wave w issues copies w + 4 k.
  uint64_t src[kXCopies];
#pragma unroll
  for (int k = 0; k < kXCopies; ++k) {
    const int q = wave + 4 * k;
    const int region = q / 8;
    const int r = 16 * (q % 8) + lane / 4;
    const int lc = (lane % 4) ^ swz64(r);
    const uint8_t* rowp;
    if (region == 0) {
      int t = t0 + r;
      t = t < L ? t : L - 1;
      const int blk = valid_block(block_table[(size_t)b * max_blocks + t / kBlk], num_blocks, status);
      rowp = (const uint8_t*)(cache + ((size_t)blk * kBlk + t % kBlk) * kRow);
    } else {
      const uint16_t* w = region == 1 ? w_uk : w_uv;
      rowp = (const uint8_t*)(w + ((size_t)h * kNope + r) * kLat);
    }
    src[k] = (uint64_t)(uintptr_t)(rowp + lc * 16);
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
  auto issue = [&](int ch) {
    const uint32_t dst = lds0 + (ch % kXStages) * kXChunk;
#pragma unroll
    for (int k = 0; k < kXCopies; ++k)
      dma16_v(src[k] + (uint64_t)ch * kXRow, __builtin_amdgcn_readfirstlane(dst + (wave + 4 * k) * 1024));
  };

  const int tq = wave >> 1;    // token quadrant: tokens 64 tq .. +63
  const int dq = wave & 1;     // feature quadrant: d 64 dq .. +63
  f32x16 acck[2][2], accv[2][2];   // acck[tj][ti]: K^C^T (d x tok); accv[ti][tj]: V (tok x d)
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acck[i][j][r] = accv[i][j][r] = 0.0f;

  issue(0);
  issue(1);
  for (int ch = 0; ch < kXChunks; ++ch) {
    // chunk ch has landed once at most chunk ch + 1's copies are in flight
    if (ch + 1 < kXChunks) __builtin_amdgcn_s_waitcnt(waitcnt_vm(kXCopies));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();   // chunk ch visible to every wave; chunk ch - 1's buffer free
    if (ch + 2 < kXChunks) issue(ch + 2);
    const MLA_LDS uint8_t* buf = lds + (ch % kXStages) * kXChunk;
#pragma unroll
    for (int ks = 0; ks < kXK / 16; ++ks) {
      const int lc = 2 * ks + g;
      u32x4 cop[2], kop[2], vop[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int rc = 64 * tq + 32 * i + n;
        const int rw = 64 * dq + 32 * i + n;
        cop[i] = lds16(buf + rc * kXRow + ((lc ^ swz64(rc)) << 4));
        kop[i] = lds16(buf + kXRegion + rw * kXRow + ((lc ^ swz64(rw)) << 4));
        vop[i] = lds16(buf + 2 * kXRegion + rw * kXRow + ((lc ^ swz64(rw)) << 4));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acck[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(kop[i]), as_bf8(cop[j]), acck[i][j], 0, 0, 0);
          accv[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(cop[i]), as_bf8(vop[j]), accv[i][j], 0, 0, 0);
        }
    }
  }

  // D layout of 32x32x16: register r holds row 8 (r / 4) + 4 g + r % 4, column n,
  // so each lane holds 4 consecutive elements of a stored row per (tile, r / 4).
  // Both 128 x 128 result tiles are staged in LDS (rows of 256 B, 16-byte chunk c
  // of row x at c ^ (x & 15)) and written out as whole rows, 16 bytes per lane.
  __syncthreads();   // every wave done with the last chunk
  MLA_LDS uint8_t* sk = lds;                  // K^C tile: row = token, 128 features
  MLA_LDS uint8_t* sv = lds + 128 * 256;      // V^T tile: row = feature, 128 stored token slots
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        {
          const int d = 64 * dq + 32 * i + 8 * q + 4 * g;     // 4 consecutive features
          const int tok = 64 * tq + 32 * j + n;
          const u32x2 v = {pack_bf2(acck[i][j][4 * q], acck[i][j][4 * q + 1]),
                           pack_bf2(acck[i][j][4 * q + 2], acck[i][j][4 * q + 3])};
          *(MLA_LDS u32x2*)(sk + tok * 256 + (((d >> 3) ^ (tok & 15)) << 4) + (d & 4) * 2) = v;
        }
        {
          const int tok = vt_pos(64 * tq + 32 * i + 8 * q + 4 * g);   // 4 consecutive tokens
          const int d = 64 * dq + 32 * j + n;
          const u32x2 v = {pack_bf2(accv[i][j][4 * q], accv[i][j][4 * q + 1]),
                           pack_bf2(accv[i][j][4 * q + 2], accv[i][j][4 * q + 3])};
          *(MLA_LDS u32x2*)(sv + d * 256 + (((tok >> 3) ^ (d & 15)) << 4) + (tok & 4) * 2) = v;
        }
      }
  __syncthreads();
  const size_t bh = (size_t)b * n_heads + h;
  uint16_t* kc_bh = kc + bh * t_ctx * kNope;
  uint16_t* vt_bh = vt + bh * kNope * (size_t)t_ctx;
  // 128 rows x 16 chunks per tile; thread tid takes chunk tid % 16 of rows tid / 16 + 16 k.
  // With an odd max_blocks the tile reaches 64 slots past t_ctx: those are not stored.
  const int c = tid & 15;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int x = (tid >> 4) + 16 * k;
    const u32x4 vk = lds16(sk + x * 256 + ((c ^ (x & 15)) << 4));
    if (t0 + x < t_ctx) *(u32x4*)(kc_bh + (size_t)(t0 + x) * kNope + 8 * c) = vk;
    const u32x4 vv = lds16(sv + x * 256 + ((c ^ (x & 15)) << 4));
    if (t0 + 8 * c < t_ctx) *(u32x4*)(vt_bh + (size_t)x * t_ctx + t0 + 8 * c) = vv;
  }
}

__global__ __launch_bounds__(512) void prefill_attn_bf16_kernel(
    const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_rope, const uint16_t* __restrict__ cache,
    int num_blocks, const int32_t* __restrict__ block_table, int max_blocks, const int32_t* __restrict__ seq_lens,
    int batch, int T, int n_heads, int t_ctx, int nqt, float scale_log2, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vt, uint16_t* __restrict__ out, float* __restrict__ lse,
    int32_t* __restrict__ status) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kFSlots * kFStage + 1024];
  MLA_LDS uint8_t* lds = (MLA_LDS uint8_t*)smem;

  // Workgroup i runs on XCD i % 8; the query tiles of one (sequence, head) go to
  // one XCD, longest first, so they share its L2 for their keys and values.
  const int x = blockIdx.x & 7;
  const int jj = blockIdx.x >> 3;
  const int grp = 8 * (jj / nqt) + x;
  const int qt = nqt - 1 - jj % nqt;
  if (grp >= batch * n_heads) return;
  const int b = grp / n_heads;
  const int h = grp - b * n_heads;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 5;
  const int n = lane & 31;

  const auto btab = scalar_ptr(block_table);
  const int cap = max_blocks * kBlk;
  int L = scalar_ptr(seq_lens)[b];
  if (L < T || L > cap) {
    if (h == 0 && qt == nqt - 1 && tid == 0 && status) atomicOr(status, MLA_STATUS_BAD_LENGTH);
    L = L < 0 ? 0 : (L > cap ? cap : L);
  }
  const int s0 = qt * kFQ;
  const int s = s0 + 32 * wave + n;                 // this lane's query row
  const bool row_ok = s < T;
  const int pos = L - T + s;                        // its position; it sees keys 0 .. pos
  const int last_s = (s0 + kFQ - 1 < T - 1) ? s0 + kFQ - 1 : T - 1;
  const int kmax = L - T + last_s;                  // the workgroup's last visible key
  // this wave's last visible key (-1: no valid row or no key)
  const int ws0 = s0 + 32 * wave;
  const int kmax_w = ws0 < T ? L - T + ((ws0 + 31 < T - 1) ? ws0 + 31 : T - 1) : -1;
  const int pos_first = L - T + ws0;                // the wave's first row position
  const int nkt = kmax >= 0 ? kmax / kFKT + 1 : 0;

  // ---- queries: B operand of S^T = K Q^T; lane holds row n, features 16 ks + 8 g .. +7
  u32x4 qreg[12];
  {
    const size_t qrow = ((size_t)b * T + (row_ok ? s : 0)) * n_heads + h;
    const uint16_t* qn = q_nope + qrow * kNope + 8 * g;
    const uint16_t* qr = q_rope + qrow * kRope + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qreg[ks] = row_ok ? *(const u32x4*)(qn + 16 * ks) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qreg[8 + ks] = row_ok ? *(const u32x4*)(qr + 16 * ks) : u32x4{0u, 0u, 0u, 0u};
  }

  // ---- copy plan.  Wave w issues copies w + 8 k (k = 0..4) of a stage: 0-15 K^C
  // rows (4 rows of 256 B per copy), 16-23 k^R rows, 24-39 V^T rows (8 rows of
  // 128 B per copy).  K^C chunk c of row r sits at c ^ (r & 15); k^R and V^T
  // chunks at c ^ swz128(r).
  const size_t bh = (size_t)b * n_heads + h;
  const uint16_t* kc_bh = kc + bh * t_ctx * kNope;
  const uint16_t* vt_bh = vt + bh * kNope * (size_t)t_ctx;
  uint32_t voff_k[2], voff_v[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int q = wave + 8 * k;                       // 0..15
    const int r = 4 * q + lane / 16;
    voff_k[k] = (uint32_t)(r * 256 + (((lane % 16) ^ (r & 15)) << 4));
    const int d = 8 * (q) + lane / 8;                 // V^T copies 24 + q: rows 8 q .. +7
    voff_v[k] = (uint32_t)((size_t)d * t_ctx * 2 + (((lane % 8) ^ swz128(d)) << 4));
  }
  const int rr = 8 * wave + lane / 8;                 // k^R copy 16 + w: rows 8 w .. +7
  const int rr_lc = (lane % 8) ^ swz128(rr);
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
  const uint64_t idle_base = uniform_addr64(cache);
  const uint32_t idle_dst = lds0 + kFSlots * kFStage;

  auto issue = [&](int kt) {
    const uint32_t dst = lds0 + (kt % kFSlots) * kFStage;
    const int t0 = kt * kFKT;
    const uint64_t bk = uniform_addr64(kc_bh + (size_t)t0 * kNope);
    const uint64_t bv = uniform_addr64(vt_bh + t0);
    // a scalar load: a vector load here would make the compiler wait for every copy in flight
    const int blk = valid_block(btab[(size_t)b * max_blocks + t0 / kBlk], num_blocks, status);
    const uint64_t br = uniform_addr64(cache + (size_t)blk * kBlk * kRow);
    int t = t0 + rr;
    t = t < L ? t : L - 1;
    const uint32_t voff_r = (uint32_t)((t % kBlk) * (kRow * 2) + kLat * 2 + (rr_lc << 4));
#pragma unroll
    for (int k = 0; k < 2; ++k) dma16(bk, voff_k[k], __builtin_amdgcn_readfirstlane(dst + (wave + 8 * k) * 1024));
    dma16(br, voff_r, __builtin_amdgcn_readfirstlane(dst + (16 + wave) * 1024));
#pragma unroll
    for (int k = 0; k < 2; ++k)
      dma16(bv, voff_v[k], __builtin_amdgcn_readfirstlane(dst + (24 + wave + 8 * k) * 1024));
  };
  auto issue_idle = [&]() {
#pragma unroll
    for (int k = 0; k < kFCopies; ++k) dma16(idle_base, (uint32_t)(lane * 16), idle_dst);
  };

  // the query loads are complete before the copies start, so no later wait
  // has to count them
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  if (nkt > 0) issue(0); else issue_idle();
  if (nkt > 1) issue(1); else issue_idle();

  float m_ref = -__builtin_inff();   // row reference maximum (log2 units)
  float l_sum = 0.0f;                // this lane's share of sum_j p_j
  f32x16 acc_o[4];                   // O^T: 128 features x 32 rows, 4 tiles
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[i][r] = 0.0f;

  for (int kt = 0; kt < nkt; ++kt) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(kFCopies));   // stage kt landed (kt + 1 may be in flight)
    __syncthreads();                                     // ... for every wave; stage kt - 1 consumed
    if (kt + 2 < nkt) issue(kt + 2); else issue_idle();
    if (kt * kFKT > kmax_w) continue;                    // every row of this wave precedes the tile
    const MLA_LDS uint8_t* st = lds + (kt % kFSlots) * kFStage;

    // ---- S^T = K . Q^T: two 32-token tiles, 12 k-steps (8 over K^C, 4 over k^R)
    f32x16 acc_s[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_s[i][r] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 12; ++ks) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = 32 * i + n;
        u32x4 a;
        if (ks < 8) a = lds16(st + row * 256 + (((2 * ks + g) ^ (row & 15)) << 4));
        else a = lds16(st + kFKc + row * 128 + (((2 * (ks - 8) + g) ^ swz128(row)) << 4));
        acc_s[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(a), as_bf8(qreg[ks]), acc_s[i], 0, 0, 0);
      }
    }

    // ---- softmax.  Lane holds row n, tokens 64 kt + 32 i + 8 (r / 4) + 4 g + r % 4.
    // The maximum is taken on the raw scores (the scale is positive) and the scale
    // enters the exponent's fma, so z = scale * s is never formed on its own.
    f32x16* sv = acc_s;   // masked in place
    if (kt * kFKT + kFKT - 1 > pos_first) {
      // a diagonal tile (some key follows some row of this wave): token offset
      // 32 i + 8 (r / 4) + r % 4 is masked when it exceeds thr.  The empty asm keeps
      // this a branch: if-converted, its selects would run on every tile.
      asm volatile("");
      const int thr = pos - kt * kFKT - 4 * g;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          sv[i][r] = (32 * i + 8 * (r >> 2) + (r & 3) > thr) ? -__builtin_inff() : sv[i][r];
    }
    float mt = sv[0][0];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sv[i][r]);
    {
      // lanes l and l ^ 32 hold the two token halves of row n
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
      mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * scale_log2;
    }
    const bool resc = mt > m_ref + kFTau;   // false while the row has seen only masked keys
    if (__builtin_amdgcn_ballot_w64(resc) != 0ull) {
      asm volatile("");   // a branch, not 64 multiplies by 1 on every tile
      const float f = resc ? __builtin_amdgcn_exp2f(m_ref - mt) : 1.0f;   // 0 on the first finite tile
      l_sum *= f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[i][r] *= f;
      m_ref = resc ? mt : m_ref;
    }
    const float neg_m = m_ref == -__builtin_inff() ? 0.0f : -m_ref;
    u32x4 pk[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int i = kk >> 1, hb = 8 * (kk & 1);
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[i][hb + e], scale_log2, neg_m));
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = pack_bf2(p[2 * e], p[2 * e + 1]);
      // the weight sum of the rounded weights the value product uses, two per dot2
      // (from the packed words themselves, not from elements of the vector below)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        l_sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[e]),
                                                __builtin_bit_cast(bf16x2, 0x3f803f80u), l_sum, false);
      pk[kk] = u32x4{w[0], w[1], w[2], w[3]};
    }

    // ---- O^T += V^T . P^T: 4 feature tiles x 4 token k-steps
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int di = 0; di < 4; ++di) {
        const int d = 32 * di + n;
        const u32x4 a = lds16(st + kFKc + kFKr + d * 128 + (((2 * kk + g) ^ swz128(d)) << 4));
        acc_o[di] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(a), as_bf8(pk[kk]), acc_o[di], 0, 0, 0);
      }
  }

  // ---- epilogue: normalise, stage each wave's 32 x 128 block through LDS, store rows
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_sum), __float_as_uint(l_sum), false, false);
    l_sum = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  const float inv = l_sum > 0.0f ? 1.0f / l_sum : 0.0f;
  if (g == 0 && row_ok && lse != nullptr)
    lse[((size_t)b * T + s) * n_heads + h] =
        l_sum > 0.0f ? (m_ref + __builtin_amdgcn_logf(l_sum)) * 0.69314718055994531f : -__builtin_inff();
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));   // idle copies into the spare kilobyte have landed
  __syncthreads();                             // every wave is done with the ring
  MLA_LDS uint8_t* ob = lds + wave * (32 * 256);
  // row n, features 32 di + 8 q + 4 g .. +3 (8 bytes); 16-byte chunk c of row n at c ^ (n & 15)
#pragma unroll
  for (int di = 0; di < 4; ++di)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int f0 = 32 * di + 8 * q + 4 * g;
      const int c = f0 >> 3;
      const u32x2 v = {pack_bf2(acc_o[di][4 * q] * inv, acc_o[di][4 * q + 1] * inv),
                       pack_bf2(acc_o[di][4 * q + 2] * inv, acc_o[di][4 * q + 3] * inv)};
      *(MLA_LDS u32x2*)(ob + n * 256 + ((c ^ (n & 15)) << 4) + (f0 & 4) * 2) = v;
    }
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's block is in LDS (read back by the same wave)
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int idx = it * 64 + lane;
    const int row = idx >> 4, c = idx & 15;
    const int srow = ws0 + row;
    const u32x4 v = lds16(ob + row * 256 + ((c ^ (row & 15)) << 4));
    if (srow < T) *(u32x4*)(out + (((size_t)b * T + srow) * n_heads + h) * kNope + c * 8) = v;
  }
}

hipError_t launch_expand_kv_bf16(const uint16_t* cache, int num_blocks, const int32_t* block_table, int max_blocks,
                                 const int32_t* seq_lens, int batch, int n_heads, const uint16_t* w_uk,
                                 const uint16_t* w_uv, uint16_t* kc, uint16_t* vt, int32_t* status, hipStream_t st) {
  const int t_ctx = max_blocks * kBlk;
  const int n_tiles = (t_ctx + kXTok - 1) / kXTok;
  // 8 XCDs x (head sets of 4 per XCD) x (groups of 8 token tiles) x 32
  const long long n_tg = ((long long)batch * n_tiles + 7) / 8;
  const long long n_hs = ((n_heads + 7) / 8 + 3) / 4;
  dim3 grid((unsigned)(8 * n_hs * n_tg * 32));
  hipLaunchKernelGGL(expand_kv_bf16_kernel, grid, dim3(256), 0, st, cache, num_blocks, block_table, max_blocks,
                     seq_lens, batch, n_heads, t_ctx, n_tiles, w_uk, w_uv, kc, vt, status);
  return hipGetLastError();
}

hipError_t launch_prefill_attn_bf16(const uint16_t* q_nope, const uint16_t* q_rope, const uint16_t* cache,
                                    int num_blocks, const int32_t* block_table, int max_blocks,
                                    const int32_t* seq_lens, int batch, int t, int n_heads, float scale,
                                    const uint16_t* kc, const uint16_t* vt, uint16_t* out, float* lse,
                                    int32_t* status, hipStream_t st) {
  const int t_ctx = max_blocks * kBlk;
  const int nqt = (t + kFQ - 1) / kFQ;
  const long long groups = (long long)batch * n_heads;
  dim3 grid((unsigned)((groups + 7) / 8 * 8 * nqt));
  const float scale_log2 = scale * 1.4426950408889634f;
  hipLaunchKernelGGL(prefill_attn_bf16_kernel, grid, dim3(kFWaves * 64), 0, st, q_nope, q_rope, cache, num_blocks,
                     block_table, max_blocks, seq_lens, batch, t, n_heads, t_ctx, nqt, scale_log2, kc, vt, out,
                     lse, status);
  return hipGetLastError();
}

size_t prefill_ws_bytes(int batch, int n_heads, int max_blocks) {
  return (size_t)batch * n_heads * (size_t)max_blocks * kBlk * kNope * 2 * 2;
}

}  // namespace mla
