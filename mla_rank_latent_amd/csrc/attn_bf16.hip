// Latent-space attention for MLA decode on gfx950 (bf16 MFMA, fp32 accumulate).
//
// What it computes ("DeepSeek-V2: Multi-Head Latent Attention (MLA) 原理与工程实现",
// §2.2 matrix absorption and §3.2 decoupled RoPE): for every query row
// (head i, query token s) with absorbed query q_lat = [W^UK_i^T q^C ‖ q^R],
// the logits z_j = scale * q_lat . [c_j ‖ k^R_j] over one range of cached
// tokens, an online softmax over them, and the latent weighted sum
// sum_j p_j c_j.  Every range leaves a partial state (latent sum, reference
// maximum, weight sum) that the merge kernel combines.
//
// Mapping onto the chip.  All heads share one latent stream, so a workgroup
// takes 128 query rows (all 128 heads at Sq = 1) against the same cache
// tiles, and the two contractions are dense GEMMs on MFMA:
//   S^T[32 tok x 32 rows]  = T[32 tok x 576] . Q^T[576 x 32 rows]     (36 MFMA 32x32x16)
//   O^T[512 x 32 rows]    += C^T[512 x 32 tok] . P^T[32 tok x 32 rows] (32 MFMA 32x32x16)
// per wave and 32-token stage.  Each of the 4 waves owns 32 rows: its Q
// (144 VGPRs) and its O accumulator (256 registers) stay in registers for
// the whole range; the cache tile is read from HBM once per workgroup.
//  - Tiles move HBM -> LDS with global_load_lds_dwordx4 (no VGPR staging)
//    into a 4-deep ring of 36 KB stages, so three stages are in flight while
//    one is consumed.
//  - LDS rows are 1152 B; 16-byte chunk k of token row t sits at chunk
//    k ^ sw(t), sw(t) = 2(t mod 4) + ((t / 4) mod 2).  With it the S operand
//    reads (ds_read_b128, 8 tokens x one chunk) and the transposing O
//    operand reads (ds_read_b64_tr_b16, 4 tokens x 4 features per 16 lanes)
//    are both bank-conflict free.
//  - The PV product needs the cache tile with tokens along K; the LDS
//    transpose read delivers exactly that from the token-major tile, and the
//    token order it produces matches the order in which the S result already
//    sits in registers, so P never leaves registers.
//  - Softmax runs in log2 units against a fixed per-row reference: the row's
//    maximum over the first 32 tokens of the range.  Scores may exceed it by
//    up to 16 (p <= 2^16, well inside bf16/fp32 range).  O is never rescaled
//    in registers (VALU writes to the MFMA accumulators would push them out
//    of AGPRs and spill); if a score ever beats the reference by more than
//    16, the workgroup re-runs the range against the largest score seen,
//    which is exact and, for real logit spreads, never happens.  The partial
//    is stored un-normalised with its (reference, weight sum); the merge
//    kernel normalises.
#include "device_util.h"

namespace mla {

namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr float kLazyTau = 16.0f;   // p = 2^(z - reference) stays <= 2^16

__device__ __forceinline__ int swz(int t) { return ((t & 3) << 1) | ((t >> 2) & 1); }

__device__ __forceinline__ bf16x8 as_bf8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ u32x4 lds_read16(const MLA_LDS uint8_t* p) {
  return *(const MLA_LDS u32x4*)p;
}

__device__ __forceinline__ u32x2 lds_read_tr(const MLA_LDS uint8_t* p) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS s16x4*)p);
  return __builtin_bit_cast(u32x2, v);
}

// Read-only tables are read through the constant address space so that
// wave-uniform lookups become scalar loads (counted by lgkmcnt, not vmcnt,
// and so never waiting on the in-flight tile copies).
#define MLA_CONST __attribute__((address_space(4)))
template <typename T>
__device__ __forceinline__ const MLA_CONST T* as_const(const T* p) {
  return (const MLA_CONST T*)p;
}

struct Ctx {
  const uint16_t* cache;
  const MLA_CONST int32_t* block_table;
  int max_blocks;
  int num_blocks;
  int32_t* status;
};

// Issue this wave's 9 direct-to-LDS loads for one 32-token stage.
// Stage chunk P (16 B) = 64 q + lane holds token t = P / 72, physical chunk
// P % 72, which is logical chunk (P % 72) ^ swz(t) of that token's row.
__device__ __forceinline__ void issue_stage(const Ctx& cx, MLA_LDS uint8_t* stage, int wave, int lane,
                                            int b, int tok0, int tlast) {
  // the 32-token stage lies inside one 64-token block
  // wave-uniform by construction; readfirstlane lets the compiler see it and use a scalar load
  const int idx = __builtin_amdgcn_readfirstlane(b * cx.max_blocks + tok0 / kBlk);
  int blk = cx.block_table[idx];
  if (blk < 0 || blk >= cx.num_blocks) {
    if (lane == 0 && cx.status) atomicOr(cx.status, MLA_STATUS_BAD_BLOCK);
    blk = 0;
  }
  const uint8_t* base = (const uint8_t*)cx.cache + ((size_t)blk * kBlk + (tok0 % kBlk)) * (size_t)(kRow * 2);
  // Recomputed per stage on purpose: hoisted out of the loop these 9 offsets
  // would be spilled, and reloading a spill waits on the in-flight copies.
  int lane_o = lane;
  asm volatile("" : "+v"(lane_o));
#pragma unroll
  for (int k = 0; k < 9; ++k) {
    int q = wave + 4 * k;
    int P = 64 * q + lane_o;
    int t = P / kChunksPerRow;
    int pc = P - t * kChunksPerRow;
    int c = pc ^ swz(t);
    int tt = t < tlast ? t : tlast;   // rows past the end re-read the last valid row
    const uint8_t* src = base + tt * (kRow * 2) + c * 16;
    // Issued as asm so the compiler does not treat every later LDS read as
    // aliasing the in-flight copy (it would wait for all of them); the ring
    // protocol below waits for exactly the stage it reads.
    uint32_t dst = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(stage + q * 1024));
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(dst) : "memory");
  }
}

}  // namespace

__global__ __launch_bounds__(256, 1) void attn_bf16_kernel(
    const uint16_t* __restrict__ cache, int num_blocks, const int32_t* __restrict__ block_table, int max_blocks,
    const int32_t* __restrict__ seq_lens, int batch, int sq, int n_heads, int hg, int W, int P,
    float scale_log2, uint8_t* __restrict__ ws, WsLayout Lw, int32_t* status) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * kStageBytes];
  MLA_LDS uint8_t* lds = (MLA_LDS uint8_t*)smem;
  __shared__ int s_retry;
  if (threadIdx.x == 0) s_retry = 0;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 31;     // row within the wave's 32 (MFMA column)
  const int hh = lane >> 5;    // lane half

  // XCD-aware order: block ids that differ by a multiple of 8 share an XCD (and
  // its L2); the G head groups of one token range take ids 8 apart.
  const int G = Lw.G;
  int bid = blockIdx.x;
  const int w = (bid / (8 * G)) * 8 + (bid % 8);
  const int g = (bid / 8) % G;
  if (w >= W) return;

  const MLA_CONST PlanHeader* hdr = as_const((const PlanHeader*)(ws + Lw.off_hdr));
  const MLA_CONST int32_t* seg = as_const((const int32_t*)(ws + Lw.off_seg));
  const MLA_CONST int32_t* piece_base = as_const((const int32_t*)(ws + Lw.off_piece));
  const MLA_CONST int32_t* wgseg = as_const((const int32_t*)(ws + Lw.off_wgseg));
  const MLA_CONST int32_t* lens = as_const(seq_lens);
  const uint16_t* q_lat = (const uint16_t*)(ws + Lw.off_qlat);
  float2* part_ml = (float2*)(ws + Lw.off_lse);
  float* part_o = (float*)(ws + Lw.off_o);

  const int total = hdr->total;
  const int quota = hdr->quota;
  const int lo = w * quota;
  if (lo >= total) return;
  const int hi = lo + quota < total ? lo + quota : total;

  Ctx cx{cache, as_const(block_table), max_blocks, num_blocks, status};

  // this lane's query row inside the head group
  const int row = wave * 32 + n;
  const int hl = row / sq;
  const int s_idx = row - hl * sq;
  const int head = g * hg + hl;
  const bool row_ok = hl < hg && head < n_heads;

  // per-lane LDS offsets for the S operand: token n, chunk (2 ks + hh) ^ swz(n)
  int s_off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) s_off[j] = n * (kRow * 2) + ((((2 * j) | hh) ^ swz(n)) * 16);
  // per-lane LDS offsets for the transposing O operand reads:
  // lane = 16 g16 + 4 e + q reads token (4 hh + e) (+16 hs + 8 r), features 32 fb + 16 (g16 % 2) + 4 q
  const int g16 = lane >> 4;
  const int e_ = (lane >> 2) & 3;
  const int q_ = lane & 3;
  int o_off[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    int clow = (4 * par + 2 * (g16 & 1) + (q_ >> 1)) ^ (2 * e_ + hh);
    o_off[par] = (4 * hh + e_) * (kRow * 2) + clow * 16 + 8 * (q_ & 1);
  }

  int seg_i = wgseg[w];
  u32x4 qreg[36];
  bool again = false;       // re-running the previous range with a raised reference
  float m_again = kNegInf;

  for (; seg_i < batch; seg_i += again ? 0 : 1) {
    const int s0 = seg[seg_i];
    const int s1 = seg[seg_i + 1];
    if (s0 >= hi) break;
    const int a = (lo > s0 ? lo : s0) - s0;
    const int e = (hi < s1 ? hi : s1) - s0;
    if (a >= e) { again = false; continue; }
    const int b = seg_i;
    const int piece = g * P + piece_base[b] + (w - s0 / quota);
    int L = lens[b];
    {
      int cap = max_blocks * kBlk;
      if (L > cap) L = cap;
      if (L < 0) L = 0;
    }
    const int tok_end = e < L ? e : L;
    // row limit: query s sees tokens j <= L - sq + s
    const int lim = L - sq + s_idx;

    {
      const uint16_t* qp = q_lat + ((size_t)(b * sq + s_idx) * n_heads + head) * kRow + 8 * hh;
#pragma unroll
      for (int ks = 0; ks < 36; ++ks) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (row_ok) v = *(const u32x4*)(qp + 16 * ks);
        qreg[ks] = v;
      }
    }

    float m_ref = again ? m_again : kNegInf;   // reference maximum (log2 units) of this lane's row
    float m_run = m_ref;                        // largest score seen so far
    float l_sum = 0.0f;                         // this lane's share of the row's sum of p
    f32x16 acc_o[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[i][r] = 0.0f;
    const int nsub = tok_end > a ? (tok_end - a + kSubTok - 1) / kSubTok : 0;
    {
      // prologue: stages 0..2
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        if (k < nsub) {
          int tok0 = a + k * kSubTok;
          int tl = tok_end - 1 - tok0;
          issue_stage(cx, lds + k * kStageBytes, wave, lane, b, tok0, tl < kSubTok - 1 ? tl : kSubTok - 1);
        }
      }
      for (int it = 0; it < nsub; ++it) {
        // wait for this wave's loads of stage `it`; later stages may stay in flight
        if (it + 2 < nsub) __builtin_amdgcn_s_waitcnt(waitcnt_vm(18));
        else if (it + 1 < nsub) __builtin_amdgcn_s_waitcnt(waitcnt_vm(9));
        else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        __syncthreads();   // all waves' loads visible; stage (it - 1) fully consumed
        if (it + 3 < nsub) {
          int tok0 = a + (it + 3) * kSubTok;
          int tl = tok_end - 1 - tok0;
          issue_stage(cx, lds + ((it + 3) & 3) * kStageBytes, wave, lane, b, tok0, tl < kSubTok - 1 ? tl : kSubTok - 1);
        }
        const MLA_LDS uint8_t* st = lds + (it & 3) * kStageBytes;
        const int tok0 = a + it * kSubTok;

        // ---- S^T = T . Q^T  (tokens x rows)
        f32x16 acc_s;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_s[r] = 0.0f;
        {
          // three operand reads in flight ahead of the MFMA chain
          u32x4 tv[4];
#pragma unroll
          for (int k = 0; k < 3; ++k) tv[k] = lds_read16(st + s_off[k & 3] + (k >> 2) * 128);
#pragma unroll
          for (int ks = 0; ks < 36; ++ks) {
            if (ks + 3 < 36) tv[(ks + 3) & 3] = lds_read16(st + s_off[(ks + 3) & 3] + ((ks + 3) >> 2) * 128);
            acc_s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(tv[ks & 3]), as_bf8(qreg[ks]), acc_s, 0, 0, 0);
          }
        }

        // ---- softmax weights of the 32 tokens against the row's reference (log2 units)
        float z[16];
        float mx = kNegInf;
        const bool need_mask = tok0 + kSubTok - 1 > L - sq;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = acc_s[r] * scale_log2;
          if (need_mask) {
            int tok = tok0 + 8 * (r >> 2) + 4 * hh + (r & 3);
            if (tok > lim) v = kNegInf;
          }
          z[r] = v;
          mx = fmaxf(mx, v);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        m_run = fmaxf(m_run, mx);
        // a row's reference is its first finite stage maximum (nothing is accumulated before it)
        if (m_ref == kNegInf) m_ref = mx;
        if (__builtin_amdgcn_ballot_w64(mx > m_ref + kLazyTau) != 0ull && lane == 0) s_retry = 1;
        const float msafe = m_ref == kNegInf ? 0.0f : m_ref;
        uint32_t pk[8];
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          float p0 = __builtin_amdgcn_exp2f(z[r] - msafe);
          float p1 = __builtin_amdgcn_exp2f(z[r + 1] - msafe);
          uint32_t pp = pack_bf2(p0, p1);
          pk[r >> 1] = pp;
          l_sum += __uint_as_float(pp << 16) + __uint_as_float(pp & 0xffff0000u);
        }

        // ---- O^T += C^T . P^T  (512 latent features x rows), two 16-token k-steps
        {
          // 32 MFMAs (16 feature blocks x 2 token halves), operands read 2 ahead
          u32x4 av[3];
#define MLA_OPERAND(j)                                                                                 \
  ({                                                                                                    \
    const MLA_LDS uint8_t* p0_ = st + o_off[(j) & 1] + (((j) & 15) >> 1) * 128 + (16 * ((j) >> 4)) * (kRow * 2); \
    u32x2 lo2_ = lds_read_tr(p0_);                                                                      \
    u32x2 hi2_ = lds_read_tr(p0_ + 8 * (kRow * 2));                                                     \
    u32x4 v_ = {lo2_[0], lo2_[1], hi2_[0], hi2_[1]};                                                    \
    v_;                                                                                                 \
  })
          av[0] = MLA_OPERAND(0);
          av[1] = MLA_OPERAND(1);
          const u32x4 pb0 = {pk[0], pk[1], pk[2], pk[3]};
          const u32x4 pb1 = {pk[4], pk[5], pk[6], pk[7]};
#pragma unroll
          for (int j = 0; j < 32; ++j) {
            if (j + 2 < 32) av[(j + 2) % 3] = MLA_OPERAND(j + 2);
            acc_o[j & 15] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(av[j % 3]), as_bf8(j < 16 ? pb0 : pb1),
                                                                    acc_o[j & 15], 0, 0, 0);
          }
#undef MLA_OPERAND
        }
      }
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      __syncthreads();   // ring drained and free; every wave's flag write visible
      const bool retry = s_retry != 0;
      __syncthreads();   // every wave has read the flag
      if (retry) {
        // a score beat the reference by more than 2^tau: run this range again
        // against the largest score seen (rare; exact either way)
        if (tid == 0) s_retry = 0;
        m_again = m_run;
        again = true;
        continue;
      }
    }
    again = false;

    // ---- partial state: un-normalised latent sum, reference max and weight sum
    const float l_tot = l_sum + __shfl_xor(l_sum, 32);
    float* op = part_o + ((size_t)piece * kRowsWG + row) * kLat;
#pragma unroll
    for (int fb = 0; fb < 16; ++fb) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        f32x4 v = {acc_o[fb][4 * rr], acc_o[fb][4 * rr + 1], acc_o[fb][4 * rr + 2], acc_o[fb][4 * rr + 3]};
        *(f32x4*)(op + fb * 32 + 8 * rr + 4 * hh) = v;
      }
    }
    if (hh == 0) part_ml[(size_t)piece * kRowsWG + row] = make_float2(m_ref, l_tot);
  }
}

hipError_t launch_attn_bf16(const WsLayout& L, const uint16_t* cache, int num_blocks, const int32_t* block_table,
                            int max_blocks, const int32_t* seq_lens, int batch, int sq, int n_heads, float scale,
                            uint8_t* ws, int32_t* status, hipStream_t st) {
  // grid: W ranges x G head groups, ordered so the groups of a range share an XCD
  int wpad = (L.W + 7) / 8 * 8;
  dim3 grid(wpad * L.G);
  const float scale_log2 = scale * 1.4426950408889634f;
  hipLaunchKernelGGL(attn_bf16_kernel, grid, dim3(256), 0, st, cache, num_blocks, block_table, max_blocks, seq_lens,
                     batch, sq, n_heads, L.hg, L.W, L.P, scale_log2, ws, L, status);
  return hipGetLastError();
}

}  // namespace mla
