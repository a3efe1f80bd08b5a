// Latent-space attention for MLA decode on gfx950 (bf16 MFMA, fp32 accumulate).
//
// What it computes ("DeepSeek-V2: Multi-Head Latent Attention (MLA) 原理与工程实现",
// §2.2 matrix absorption and §3.2 decoupled RoPE): for every query row
// (head i, query token s) with absorbed query q_lat = [W^UK_i^T q^C ‖ q^R]
// (pre-scaled by a power of two s2, which rounds nothing), the logits in log2
// units z_j = zscale * q_lat . [c_j ‖ k^R_j], zscale * s2 = softmax scale *
// log2(e), over one range of cached tokens,
// softmax weights against a per-row reference maximum, and the latent
// weighted sum sum_j p_j c_j.  Every range leaves a partial state (latent
// sum, reference maximum, weight sum) that the merge kernel combines.
//
// Mapping onto the chip.  All heads share one latent stream, so a workgroup
// takes 128 query rows (all 128 heads at Sq = 1) against the same cache
// tiles, and both contractions are dense GEMMs on MFMA 32x32x16 (the shape
// one wave can issue at the matrix core's full rate).  Four waves, one per
// SIMD; per wave and 32-token stage:
//   scores  S^T[32 tok x 32 rows] = T[32 tok x 576] . Q^T[576 x 32 rows] for the
//           wave's own 32 rows (36 MFMAs, one accumulation chain: dependent
//           MFMAs of one opcode issue back to back);
//   latent  O^T[128 feat x 128 rows] += C^T[128 feat x 32 tok] . P^T[32 tok x 128 rows]
//           for the wave's own quarter of the 512 latent features and all 128
//           rows (32 MFMAs).
// A wave keeps its Q (144 VGPRs) and its O quarter (256 AGPRs) in registers
// for the whole range; Q arrives as 36 contiguous 1 KB runs, the absorbed
// queries being stored in the MFMA operand order (qlat_byte).  The softmax weights P of a stage go through LDS
// (8 KB, double-buffered), so every tile operand a wave reads for the latent
// product feeds four MFMAs (one per row block) and the transposing tile reads
// drop to a quarter.  The cache tile is read from HBM once per workgroup.
//  - Software pipeline: iteration it scores stage it, then runs the latent
//    product of stage it - 1 with stage it's softmax interleaved between its
//    MFMAs step by step (one exponential per MFMA).  The product's last four
//    MFMAs run after the next iteration's barrier, from operands kept in
//    registers, while that iteration's first score operands are read; the next
//    product's first operands are read during the score chain; and the chain's
//    result is first read four product MFMAs after its last MFMA, so the matrix
//    core waits on neither LDS latency nor a result hazard at either phase edge.
//    The score accumulators live in VGPRs (the score MFMAs are issued as asm
//    in their VGPR form), the latent accumulators in AGPRs, so no accumulator
//    is ever moved between the two register files.
//  - Tiles move HBM -> LDS with global_load_lds_dwordx4 (no VGPR staging)
//    into a 4-slot ring of 36 KB stages: one being multiplied, one being
//    scored, two in flight.  A wave's copies are issued between its score
//    MFMAs.
//  - LDS rows are 1152 B.  16-byte chunk k of token row t sits at chunk
//    k ^ sw(t), sw(t) = 2 (t mod 4) ^ ((t / 4) mod 8) (XOR within groups of 8
//    chunks).  Measured with the LDS bank-conflict counter on gfx950, this
//    makes both the score operand reads (ds_read_b128: 32 rows x 2 chunks)
//    and the transposing PV operand reads (ds_read_b64_tr_b16: 4 rows x 4
//    feature quads per 16 lanes) conflict free.
//  - The PV product needs the tile with tokens along K; the LDS transpose
//    read delivers that from the token-major tile, in the token order in
//    which the S result sits in registers, which is also the order in which
//    P is stored and read back as the MFMA's B operand.
//  - Scores against a fixed per-row reference (the first stage's maximum):
//    p = 2^(z - ref) <= 2^16 unless a later score beats the reference by
//    more than 16, in which case the range is re-run against the largest
//    score seen (exact; for real logit spreads it never happens).  O is never
//    rescaled in registers, so its accumulators are written only by MFMAs
//    and stay in AGPRs.  The weight sum adds the bf16-rounded weights (a
//    packed dot product with ones), the same values the latent product uses.
#include "attn_common.h"

namespace mla {

namespace {
using namespace attn;

constexpr float kNegInf = -__builtin_inff();
constexpr float kLazyTau = 16.0f;   // p = 2^(z - reference) stays <= 2^16
constexpr int kWaves = 4;
constexpr int kRowsPerWave = 32;
static_assert(kWaves * kRowsPerWave == kRowsWG, "rows per workgroup");
constexpr int kLoadsPerWave = kStageBytes / 1024 / kWaves;   // 9 copies of 1 KB per wave and stage
constexpr int kPfS = 3;   // score operands read ahead (measured: 3 beats 2 and 4)
constexpr int kPBytes = kRowsWG * kSubTok * 2;   // one stage's weights for all rows: 8 KB

constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};   // weight sum as a packed dot product
__device__ __forceinline__ int swz(int t) { return ((t & 3) << 1) ^ ((t >> 2) & 7); }

// Maxima of scores: -inf (masked) and finite values only, so the canonicalising moves
// the compiler adds around fmaxf are not needed.
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float vmax2(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

}  // namespace

__global__ __launch_bounds__(kWaves * 64, 1) void attn_bf16_kernel(
    const uint16_t* __restrict__ cache, int num_blocks, const int32_t* __restrict__ block_table, int max_blocks,
    const int32_t* __restrict__ seq_lens, int batch, int sq, int n_heads, int hg, int W, int P,
    float zscale, uint8_t* __restrict__ ws, WsLayout Lw, int32_t* status) {
  // the ring, then two 8 KB slots of softmax weights (bf16) shared by the waves
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * kStageBytes + 2 * kPBytes];
  MLA_LDS uint8_t* lds = (MLA_LDS uint8_t*)smem;
  MLA_LDS uint8_t* pbuf = lds + kStages * kStageBytes;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 31;     // row within the wave's 32 (MFMA column)
  const int hh = lane >> 5;    // lane half

  // XCD-aware order: block ids equal modulo 8 share an XCD (and its L2).  The G head
  // groups of a token range run on one XCD, so the range's cache rows leave HBM once.
  // With W a multiple of 8, XCD x also takes the consecutive ranges x W/8 .. +W/8-1, so
  // the ranges of one sequence share its absorbed queries in L2; otherwise ranges go to
  // the XCDs in turn.
  const int G = Lw.G;
  const int bid = blockIdx.x;
  int w, g;
  if (W % 8 == 0) {
    const int j = bid / 8;
    g = j % G;
    w = (bid % 8) * (W / 8) + j / G;
  } else {
    w = (bid / (8 * G)) * 8 + (bid % 8);
    g = (bid / 8) % G;
  }
  if (w >= W) return;

  const MLA_CONST int32_t* seg = as_const((const int32_t*)(ws + Lw.off_seg));
  const MLA_CONST int32_t* piece_base = as_const((const int32_t*)(ws + Lw.off_piece));
  const MLA_CONST int32_t* wgseg = as_const((const int32_t*)(ws + Lw.off_wgseg));
  const MLA_CONST int32_t* lens = as_const(seq_lens);
  const MLA_CONST int32_t* btab = as_const(block_table);
  const uint8_t* q_lat = ws + Lw.off_qlat;   // absorbed queries in operand order (qlat_byte)
  float2* part_ml = (float2*)(ws + Lw.off_lse);
  uint16_t* part_o = (uint16_t*)(ws + Lw.off_o);   // bf16

  // this range's tokens [lo, hi) of the concatenated sequences (empty past the plan's ranges)
  const MLA_CONST int32_t* rcut = as_const((const int32_t*)(ws + Lw.off_rcut));
  const MLA_CONST int32_t* firstr = as_const((const int32_t*)(ws + Lw.off_firstr));
  const int lo = rcut[w];
  const int hi = rcut[w + 1];
  if (lo >= hi) return;

  // this lane's query row inside the head group
  const int row = wave * kRowsPerWave + n;
  const int hl = row / sq;
  const int s_idx = row - hl * sq;
  const int head = g * hg + hl;
  const bool row_ok = hl < hg && head < n_heads;

  // score operand (A of 32x32x16): lane reads token n, features 16 ks + 8 hh .. +7:
  // logical chunk 2 ks + hh at physical ((2 ks + hh) & ~7) | ((2 (ks & 3) + hh) ^ swz(n))
  int s_off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) s_off[j] = n * (kRow * 2) + (((2 * j + hh) ^ swz(n)) * 16);
  // PV operand (A of 32x32x16, transposing read): lane 16 g + 4 e + q (hh = g / 2) reads
  // token 16 hs + 8 r + 4 hh + e, features 32 fb + 16 (g % 2) + 4 q .. +3, i.e. chunk
  // 4 fb + 2 (g % 2) + q / 2, half q % 2.  swz(token) = 2 e ^ (4 hs + 2 r + hh): the
  // (4 hs + 2 r) part is applied below as an XOR of 16 (4 hs + 2 r) on the byte offset.
  const int g16 = lane >> 4;
  const int e_ = (lane >> 2) & 3;
  const int q_ = lane & 3;
  int o_off[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int clow = (4 * par + 2 * (g16 & 1) + (q_ >> 1)) ^ ((2 * e_) ^ hh);
    o_off[par] = (4 * hh + e_) * (kRow * 2) + clow * 16 + 8 * (q_ & 1);
  }
  // Stage copy plan: copy q (0..35) of a stage moves stage bytes [1024 q, 1024 q + 1024);
  // wave w issues copies w, w + 4, ... .  Lane l's 16 B land at stage chunk 64 q + l:
  // token (64 q + l) / 72, physical chunk (64 q + l) % 72, holding logical chunk
  // (physical ^ swz(token)) of that token.  ld_off = its byte offset inside the 32 rows;
  // two offsets per register.  For a ragged stage (rows past tlast invalid) the rows past
  // tlast re-read row tlast, so every LDS row holds finite cache data.
  uint32_t ld_off2[(kLoadsPerWave + 1) / 2];
  auto set_ld_off = [&](int tlast) {
#pragma unroll
    for (int k = 0; k < 2 * ((kLoadsPerWave + 1) / 2); ++k) {
      uint32_t o = 0;
      if (k < kLoadsPerWave) {
        const int Pc = 64 * (wave + kWaves * k) + lane;
        const int t = Pc / kChunksPerRow;
        const int pc = Pc % kChunksPerRow;
        o = (uint32_t)((t < tlast ? t : tlast) * (kRow * 2) + (pc ^ swz(t)) * 16);
      }
      if (k & 1) ld_off2[k >> 1] |= o << 16;
      else ld_off2[k >> 1] = o;
    }
  };
  auto ld_off = [&](int k) { return (k & 1) ? (ld_off2[k >> 1] >> 16) : (ld_off2[k >> 1] & 0xffffu); };

  // The block-table entry for token tok0 of sequence b: a scalar load whose
  // value is checked only when the copies are issued, so that its latency can
  // hide behind a whole stage of work.
  auto lookup_block = [&](int b, int tok0) {
    return btab[__builtin_amdgcn_readfirstlane(b * max_blocks + tok0 / kBlk)];
  };
  // Global address of the 32-token stage starting at token tok0, inside cache
  // block blk.  A block id outside the pool is reported and replaced by block 0.
  const uint64_t cache_u = uniform_addr(cache);
  auto stage_base = [&](int blk, int tok0) {
    const bool bad = blk < 0 || blk >= num_blocks;   // wave-uniform; the address math stays scalar
    if (bad && lane == 0 && status) atomicOr(status, MLA_STATUS_BAD_BLOCK);
    const uint32_t row = (uint32_t)(bad ? 0 : blk) * kBlk + (uint32_t)(tok0 % kBlk);
    return cache_u + (uint64_t)__builtin_amdgcn_readfirstlane(row) * (uint64_t)(kRow * 2);
  };
  // Issue all of this wave's copies of a stage into ring slot `slot` at once, with the
  // offsets set_ld_off last produced (clamped for a ragged stage).
  auto issue_stage = [&](int slot, uint64_t base) {
    const uint32_t dst0 = (uint32_t)(uintptr_t)(lds + slot * kStageBytes + wave * 1024);
#pragma unroll
    for (int k = 0; k < kLoadsPerWave; ++k)
      copy16_to_lds(base, ld_off(k), __builtin_amdgcn_readfirstlane(dst0 + kWaves * 1024 * k));
  };
  // Copies that fetch nothing needed: an in-bounds read of the pool's first rows
  // into a ring slot no later iteration of the range reads.  Every iteration
  // issues the same number of copies, so one fixed wait count finds each stage
  // landed.
  const uint64_t idle_base = uniform_addr(cache);

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
    if (a >= e) {
      again = false;
      continue;
    }
    const int b = seg_i;
    const int piece = g * P + piece_base[b] + (w - firstr[b]);
    int L = lens[b];
    {
      const int cap = max_blocks * kBlk;
      L = L > cap ? cap : (L < 0 ? 0 : L);
    }
    const int tok_end = e < L ? e : L;
    const int lim = L - sq + s_idx;   // query s sees tokens j <= L - sq + s

    const int nsub = tok_end > a ? (tok_end - a + kSubTok - 1) / kSubTok : 0;
    // block ids of the first three stages: scalar loads issued ahead of the query loads
    const int blk0 = 0 < nsub ? lookup_block(b, a) : 0;
    const int blk1 = 1 < nsub ? lookup_block(b, a + kSubTok) : 0;
    int blk_next = 2 < nsub ? lookup_block(b, a + 2 * kSubTok) : 0;
    {
      // row r of the absorbed queries (for a padding row, the sequence's row 0, zeroed):
      // k-step ks of this lane's operand is the 16 bytes at qlat_byte(r, 16 ks + 8 hh), so
      // each load of the wave is one 1 KB run
      const size_t r = row_ok ? ((size_t)b * n_heads + head) * sq + s_idx : (size_t)b * n_heads * sq;
      const uint8_t* qp = q_lat + qlat_byte(r, 8 * hh);
#pragma unroll
      for (int ks = 0; ks < 36; ++ks) {
        const u32x4 v = *(const u32x4*)(qp + 1024 * ks);
        qreg[ks] = row_ok ? v : u32x4{0u, 0u, 0u, 0u};
      }
    }

    float m_ref = again ? m_again : kNegInf;   // reference maximum (log2 units) of this lane's row
    float m_run = m_ref;                       // largest score seen
    float l_sum = 0.0f;                        // this lane's share of sum_j p_j
    bool bad = false;                          // a score beat the reference by more than 2^tau
    f32x16 acc_o[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[i][r] = 0.0f;
    auto tlast_of = [&](int k) {
      const int t = tok_end - 1 - (a + k * kSubTok);
      return t < kSubTok - 1 ? t : kSubTok - 1;
    };
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      set_ld_off(k < nsub ? tlast_of(k) : kSubTok - 1);
      if (k < nsub) {
        issue_stage(k, stage_base(k == 0 ? blk0 : blk1, a + k * kSubTok));
      } else {
        const uint32_t idle_dst = (uint32_t)(uintptr_t)(lds + k * kStageBytes + wave * 1024);
#pragma unroll
        for (int c = 0; c < kLoadsPerWave; ++c) copy16_to_lds(idle_base, ld_off(c), __builtin_amdgcn_readfirstlane(idle_dst));
      }
    }
    // the weights of the (empty) stage before the first: zero
    *(MLA_LDS u32x4*)(pbuf + kPBytes + wave * 2048 + lane * 16) = u32x4{0u, 0u, 0u, 0u};
    *(MLA_LDS u32x4*)(pbuf + kPBytes + wave * 2048 + 1024 + lane * 16) = u32x4{0u, 0u, 0u, 0u};
    // later block ids are looked up one stage ahead of their copies, so that the
    // scalar load's latency is hidden behind a whole stage of work

    // Iteration it scores stage it and, interleaved with that stage's softmax,
    // runs the latent product of stage it - 1, so the softmax's vector work
    // overlaps matrix work.  Iteration nsub only finishes the last product.  The
    // product's last four MFMAs (token half 1, feature block 3, the four row blocks)
    // run at the start of the next iteration, right after its barrier, from operands
    // kept in registers: that matrix work covers the latency of the first score-operand
    // reads.  Before the first iteration the kept operands are zero (0 x 0 is added).
    u32x4 tail_a = u32x4{0u, 0u, 0u, 0u};
    u32x4 tail_b[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) tail_b[rb] = u32x4{0u, 0u, 0u, 0u};
    for (int it = 0; it <= nsub; ++it) {
      // This wave's copies of stage it have landed once at most one stage's worth
      // (issued by the previous iteration) remains in flight.
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(kLoadsPerWave));
      __syncthreads();   // stage it visible to all waves; stage it - 2 fully consumed
      // The copies of stage it + 2 ride along the score MFMAs below.  A ragged stage (a
      // sequence's last) re-reads its last valid row in place of the rows past it.  With no
      // stage left to fetch, the copies land in the slot stage it + 2 would use: no later
      // iteration of this range reads it.
      uint64_t nbase = idle_base;
      uint32_t ndst = (uint32_t)(uintptr_t)(lds + ((it + 2) & 3) * kStageBytes + wave * 1024), nstride = 0;
      if (it + 2 < nsub) {
        nbase = stage_base(blk_next, a + (it + 2) * kSubTok);
        nstride = kWaves * 1024;
        const int ntl = tlast_of(it + 2);
        if (ntl < kSubTok - 1) set_ld_off(ntl);   // the range's last stage: later copies are idle
      }
      const bool valid = it < nsub;
      const MLA_LDS uint8_t* st = lds + (it & 3) * kStageBytes;
      // the latent product's stage (stage 0 for the empty product of iteration 0:
      // finite data times zero weights)
      const MLA_LDS uint8_t* sto = lds + ((it > 0 ? it - 1 : 0) & 3) * kStageBytes;
      const int tok0 = a + it * kSubTok;

      // latent-product operands (stage it - 1), the first of them read during the score MFMAs
      const MLA_LDS uint8_t* pp = pbuf + ((it + 1) & 1) * kPBytes + lane * 16;
      // A operand ai = 4 hs + fb: feature block 4 wave + fb, token half hs; its two reads
      // take tokens 16 hs + 4 hh + e (r = 0) and 16 hs + 8 + 4 hh + e (r = 1)
      auto rd = [&](int ai) {
        const int hs = ai >> 2, FB = 4 * wave + (ai & 3);
        const int o0 = (o_off[FB & 1] ^ (16 * (4 * hs))) + (FB >> 1) * 128 + (16 * hs) * (kRow * 2);
        const int o1 = (o_off[FB & 1] ^ (16 * (4 * hs + 2))) + (FB >> 1) * 128 + (16 * hs + 8) * (kRow * 2);
        const u32x2 lo2 = lds_read_tr16(sto + o0);
        const u32x2 hi2 = lds_read_tr16(sto + o1);
        return u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
      };
      u32x4 pb[2][4], av[8];

      // ---- S^T = T . Q^T (32 tokens x 32 rows), 36 k-steps of 16 features
      // one accumulation chain: dependent MFMAs of one opcode issue back to back
      f32x16 acc_s;
      {
        u32x4 tv[kPfS];
#pragma unroll
        for (int k = 0; k < kPfS; ++k) tv[k] = lds_read16(st + s_off[k & 3] + (k >> 2) * 128);
        __builtin_amdgcn_sched_barrier(0);
        // the previous product's last four MFMAs while the first reads land
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          acc_o[12 + rb] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(tail_a), as_bf8(tail_b[rb]), acc_o[12 + rb], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int ks = 0; ks < 36; ++ks) {
          const u32x4 t = tv[ks % kPfS];
          if (ks + kPfS < 36) tv[ks % kPfS] = lds_read16(st + s_off[(ks + kPfS) & 3] + ((ks + kPfS) >> 2) * 128);
          if (ks == 0) mfma_s_first(acc_s, t, qreg[ks]);
          else mfma_s(acc_s, t, qreg[ks]);
          if ((ks & 3) == 2)
            copy16_to_lds(nbase, ld_off(ks >> 2), __builtin_amdgcn_readfirstlane(ndst + nstride * (ks >> 2)));
          if (ks == 27) av[0] = rd(0);
          if (ks == 31) av[1] = rd(1);
          if (ks == 32) {
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) pb[0][rb] = lds_read16(pp + rb * 2048);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (!valid || tok0 + kSubTok - 1 > L - sq) {   // past some row's last visible token, or no stage
        settle_s(acc_s);   // the chain's result is read right away here
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int tok = tok0 + 8 * (r >> 2) + 4 * hh + (r & 3);
          const bool off = !valid || tok > lim;
          acc_s[r] = off ? kNegInf : acc_s[r];
        }
      }

      // ---- softmax weights of stage it against the row reference (log2 units; the lane
      // holds row n and tokens 8 (r / 4) + 4 hh + r % 4, r = 0..15), interleaved step by
      // step with the latent product of stage it - 1:
      //   O^T += C^T . P^T over this wave's 128 features (4 blocks of 32) x all 128 rows
      //   (4 row blocks) x 2 token halves, 32 MFMAs.  P comes from LDS, written there by
      //   the wave that owns each row block.  The chain's result is first read after four
      //   of these MFMAs, i.e. over a hundred cycles after the chain's last MFMA issued,
      //   well past the wait an 8-pass MFMA's result needs.
      {
        uint32_t pk[8];
        float p[16];
        float mx = 0.0f, msafe = 0.0f;
#pragma unroll
        for (int j = 0; j < 28; ++j) {
          const int hs = j >> 4, fb = (j >> 2) & 3, rb = j & 3, ai = 4 * hs + fb;
          acc_o[4 * fb + rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(av[ai]), as_bf8(pb[hs][rb]),
                                                                       acc_o[4 * fb + rb], 0, 0, 0);
          if (rb == 0 && ai + 2 < 8) av[ai + 2] = rd(ai + 2);
          if (j == 10) {
#pragma unroll
            for (int r2 = 0; r2 < 4; ++r2) pb[1][r2] = lds_read16(pp + r2 * 2048 + 1024);
          }
          if (j == 5) {
            mx = vmax3(vmax3(acc_s[0], acc_s[1], acc_s[2]), vmax3(acc_s[3], acc_s[4], acc_s[5]),
                       vmax3(acc_s[6], acc_s[7], acc_s[8]));
          } else if (j == 6) {
            mx = vmax3(mx, vmax3(acc_s[9], acc_s[10], acc_s[11]), vmax3(acc_s[12], acc_s[13], vmax2(acc_s[14], acc_s[15])));
          } else if (j == 7) {
            // the other lane half holds the same row's other 16 tokens
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
            mx = vmax2(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * zscale;   // zscale > 0
          } else if (j == 9) {
            m_run = vmax2(m_run, mx);
            m_ref = m_ref == kNegInf ? mx : m_ref;   // a row's reference: its first finite stage maximum
          } else if (j == 11) {
            bad = bad || (mx > m_ref + kLazyTau);
            msafe = m_ref == kNegInf ? 0.0f : m_ref;
          } else if (j >= 12) {
            // one weight per MFMA; each pair packed to bf16, and summed as rounded
            const int r = j - 12;
            p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(acc_s[r], zscale, -msafe));
            if (r & 1) {
              pk[r >> 1] = pack_bf2(p[r - 1], p[r]);
              l_sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[r >> 1]), kOnes2, l_sum, false);
            }
            if (j == 27) {
              // this stage's weights, for every wave's latent product in the next iteration
              *(MLA_LDS u32x4*)(pbuf + (it & 1) * kPBytes + wave * 2048 + lane * 16) =
                  u32x4{pk[0], pk[1], pk[2], pk[3]};
              *(MLA_LDS u32x4*)(pbuf + (it & 1) * kPBytes + wave * 2048 + 1024 + lane * 16) =
                  u32x4{pk[4], pk[5], pk[6], pk[7]};
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        tail_a = av[7];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) tail_b[rb] = pb[1][rb];
      }
      // The block id of stage it + 3 (its copies go out in the next iteration).  A scalar
      // load is counted with the LDS reads and returns out of order, so any LDS wait after
      // it must wait for it too: issued here, its latency hides under the barrier's wait
      // instead of the next score chain's first operand wait.
      if (it + 3 < nsub) blk_next = lookup_block(b, a + (it + 3) * kSubTok);
      __builtin_amdgcn_sched_barrier(0);
    }
    // the last product's last four MFMAs
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
      acc_o[12 + rb] =
          __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(tail_a), as_bf8(tail_b[rb]), acc_o[12 + rb], 0, 0, 0);
    const bool wbad = __builtin_amdgcn_ballot_w64(bad) != 0ull;
    // The last two iterations' copies (idle ones, into ring slots (nsub + 1) & 3 and
    // (nsub + 2) & 3) may still be in flight; they are asm, so the compiler does not wait
    // for them.  The epilogue below reuses ring slots 0 and 1 and a retried range refills
    // the ring, so every copy of this wave lands before the barrier.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();   // ring and weight slots free
    MLA_LDS int* flags = (MLA_LDS int*)pbuf;
    if (lane == 0) flags[wave] = wbad ? 1 : 0;
    __syncthreads();   // every wave's flag visible
    const bool retry = (flags[0] | flags[1] | flags[2] | flags[3]) != 0;
    __syncthreads();   // every wave has read the flags
    if (retry) {
      // a score beat the reference by more than 2^tau: run this range again
      // against the largest score seen (rare; exact either way)
      m_again = m_run;
      again = true;
      continue;
    }
    again = false;

    // ---- partial state: un-normalised latent sum, reference max and weight sum
    const float l_tot = l_sum + __shfl_xor(l_sum, 32);
    // (rounded to bf16 on the way out, through LDS: the ring is free once every wave has
    // left the loop, which the flag barriers above guarantee)
    uint16_t* prow = part_o + (size_t)piece * kRowsWG * kLat;
    // two passes of 64 rows (two 32-row blocks staged side by side)
    static_assert(2 * kEpiRows * kEpiStride <= kStages * kStageBytes, "two epilogue blocks fit the ring");
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int fb = 0; fb < 4; ++fb) {
          const f32x16& A = acc_o[4 * fb + 2 * pass + half];
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
            stage_row_f4(lds + half * kEpiRows * kEpiStride, n, 128 * wave + 32 * fb + 8 * rr + 4 * hh,
                         f32x4{A[4 * rr], A[4 * rr + 1], A[4 * rr + 2], A[4 * rr + 3]});
        }
      __syncthreads();
      store_pass_bf16(lds, prow + (size_t)kEpiRows * 2 * pass * kLat, tid);
      store_pass_bf16(lds + kEpiRows * kEpiStride, prow + (size_t)kEpiRows * (2 * pass + 1) * kLat, tid);
      __syncthreads();   // LDS free for the next pass (or the next range)
    }
    if (hh == 0) part_ml[(size_t)piece * kRowsWG + row] = make_float2(m_ref, l_tot);
  }
}

hipError_t launch_attn_bf16(const WsLayout& L, const uint16_t* cache, int num_blocks, const int32_t* block_table,
                            int max_blocks, const int32_t* seq_lens, int batch, int sq, int n_heads, float zscale,
                            uint8_t* ws, int32_t* status, hipStream_t st) {
  // grid: W ranges x G head groups, ordered so the groups of a range share an XCD
  const int wpad = (L.W + 7) / 8 * 8;
  dim3 grid(wpad * L.G);
  hipLaunchKernelGGL(attn_bf16_kernel, grid, dim3(kWaves * 64), 0, st, cache, num_blocks, block_table, max_blocks,
                     seq_lens, batch, sq, n_heads, L.hg, L.W, L.P, zscale, ws, L, status);
  return hipGetLastError();
}

}  // namespace mla
