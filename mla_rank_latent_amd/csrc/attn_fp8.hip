// Latent-space attention for MLA decode over the FP8 latent cache (gfx950).
//
// Same computation as the bf16-cache kernel ("DeepSeek-V2: Multi-Head Latent
// Attention (MLA) 原理与工程实现", §2.2 matrix absorption and §3.2 decoupled
// RoPE): for every query row with absorbed query q_lat = [W^UK_i^T q^C ‖ q^R]
// (pre-scaled by a power of two s2), logits in log2 units
// z_j = zscale * q_lat . [c_j ‖ k^R_j], zscale * s2 = softmax scale * log2(e),
// over one range of cached tokens,
// softmax weights against a per-row reference maximum, and the latent weighted
// sum sum_j p_j c_j, left as a partial state for the merge kernel.  Here the
// cache stores c_j = s_j * v(code_j) (E4M3 codes, one power-of-two scale per
// token), and the kernel computes on those values exactly: s_j * v(code) is a
// bf16 value, produced by the hardware's scaled conversion, so the score reads
// [s_j v(code_j) ‖ k^R_j] as the bf16 kernel reads [c_j ‖ k^R_j]; the weighted
// sum takes the codes unscaled and the scale on the weight,
//   sum_j p_j c_j = sum_j (p_j s_j) v(code_j),
// so the only roundings are those of the bf16 path (the weights p_j s_j go to
// bf16 as the bf16 kernel's p_j do).
//
// Mapping onto the chip: as the bf16 kernel (128 query rows per workgroup, four
// waves, one per SIMD: a wave scores its own 32 rows and accumulates its quarter
// of the 512 latent features for all 128 rows, with the bf16 weights shared
// through LDS; MFMA 32x32x16 bf16 for both products, the score MFMAs in their
// VGPR form in one chain, the latent product of stage it - 1 interleaved step by
// step with stage it's softmax, restart-on-overflow reference).  What the
// format changes:
//  - A 32-token stage is 21 KB instead of 36 KB (16 KB of codes, 4 KB of k^R,
//    the 128 B of scales in a 1 KB slot), so the ring holds six stages and
//    four are in flight while one is scored and one multiplied.
//  - Score operands: one 16-byte LDS read gives 16 codes of a token, which
//    convert (v_cvt_scalef32_pk_bf16_fp8 with the token's scale) to the
//    operands of two k-steps; the query registers are loaded in the matching
//    feature order.
//  - Latent-product operands come from ds_read_b64_tr_b8, which hands each
//    lane one feature of eight tokens (the order in which the score result
//    holds its tokens), converted with scale 1; the scale rides on the weight.
//    A wave converts only its feature quarter, and each converted operand
//    feeds the four row blocks' MFMAs.
//  - LDS rows: 16-byte chunk c of a token's 512-byte code row sits at
//    c ^ swf(t), swf a permutation of t's low four bits chosen so that the
//    16 tokens of a score read and the 8 tokens x 2 chunks of a transposing
//    read each fall in distinct banks; k^R rows (128 B) use c ^ ((t >> 1) & 7).
#include "attn_common.h"

namespace mla {

namespace {
using namespace attn;

constexpr float kNegInf = -__builtin_inff();
constexpr float kLazyTau = 16.0f;   // p = 2^(z - reference) stays <= 2^16
constexpr int kWaves = 4;
constexpr int kRowsPerWave = 32;
static_assert(kWaves * kRowsPerWave == kRowsWG, "rows per workgroup");
constexpr int kQLat = kSubTok * kLat;            // 16384: code rows of a stage
constexpr int kQRope = kSubTok * kRope * 2;      // 4096: k^R rows of a stage
constexpr int kQScale = kQLat + kQRope;          // offset of the 32 scales
constexpr int kQStage = kQScale + 1024;          // 21504
constexpr int kQSlots = 6;                       // ring slots
constexpr int kQAhead = kQSlots - 2;             // stages in flight
constexpr int kQCopies = 6;                      // 1 KB copies per wave and stage (21 used of 24)
constexpr int kPfS = 3;                          // score reads ahead (each feeds two k-steps)
constexpr int kQIdle = kQSlots * kQStage;       // the spare kilobyte
constexpr int kQRq = kQIdle + 1024;              // q^R of the 128 rows (128 B each)
constexpr int kPBytes = kRowsWG * kSubTok * 2;   // one stage's weights for all rows: 8 KB
constexpr int kQP = kQRq + kRowsWG * kRope * 2;   // two slots of softmax weights (bf16)
constexpr int kQLds = kQP + 2 * kPBytes;
static_assert(kQStage % 1024 == 0 && kQLds <= 160 * 1024, "LDS budget");

__device__ __forceinline__ int swf(int t) { return ((t & 3) << 1) | ((t >> 2) & 1) | (t & 8); }
__device__ __forceinline__ int swr(int t) { return (t >> 1) & 7; }

// four E4M3 codes (one dword, code k in byte k) times a power of two s -> four bf16, exactly
__device__ __forceinline__ u32x2 cvt4(uint32_t w, float s) {
  const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, s, false);
  const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, s, true);
  return u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

// Score MFMAs (VGPR form, as mfma_s_first / mfma_s) whose A operand the vector unit has just
// written (the code conversion): an MFMA may read a VGPR only two wait states after a VALU
// instruction wrote it, and the compiler cannot see the MFMA inside the asm, so the asm
// issues the wait states itself.
__device__ __forceinline__ void mfma_sv_first(f32x16& acc, u32x4 a, u32x4 b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_sv(f32x16& acc, u32x4 a, u32x4 b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}

// ds_read_b64_tr_b8: in each group of 16 lanes, lanes 2 e and 2 e + 1 point at bytes 0..7 and
// 8..15 of row e (e = 0..7); lane i of the group receives byte i of every row, row e in byte e
__device__ __forceinline__ u32x2 lds_read_tr8(const MLA_LDS uint8_t* p) {
  typedef int i32x2 __attribute__((ext_vector_type(2)));
  const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((MLA_LDS i32x2*)p);
  return __builtin_bit_cast(u32x2, v);
}

}  // namespace

__global__ __launch_bounds__(kWaves * 64, 1) void attn_fp8_kernel(
    const uint8_t* __restrict__ pages, int num_blocks, const int32_t* __restrict__ block_table, int max_blocks,
    const int32_t* __restrict__ seq_lens, int batch, int sq, int n_heads, int hg, int W, int P,
    float zscale, uint8_t* __restrict__ ws, WsLayout Lw, int32_t* status) {
  // the ring, 1 KB that absorbs the copies that fetch nothing needed, and the rows' q^R
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kQLds];
  MLA_LDS uint8_t* lds = (MLA_LDS uint8_t*)smem;
  __shared__ int s_retry;
  if (threadIdx.x == 0) s_retry = 0;

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

  // Score operands (A of 32x32x16: lane = token n, K half hh).  Code pair j (k-steps 2 j and
  // 2 j + 1): logical chunk 2 j + hh of token n, at physical (2 j + hh) ^ swf(n) =
  // 2 (j ^ (swf >> 1)) + (hh ^ (swf & 1)); as a byte offset, sl_off ^ 32 j for j < 8, plus 256
  // for j >= 8.  k^R k-step k (0..3): chunk 2 k + hh of the token's k^R row, sr_off ^ 32 k.
  const int sf = swf(n);
  const int sl_off = n * kLat + 32 * (sf >> 1) + 16 * (hh ^ (sf & 1));
  const int sr = swr(n);
  const int sr_off = kQLat + n * (kRope * 2) + 32 * (sr >> 1) + 16 * (hh ^ (sr & 1));
  // The rows' q^R live in LDS, not in registers (a lane writes and reads only its own
  // chunks): chunk 2 k + hh of row r at (2 k + hh) ^ swr(r), swr(r) = swr(n).
  const int qr_off = kQRq + row * (kRope * 2) + 32 * (sr >> 1) + 16 * (hh ^ (sr & 1));
  // Latent-product operands (A of 32x32x16 from the transposing read): lane 16 g4 + 2 e + q2
  // (hh = g4 / 2, gp = g4 % 2) points at token row e of the group, 16 hs + tpv, and bytes
  // 8 q2 .. +7 of chunk 2 fb + gp (features 32 fb + 16 gp .. +15), at physical
  // (2 fb + gp) ^ swf(tpv): o8_off ^ 32 (fb & 7), plus 256 for fb >= 8, plus 8192 hs.
  const int e8 = (lane & 15) >> 1;
  const int tpv = 8 * (e8 >> 2) + 4 * hh + (e8 & 3);
  const int sp = swf(tpv);
  const int gp = (lane >> 4) & 1;
  const int o8_off = tpv * kLat + 32 * (sp >> 1) + 16 * (gp ^ (sp & 1)) + 8 * (lane & 1);

  // Stage copy plan: copy q (0..23) fills stage bytes [1024 q, 1024 q + 1024); wave w issues
  // copies w + 4 i, i = 0..5.  q < 16: code rows (lane l: token 2 q + l / 32, physical chunk
  // l % 32 holding logical chunk (l % 32) ^ swf(token)); 16..19: k^R rows (token
  // 8 (q - 16) + l / 8, physical chunk l % 8 holding (l % 8) ^ swr(token)); 20: the 32 scales
  // (lanes 8..63 repeat lanes 0..7); 21..23 fetch nothing needed.  Offsets are relative to the
  // start of the region (codes, k^R, scales) of the stage's half page.
  uint32_t cp2[kQCopies / 2];
#pragma unroll
  for (int i = 0; i < kQCopies; ++i) {
    const int q = wave + kWaves * i;
    uint32_t o = 0;
    if (q < 16) {
      const int t = 2 * q + (lane >> 5);
      o = (uint32_t)(t * kLat + 16 * ((lane & 31) ^ swf(t)));
    } else if (q < 20) {
      const int t = 8 * (q - 16) + (lane >> 3);
      o = (uint32_t)(t * (kRope * 2) + 16 * ((lane & 7) ^ swr(t)));
    } else if (q == 20) {
      o = (uint32_t)(16 * (lane & 7));
    }
    if (i & 1) cp2[i >> 1] |= o << 16;
    else cp2[i >> 1] = o;
  }
  auto cp_off = [&](int i) { return (i & 1) ? (cp2[i >> 1] >> 16) : (cp2[i >> 1] & 0xffffu); };

  auto lookup_block = [&](int b, int tok0) {
    return btab[__builtin_amdgcn_readfirstlane(b * max_blocks + tok0 / kBlk)];
  };
  // global start of the stage's three regions (codes, k^R, scales) inside page blk; the
  // stage is the first or second half of the page.  A block id outside the pool is
  // reported and replaced by block 0.
  // Where one stage's copies go: the global start of its three regions (codes, k^R, scales)
  // inside page blk (the stage is the first or second half of the page) and its ring slot.
  // Copy 5 is the scales for wave 0 and a copy of nothing needed for the other waves.  A block
  // id outside the pool is reported and replaced by block 0.  An idle target sends every copy
  // to the spare kilobyte.
  struct Target {
    uint64_t lat, rope, sc5;
    uint32_t dst, stride, dst5;
  };
  const uint64_t idle_base = uniform_addr(pages);
  const uint32_t idle_dst = (uint32_t)(uintptr_t)(lds + kQIdle);
  const Target idle_target{idle_base, idle_base, idle_base, idle_dst, 0u, idle_dst};
  auto target_of = [&](int blk, int tok0, int slot) {
    const bool bad = blk < 0 || blk >= num_blocks;   // wave-uniform; the address math stays scalar
    if (bad && lane == 0 && status) atomicOr(status, MLA_STATUS_BAD_BLOCK);
    const uint32_t ub = __builtin_amdgcn_readfirstlane((uint32_t)(bad ? 0 : blk));
    const uint32_t half = (uint32_t)((tok0 % kBlk) / kSubTok);
    const uint64_t pg = idle_base + (uint64_t)ub * (uint64_t)kFp8PageBytes;
    const uint32_t d0 = (uint32_t)(uintptr_t)(lds + slot * kQStage + 1024 * wave);
    return Target{pg + half * kQLat, pg + kFp8RopeOff + half * kQRope,
                  wave == 0 ? pg + kFp8ScaleOff + half * (kSubTok * 4) : idle_base, d0,
                  (uint32_t)(kWaves * 1024), wave == 0 ? d0 + kWaves * 1024 * 5 : idle_dst};
  };
  // Copy i of this wave; with tlast < 31 (a sequence's last stage) rows past tlast re-read row
  // tlast (the last valid token), so every LDS row holds finite cache data.
  auto copy_i = [&](const Target& T, int i, int tlast) {
    uint32_t o = cp_off(i);
    if (i <= 4 && tlast < kSubTok - 1) {
      const int sh = i < 4 ? 9 : 7;   // log2 of the row bytes (512 codes, 128 of k^R)
      const int over = (int)(o >> sh) - tlast;
      o -= (uint32_t)((over > 0 ? over : 0) << sh);
    }
    const uint64_t base = i < 4 ? T.lat : (i == 4 ? T.rope : T.sc5);
    const uint32_t dst = i < 5 ? T.dst + T.stride * i : T.dst5;
    copy16_to_lds(base, o, __builtin_amdgcn_readfirstlane(dst));
  };

  int seg_i = wgseg[w];
  u32x4 qreg[32];
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

    {
      // code k-step ks < 32 takes features 32 (ks / 2) + 16 hh + 8 (ks % 2) .. +7; k^R k-step
      // 32 + k takes features 512 + 16 k + 8 hh .. +7
      // row r of the absorbed queries (for a padding row, the sequence's row 0, zeroed)
      const size_t r = row_ok ? ((size_t)b * n_heads + head) * sq + s_idx : (size_t)b * n_heads * sq;
#pragma unroll
      for (int ks = 0; ks < 36; ++ks) {
        const int f = ks < 32 ? 32 * (ks >> 1) + 16 * hh + 8 * (ks & 1) : 16 * ks + 8 * hh;
        u32x4 v = *(const u32x4*)(q_lat + qlat_byte(r, f));
        v = row_ok ? v : u32x4{0u, 0u, 0u, 0u};
        if (ks < 32) qreg[ks] = v;
        else *(MLA_LDS u32x4*)(lds + (qr_off ^ (32 * (ks - 32)))) = v;
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
    const int nsub = tok_end > a ? (tok_end - a + kSubTok - 1) / kSubTok : 0;
    auto tlast_of = [&](int k) {
      const int t = tok_end - 1 - (a + k * kSubTok);
      return t < kSubTok - 1 ? t : kSubTok - 1;
    };
#pragma unroll
    for (int k = 0; k < kQAhead; ++k) {
      const Target T = k < nsub ? target_of(lookup_block(b, a + k * kSubTok), a + k * kSubTok, k) : idle_target;
      const int tl = k < nsub ? tlast_of(k) : kSubTok - 1;
#pragma unroll
      for (int i = 0; i < kQCopies; ++i) copy_i(T, i, tl);
    }
    // block ids are looked up one stage ahead of their copies
    int blk_next = kQAhead < nsub ? lookup_block(b, a + kQAhead * kSubTok) : 0;
    // softmax weights (times scales) of the previous stage, bf16 pairs, consumed one iteration later
    // the weights of the (empty) stage before the first: zero
    *(MLA_LDS u32x4*)(lds + kQP + kPBytes + wave * 2048 + lane * 16) = u32x4{0u, 0u, 0u, 0u};
    *(MLA_LDS u32x4*)(lds + kQP + kPBytes + wave * 2048 + 1024 + lane * 16) = u32x4{0u, 0u, 0u, 0u};

    for (int it = 0; it <= nsub; ++it) {
      // This wave's copies of stage it have landed once at most kQAhead - 1 stages' worth
      // (issued later) remain in flight.
      __builtin_amdgcn_s_waitcnt(waitcnt_vm((kQAhead - 1) * kQCopies));
      __syncthreads();   // stage it visible to all waves; stage it - 2 fully consumed
      // The copies of stage it + kQAhead ride along the score MFMAs below; a ragged stage (a
      // sequence's last) goes out here in full, with its rows clamped.
      const int nx = it + kQAhead;
      Target nt = idle_target;
      if (nx < nsub) {
        const Target T = target_of(blk_next, a + nx * kSubTok, nx % kQSlots);
        const int tl = tlast_of(nx);
        if (tl == kSubTok - 1) {
          nt = T;
        } else {
#pragma unroll
          for (int i = 0; i < kQCopies; ++i) copy_i(T, i, tl);
        }
      }
      if (nx + 1 < nsub) blk_next = lookup_block(b, a + (nx + 1) * kSubTok);
      const bool valid = it < nsub;
      const MLA_LDS uint8_t* st = lds + (it % kQSlots) * kQStage;
      const MLA_LDS uint8_t* sto = lds + ((it > 0 ? it - 1 : 0) % kQSlots) * kQStage;
      const int tok0 = a + it * kSubTok;

      // ---- S^T = T . Q^T (32 tokens x 32 rows): 16 code pairs and 4 k^R k-steps in one
      // accumulation chain (dependent MFMAs of one opcode issue back to back).  Lane n's
      // operands are token n's, scaled by its s_n.
      f32x16 acc_s;
      {
        const float s_n = *(const MLA_LDS float*)(st + kQScale + 4 * n);
        u32x4 tv[kPfS];
#pragma unroll
        for (int k = 0; k < kPfS; ++k) tv[k] = lds_read16(st + ((sl_off ^ (32 * (k & 7))) + 256 * (k >> 3)));
        u32x4 rv = lds_read16(st + sr_off);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const u32x4 raw = tv[j % kPfS];
          if (j + kPfS < 16) {
            const int jj = j + kPfS;
            tv[j % kPfS] = lds_read16(st + ((sl_off ^ (32 * (jj & 7))) + 256 * (jj >> 3)));
          }
          const u32x2 c0 = cvt4(raw[0], s_n), c1 = cvt4(raw[1], s_n);
          const u32x2 c2 = cvt4(raw[2], s_n), c3 = cvt4(raw[3], s_n);
          const u32x4 opa = {c0[0], c0[1], c1[0], c1[1]};
          const u32x4 opb = {c2[0], c2[1], c3[0], c3[1]};
          if (j == 0) mfma_sv_first(acc_s, opa, qreg[0]);
          else mfma_sv(acc_s, opa, qreg[0 + 2 * j]);
          mfma_sv(acc_s, opb, qreg[2 * j + 1]);
          if ((j & 3) == 1) {
            // a k^R k-step every fourth pair, alternating chains
            const int k = j >> 2;
            const u32x4 r = rv;
            if (k < 3) rv = lds_read16(st + (sr_off ^ (32 * (k + 1))));
            mfma_s(acc_s, r, lds_read16(lds + (qr_off ^ (32 * k))));
          }
          if (j >= 2 && j < 2 + 2 * kQCopies && (j & 1) == 0) copy_i(nt, (j - 2) >> 1, kSubTok - 1);
        }
        settle_s(acc_s);
      }

      // ---- softmax weights of stage it against the row reference (log2 units; lane holds row
      // n and tokens 8 (r / 4) + 4 hh + r % 4, r = 0..15, whose scales it reads here),
      // interleaved step by step with the latent product of stage it - 1:
      //   O^T += C^T . (P S)^T over this wave's 128 features (4 blocks of 32) x all 128 rows
      //   (4 row blocks) x 2 token halves, 32 MFMAs.  The weights come from LDS, written
      //   there by the wave that owns each row block; each converted tile operand feeds
      //   four MFMAs.
      uint32_t pk[8];
      {
        float z[16], sc[16];
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const f32x4 v = *(const MLA_LDS f32x4*)(st + kQScale + 4 * (8 * qd + 4 * hh));
#pragma unroll
          for (int c = 0; c < 4; ++c) sc[4 * qd + c] = v[c];
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) z[r] = acc_s[r];
        if (!valid || tok0 + kSubTok - 1 > L - sq) {   // past some row's last visible token, or no stage
          asm volatile("");   // a branch taken on a sequence's last stage only: keep it one
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int tok = tok0 + 8 * (r >> 2) + 4 * hh + (r & 3);
            const bool off = !valid || tok > lim;
            z[r] = off ? kNegInf : z[r];
            sc[r] = off ? 0.0f : sc[r];   // a slot past the sequence may hold any bits
          }
        }
        const MLA_LDS uint8_t* pp = lds + kQP + ((it + 1) & 1) * kPBytes + lane * 16;
        // A operand ai = 4 hs + fb: feature block 4 wave + fb, token half hs
        auto rd = [&](int ai) {
          const int hs = ai >> 2, FB = 4 * wave + (ai & 3);
          const u32x2 raw = lds_read_tr8(sto + ((o8_off ^ (32 * (FB & 7))) + 256 * (FB >> 3) + hs * (16 * kLat)));
          const u32x2 c0 = cvt4(raw[0], 1.0f), c1 = cvt4(raw[1], 1.0f);
          return u32x4{c0[0], c0[1], c1[0], c1[1]};
        };
        u32x4 pb[2][4], av[8];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) pb[0][rb] = lds_read16(pp + rb * 2048);
        av[0] = rd(0);
        av[1] = rd(1);
        float mx = 0.0f, msafe = 0.0f;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int jj = 0; jj < 32; ++jj) {
          const int hs = jj >> 4, fb = (jj >> 2) & 3, rb = jj & 3, ai = 4 * hs + fb;
          acc_o[4 * fb + rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(av[ai]), as_bf8(pb[hs][rb]),
                                                                       acc_o[4 * fb + rb], 0, 0, 0);
          if (rb == 0 && ai + 2 < 8) av[ai + 2] = rd(ai + 2);
          if (jj == 8) {
#pragma unroll
            for (int r2 = 0; r2 < 4; ++r2) pb[1][r2] = lds_read16(pp + r2 * 2048 + 1024);
          }
          if (jj == 0) {
            mx = __builtin_fmaxf(__builtin_fmaxf(z[0], __builtin_fmaxf(z[1], z[2])),
                                 __builtin_fmaxf(__builtin_fmaxf(z[3], __builtin_fmaxf(z[4], z[5])), __builtin_fmaxf(z[6], z[7])));
          } else if (jj == 1) {
            mx = fmaxf(mx, __builtin_fmaxf(__builtin_fmaxf(z[8], __builtin_fmaxf(z[9], z[10])),
                                           __builtin_fmaxf(__builtin_fmaxf(z[11], __builtin_fmaxf(z[12], z[13])),
                                                           __builtin_fmaxf(z[14], z[15]))));
          } else if (jj == 2) {
            // the other lane half holds the same row's other 16 tokens
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
            mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * zscale;   // zscale > 0
            m_run = fmaxf(m_run, mx);
            m_ref = m_ref == kNegInf ? mx : m_ref;   // a row's reference: its first finite stage maximum
            bad = bad || (mx > m_ref + kLazyTau);
            msafe = m_ref == kNegInf ? 0.0f : m_ref;
          } else if (jj >= 3 && jj < 27 && (jj - 3) % 3 == 0) {
            const int r = 2 * ((jj - 3) / 3);
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(z[r], zscale, -msafe));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(z[r + 1], zscale, -msafe));
            l_sum += p0 + p1;
            pk[r >> 1] = pack_bf2(p0 * sc[r], p1 * sc[r + 1]);
          } else if (jj == 27) {
            // this stage's weights, for every wave's latent product in the next iteration
            MLA_LDS uint8_t* pw = lds + kQP + (it & 1) * kPBytes + wave * 2048 + lane * 16;
            *(MLA_LDS u32x4*)pw = u32x4{pk[0], pk[1], pk[2], pk[3]};
            *(MLA_LDS u32x4*)(pw + 1024) = u32x4{pk[4], pk[5], pk[6], pk[7]};
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    if (__builtin_amdgcn_ballot_w64(bad) != 0ull && lane == 0) s_retry = 1;
    // every copy of this wave (asm, so not waited for by the compiler) lands before the
    // epilogue or a retried range reuses the ring
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();   // ring free for the next range; every wave's flag visible
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
    again = false;

    // ---- partial state: un-normalised latent sum, reference max and weight sum
    const float l_tot = l_sum + __shfl_xor(l_sum, 32);
    // (rounded to bf16 on the way out, through LDS in passes of 32 rows, one row block each;
    // the ring is free once every wave has left the loop)
    uint16_t* prow = part_o + (size_t)piece * kRowsWG * kLat;
#pragma unroll
    for (int pass = 0; pass < kRowsWG / kEpiRows; ++pass) {
#pragma unroll
      for (int fb = 0; fb < 4; ++fb) {
        const f32x16& A = acc_o[4 * fb + pass];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          stage_row_f4(lds, n, 128 * wave + 32 * fb + 8 * rr + 4 * hh,
                       f32x4{A[4 * rr], A[4 * rr + 1], A[4 * rr + 2], A[4 * rr + 3]});
      }
      __syncthreads();
      store_pass_bf16(lds, prow + (size_t)kEpiRows * pass * kLat, tid);
      __syncthreads();   // LDS free for the next pass (or the next range)
    }
    if (hh == 0) part_ml[(size_t)piece * kRowsWG + row] = make_float2(m_ref, l_tot);
  }
}

hipError_t launch_attn_fp8(const WsLayout& L, const uint8_t* pages, int num_blocks, const int32_t* block_table,
                           int max_blocks, const int32_t* seq_lens, int batch, int sq, int n_heads, float zscale,
                           uint8_t* ws, int32_t* status, hipStream_t st) {
  // grid: W ranges x G head groups, ordered so the groups of a range share an XCD
  const int wpad = (L.W + 7) / 8 * 8;
  dim3 grid(wpad * L.G);
  hipLaunchKernelGGL(attn_fp8_kernel, grid, dim3(kWaves * 64), 0, st, pages, num_blocks, block_table, max_blocks,
                     seq_lens, batch, sq, n_heads, L.hg, L.W, L.P, zscale, ws, L, status);
  return hipGetLastError();
}

}  // namespace mla
