// Log-sum-exp merge of the split partial states and the W^UV up-projection,
// gfx950 bf16 MFMA with fp32 accumulate.
//
// Each range of cached tokens left, per query row, an un-normalised latent
// sum O_k = sum_j 2^(z_j - m_k) c_j (bf16) with its reference m_k and weight
// sum l_k (log2 units).  The exact merge is
//   M = max_k m_k,  w_k = 2^(m_k - M),
//   o_lat = sum_k w_k O_k / sum_k w_k l_k,   lse = ln 2 * (M + log2 sum_k w_k l_k).
// Then the value side of matrix absorption ("DeepSeek-V2: Multi-Head Latent
// Attention (MLA) 原理与工程实现" §2.2: sum_j p_j W^UV_i c_j = W^UV_i sum_j p_j c_j)
// restores the head's output, out_i = W^UV_i o_lat (W^UV_i = rows 128 i ..
// 128 i + 127 of W^UV, §2.1).
//
// One workgroup of eight waves per (head, 32 query rows), or two (each with half of the
// head's output columns) when all query rows fit one block of 32.
//  - Merge: sixteen threads per row, each owning 32 of its 512 columns
//    (8 bytes at 128-byte strides, so the sixteen lanes of a row read whole
//    128-byte blocks).  Up to four pieces' loads are in flight per thread and the
//    piece weights are applied branch-free, so the partial states stream at
//    memory rate instead of one round trip per piece.  Rows with many pieces (small
//    batches) split them over several thread slots, shared out in proportion to the
//    rows' piece counts and combined through LDS.
//  - The merged latent goes to LDS as a bf16 high part and a bf16 remainder
//    (two MFMAs per step keep the product close to fp32 accuracy).
//  - A block with one query row (batch 1 at one query token) takes the row in fp32 and
//    multiplies it with the W^UV slice on the vector units (each output column a product of
//    512, split over 4 or 8 adjacent threads); otherwise:
//  - Up-projection [32 x 512] . [512 x columns] on MFMA 32x32x16, computed
//    transposed so that each lane ends with four adjacent output columns per
//    register group (8-byte stores): each wave takes 32 output columns over one
//    latent part (halves with 128 columns per workgroup, quarters with 64), with its
//    W^UV slice loaded into registers before the merge starts; the parts are
//    summed through LDS in part order.
#include "device_util.h"

namespace mla {

namespace {
__device__ __forceinline__ bf16x8 as_bf8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
constexpr int kMergeRows = 32;
}  // namespace

// NCS = workgroups per (head, row block), each taking 128 / NCS output columns: 1 when the
// rows fill several blocks (the blocks of a head then share its W^UV slice in L2), 2 for a
// single block (small batches), so that twice the workgroups each load half the slice.
template <int NCS>
__global__ __launch_bounds__(512) void merge_upv_bf16_kernel(const uint16_t* __restrict__ w_uv, int batch, int sq,
                                                             int n_heads, int hg, int P,
                                                             const uint8_t* __restrict__ ws, WsLayout Lw,
                                                             uint16_t* __restrict__ out, float* __restrict__ lse) {
  // hi and lo parts of the merged latent (32 rows x 512, swizzled 16-byte chunks), then
  // the slots' partial sums when rows are shared by several slots (32 x 512 fp32), whose
  // space later takes the latent parts' partial products (up to 3 x 32 x 64 fp32)
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kMergeRows * kLat * 2 + kMergeRows * kLat * 4];
  __shared__ float s_mx[kMergeRows], s_den[kMergeRows];
  __shared__ int s_first[kMergeRows / 2], s_nsl[kMergeRows / 2];   // a shared row's first slot and slot count
  MLA_LDS uint8_t* s_hi = (MLA_LDS uint8_t*)smem;
  MLA_LDS uint8_t* s_lo = s_hi + kMergeRows * kLat * 2;
  MLA_LDS uint8_t* s_comb = s_lo + kMergeRows * kLat * 2;
  MLA_LDS float* s_red = (MLA_LDS float*)s_comb;

  constexpr int kCols = kNope / NCS;        // output columns of the workgroup
  constexpr int kWc = kCols / 32;           // 32-column blocks: 4 or 2
  constexpr int kParts = 8 / kWc;           // latent parts: 2 or 4
  constexpr int kSteps = kLat / kParts / 16;   // k-steps of 16 per part: 16 or 8
  const int M = batch * sq;
  const int nmb = (M + kMergeRows - 1) / kMergeRows;
  // the column parts of a (head, row block) take ids n_heads * nmb apart (one XCD when
  // that is a multiple of 8), the row blocks of a head ids n_heads apart
  const int h = blockIdx.x % n_heads;
  const int mb = (blockIdx.x / n_heads) % nmb;
  const int ch = blockIdx.x / (n_heads * nmb);
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int hh = lane >> 5;
  const int n = lane & 31;
  const int kp = wave / kWc;    // latent part of the up-projection
  const int wc = wave % kWc;    // output column block
  const int col0 = ch * kCols + 32 * wc;

  // The rows' piece ranges are loaded first: the memory wait for them then leaves the W^UV
  // slice below in flight.  Lane k < rv of every wave holds row k's when rows are shared
  // out (rv <= 16, see the merge), else every slot its own row's.
  const int rv = M - mb * kMergeRows < kMergeRows ? M - mb * kMergeRows : kMergeRows;
  const bool shared_rows = rv <= kMergeRows / 2;
  const int slot = tid >> 4;
  const int c16 = tid & 15;
  int i = slot, pl = 0, npl = 1;   // row within the block, piece lane of the row, its slots
  bool row_ok = slot < rv;
  int pb0 = 0, pb1 = 0;
  if (shared_rows ? lane < rv : row_ok) {
    const int32_t* piece_base = (const int32_t*)(ws + Lw.off_piece);
    const int bk = (mb * kMergeRows + (shared_rows ? lane : i)) / sq;
    pb0 = piece_base[bk];
    pb1 = piece_base[bk + 1];
  }

  // The workgroup's W^UV slice, loaded before the merge starts.  Several rows: the B operand
  // of the MFMA up-projection (K = latent, N = output column), lane holding
  // W^UV[128 h + col0 + n][kLat / kParts * kp + 16 ks + 8 hh .. +7], ks = 0 .. kSteps - 1.
  // One row (rv = 1: batch 1 at one query token): a product of the row with the slice, thread
  // t holding latent elements 8 (t % kTpc + kTpc ks) .. +7, ks = 0 .. kSteps - 1, of output
  // column t / kTpc of the workgroup's kCols (the kTpc threads of a column read whole 128-byte
  // runs of its row at each step).
  constexpr int kTpc = 512 / kCols;   // threads per output column on the one-row path
  static_assert(kTpc * 8 * kSteps == kLat, "one-row slice covers the latent");
  u32x4 bop[kSteps];
  if (rv == 1) {
    const uint16_t* wp = w_uv + ((size_t)h * kNope + ch * kCols + tid / kTpc) * kLat + (tid % kTpc) * 8;
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks) bop[ks] = *(const u32x4*)(wp + 8 * kTpc * ks);
  } else {
    const uint16_t* wp = w_uv + ((size_t)h * kNope + col0 + n) * kLat + (kLat / kParts) * kp + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks) bop[ks] = *(const u32x4*)(wp + 16 * ks);
  }

  // ---- merge.  Sixteen threads (a slot) own one row's 512 columns: thread c16 of a slot
  // holds columns 64 j + 4 c16 .. +3, j = 0..7.  With rv <= 16 valid rows (small batches,
  // whose sequences are split into many pieces) the 32 slots are shared out by piece
  // count: each row takes one slot, and the other 32 - rv go to the rows in proportion to
  // their pieces (rounded down), so a long sequence's row, which sets the block's time,
  // takes the most.  A row's slots are consecutive and take every npl-th piece; their
  // states are combined through LDS in slot order.
  {
    const int g = h / hg;
    if (rv > 1 && rv < kMergeRows) {
      // rows without a slot (or past M) must still hold finite values for the MFMAs
      for (int k = tid; k < kMergeRows * kLat / 4; k += 512) {
        ((MLA_LDS u32x2*)s_hi)[k] = u32x2{0u, 0u};
        ((MLA_LDS u32x2*)s_lo)[k] = u32x2{0u, 0u};
      }
      __syncthreads();   // the rows' own values land after the fill
    }
    int p0 = g * P + pb0, p1 = g * P + pb1;
    if (shared_rows) {
      // the shares, from the rows' counts in scalar registers
      int tot = 0;
#pragma unroll
      for (int k = 0; k < kMergeRows / 2; ++k) tot += __builtin_amdgcn_readlane(pb1 - pb0, k);
      const int ns = 1 + (tot > 0 ? (pb1 - pb0) * (kMergeRows - rv) / tot : 0);   // lane k < rv: row k's slots
      int start = 0, my_start = 0;
      row_ok = false;
      i = 0;   // a slot left over keeps row 0 and no pieces
#pragma unroll
      for (int k = 0; k < kMergeRows / 2; ++k) {
        if (k < rv) {
          const int nk = __builtin_amdgcn_readlane(ns, k);
          const int b0k = __builtin_amdgcn_readlane(pb0, k), b1k = __builtin_amdgcn_readlane(pb1, k);
          if (slot >= start && slot < start + nk) {
            i = k;
            pl = slot - start;
            npl = nk;
            row_ok = true;
            p0 = g * P + b0k;
            p1 = g * P + b1k;
          }
          if (lane == k) my_start = start;
          start += nk;
        }
      }
      if (wave == 0 && lane < rv) {
        s_first[lane] = my_start;
        s_nsl[lane] = ns;
      }
    }
    const int m = mb * kMergeRows + i;
    f32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float den = 0.0f, Mx = -__builtin_inff();
    int r = 0;
    const float2* part_ml = (const float2*)(ws + Lw.off_lse);
    const uint16_t* part_o = (const uint16_t*)(ws + Lw.off_o);   // bf16
    if (row_ok) {
      const int b = m / sq;
      const int s = m - b * sq;
      r = (h - g * hg) * sq + s;
      // online merge: the running maximum rises as pieces arrive and the sums so far are
      // rescaled; up to four pieces' loads (states and weights together) share one round trip
      for (int p = p0 + pl; p < p1; p += 4 * npl) {
        int q[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) q[k] = p + k * npl < p1 ? p + k * npl : p;   // past the end: weight 0
        float2 ml[4];
        u32x2 bv[4][8];
#pragma unroll
        for (int k = 0; k < 4; ++k) ml[k] = part_ml[(size_t)q[k] * Lw.rows + r];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const u32x2* o = (const u32x2*)(part_o + ((size_t)q[k] * Lw.rows + r) * kLat) + c16;
#pragma unroll
          for (int j = 0; j < 8; ++j) bv[k][j] = o[16 * j];
        }
        // an empty piece has l = 0 (m = -inf, O = 0): weight 0
        float mk[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) mk[k] = ((k == 0 || q[k] != p) && ml[k].y > 0.0f) ? ml[k].x : -__builtin_inff();
        // no branch on the weights: the states' loads then issue with the weights' in one
        // round trip.  Nothing seen yet (mn = -inf) gives sc = 0 and w = 0: the sums stay 0.
        const float mn = fmaxf(fmaxf(Mx, fmaxf(mk[0], mk[1])), fmaxf(mk[2], mk[3]));
        const float sc = Mx == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(Mx - mn);
        float w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) w[k] = mk[k] == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(mk[k] - mn);
        auto widen = [](u32x2 v) {
          return f32x4{__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xffff0000u), __uint_as_float(v[1] << 16),
                       __uint_as_float(v[1] & 0xffff0000u)};
        };
        den = den * sc + w[0] * ml[0].y + w[1] * ml[1].y + w[2] * ml[2].y + w[3] * ml[3].y;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          acc[j] = acc[j] * sc + w[0] * widen(bv[0][j]) + w[1] * widen(bv[1][j]) + w[2] * widen(bv[2][j]) +
                   w[3] * widen(bv[3][j]);
        Mx = mn;
      }
    }
    // the merged row, normalised, as a bf16 high part and remainder: columns 64 j + 4 c16 .. +3
    // are half (c16 & 1) of logical chunk 8 j + c16 / 2, stored at chunk 8 j + ((c16 / 2) ^ (i % 8))
    auto put_row = [&](int ii, int cc, const f32x4* a, float inv) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        u32x2 vh, vl;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float x0 = a[j][2 * e] * inv, x1 = a[j][2 * e + 1] * inv;
          const uint32_t hp = pack_bf2(x0, x1);
          vh[e] = hp;
          vl[e] = pack_bf2(x0 - bf2f((uint16_t)(hp & 0xffffu)), x1 - bf2f((uint16_t)(hp >> 16)));
        }
        const int off = ii * (kLat * 2) + (8 * j + ((cc >> 1) ^ (ii & 7))) * 16 + 8 * (cc & 1);
        *(MLA_LDS u32x2*)(s_hi + off) = vh;
        *(MLA_LDS u32x2*)(s_lo + off) = vl;
      }
    };
    auto put_lse = [&](int mm, float mx, float dn) {
      if (lse != nullptr && ch == 0)
        lse[(size_t)mm * n_heads + h] = dn > 0.0f ? (mx + __builtin_amdgcn_logf(dn)) * 0.69314718055994531f
                                                  : -__builtin_inff();
    };
    if (rv > kMergeRows / 2) {
      if (row_ok) {
        if (c16 == 0) put_lse(m, Mx, den);
        put_row(i, c16, acc, den > 0.0f ? 1.0f / den : 0.0f);
      }
    } else {
      // A row's slots leave their sums, maxima and weight sums in LDS; every thread then
      // finishes some (row, column-quad) pairs, bringing the row's slots to the row's maximum
      // and adding them in slot order (npl reads per pair, 128 threads per row).
      MLA_LDS f32x4* comb = (MLA_LDS f32x4*)s_comb;
#pragma unroll
      for (int j = 0; j < 8; ++j) comb[(slot * 16 + c16) * 8 + j] = acc[j];
      if (c16 == 0) {
        s_mx[slot] = Mx;
        s_den[slot] = den;
      }
      __syncthreads();
      for (int task = tid; task < rv * 128; task += 512) {
        // a wave's 64 tasks share their row: the slot range and the maxima are uniform
        const int ii = __builtin_amdgcn_readfirstlane(task >> 7), quad = task & 127, jj = quad >> 4, cc = quad & 15;
        const int q0 = __builtin_amdgcn_readfirstlane(s_first[ii]);
        const int q1 = q0 + __builtin_amdgcn_readfirstlane(s_nsl[ii]);
        float mg = -__builtin_inff();
#pragma unroll 8
        for (int q = q0; q < q1; ++q) mg = fmaxf(mg, s_mx[q]);
        f32x4 sum = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        float dn = 0.0f;
#pragma unroll 8
        for (int q = q0; q < q1; ++q) {
          const float mq = s_mx[q];
          const float wq = mq == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(mq - mg);   // slot without weight: 0
          sum += comb[(q * 16 + cc) * 8 + jj] * wq;
          dn += s_den[q] * wq;
        }
        if (quad == 0) put_lse(mb * kMergeRows + ii, mg, dn);
        const float inv = dn > 0.0f ? 1.0f / dn : 0.0f;
        if (rv == 1) {   // the one row, fp32, for the one-row product: columns 64 jj + 4 cc .. +3
          *(MLA_LDS f32x4*)((MLA_LDS float*)s_hi + 64 * jj + 4 * cc) = sum * inv;
          continue;
        }
        u32x2 vh, vl;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float x0 = sum[2 * e] * inv, x1 = sum[2 * e + 1] * inv;
          const uint32_t hp = pack_bf2(x0, x1);
          vh[e] = hp;
          vl[e] = pack_bf2(x0 - bf2f((uint16_t)(hp & 0xffffu)), x1 - bf2f((uint16_t)(hp >> 16)));
        }
        const int off = ii * (kLat * 2) + (8 * jj + ((cc >> 1) ^ (ii & 7))) * 16 + 8 * (cc & 1);
        *(MLA_LDS u32x2*)(s_hi + off) = vh;
        *(MLA_LDS u32x2*)(s_lo + off) = vl;
      }
    }
  }
  __syncthreads();

  if (rv == 1) {
    // ---- one row: out[column] = W^UV row . o_lat in fp32, the kTpc partial sums of a column
    // (adjacent lanes) added by a butterfly in a fixed order
    const MLA_LDS float* ol = (const MLA_LDS float*)s_hi + (tid % kTpc) * 8;
    float a = 0.0f;
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks) {
      const f32x4 o0 = *(const MLA_LDS f32x4*)(ol + 8 * kTpc * ks);
      const f32x4 o1 = *(const MLA_LDS f32x4*)(ol + 8 * kTpc * ks + 4);
      const u32x4 wv = bop[ks];
      a += bf2f((uint16_t)(wv[0] & 0xffffu)) * o0[0] + bf2f((uint16_t)(wv[0] >> 16)) * o0[1] +
           bf2f((uint16_t)(wv[1] & 0xffffu)) * o0[2] + bf2f((uint16_t)(wv[1] >> 16)) * o0[3] +
           bf2f((uint16_t)(wv[2] & 0xffffu)) * o1[0] + bf2f((uint16_t)(wv[2] >> 16)) * o1[1] +
           bf2f((uint16_t)(wv[3] & 0xffffu)) * o1[2] + bf2f((uint16_t)(wv[3] >> 16)) * o1[3];
    }
#pragma unroll
    for (int off = kTpc / 2; off >= 1; off >>= 1) a += __shfl_xor(a, off);
    if (tid % kTpc == 0) out[((size_t)(mb * kMergeRows) * n_heads + h) * kNope + ch * kCols + tid / kTpc] = f2bf(a);
    return;
  }

  // ---- out[32 rows x 32 cols of this wave] over latent part kp
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
  for (int ks = 0; ks < kSteps; ++ks) {
    const int chunk = (kLat / kParts / 8) * kp + 2 * ks + hh;
    const int off = n * (kLat * 2) + ((chunk & ~7) | ((chunk & 7) ^ (n & 7))) * 16;
    const u32x4 ah = *(const MLA_LDS u32x4*)(s_hi + off);
    const u32x4 al = *(const MLA_LDS u32x4*)(s_lo + off);
    // operands in swapped roles: the product is out^T, [output column x row]
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(bop[ks]), as_bf8(ah), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(bop[ks]), as_bf8(al), acc, 0, 0, 0);
  }
  // out^T layout: lane holds row n, register r column 32 wc + 8 (r / 4) + 4 hh + r % 4, so each
  // group of four registers is four adjacent columns.  Parts 1 .. kParts - 1 go through LDS
  // (the combine's space is free again), part 0 adds them in part order and stores.
  if (kp > 0) {
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *(MLA_LDS f32x4*)(s_red + ((kp - 1) * kMergeRows + n) * kCols + 32 * wc + 8 * g + 4 * hh) =
          f32x4{acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
  }
  __syncthreads();
  if (kp == 0) {
    const int m = mb * kMergeRows + n;
    if (m < M) {
      uint16_t* dst = out + ((size_t)m * n_heads + h) * kNope + col0 + 4 * hh;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 v = f32x4{acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
#pragma unroll
        for (int q = 1; q < kParts; ++q)
          v += *(const MLA_LDS f32x4*)(s_red + ((q - 1) * kMergeRows + n) * kCols + 32 * wc + 8 * g + 4 * hh);
        *(u32x2*)(dst + 8 * g) = u32x2{pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3])};
      }
    }
  }
}

hipError_t launch_merge_upv_bf16(const WsLayout& L, const uint16_t* w_uv, int batch, int sq, int n_heads, uint8_t* ws,
                                 uint16_t* out, float* lse, hipStream_t st) {
  const int M = batch * sq;
  const int nmb = (M + kMergeRows - 1) / kMergeRows;
  if (nmb == 1) {
    hipLaunchKernelGGL(merge_upv_bf16_kernel<2>, dim3(n_heads * 2), dim3(512), 0, st, w_uv, batch, sq, n_heads, L.hg,
                       L.P, (const uint8_t*)ws, L, out, lse);
  } else {
    hipLaunchKernelGGL(merge_upv_bf16_kernel<1>, dim3(n_heads * nmb), dim3(512), 0, st, w_uv, batch, sq, n_heads,
                       L.hg, L.P, (const uint8_t*)ws, L, out, lse);
  }
  return hipGetLastError();
}

}  // namespace mla
