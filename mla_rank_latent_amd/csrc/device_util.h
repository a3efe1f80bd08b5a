// Device-side helpers for the gfx950 kernels: vector types, bf16 rounding,
// wait-count encoding, the split planner and fp64 RoPE.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_internal.h"

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

#define MLA_LDS __attribute__((address_space(3)))

// bf16 bits -> float (exact)
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float -> bf16 bits, round to nearest, ties to even (gfx950's v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// two floats -> packed bf16x2 (low half = a), one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// double -> bf16 bits with a single rounding: first to float rounding toward
// zero with a sticky bit (round-to-odd, exact for the later 8-bit rounding),
// then nearest-even to bf16.
__device__ __forceinline__ uint16_t d2bf(double x) {
  float f = __double2float_rz(x);
  if ((double)f != x) f = __uint_as_float(__float_as_uint(f) | 1u);
  return f2bf(f);
}

// s_waitcnt immediate for gfx9-family: vmcnt = n, expcnt and lgkmcnt left at max.
__host__ __device__ constexpr int waitcnt_vm(int n) {
  return (n & 0xf) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8);
}

// ---------------------------------------------------------------------------
// Split planner: one 256-thread workgroup writes the plan for `batch` sequences into the
// workspace.  seg_start[b] = sum over b' < b of roundup(clamped len, align); the token
// space [0, total) is cut into at most num_wg ranges, range w = [rcut[w], rcut[w + 1]);
// piece_base[b] = number of pieces before sequence b; first_range[b] = the range holding
// sequence b's first token; wg_seg[w] = the sequence holding range w's first token.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int clamp_len(int L, int sq, int max_blocks, int bsz, int32_t* status) {
  int cap = max_blocks * bsz;
  if (L < sq || L > cap) {
    if (status) atomicOr(status, MLA_STATUS_BAD_LENGTH);
    L = L < 0 ? 0 : (L > cap ? cap : L);
  }
  return L;
}

// number of v[0 .. n) below x (lower bound) / at most x (upper bound); v nondecreasing
__device__ __forceinline__ int count_below(const int* v, int n, int x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (v[mid] < x) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}
__device__ __forceinline__ int count_upto(const int* v, int n, int x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (v[mid] <= x) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

__device__ void plan_build(const int32_t* seq_lens, int batch, int sq, int max_blocks, int bsz, int align,
                           int num_wg, uint8_t* ws, const WsLayout& Lw, int32_t* status) {
  __shared__ int s_scan[256];
  __shared__ int s_carry;
  __shared__ int s_cut[kPlanBins];   // range starts of a cost-balanced plan; the quota search's bins
  __shared__ int s_most;
  PlanHeader* hdr = (PlanHeader*)(ws + Lw.off_hdr);
  int32_t* seg = (int32_t*)(ws + Lw.off_seg);
  int32_t* piece = (int32_t*)(ws + Lw.off_piece);
  int32_t* wgseg = (int32_t*)(ws + Lw.off_wgseg);
  int32_t* rcut = (int32_t*)(ws + Lw.off_rcut);
  int32_t* firstr = (int32_t*)(ws + Lw.off_firstr);
  const int t = threadIdx.x;
  // pass 1: prefix sums of rounded lengths -> seg_start, and the total.  With at most 256
  // sequences each thread keeps its segment for pass 2 instead of reading it back, and
  // s_scan[b - 1] keeps boundary b (the start of sequence b) until pass 2.
  int my_s0 = 0, my_s1 = 0;
  if (t == 0) s_carry = 0;
  __syncthreads();
  for (int base = 0; base < batch; base += 256) {
    int b = base + t;
    int v = 0;
    if (b < batch) {
      int L = clamp_len(seq_lens[b], sq, max_blocks, bsz, status);
      v = (L + align - 1) / align * align;
    }
    s_scan[t] = v;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      int add = t >= off ? s_scan[t - off] : 0;
      __syncthreads();
      s_scan[t] += add;
      __syncthreads();
    }
    if (b < batch) {
      my_s0 = s_carry + s_scan[t] - v;
      my_s1 = my_s0 + v;
      seg[b] = my_s0;
    }
    __syncthreads();
    if (t == 255) s_carry += s_scan[255];
    __syncthreads();
  }
  const int total = s_carry;
  if (t == 0) seg[batch] = total;
  int quota = (total + num_wg - 1) / num_wg;
  quota = (quota + align - 1) / align * align;
  if (quota < align) quota = align;
  // A range's partial state (128 rows x 512 bf16 latent sums) is 128 KB, which 114 cached
  // tokens (1152 B each) would cost to read: ranges of the bf16 kernels take at least two
  // 64-token blocks, so that small batches do not write (and merge) more partial-state bytes
  // than the cache bytes they read.
  const int min_range = align == kBlk ? kMinRangeTokens : align;
  if (quota < min_range) quota = min_range;
  // A range that holds a sequence boundary runs a second piece, which costs about
  // kPieceCostTokens of attention work, and the slowest range sets the kernel's time.  When
  // the range count is the library's choice, two plans are weighed by that cost of their
  // slowest range (tokens + kPieceCostTokens per boundary inside), and the cheaper is kept
  // (the even one on ties):
  //  - even ranges of q tokens, q = q0, q0 + align, ... (fewer ranges): the cost is
  //    q + kPieceCostTokens * (most boundaries inside one range).  Batch 4 with
  //    128K/64K/32K/16K contexts gets 240 ranges of 1024 tokens that each hold one
  //    sequence's tokens, not 256 ranges of 960 of which three hold two sequences;
  //  - (up to 256 sequences) cost-balanced ranges: with C(x) = x + kPieceCostTokens *
  //    (boundaries below token x), range w starts where C reaches w / W of its total, at the
  //    next multiple of align, or at the boundary itself when that is at most one align
  //    step back or the cost target falls inside a boundary's step.  Ragged batches, whose
  //    even ranges hold several boundaries each, get ranges that are shorter where they
  //    hold boundaries.
  // Boundaries are seg[1 .. batch-1] below total (multiples of align).
  bool balanced = false;
  int nwb = 0;   // ranges of the balanced plan
  if (Lw.tune && batch > 1 && num_wg <= kPlanBins) {
    int best_q = quota, best_cost = 0x7fffffff;
    for (int c = 0; c < kQuotaTries; ++c) {
      const int q = quota + c * align;
      const int nr = (total + q - 1) / q;   // ranges at this quota (<= num_wg)
      for (int i = t; i < nr; i += 256) s_cut[i] = 0;
      if (t == 0) s_most = 0;
      __syncthreads();
      for (int b = t; b < batch; b += 256) {
        const int s0 = batch <= 256 ? my_s0 : seg[b];   // thread b kept its segment start
        if (b > 0 && s0 < total && s0 % q != 0) atomicAdd(&s_cut[s0 / q], 1);
      }
      __syncthreads();
      int most = 0;
      for (int i = t; i < nr; i += 256) most = s_cut[i] > most ? s_cut[i] : most;
      if (most > 0) atomicMax(&s_most, most);
      __syncthreads();
      const int cost = q + kPieceCostTokens * s_most;
      if (cost < best_cost) {
        best_cost = cost;
        best_q = q;
      }
      const bool done = s_most == 0;   // no boundary inside a range: larger quotas cost more
      __syncthreads();                 // s_cut and s_most are reset by the next try
      if (done) break;
    }
    quota = best_q;
    if (batch <= 256 && best_cost > quota) {
      // boundaries s_scan[0 .. nb) (sequence b + 1 starts at s_scan[b])
      const int nb = count_below(s_scan, batch - 1, total);
      const long long ctot = (long long)total + (long long)kPieceCostTokens * nb;
      long long wl = ctot / min_range;
      wl = wl < 1 ? 1 : wl;
      const int wb = wl < num_wg ? (int)wl : num_wg;
      for (int w = t; w < wb; w += 256) {
        int cut = 0;
        if (w > 0) {
          const long long y = (long long)w * ctot / wb;
          // k = boundaries whose step C has fully passed below y
          int lo = 0, hi = nb;
          while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if ((long long)s_scan[mid] + (long long)kPieceCostTokens * (mid + 1) < y) lo = mid + 1;
            else hi = mid;
          }
          const int sk = lo > 0 ? s_scan[lo - 1] : 0;
          const int sk1 = lo < nb ? s_scan[lo] : total;
          const long long x = y - (long long)kPieceCostTokens * lo;
          long long tc = (x + align - 1) / align * align;
          if (tc > sk1) tc = sk1;
          cut = lo > 0 && (int)tc - sk <= align ? sk : (int)tc;   // sk: a boundary when lo > 0
        }
        s_cut[w] = cut;
      }
      if (t == 0) s_most = 0;
      __syncthreads();
      for (int w = t; w < wb; w += 256) {
        const int lo = s_cut[w], hi = w + 1 < wb ? s_cut[w + 1] : total;
        if (hi > lo) {
          const int inside = count_below(s_scan, nb, hi) - count_upto(s_scan, nb, lo);
          atomicMax(&s_most, hi - lo + kPieceCostTokens * inside);
        }
      }
      __syncthreads();
      balanced = s_most < best_cost;
      nwb = wb;
    }
  }
  __syncthreads();
  // the plan's ranges: their count, where range w starts, and the range holding token x
  // (balanced is uniform: each branch reads the LDS cuts only on the plan that has them)
  const int nw = balanced ? nwb : (total + quota - 1) / quota;
  auto cut_of = [&](int w) {
    if (w >= nw) return total;
    if (balanced) return s_cut[w];
    return w * quota;
  };
  auto range_of = [&](int x) {
    if (balanced) return count_upto(s_cut, nw, x) - 1;
    return x / quota;
  };
  for (int w = t; w <= num_wg; w += 256) rcut[w] = cut_of(w);
  // pass 2: pieces per sequence = number of ranges its segment meets
  if (t == 0) s_carry = 0;
  __syncthreads();
  for (int base = 0; base < batch; base += 256) {
    int b = base + t;
    int v = 0, s0 = 0, s1 = 0, r0 = 0, r1 = -1;
    if (b < batch) {
      s0 = batch <= 256 ? my_s0 : seg[b];
      s1 = batch <= 256 ? my_s1 : seg[b + 1];
      if (s1 > s0) {
        r0 = range_of(s0);
        r1 = range_of(s1 - 1);
        v = r1 - r0 + 1;
      }
    }
    s_scan[t] = v;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      int add = t >= off ? s_scan[t - off] : 0;
      __syncthreads();
      s_scan[t] += add;
      __syncthreads();
    }
    if (b < batch) {
      piece[b] = s_carry + s_scan[t] - v;
      firstr[b] = r0;
      // ranges whose first token falls in this segment start their walk here
      if (s1 > s0) {
        for (int w = cut_of(r0) < s0 ? r0 + 1 : r0; w <= r1; ++w) wgseg[w] = b;
      }
    }
    __syncthreads();
    if (t == 255) s_carry += s_scan[255];
    __syncthreads();
  }
  if (t == 0) {
    piece[batch] = s_carry;
    hdr->total = total;
    hdr->quota = balanced ? 0 : quota;
    hdr->pieces = s_carry;
    hdr->status = 0;
  }
}

// RoPE on one pair at position pos: angle pos * base^(-2i/d), evaluated in fp64.
__device__ __forceinline__ void rope_angle(int pos, int i, int d, double base, double* s, double* c) {
  double theta = pow(base, -2.0 * (double)i / (double)d);
  sincos((double)pos * theta, s, c);
}
__device__ __forceinline__ void rope_pair(double x0, double x1, int pos, int i, int d, double base,
                                          double* y0, double* y1) {
  double s, c;
  rope_angle(pos, i, d, base, &s, &c);
  *y0 = x0 * c - x1 * s;
  *y1 = x0 * s + x1 * c;
}

}  // namespace mla
