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
// Split planner: one 256-thread workgroup writes the plan for `batch`
// sequences into the workspace.  seg_start[b] = sum over b' < b of
// roundup(clamped len, align); piece_base[b] = number of pieces before
// sequence b; wg_seg[w] = the sequence holding token w * quota.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int clamp_len(int L, int sq, int max_blocks, int bsz, int32_t* status) {
  int cap = max_blocks * bsz;
  if (L < sq || L > cap) {
    if (status) atomicOr(status, MLA_STATUS_BAD_LENGTH);
    L = L < 0 ? 0 : (L > cap ? cap : L);
  }
  return L;
}

__device__ void plan_build(const int32_t* seq_lens, int batch, int sq, int max_blocks, int bsz, int align,
                           int num_wg, uint8_t* ws, const WsLayout& Lw, int32_t* status) {
  __shared__ int s_scan[256];
  __shared__ int s_carry;
  PlanHeader* hdr = (PlanHeader*)(ws + Lw.off_hdr);
  int32_t* seg = (int32_t*)(ws + Lw.off_seg);
  int32_t* piece = (int32_t*)(ws + Lw.off_piece);
  int32_t* wgseg = (int32_t*)(ws + Lw.off_wgseg);
  const int t = threadIdx.x;
  // pass 1: prefix sums of rounded lengths -> seg_start, and the total.  With at most 256
  // sequences each thread keeps its segment for pass 2 instead of reading it back.
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
  if (align == kBlk && quota < kMinRangeTokens) quota = kMinRangeTokens;
  // A range that holds a sequence boundary runs a second piece, which costs about
  // kPieceCostTokens of attention work, and the slowest range sets the kernel's time.  When
  // the range count is the library's choice, quotas q0, q0 + align, ... (fewer ranges) are
  // weighed by q + kPieceCostTokens * (most boundaries inside one range), and the cheapest is
  // taken (the first on ties): batch 4 with 128K/64K/32K/16K contexts, for one, gets 240
  // ranges of 1024 tokens that each hold one sequence's tokens only, not 256 ranges of 960
  // of which three hold two sequences.  Boundaries at seg[1 .. batch-1] (multiples of align).
  if (Lw.tune && batch > 1 && num_wg <= kPlanBins) {
    __shared__ int s_bins[kPlanBins];
    __shared__ int s_most;
    int best_q = quota, best_cost = 0x7fffffff;
    for (int c = 0; c < kQuotaTries; ++c) {
      const int q = quota + c * align;
      const int nr = (total + q - 1) / q;   // ranges at this quota (<= num_wg)
      for (int i = t; i < nr; i += 256) s_bins[i] = 0;
      if (t == 0) s_most = 0;
      __syncthreads();
      for (int b = t; b < batch; b += 256) {
        const int s0 = batch <= 256 ? my_s0 : seg[b];   // thread b kept its segment start
        if (b > 0 && s0 < total && s0 % q != 0) atomicAdd(&s_bins[s0 / q], 1);
      }
      __syncthreads();
      int most = 0;
      for (int i = t; i < nr; i += 256) most = s_bins[i] > most ? s_bins[i] : most;
      if (most > 0) atomicMax(&s_most, most);
      __syncthreads();
      const int cost = q + kPieceCostTokens * s_most;
      if (cost < best_cost) {
        best_cost = cost;
        best_q = q;
      }
      const bool done = s_most == 0;   // no boundary inside a range: larger quotas cost more
      __syncthreads();                 // s_bins and s_most are reset by the next try
      if (done) break;
    }
    quota = best_q;
  }
  __syncthreads();
  // pass 2: pieces per sequence = number of ranges its segment meets
  if (t == 0) s_carry = 0;
  __syncthreads();
  for (int base = 0; base < batch; base += 256) {
    int b = base + t;
    int v = 0, s0 = 0, s1 = 0;
    if (b < batch) {
      s0 = batch <= 256 ? my_s0 : seg[b];
      s1 = batch <= 256 ? my_s1 : seg[b + 1];
      v = s1 > s0 ? (s1 - 1) / quota - s0 / quota + 1 : 0;
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
      // ranges whose first token falls in this segment start their walk here
      if (s1 > s0) {
        for (int w = (s0 + quota - 1) / quota; w * quota < s1 && w < num_wg; ++w) wgseg[w] = b;
      }
    }
    __syncthreads();
    if (t == 255) s_carry += s_scan[255];
    __syncthreads();
  }
  if (t == 0) {
    piece[batch] = s_carry;
    hdr->total = total;
    hdr->quota = quota;
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
