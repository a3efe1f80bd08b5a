// Plain fp32 kernels for any MLA widths, plus the query projection for both
// element types.  They compute the same steps as the bf16 MFMA kernels
// ("DeepSeek-V2: Multi-Head Latent Attention (MLA) 原理与工程实现" §2.1 joint
// compression, §2.2 absorption, §3.2 decoupled RoPE) in fp32 throughout, with
// the same split plan and partial-state format, so the split/merge logic is
// exercised at fp32 accuracy as well.  They are sized for small models; the
// DeepSeek-V2 widths in bf16 run on the MFMA kernels.
#include "device_util.h"

namespace mla {

namespace {

__device__ __forceinline__ float ld(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ float ld(const uint16_t* p, size_t i) { return bf2f(p[i]); }
__device__ __forceinline__ void st(float* p, size_t i, double v) { p[i] = (float)v; }
__device__ __forceinline__ void st(uint16_t* p, size_t i, double v) { p[i] = d2bf(v); }

__device__ float block_max(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) r = fmaxf(r, red[w]);
  return r;
}

__device__ float block_sum(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = 0.0f;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) r += red[w];
  return r;
}

}  // namespace

// ---------------------------------------------------------------------------
// append: one thread per (token, rotary pair or latent column); dot products
// accumulate in fp32 in index order, RoPE in fp64.
// ---------------------------------------------------------------------------
__global__ void append_f32_kernel(mla_dims d, const float* __restrict__ h, const float* __restrict__ w_dkv,
                                  const float* __restrict__ w_kr, const int32_t* __restrict__ positions,
                                  const int32_t* __restrict__ block_table, int max_blocks, float* __restrict__ cache,
                                  int num_blocks, int tokens, int t_per_seq, int32_t* status) {
  const int per_tok = d.d_latent + d.d_rope / 2;
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long long)tokens * per_tok) return;
  const int tok = (int)(gid / per_tok);
  const int j = (int)(gid % per_tok);
  const int b = tok / t_per_seq;
  const int pos = positions[tok];
  if (pos < 0 || pos >= max_blocks * d.block_size) {
    if (status) atomicOr(status, MLA_STATUS_BAD_POS);
    return;
  }
  const int blk = block_table[(size_t)b * max_blocks + pos / d.block_size];
  if (blk < 0 || blk >= num_blocks) {
    if (status) atomicOr(status, MLA_STATUS_BAD_BLOCK);
    return;
  }
  const int R = d.d_latent + d.d_rope;
  float* row = cache + ((size_t)blk * d.block_size + pos % d.block_size) * R;
  const float* hv = h + (size_t)tok * d.d_model;
  if (j < d.d_latent) {
    const float* w = w_dkv + (size_t)j * d.d_model;
    float acc = 0.0f;
    for (int k = 0; k < d.d_model; ++k) acc = fmaf(w[k], hv[k], acc);
    row[j] = acc;
  } else {
    const int i = j - d.d_latent;   // rotary pair
    const float* w0 = w_kr + (size_t)(2 * i) * d.d_model;
    const float* w1 = w0 + d.d_model;
    float a0 = 0.0f, a1 = 0.0f;
    for (int k = 0; k < d.d_model; ++k) {
      a0 = fmaf(w0[k], hv[k], a0);
      a1 = fmaf(w1[k], hv[k], a1);
    }
    double y0, y1;
    rope_pair(a0, a1, pos, i, d.d_rope, (double)d.rope_base, &y0, &y1);
    row[d.d_latent + 2 * i] = (float)y0;
    row[d.d_latent + 2 * i + 1] = (float)y1;
  }
}

hipError_t launch_append_f32(const mla_dims* d, const float* h, const float* w_dkv, const float* w_kr,
                             const int32_t* positions, const int32_t* block_table, int max_blocks, float* cache,
                             int num_blocks, int tokens, int t_per_seq, int32_t* status, hipStream_t st) {
  long long n = (long long)tokens * (d->d_latent + d->d_rope / 2);
  dim3 grid((unsigned)((n + 255) / 256));
  hipLaunchKernelGGL(append_f32_kernel, grid, dim3(256), 0, st, *d, h, w_dkv, w_kr, positions, block_table,
                     max_blocks, cache, num_blocks, tokens, t_per_seq, status);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// query projection (both element types): thread per (token, head, nope column
// or rotary pair); fp32 accumulation, RoPE in fp64, one rounding to the type.
// ---------------------------------------------------------------------------
template <typename T>
__global__ void qproj_kernel(mla_dims d, const T* __restrict__ h, const T* __restrict__ w_q,
                             const T* __restrict__ w_qr, const int32_t* __restrict__ positions,
                             T* __restrict__ q_nope, T* __restrict__ q_rope, int tokens) {
  const int per_head = d.d_nope + d.d_rope / 2;
  const int per_tok = d.n_heads * per_head;
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long long)tokens * per_tok) return;
  const int tok = (int)(gid / per_tok);
  const int rem = (int)(gid % per_tok);
  const int head = rem / per_head;
  const int j = rem % per_head;
  const T* hv = h + (size_t)tok * d.d_model;
  if (j < d.d_nope) {
    const T* w = w_q + ((size_t)head * d.d_nope + j) * d.d_model;
    float acc = 0.0f;
    for (int k = 0; k < d.d_model; ++k) acc = fmaf(ld(w, k), ld(hv, k), acc);
    st(q_nope, ((size_t)tok * d.n_heads + head) * d.d_nope + j, (double)acc);
  } else {
    const int i = j - d.d_nope;
    const T* w0 = w_qr + ((size_t)head * d.d_rope + 2 * i) * d.d_model;
    const T* w1 = w0 + d.d_model;
    float a0 = 0.0f, a1 = 0.0f;
    for (int k = 0; k < d.d_model; ++k) {
      float x = ld(hv, k);
      a0 = fmaf(ld(w0, k), x, a0);
      a1 = fmaf(ld(w1, k), x, a1);
    }
    double y0, y1;
    rope_pair(a0, a1, positions[tok], i, d.d_rope, (double)d.rope_base, &y0, &y1);
    size_t base = ((size_t)tok * d.n_heads + head) * d.d_rope + 2 * i;
    st(q_rope, base, y0);
    st(q_rope, base + 1, y1);
  }
}

hipError_t launch_qproj(const mla_dims* d, const void* h, const void* w_q, const void* w_qr, const int32_t* positions,
                        void* q_nope, void* q_rope, int tokens, hipStream_t st) {
  long long n = (long long)tokens * d->n_heads * (d->d_nope + d->d_rope / 2);
  dim3 grid((unsigned)((n + 255) / 256));
  if (d->dtype == MLA_DTYPE_F32)
    hipLaunchKernelGGL(qproj_kernel<float>, grid, dim3(256), 0, st, *d, (const float*)h, (const float*)w_q,
                       (const float*)w_qr, positions, (float*)q_nope, (float*)q_rope, tokens);
  else
    hipLaunchKernelGGL(qproj_kernel<uint16_t>, grid, dim3(256), 0, st, *d, (const uint16_t*)h, (const uint16_t*)w_q,
                       (const uint16_t*)w_qr, positions, (uint16_t*)q_nope, (uint16_t*)q_rope, tokens);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// decode, fp32
// ---------------------------------------------------------------------------
// absorbed query q_lat[m, i] = [W^UK_i^T q^C ‖ q^R]; the last workgroup builds the split plan
__global__ void absorb_f32_kernel(mla_dims d, const float* __restrict__ q_nope, const float* __restrict__ q_rope,
                                  const float* __restrict__ w_uk, const int32_t* __restrict__ seq_lens,
                                  int max_blocks, int batch, int sq, uint8_t* __restrict__ ws, WsLayout Lw,
                                  int32_t* status) {
  if (blockIdx.x == gridDim.x - 1) {
    plan_build(seq_lens, batch, sq, max_blocks, d.block_size, Lw.align, Lw.W, ws, Lw, status);
    return;
  }
  const int H = d.n_heads, R = d.d_latent + d.d_rope;
  const int mh = blockIdx.x;   // m * H + head
  const int head = mh % H;
  float* q_lat = (float*)(ws + Lw.off_qlat);
  const float* qn = q_nope + (size_t)mh * d.d_nope;
  for (int c = threadIdx.x; c < R; c += blockDim.x) {
    float v;
    if (c < d.d_latent) {
      v = 0.0f;
      for (int k = 0; k < d.d_nope; ++k) v = fmaf(qn[k], w_uk[((size_t)head * d.d_nope + k) * d.d_latent + c], v);
    } else {
      v = q_rope[(size_t)mh * d.d_rope + (c - d.d_latent)];
    }
    q_lat[(size_t)mh * R + c] = v;
  }
}

// one workgroup per (range, query row): online softmax over the range in
// chunks of 256 tokens; partial = un-normalised latent sum, reference, weight sum
__global__ __launch_bounds__(256) void attn_f32_kernel(mla_dims d, const float* __restrict__ cache, int num_blocks,
                                                       const int32_t* __restrict__ block_table, int max_blocks,
                                                       const int32_t* __restrict__ seq_lens, int batch, int sq,
                                                       float scale_log2, uint8_t* __restrict__ ws, WsLayout Lw,
                                                       int32_t* status) {
  __shared__ float s_p[256];
  __shared__ int s_row[256];
  __shared__ float s_red[8];
  const int w = blockIdx.x;
  const int r = blockIdx.y;   // row = head * sq + s
  const int H = d.n_heads, R = d.d_latent + d.d_rope, dc = d.d_latent, bs = d.block_size;
  const int head = r / sq, s = r % sq;
  const int32_t* seg = (const int32_t*)(ws + Lw.off_seg);
  const int32_t* piece_base = (const int32_t*)(ws + Lw.off_piece);
  const int32_t* wgseg = (const int32_t*)(ws + Lw.off_wgseg);
  const float* q_lat = (const float*)(ws + Lw.off_qlat);
  float* part_o = (float*)(ws + Lw.off_o);
  float2* part_ml = (float2*)(ws + Lw.off_lse);
  const int32_t* rcut = (const int32_t*)(ws + Lw.off_rcut);
  const int32_t* firstr = (const int32_t*)(ws + Lw.off_firstr);
  const int lo = rcut[w], hi = rcut[w + 1];   // this range's tokens (empty past the plan's ranges)
  if (lo >= hi) return;
  constexpr int kPer = kF32MaxWidth / 256;   // latent columns per thread
  for (int b = wgseg[w]; b < batch; ++b) {
    const int s0 = seg[b], s1 = seg[b + 1];
    if (s0 >= hi) break;
    const int a = max(lo, s0) - s0, e = min(hi, s1) - s0;
    if (a >= e) continue;
    const int piece = piece_base[b] + (w - firstr[b]);
    const int L = min(max(seq_lens[b], 0), max_blocks * bs);
    const int lim = L - sq + s;   // last visible token
    const int tend = min(e, lim + 1);
    const float* q = q_lat + ((size_t)(b * sq + s) * H + head) * R;
    float m_ref = -__builtin_inff(), l_sum = 0.0f;
    float o[kPer];
    for (int k = 0; k < kPer; ++k) o[k] = 0.0f;
    for (int t0 = a; t0 < tend; t0 += 256) {
      const int t = t0 + threadIdx.x;
      float z = -__builtin_inff();
      int rowi = -1;
      if (t < tend) {
        int blk = block_table[(size_t)b * max_blocks + t / bs];
        if (blk < 0 || blk >= num_blocks) {
          if (status) atomicOr(status, MLA_STATUS_BAD_BLOCK);
          blk = 0;
        }
        rowi = blk * bs + t % bs;
        const float* kv = cache + (size_t)rowi * R;
        float acc = 0.0f;
        for (int k = 0; k < R; ++k) acc = fmaf(q[k], kv[k], acc);
        z = acc * scale_log2;
      }
      const float cmax = block_max(z, s_red);
      const float m_new = fmaxf(m_ref, cmax);
      const float alpha = m_ref == -__builtin_inff() ? 0.0f : exp2f(m_ref - m_new);
      const float p = t < tend ? exp2f(z - m_new) : 0.0f;
      s_p[threadIdx.x] = p;
      s_row[threadIdx.x] = rowi;
      const float psum = block_sum(p, s_red);
      l_sum = l_sum * alpha + psum;
      m_ref = m_new;
      __syncthreads();
      const int n = min(256, tend - t0);
      for (int k = 0; k < kPer; ++k) {
        const int c = threadIdx.x + 256 * k;
        if (c >= dc) break;
        float acc = o[k] * alpha;
        for (int j = 0; j < n; ++j) acc = fmaf(s_p[j], cache[(size_t)s_row[j] * R + c], acc);
        o[k] = acc;
      }
      __syncthreads();
    }
    float* op = part_o + ((size_t)piece * Lw.rows + r) * dc;
    for (int k = 0; k < kPer; ++k) {
      const int c = threadIdx.x + 256 * k;
      if (c < dc) op[c] = o[k];
    }
    if (threadIdx.x == 0) part_ml[(size_t)piece * Lw.rows + r] = make_float2(m_ref, l_sum);
  }
}

// merge the partials of one (query, head) and apply W^UV_i
__global__ __launch_bounds__(256) void merge_upv_f32_kernel(mla_dims d, const float* __restrict__ w_uv, int batch,
                                                            int sq, const uint8_t* __restrict__ ws, WsLayout Lw,
                                                            float* __restrict__ out, float* __restrict__ lse) {
  __shared__ float s_o[kF32MaxWidth];
  const int H = d.n_heads, dc = d.d_latent, dn = d.d_nope;
  const int mh = blockIdx.x;
  const int m = mh / H, head = mh % H;
  const int b = m / sq, s = m % sq;
  const int r = head * sq + s;
  const int32_t* piece_base = (const int32_t*)(ws + Lw.off_piece);
  const float2* part_ml = (const float2*)(ws + Lw.off_lse);
  const float* part_o = (const float*)(ws + Lw.off_o);
  const int p0 = piece_base[b], p1 = piece_base[b + 1];
  float Mx = -__builtin_inff();
  for (int p = p0; p < p1; ++p) {
    float2 ml = part_ml[(size_t)p * Lw.rows + r];
    if (ml.y > 0.0f) Mx = fmaxf(Mx, ml.x);
  }
  float den = 0.0f;
  for (int p = p0; p < p1; ++p) {
    float2 ml = part_ml[(size_t)p * Lw.rows + r];
    if (ml.y > 0.0f) den += exp2f(ml.x - Mx) * ml.y;
  }
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
  for (int c = threadIdx.x; c < dc; c += blockDim.x) {
    float acc = 0.0f;
    for (int p = p0; p < p1; ++p) {
      float2 ml = part_ml[(size_t)p * Lw.rows + r];
      if (ml.y > 0.0f) acc = fmaf(exp2f(ml.x - Mx), part_o[((size_t)p * Lw.rows + r) * dc + c], acc);
    }
    s_o[c] = acc * inv;
  }
  __syncthreads();
  for (int j = threadIdx.x; j < dn; j += blockDim.x) {
    const float* wv = w_uv + ((size_t)head * dn + j) * dc;
    float acc = 0.0f;
    for (int c = 0; c < dc; ++c) acc = fmaf(wv[c], s_o[c], acc);
    out[(size_t)mh * dn + j] = acc;
  }
  if (threadIdx.x == 0 && lse != nullptr)
    lse[mh] = den > 0.0f ? (Mx + log2f(den)) * 0.69314718055994531f : -__builtin_inff();
}

hipError_t launch_decode_f32(int phases, const mla_dims* d, const WsLayout& L, const float* q_nope,
                             const float* q_rope, const float* w_uk, const float* w_uv, const float* cache,
                             int num_blocks, const int32_t* block_table, int max_blocks, const int32_t* seq_lens,
                             int batch, int sq, float scale, uint8_t* ws, float* out, float* lse, int32_t* status,
                             hipStream_t st) {
  const int MH = batch * sq * d->n_heads;
  if (phases & 1) {
    hipLaunchKernelGGL(absorb_f32_kernel, dim3(MH + 1), dim3(256), 0, st, *d, q_nope, q_rope, w_uk, seq_lens,
                       max_blocks, batch, sq, ws, L, status);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (phases & 2) {
    hipLaunchKernelGGL(attn_f32_kernel, dim3(L.W, L.rows), dim3(256), 0, st, *d, cache, num_blocks, block_table,
                       max_blocks, seq_lens, batch, sq, scale * 1.4426950408889634f, ws, L, status);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (phases & 4) {
    hipLaunchKernelGGL(merge_upv_f32_kernel, dim3(MH), dim3(256), 0, st, *d, w_uv, batch, sq, (const uint8_t*)ws, L,
                       out, lse);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace mla
