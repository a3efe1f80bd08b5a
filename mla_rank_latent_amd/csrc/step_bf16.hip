// The preparation of a decode step that appends its own tokens, in one launch.
//
// A decode step over a latent cache first appends the step's new tokens (their rows
// [c^KV ‖ k^R] = [W^DKV h ‖ RoPE(W^KR h)], "DeepSeek-V2: Multi-Head Latent Attention (MLA)
// 原理与工程实现" §2.1, §3.2) and then attends with absorbed queries (W^UK_i^T q^C_i, §2.2).
// The append's partial products over slices of d_model, the absorbed queries and the split
// plan depend on nothing from one another, so one grid runs them side by side: block 0
// builds the plan, the next blocks are the append's [64 tokens x 32 columns] tiles of every
// slice, the rest the absorbed queries' (head, 128 columns) blocks.  Each part is the very
// code the stand-alone kernels run (prep_tiles.h), so the results are bit for bit those of
// mla_cache_append followed by mla_decode.  The append's second kernel (the slices summed
// in order, RoPE, the rows written through the block table) follows; the attention reads
// the rows after it.
#include "prep_tiles.h"

namespace mla {

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void step_prepare_bf16_kernel(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ w_dkv, const uint16_t* __restrict__ w_kr,
    int tokens, int d_model, int nslice, float* __restrict__ part, int n_app, const uint16_t* __restrict__ q_nope,
    const uint16_t* __restrict__ q_rope, const uint16_t* __restrict__ w_uk, const int32_t* __restrict__ seq_lens,
    int max_blocks, int batch, int sq, int n_heads, float qscale, uint8_t* __restrict__ ws, WsLayout Lw,
    int32_t* status) {
  constexpr int kLds = prep::kAppendPartialLds > prep::kAbsorbLds ? prep::kAppendPartialLds : prep::kAbsorbLds;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kLds];
  const int bid = blockIdx.x;
  if (bid == 0) {
    plan_build(seq_lens, batch, sq, max_blocks, kBlk, Lw.align, Lw.W, ws, Lw, status);
    return;
  }
  if (bid <= n_app) {
    int ct, tg, sl;
    prep::append_tile_of(bid - 1, kRow / 32, (tokens + 63) / 64, nslice, &ct, &tg, &sl);
    prep::append_partial_tile(h, w_dkv, w_kr, tokens, d_model, nslice, part, (MLA_LDS uint8_t*)smem, ct, tg, sl);
    return;
  }
  prep::absorb_tile(q_nope, q_rope, w_uk, batch, sq, n_heads, qscale, ws, Lw, (MLA_LDS uint8_t*)smem,
                    bid - 1 - n_app);
}

hipError_t launch_step_prepare_bf16(const uint16_t* h, const uint16_t* w_dkv, const uint16_t* w_kr,
                                    const int32_t* positions, const int32_t* block_table, int max_blocks,
                                    uint16_t* cache, int num_blocks, int t_per_seq, int d_model, float rope_base,
                                    float* part, const WsLayout& L, const uint16_t* q_nope, const uint16_t* q_rope,
                                    const uint16_t* w_uk, const int32_t* seq_lens, int batch, int sq, int n_heads,
                                    float qscale, uint8_t* ws, int32_t* status, hipStream_t st) {
  const int tokens = batch * t_per_seq;
  const int nslice = append_split_slices(d_model);
  const int n_app = (kRow / 32) * ((tokens + 63) / 64) * nslice;
  dim3 grid(1 + n_app + 4 * n_heads);
  hipLaunchKernelGGL(step_prepare_bf16_kernel, grid, dim3(256), 0, st, h, w_dkv, w_kr, tokens, d_model, nslice, part,
                     n_app, q_nope, q_rope, w_uk, seq_lens, max_blocks, batch, sq, n_heads, qscale, ws, L, status);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_append_finish_bf16(part, nslice, positions, block_table, max_blocks, cache, num_blocks, tokens,
                                   t_per_seq, rope_base, status, st);
}

}  // namespace mla
