// Internal declarations shared by the HIP kernels and the host entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "mla.h"

namespace mla {

// ---------------------------------------------------------------------------
// Fixed widths of the bf16 MFMA kernels (DeepSeek-V2's MLA: d_c = 512,
// d_h^R = 64, d_h = 128, as the DeepSeek-V2 MLA page gives in §1.1 and §3.3).
// ---------------------------------------------------------------------------
constexpr int kLat = 512;            // d_latent
constexpr int kRope = 64;            // d_rope
constexpr int kRow = kLat + kRope;   // cached row: [c^KV ‖ k^R]
constexpr int kNope = 128;           // d_nope
constexpr int kBlk = 64;             // tokens per cache block
constexpr int kRowsWG = 128;         // query rows (head, query-token) per attention workgroup
constexpr int kSubTok = 32;          // tokens per LDS stage
constexpr int kStages = 4;           // LDS ring depth
constexpr int kStageBytes = kSubTok * kRow * 2;        // 36864
constexpr int kChunksPerRow = kRow * 2 / 16;           // 72 chunks of 16 B
constexpr int kMaxSqBf16 = 8;
constexpr int kMinRangeTokens = 2 * kBlk;   // smallest token range of the bf16 split plan
// What a range pays for each sequence boundary inside it (a second piece: another query
// load, another partial state written, the copy pipeline refilled), in cached tokens'
// worth of attention work: 14.9 us measured at 960-token ranges and ~1.9 GHz, ~234 tokens.
constexpr int kPieceCostTokens = 4 * kBlk;
constexpr int kQuotaTries = 8;              // quotas the planner weighs (q0, q0 + align, ...)
constexpr int kPlanBins = 512;              // most ranges the planner weighs them for
// FP8 latent cache page (MLA_DTYPE_BF16_FP8): 64 rows of E4M3 codes, then 64 bf16
// k^R rows, then 64 fp32 scales
constexpr int kFp8RopeOff = kBlk * kLat;                       // 32768
constexpr int kFp8ScaleOff = kFp8RopeOff + kBlk * kRope * 2;   // 40960
constexpr int kFp8PageBytes = kFp8ScaleOff + kBlk * 4;         // 41216

// Absorbed queries of the bf16 kernels, in the order the attention kernels load them.
// Query row r = (b n_heads + head) sq + s (a sequence's heads, each with its query
// tokens); rows in blocks of 32; inside a block, 16-feature step ks (0..35) takes 1 KB,
// in which lane 32 hh + (r % 32) holds features 16 ks + 8 hh .. +7 of row r: the
// operand layout of MFMA 32x32x16 with the rows on its 32-wide side.  A wave that reads
// 32 consecutive rows then loads whole 1 KB runs.
constexpr int kQBlockRows = 32;
constexpr size_t kQBlockBytes = (size_t)kQBlockRows * kRow * 2;   // 36864
__host__ __device__ inline size_t qlat_padded_rows(size_t rows) {
  return (rows + kQBlockRows - 1) / kQBlockRows * kQBlockRows;
}
// byte offset of feature f (0..575) of row r
__host__ __device__ inline size_t qlat_byte(size_t r, int f) {
  return (r / kQBlockRows) * kQBlockBytes + (size_t)(f >> 4) * 1024 +
         (size_t)((((f >> 3) & 1) * kQBlockRows) + (int)(r % kQBlockRows)) * 16 + (size_t)(f & 7) * 2;
}

// f32 generic path limits
constexpr int kF32MaxWidth = 1024;
constexpr int kF32MaxSq = 64;

// ---------------------------------------------------------------------------
// Split plan.  The per-group token space is the concatenation over sequences
// of seq_len rounded up to `align`; it is cut into at most `num_wg` ranges (equal ones of
// `quota` tokens, or cost-balanced ones, quota 0), range w = [rcut[w], rcut[w + 1]).  Every
// (range, sequence) intersection is one piece with its own partial softmax state.  Written
// on the device by plan_build().
// ---------------------------------------------------------------------------
struct PlanHeader {
  int32_t total;      // tokens in the (rounded) space of one head group
  int32_t quota;      // tokens per range (multiple of align); 0 for cost-balanced ranges
  int32_t pieces;     // pieces per head group
  int32_t status;     // reserved
};

// Workspace layout, computed identically by the size query and by decode.
struct WsLayout {
  int G;              // head groups
  int hg;             // heads per group
  int rows;           // query rows per group (padded for bf16)
  int W;              // ranges (workgroups) per head group
  int P;              // max pieces per head group = W + batch
  int align;          // token alignment of ranges
  int tune;           // the range count was left to the library: the planner may use fewer
  size_t off_hdr, off_seg, off_piece, off_wgseg, off_rcut, off_firstr, off_qlat, off_lse, off_o, total;
};

bool ws_layout(const mla_dims* d, int batch, int sq, int num_splits, WsLayout* L);
int device_cu_count();

// ---------------------------------------------------------------------------
// Launchers (one per kernel family).  Each returns hipSuccess or the launch error.
// ---------------------------------------------------------------------------
// split append: K slices, workspace bytes, launcher (workspace = fp32 partial products)
int append_split_slices(int d_model);
size_t append_split_ws_bytes(int d_model, long long tokens);
hipError_t launch_append_split_bf16(const uint16_t* h, const uint16_t* w_dkv, const uint16_t* w_kr,
                                    const int32_t* positions, const int32_t* block_table, int max_blocks,
                                    uint16_t* cache, int num_blocks, int tokens, int t_per_seq, int d_model,
                                    float rope_base, float* ws, int32_t* status, hipStream_t st);
// the split append's second kernel alone (the slices summed in order, RoPE, the rows written)
hipError_t launch_append_finish_bf16(const float* part, int nslice, const int32_t* positions,
                                     const int32_t* block_table, int max_blocks, uint16_t* cache, int num_blocks,
                                     int tokens, int t_per_seq, float rope_base, int32_t* status, hipStream_t st);
// a decode step's append partial products, absorbed queries and split plan in one launch,
// then the append's second kernel
hipError_t launch_step_prepare_bf16(const uint16_t* h, const uint16_t* w_dkv, const uint16_t* w_kr,
                                    const int32_t* positions, const int32_t* block_table, int max_blocks,
                                    uint16_t* cache, int num_blocks, int t_per_seq, int d_model, float rope_base,
                                    float* part, const WsLayout& L, const uint16_t* q_nope, const uint16_t* q_rope,
                                    const uint16_t* w_uk, const int32_t* seq_lens, int batch, int sq, int n_heads,
                                    float qscale, uint8_t* ws, int32_t* status, hipStream_t st);
hipError_t launch_append_bf16(const uint16_t* h, const uint16_t* w_dkv, const uint16_t* w_kr,
                              const int32_t* positions, const int32_t* block_table, int max_blocks,
                              uint16_t* cache, int num_blocks, int tokens, int t_per_seq, int d_model,
                              float rope_base, int32_t* status, hipStream_t st);
hipError_t launch_append_f32(const mla_dims* d, const float* h, const float* w_dkv, const float* w_kr,
                             const int32_t* positions, const int32_t* block_table, int max_blocks,
                             float* cache, int num_blocks, int tokens, int t_per_seq,
                             int32_t* status, hipStream_t st);
hipError_t launch_qproj(const mla_dims* d, const void* h, const void* w_q, const void* w_qr,
                        const int32_t* positions, void* q_nope, void* q_rope, int tokens, hipStream_t st);
// Softmax scale split: softmax scale * log2(e) = qscale * zscale with qscale a power of two
// (applied exactly to the absorbed query) and zscale in [0.71, 1.42] (applied to the logits).
void split_softmax_scale(float softmax_scale, float* qscale, float* zscale);
// absorb: q_lat = qscale * [W^UK_i^T q^C | q^R]
hipError_t launch_absorb_bf16(const WsLayout& L, const uint16_t* q_nope, const uint16_t* q_rope,
                              const uint16_t* w_uk, const int32_t* seq_lens, int max_blocks, int batch,
                              int sq, int n_heads, float qscale, uint8_t* ws, int32_t* status, hipStream_t st);
hipError_t launch_attn_bf16(const WsLayout& L, const uint16_t* cache, int num_blocks,
                            const int32_t* block_table, int max_blocks, const int32_t* seq_lens,
                            int batch, int sq, int n_heads, float zscale, uint8_t* ws, int32_t* status,
                            hipStream_t st);
hipError_t launch_attn_fp8(const WsLayout& L, const uint8_t* pages, int num_blocks, const int32_t* block_table,
                           int max_blocks, const int32_t* seq_lens, int batch, int sq, int n_heads, float zscale,
                           uint8_t* ws, int32_t* status, hipStream_t st);
// FP8 cache rows: quantise bf16 rows [n_rows][576] into pages.  positions == null: row r is
// slot r % 64 of page r / 64 (a whole pool); otherwise token r goes to its position's slot
// (t_per_seq tokens per sequence), invalid positions and blocks reported and skipped.
hipError_t launch_quant_rows_fp8(const uint16_t* src, long long n_rows, const int32_t* positions,
                                 const int32_t* block_table, int max_blocks, int t_per_seq, int num_blocks,
                                 uint8_t* pages, int32_t* status, hipStream_t st);
hipError_t launch_merge_upv_bf16(const WsLayout& L, const uint16_t* w_uv, int batch, int sq, int n_heads,
                                 uint8_t* ws, uint16_t* out, float* lse, hipStream_t st);
// many-token append (prefill chunks): one GEMM kernel, no workspace; used for bf16 when
// batch * t >= kAppendGemmMinTokens and d_model is a multiple of 64
constexpr int kAppendGemmMinTokens = 2048;
hipError_t launch_append_gemm_bf16(const uint16_t* h, const uint16_t* w_dkv, const uint16_t* w_kr,
                                   const int32_t* positions, const int32_t* block_table, int max_blocks,
                                   uint16_t* cache, int num_blocks, int tokens, int t_per_seq, int d_model,
                                   float rope_base, int32_t* status, hipStream_t st);
// full-layer projections: y = x W^T for a few rows, split over K, summed in order
int proj_splits(int M, int N, int K);
size_t proj_ws_bytes(int M, int N, int K);
hipError_t launch_proj_bf16(const uint16_t* x, const uint16_t* w0, const uint16_t* w1, int n_w0, int M, int N, int K,
                            float* part, int rope_from, int rope_width, const int32_t* positions, float rope_base,
                            uint16_t* y0, int ld0, uint16_t* y1, int ld1, hipStream_t st);
// prefill (expanded form): workspace bytes, K^C / V^T expansion, causal attention
size_t prefill_ws_bytes(int batch, int n_heads, int max_blocks);
hipError_t launch_expand_kv_bf16(const uint16_t* cache, int num_blocks, const int32_t* block_table, int max_blocks,
                                 const int32_t* seq_lens, int batch, int n_heads, const uint16_t* w_uk,
                                 const uint16_t* w_uv, uint16_t* kc, uint16_t* vt, int32_t* status, hipStream_t st);
hipError_t launch_prefill_attn_bf16(const uint16_t* q_nope, const uint16_t* q_rope, const uint16_t* cache,
                                    int num_blocks, const int32_t* block_table, int max_blocks,
                                    const int32_t* seq_lens, int batch, int t, int n_heads, float scale,
                                    const uint16_t* kc, const uint16_t* vt, uint16_t* out, float* lse,
                                    int32_t* status, hipStream_t st);
hipError_t launch_decode_f32(int phases, const mla_dims* d, const WsLayout& L, const float* q_nope, const float* q_rope,
                             const float* w_uk, const float* w_uv, const float* cache, int num_blocks,
                             const int32_t* block_table, int max_blocks, const int32_t* seq_lens,
                             int batch, int sq, float scale, uint8_t* ws, float* out, float* lse,
                             int32_t* status, hipStream_t st);

}  // namespace mla
