// Host entry points of the MLA decode library (the C ABI declared in mla.h).
// Every check that the arguments allow is made here, before anything is
// launched; the kernels only guard against what the data alone can reveal.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>

#include "mla_internal.h"

// Device scratch of mla_decode_noalloc, for callers that cannot allocate: one copy per GPU,
// held until the process ends.  In host code this name is only a stand-in for the symbol;
// the device address comes from hipGetSymbolAddress (noalloc_scratch() below).
static __device__ __align__(256) uint8_t scratch[MLA_NOALLOC_SCRATCH_BYTES];

namespace mla {

namespace {

constexpr size_t kAlign = 256;
size_t up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// bf16 tensors: MLA_DTYPE_BF16, and MLA_DTYPE_BF16_FP8 (which differs only in the cache)
bool is_bf(const mla_dims* d) { return d->dtype == MLA_DTYPE_BF16 || d->dtype == MLA_DTYPE_BF16_FP8; }
bool is_fp8(const mla_dims* d) { return d->dtype == MLA_DTYPE_BF16_FP8; }
size_t elem_size(int dtype) { return dtype == MLA_DTYPE_F32 ? 4 : 2; }

// Checks that hold for every entry point.
int check_dims(const mla_dims* d) {
  if (d == nullptr) return MLA_ERR_NULL_PTR;
  if (d->dtype != MLA_DTYPE_F32 && d->dtype != MLA_DTYPE_BF16 && d->dtype != MLA_DTYPE_BF16_FP8)
    return MLA_ERR_BAD_DTYPE;
  if (d->n_heads < 1 || d->d_nope < 1 || d->d_rope < 0 || d->d_latent < 1 || d->d_model < 1 || d->block_size < 1)
    return MLA_ERR_BAD_DIMS;
  if (d->d_rope % 2 != 0) return MLA_ERR_BAD_DIMS;   // RoPE turns pairs
  if (!(d->rope_base > 0.0f) || !std::isfinite(d->rope_base)) return MLA_ERR_BAD_DIMS;
  if (is_bf(d)) {
    if (d->d_nope != kNope || d->d_rope != kRope || d->d_latent != kLat || d->block_size != kBlk)
      return MLA_ERR_UNSUPPORTED;
    if (d->n_heads > 1024 || d->d_model % 32 != 0) return MLA_ERR_UNSUPPORTED;
  } else {
    if (d->d_nope > kF32MaxWidth || d->d_latent > kF32MaxWidth || d->d_latent + d->d_rope > kF32MaxWidth ||
        d->n_heads > 1024 || d->block_size > 1024)
      return MLA_ERR_CAPACITY;
  }
  if (d->d_model > (1 << 20)) return MLA_ERR_CAPACITY;
  return MLA_OK;
}

int check_sq(const mla_dims* d, int sq) {
  if (sq < 1) return MLA_ERR_BAD_DIMS;
  if (sq > (is_bf(d) ? kMaxSqBf16 : kF32MaxSq)) return MLA_ERR_CAPACITY;
  if (d->dtype == MLA_DTYPE_F32 && d->n_heads * sq > 65535) return MLA_ERR_CAPACITY;   // one grid row per query row
  return MLA_OK;
}

int check_pool(const mla_dims* d, int num_blocks, int max_blocks, int batch) {
  if (num_blocks < 1 || max_blocks < 1 || batch < 1) return MLA_ERR_BAD_DIMS;
  if (batch > 65536) return MLA_ERR_CAPACITY;
  const long long R = d->d_latent + d->d_rope;
  if ((long long)num_blocks * d->block_size >= (1ll << 31)) return MLA_ERR_CAPACITY;
  if ((long long)num_blocks * d->block_size * R >= (1ll << 40)) return MLA_ERR_CAPACITY;
  if ((long long)batch * max_blocks >= (1ll << 31)) return MLA_ERR_CAPACITY;
  if ((long long)batch * max_blocks * d->block_size >= (1ll << 31)) return MLA_ERR_CAPACITY;
  return MLA_OK;
}

std::atomic<int> g_cus[64];

}  // namespace

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    int c = g_cus[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) return 0;
  if (dev < 64) g_cus[dev].store(n, std::memory_order_relaxed);
  return n;
}

bool ws_layout(const mla_dims* d, int batch, int sq, int num_splits, WsLayout* L) {
  const bool bf = is_bf(d);
  if (bf) {
    L->hg = d->n_heads < kRowsWG / sq ? d->n_heads : kRowsWG / sq;
    L->G = (d->n_heads + L->hg - 1) / L->hg;
    L->rows = kRowsWG;
    L->align = kBlk;
  } else {
    L->hg = d->n_heads;
    L->G = 1;
    L->rows = d->n_heads * sq;
    L->align = 16;
  }
  int W = num_splits;
  if (W <= 0) {
    int cus = device_cu_count();
    if (cus <= 0) return false;
    W = bf ? (cus / L->G > 0 ? cus / L->G : 1) : cus;
  }
  if (W > (1 << 20)) return false;
  L->W = W;
  L->tune = num_splits <= 0 ? 1 : 0;
  L->P = W + batch;
  const size_t R = (size_t)d->d_latent + d->d_rope;
  size_t off = 0;
  L->off_hdr = off;   off += up(sizeof(PlanHeader));
  L->off_seg = off;   off += up((size_t)(batch + 1) * 4);
  L->off_piece = off; off += up((size_t)(batch + 1) * 4);
  L->off_wgseg = off; off += up((size_t)W * 4);
  L->off_rcut = off;  off += up((size_t)(W + 1) * 4);
  L->off_firstr = off; off += up((size_t)batch * 4);
  const size_t qrows = (size_t)batch * sq * d->n_heads;
  L->off_qlat = off;  off += up((bf ? qlat_padded_rows(qrows) : qrows) * R * elem_size(d->dtype));
  L->off_lse = off;   off += up((size_t)L->G * L->P * L->rows * 8);
  // partial latent sums: bf16 for the bf16 kernels, fp32 for the fp32 ones
  L->off_o = off;     off += up((size_t)L->G * L->P * L->rows * d->d_latent * (bf ? 2 : 4));
  L->total = off;
  return true;
}

void split_softmax_scale(float softmax_scale, float* qscale, float* zscale) {
  const double s = (double)softmax_scale * 1.4426950408889634;   // log2(e): exponentials in base 2
  if (s == 0.0) {   // every logit is zero
    *qscale = 0.0f;
    *zscale = 1.0f;
    return;
  }
  // the exponent is clamped so that qscale stays a normal float for any finite scale
  const double p2 = std::exp2(std::fmin(std::fmax(std::nearbyint(std::log2(std::fabs(s))), -100.0), 100.0));
  *qscale = (float)(s < 0.0 ? -p2 : p2);
  *zscale = (float)(std::fabs(s) / p2);
}

}  // namespace mla

using namespace mla;

extern "C" {

const char* mla_status_str(int code) {
  switch (code) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL_PTR: return "a required pointer is NULL";
    case MLA_ERR_BAD_DIMS: return "a size is out of range or inconsistent";
    case MLA_ERR_BAD_DTYPE: return "unknown element type";
    case MLA_ERR_BAD_ALIGN: return "a device pointer is not 16-byte aligned (workspace: 256-byte)";
    case MLA_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than mla_decode_workspace_bytes()";
    case MLA_ERR_CAPACITY: return "a size exceeds what the kernels can index";
    case MLA_ERR_HIP: return "the HIP runtime refused a launch";
    case MLA_ERR_UNSUPPORTED: return "dims or an element type this entry point is not built for";
    case MLA_ERR_SCRATCH_TOO_SMALL:
      return "the shape needs more than the MLA_NOALLOC_SCRATCH_BYTES of scratch mla_decode_noalloc holds";
    default: return "unknown status code";
  }
}

size_t mla_cache_bytes(const mla_dims* dims, int64_t tokens) {
  if (check_dims(dims) != MLA_OK || tokens < 0) return 0;
  if (is_fp8(dims)) return (size_t)((tokens + kBlk - 1) / kBlk) * kFp8PageBytes;   // whole pages
  return (size_t)tokens * ((size_t)dims->d_latent + dims->d_rope) * elem_size(dims->dtype);
}

}  // extern "C"

namespace {
bool append_uses_gemm(const mla_dims* d, long long tokens) {
  return is_bf(d) && tokens >= kAppendGemmMinTokens && d->d_model % 64 == 0;
}
// FP8 append: the bf16 rows are first written densely to the workspace, then quantised into
// their pages; the split path's partial products follow the staging rows
size_t fp8_staging_bytes(long long tokens) { return up((size_t)tokens * kRow * 2); }
}  // namespace

extern "C" {

size_t mla_cache_append_workspace_bytes(const mla_dims* dims, int32_t batch, int32_t t) {
  if (check_dims(dims) != MLA_OK || batch < 1 || t < 1 || (long long)batch * t >= (1ll << 30)) return 0;
  const long long tokens = (long long)batch * t;
  const size_t split = append_uses_gemm(dims, tokens) ? 0 : append_split_ws_bytes(dims->d_model, tokens);
  if (is_fp8(dims)) return fp8_staging_bytes(tokens) + split;
  if (dims->dtype != MLA_DTYPE_BF16) return 0;
  return split;
}

}  // extern "C"

namespace {
// mla_cache_append's argument checks (dims checked already)
int check_append(const mla_dims* dims, const void* h, const void* w_dkv, const void* w_kr, const int32_t* positions,
                 const int32_t* block_table, int32_t max_blocks, const void* cache, int32_t num_blocks,
                 int32_t batch, int32_t t, const void* workspace, const int32_t* status) {
  int rc;
  if (!h || !w_dkv || !w_kr || !positions || !block_table || !cache) return MLA_ERR_NULL_PTR;
  if (t < 1) return MLA_ERR_BAD_DIMS;
  if ((rc = check_pool(dims, num_blocks, max_blocks, batch)) != MLA_OK) return rc;
  if ((long long)batch * t >= (1ll << 30)) return MLA_ERR_CAPACITY;
  if (!aligned16(h) || !aligned16(w_dkv) || !aligned16(w_kr) || !aligned16(positions) || !aligned16(block_table) ||
      !aligned16(cache) || (status && ((uintptr_t)status & 3u)) || (workspace && !aligned16(workspace)))
    return MLA_ERR_BAD_ALIGN;
  return MLA_OK;
}
}  // namespace

extern "C" {

int mla_cache_append(const mla_dims* dims, const void* h, const void* w_dkv, const void* w_kr, const int32_t* positions,
                     const int32_t* block_table, int32_t max_blocks, void* cache, int32_t num_blocks, int32_t batch,
                     int32_t t, void* workspace, size_t workspace_bytes, int32_t* status, void* stream) {
  int rc = check_dims(dims);
  if (rc != MLA_OK) return rc;
  if ((rc = check_append(dims, h, w_dkv, w_kr, positions, block_table, max_blocks, cache, num_blocks, batch, t,
                         workspace, status)) != MLA_OK)
    return rc;
  const bool gemm = append_uses_gemm(dims, (long long)batch * t);
  hipStream_t st = (hipStream_t)stream;
  if (is_fp8(dims)) {
    // bf16 rows into the workspace (dense, row = token), then quantised into their pages
    const long long tokens = (long long)batch * t;
    if (workspace == nullptr || workspace_bytes < mla_cache_append_workspace_bytes(dims, batch, t))
      return MLA_ERR_WORKSPACE_TOO_SMALL;
    uint16_t* rows = (uint16_t*)workspace;
    float* part = (float*)((uint8_t*)workspace + fp8_staging_bytes(tokens));
    hipError_t e =
        gemm ? launch_append_gemm_bf16((const uint16_t*)h, (const uint16_t*)w_dkv, (const uint16_t*)w_kr, positions,
                                       nullptr, max_blocks, rows, num_blocks, batch * t, t, dims->d_model,
                                       dims->rope_base, status, st)
             : launch_append_split_bf16((const uint16_t*)h, (const uint16_t*)w_dkv, (const uint16_t*)w_kr, positions,
                                        nullptr, max_blocks, rows, num_blocks, batch * t, t, dims->d_model,
                                        dims->rope_base, part, status, st);
    if (e == hipSuccess)
      e = launch_quant_rows_fp8(rows, tokens, positions, block_table, max_blocks, t, num_blocks, (uint8_t*)cache,
                                status, st);
    return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
  }
  const bool split = !gemm && workspace != nullptr && dims->dtype == MLA_DTYPE_BF16;
  if (split && workspace_bytes < append_split_ws_bytes(dims->d_model, (long long)batch * t))
    return MLA_ERR_WORKSPACE_TOO_SMALL;
  hipError_t e;
  if (gemm)
    e = launch_append_gemm_bf16((const uint16_t*)h, (const uint16_t*)w_dkv, (const uint16_t*)w_kr, positions,
                                block_table, max_blocks, (uint16_t*)cache, num_blocks, batch * t, t, dims->d_model,
                                dims->rope_base, status, st);
  else if (split)
    e = launch_append_split_bf16((const uint16_t*)h, (const uint16_t*)w_dkv, (const uint16_t*)w_kr, positions,
                                 block_table, max_blocks, (uint16_t*)cache, num_blocks, batch * t, t, dims->d_model,
                                 dims->rope_base, (float*)workspace, status, st);
  else if (dims->dtype == MLA_DTYPE_BF16)
    e = launch_append_bf16((const uint16_t*)h, (const uint16_t*)w_dkv, (const uint16_t*)w_kr, positions, block_table,
                           max_blocks, (uint16_t*)cache, num_blocks, batch * t, t, dims->d_model, dims->rope_base,
                           status, st);
  else
    e = launch_append_f32(dims, (const float*)h, (const float*)w_dkv, (const float*)w_kr, positions, block_table,
                          max_blocks, (float*)cache, num_blocks, batch * t, t, status, st);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int mla_cache_quantize(const mla_dims* dims, const void* src, void* pages, int32_t num_blocks, void* stream) {
  int rc = check_dims(dims);
  if (rc != MLA_OK) return rc;
  if (!is_fp8(dims)) return MLA_ERR_BAD_DTYPE;
  if (!src || !pages) return MLA_ERR_NULL_PTR;
  if (num_blocks < 1) return MLA_ERR_BAD_DIMS;
  if ((long long)num_blocks * kBlk >= (1ll << 31)) return MLA_ERR_CAPACITY;
  if (!aligned16(src) || !aligned16(pages)) return MLA_ERR_BAD_ALIGN;
  hipError_t e = launch_quant_rows_fp8((const uint16_t*)src, (long long)num_blocks * kBlk, nullptr, nullptr, 0, 1,
                                       num_blocks, (uint8_t*)pages, nullptr, (hipStream_t)stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // extern "C"

namespace {
// the full layer's projections run on bf16 tiles of 64 features (d_qlat 0: not used by the call)
int check_layer(const mla_dims* d, int d_qlat, int batch, int sq) {
  int rc = check_dims(d);
  if (rc != MLA_OK) return rc;
  if (!is_bf(d)) return MLA_ERR_UNSUPPORTED;
  if (d_qlat != 0 && (d_qlat < 64 || d_qlat % 64 != 0)) return MLA_ERR_UNSUPPORTED;
  if (d->d_model % 64 != 0) return MLA_ERR_UNSUPPORTED;
  if (d_qlat > (1 << 16)) return MLA_ERR_CAPACITY;
  if (batch < 1 || sq < 1) return MLA_ERR_BAD_DIMS;
  if ((long long)batch * sq > (1 << 20)) return MLA_ERR_CAPACITY;
  return MLA_OK;
}
size_t q_compress_bytes(const mla_dims* d, int d_qlat, int M) {
  const size_t cq = up((size_t)M * d_qlat * 2);
  size_t part = proj_ws_bytes(M, d_qlat, d->d_model);
  part = std::max(part, proj_ws_bytes(M, d->n_heads * (d->d_nope + d->d_rope), d_qlat));
  return cq + up(part);
}
}  // namespace

extern "C" {

size_t mla_layer_workspace_bytes(const mla_dims* dims, int32_t d_qlat, int32_t batch, int32_t sq) {
  if (check_layer(dims, d_qlat, batch, sq) != MLA_OK) return 0;
  const int M = batch * sq;
  return std::max(q_compress_bytes(dims, d_qlat, M),
                  up(proj_ws_bytes(M, dims->d_model, dims->n_heads * dims->d_nope)));
}

int mla_q_compress(const mla_dims* dims, int32_t d_qlat, const void* h, const void* w_dq, const void* w_uq,
                   const void* w_qr, const int32_t* positions, void* q_nope, void* q_rope, int32_t batch, int32_t sq,
                   void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_layer(dims, d_qlat, batch, sq);
  if (rc != MLA_OK) return rc;
  if (!h || !w_dq || !w_uq || !w_qr || !positions || !q_nope || !q_rope || !workspace) return MLA_ERR_NULL_PTR;
  if (!aligned16(h) || !aligned16(w_dq) || !aligned16(w_uq) || !aligned16(w_qr) || !aligned16(positions) ||
      !aligned16(q_nope) || !aligned16(q_rope) || ((uintptr_t)workspace & (kAlign - 1)))
    return MLA_ERR_BAD_ALIGN;
  const int M = batch * sq;
  if (workspace_bytes < q_compress_bytes(dims, d_qlat, M)) return MLA_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t st = (hipStream_t)stream;
  uint16_t* cq = (uint16_t*)workspace;
  float* part = (float*)((uint8_t*)workspace + up((size_t)M * d_qlat * 2));
  const int HN = dims->n_heads * dims->d_nope, HR = dims->n_heads * dims->d_rope;
  // c^Q = W^DQ h (kept in bf16, the activation type), then q^C = W^UQ c^Q and q^R = RoPE(W^QR c^Q) as one
  // product over the stacked rows [W^UQ; W^QR]
  const uint16_t* wdq = (const uint16_t*)w_dq;
  hipError_t e = launch_proj_bf16((const uint16_t*)h, wdq, wdq, d_qlat, M, d_qlat, dims->d_model, part, d_qlat,
                                  dims->d_rope, positions, dims->rope_base, cq, d_qlat, nullptr, 0, st);
  if (e == hipSuccess)
    e = launch_proj_bf16(cq, (const uint16_t*)w_uq, (const uint16_t*)w_qr, HN, M, HN + HR, d_qlat, part, HN,
                         dims->d_rope, positions, dims->rope_base, (uint16_t*)q_nope, HN, (uint16_t*)q_rope, HR, st);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int mla_out_project(const mla_dims* dims, const void* o, const void* w_o, void* u, int32_t batch, int32_t sq,
                    void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_layer(dims, 0, batch, sq);
  if (rc != MLA_OK) return rc;
  if (!o || !w_o || !u || !workspace) return MLA_ERR_NULL_PTR;
  if (!aligned16(o) || !aligned16(w_o) || !aligned16(u) || ((uintptr_t)workspace & (kAlign - 1)))
    return MLA_ERR_BAD_ALIGN;
  const int M = batch * sq;
  const int HN = dims->n_heads * dims->d_nope;
  if (workspace_bytes < std::max<size_t>(proj_ws_bytes(M, dims->d_model, HN), 1)) return MLA_ERR_WORKSPACE_TOO_SMALL;
  const uint16_t* wo = (const uint16_t*)w_o;
  hipError_t e = launch_proj_bf16((const uint16_t*)o, wo, wo, dims->d_model, M, dims->d_model, HN, (float*)workspace,
                                  dims->d_model, dims->d_rope, nullptr, dims->rope_base, (uint16_t*)u, dims->d_model,
                                  nullptr, 0, (hipStream_t)stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int mla_q_project(const mla_dims* dims, const void* h, const void* w_q, const void* w_qr, const int32_t* positions,
                  void* q_nope, void* q_rope, int32_t batch, int32_t sq, void* stream) {
  int rc = check_dims(dims);
  if (rc != MLA_OK) return rc;
  if (!h || !w_q || !positions || !q_nope || ((!w_qr || !q_rope) && dims->d_rope > 0)) return MLA_ERR_NULL_PTR;
  if (batch < 1 || sq < 1) return MLA_ERR_BAD_DIMS;
  if ((long long)batch * sq * dims->n_heads * (dims->d_nope + dims->d_rope) >= (1ll << 31)) return MLA_ERR_CAPACITY;
  if (!aligned16(h) || !aligned16(w_q) || (w_qr && !aligned16(w_qr)) || !aligned16(positions) ||
      !aligned16(q_nope) || (q_rope && !aligned16(q_rope)))
    return MLA_ERR_BAD_ALIGN;
  hipError_t e = launch_qproj(dims, h, w_q, w_qr, positions, q_nope, q_rope, batch * sq, (hipStream_t)stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

size_t mla_decode_workspace_bytes(const mla_dims* dims, int32_t batch, int32_t sq, int32_t num_splits) {
  if (check_dims(dims) != MLA_OK || check_sq(dims, sq) != MLA_OK || batch < 1 || batch > 65536 || num_splits < 0)
    return 0;
  WsLayout L;
  if (!ws_layout(dims, batch, sq, num_splits, &L)) return 0;
  return L.total;
}

}  // extern "C"

namespace {

constexpr int kPhasePrepare = 1, kPhaseAttend = 2, kPhaseFinish = 4;

// The scratch array's device address on the current device, looked up once per device
// (hipGetSymbolAddress, with that device current) and kept.
std::atomic<void*> g_scratch[64];
std::mutex g_scratch_mu;

int noalloc_scratch(void** ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MLA_ERR_HIP;
  if (dev >= 64) return MLA_ERR_CAPACITY;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MLA_ERR_HIP;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return MLA_OK;
}

// use_scratch: the phases run in this device's scratch array (mla_decode_noalloc), and
// workspace / workspace_bytes are ignored
int decode_impl(int phases, bool use_scratch, const mla_dims* dims, const void* q_nope, const void* q_rope,
                const void* w_uk, const void* w_uv, const void* cache, int32_t num_blocks, const int32_t* block_table,
                int32_t max_blocks, const int32_t* seq_lens, int32_t batch, int32_t sq, float softmax_scale,
                int32_t num_splits, void* workspace, size_t workspace_bytes, void* out, float* lse, int32_t* status,
                void* stream) {
  int rc = check_dims(dims);
  if (rc != MLA_OK) return rc;
  if (use_scratch) workspace_bytes = MLA_NOALLOC_SCRATCH_BYTES;
  if (!q_nope || !w_uk || !w_uv || !cache || !block_table || !seq_lens || (!workspace && !use_scratch) || !out)
    return MLA_ERR_NULL_PTR;
  if (dims->d_rope > 0 && !q_rope) return MLA_ERR_NULL_PTR;
  if ((rc = check_sq(dims, sq)) != MLA_OK) return rc;
  if ((rc = check_pool(dims, num_blocks, max_blocks, batch)) != MLA_OK) return rc;
  if (num_splits < 0 || !std::isfinite(softmax_scale)) return MLA_ERR_BAD_DIMS;
  if (!aligned16(q_nope) || (q_rope && !aligned16(q_rope)) || !aligned16(w_uk) || !aligned16(w_uv) ||
      !aligned16(cache) || !aligned16(block_table) || !aligned16(seq_lens) || !aligned16(out) ||
      (!use_scratch && ((uintptr_t)workspace & (kAlign - 1))) || (lse && ((uintptr_t)lse & 3u)) ||
      (status && ((uintptr_t)status & 3u)))
    return MLA_ERR_BAD_ALIGN;
  WsLayout L;
  if (!ws_layout(dims, batch, sq, num_splits, &L)) return MLA_ERR_HIP;
  if (workspace_bytes < L.total) return use_scratch ? MLA_ERR_SCRATCH_TOO_SMALL : MLA_ERR_WORKSPACE_TOO_SMALL;
  if (use_scratch && (rc = noalloc_scratch(&workspace)) != MLA_OK) return rc;
  hipStream_t st = (hipStream_t)stream;
  uint8_t* ws = (uint8_t*)workspace;
  hipError_t e = hipSuccess;
  if (is_bf(dims)) {
    float qscale, zscale;
    split_softmax_scale(softmax_scale, &qscale, &zscale);
    if (phases & kPhasePrepare)
      e = launch_absorb_bf16(L, (const uint16_t*)q_nope, (const uint16_t*)q_rope, (const uint16_t*)w_uk, seq_lens,
                             max_blocks, batch, sq, dims->n_heads, qscale, ws, status, st);
    if (e == hipSuccess && (phases & kPhaseAttend))
      e = is_fp8(dims) ? launch_attn_fp8(L, (const uint8_t*)cache, num_blocks, block_table, max_blocks, seq_lens,
                                         batch, sq, dims->n_heads, zscale, ws, status, st)
                       : launch_attn_bf16(L, (const uint16_t*)cache, num_blocks, block_table, max_blocks, seq_lens,
                                          batch, sq, dims->n_heads, zscale, ws, status, st);
    if (e == hipSuccess && (phases & kPhaseFinish))
      e = launch_merge_upv_bf16(L, (const uint16_t*)w_uv, batch, sq, dims->n_heads, ws, (uint16_t*)out, lse, st);
  } else {
    e = launch_decode_f32(phases, dims, L, (const float*)q_nope, (const float*)q_rope, (const float*)w_uk,
                          (const float*)w_uv, (const float*)cache, num_blocks, block_table, max_blocks, seq_lens,
                          batch, sq, softmax_scale, ws, (float*)out, lse, status, st);
  }
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // namespace

extern "C" {

#define MLA_DECODE_ARGS                                                                                          \
  dims, q_nope, q_rope, w_uk, w_uv, cache, num_blocks, block_table, max_blocks, seq_lens, batch, sq, softmax_scale, \
      num_splits, workspace, workspace_bytes, out, lse, status, stream
#define MLA_DECODE_PARAMS                                                                                        \
  const mla_dims *dims, const void *q_nope, const void *q_rope, const void *w_uk, const void *w_uv,                \
      const void *cache, int32_t num_blocks, const int32_t *block_table, int32_t max_blocks,                       \
      const int32_t *seq_lens, int32_t batch, int32_t sq, float softmax_scale, int32_t num_splits, void *workspace, \
      size_t workspace_bytes, void *out, float *lse, int32_t *status, void *stream

int mla_decode(MLA_DECODE_PARAMS) {
  return decode_impl(kPhasePrepare | kPhaseAttend | kPhaseFinish, false, MLA_DECODE_ARGS);
}
int mla_decode_prepare(MLA_DECODE_PARAMS) { return decode_impl(kPhasePrepare, false, MLA_DECODE_ARGS); }
int mla_decode_attend(MLA_DECODE_PARAMS) { return decode_impl(kPhaseAttend, false, MLA_DECODE_ARGS); }
int mla_decode_finish(MLA_DECODE_PARAMS) { return decode_impl(kPhaseFinish, false, MLA_DECODE_ARGS); }

size_t mla_decode_step_workspace_bytes(const mla_dims* dims, int32_t batch, int32_t sq, int32_t num_splits) {
  if (check_dims(dims) != MLA_OK || dims->dtype != MLA_DTYPE_BF16) return 0;
  const size_t dec = mla_decode_workspace_bytes(dims, batch, sq, num_splits);
  if (dec == 0 || (long long)batch * sq >= (1ll << 30)) return 0;
  const long long tokens = (long long)batch * sq;
  return up(dec) + (append_uses_gemm(dims, tokens) ? 0 : up(append_split_ws_bytes(dims->d_model, tokens)));
}

int mla_decode_step(const mla_dims* dims, const mla_step_args* args, int32_t phases, void* stream) {
  int rc = check_dims(dims);
  if (rc != MLA_OK) return rc;
  if (args == nullptr) return MLA_ERR_NULL_PTR;
  if (dims->dtype != MLA_DTYPE_BF16) return MLA_ERR_UNSUPPORTED;
  if (phases < 1 || phases > (kPhasePrepare | kPhaseAttend | kPhaseFinish)) return MLA_ERR_BAD_DIMS;
  const mla_step_args& a = *args;
  // the append's checks (t = sq tokens per sequence), then decode's, without launching anything
  if ((rc = check_append(dims, a.h, a.w_dkv, a.w_kr, a.positions, a.block_table, a.max_blocks, a.cache,
                         a.num_blocks, a.batch, a.sq, a.workspace, a.status)) != MLA_OK)
    return rc;
  if ((rc = decode_impl(0, false, dims, a.q_nope, a.q_rope, a.w_uk, a.w_uv, a.cache, a.num_blocks, a.block_table,
                        a.max_blocks, a.seq_lens, a.batch, a.sq, a.softmax_scale, a.num_splits, a.workspace,
                        a.workspace_bytes, a.out, a.lse, a.status, stream)) != MLA_OK)
    return rc;
  if (a.workspace_bytes < mla_decode_step_workspace_bytes(dims, a.batch, a.sq, a.num_splits))
    return MLA_ERR_WORKSPACE_TOO_SMALL;
  WsLayout L;
  if (!ws_layout(dims, a.batch, a.sq, a.num_splits, &L)) return MLA_ERR_HIP;
  hipStream_t st = (hipStream_t)stream;
  uint8_t* ws = (uint8_t*)a.workspace;
  hipError_t e = hipSuccess;
  if (phases & kPhasePrepare) {
    float qscale, zscale;
    split_softmax_scale(a.softmax_scale, &qscale, &zscale);
    const uint16_t *h = (const uint16_t*)a.h, *w_dkv = (const uint16_t*)a.w_dkv, *w_kr = (const uint16_t*)a.w_kr;
    if (append_uses_gemm(dims, (long long)a.batch * a.sq)) {
      // many tokens: mla_cache_append's GEMM path, then the absorbed queries and the plan
      e = launch_append_gemm_bf16(h, w_dkv, w_kr, a.positions, a.block_table, a.max_blocks, (uint16_t*)a.cache,
                                  a.num_blocks, a.batch * a.sq, a.sq, dims->d_model, dims->rope_base, a.status, st);
      if (e == hipSuccess)
        e = launch_absorb_bf16(L, (const uint16_t*)a.q_nope, (const uint16_t*)a.q_rope, (const uint16_t*)a.w_uk,
                               a.seq_lens, a.max_blocks, a.batch, a.sq, dims->n_heads, qscale, ws, a.status, st);
    } else {
      e = launch_step_prepare_bf16(h, w_dkv, w_kr, a.positions, a.block_table, a.max_blocks, (uint16_t*)a.cache,
                                   a.num_blocks, a.sq, dims->d_model, dims->rope_base, (float*)(ws + up(L.total)), L,
                                   (const uint16_t*)a.q_nope, (const uint16_t*)a.q_rope, (const uint16_t*)a.w_uk,
                                   a.seq_lens, a.batch, a.sq, dims->n_heads, qscale, ws, a.status, st);
    }
    if (e != hipSuccess) return MLA_ERR_HIP;
  }
  if (phases & (kPhaseAttend | kPhaseFinish))
    return decode_impl(phases & (kPhaseAttend | kPhaseFinish), false, dims, a.q_nope, a.q_rope, a.w_uk, a.w_uv,
                       a.cache, a.num_blocks, a.block_table, a.max_blocks, a.seq_lens, a.batch, a.sq, a.softmax_scale,
                       a.num_splits, a.workspace, a.workspace_bytes, a.out, a.lse, a.status, stream);
  return MLA_OK;
}

int mla_decode_noalloc(const mla_dims* dims, const void* q_nope, const void* q_rope, const void* w_uk,
                       const void* w_uv, const void* cache, int32_t num_blocks, const int32_t* block_table,
                       int32_t max_blocks, const int32_t* seq_lens, int32_t batch, int32_t sq, float softmax_scale,
                       int32_t num_splits, void* out, float* lse, int32_t* status, void* stream) {
  return decode_impl(kPhasePrepare | kPhaseAttend | kPhaseFinish, true, dims, q_nope, q_rope, w_uk, w_uv, cache,
                     num_blocks, block_table, max_blocks, seq_lens, batch, sq, softmax_scale, num_splits, nullptr,
                     0, out, lse, status, stream);
}

size_t mla_prefill_workspace_bytes(const mla_dims* dims, int32_t batch, int32_t max_blocks) {
  if (check_dims(dims) != MLA_OK || dims->dtype != MLA_DTYPE_BF16 || batch < 1 || batch > 65536 || max_blocks < 1 ||
      (long long)max_blocks * dims->block_size > (1ll << 23))
    return 0;
  return prefill_ws_bytes(batch, dims->n_heads, max_blocks);
}

}  // extern "C"

namespace {

constexpr int kPrefillExpand = 1, kPrefillAttend = 2;

int prefill_phases(int phases, const mla_dims* dims, const void* q_nope, const void* q_rope, const void* w_uk,
                   const void* w_uv, const void* cache, int32_t num_blocks, const int32_t* block_table,
                   int32_t max_blocks, const int32_t* seq_lens, int32_t batch, int32_t t, float softmax_scale,
                   void* workspace, size_t workspace_bytes, void* out, float* lse, int32_t* status, void* stream) {
  int rc = check_dims(dims);
  if (rc != MLA_OK) return rc;
  if (dims->dtype != MLA_DTYPE_BF16) return MLA_ERR_UNSUPPORTED;
  if (!q_nope || !q_rope || !w_uk || !w_uv || !cache || !block_table || !seq_lens || !workspace || !out)
    return MLA_ERR_NULL_PTR;
  if ((rc = check_pool(dims, num_blocks, max_blocks, batch)) != MLA_OK) return rc;
  if ((long long)max_blocks * dims->block_size > (1ll << 23)) return MLA_ERR_CAPACITY;
  if (t < 1 || (long long)t > (long long)max_blocks * dims->block_size || !std::isfinite(softmax_scale) ||
      !(softmax_scale > 0.0f))
    return MLA_ERR_BAD_DIMS;
  if ((long long)batch * t * dims->n_heads >= (1ll << 31)) return MLA_ERR_CAPACITY;
  {
    // launch grids: expansion (8 XCDs x head sets x token-tile groups x 32) and attention
    // ((sequence x head) rounded to 8, x 256-row query tiles)
    const long long tiles = ((long long)max_blocks * dims->block_size + 127) / 128;
    const long long qtiles = ((long long)t + 255) / 256;
    const long long xgrid = 8 * (((dims->n_heads + 7) / 8 + 3) / 4) * (((long long)batch * tiles + 7) / 8) * 32;
    if (xgrid >= (1ll << 31) ||
        ((long long)batch * dims->n_heads + 7) / 8 * 8 * qtiles >= (1ll << 31))
      return MLA_ERR_CAPACITY;
  }
  if (!aligned16(q_nope) || !aligned16(q_rope) || !aligned16(w_uk) || !aligned16(w_uv) || !aligned16(cache) ||
      !aligned16(block_table) || !aligned16(seq_lens) || !aligned16(out) || ((uintptr_t)workspace & (kAlign - 1)) ||
      (lse && ((uintptr_t)lse & 3u)) || (status && ((uintptr_t)status & 3u)))
    return MLA_ERR_BAD_ALIGN;
  // The expanded keys and values of one sequence take per_seq bytes.  The phase calls need
  // room for every sequence (expand writes them all before attend reads them); the whole
  // call processes the sequences in groups that fit the workspace given, each group
  // expanded and then attended, so its workspace need not grow with the batch.
  const size_t per_seq = prefill_ws_bytes(1, dims->n_heads, max_blocks);
  const bool both = (phases & kPrefillExpand) && (phases & kPrefillAttend);
  int group = batch;
  if (workspace_bytes < prefill_ws_bytes(batch, dims->n_heads, max_blocks)) {
    if (!both || workspace_bytes < per_seq) return MLA_ERR_WORKSPACE_TOO_SMALL;
    group = (int)(workspace_bytes / per_seq);
  }
  hipStream_t st = (hipStream_t)stream;
  const int H = dims->n_heads;
  hipError_t e = hipSuccess;
  for (int b0 = 0; b0 < batch && e == hipSuccess; b0 += group) {
    const int nb = batch - b0 < group ? batch - b0 : group;
    uint16_t* kc = (uint16_t*)workspace;
    uint16_t* vt = kc + prefill_ws_bytes(nb, H, max_blocks) / 4;   // the second half: V^T
    const int32_t* bt = block_table + (size_t)b0 * max_blocks;
    const int32_t* lens = seq_lens + b0;
    if (phases & kPrefillExpand)
      e = launch_expand_kv_bf16((const uint16_t*)cache, num_blocks, bt, max_blocks, lens, nb, H,
                                (const uint16_t*)w_uk, (const uint16_t*)w_uv, kc, vt, status, st);
    if (e == hipSuccess && (phases & kPrefillAttend)) {
      const size_t rows = (size_t)b0 * t * H;   // query rows before this group
      e = launch_prefill_attn_bf16((const uint16_t*)q_nope + rows * dims->d_nope,
                                   (const uint16_t*)q_rope + rows * dims->d_rope, (const uint16_t*)cache, num_blocks,
                                   bt, max_blocks, lens, nb, t, H, softmax_scale, kc, vt,
                                   (uint16_t*)out + rows * dims->d_nope, lse ? lse + rows : nullptr, status, st);
    }
  }
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // namespace

#define MLA_PREFILL_PARAMS                                                                                     \
  const mla_dims *dims, const void *q_nope, const void *q_rope, const void *w_uk, const void *w_uv,              \
      const void *cache, int32_t num_blocks, const int32_t *block_table, int32_t max_blocks,                     \
      const int32_t *seq_lens, int32_t batch, int32_t t, float softmax_scale, void *workspace,                   \
      size_t workspace_bytes, void *out, float *lse, int32_t *status, void *stream
#define MLA_PREFILL_ARGS                                                                                          \
  dims, q_nope, q_rope, w_uk, w_uv, cache, num_blocks, block_table, max_blocks, seq_lens, batch, t, softmax_scale, \
      workspace, workspace_bytes, out, lse, status, stream

extern "C" {

int mla_prefill(MLA_PREFILL_PARAMS) { return prefill_phases(kPrefillExpand | kPrefillAttend, MLA_PREFILL_ARGS); }
int mla_prefill_expand(MLA_PREFILL_PARAMS) { return prefill_phases(kPrefillExpand, MLA_PREFILL_ARGS); }
int mla_prefill_attend(MLA_PREFILL_PARAMS) { return prefill_phases(kPrefillAttend, MLA_PREFILL_ARGS); }

}  // extern "C"
