/*
 * mla.h - C ABI of the MI355X (gfx950) MLA decode library.
 *
 * Multi-head Latent Attention decode over a paged latent KV cache.  Each cached
 * token keeps only its joint latent c^KV (d_latent wide) followed by its
 * rotary key k^R (d_rope wide), as "DeepSeek-V2: Multi-Head Latent Attention
 * (MLA) 原理与工程实现" §2.1 (joint low-rank K/V compression) and §3.3 (cache of
 * d_c + d_h^R per token) describe.  Decode runs in latent space through matrix
 * absorption (same page, §2.2): every head's q^C is turned into a latent query
 * with W^UK_i, scored against [c^KV ‖ k^R] together with the rotated q^R
 * (§3.2, decoupled RoPE), the softmax weights sum the latents, and W^UV_i
 * restores the head's output.
 *
 * Conventions for every entry point
 *  - Return 0 (MLA_OK) or a negative MLA_ERR_* code.  All shape, dtype,
 *    pointer and alignment errors are found on the host before anything is
 *    launched; on error nothing is launched and no memory is touched.
 *  - Array pointers are DEVICE pointers owned by the caller (unless a comment
 *    says host).  The library never allocates, frees or synchronises; every
 *    launch is asynchronous on the caller's stream (`stream` is a hipStream_t,
 *    NULL = the default stream).  Kernel launches are the only stream work
 *    (no memset or copy), so a stream under HIP graph capture records them as
 *    they are, and a replay with the same buffers repeats the call.
 *  - Arrays are dense, row-major, in the element type named by dims->dtype
 *    (MLA_DTYPE_F32: float, MLA_DTYPE_BF16 and MLA_DTYPE_BF16_FP8: bfloat16)
 *    unless typed int32/float; with MLA_DTYPE_BF16_FP8 the cache alone is in
 *    the FP8 page format described below.
 *    Device arrays must be 16-byte aligned.
 *  - Weights are stored out x in, as the page writes W in R^{out x in}.
 *  - Problems that only the data can reveal (a block id outside the pool, a
 *    sequence longer than its block-table row, an append position outside
 *    its table row) are never turned into out-of-bounds accesses: the access
 *    is clamped or skipped and the matching MLA_STATUS_* bit is OR-ed into
 *    the optional device word `status`.
 *  - The library's mutable global state is a per-device cache of the compute-unit
 *    count and of the scratch array's address (each written once, atomically), and
 *    that scratch array itself, which only mla_decode_noalloc uses; concurrent calls
 *    on different streams are safe as long as they do not share output or workspace
 *    memory (mla_decode_noalloc: see there).
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* return codes */
#define MLA_OK                        0
#define MLA_ERR_NULL_PTR             -1  /* a required pointer is NULL */
#define MLA_ERR_BAD_DIMS             -2  /* a size is out of range or inconsistent */
#define MLA_ERR_BAD_DTYPE            -3  /* dims->dtype is not a known type */
#define MLA_ERR_BAD_ALIGN            -4  /* a device pointer is not 16-byte aligned */
#define MLA_ERR_WORKSPACE_TOO_SMALL  -5  /* workspace_bytes < mla_decode_workspace_bytes(...) */
#define MLA_ERR_CAPACITY             -6  /* a size exceeds what the kernels index (see below) */
#define MLA_ERR_HIP                  -7  /* the HIP runtime refused a launch */
#define MLA_ERR_UNSUPPORTED          -8  /* valid dims or dtype this entry point is not built for */
#define MLA_ERR_SCRATCH_TOO_SMALL    -9  /* mla_decode_noalloc: the shape needs more than its scratch */

/* bits OR-ed into *status by the kernels */
#define MLA_STATUS_BAD_BLOCK   0x1  /* block_table named a block outside [0, num_blocks) */
#define MLA_STATUS_BAD_LENGTH  0x2  /* seq_lens[b] < sq or > max_blocks * block_size */
#define MLA_STATUS_BAD_POS     0x4  /* append position < 0 or >= max_blocks * block_size */

#define MLA_DTYPE_F32       0
#define MLA_DTYPE_BF16      1
#define MLA_DTYPE_BF16_FP8  2   /* bf16 tensors, latent cache in FP8 E4M3 pages */

/*
 * The FP8 latent cache (MLA_DTYPE_BF16_FP8).  The "DeepSeek-V2 ... MLA" page
 * §5.1 (item 3) names quantisation error as the risk of a low-precision form
 * and fixes no format; this library's format:
 *  - c^KV is stored as OCP FP8 E4M3 codes (bias 7, 3 mantissa bits, no
 *    infinities, largest finite 448) with one power-of-two scale per token,
 *    s = 2^k for the smallest k >= -124 with max_i |c_i| <= 448 s (s = 1 for an
 *    all-zero c), code_i = round-to-nearest-even(c_i / s) (an exact division;
 *    the sign of zero is kept).  The value a code stands for is s * e4m3(code),
 *    exactly a bfloat16 value for rows with max |c_i| < 2^127.
 *  - k^R stays bfloat16.
 *  - What is quantised is the bf16 row [c ‖ k^R] a MLA_DTYPE_BF16 cache holds,
 *    so an FP8 cache equals mla_cache_quantize() of the bf16 cache.
 *  - Block size 64.  Page b (MLA_FP8_PAGE_BYTES bytes) holds the 64 rows of
 *    512 codes (bytes [0, 32768)), then the 64 k^R rows of 64 bf16
 *    ([32768, 40960)), then the 64 scales as little-endian fp32 ([40960, 41216)).
 *    A cache of num_blocks pages is num_blocks * MLA_FP8_PAGE_BYTES bytes.
 *  - Decode computes on the dequantised values s * e4m3(code) exactly (the
 *    products see the same bfloat16 values a bf16 cache of those values would
 *    hold), so results match the bf16 path on the dequantised cache.
 */
#define MLA_FP8_PAGE_BYTES 41216

/* Model dimensions (names follow the DeepSeek-V2 MLA page's notation). */
typedef struct mla_dims {
  int32_t n_heads;     /* n_h                                                   */
  int32_t d_nope;      /* d_h: per-head width of q^C, k^C and v                 */
  int32_t d_rope;      /* d_h^R: width of the decoupled rotary q^R_i and k^R    */
  int32_t d_latent;    /* d_c: width of the joint latent c^KV                   */
  int32_t d_model;     /* d: hidden size the down-projections read              */
  int32_t block_size;  /* tokens per cache block                                */
  int32_t dtype;       /* MLA_DTYPE_F32 or MLA_DTYPE_BF16                       */
  float rope_base;     /* RoPE base b: pair i turns by pos * b^(-2i/d_rope)     */
} mla_dims;

/*
 * Size limits.
 *  - MLA_DTYPE_BF16 and MLA_DTYPE_BF16_FP8 run the MFMA kernels, built for
 *    DeepSeek-V2's widths:
 *    d_nope = 128, d_rope = 64, d_latent = 512, block_size = 64, n_heads in
 *    1..1024, d_model a multiple of 32, sq in 1..8.  Other bf16 dims give
 *    MLA_ERR_UNSUPPORTED (sq above 8: MLA_ERR_CAPACITY).
 *  - MLA_DTYPE_F32 runs plain fp32 kernels for any dims with d_nope, d_rope
 *    (even) and d_latent in 1..1024, d_latent + d_rope <= 1024,
 *    n_heads <= 1024, block_size 1..1024, sq in 1..64.
 *  - batch <= 65536; num_blocks * block_size * (d_latent + d_rope) < 2^40.
 */

/* A short English description of a return code (static storage; never NULL). */
const char* mla_status_str(int code);

/*
 * Bytes the latent cache needs for `tokens` tokens: tokens * (d_latent + d_rope)
 * * sizeof(dtype) ("DeepSeek-V2 ... MLA" page §3.3: d_c + d_h^R elements per
 * token per layer, against MHA's 2 n_h d_h in §1.1); for MLA_DTYPE_BF16_FP8,
 * whole pages: ceil(tokens / 64) * MLA_FP8_PAGE_BYTES.  Returns 0 for invalid
 * dims or a negative token count.  Pure host arithmetic.
 */
size_t mla_cache_bytes(const mla_dims* dims, int64_t tokens);

/*
 * Append `t` new tokens per sequence to the paged latent cache.
 *
 * For token (b, j) at position p = positions[b*t + j] with hidden state
 * h[b, j, :] (d_model wide):
 *   c   = W^DKV h                    (W^DKV: w_dkv [d_latent, d_model])  §2.1
 *   k^R = RoPE_p(W^KR h)             (W^KR:  w_kr  [d_rope,   d_model])  §3.2
 *   cache[block_table[b*max_blocks + p / block_size]][p % block_size][:]
 *       = [c ‖ k^R] rounded to dtype (bf16: nearest-even)
 * RoPE turns pairs (x_{2i}, x_{2i+1}) by angle p * rope_base^(-2i/d_rope); the
 * angle and its sine/cosine are evaluated in fp64.
 * Dot products accumulate in fp32.  Exactly batch*t rows of d_latent + d_rope
 * elements are written and nothing else.  The caller advances its seq_lens.
 *
 * h          [batch, t, d_model]            dtype
 * w_dkv      [d_latent, d_model]            dtype
 * w_kr       [d_rope, d_model]              dtype
 * positions  [batch, t]                     int32 (device)
 * block_table[batch, max_blocks]            int32 (device)
 * cache      [num_blocks, block_size, d_latent + d_rope]  dtype, written in place
 * workspace  optional device scratch of mla_cache_append_workspace_bytes(dims,
 *            batch, t) bytes, 16-byte aligned, contents irrelevant and clobbered.
 *            With it (bf16) the products are split over the d_model axis across
 *            many workgroups and summed in a fixed order by a second kernel, so
 *            the weights stream at memory rate; NULL (with workspace_bytes 0)
 *            runs one kernel that needs no scratch.  From 2048 rows (batch*t)
 *            with d_model a multiple of 64 (bf16), a third path runs: one GEMM
 *            kernel over the whole d_model per tile, which needs no scratch and
 *            ignores the workspace (mla_cache_append_workspace_bytes returns 0
 *            there).  Every path's result is independent of timing; paths may
 *            differ in the last bit, because they sum in different orders.
 * status     optional int32 (device), OR-ed with MLA_STATUS_BAD_POS/BAD_BLOCK; a
 *            row whose position or block is invalid is skipped.
 * MLA_DTYPE_BF16_FP8: cache is the FP8 page pool; the bf16 row is computed as
 * above (the split or GEMM path), written to the workspace, then quantised into
 * its page slot.  The workspace is required (mla_cache_append_workspace_bytes;
 * MLA_ERR_WORKSPACE_TOO_SMALL without it).
 */
int mla_cache_append(const mla_dims* dims, const void* h, const void* w_dkv, const void* w_kr,
                     const int32_t* positions, const int32_t* block_table, int32_t max_blocks,
                     void* cache, int32_t num_blocks, int32_t batch, int32_t t,
                     void* workspace, size_t workspace_bytes, int32_t* status, void* stream);

/*
 * Workspace bytes for mla_cache_append's split path with this batch shape, or
 * 0 when the path needs none (fp32) or the arguments are invalid.
 */
size_t mla_cache_append_workspace_bytes(const mla_dims* dims, int32_t batch, int32_t t);

/*
 * Quantise a whole bf16 cache into the FP8 page format (the format described
 * at MLA_DTYPE_BF16_FP8): page b of `pages` from block b of `src`, for
 * b < num_blocks.  dims->dtype must be MLA_DTYPE_BF16_FP8 (MLA_ERR_BAD_DTYPE
 * otherwise) and the other dims the MFMA kernels' widths.
 *
 * src        [num_blocks, 64, 576]             bfloat16, finite (device)
 * pages      [num_blocks, MLA_FP8_PAGE_BYTES]  bytes, written (device)
 */
int mla_cache_quantize(const mla_dims* dims, const void* src, void* pages, int32_t num_blocks, void* stream);

/*
 * Project the query hidden states of `sq` tokens per sequence:
 *   q_nope[b, s, i, :] = W^Q_i h[b, s, :]            (w_q  [n_heads*d_nope, d_model])
 *   q_rope[b, s, i, :] = RoPE_p(W^QR_i h[b, s, :])   (w_qr [n_heads*d_rope, d_model])
 * with p = positions[b*sq + s] ("DeepSeek-V2 ... MLA" page §1.1 for W^Q on h,
 * §3.2 for the multi-head rotary query).  Same RoPE and accumulation rules as
 * mla_cache_append.  Outputs are in dtype.
 */
int mla_q_project(const mla_dims* dims, const void* h, const void* w_q, const void* w_qr,
                  const int32_t* positions, void* q_nope, void* q_rope,
                  int32_t batch, int32_t sq, void* stream);

/*
 * Workspace bytes mla_decode needs for this batch shape.  num_splits is the
 * number of attention workgroups the token space is cut into (0 = one per
 * compute unit of the current device); pass the same value to mla_decode.
 * Returns 0 for invalid arguments.
 */
size_t mla_decode_workspace_bytes(const mla_dims* dims, int32_t batch, int32_t sq, int32_t num_splits);

/*
 * Decode attention for `sq` query tokens per sequence ("DeepSeek-V2 ... MLA"
 * page §2.2 absorption and §3.2 decoupled RoPE):
 *   q~_i   = W^UK_i^T q^C_i                     latent query, d_latent wide
 *   z_j    = scale * ([q~_i ‖ q^R_i] . [c_j ‖ k^R_j])
 *   p      = softmax over the visible tokens j
 *   out_i  = W^UV_i (sum_j p_j c_j)
 * W^UK_i, W^UV_i are rows i*d_nope .. (i+1)*d_nope-1 of w_uk, w_uv.
 * Query s of sequence b sits at position seq_lens[b] - sq + s and sees cached
 * tokens 0 .. seq_lens[b] - sq + s (itself included; causal inside the group).
 * The token space is cut into num_splits equal ranges processed in parallel;
 * the partial softmax states are merged exactly by log-sum-exp.
 *
 * q_nope     [batch, sq, n_heads, d_nope]   dtype
 * q_rope     [batch, sq, n_heads, d_rope]   dtype, already rotated
 * w_uk, w_uv [n_heads*d_nope, d_latent]     dtype
 * cache      [num_blocks, block_size, d_latent + d_rope]  dtype
 *            (MLA_DTYPE_BF16_FP8: [num_blocks, MLA_FP8_PAGE_BYTES] pages)
 * block_table[batch, max_blocks]            int32 (device)
 * seq_lens   [batch]                        int32 (device), query tokens included
 * softmax_scale  e.g. 1/sqrt(d_nope + d_rope)
 * num_splits 0 = at most one attention workgroup per compute unit, the token ranges
 *            chosen by the library (even ranges, or for ragged batches of up to
 *            256 sequences ranges that are shorter where they hold a sequence
 *            boundary, whichever makes the slowest range cheaper); >0 forces the
 *            count, with even ranges
 * workspace  device scratch of at least mla_decode_workspace_bytes(dims, batch,
 *            sq, num_splits) bytes, 256-byte aligned; its contents on entry do
 *            not matter and are clobbered
 * out        [batch, sq, n_heads, d_nope]   dtype
 * lse        optional [batch, sq, n_heads] float: natural log of sum_j exp(z_j);
 *            -inf (and out = 0) for a query that sees no token
 * status     optional int32 (device), OR-ed with MLA_STATUS_BAD_BLOCK/BAD_LENGTH
 */
int mla_decode(const mla_dims* dims, const void* q_nope, const void* q_rope,
               const void* w_uk, const void* w_uv, const void* cache, int32_t num_blocks,
               const int32_t* block_table, int32_t max_blocks, const int32_t* seq_lens,
               int32_t batch, int32_t sq, float softmax_scale, int32_t num_splits,
               void* workspace, size_t workspace_bytes, void* out, float* lse,
               int32_t* status, void* stream);

/*
 * The three phases of mla_decode, for callers that schedule them separately
 * (to overlap the first with other work, or to time the attention kernel on
 * its own).  Same arguments, same checks and same conventions as mla_decode;
 * calling all three in order on one stream with the same arguments and
 * workspace is exactly mla_decode.
 *  - prepare: absorbed latent queries q~_i = W^UK_i^T q^C_i ‖ q^R_i ("DeepSeek-V2
 *    ... MLA" page §2.2) and the split plan, into the workspace.
 *  - attend:  scores over [c ‖ k^R], softmax weights and latent weighted sums
 *    for every token range (§2.2, §3.2), as partial states in the workspace.
 *  - finish:  log-sum-exp merge of the partial states and out_i = W^UV_i o_lat
 *    (§2.2 value-side absorption); writes out and lse.
 */
int mla_decode_prepare(const mla_dims* dims, const void* q_nope, const void* q_rope,
                       const void* w_uk, const void* w_uv, const void* cache, int32_t num_blocks,
                       const int32_t* block_table, int32_t max_blocks, const int32_t* seq_lens,
                       int32_t batch, int32_t sq, float softmax_scale, int32_t num_splits,
                       void* workspace, size_t workspace_bytes, void* out, float* lse,
                       int32_t* status, void* stream);
int mla_decode_attend(const mla_dims* dims, const void* q_nope, const void* q_rope,
                      const void* w_uk, const void* w_uv, const void* cache, int32_t num_blocks,
                      const int32_t* block_table, int32_t max_blocks, const int32_t* seq_lens,
                      int32_t batch, int32_t sq, float softmax_scale, int32_t num_splits,
                      void* workspace, size_t workspace_bytes, void* out, float* lse,
                      int32_t* status, void* stream);
int mla_decode_finish(const mla_dims* dims, const void* q_nope, const void* q_rope,
                      const void* w_uk, const void* w_uv, const void* cache, int32_t num_blocks,
                      const int32_t* block_table, int32_t max_blocks, const int32_t* seq_lens,
                      int32_t batch, int32_t sq, float softmax_scale, int32_t num_splits,
                      void* workspace, size_t workspace_bytes, void* out, float* lse,
                      int32_t* status, void* stream);

/*
 * A decode step that appends its own tokens: exactly mla_cache_append of the sq new
 * tokens of every sequence (t = sq, with a workspace) followed by mla_decode of those
 * tokens as the query group, bit for bit the same results, in fewer launches.
 * ("DeepSeek-V2: Multi-Head Latent Attention (MLA) 原理与工程实现" §2.1 and §3.2 for
 * the cached row of a new token, §2.2 for the absorbed decode.)  The append's partial
 * products, the absorbed queries and the split plan depend on nothing from one another
 * and run in one launch.  MLA_DTYPE_BF16 only (others: MLA_ERR_UNSUPPORTED).
 *
 * Each field means what the argument of the same name means for mla_cache_append
 * (h, w_dkv, w_kr, positions; t = sq) or mla_decode (the rest); seq_lens include the
 * new tokens.  workspace: at least mla_decode_step_workspace_bytes(dims, batch, sq,
 * num_splits) bytes, 256-byte aligned, clobbered.  Every argument is checked on the host
 * before anything is launched, as by those two calls.
 * phases: MLA_PHASE_ALL, or any of
 *  - MLA_PHASE_PREPARE: the new rows written to the cache, the absorbed queries and the
 *    split plan (into the workspace);
 *  - MLA_PHASE_ATTEND / MLA_PHASE_FINISH: mla_decode_attend / mla_decode_finish.
 * Calling the phases in order on one stream with the same arguments equals MLA_PHASE_ALL.
 */
typedef struct mla_step_args {
  const void* h;               /* [batch, sq, d_model]                          */
  const void* w_dkv;           /* [d_latent, d_model]                           */
  const void* w_kr;            /* [d_rope, d_model]                             */
  const int32_t* positions;    /* [batch, sq] int32 (device)                    */
  const void* q_nope;          /* [batch, sq, n_heads, d_nope]                  */
  const void* q_rope;          /* [batch, sq, n_heads, d_rope], rotated         */
  const void* w_uk;            /* [n_heads * d_nope, d_latent]                  */
  const void* w_uv;            /* [n_heads * d_nope, d_latent]                  */
  void* cache;                 /* [num_blocks, block_size, d_latent + d_rope]   */
  int32_t num_blocks;
  const int32_t* block_table;  /* [batch, max_blocks] int32 (device)            */
  int32_t max_blocks;
  const int32_t* seq_lens;     /* [batch] int32 (device), new tokens included   */
  int32_t batch;
  int32_t sq;                  /* new tokens = query tokens per sequence        */
  float softmax_scale;
  int32_t num_splits;
  void* workspace;
  size_t workspace_bytes;
  void* out;                   /* [batch, sq, n_heads, d_nope]                  */
  float* lse;                  /* optional [batch, sq, n_heads]                 */
  int32_t* status;             /* optional                                      */
} mla_step_args;

#define MLA_PHASE_PREPARE 1
#define MLA_PHASE_ATTEND  2
#define MLA_PHASE_FINISH  4
#define MLA_PHASE_ALL     7

/* Workspace bytes mla_decode_step needs (0 for invalid arguments or non-bf16 dims). */
size_t mla_decode_step_workspace_bytes(const mla_dims* dims, int32_t batch, int32_t sq, int32_t num_splits);
int mla_decode_step(const mla_dims* dims, const mla_step_args* args, int32_t phases, void* stream);

/*
 * mla_decode without a caller workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, checks, results and conventions as mla_decode with
 * the same num_splits, minus workspace and workspace_bytes: the workspace is a
 * static device array of MLA_NOALLOC_SCRATCH_BYTES inside the library, one per GPU,
 * held from the first call on that GPU until the process ends (the first call on a
 * device looks up its address; no call allocates or frees anything).
 *  - A shape whose mla_decode_workspace_bytes(dims, batch, sq, num_splits) exceeds
 *    MLA_NOALLOC_SCRATCH_BYTES returns MLA_ERR_SCRATCH_TOO_SMALL before anything is
 *    launched (64 MiB holds batch 64 x 128 heads at one query token, the decode
 *    benchmark's shape, with room to spare; use mla_decode for larger shapes).
 *  - The GPU is the calling thread's current device (hipGetDevice): the stream must
 *    belong to it, as for any launch of that device's kernels.
 *  - Every call on one GPU uses that GPU's one array, and nothing in it has to start
 *    at any value (each call writes what it reads).  Calls that overlap in time on
 *    one GPU (other streams, other host threads) race on it and give wrong results:
 *    order them on one stream, or use mla_decode with separate workspaces.
 *  - Under HIP graph capture: make one call on the device before capturing, so the
 *    address lookup is not part of the captured region; a replay then runs in the
 *    same array, and replays overlapping other calls on that GPU race like calls do.
 */
#define MLA_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
int mla_decode_noalloc(const mla_dims* dims, const void* q_nope, const void* q_rope,
                       const void* w_uk, const void* w_uv, const void* cache, int32_t num_blocks,
                       const int32_t* block_table, int32_t max_blocks, const int32_t* seq_lens,
                       int32_t batch, int32_t sq, float softmax_scale, int32_t num_splits,
                       void* out, float* lse, int32_t* status, void* stream);

/*
 * The full layer's projections around attention ("DeepSeek-V2 ... MLA" page
 * §2.3 query compression; "【深度学习】DeepSeek焦点架构-MLA" page 02 (3) and
 * (5): the compressed query's up-projections give each head's q^C and its
 * rotary q^R, and the heads' outputs, concatenated, pass through W^O).
 * bf16 tensors only (f32: MLA_ERR_UNSUPPORTED); d_model and d_qlat multiples of 64;
 * batch * sq <= 2^20.  Products accumulate in fp32, split over the input
 * features across workgroups and summed in a fixed order, so results do not
 * depend on timing.
 *
 * Workspace bytes for mla_q_compress and mla_out_project with this shape
 * (the larger of the two); 0 for invalid or unsupported arguments.
 */
size_t mla_layer_workspace_bytes(const mla_dims* dims, int32_t d_qlat, int32_t batch, int32_t sq);

/*
 *   c^Q          = W^DQ h              (w_dq [d_qlat, d_model]); kept in bf16
 *   q_nope[.., i] = W^UQ_i c^Q         (w_uq [n_heads*d_nope, d_qlat])
 *   q_rope[.., i] = RoPE_p(W^QR_i c^Q) (w_qr [n_heads*d_rope, d_qlat]), p = positions[b*sq + s]
 * h [batch, sq, d_model]; positions [batch, sq] int32 (device); q_nope and
 * q_rope as mla_decode takes them.  RoPE as in mla_cache_append.
 */
int mla_q_compress(const mla_dims* dims, int32_t d_qlat, const void* h, const void* w_dq,
                   const void* w_uq, const void* w_qr, const int32_t* positions,
                   void* q_nope, void* q_rope, int32_t batch, int32_t sq,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 *   u[b, s, :] = W^O [o_1; ...; o_{n_heads}]   (w_o [d_model, n_heads*d_nope])
 * o [batch, sq, n_heads, d_nope] (mla_decode's out); u [batch, sq, d_model].
 */
int mla_out_project(const mla_dims* dims, const void* o, const void* w_o, void* u,
                    int32_t batch, int32_t sq, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * Workspace bytes for the expanded per-head keys and values of every token slot
 * the block table can address, for `batch` sequences:
 *   2 * batch * n_heads * (max_blocks * block_size) * d_nope * 2 bytes.
 * mla_prefill_expand and mla_prefill_attend need it for the whole batch;
 * mla_prefill runs with any workspace of at least one sequence's worth
 * (mla_prefill_workspace_bytes(dims, 1, max_blocks)), taking the sequences in
 * groups that fit, so its memory need not grow with the batch.
 * bf16 only; returns 0 for invalid arguments or f32 dims.
 */
size_t mla_prefill_workspace_bytes(const mla_dims* dims, int32_t batch, int32_t max_blocks);

/*
 * Prefill attention in expanded form for the last `t` tokens of each sequence
 * ("DeepSeek-V2 ... MLA" page §2.1 up-projections, §3.2 decoupled RoPE).  The
 * result is the attention mla_decode defines for a query group of t tokens;
 * the computation decompresses instead of absorbing, which is the cheaper
 * order when many queries read each cached token:
 *   k^C_{j,i} = W^UK_i c_j,  v_{j,i} = W^UV_i c_j          (every context token j)
 *   z_j    = scale * ([q^C_i ‖ q^R_i] . [k^C_{j,i} ‖ k^R_j])
 *   out_i  = sum_j softmax(z)_j v_{j,i}
 * Query s of sequence b sits at position seq_lens[b] - t + s and sees tokens
 * 0 .. seq_lens[b] - t + s.  The t new tokens' rows must already be in the
 * cache (mla_cache_append with the same t).
 *
 * q_nope     [batch, t, n_heads, d_nope]   bf16
 * q_rope     [batch, t, n_heads, d_rope]   bf16, already rotated
 * w_uk, w_uv, cache, block_table, seq_lens, lse, status: as for mla_decode
 * softmax_scale  positive and finite (MLA_ERR_BAD_DIMS otherwise)
 * t          query tokens per sequence, 1 .. max_blocks * block_size
 * workspace  device scratch, 256-byte aligned, clobbered: at least
 *            mla_prefill_workspace_bytes(dims, 1, max_blocks) bytes (one
 *            sequence); with less than the whole batch's
 *            mla_prefill_workspace_bytes(dims, batch, max_blocks) the sequences
 *            are expanded and attended in groups that fit, one after another on
 *            the stream (same results)
 * out        [batch, t, n_heads, d_nope]   bf16
 * Limits: MLA_DTYPE_BF16 only (f32 and the FP8 cache: MLA_ERR_UNSUPPORTED);
 * max_blocks * block_size <= 2^23.
 */
int mla_prefill(const mla_dims* dims, const void* q_nope, const void* q_rope,
                const void* w_uk, const void* w_uv, const void* cache, int32_t num_blocks,
                const int32_t* block_table, int32_t max_blocks, const int32_t* seq_lens,
                int32_t batch, int32_t t, float softmax_scale,
                void* workspace, size_t workspace_bytes, void* out, float* lse,
                int32_t* status, void* stream);

/*
 * The two phases of mla_prefill, for callers that schedule or time them
 * separately.  Same arguments, checks and conventions; calling both in order
 * on one stream with the same arguments and workspace is exactly mla_prefill.
 * The phases need the whole batch's workspace (MLA_ERR_WORKSPACE_TOO_SMALL
 * otherwise), since expand writes every sequence before attend reads them.
 *  - expand: k^C_{j,i} = W^UK_i c_j and v_{j,i} = W^UV_i c_j for every context
 *    token j and head i ("DeepSeek-V2 ... MLA" page §2.1), into the workspace.
 *  - attend: causal attention of the t queries over [k^C_{j,i} ‖ k^R_j] and
 *    v_{j,i} (§3.2); writes out and lse.
 */
int mla_prefill_expand(const mla_dims* dims, const void* q_nope, const void* q_rope,
                       const void* w_uk, const void* w_uv, const void* cache, int32_t num_blocks,
                       const int32_t* block_table, int32_t max_blocks, const int32_t* seq_lens,
                       int32_t batch, int32_t t, float softmax_scale,
                       void* workspace, size_t workspace_bytes, void* out, float* lse,
                       int32_t* status, void* stream);
int mla_prefill_attend(const mla_dims* dims, const void* q_nope, const void* q_rope,
                       const void* w_uk, const void* w_uv, const void* cache, int32_t num_blocks,
                       const int32_t* block_table, int32_t max_blocks, const int32_t* seq_lens,
                       int32_t batch, int32_t t, float softmax_scale,
                       void* workspace, size_t workspace_bytes, void* out, float* lse,
                       int32_t* status, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
