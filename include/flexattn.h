/*
 * flexattn.h -- C ABI of the MI355X (gfx950) block-sparse masked attention
 * forward library, libflexattn.so.
 *
 * The operation is the FlexAttention forward pass: a block mask lists, per
 * Q_BLOCK-row block of queries, which KV_BLOCK-wide key blocks are partially
 * visible (kv_num_blocks / kv_indices) and which are fully visible
 * (full_kv_num_blocks / full_kv_indices); the forward walks those lists,
 * forms S = scale * Q K^T tile by tile, applies the score modification on
 * every visited tile and the mask only on partial tiles, runs the online
 * softmax (running row max, alpha rescale of the accumulator and row sum)
 * and accumulates P V, optionally writing the log-sum-exp.
 *   - Block-mask tuple fields: "[Inductor][Flex Attention] Add Subtiling
 *     Option for Alpha Scaling", test/inductor/test_flex_attention.py hunk
 *     (the tuple passed to the flex_attention higher-order op).
 *   - Online-softmax step and the alpha-rescale subtiling option: same page,
 *     common.py.jinja hunk in forward_block_mn, and the USE_SUBTILING entry
 *     of FlexKernelOptions in torch/nn/attention/flex_attention.py.
 *   - Mask semantics (prefix-bidirectional OR causal, inclusive bound,
 *     masked score = -inf): "Performance for templated attention strangely
 *     bad for a combination of causal + upper square mask", bad.py -> bad2.py.
 *
 * Conventions for every entry point:
 *   - Returns FLEX_OK (0) or a FLEX_E_* code; never throws, never aborts.
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library never allocates or frees device memory, never synchronises the
 *     stream, keeps no pointer after it returns and holds no state between
 *     calls.  Work is enqueued on `stream` (a hipStream_t; NULL = the null
 *     stream); results are ready when that stream reaches them.
 *   - Argument errors are detected on the host before anything is enqueued;
 *     on such an error nothing is launched and no output is touched.
 *   - FLEX_E_HIP means a HIP launch reported an error (hipGetLastError);
 *     outputs are then undefined.
 *   - Calls are thread-safe (no shared mutable state).
 */
#ifndef FLEXATTN_H
#define FLEXATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FLEXATTN_ABI_VERSION 8

/* ---- status codes ---- */
#define FLEX_OK 0
#define FLEX_E_INVALID_ARG 1 /* null pointer, negative or mismatched size */
#define FLEX_E_UNSUPPORTED 2 /* valid but not built: head dim, block size, dtype */
#define FLEX_E_HIP 3         /* a HIP launch failed */
#define FLEX_E_SCRATCH_LIMIT 4 /* beyond flex_attn_bwd_noalloc's scratch: 2 B H q_len > FLEX_NOALLOC_SCRATCH_FLOATS */

/* ---- element types ---- */
#define FLEX_DTYPE_BF16 0
#define FLEX_DTYPE_FP32 1

/* ---- mask kinds (mask_mod) ----
 * For query index i and key index j (0-based, i < q_len, j < kv_len):
 *   NOOP            every key is visible
 *   CAUSAL          i >= j
 *   SLIDING_WINDOW  window_min <= i - j <= window   (window_min = 0: the
 *                   causal sliding window of width window + 1)
 *   PREFIX_CAUSAL   (i <= prefix AND j <= prefix) OR i >= j   (inclusive
 *                   bound, as in the bad.py mask of the templated-attention
 *                   performance issue)
 *   DOCUMENT        q_doc[i] == kv_doc[j]
 *   DOCUMENT_CAUSAL q_doc[i] == kv_doc[j] AND i >= j
 * The document kinds are a mask_mod that closes over a tensor (the op's
 * mask_mod_other_buffers slot, which the subtiling page's test hunks show
 * holding a captured tensor): per-token document ids of packed or jagged
 * sequences.  Both id arrays must be non-decreasing (each document one run
 * of positions); then every query sees one interval of keys, which the
 * builder computes once into the block mask's row_bounds. */
#define FLEX_MASK_NOOP 0
#define FLEX_MASK_CAUSAL 1
#define FLEX_MASK_SLIDING_WINDOW 2
#define FLEX_MASK_PREFIX_CAUSAL 3
#define FLEX_MASK_DOCUMENT 4
#define FLEX_MASK_DOCUMENT_CAUSAL 5

typedef struct flex_mask_desc {
  int32_t kind;       /* FLEX_MASK_* */
  int32_t window;     /* SLIDING_WINDOW: largest visible i - j (>= window_min) */
  int32_t window_min; /* SLIDING_WINDOW: smallest visible i - j (>= 0) */
  int32_t prefix;     /* PREFIX_CAUSAL: last index of the bidirectional prefix (>= 0) */
  const int32_t* q_doc;  /* DOCUMENT*: device int32 [q_len], non-decreasing */
  const int32_t* kv_doc; /* DOCUMENT*: device int32 [kv_len], non-decreasing */
} flex_mask_desc;

/* ---- score modifications (score_mod), applied to the SCALED score s ----
 *   IDENTITY  s
 *   REL_BIAS  s - slope_h * (i - j),  slope_h = 2^(-bias_max * (h + 1) / H),
 *             h the head index, H = num_heads (an ALiBi-style bias); or,
 *             with a slope table, slope_h = slopes[h]: a score_mod that
 *             closes over a tensor (what the op's score_mod_other_buffers
 *             slot in the subtiling page's test hunks carries).  The table
 *             is read, never differentiated: the backward gives no gradient
 *             for it. */
#define FLEX_SCORE_IDENTITY 0
#define FLEX_SCORE_REL_BIAS 1

typedef struct flex_score_desc {
  int32_t kind;      /* FLEX_SCORE_* */
  int32_t num_heads; /* REL_BIAS: H in the slope formula; must equal the call's H */
  float bias_max;    /* REL_BIAS without a table: 8 for the usual ALiBi slopes; finite */
  const float* slopes; /* REL_BIAS: NULL, or device fp32 [num_heads], 4-byte aligned,
                          finite values (any sign), read by the kernels; bias_max
                          is then ignored.  The caller keeps it alive until the
                          call's work on the stream is done. */
} flex_score_desc;

/* ---- block mask, as consumed by flex_attn_fwd ----
 * Built by flex_attn_build_block_mask (or by the caller, in the same format):
 *   kv_num_blocks[qb]            number of partial tiles of q-block qb
 *   kv_indices[qb * n_kv_blocks + n], n < kv_num_blocks[qb]: their kv-block
 *                                indices (the rest of the row is padding)
 *   full_kv_num_blocks / full_kv_indices: the same for full tiles.
 * A tile is full when every (i, j) in it is visible and in range, partial
 * when some are, and listed in neither array when none are.  The mask
 * descriptor travels with the arrays because partial tiles evaluate it per
 * element.  The forward reads the arrays on the device; entries outside
 * [0, n_kv_blocks) are clamped, so a malformed array gives wrong results but
 * no out-of-bounds access. */
typedef struct flex_block_mask {
  flex_mask_desc mask;
  int32_t q_len, kv_len;           /* sequence lengths the mask was built for */
  int32_t q_block, kv_block;       /* Q_BLOCK, KV_BLOCK */
  int32_t n_q_blocks, n_kv_blocks; /* ceil(q_len / q_block), ceil(kv_len / kv_block) */
  const int32_t* kv_num_blocks;      /* device, [n_q_blocks] */
  const int32_t* kv_indices;         /* device, [n_q_blocks, n_kv_blocks] */
  const int32_t* full_kv_num_blocks; /* device, [n_q_blocks] */
  const int32_t* full_kv_indices;    /* device, [n_q_blocks, n_kv_blocks] */
  /* DOCUMENT*: device int32 [2 * q_len], the keys query i sees are
   * row_bounds[2i] .. row_bounds[2i + 1] (empty when the first is larger),
   * written by flex_attn_build_block_mask.  NULL for the other kinds. */
  const int32_t* row_bounds;
} flex_block_mask;

/* ---- transposed block mask, as consumed by the backward ----
 * The same tile classes listed per kv-block column: the q_num_blocks /
 * q_indices / full_q_num_blocks / full_q_indices fields of the block-mask
 * tuple passed to the flex_attention higher-order op in the test hunks of
 * "[Inductor][Flex Attention] Add Subtiling Option for Alpha Scaling".
 * q_num_blocks[kb] partial q-blocks of column kb are listed ascending at
 * q_indices[kb * n_q_blocks ...], followed by every other q-block ascending
 * (each column a permutation of 0 .. n_q_blocks - 1); the same for the full
 * tiles.  Built by flex_attn_build_block_mask_t.  All pointers are device
 * pointers owned by the caller. */
typedef struct flex_block_mask_t {
  int32_t q_block, kv_block;      /* the forward block mask's block sizes */
  int32_t n_q_blocks, n_kv_blocks;
  const int32_t* q_num_blocks;       /* [n_kv_blocks] */
  const int32_t* q_indices;          /* [n_kv_blocks * n_q_blocks] */
  const int32_t* full_q_num_blocks;  /* [n_kv_blocks] */
  const int32_t* full_q_indices;     /* [n_kv_blocks * n_q_blocks] */
  /* DOCUMENT*: device int32 [2 * kv_len], the queries that see key j are
   * col_bounds[2j] .. col_bounds[2j + 1], written by
   * flex_attn_build_block_mask_t.  NULL for the other kinds. */
  const int32_t* col_bounds;
} flex_block_mask_t;

/* Forward kernel options: the entries of the kernel_options dict the
 * flex_attention higher-order op receives in the test hunks of the subtiling
 * page (all False by default there, and 0 here).  The page names them but
 * does not define them; the meanings below are the plain readings. */
typedef struct flex_fwd_options {
  /* USE_SUBTILING: rescale the output accumulator by alpha in two halves of
   * the head dimension, each just before the P V products that update it.
   * Results are bitwise identical either way; only instruction order changes. */
  int32_t use_subtiling;
  /* PRESCALE_QK: multiply q by scale (times log2 e, the kernel's base-2
   * units) and round it to the input type once, before Q K^T, instead of
   * scaling each score.  The scores then carry the rounding of q: for bf16
   * inputs up to 2^-9 * scale * sum_d |q_d k_d| per score. */
  int32_t prescale_qk;
  /* ROWS_GUARANTEED_SAFE: the caller promises that every query row sees at
   * least one key; the guards that give such a row out = 0 and lse = -inf
   * are dropped.  A row that sees no key then gets undefined out and lse. */
  int32_t rows_guaranteed_safe;
  /* BLOCKS_ARE_CONTIGUOUS: the caller promises that each index list is
   * consecutive, kv_indices[qb, n] = kv_indices[qb, 0] + n for n below the
   * count (and the same for full_kv_indices); only the first entry of each
   * list is read.  Results are undefined (never out of bounds) if not. */
  int32_t blocks_are_contiguous;
} flex_fwd_options;

/* Returns FLEXATTN_ABI_VERSION. */
int32_t flex_attn_abi_version(void);

/* Human-readable text for a status code; a static string, never NULL. */
const char* flex_attn_strerror(int32_t code);

/* Host only.  n_q_blocks = ceil(q_len / q_block), n_kv_blocks =
 * ceil(kv_len / kv_block).  Lengths may be 0; block sizes must be > 0.
 * Errors: FLEX_E_INVALID_ARG (null output pointer, negative length,
 * non-positive block size). */
int32_t flex_attn_block_mask_dims(int32_t q_len, int32_t kv_len, int32_t q_block,
                                  int32_t kv_block, int32_t* n_q_blocks,
                                  int32_t* n_kv_blocks);

/* Build the four block arrays for a mask kind on the device.
 *   mask        host pointer to the mask descriptor.
 *   q_len, kv_len >= 0 (any value: the last blocks may be ragged).
 *   q_block, kv_block: 1 .. 1024.
 *   outputs: device int32 arrays, [n_q_blocks] and [n_q_blocks * n_kv_blocks].
 *   Every index row is written in full: the selected kv-blocks in ascending
 *   order, then every other kv-block in ascending order.
 *   row_bounds: DOCUMENT*: device int32 [2 * q_len], receives each query's
 *   visible key interval (pass it on in flex_block_mask.row_bounds); may be
 *   NULL for the other kinds.  The id arrays are read on the device and
 *   checked there: if either array has an id below its predecessor, every
 *   query's interval is set to the empty pair (INT32_MAX, INT32_MIN), no
 *   kv-block is listed, and the forward writes NaN to every output row and
 *   log-sum-exp of the call (the backward NaN to every dq, dk and dv row),
 *   so the broken precondition shows in the results.  No error code: the
 *   check runs on the stream, after the call has returned.
 * Errors: FLEX_E_INVALID_ARG (null pointer with a non-empty output, bad sizes,
 * bad mask parameters), FLEX_E_UNSUPPORTED (unknown mask kind), FLEX_E_HIP. */
int32_t flex_attn_build_block_mask(const flex_mask_desc* mask, int32_t q_len,
                                   int32_t kv_len, int32_t q_block,
                                   int32_t kv_block, int32_t* kv_num_blocks,
                                   int32_t* kv_indices,
                                   int32_t* full_kv_num_blocks,
                                   int32_t* full_kv_indices, int32_t* row_bounds,
                                   void* stream);

/* Build the four transposed block arrays (the q_num_blocks / q_indices /
 * full_q_num_blocks / full_q_indices fields of the block-mask tuple in the
 * test hunks of the subtiling page) on the device.
 *   mask, q_len, kv_len, q_block, kv_block: as flex_attn_build_block_mask.
 *   outputs: device int32 arrays, [n_kv_blocks] and [n_kv_blocks * n_q_blocks];
 *   every column is written in full (selected q-blocks ascending, then the
 *   others ascending).
 *   col_bounds: DOCUMENT*: device int32 [2 * kv_len], receives the interval
 *   of queries that see each key (pass it on in flex_block_mask_t.col_bounds);
 *   may be NULL for the other kinds.  Ids out of order are caught as in
 *   flex_attn_build_block_mask: every key's interval becomes the empty pair
 *   (INT32_MAX, INT32_MIN), no q-block is listed, and the backward writes
 *   NaN to every dk and dv row.
 * Errors: as flex_attn_build_block_mask. */
int32_t flex_attn_build_block_mask_t(const flex_mask_desc* mask, int32_t q_len,
                                     int32_t kv_len, int32_t q_block,
                                     int32_t kv_block, int32_t* q_num_blocks,
                                     int32_t* q_indices,
                                     int32_t* full_q_num_blocks,
                                     int32_t* full_q_indices, int32_t* col_bounds,
                                     void* stream);

/* Attention forward.
 *   q [B, H, q_len, head_dim], k [B, H, kv_len, head_dim],
 *   v [B, H, kv_len, v_head_dim]: contiguous, element type in_dtype, 16-byte
 *   aligned device pointers.  v_head_dim may differ from head_dim (the
 *   V_HEAD_DIM of the pages' kernel template).
 *   bm: host pointer; bm->q_len / kv_len must equal the call's; its block
 *   sizes select the kernel.  bm->mask is applied on partial tiles.
 *   score: host pointer, NULL = identity.
 *   scale: finite and non-zero (pass 1/sqrt(head_dim) for the usual default).
 *   out [B, H, q_len, v_head_dim] of out_dtype, contiguous, 16-byte aligned.
 *   lse: NULL, or fp32 [B, H, q_len]: natural-log log-sum-exp of the scores
 *   of each row; -inf (and out = 0) for a row that sees no key
 *   (OUTPUT_LOGSUMEXP of the test hunks).
 *   max_out: NULL, or fp32 [B, H, q_len]: the largest visible score of each
 *   row (scaled, after the score modification; -inf for a row that sees no
 *   key), the third output of the op (OUTPUT_MAX).  Requesting it runs the
 *   exact running max on every block.
 *   opt: host pointer, NULL = defaults (every option 0).
 * Built instances: in_dtype BF16 or FP32, head_dim and v_head_dim each 64 or
 * 128; (q_block, kv_block) in {(64, 64), (128, 64), (128, 128)}; any mask
 * kind and score kind; out_dtype BF16 or FP32.  q_len, kv_len >= 0 (ragged last
 * blocks are fine), B, H >= 0, B * H * n_q_blocks < 2^31.
 * Debugging: with the environment variable FLEXATTN_DEBUG_LDS_POISON set
 * (to anything but "0"; read on every call) the BF16-input forward fills
 * each K/V staging buffer in LDS with NaN, behind a work-group barrier,
 * before the loads that refill it are issued.  A read of a buffer before its
 * loads have landed, or after the next loads began to overwrite it, then
 * gives NaN output instead of plausible wrong values.  The results are
 * otherwise bit-identical; the calls are slower.
 * Errors: FLEX_E_INVALID_ARG, FLEX_E_UNSUPPORTED, FLEX_E_HIP. */
int32_t flex_attn_fwd(const void* q, const void* k, const void* v,
                      int32_t in_dtype, int32_t B, int32_t H, int32_t q_len,
                      int32_t kv_len, int32_t head_dim, int32_t v_head_dim,
                      const flex_block_mask* bm, const flex_score_desc* score,
                      float scale, void* out, int32_t out_dtype, float* lse,
                      float* max_out, const flex_fwd_options* opt, void* stream);

/* Host only.  Floats of device workspace flex_attn_bwd needs:
 * 2 * B * H * q_len.  Errors: FLEX_E_INVALID_ARG (null output, negative size). */
int32_t flex_attn_bwd_workspace_floats(int32_t B, int32_t H, int32_t q_len,
                                       int64_t* n_floats);

/* Attention backward: gradients of q, k and v (the outputs of the
 * flex_attention_backward higher-order op in the test hunks of the subtiling
 * page, which takes q, k, v, the forward output and log-sum-exp, the output
 * gradient and a log-sum-exp gradient).  For every visible pair (i, j), with
 * p_ij = exp(s_ij - lse_i) and delta_i = <dout_i, out_i> - dlse_i:
 *   ds_ij = p_ij (<dout_i, v_j> - delta_i),
 *   dq_i = scale sum_j ds_ij k_j,  dk_j = scale sum_i ds_ij q_i,
 *   dv_j = sum_i p_ij dout_i.
 *   q [B, H, q_len, head_dim], k [B, H, kv_len, head_dim],
 *   v [B, H, kv_len, v_head_dim], out, dout [B, H, q_len, v_head_dim]:
 *   contiguous, element type in_dtype, 16-byte aligned device pointers; out
 *   and lse must be the forward's results for these inputs, mask and score.
 *   lse: fp32 [B, H, q_len] (natural log; -inf for a row that sees no key).
 *   dlse: NULL (zero) or fp32 [B, H, q_len].
 *   bm: the forward's block mask; bmt: its transpose (same mask and block
 *   sizes), both host pointers to structs of device arrays.
 *   score, scale: as in the forward call.
 *   dq [B, H, q_len, head_dim], dk [B, H, kv_len, head_dim],
 *   dv [B, H, kv_len, v_head_dim] of grad_dtype (BF16 or FP32), 16-byte
 *   aligned, written in full (zero where nothing contributes).
 *   dq may be NULL: the WRITE_DQ kernel option of the test hunks set to
 *   False (the flex_attention_backward call there passes it among its
 *   kernel options).  The dq kernel is then not run, nothing is written in
 *   its place, and dk and dv are the same as with dq requested.
 *   workspace: device fp32, flex_attn_bwd_workspace_floats() floats, owned by
 *   the caller; its contents on entry are ignored and left undefined.
 * Built instances: in_dtype BF16 or FP32, head_dim and v_head_dim each 64 or
 * 128; (q_block, kv_block) in {(64, 64), (128, 64), (128, 128)}, any mask
 * kind and score kind.  BF16 inputs take the products on the matrix cores (p and ds rounded
 * to bf16, fp32 sums); FP32 inputs keep every product and sum in fp32.
 * Errors: FLEX_E_INVALID_ARG, FLEX_E_UNSUPPORTED (other instances, scale 0
 * or not finite), FLEX_E_HIP. */
int32_t flex_attn_bwd(const void* q, const void* k, const void* v, const void* out,
                      const void* dout, const float* lse, const float* dlse,
                      int32_t in_dtype, int32_t B, int32_t H, int32_t q_len,
                      int32_t kv_len, int32_t head_dim, int32_t v_head_dim,
                      const flex_block_mask* bm, const flex_block_mask_t* bmt,
                      const flex_score_desc* score, float scale, void* dq, void* dk,
                      void* dv, int32_t grad_dtype, float* workspace, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * as flex_attn_bwd, with the same arguments and errors, but without the
 * workspace argument.  The workspace is a file-scope device array of the
 * library, FLEX_NOALLOC_SCRATCH_FLOATS floats (32 MiB), one copy per GPU,
 * held until the process ends; the call itself allocates nothing.
 *   Limit: 2 * B * H * q_len <= FLEX_NOALLOC_SCRATCH_FLOATS (2^22 query rows
 *   in all); larger calls return FLEX_E_SCRATCH_LIMIT before anything is
 *   launched.
 *   Every call on a GPU uses that GPU's one array, so calls whose work
 *   overlaps on one GPU (concurrent streams, other threads) race on it: the
 *   caller orders them.  Nothing in the array needs to start at zero (each
 *   call writes every element it reads first). */
#define FLEX_NOALLOC_SCRATCH_FLOATS (1 << 23)
int32_t flex_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* out,
                              const void* dout, const float* lse, const float* dlse,
                              int32_t in_dtype, int32_t B, int32_t H, int32_t q_len,
                              int32_t kv_len, int32_t head_dim, int32_t v_head_dim,
                              const flex_block_mask* bm, const flex_block_mask_t* bmt,
                              const flex_score_desc* score, float scale, void* dq, void* dk,
                              void* dv, int32_t grad_dtype, void* stream);

/* Measurement helper, not part of the attention path: the matrix-unit peak
 * the forward's rate is compared with.  Launches n_workgroups work-groups of
 * 256 threads (4 waves); every wave runs `iters` rounds of 4 independent
 * v_mfma_f32_32x32x16_bf16 (32 * 32 * 16 * 2 = 32768 FLOPs each), so the
 * launch does n_workgroups * 4 * iters * 4 * 32768 FLOPs; the caller times
 * it on `stream`.  Launch 4 work-groups per compute unit (4 waves per SIMD)
 * or more to fill the part.
 *   sink: device fp32 [n_workgroups * 256] (receives sums of the
 *   accumulators, so that no product is dead code).
 *   clocks: device uint64 [n_workgroups * 4 * 2]; wave w writes
 *   clocks[2w] = shader clock cycles (s_memtime) and clocks[2w + 1] = ticks
 *   of the 100 MHz real-time counter (s_memrealtime) over its chains, so the
 *   shader clock under this load is 0.1 GHz * clocks[2w] / clocks[2w + 1].
 * Errors: FLEX_E_INVALID_ARG (non-positive sizes, null or misaligned
 * pointers), FLEX_E_HIP. */
int32_t flex_attn_mfma_peak_probe(int32_t n_workgroups, int32_t iters, float* sink,
                                  uint64_t* clocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FLEXATTN_H */
