/*
 * msa.h - C ABI of the MiniMax Sparse Attention (MSA) forward path on AMD
 * Instinct MI355X (gfx950).
 *
 * The path has three stages, in the order the MiniMax-AI/MSA README (section
 * "Usage") runs them and the MSA news summary ("MSA; MiniMax sparse attention
 * kernels for SM100 GPUs", paragraph on the three-step flow) describes:
 *
 *   1. msa_proxy_block_maxscore - a cheap dense proxy pass whose only output
 *      is, per query row, proxy head and 128-token KV block, the largest
 *      scaled proxy logit in that block (causal).
 *   2. msa_topk_select          - per (row, KV group) the `topk` best blocks,
 *      the row's own (local) block always kept (Flash-MSA article, paragraph
 *      on the forward kernels).
 *      msa_proxy_topk_select runs 1 and 2 as one pass, keeping each row's
 *      best blocks in registers instead of writing max_score.
 *   3. msa_sparse_attn_prefill  - GQA attention over only the selected blocks
 *      of a paged K/V cache (README "Usage": kv_block_indexes argument),
 *      msa_sparse_attn_decode   - its one-token-per-sequence paged decode
 *      form with fp8 or bf16 K/V (README "Stacks": paged FP8 decode wrapper).
 *
 * msa_plan turns the per-sequence lengths into a host plan (README "Usage":
 * the plan is built from qo_lens / kv_lens, heads and page size, then run).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers named *_host are host memory; every other tensor pointer is
 *    device memory on the current HIP device.  All tensors are dense,
 *    row-major and 16-byte aligned.  The caller owns every buffer.
 *  - The library allocates no device memory.  Each call is enqueued on the
 *    caller's `stream` and returns without synchronising; results are ready
 *    when the stream reaches that point.  Every compute call therefore takes
 *    the plan's device workspace (workspace, workspace_bytes: at least what
 *    msa_plan returned) for its scratch: CSR lists, partial outputs, the
 *    plan's metadata.
 *  - max_score (stage 1's output, stage 2's input) is [P, nb_max, row_count]
 *    with rows fastest, not [rows, P, nb_max]: the proxy kernel writes 64
 *    consecutive rows per wave per block and the top-k kernel reads 64
 *    consecutive rows per load, both as whole 256-byte lines.
 *  - Rows: the query rows of all sequences are concatenated, T = sum(qo_len).
 *    Row i of sequence s sits at KV position kv_len[s] - qo_len[s] + i
 *    (causal, bottom-right aligned).  Key j is visible to it iff j <= that
 *    position (the diagonal counts) and j < kv_len[s].
 *  - Pages: page_size = 128 = block size.  kv_indices is one flat int32 list;
 *    sequence s owns its ceil(kv_len[s]/128) entries starting right after
 *    those of sequences 0..s-1.  Key j of sequence s is slot j % 128 of page
 *    kv_indices[start_s + j / 128].  Page pools are
 *    [num_pages, heads, 128, head_dim] (the README's k_pages.shape[1] is the
 *    KV head count).  Slots past kv_len in a sequence's last page are never
 *    read into results (they may hold anything, NaN included).
 *  - Block ids in kv_block_indexes are logical blocks of the row's sequence
 *    (0-based), ascending, padded with -1.
 *  - head_dim = proxy head_dim = 128; page_size = 128.
 *  - bf16 = IEEE bfloat16; fp8 = OCP E4M3FN.  fp8 tensors carry one fp32
 *    scale per head (value = code x scale).
 *  - Every call returns msa_status_t; on failure msa_last_error() gives a
 *    message (thread-local, valid until the thread's next call).  No C++
 *    exception crosses this boundary.  Argument errors are detected on the
 *    host before anything is enqueued.  Device-side data errors (page ids
 *    outside the pool, block ids beyond the row's local block) are not
 *    checked and lead to undefined results.
 */
#ifndef MSA_H_
#define MSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct msa_plan_s* msa_plan_t;
typedef void* msa_stream_t; /* a hipStream_t; NULL = the null stream */

typedef enum {
  MSA_OK = 0,
  MSA_ERR_INVALID_ARG = 1,         /* bad pointer, size, range or combination */
  MSA_ERR_UNSUPPORTED = 2,         /* valid but not built (head_dim != 128 ...) */
  MSA_ERR_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes smaller than the plan's */
  MSA_ERR_HIP = 4                  /* the HIP runtime reported an error */
} msa_status_t;

/* MSA_MXFP4 and MSA_MXFP4_QK are proxy dtypes only (desc.proxy_dtype): the
 * low-precision block-score indexer of the README's "Stacks" list, in the FP4
 * format gfx950 matrix cores consume (OCP microscaling FP4: E2M1 codes, one
 * E8M0 scale per 32 dims, value = e2m1(code) * 2^(scale - 127)).
 *   MSA_MXFP4     proxy q fp8 e4m3 with per-head scales, proxy K MXFP4;
 *   MSA_MXFP4_QK  proxy q and proxy K both MXFP4 (twice the matrix-core rate
 *                 of fp8 in the prefill proxy pass).
 * An MXFP4 proxy-K page of one head is a record of 128 * 64 bytes of codes
 * (slot-major; element 2i of a row in the low nibble of byte i) followed by
 * 128 * 4 scale bytes (slot-major; byte c scales dims 32c..32c+31): 8704
 * bytes.  An MXFP4 proxy q row (one row, one head) is its 64 code bytes then
 * its 4 scale bytes: 68 bytes, rows contiguous ([T, P, 68]). */
typedef enum { MSA_BF16 = 0, MSA_FP8_E4M3 = 1, MSA_MXFP4 = 2, MSA_MXFP4_QK = 3 } msa_dtype_t;
typedef enum { MSA_PREFILL = 0, MSA_DECODE = 1 } msa_mode_t;

typedef struct {
  int32_t batch;               /* number of sequences, >= 1 */
  const int32_t* qo_lens_host; /* [batch] query rows per sequence (copied) */
  const int32_t* kv_lens_host; /* [batch] keys per sequence, >= qo_len (copied) */
  int32_t num_qo_heads;        /* H_q */
  int32_t num_kv_heads;        /* H_kv; H_q % H_kv == 0, G = H_q / H_kv in {1,2,4,8,16} */
  int32_t num_proxy_heads;     /* P == H_kv (prefill); proxy head p drives KV group p */
  int32_t num_proxy_kv_heads;  /* P_k: 1 (shared) or P */
  int32_t head_dim;            /* 128 */
  int32_t page_size;           /* 128 */
  int32_t topk;                /* slots per (row, group), local block included; 1..64 */
  msa_dtype_t kv_dtype;        /* K/V pages: bf16 or fp8 (prefill, decode), MXFP4 (prefill) */
  msa_dtype_t proxy_dtype;     /* proxy q and proxy k pages: bf16, fp8, MXFP4 (fp8 q,
                                  MXFP4 K) or MXFP4_QK (both MXFP4) */
  float sm_scale;              /* main attention logit scale */
  float proxy_sm_scale;        /* proxy logit scale */
  msa_mode_t mode;             /* which entry points the plan serves */
  int64_t max_rows_per_call;   /* prefill: rows per proxy/top-k call; 0 = min(T, 32768) */
  int64_t attn_window_rows;    /* prefill: rows whose attention partials are live at
                                  once (workspace scales with it); 0 = automatic.
                                  Capped at (2^27 - 256) / (num_qo_heads * topk) */
  int32_t decode_splits;       /* decode: workgroups sharing one (sequence, group),
                                  merged by log-sum-exp; 0 = automatic, else 1..64 */
} msa_plan_desc_t;

/* Build a host plan from `desc`.  Validates every field; touches no device.
 * *workspace_bytes receives the device workspace size the compute calls need
 * (the caller allocates it).  The plan is released by msa_plan_destroy.
 *
 * Environment, read here: MSA_XCD_PIN=1 makes the plan's sparse attention
 * deal each KV group's work items to one XCD (Hkv a multiple of 8) or to
 * 8 / Hkv XCDs (Hkv dividing 8), so that with a small attn_window_rows the
 * group's gathered query rows stay in that XCD's L2.  Results are
 * bit-identical; with the default window it is slower (a tuning knob, off
 * by default).
 *
 * Workspace metadata: the first call that uses a workspace with a plan
 * copies the plan's small metadata (row and page offsets, proxy row tiles)
 * into it, enqueued on that call's stream.  The library records which plan's
 * metadata each workspace holds and copies it again whenever that record does
 * not match: another plan, another stream, or another plan's call whose
 * workspace overlaps this metadata.  Memory written by anything outside the
 * library must be announced with msa_workspace_reset before it is used as a
 * workspace again.  Calls sharing one workspace must not overlap in time
 * (their streams must be ordered).
 * Errors: INVALID_ARG for bad fields; UNSUPPORTED for shapes that are valid
 * but not built (head_dim or page_size != 128, G not in {1,2,4,8,16}, a
 * sequence of more than 65536 blocks = 8388608 keys). */
msa_status_t msa_plan(const msa_plan_desc_t* desc, msa_plan_t* plan, size_t* workspace_bytes);

msa_status_t msa_plan_destroy(msa_plan_t plan);

/* Forget the metadata records of every workspace whose metadata lies in
 * [workspace, workspace + bytes) (host only, nothing is enqueued): the next
 * call using such a workspace copies its plan's metadata again.  Call it when
 * that memory was freed and reallocated, or written by anything other than
 * this library.  Errors: INVALID_ARG for a NULL workspace. */
msa_status_t msa_workspace_reset(const void* workspace, size_t bytes);

/* Stage 1: proxy block max scores (README "Usage", proxy pass with
 * output_maxscore; Flash-MSA article, max-pooling of proxy scores over
 * 128-token blocks).
 *
 * For rows r in [row_begin, row_begin + row_count), proxy head p and block b
 * of r's sequence with b <= local(r) = position(r) / 128:
 *   max_score[p][b][r - row_begin] = max over visible keys j of block b of
 *       proxy_sm_scale * qs[p] * ks[pk(p)] * <proxy_q[r][p], proxy_k[j][pk(p)]>
 * where pk(p) = p if P_k = P else 0, and qs/ks are the fp8 scales (1 for
 * bf16).  Entries with b > local(r) are left unspecified (may be written).
 *
 *   proxy_q        [T, P, 128]  bf16 or fp8 (desc.proxy_dtype; fp8 for MXFP4);
 *                  MXFP4_QK: [T, P, 68 B] rows (see MSA_MXFP4)
 *   proxy_k_pages  [num_pages, P_k, 128, 128], bf16 or fp8; MXFP4 and
 *                  MXFP4_QK: [num_pages, P_k, 8704 B] records
 *   proxy_q_scale  [P]   fp32, device; given iff proxy q is fp8 (fp8, MXFP4)
 *   proxy_k_scale  [P_k] fp32, device; given iff proxy K is fp8
 *   kv_indices     int32 flat page table (see conventions)
 *   max_score      fp32 [P, nb_max, row_count], nb_max = max over sequences
 *                  of ceil(kv_len / 128); row_count <= plan's max_rows_per_call
 * Plans whose every sequence has exactly one query row (the indexer pass of a
 * decode step) run a kernel that streams each sequence's proxy-K blocks
 * once for all proxy heads; the results are the same.
 * Errors: INVALID_ARG for a null pointer, a row range outside [0, T), an
 * empty range, or a scale pointer that does not match the dtype;
 * UNSUPPORTED if the plan is a decode plan. */
msa_status_t msa_proxy_block_maxscore(msa_plan_t plan, const void* proxy_q, const void* proxy_k_pages,
                                      const float* proxy_q_scale, const float* proxy_k_scale,
                                      const int32_t* kv_indices, int64_t row_begin, int64_t row_count,
                                      float* max_score, void* workspace, size_t workspace_bytes,
                                      msa_stream_t stream);

/* Stage 2: top-k block selection (README "Usage", sparse_topk_select with
 * `topk` slots; Flash-MSA article: each token's local block always stays
 * visible, each proxy head selects for its own KV group).
 *
 * For each row r in the range and group g (= proxy head g): the local block
 * plus the topk-1 highest-scoring blocks among 0..local-1 (ties: lower block
 * id), ascending, -1 padded, written to kv_block_indexes[r][g][0..topk).
 * When local < topk - 1 every block 0..local is selected.
 *
 *   max_score         fp32 [P, nb_max, row_count] as written by stage 1
 *   kv_block_indexes  int32 [T, H_kv, topk]; only the rows of the range are written
 * Errors: as stage 1. */
msa_status_t msa_topk_select(msa_plan_t plan, const float* max_score, int64_t row_begin, int64_t row_count,
                             int32_t* kv_block_indexes, void* workspace, size_t workspace_bytes,
                             msa_stream_t stream);

/* Stages 1 and 2 fused: the proxy pass keeps each row's best blocks as it
 * goes and writes the selection directly, with no max_score round trip (the
 * streaming selection with an in-register insertion sort that the Flash-MSA
 * article describes for its proxy attention, paragraph on the forward
 * kernels).  The result equals msa_proxy_block_maxscore followed by
 * msa_topk_select on the same inputs, bit for bit (same fp32 scores, same
 * tie rule).
 *
 * Arguments as in stages 1 and 2; rows [row_begin, row_begin + row_count)
 * may span the whole batch (no max_rows_per_call limit: nothing is staged).
 * Errors: as stage 1; UNSUPPORTED if the plan's topk exceeds 17 (at most 16
 * competing blocks are kept per row; use the two separate calls then). */
msa_status_t msa_proxy_topk_select(msa_plan_t plan, const void* proxy_q, const void* proxy_k_pages,
                                   const float* proxy_q_scale, const float* proxy_k_scale,
                                   const int32_t* kv_indices, int64_t row_begin, int64_t row_count,
                                   int32_t* kv_block_indexes, void* workspace, size_t workspace_bytes,
                                   msa_stream_t stream);

/* Stage 3a: block-sparse GQA prefill attention (README "Usage", attention
 * run with kv_block_indexes; Flash-MSA article: GQA main attention,
 * block-sparse flash attention reformulated as variable-length attention).
 *
 * For every row r and query head h (group g = h / G):
 *   keys K = { j : j / 128 in kv_block_indexes[r][g][:], j visible to r }
 *   out[r][h] = sum_j softmax_j(sm_scale * <q[r][h], k[j][g]>) v[j][g]
 *   lse[r][h] = natural log of sum_j exp(sm_scale * <q[r][h], k[j][g]>)
 * Every selection must contain the row's local block (stage 2 guarantees it).
 *
 *   q                 bf16 [T, H_q, 128]
 *   k_pages, v_pages  [num_pages, H_kv, 128, 128] bf16 or fp8 (desc.kv_dtype),
 *                     or MXFP4 records [num_pages, H_kv, 8704 B] (the record
 *                     layout of MSA_MXFP4 proxy K pages)
 *   k_scale, v_scale  fp32 [H_kv] device, given iff K/V are fp8 (value = code
 *                     x scale); NULL for bf16 and MXFP4
 *   kv_block_indexes  int32 [T, H_kv, topk]
 *   out               bf16 [T, H_q, 128]
 *   lse               fp32 [T, H_q] or NULL
 * fp8 and MXFP4 codes are widened to bf16 exactly (MXFP4 with its block
 * scale) before the bf16 matrix products; fp8 per-head scales multiply the
 * logits and the output.
 * Errors: INVALID_ARG for null pointers or scales that do not match the K/V
 * dtype; UNSUPPORTED for a decode plan; WORKSPACE_TOO_SMALL. */
msa_status_t msa_sparse_attn_prefill(msa_plan_t plan, const void* q, const void* k_pages, const void* v_pages,
                                     const float* k_scale, const float* v_scale, const int32_t* kv_indices,
                                     const int32_t* kv_block_indexes, void* out, float* lse, void* workspace,
                                     size_t workspace_bytes, msa_stream_t stream);

/* Stage 3a on the rows [row_begin, row_begin + row_count) only: the same
 * results for those rows, nothing else written.  Lets a caller overlap the
 * attention of one row range with the selection pass of the next (a second
 * stream); calls sharing one workspace must not overlap each other.
 * Arguments as in msa_sparse_attn_prefill; out and lse are the full [T, ...]
 * tensors.  Errors: as msa_sparse_attn_prefill, plus INVALID_ARG for a row
 * range outside [0, T) or an empty range. */
msa_status_t msa_sparse_attn_prefill_rows(msa_plan_t plan, const void* q, const void* k_pages, const void* v_pages,
                                          const float* k_scale, const float* v_scale, const int32_t* kv_indices,
                                          const int32_t* kv_block_indexes, void* out, float* lse, int64_t row_begin,
                                          int64_t row_count, void* workspace, size_t workspace_bytes,
                                          msa_stream_t stream);

/* Training backward of stage 3a (Flash-MSA article, backward paragraphs:
 * the forward pass's block indexes are cached and reused, so the backward
 * runs over the same selection).  With P the softmax of row r, head h over
 * its keys K(r, g) and dout the upstream gradient:
 *   dv[j] += P_j dout[r][h]
 *   ds_j   = P_j (<dout[r][h], v_j> - <dout[r][h], out[r][h]>)
 *   dq[r][h] = sm_scale sum_j ds_j k_j,   dk[j] += sm_scale ds_j q[r][h]
 *
 *   q, k_pages, v_pages, kv_indices, kv_block_indexes: as in the forward
 *                     (bf16 K/V only)
 *   out, lse          the forward's output (bf16) and log-sum-exp (fp32,
 *                     natural log) for the same inputs
 *   dout              bf16 [T, H_q, 128]
 *   dq                fp32 [T, H_q, 128], fully written
 *   dk_pages, dv_pages fp32 [num_pages, H_kv, 128, 128]: every (page, head)
 *                     that holds a block of some sequence is written (0 where
 *                     no row attends to it); other pages are not touched
 * Results are bit-reproducible when the plan's attention window is at most
 * 65536 rows (the default window is): the rows that selected a block are then
 * summed in a fixed order for dk/dv (ascending rows, in two interleaved chunk
 * groups added at the end), and the per-slot dq partials in slot order.
 * Errors: INVALID_ARG for null or misaligned pointers; UNSUPPORTED for a
 * decode plan or non-bf16 K/V; WORKSPACE_TOO_SMALL. */
msa_status_t msa_sparse_attn_prefill_backward(msa_plan_t plan, const void* q, const void* k_pages,
                                              const void* v_pages, const int32_t* kv_indices,
                                              const int32_t* kv_block_indexes, const void* out, const float* lse,
                                              const void* dout, float* dq, float* dk_pages, float* dv_pages,
                                              void* workspace, size_t workspace_bytes, msa_stream_t stream);

/* Fused training backward of the main attention and of the proxy's
 * distillation loss (Flash-MSA article, backward paragraph: the KL divergence
 * between the proxy's and the main attention's distributions needs both at
 * once, and its gradient with respect to a proxy score is the proxy
 * probability minus the main probability).  Computes everything
 * msa_sparse_attn_prefill_backward computes, plus, for row r and KV group g
 * (driven by proxy head g) over the row's visible keys j (j <= pos, j < kv_len):
 *   p_proxy_j = softmax_j(z_j),  z_j = proxy_sm_scale <proxy_q[r][g], proxy_k[j][g]>
 *   p_main_j  = (1/G) sum over the group's heads h of the main attention
 *               probability of key j (0 off the cached selection)
 *   dz_j      = kl_grad_scale (p_proxy_j - p_main_j)
 *   dproxy_q[r][g]  = proxy_sm_scale sum_j dz_j proxy_k[j][g]
 *   dproxy_k[j][g] += proxy_sm_scale dz_j proxy_q[r][g]
 * i.e. the gradient of kl_grad_scale * sum_(r,g) KL(p_main || p_proxy) with
 * p_main held fixed.  The main probabilities use the forward's lse, as the
 * main gradients do.
 *
 *   main operands as in msa_sparse_attn_prefill_backward
 *   proxy_q           bf16 [T, H_kv, 128]
 *   proxy_k_pages     bf16 [num_pages, H_kv, 128, 128] (same page table)
 *   kl_grad_scale     upstream gradient of the summed KL (finite)
 *   dproxy_q          fp32 [T, H_kv, 128], fully written
 *   dproxy_k_pages    fp32 [num_pages, H_kv, 128, 128]: pages of sequences
 *                     written, other pages not touched
 *   proxy_lse         fp32 [T, H_kv]: log-sum-exp (natural log) of z over the
 *                     row's visible keys, written
 * The plan needs proxy_dtype BF16 and num_proxy_heads == num_proxy_kv_heads
 * == num_kv_heads; its workspace then holds the proxy term's per-slot
 * partials.  Errors: INVALID_ARG for null or misaligned pointers or a
 * non-finite kl_grad_scale; UNSUPPORTED for a decode plan, non-bf16 K/V or a
 * plan without that proxy shape; WORKSPACE_TOO_SMALL. */
msa_status_t msa_sparse_attn_prefill_backward_kl(msa_plan_t plan, const void* q, const void* k_pages,
                                                 const void* v_pages, const int32_t* kv_indices,
                                                 const int32_t* kv_block_indexes, const void* out, const float* lse,
                                                 const void* dout, const void* proxy_q, const void* proxy_k_pages,
                                                 float kl_grad_scale, float* dq, float* dk_pages, float* dv_pages,
                                                 float* dproxy_q, float* dproxy_k_pages, float* proxy_lse,
                                                 void* workspace, size_t workspace_bytes, msa_stream_t stream);

/* Warm-up mode, forward (Flash-MSA article, backward paragraph: a warm-up in
 * which the main attention runs densely, without block indexes, while the
 * proxy learns only in the backward pass): causal GQA attention of every
 * query row over all of its visible keys (j <= pos, j < kv_len),
 *   out[r][h] = sum_j softmax_j(sm_scale * <q[r][h], k[j][g]>) v[j][g],
 *   lse[r][h] = natural log of sum_j exp(sm_scale * <q[r][h], k[j][g]>).
 * Operands and layouts as in msa_sparse_attn_prefill without the selection;
 * bf16 K/V only.  Errors: INVALID_ARG for null or misaligned pointers;
 * UNSUPPORTED for a decode plan or non-bf16 K/V; WORKSPACE_TOO_SMALL. */
msa_status_t msa_dense_attn_prefill(msa_plan_t plan, const void* q, const void* k_pages, const void* v_pages,
                                    const int32_t* kv_indices, void* out, float* lse, void* workspace,
                                    size_t workspace_bytes, msa_stream_t stream);

/* Warm-up mode, backward: the gradients of msa_dense_attn_prefill (the
 * formulas of msa_sparse_attn_prefill_backward with every visible key), and,
 * when proxy_q and proxy_k_pages are given, the proxy distillation gradient
 * of msa_sparse_attn_prefill_backward_kl with p_main the group mean of this
 * dense attention (nonzero on every visible key).  With proxy_q and
 * proxy_k_pages NULL the proxy arguments are ignored and may be NULL.
 *   out, lse          msa_dense_attn_prefill's results for the same inputs
 *   dq                fp32 [T, H_q, 128], fully written
 *   dk_pages, dv_pages fp32 [num_pages, H_kv, 128, 128]: pages of sequences
 *                     written, other pages not touched
 *   proxy operands and outputs as in msa_sparse_attn_prefill_backward_kl
 * The plan's partial-output area holds D = <dout, out> of every row, so very
 * long batches need an attention window of at least T / (64 topk) rows.
 * Errors: INVALID_ARG for null or misaligned pointers or a non-finite
 * kl_grad_scale; UNSUPPORTED for a decode plan, non-bf16 K/V, a proxy term on
 * a plan without one bf16 proxy head and proxy-K head per KV group, or too
 * short an attention window; WORKSPACE_TOO_SMALL. */
msa_status_t msa_dense_attn_prefill_backward(msa_plan_t plan, const void* q, const void* k_pages,
                                             const void* v_pages, const int32_t* kv_indices, const void* out,
                                             const float* lse, const void* dout, const void* proxy_q,
                                             const void* proxy_k_pages, float kl_grad_scale, float* dq,
                                             float* dk_pages, float* dv_pages, float* dproxy_q,
                                             float* dproxy_k_pages, float* proxy_lse, void* workspace,
                                             size_t workspace_bytes, msa_stream_t stream);

/* Stage 3b: paged sparse decode (README "Stacks": paged FP8 decode).  Stage
 * 3a with qo_len = 1 for every sequence: the new token is already the last
 * key of its sequence (position kv_len - 1), so its local block is the last.
 *
 *   q                 bf16 [batch, H_q, 128]
 *   k_pages, v_pages  fp8 or bf16 (desc.kv_dtype) [num_pages, H_kv, 128, 128]
 *   k_scale, v_scale  fp32 [H_kv] device, NULL iff bf16
 *   kv_block_indexes  int32 [batch, H_kv, topk]
 *   out               bf16 [batch, H_q, 128];  lse fp32 [batch, H_q] or NULL
 * Errors: INVALID_ARG; UNSUPPORTED for a prefill plan; WORKSPACE_TOO_SMALL. */
msa_status_t msa_sparse_attn_decode(msa_plan_t plan, const void* q, const void* k_pages, const void* v_pages,
                                    const float* k_scale, const float* v_scale, const int32_t* kv_indices,
                                    const int32_t* kv_block_indexes, void* out, float* lse, void* workspace,
                                    size_t workspace_bytes, msa_stream_t stream);

/* Allocation-free form of msa_sparse_attn_decode, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same arguments and results, without
 * a workspace.  The plan metadata and split partials go to a static scratch
 * array of 16 MiB per device, part of the library's code object (each device
 * the library runs on holds its own copy until the process ends).  The call
 * allocates nothing.  Every call on one device shares that device's scratch:
 * calls that overlap in time on one device (different streams, or different
 * host threads without stream ordering) race.  Nothing in the scratch needs
 * to start at zero.  Errors: as msa_sparse_attn_decode, plus INVALID_ARG when
 * the plan's workspace size (msa_plan's workspace_bytes) exceeds 16 MiB. */
msa_status_t msa_sparse_attn_decode_noalloc(msa_plan_t plan, const void* q, const void* k_pages,
                                            const void* v_pages, const float* k_scale, const float* v_scale,
                                            const int32_t* kv_indices, const int32_t* kv_block_indexes, void* out,
                                            float* lse, msa_stream_t stream);

/* Message for the calling thread's last non-OK status ("" if none). */
const char* msa_last_error(void);

/* Plan introspection (host only): total rows T, max blocks per sequence
 * nb_max, and the row bound of one proxy / top-k call. */
msa_status_t msa_plan_info(msa_plan_t plan, int64_t* total_rows, int32_t* nb_max, int64_t* max_rows_per_call);

/* Diagnostics, not part of the path.  When `kernel` names one of the
 * library's internal kernels ("proxy_maxscore", "topk_select", "proxy_topk", "csr",
 * "partial_attn", "merge", "decode", "decode_merge", "bwd_dq", "bwd_dq_sum", "bwd_dkv",
 * "kl_dq_sum", "kl_dense_dq", "kl_dense_dk", "dense_fwd", "dense_dq", "dense_dkv"), each later launch of it
 * for this plan carries two HIP events that the runtime stamps with the
 * dispatch's begin and end (events are created on first use and reused; no
 * device memory).  NULL
 * switches it off.  msa_profile_read waits for the recorded events, returns
 * the summed kernel time in milliseconds and the number of launches, and
 * clears the record.  Errors: INVALID_ARG for an unknown name; HIP. */
msa_status_t msa_profile_kernel(msa_plan_t plan, const char* kernel);
msa_status_t msa_profile_read(msa_plan_t plan, double* total_ms, int64_t* launches);

/* Diagnostic, not part of the path: the matrix-core rate the current device
 * sustains.  dtype MSA_BF16 (v_mfma_f32_32x32x16_bf16), MSA_FP8_E4M3 or
 * MSA_MXFP4_QK (v_mfma_scale_f32_32x32x64_f8f6f4 on e4m3 or E2M1 operands,
 * unit block scales); every SIMD runs two waves of `iters`
 * rounds of four independent accumulations on register operands.  Runs on the
 * null stream and waits for it; *tflops receives dense TFLOP/s.  Errors:
 * INVALID_ARG (bad dtype, iters < 1, NULL), HIP. */
msa_status_t msa_diag_mfma_rate(int32_t dtype, int32_t iters, double* tflops);

#ifdef __cplusplus
}
#endif
#endif /* MSA_H_ */
