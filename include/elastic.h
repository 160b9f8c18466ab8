/*
 * elastic.h - C ABI of libelastic: Elastic Attention prefill on AMD Instinct MI355X (gfx950).
 *
 * Method: "Elastic Attention: Test-time Adaptive Sparsity Ratios for Efficient Transformers"
 * (arXiv 2601.17367), as summarised on paperlayer.ai (abs/2601.17367v2).  An Attention
 * Router reads a layer's hidden states and gives every key/value head a binary choice
 * between full attention and sparse attention (summary section 3, "Attention Router");
 * heads then run in one hybrid launch and their outputs are concatenated (section 2,
 * "Hybrid Head Mechanism"; appendix D.1, "Sparse Inference": routing metadata goes
 * straight to one unified kernel launch).
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers owned by the caller, unless a comment says
 *    "host".  The library never allocates, frees or synchronises; each call only enqueues
 *    work on `stream` (a hipStream_t; NULL = the null stream) and returns.
 *  - Layouts are dense, row-major and token-major: q and o are [T, Hq, D], k and v are
 *    [T, Hkv, D], hidden is [T, d_model].  Sequences of a batch are packed back to back;
 *    `cu_seqlens` (device, int32 [batch+1], cu_seqlens[0] = 0, non-decreasing,
 *    cu_seqlens[batch] = total_tokens) gives their offsets.  cu_seqlens == NULL is allowed
 *    only with batch == 1 and means one sequence of total_tokens tokens.
 *  - Positions are local to a sequence; no token attends across sequences.
 *  - Query head h reads key/value head h / G with G = Hq / Hkv (grouped-query attention)
 *    and takes that head's full/sparse mode: the router decides per key/value head.
 *  - Arguments are validated on the host before any HIP call; a failure returns
 *    ELASTIC_EINVAL / ELASTIC_EUNSUPPORTED / ELASTIC_EWORKSPACE and enqueues nothing.
 *    Device-resident values (cu_seqlens, head masks) are never read on the host, so the
 *    caller must pass consistent ones; a launch error returns ELASTIC_EHIP and
 *    elastic_last_error() gives the HIP message (thread-local).
 *  - Concurrent calls are safe when each uses its own workspace; calls that share a
 *    workspace must be ordered on one stream.
 *  - Tensors the kernels read or write row by row (q, k, v, o, hidden, and the o arrays of
 *    elastic_lse_merge) must start on a 16-byte boundary: rows move with 16-byte loads,
 *    stores and LDS copies.  A misaligned pointer returns ELASTIC_EINVAL.
 */
#ifndef ELASTIC_H_
#define ELASTIC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ELASTIC_ABI_VERSION 4

enum elastic_status {
  ELASTIC_OK = 0,
  ELASTIC_EINVAL = 1,       /* null required pointer, non-positive size, inconsistent shapes */
  ELASTIC_EUNSUPPORTED = 2, /* valid but not implemented: head_dim, dtype, pattern geometry */
  ELASTIC_EWORKSPACE = 3,   /* workspace_bytes below the matching *_workspace_size() */
  ELASTIC_EHIP = 4          /* a HIP launch or runtime call failed */
};

enum elastic_dtype { ELASTIC_BF16 = 0, ELASTIC_FP32 = 1 };

enum elastic_sparse_kind {
  /* Streaming sparse attention (summary section 4 and appendix B.2; appendix D.1 gives
   * 128 sink tokens): query i sees key j <= i iff j < sink_tokens or i - j < window_tokens
   * (the window counts the query itself), so it sees min(i + 1, sink + window) keys. */
  ELASTIC_SPARSE_STREAMING = 0,
  /* Fixed block-sparse pattern (appendix D.1, "unified block-sparse kernel"): with
   * qb = i / block_size and kb = j / block_size, query i sees key j <= i iff
   * kb < sink_blocks, or qb - kb <= local_blocks, or (stride_blocks > 0 and
   * kb % stride_blocks == 0).  Blocks strictly below the diagonal are fully visible; the
   * diagonal block is causal inside. */
  ELASTIC_SPARSE_BLOCK = 1,
  /* Explicit block lists per sequence and key/value head, the consumer side of a
   * content-based block selection (summary section 4 and appendix G.2 name XAttention's
   * block selection).  For sequence b, KV head g and query block qb = i / block_size, CSR
   * row r = (b * n_kv_heads + g) * list_qblocks + qb lists the key blocks
   * list_col_idx[list_row_ptr[r] .. list_row_ptr[r+1]); query i sees key j <= i iff
   * j / block_size is listed.  Listed blocks after qb are ignored; a query block with an
   * empty list leaves its rows without keys (o = 0, lse = -inf). */
  ELASTIC_SPARSE_BLOCK_LIST = 2
};

/* Pattern of the sparse heads.  The struct is read on the host during the call; the block
 * lists it points at are read by the kernels on the device. */
typedef struct elastic_sparse_cfg {
  int32_t kind;          /* enum elastic_sparse_kind */
  int32_t sink_tokens;   /* streaming: >= 0 */
  int32_t window_tokens; /* streaming: >= 1 */
  int32_t block_size;    /* block, block list: 64 or 128 */
  int32_t sink_blocks;   /* block: >= 0 */
  int32_t local_blocks;  /* block: >= 0 (blocks strictly before the diagonal block) */
  int32_t stride_blocks; /* block: >= 0, 0 = no strided blocks */
  int32_t list_qblocks;  /* block list: CSR rows per (sequence, KV head), >= query blocks */
  const int32_t* list_row_ptr; /* block list: device int32 [batch * n_kv_heads * list_qblocks + 1],
                                  non-decreasing, list_row_ptr[0] = 0 */
  const int32_t* list_col_idx; /* block list: device int32 key-block indices, each row ascending
                                  without repeats */
} elastic_sparse_cfg;

/* ABI version compiled into the library (ELASTIC_ABI_VERSION). */
int elastic_abi_version(void);

/* Static text for a status code. */
const char* elastic_status_string(int status);

/* Text of the last ELASTIC_EHIP error on the calling thread ("" if none), or of the last
 * ELASTIC_EWORKSPACE from elastic_attn_prefill_noalloc. */
const char* elastic_last_error(void);

/* Bytes of workspace elastic_route needs for these sizes (device memory, any alignment
 * of at least 256 bytes; contents need not be initialised). */
size_t elastic_route_workspace_size(int32_t batch, int64_t total_tokens, int32_t d_model);

/*
 * Attention Router forward (summary section 1: the router reads the input hidden states
 * and routes per head; section 3 "Attention Router": pooled hidden states, a task MLP and
 * a router MLP give head-wise logits that pick full or sparse attention; appendix H.4
 * "Router Input Length": boundary pooling of the first and last tokens).
 *
 * For every sequence b:  h = mean of hidden rows of b (all rows when pool_head ==
 * pool_tail == 0; otherwise the first pool_head and last pool_tail rows, each row at most
 * once), z = W1 h, a = max(z, 0), logit = W2 a, mask = (logit > threshold).
 *
 *  hidden      [total_tokens, d_model], dtype hidden_dtype (ELASTIC_BF16 or ELASTIC_FP32)
 *  w1          [d_router, d_model] fp32 row-major;   d_router in [1, 256]
 *  w2          [n_kv_heads, d_router] fp32 row-major; n_kv_heads in [1, 256]
 *  logits_out  [batch, n_kv_heads] fp32, may be NULL
 *  mask_out    [batch, n_kv_heads] int32, 1 = full attention, 0 = sparse (required)
 *  d_model     multiple of 8.  Sums are fp32 in a fixed order: results are bitwise
 *              reproducible run to run.  A sequence of length 0 pools nothing: its
 *              logits are 0, so its mask is (0 > threshold): all sparse for threshold >= 0.
 * The workspace holds intermediate sums and per-sequence completion counts that the call
 * itself clears; two calls in flight at once need two workspaces.
 */
int elastic_route(const void* hidden, int32_t hidden_dtype, const int32_t* cu_seqlens,
                  int32_t batch, int64_t total_tokens, int32_t d_model, int32_t pool_head,
                  int32_t pool_tail, const float* w1, int32_t d_router, const float* w2,
                  int32_t n_kv_heads, float threshold, float* logits_out, int32_t* mask_out,
                  void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace elastic_attn_prefill needs (device memory, 256-byte aligned). */
size_t elastic_attn_workspace_size(int32_t dtype, int32_t batch, int64_t total_tokens,
                                   int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim);

/*
 * Hybrid-head GQA prefill attention in one scheduled launch (summary section 2 "Hybrid
 * Head Mechanism"; section 3 "Efficient Deployment": one fused kernel computes retrieval
 * (full) and sparse heads on a single GPU; appendix D.1: routing metadata is passed
 * directly to one launch without splitting tensors).
 *
 * For query head h of sequence b with key/value head g = h / G:
 *   mode = head_mask[b * n_kv_heads + g] != 0 ? full causal : the `sparse` pattern,
 *   o[i, h, :] = sum_{j in A(i)} softmax_j(scale * <q_i, k_j>) v_j,
 *   lse[h, i]  = log sum_{j in A(i)} exp(scale * <q_i, k_j>)      (natural log)
 *
 *  q, o        [total_tokens, n_q_heads, head_dim]   dtype (bf16 or fp32; o same dtype)
 *  k, v        [total_tokens, n_kv_heads, head_dim]
 *  head_mask   [batch, n_kv_heads] int32 (router output or a forced mask); NULL = all full
 *  sparse      host pointer, pattern of the sparse heads (required unless head_mask NULL)
 *  lse_out     [n_q_heads, total_tokens] fp32, may be NULL
 *  softmax_scale <= 0 selects head_dim^-1/2.
 *  max_seqlen  >= every sequence length (used for sizing only).
 * Supported: head_dim 64 or 128; bf16 (bf16 MFMA, fp32 accumulation and softmax) or fp32
 * (fp32 throughout); n_q_heads % n_kv_heads == 0.
 */
int elastic_attn_prefill(const void* q, const void* k, const void* v, void* o, int32_t dtype,
                         const int32_t* cu_seqlens, int32_t batch, int64_t total_tokens,
                         int32_t max_seqlen, int32_t n_q_heads, int32_t n_kv_heads,
                         int32_t head_dim, float softmax_scale, const int32_t* head_mask,
                         const elastic_sparse_cfg* sparse, float* lse_out, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * Prefill of query rows against a separate range of key rows: chunked prefill and key-range
 * splits (summary appendix D.1 "Sparse Inference": prefill runs in chunks of 16,384 queries;
 * the partial results of split key ranges combine with elastic_lse_merge).
 *
 * Sequence b owns query rows [cu_seqlens_q[b], cu_seqlens_q[b+1]) of q/o/lse and key rows
 * [cu_seqlens_k[b], cu_seqlens_k[b+1]) of k/v.  Positions are absolute within the sequence:
 * query row t sits at q_pos + t and key row j at k_pos + j; every pattern (causal, sink,
 * window, blocks) is evaluated on these positions and restricted to the keys present.
 *   q_pos   >= 0: position of every sequence's first query row;
 *           -1: bottom-right alignment, the queries are the sequence's last key positions
 *           (q_pos = k_pos + n_k - n_q per sequence): one prefill chunk over its whole prefix.
 *   k_pos   >= 0, a multiple of 64 (and of block_size for the block pattern).
 * A query row that sees no key gets o = 0 and lse = -inf.
 *
 *  q, o        [total_q, n_q_heads, head_dim];  k, v [total_k, n_kv_heads, head_dim]
 *  lse_out     [n_q_heads, total_q] fp32, may be NULL
 *  cu_seqlens_q / cu_seqlens_k  int32 [batch + 1] device arrays; both NULL only when batch == 1
 *  max_seqlen_q, max_seqlen_k   >= every sequence's query / key rows (sizing and checks)
 *  workspace   elastic_attn_workspace_size(dtype, batch, total_q, n_q_heads, n_kv_heads,
 *              head_dim) bytes.
 * Other arguments, supported shapes and errors as for elastic_attn_prefill;
 * ELASTIC_EINVAL also for a misaligned k_pos, q_pos < -1, positions past 2^31 - 1, or block
 * lists with fewer than (last query position / block_size + 1) rows per (sequence, head);
 * ELASTIC_EUNSUPPORTED for block lists over more than 4095 key blocks.
 * elastic_attn_prefill is this call with q = k rows, q_pos = k_pos = 0.
 */
int elastic_attn_prefill_kv(const void* q, const void* k, const void* v, void* o, int32_t dtype,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                            int32_t batch, int64_t total_q, int64_t total_k,
                            int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t q_pos,
                            int32_t k_pos, int32_t n_q_heads, int32_t n_kv_heads,
                            int32_t head_dim, float softmax_scale, const int32_t* head_mask,
                            const elastic_sparse_cfg* sparse, float* lse_out, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): elastic_attn_prefill without a workspace argument.
 * The scheduler's queue header and work list go to a scratch array that the library holds in
 * device memory, ELASTIC_NOALLOC_SCRATCH_BYTES on every GPU it runs on, until the process ends;
 * the call itself allocates nothing.  Every call on a GPU shares that GPU's array, so calls
 * that overlap on one GPU (other streams, other threads) race: the caller must serialise them.
 * A problem whose workspace (elastic_attn_workspace_size) exceeds the array returns
 * ELASTIC_EWORKSPACE before any HIP call, with both sizes in elastic_last_error().  8 MiB holds
 * about 419,000 work items: one bf16 sequence of up to 3.35M tokens with 32 query / 8 KV heads
 * (1.67M with 64 / 8).  Arguments, results and other errors as for elastic_attn_prefill.
 */
#define ELASTIC_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
int elastic_attn_prefill_noalloc(const void* q, const void* k, const void* v, void* o,
                                 int32_t dtype, const int32_t* cu_seqlens, int32_t batch,
                                 int64_t total_tokens, int32_t max_seqlen, int32_t n_q_heads,
                                 int32_t n_kv_heads, int32_t head_dim, float softmax_scale,
                                 const int32_t* head_mask, const elastic_sparse_cfg* sparse,
                                 float* lse_out, void* stream);

/*
 * Combines two attention results of the same query rows over disjoint key sets (for example
 * the two halves of a split key range, or a sequence shard's partial and its halo part):
 *   lse = log(exp(lse_a) + exp(lse_b)),  o = exp(lse_a - lse) o_a + exp(lse_b - lse) o_b,
 * per (row, head); a row with lse_a = lse_b = -inf stays o = 0, lse = -inf.
 *
 *  o_a, o_b, o_out        [rows, n_heads, head_dim], dtype (bf16 or fp32)
 *  lse_a, lse_b, lse_out  [n_heads, rows] fp32 natural log (the layout elastic_attn_* write)
 * o_out / lse_out may alias o_a or o_b / lse_a or lse_b (in-place merge).  All pointers are
 * device pointers and required; head_dim 64 or 128.  Enqueues one elementwise kernel.
 */
int elastic_lse_merge(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
                      void* o_out, float* lse_out, int32_t dtype, int64_t rows, int32_t n_heads,
                      int32_t head_dim, void* stream);

/*
 * Retrieval scores of the pages' static head assignment (summary appendix C.1 "Retrieval
 * Score Calculation"): for sequence b and query head h, the attention weight that the last
 * token of b puts on the needle span [needle[2b], needle[2b+1]) (local key positions, clipped
 * to the sequence), softmax over all keys of b with scale softmax_scale (<= 0: head_dim^-1/2):
 *   scores_q[b, h]  = sum_{j in needle} exp(s_j) / sum_j exp(s_j),  s_j = scale <q_last, k_j>
 *   scores_kv[b, g] = mean of scores_q[b, h] over the G query heads of KV head g.
 * An empty sequence scores 0.  q [total_tokens, n_q_heads, head_dim] (only each sequence's
 * last row is read), k [total_tokens, n_kv_heads, head_dim]; cu_seqlens as for
 * elastic_attn_prefill; needle int32 [batch, 2] device; scores_q fp32 [batch, n_q_heads] and
 * scores_kv fp32 [batch, n_kv_heads] device, either may be NULL (not both).  q and k 16-byte
 * aligned.  fp32 accumulation; reads every key once (HBM-bound).
 * Errors: ELASTIC_EINVAL (pointers, shapes, alignment), ELASTIC_EUNSUPPORTED (dtype,
 * head_dim, more than 65535 sequences or 1024 query heads per KV head), ELASTIC_EWORKSPACE.
 */
size_t elastic_retrieval_workspace_size(int32_t batch, int32_t max_seqlen, int32_t n_q_heads);
int elastic_retrieval_scores(const void* q, const void* k, int32_t dtype,
                             const int32_t* cu_seqlens, int32_t batch, int64_t total_tokens,
                             int32_t max_seqlen, int32_t n_q_heads, int32_t n_kv_heads,
                             int32_t head_dim, float softmax_scale, const int32_t* needle,
                             float* scores_q, float* scores_kv, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * Static head assignment (summary appendix C.1 "Sparsity Assignment"): of the n_units
 * scores (device fp32, e.g. [layers, n_kv_heads] flattened), the
 *   k = floor((1 - omega_msr) * n_units)       (evaluated in double)
 * highest stay full: mask_out[i] = 1, the rest 0 (device int32 [n_units]).  Equal scores rank
 * by lower index; NaN ranks below every number.  A layer's slice of mask_out is a forced head
 * mask for elastic_attn_prefill.  One kernel, O(n_units^2) comparisons spread over up to 4096
 * waves.
 * Errors: ELASTIC_EINVAL (pointers, omega_msr outside [0, 1]), ELASTIC_EUNSUPPORTED
 * (n_units > ELASTIC_ASSIGN_MAX_UNITS).
 */
#define ELASTIC_ASSIGN_MAX_UNITS 16384
int elastic_static_assignment(const float* scores, int32_t n_units, double omega_msr,
                              int32_t* mask_out, void* stream);

/*
 * Host-only work counter (no HIP call): the number of allowed (query, key) score entries
 * over all query heads, for sequences of the given lengths (host int32 [batch]) and head
 * modes (host int32 [batch, n_kv_heads], NULL = all full).  Effective attention FLOPs are
 * 4 * head_dim * entries.  Closed forms: full n(n+1)/2 per head; streaming
 * c(c+1)/2 + (n-c)c with c = min(n, sink+window); block: per query block, the visible
 * earlier blocks times block_size plus the causal diagonal block.  Block lists live on the
 * device: a call with block-list sparse heads returns ELASTIC_EUNSUPPORTED (count those with
 * elastic_attn_entries_lists from a host copy of the lists).
 */
int elastic_attn_entries(const int32_t* seqlens_host, int32_t batch,
                         const int32_t* head_mask_host, int32_t n_q_heads, int32_t n_kv_heads,
                         const elastic_sparse_cfg* sparse, int64_t* entries_out);

/*
 * Host-only work counter for sparse heads given by explicit block lists (the
 * ELASTIC_SPARSE_BLOCK_LIST pattern, read from HOST copies of its CSR arrays): allowed score
 * entries over all query heads.  Full heads count n(n+1)/2 each; for a sparse head, query
 * block qb counts its listed earlier key blocks whole (block_size keys per query row) and its
 * own block causally if listed.  Listed blocks after qb, repeated and negative indices count
 * nothing, as in the kernels.
 *  seqlens_host       int32 [batch], host
 *  head_mask_host     int32 [batch, n_kv_heads], host, NULL = all full
 *  list_row_ptr_host  int32 [batch * n_kv_heads * list_qblocks + 1], host, non-decreasing from 0
 *  list_col_idx_host  int32 [list_row_ptr_host[last]], host (may be NULL when that is 0)
 * Errors: ELASTIC_EINVAL (pointers, sizes, a sequence with more query blocks than
 * list_qblocks, a decreasing row_ptr), ELASTIC_EUNSUPPORTED (block_size not 64 or 128).
 */
int elastic_attn_entries_lists(const int32_t* seqlens_host, int32_t batch,
                               const int32_t* head_mask_host, int32_t n_q_heads,
                               int32_t n_kv_heads, int32_t block_size, int32_t list_qblocks,
                               const int32_t* list_row_ptr_host, const int32_t* list_col_idx_host,
                               int64_t* entries_out);

#ifdef __cplusplus
}
#endif

#endif /* ELASTIC_H_ */
