// C ABI of libelastic: argument validation, workspace layout and launch sequencing.
// Every entry point validates on the host before touching HIP and never reads device memory,
// so a call only enqueues work on the caller's stream.
#include <stdio.h>
#include <string.h>

#include <math.h>
#include <mutex>
#include <vector>

#include "elastic_internal.hpp"

using namespace elastic;

// ---------------------------------------------------------------- persistent grids
hipError_t elastic::resident_grid(const void* kernel, int threads, int64_t* grid) {
  struct Entry {
    int dev;
    const void* kernel;
    int64_t grid;
  };
  static std::mutex mu;
  static Entry cache[64];
  static int cached = 0;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  {
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < cached; ++i)
      if (cache[i].dev == dev && cache[i].kernel == kernel) {
        *grid = cache[i].grid;
        return hipSuccess;
      }
  }
  int cus = 0, per_cu = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0);
  if (e != hipSuccess) return e;
  *grid = (int64_t)(cus > 0 ? cus : 1) * (per_cu > 0 ? per_cu : 1);
  std::lock_guard<std::mutex> lock(mu);
  if (cached < 64) cache[cached++] = Entry{dev, kernel, *grid};
  return hipSuccess;
}

namespace {

thread_local char g_last_error[512] = "";

int hip_fail(hipError_t e, const char* where) {
  snprintf(g_last_error, sizeof(g_last_error), "%s: %s", where, hipGetErrorString(e));
  return ELASTIC_EHIP;
}

constexpr size_t ALIGN = 256;
inline size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

// The kernels move tensor rows with 16-byte loads, stores and LDS copies.
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// ---------------------------------------------------------------- attention sizing
int attn_rows_per_item(int32_t dtype) { return dtype == ELASTIC_BF16 ? BF16_ROWS : F32_ROWS; }
int attn_key_tile(int32_t dtype) { return dtype == ELASTIC_BF16 ? BF16_BK : F32_BK; }

int64_t attn_max_items(int32_t dtype, int32_t batch, int64_t total_tokens, int32_t n_q_heads,
                       int32_t n_kv_heads) {
  const int G = n_q_heads / n_kv_heads;
  const int BT = tokens_per_item(attn_rows_per_item(dtype), G);
  return ((total_tokens + BT - 1) / BT + batch) * (int64_t)n_kv_heads;
}

struct AttnWorkspace {
  size_t sched, items, tile_prefix, cost_tmp, total;
};

AttnWorkspace attn_layout(int64_t max_items, int32_t batch) {
  AttnWorkspace w;
  w.sched = 0;
  w.items = align_up(SCHED_INTS * sizeof(int32_t));
  w.tile_prefix = align_up(w.items + (size_t)max_items * sizeof(WorkItem));
  w.cost_tmp = align_up(w.tile_prefix + (size_t)(batch + 1) * sizeof(int32_t));
  w.total = align_up(w.cost_tmp + (size_t)max_items * sizeof(int32_t));
  return w;
}

// ---------------------------------------------------------------- router sizing
struct RouteWorkspace {
  int64_t max_slabs;
  size_t partials, zpart, done, total;
};

RouteWorkspace route_layout(int32_t batch, int64_t total_tokens, int32_t d_model) {
  RouteWorkspace w;
  w.max_slabs = (total_tokens + ROUTE_SLAB - 1) / ROUTE_SLAB + batch;
  const size_t strips = (size_t)(d_model + ROUTE_HCOLS - 1) / ROUTE_HCOLS;
  w.partials = 0;
  w.zpart = align_up((size_t)w.max_slabs * d_model * sizeof(float));
  w.done = align_up(w.zpart + (size_t)batch * strips * ROUTE_MAX_DR * sizeof(float));
  w.total = align_up(w.done + (size_t)batch * sizeof(int32_t));
  return w;
}

int check_pattern(const elastic_sparse_cfg* s) {
  if (s->kind == ELASTIC_SPARSE_STREAMING) {
    if (s->sink_tokens < 0 || s->window_tokens < 1) return ELASTIC_EINVAL;
    return ELASTIC_OK;
  }
  if (s->kind == ELASTIC_SPARSE_BLOCK) {
    if (s->sink_blocks < 0 || s->local_blocks < 0 || s->stride_blocks < 0) return ELASTIC_EINVAL;
    if (s->block_size != 64 && s->block_size != 128) return ELASTIC_EUNSUPPORTED;
    return ELASTIC_OK;
  }
  if (s->kind == ELASTIC_SPARSE_BLOCK_LIST) {
    if (s->list_qblocks < 1 || s->list_row_ptr == nullptr || s->list_col_idx == nullptr)
      return ELASTIC_EINVAL;
    if (s->block_size != 64 && s->block_size != 128) return ELASTIC_EUNSUPPORTED;
    return ELASTIC_OK;
  }
  return ELASTIC_EINVAL;
}

// Block lists: the CSR must hold a row for every query block the call reaches, and one item's
// key blocks must fit the kernels' LDS visibility words.
int check_lists(const elastic_sparse_cfg* s, int64_t max_q_pos, int64_t max_k) {
  if (s == nullptr || s->kind != ELASTIC_SPARSE_BLOCK_LIST) return ELASTIC_OK;
  if (max_q_pos >= 0 && max_q_pos / s->block_size >= s->list_qblocks) return ELASTIC_EINVAL;
  if ((max_k + s->block_size - 1) / s->block_size + 1 > LIST_MAX_KB) return ELASTIC_EUNSUPPORTED;
  return ELASTIC_OK;
}

Pattern to_pattern(const elastic_sparse_cfg* s) {
  Pattern p{};
  if (s == nullptr) {
    p.kind = ELASTIC_SPARSE_STREAMING;
    p.window = 1;
    p.block = 64;
    return p;
  }
  p.kind = s->kind;
  p.sink = s->sink_tokens;
  p.window = s->window_tokens;
  p.block = s->block_size > 0 ? s->block_size : 64;
  p.sink_blocks = s->sink_blocks;
  p.local_blocks = s->local_blocks;
  p.stride_blocks = s->stride_blocks;
  p.qblocks = s->kind == ELASTIC_SPARSE_BLOCK_LIST ? s->list_qblocks : 0;
  p.row_ptr = s->kind == ELASTIC_SPARSE_BLOCK_LIST ? s->list_row_ptr : nullptr;
  p.col_idx = s->kind == ELASTIC_SPARSE_BLOCK_LIST ? s->list_col_idx : nullptr;
  return p;
}

// Allowed entries of one query head over a sequence of length n.
int64_t head_entries(int64_t n, bool full, const elastic_sparse_cfg* s) {
  if (n <= 0) return 0;
  if (full) return n * (n + 1) / 2;
  if (s->kind == ELASTIC_SPARSE_STREAMING) {
    int64_t c = (int64_t)s->sink_tokens + s->window_tokens;
    if (c > n) c = n;
    return c * (c + 1) / 2 + (n - c) * c;
  }
  const int64_t B = s->block_size, stride = s->stride_blocks;
  const int64_t nb = (n + B - 1) / B;
  int64_t total = 0;
  for (int64_t qb = 0; qb < nb; ++qb) {
    // visible blocks strictly before qb: [0, a) U [bstart, qb) U {multiples of stride}
    const int64_t a = s->sink_blocks < qb ? s->sink_blocks : qb;
    int64_t bstart = qb - s->local_blocks;
    if (bstart < 0) bstart = 0;
    int64_t e;
    if (a >= bstart) {
      e = qb;
    } else {
      e = a + (qb - bstart);
      if (stride > 0) e += (bstart + stride - 1) / stride - (a + stride - 1) / stride;
    }
    const int64_t r0 = qb * B;
    const int64_t nr = (r0 + B < n ? r0 + B : n) - r0;
    total += nr * e * B + nr * (nr + 1) / 2;
  }
  return total;
}

}  // namespace

extern "C" {

int elastic_abi_version(void) { return ELASTIC_ABI_VERSION; }

const char* elastic_status_string(int status) {
  switch (status) {
    case ELASTIC_OK: return "ok";
    case ELASTIC_EINVAL: return "invalid argument";
    case ELASTIC_EUNSUPPORTED: return "unsupported configuration";
    case ELASTIC_EWORKSPACE: return "workspace too small";
    case ELASTIC_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* elastic_last_error(void) { return g_last_error; }

size_t elastic_route_workspace_size(int32_t batch, int64_t total_tokens, int32_t d_model) {
  if (batch < 1 || total_tokens < 0 || d_model < 1) return 0;
  return route_layout(batch, total_tokens, d_model).total;
}

int elastic_route(const void* hidden, int32_t hidden_dtype, const int32_t* cu_seqlens,
                  int32_t batch, int64_t total_tokens, int32_t d_model, int32_t pool_head,
                  int32_t pool_tail, const float* w1, int32_t d_router, const float* w2,
                  int32_t n_kv_heads, float threshold, float* logits_out, int32_t* mask_out,
                  void* workspace, size_t workspace_bytes, void* stream) {
  if (w1 == nullptr || w2 == nullptr || mask_out == nullptr) return ELASTIC_EINVAL;
  if (hidden == nullptr && total_tokens > 0) return ELASTIC_EINVAL;
  if (batch < 1 || total_tokens < 0 || total_tokens > INT32_MAX) return ELASTIC_EINVAL;
  if (cu_seqlens == nullptr && batch != 1) return ELASTIC_EINVAL;
  if (pool_head < 0 || pool_tail < 0) return ELASTIC_EINVAL;
  if (d_model < 1 || d_router < 1 || n_kv_heads < 1) return ELASTIC_EINVAL;
  if (hidden_dtype != ELASTIC_BF16 && hidden_dtype != ELASTIC_FP32) return ELASTIC_EUNSUPPORTED;
  if (d_model % 8 != 0 || d_router > ROUTE_MAX_DR || n_kv_heads > ROUTE_MAX_HKV)
    return ELASTIC_EUNSUPPORTED;
  if (total_tokens > 0 && !aligned16(hidden)) return ELASTIC_EINVAL;
  const RouteWorkspace lay = route_layout(batch, total_tokens, d_model);
  if (workspace == nullptr || workspace_bytes < lay.total) return ELASTIC_EWORKSPACE;
  char* ws = static_cast<char*>(workspace);
  const hipError_t e = launch_route(
      hidden, hidden_dtype, cu_seqlens, batch, total_tokens, d_model, pool_head, pool_tail, w1,
      d_router, w2, n_kv_heads, threshold, logits_out, mask_out,
      reinterpret_cast<float*>(ws + lay.partials), total_tokens > 0 ? lay.max_slabs : 0,
      reinterpret_cast<float*>(ws + lay.zpart), reinterpret_cast<int32_t*>(ws + lay.done),
      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ELASTIC_OK : hip_fail(e, "elastic_route");
}

size_t elastic_attn_workspace_size(int32_t dtype, int32_t batch, int64_t total_tokens,
                                   int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim) {
  (void)head_dim;
  if ((dtype != ELASTIC_BF16 && dtype != ELASTIC_FP32) || batch < 1 || total_tokens < 0 ||
      n_q_heads < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads != 0 ||
      n_q_heads / n_kv_heads > attn_rows_per_item(dtype))
    return 0;
  return attn_layout(attn_max_items(dtype, batch, total_tokens, n_q_heads, n_kv_heads), batch).total;
}

}  // extern "C"

namespace {

// Shared body of the two attention entry points: validation, then scheduler + attention.
int attn_call(const char* who, const void* q, const void* k, const void* v, void* o, int32_t dtype,
              const int32_t* cu_q, const int32_t* cu_k, int32_t batch, int64_t total_q,
              int64_t total_k, int32_t max_q, int32_t max_k, int32_t q_pos, int32_t k_pos,
              int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, float softmax_scale,
              const int32_t* head_mask, const elastic_sparse_cfg* sparse, float* lse_out,
              void* workspace, size_t workspace_bytes, void* stream, bool validate_only = false) {
  if (batch < 1 || total_q < 0 || total_q > INT32_MAX || total_k < 0 || total_k > INT32_MAX ||
      max_q < 0 || max_k < 0)
    return ELASTIC_EINVAL;
  if (total_q > 0 && (q == nullptr || o == nullptr)) return ELASTIC_EINVAL;
  if (total_k > 0 && (k == nullptr || v == nullptr)) return ELASTIC_EINVAL;
  if (total_q > 0 && !(aligned16(q) && aligned16(o))) return ELASTIC_EINVAL;
  if (total_k > 0 && !(aligned16(k) && aligned16(v))) return ELASTIC_EINVAL;
  if ((cu_q == nullptr || cu_k == nullptr) && batch != 1) return ELASTIC_EINVAL;
  if (q_pos < -1 || k_pos < 0 || k_pos % 64 != 0) return ELASTIC_EINVAL;
  // absolute positions stay within int32: keys up to k_pos + max_k, queries up to q_pos + max_q
  if ((int64_t)k_pos + max_k > INT32_MAX || (q_pos >= 0 && (int64_t)q_pos + max_q > INT32_MAX))
    return ELASTIC_EINVAL;
  if (n_q_heads < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads != 0) return ELASTIC_EINVAL;
  if (head_mask != nullptr && sparse == nullptr) return ELASTIC_EINVAL;
  if (sparse != nullptr) {
    const int st = check_pattern(sparse);
    if (st != ELASTIC_OK) return st;
    if (sparse->kind != ELASTIC_SPARSE_STREAMING && k_pos % sparse->block_size != 0) return ELASTIC_EINVAL;
    // last query position any sequence can reach: q_pos + max_q - 1, or k_pos + max_k - 1
    const int64_t max_q_pos = q_pos >= 0 ? (int64_t)q_pos + max_q - 1 : (int64_t)k_pos + max_k - 1;
    const int lst = check_lists(sparse, max_q_pos, max_k);
    if (lst != ELASTIC_OK) return lst;
  }
  if (dtype != ELASTIC_BF16 && dtype != ELASTIC_FP32) return ELASTIC_EUNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return ELASTIC_EUNSUPPORTED;
  if (n_q_heads / n_kv_heads > attn_rows_per_item(dtype)) return ELASTIC_EUNSUPPORTED;
  const int64_t max_items = attn_max_items(dtype, batch, total_q, n_q_heads, n_kv_heads);
  if (max_items > INT32_MAX) return ELASTIC_EUNSUPPORTED;
  const AttnWorkspace lay = attn_layout(max_items, batch);
  if (workspace == nullptr || workspace_bytes < lay.total) return ELASTIC_EWORKSPACE;
  if (total_q == 0 || validate_only) return ELASTIC_OK;

  const int G = n_q_heads / n_kv_heads;
  const int BT = tokens_per_item(attn_rows_per_item(dtype), G);
  const int BK = attn_key_tile(dtype);
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)head_dim);
  const Pattern pat = to_pattern(sparse);
  const SeqGeom geo{cu_q, cu_k, total_q, total_k, q_pos, k_pos};
  char* ws = static_cast<char*>(workspace);
  int32_t* sched = reinterpret_cast<int32_t*>(ws + lay.sched);
  WorkItem* items = reinterpret_cast<WorkItem*>(ws + lay.items);
  int32_t* tile_prefix = reinterpret_cast<int32_t*>(ws + lay.tile_prefix);
  int32_t* cost_tmp = reinterpret_cast<int32_t*>(ws + lay.cost_tmp);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  char where[96];

  hipError_t e = launch_plan(geo, batch, n_kv_heads, head_mask, pat, BT, BK, max_items,
                             tile_prefix, cost_tmp, items, sched, st);
  if (e != hipSuccess) {
    snprintf(where, sizeof(where), "%s: plan", who);
    return hip_fail(e, where);
  }
  if (dtype == ELASTIC_BF16)
    e = launch_attn_bf16(head_dim, q, k, v, o, lse_out, geo, n_q_heads, n_kv_heads, BT, scale,
                         head_mask, pat, items, sched, max_items, st);
  else
    e = launch_attn_f32(head_dim, q, k, v, o, lse_out, geo, n_q_heads, n_kv_heads, BT, scale,
                        pat, items, sched, max_items, st);
  if (e != hipSuccess) {
    snprintf(where, sizeof(where), "%s: attention", who);
    return hip_fail(e, where);
  }
  return ELASTIC_OK;
}

}  // namespace

extern "C" {

int elastic_attn_prefill(const void* q, const void* k, const void* v, void* o, int32_t dtype,
                         const int32_t* cu_seqlens, int32_t batch, int64_t total_tokens,
                         int32_t max_seqlen, int32_t n_q_heads, int32_t n_kv_heads,
                         int32_t head_dim, float softmax_scale, const int32_t* head_mask,
                         const elastic_sparse_cfg* sparse, float* lse_out, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return attn_call("elastic_attn_prefill", q, k, v, o, dtype, cu_seqlens, cu_seqlens, batch,
                   total_tokens, total_tokens, max_seqlen, max_seqlen, 0, 0, n_q_heads, n_kv_heads,
                   head_dim, softmax_scale, head_mask, sparse, lse_out, workspace, workspace_bytes,
                   stream);
}

int elastic_attn_prefill_kv(const void* q, const void* k, const void* v, void* o, int32_t dtype,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                            int32_t batch, int64_t total_q, int64_t total_k,
                            int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t q_pos,
                            int32_t k_pos, int32_t n_q_heads, int32_t n_kv_heads,
                            int32_t head_dim, float softmax_scale, const int32_t* head_mask,
                            const elastic_sparse_cfg* sparse, float* lse_out, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return attn_call("elastic_attn_prefill_kv", q, k, v, o, dtype, cu_seqlens_q, cu_seqlens_k,
                   batch, total_q, total_k, max_seqlen_q, max_seqlen_k, q_pos, k_pos, n_q_heads,
                   n_kv_heads, head_dim, softmax_scale, head_mask, sparse, lse_out, workspace,
                   workspace_bytes, stream);
}

// ---------------------------------------------------------------- allocation-free variant
// The scheduler's header, work list, tile prefix and cost table of elastic_attn_prefill_noalloc
// live in this array (one copy per GPU, held until the process ends) instead of a caller
// workspace.  Nothing in it has to start at zero: the scheduler kernel writes the queue header
// (and zeroes the claim counters) and every item before the attention kernel reads them, so
// the contents a previous call left are never read.  Calls that overlap on one GPU share the
// array and race.
}  // extern "C"

namespace {

static __device__ __align__(256) unsigned char scratch[ELASTIC_NOALLOC_SCRATCH_BYTES];

// Device address of `scratch` on the current device, looked up once per device with that
// device current.  In host code the array's name is only a stand-in, never a device address.
int noalloc_scratch(void** out) {
  constexpr int MAX_DEVICES = 64;
  static std::mutex mu;
  static void* addr[MAX_DEVICES] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "elastic_attn_prefill_noalloc: hipGetDevice");
  if (dev < 0 || dev >= MAX_DEVICES) return ELASTIC_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "elastic_attn_prefill_noalloc: hipGetSymbolAddress");
    if (p == nullptr) return hip_fail(hipErrorInvalidSymbol, "elastic_attn_prefill_noalloc: scratch");
    addr[dev] = p;
  }
  *out = addr[dev];
  return ELASTIC_OK;
}

}  // namespace

extern "C" {

int elastic_attn_prefill_noalloc(const void* q, const void* k, const void* v, void* o,
                                 int32_t dtype, const int32_t* cu_seqlens, int32_t batch,
                                 int64_t total_tokens, int32_t max_seqlen, int32_t n_q_heads,
                                 int32_t n_kv_heads, int32_t head_dim, float softmax_scale,
                                 const int32_t* head_mask, const elastic_sparse_cfg* sparse,
                                 float* lse_out, void* stream) {
  static const char* who = "elastic_attn_prefill_noalloc";
  // host-only validation first, against a stand-in workspace of the array's size
  char stand_in = 0;
  int st = attn_call(who, q, k, v, o, dtype, cu_seqlens, cu_seqlens, batch, total_tokens,
                     total_tokens, max_seqlen, max_seqlen, 0, 0, n_q_heads, n_kv_heads, head_dim,
                     softmax_scale, head_mask, sparse, lse_out, &stand_in,
                     ELASTIC_NOALLOC_SCRATCH_BYTES, stream, /*validate_only=*/true);
  if (st == ELASTIC_EWORKSPACE) {
    snprintf(g_last_error, sizeof(g_last_error),
             "%s: the problem needs %zu bytes of scheduler scratch; the library holds %zu "
             "(use elastic_attn_prefill with a caller workspace)", who,
             elastic_attn_workspace_size(dtype, batch, total_tokens, n_q_heads, n_kv_heads, head_dim),
             (size_t)ELASTIC_NOALLOC_SCRATCH_BYTES);
    return st;
  }
  if (st != ELASTIC_OK || total_tokens == 0) return st;
  void* ws = nullptr;
  st = noalloc_scratch(&ws);
  if (st != ELASTIC_OK) return st;
  return attn_call(who, q, k, v, o, dtype, cu_seqlens, cu_seqlens, batch, total_tokens,
                   total_tokens, max_seqlen, max_seqlen, 0, 0, n_q_heads, n_kv_heads, head_dim,
                   softmax_scale, head_mask, sparse, lse_out, ws, ELASTIC_NOALLOC_SCRATCH_BYTES,
                   stream);
}

int elastic_lse_merge(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
                      void* o_out, float* lse_out, int32_t dtype, int64_t rows, int32_t n_heads,
                      int32_t head_dim, void* stream) {
  if (rows < 0 || n_heads < 1) return ELASTIC_EINVAL;
  if (dtype != ELASTIC_BF16 && dtype != ELASTIC_FP32) return ELASTIC_EUNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return ELASTIC_EUNSUPPORTED;
  if (rows == 0) return ELASTIC_OK;
  if (!o_a || !lse_a || !o_b || !lse_b || !o_out || !lse_out) return ELASTIC_EINVAL;
  if (!(aligned16(o_a) && aligned16(o_b) && aligned16(o_out))) return ELASTIC_EINVAL;
  const hipError_t e = launch_lse_merge(dtype, o_a, lse_a, o_b, lse_b, o_out, lse_out, rows,
                                        n_heads, head_dim, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "elastic_lse_merge");
  return ELASTIC_OK;
}

size_t elastic_retrieval_workspace_size(int32_t batch, int32_t max_seqlen, int32_t n_q_heads) {
  if (batch < 0 || n_q_heads < 1) return 0;
  return align_up((size_t)batch * n_q_heads * (size_t)retrieval_chunks(max_seqlen) * 3 *
                  sizeof(float)) + ALIGN;
}

int elastic_retrieval_scores(const void* q, const void* k, int32_t dtype,
                             const int32_t* cu_seqlens, int32_t batch, int64_t total_tokens,
                             int32_t max_seqlen, int32_t n_q_heads, int32_t n_kv_heads,
                             int32_t head_dim, float softmax_scale, const int32_t* needle,
                             float* scores_q, float* scores_kv, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (batch < 0 || total_tokens < 0 || max_seqlen < 0) return ELASTIC_EINVAL;
  if (n_q_heads < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads != 0) return ELASTIC_EINVAL;
  if (cu_seqlens == nullptr && batch > 1) return ELASTIC_EINVAL;
  if (cu_seqlens == nullptr && batch == 1 && total_tokens > max_seqlen) return ELASTIC_EINVAL;
  if (dtype != ELASTIC_BF16 && dtype != ELASTIC_FP32) return ELASTIC_EUNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return ELASTIC_EUNSUPPORTED;
  if (batch == 0) return ELASTIC_OK;
  if (!q || !k || !needle || (!scores_q && !scores_kv)) return ELASTIC_EINVAL;
  if (!(aligned16(q) && aligned16(k))) return ELASTIC_EINVAL;
  if (n_q_heads / n_kv_heads > RET_MAX_G) return ELASTIC_EUNSUPPORTED;
  // grid: chunks x (KV heads x slices of 8 query heads) x sequences
  if (batch > 65535 || (int64_t)n_kv_heads * ((n_q_heads / n_kv_heads + 7) / 8) > 65535)
    return ELASTIC_EUNSUPPORTED;
  const size_t need = elastic_retrieval_workspace_size(batch, max_seqlen, n_q_heads);
  if (workspace == nullptr || workspace_bytes < need) return ELASTIC_EWORKSPACE;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)head_dim);
  const hipError_t e = launch_retrieval(dtype, head_dim, q, k, cu_seqlens, total_tokens, batch,
                                        max_seqlen, n_q_heads, n_kv_heads, scale, needle,
                                        static_cast<float*>(workspace), scores_q, scores_kv,
                                        static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "elastic_retrieval_scores");
  return ELASTIC_OK;
}

int elastic_static_assignment(const float* scores, int32_t n_units, double omega_msr,
                              int32_t* mask_out, void* stream) {
  if (n_units < 0 || !(omega_msr >= 0.0 && omega_msr <= 1.0)) return ELASTIC_EINVAL;
  if (n_units > ELASTIC_ASSIGN_MAX_UNITS) return ELASTIC_EUNSUPPORTED;
  if (n_units == 0) return ELASTIC_OK;
  if (!scores || !mask_out) return ELASTIC_EINVAL;
  int k = (int)floor((1.0 - omega_msr) * (double)n_units);  // the pages' formula, in fp64
  k = k < 0 ? 0 : (k > n_units ? n_units : k);
  const hipError_t e = launch_assign(scores, n_units, k, mask_out, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "elastic_static_assignment");
  return ELASTIC_OK;
}

int elastic_attn_entries(const int32_t* seqlens_host, int32_t batch,
                         const int32_t* head_mask_host, int32_t n_q_heads, int32_t n_kv_heads,
                         const elastic_sparse_cfg* sparse, int64_t* entries_out) {
  if (seqlens_host == nullptr || entries_out == nullptr || batch < 1) return ELASTIC_EINVAL;
  if (n_q_heads < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads != 0) return ELASTIC_EINVAL;
  if (head_mask_host != nullptr && sparse == nullptr) return ELASTIC_EINVAL;
  if (sparse != nullptr) {
    const int st = check_pattern(sparse);
    if (st != ELASTIC_OK) return st;
  }
  const int64_t G = n_q_heads / n_kv_heads;
  int64_t total = 0;
  for (int32_t b = 0; b < batch; ++b) {
    if (seqlens_host[b] < 0) return ELASTIC_EINVAL;
    int64_t full_e = -1, sparse_e = -1;
    for (int32_t g = 0; g < n_kv_heads; ++g) {
      const bool full = head_mask_host == nullptr || head_mask_host[(int64_t)b * n_kv_heads + g] != 0;
      if (!full && sparse->kind == ELASTIC_SPARSE_BLOCK_LIST) return ELASTIC_EUNSUPPORTED;
      int64_t& slot = full ? full_e : sparse_e;
      if (slot < 0) slot = head_entries(seqlens_host[b], full, sparse);
      total += G * slot;
    }
  }
  *entries_out = total;
  return ELASTIC_OK;
}


int elastic_attn_entries_lists(const int32_t* seqlens_host, int32_t batch,
                               const int32_t* head_mask_host, int32_t n_q_heads,
                               int32_t n_kv_heads, int32_t block_size, int32_t list_qblocks,
                               const int32_t* list_row_ptr_host, const int32_t* list_col_idx_host,
                               int64_t* entries_out) {
  if (seqlens_host == nullptr || entries_out == nullptr || batch < 1) return ELASTIC_EINVAL;
  if (n_q_heads < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads != 0) return ELASTIC_EINVAL;
  if (list_qblocks < 1 || list_row_ptr_host == nullptr) return ELASTIC_EINVAL;
  if (block_size != 64 && block_size != 128) return ELASTIC_EUNSUPPORTED;
  const int64_t rows = (int64_t)batch * n_kv_heads * list_qblocks;
  if (list_row_ptr_host[0] != 0) return ELASTIC_EINVAL;
  for (int64_t r = 0; r < rows; ++r)
    if (list_row_ptr_host[r + 1] < list_row_ptr_host[r]) return ELASTIC_EINVAL;
  if (list_row_ptr_host[rows] > 0 && list_col_idx_host == nullptr) return ELASTIC_EINVAL;
  const int64_t G = n_q_heads / n_kv_heads, B = block_size;
  std::vector<uint8_t> seen((size_t)list_qblocks);
  int64_t total = 0;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t n = seqlens_host[b];
    if (n < 0) return ELASTIC_EINVAL;
    const int64_t nqb = (n + B - 1) / B;
    if (nqb > list_qblocks) return ELASTIC_EINVAL;  // a query block without a list row
    for (int32_t g = 0; g < n_kv_heads; ++g) {
      const bool full = head_mask_host == nullptr || head_mask_host[(int64_t)b * n_kv_heads + g] != 0;
      if (full) {
        total += G * (n * (n + 1) / 2);
        continue;
      }
      // query block qb sees its listed earlier blocks whole and its own block causally; blocks
      // after qb, repeats and negative indices add nothing
      for (int64_t qb = 0; qb < nqb; ++qb) {
        const int64_t r = ((int64_t)b * n_kv_heads + g) * list_qblocks + qb;
        int64_t below = 0;
        bool diag = false;
        for (int64_t e = list_row_ptr_host[r]; e < list_row_ptr_host[r + 1]; ++e) {
          const int64_t kb = list_col_idx_host[e];
          if (kb < 0 || kb > qb || seen[(size_t)kb]) continue;
          seen[(size_t)kb] = 1;
          if (kb == qb) diag = true;
          else ++below;
        }
        for (int64_t e = list_row_ptr_host[r]; e < list_row_ptr_host[r + 1]; ++e) {
          const int64_t kb = list_col_idx_host[e];
          if (kb >= 0 && kb <= qb) seen[(size_t)kb] = 0;
        }
        const int64_t nr = (qb * B + B < n ? qb * B + B : n) - qb * B;  // query rows of the block
        total += G * (nr * below * B + (diag ? nr * (nr + 1) / 2 : 0));
      }
    }
  }
  *entries_out = total;
  return ELASTIC_OK;
}

}  // extern "C"
