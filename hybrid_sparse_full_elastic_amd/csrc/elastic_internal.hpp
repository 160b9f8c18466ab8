// Internal declarations of libelastic (gfx950).  Not part of the public ABI.
//
// Key-tile geometry shared by the scheduler and the attention kernels.  Positions are local
// to a sequence.  A work item is (sequence, KV head, query tile of BT tokens); it visits the
// key tiles (BK keys each) that hold at least one key some query of the tile may see, in
// increasing order.  Mode rules follow "Elastic Attention" (arXiv 2601.17367; paperlayer
// summary, section 2 "Hybrid Head Mechanism", appendix D.1 "Sparse Inference"): full heads
// are causal; sparse heads use sink + local window streaming or a fixed block pattern.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/elastic.h"

namespace elastic {

enum : int {
  MODE_STREAM = ELASTIC_SPARSE_STREAMING,
  MODE_BLOCK = ELASTIC_SPARSE_BLOCK,
  MODE_LIST = ELASTIC_SPARSE_BLOCK_LIST,
  MODE_FULL = 3
};

// Sparse pattern as the kernels see it (by value in kernel arguments).
struct Pattern {
  int kind;                  // ELASTIC_SPARSE_*
  int sink, window;          // streaming
  int block, sink_blocks, local_blocks, stride_blocks;
  int qblocks;               // block list: CSR rows per (sequence, KV head)
  const int32_t* row_ptr;    // block list (device)
  const int32_t* col_idx;
};

// Block lists: the key blocks an item may visit are marked in LDS, one word per key block
// (bit i = visible to the item's (i+1)-th query block); LIST_MAX_KB words per workgroup.
constexpr int LIST_MAX_KB = 4096;
constexpr int LIST_MAX_QB = 8;  // query blocks one item may span

// Key tiles of one block-list item, read from the LDS visibility words vis[kb - kb0].  Same
// interface as KeyTilesT; every call is made by the whole workgroup with uniform arguments.
struct ListTiles {
  int BK, tpb, tpb_shift, t0, t1, lo, last, k_end, qb0, kb0, kb_last;  // tpb = 1 << tpb_shift
  unsigned full_mask;  // every query block of the item
  const uint32_t* vis;

  __device__ unsigned vis_of(int kt) const { return vis[(kt >> tpb_shift) - kb0]; }

  // Does the list of query block qblk (absolute) hold the key block of tile kt?
  __device__ bool lists(int kt, int qblk) const {
    const int bit = qblk - qb0;
    return bit >= 0 && bit < LIST_MAX_QB && ((vis_of(kt) >> bit) & 1u);
  }

  __device__ int next(int kt) const {
    if (kt < lo) kt = lo;
    if (kt > last) return -1;
    const int kb = kt >> tpb_shift;
    if (vis[kb - kb0] != 0) return kt;
    const int lane = __lane_id();
    for (int base = kb + 1; base <= kb_last; base += 64) {
      const int b = base + lane;
      const uint64_t m = __ballot(b <= kb_last && vis[b - kb0] != 0);
      if (m != 0) {
        const int t = (base + __ffsll((unsigned long long)m) - 1) << tpb_shift;
        return t <= last ? t : -1;
      }
    }
    return -1;
  }

  __device__ bool needs_mask(int kt) const {
    const int k0 = kt * BK, k1 = k0 + BK - 1;
    return k1 > t0 || k1 >= k_end || vis_of(kt) != full_mask;
  }

  __device__ bool steady_pair(int) const { return false; }
};

// Builds the ListTiles of one block-list item: marks in vis the key blocks of the range that
// the item's query blocks list (ignoring blocks after the query block), then returns the
// walker.  The whole workgroup calls it (two barriers).  a0, a1: absolute positions of the
// item's first and last query; [k_begin, k_end): its key range.
__device__ inline ListTiles list_tiles(uint32_t* vis, const Pattern& p, int b, int g,
                                       int n_kv_heads, int a0, int a1, int k_begin, int k_end,
                                       int BK, int tid, int nt) {
  ListTiles t;
  t.BK = BK;
  t.tpb = p.block / BK;
  t.tpb_shift = __builtin_ctz((unsigned)t.tpb);  // block and BK are powers of two
  t.t0 = a0;
  t.t1 = a1;
  t.k_end = k_end;
  t.vis = vis;
  t.lo = k_begin / BK;
  t.kb0 = k_begin / p.block;
  const int qb0 = a0 > 0 ? a0 / p.block : 0;
  const int qb1 = a1 >= 0 ? a1 / p.block : -1;
  t.qb0 = qb0;
  const int kb_end = k_end > k_begin ? (k_end - 1) / p.block : t.kb0 - 1;
  t.kb_last = qb1 < kb_end ? qb1 : kb_end;
  const int diag = a1 >= 0 ? a1 / BK : -1;
  const int hi = k_end > k_begin ? (k_end - 1) / BK : t.lo - 1;
  t.last = diag < hi ? diag : hi;
  if (t.kb_last - t.kb0 + 1 > LIST_MAX_KB) t.kb_last = t.kb0 + LIST_MAX_KB - 1;  // checked on the host
  const int nqb = qb1 - qb0 + 1;
  t.full_mask = nqb >= 32 ? 0xffffffffu : (1u << (nqb > 0 ? nqb : 0)) - 1u;
  for (int i = tid; i <= t.kb_last - t.kb0; i += nt) vis[i] = 0;
  __syncthreads();
  for (int qb = qb0; qb <= qb1 && qb - qb0 < LIST_MAX_QB; ++qb) {
    if (qb >= p.qblocks) break;
    const int64_t r = ((int64_t)b * n_kv_heads + g) * p.qblocks + qb;
    const int e0 = p.row_ptr[r], e1 = p.row_ptr[r + 1];
    for (int e = e0 + tid; e < e1; e += nt) {
      const int kb = p.col_idx[e];
      if (kb >= t.kb0 && kb <= t.kb_last && kb <= qb) atomicOr(&vis[kb - t.kb0], 1u << (qb - qb0));
    }
  }
  __syncthreads();
  return t;
}

// Query/key geometry of one attention call.  Sequence b has queries at rows
// [cu_q[b], cu_q[b+1]) of q/o and keys at rows [cu_k[b], cu_k[b+1]) of k/v (a null array
// means one sequence of total_q / total_k rows).  Positions are absolute: query t of the
// sequence sits at q_pos + t (q_pos < 0: the queries are the last key positions,
// k_pos + n_k - n_q) and key j at k_pos + j (k_pos a multiple of 64).
struct SeqGeom {
  const int32_t* cu_q;
  const int32_t* cu_k;
  int64_t total_q, total_k;
  int q_pos, k_pos;
};

struct SeqSpan {
  int64_t q0, k0;  // first row of the sequence in q/o and in k/v
  int nq, nk;      // query and key rows
  int qp;          // absolute position of query row 0
};

__host__ __device__ inline SeqSpan seq_span(const SeqGeom& g, int b) {
  SeqSpan s;
  s.q0 = g.cu_q ? g.cu_q[b] : 0;
  s.nq = g.cu_q ? g.cu_q[b + 1] - (int)s.q0 : (int)g.total_q;
  s.k0 = g.cu_k ? g.cu_k[b] : 0;
  s.nk = g.cu_k ? g.cu_k[b + 1] - (int)s.k0 : (int)g.total_k;
  s.qp = g.q_pos >= 0 ? g.q_pos : g.k_pos + s.nk - s.nq;
  return s;
}

// One scheduled unit of attention work.
struct WorkItem {
  int seq;    // sequence index b
  int group;  // KV head g
  int qtile;  // query tile index: tokens [qtile * BT, min(n, (qtile + 1) * BT))
  int full;   // 1: the KV head runs full attention, 0: its sparse pattern (from the head mask)
};

// Is key j visible to query i (local positions) under `mode`?
__host__ __device__ inline bool key_allowed(int mode, const Pattern& p, int i, int j) {
  if (j > i) return false;
  if (mode == MODE_FULL) return true;
  if (mode == MODE_STREAM) return j < p.sink || i - j < p.window;
  const int qb = i / p.block, kb = j / p.block;
  return kb < p.sink_blocks || qb - kb <= p.local_blocks ||
         (p.stride_blocks > 0 && kb % p.stride_blocks == 0);
}

// Key tiles visited by the query tokens [t0, t1] (inclusive) of one work item.  Positions
// are absolute: queries and keys of a sequence share one axis, so a chunk of queries can
// attend a range of keys [k_begin, k_end) (k_begin a multiple of BK, and of the block size
// for the block pattern).  Tile index kt holds keys [kt * BK, kt * BK + BK).  M is the mode
// when it is known at compile time (MODE_*), or -1 to take it from the constructor.
template <int M = -1>
struct KeyTilesT {
  int mode_rt, BK, t0, t1;
  int diag;                 // tile of the last query: the causal limit
  int lo, last;             // visited tiles lie in [lo, last]; last < lo when none
  int k_end;                // one past the last key present
  Pattern p;
  int sink_end, win_begin;  // streaming: tiles [0, sink_end) and [win_begin, diag]
  int tpb, qb0, qb1;        // block: tiles per block, query blocks of t0 and t1
  // block: log2 of tiles per block and of the block size (both powers of two), and
  // stride_blocks - 1 when the stride is a power of two (else -1): the per-step tile walk
  // then takes shifts and masks instead of scalar divisions
  int tpb_shift, blk_shift, stride_mask, stride_shift;

  __host__ __device__ int mode() const { return M >= 0 ? M : mode_rt; }

  __host__ __device__ KeyTilesT(int mode_, const Pattern& p_, int t0_, int t1_, int BK_,
                                int k_begin = 0, int k_end_ = 0x7fffffff)
      : mode_rt(mode_), BK(BK_), t0(t0_), t1(t1_), diag(t1_ >= 0 ? t1_ / BK_ : -1), k_end(k_end_), p(p_) {
    // (queries at negative positions -- more query rows than keys under bottom-right
    // alignment -- see no key: their tiles are skipped or fully masked)
    lo = k_begin / BK;
    const int hi = k_end > k_begin ? (k_end - 1) / BK : lo - 1;
    last = diag < hi ? diag : hi;
    sink_end = 0;
    win_begin = 0;
    tpb = 1;
    qb0 = qb1 = 0;
    tpb_shift = blk_shift = stride_shift = 0;
    stride_mask = -1;
    if (mode() == MODE_STREAM) {
      const int sink_keys = p.sink < t1 + 1 ? p.sink : t1 + 1;
      sink_end = (sink_keys + BK - 1) / BK;
      const int w0 = t0 - p.window + 1;
      win_begin = w0 > 0 ? w0 / BK : 0;
    } else if (mode() == MODE_BLOCK) {
      tpb = p.block / BK;  // block_size is a multiple of BK (checked on the host)
      qb0 = t0 / p.block;
      qb1 = t1 / p.block;
      tpb_shift = __builtin_ctz((unsigned)tpb);
      blk_shift = __builtin_ctz((unsigned)p.block);
      if (p.stride_blocks > 0 && (p.stride_blocks & (p.stride_blocks - 1)) == 0) {
        stride_mask = p.stride_blocks - 1;
        stride_shift = __builtin_ctz((unsigned)p.stride_blocks);
      }
    }
  }

  // Block lists only (ListTiles): closed-form patterns have no lists.
  __host__ __device__ bool lists(int, int) const { return true; }

  // Smallest key block >= kb that some query block in [qb0, qb1] may see.
  __host__ __device__ int next_block(int kb) const {
    if (kb < p.sink_blocks || kb >= qb0 - p.local_blocks) return kb;
    int c = qb0 - p.local_blocks;
    if (p.stride_blocks > 0) {
      const int m = stride_mask >= 0 ? (kb + stride_mask) & ~stride_mask
                                     : ((kb + p.stride_blocks - 1) / p.stride_blocks) * p.stride_blocks;
      if (m < c) c = m;
    }
    return c;
  }

  // Smallest visited tile >= kt, or -1 when there is none.
  __host__ __device__ int next(int kt) const {
    if (kt < lo) kt = lo;
    if (kt > last) return -1;
    if (mode() == MODE_STREAM) {
      if (kt >= sink_end && kt < win_begin) kt = win_begin;
    } else if (mode() == MODE_BLOCK) {
      const int kb = kt >> tpb_shift;
      const int nb = next_block(kb);
      if (nb != kb) kt = nb << tpb_shift;
    }
    return kt <= last ? kt : -1;
  }

  // Does tile kt need per-element masking for some (query, key) pair of this item?
  __host__ __device__ bool needs_mask(int kt) const {
    const int k0 = kt * BK, k1 = k0 + BK - 1;
    if (k1 > t0) return true;      // causal edge
    if (k1 >= k_end) return true;  // keys past the end of the range (or of the sequence)
    if (mode() == MODE_FULL) return false;
    if (mode() == MODE_STREAM) return !(k1 < p.sink || k0 > t1 - p.window);
    const int kb = k0 >> blk_shift;
    const bool on_stride = p.stride_blocks > 0 &&
                           (stride_mask >= 0 ? (kb & stride_mask) == 0 : kb % p.stride_blocks == 0);
    return !(kb < p.sink_blocks || kb >= qb1 - p.local_blocks || on_stride);
  }

  // Visited tiles in [0, x] for x <= diag, ignoring the key range, without enumeration.
  __host__ __device__ int cnt_upto(int x) const {
    if (x < 0) return 0;
    if (mode() == MODE_FULL) return x + 1;
    if (mode() == MODE_STREAM) {  // [0, sink_end) U [win_begin, diag], clipped to [0, diag]
      const int se = sink_end < diag + 1 ? sink_end : diag + 1;
      const int wb = win_begin > se ? win_begin : se;
      return (x + 1 < se ? x + 1 : se) + (x >= wb ? x - wb + 1 : 0);
    }
    // block: key blocks below qb1 are visible when in [0, a), [b0, qb1) or a stride multiple;
    // the diagonal block qb1 is visited up to diag
    const int a = p.sink_blocks < qb1 ? p.sink_blocks : qb1;
    const int b0 = qb0 - p.local_blocks > 0 ? qb0 - p.local_blocks : 0;
    const int xb = x >> tpb_shift;
    const int m = xb < qb1 ? xb : qb1;  // whole visible blocks in [0, m)
    int nb;
    if (a >= b0) {
      nb = m;
    } else {
      nb = (m < a ? m : a) + (m > b0 ? m - b0 : 0);
      const int top = m < b0 ? m : b0;
      if (p.stride_blocks > 0 && top > a)  // stride multiples in [a, top) (both >= 0)
        nb += stride_mask >= 0
                  ? ((top + stride_mask) >> stride_shift) - ((a + stride_mask) >> stride_shift)
                  : (top + p.stride_blocks - 1) / p.stride_blocks - (a + p.stride_blocks - 1) / p.stride_blocks;
    }
    if (xb >= qb1) return nb * tpb + (x - qb1 * tpb + 1);
    const bool vis = xb < a || xb >= b0 ||
                     (p.stride_blocks > 0 && (stride_mask >= 0 ? (xb & stride_mask) == 0 : xb % p.stride_blocks == 0));
    return nb * tpb + (vis ? x - xb * tpb + 1 : 0);
  }

  __host__ __device__ int count() const {
    return last < lo ? 0 : cnt_upto(last) - cnt_upto(lo - 1);
  }

  // May a pair of steady steps start at visited tile j?  Then tiles j..j+6 are visited
  // consecutively, tiles j..j+5 hold BK keys of the range each, and tiles j+1, j+2 need no
  // mask: the pair loads (K up to tile j+5), computes and advances (the schedule looks six
  // tiles ahead) without any bound decision.  Such runs are
  // a full item's tiles below the diagonal, a streaming item's window interior, and the
  // local blocks every query of a block item sees.
  __host__ __device__ bool steady_pair(int j) const {
    const int whole_end = k_end / BK;
    const int causal = (t0 + 1) / BK;  // tiles below hold only keys <= t0
    const int mask_from = causal < whole_end ? causal : whole_end;
    if (!(j + 6 <= last && j + 5 < whole_end && j + 2 < mask_from)) return false;
    if (mode() == MODE_FULL) return true;
    if (mode() == MODE_STREAM) return j >= win_begin && (j + 1) * BK > t1 - p.window;
    const int run = (qb0 - p.local_blocks > 0 ? qb0 - p.local_blocks : 0) * tpb;
    const int free = (qb1 - p.local_blocks > 0 ? qb1 - p.local_blocks : 0) * tpb;
    return j >= run && j + 1 >= free;
  }
};
using KeyTiles = KeyTilesT<-1>;

// ------------------------------------------------------------------ tile configurations
// bf16 MFMA attention: NW waves x NB blocks of 32 query rows per workgroup, 64-key tiles.
constexpr int BF16_NW = 8;
constexpr int BF16_NB = 1;
constexpr int BF16_ROWS = BF16_NW * BF16_NB * 32;  // query rows (token, head) per workgroup
constexpr int BF16_BK = 64;
// fp32 attention: one thread per query row, 32-key tiles.
constexpr int F32_ROWS = 256;
constexpr int F32_BK = 32;

// Query tokens per work item: the workgroup's rows hold whole tokens' G heads.
inline int tokens_per_item(int rows, int G) { return rows / G; }

// ------------------------------------------------------------------ per-XCD work queues
// The scheduler splits the work list into one queue per XCD.  Each queue holds the items of
// a few (sequence, KV head) groups -- a cut of the groups laid end to end, balanced by cost --
// heaviest first, so the workgroups of one XCD stream the same K/V through their shared L2.
// Workgroup b runs on XCD b % SCHED_NX (the dispatcher deals workgroups out round-robin); it
// claims items from its own queue and, once that is empty, from the others (the largest
// remaining item first), so XCDs that run ahead take over work.  Correctness does not depend
// on the XCD mapping: every item is claimed exactly once by a counter increment.
//
// Header (int32, in the workspace): [0] item count, [1 + x] first item of queue x
// (x = 0..SCHED_NX, the last entry is the count), and the claim counter of queue x at
// [SCHED_CTR * (1 + x)], each on a 128-byte line of its own.
constexpr int SCHED_NX = 8;
constexpr int SCHED_CTR = 32;
constexpr int SCHED_INTS = SCHED_CTR * (SCHED_NX + 1);

// Index of the next item for the calling workgroup, or -1 when every queue is empty.  One
// thread calls it; the result is broadcast to the workgroup.
__device__ inline int claim_item(int32_t* sched) {
  const int x = (int)(blockIdx.x % SCHED_NX);
  for (int i = 0; i < SCHED_NX; ++i) {
    const int y = (x + i) % SCHED_NX;
    const int q0 = sched[1 + y], len = sched[2 + y] - q0;
    int* ctr = sched + SCHED_CTR * (1 + y);
    if (len <= 0) continue;
    // other queues: skip them without an increment when already empty
    if (i > 0 && __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= len) continue;
    const int k = atomicAdd(ctr, 1);
    if (k < len) return q0 + k;
  }
  return -1;
}

// Workgroups of `kernel` (block `threads`, static LDS only) that fit on the current device at
// once: compute units x resident workgroups per unit (cached per device and kernel).
hipError_t resident_grid(const void* kernel, int threads, int64_t* grid);

// ------------------------------------------------------------------ launchers (device code)
hipError_t launch_plan(const SeqGeom& geo, int batch, int n_kv_heads, const int32_t* head_mask,
                       const Pattern& pat, int BT, int BK, int64_t max_items, int32_t* tile_prefix,
                       int32_t* cost_tmp, WorkItem* items, int32_t* sched, hipStream_t stream);

hipError_t launch_attn_bf16(int head_dim, const void* q, const void* k, const void* v, void* o,
                            float* lse, const SeqGeom& geo, int n_q_heads, int n_kv_heads, int BT,
                            float scale, const int32_t* head_mask, const Pattern& pat,
                            const WorkItem* items, int32_t* sched, int64_t max_items,
                            hipStream_t stream);

hipError_t launch_attn_f32(int head_dim, const void* q, const void* k, const void* v, void* o,
                           float* lse, const SeqGeom& geo, int n_q_heads, int n_kv_heads, int BT,
                           float scale, const Pattern& pat,
                           const WorkItem* items, int32_t* sched, int64_t max_items,
                           hipStream_t stream);

// Retrieval scores: keys per partial workgroup, chunk count for a sequence length bound.
constexpr int RET_CHUNK = 256;
constexpr int RET_MAX_G = 1024;  // query heads per KV head the score combine supports
int64_t retrieval_chunks(int32_t max_seqlen);
hipError_t launch_retrieval(int dtype, int head_dim, const void* q, const void* k,
                            const int32_t* cu, int64_t total, int batch, int max_seqlen, int Hq,
                            int Hkv, float scale, const int32_t* needle, float* part,
                            float* scores_q, float* scores_kv, hipStream_t stream);
hipError_t launch_assign(const float* scores, int n, int k, int32_t* mask, hipStream_t stream);

hipError_t launch_lse_merge(int dtype, const void* o_a, const float* lse_a, const void* o_b,
                            const float* lse_b, void* o_out, float* lse_out, int64_t rows,
                            int heads, int head_dim, hipStream_t stream);

// Router: rows of sequence b are pooled in slabs of ROUTE_SLAB rows.
constexpr int ROUTE_SLAB = 128;
constexpr int ROUTE_MAX_DR = 256;   // d_router limit
constexpr int ROUTE_MAX_HKV = 256;  // n_kv_heads limit

hipError_t launch_route(const void* hidden, int hidden_dtype, const int32_t* cu_seqlens, int batch,
                        int64_t total_tokens, int d_model, int pool_head, int pool_tail,
                        const float* w1, int d_router, const float* w2, int n_kv_heads,
                        float threshold, float* logits_out, int32_t* mask_out, float* partials,
                        int64_t max_slabs, float* zpart, int32_t* done, hipStream_t stream);
constexpr int ROUTE_HCOLS = 64;  // columns per route_strip workgroup

}  // namespace elastic
