// Scheduler: turns (sequence, KV head, query tile) units and the device-resident head mask
// into one work list, heaviest first, for the single hybrid attention launch.  Query tiles
// cover each sequence's query rows; costs count the key tiles of the sequence's key range
// that the tile's queries may see (absolute positions, so query chunks and key ranges cost
// what they visit).
//
// The pages describe the deployment problem this solves: mixed full and sparse heads are
// slow when run as separate passes on one GPU, so routing metadata goes straight into one
// unified launch without splitting tensors ("Elastic Attention", arXiv 2601.17367;
// paperlayer summary, section 3 "Efficient Deployment" and appendix D.1 "Sparse
// Inference").  Here the mask never leaves the device: one workgroup reads it, costs every
// item by the number of key tiles it visits (O(n) for full items, O(sink + window) for
// streaming ones), and counting-sorts the items by decreasing cost (longest processing time
// first), so the hardware dispatcher hands the long causal items out first and the short
// sparse items fill the tail.
#include "elastic_internal.hpp"

namespace elastic {
namespace {

constexpr int PLAN_THREADS = 1024;
constexpr int PLAN_BUCKETS = 4096;   // costs >= PLAN_BUCKETS - 1 share the last bucket
constexpr int PLAN_LDS_SEQ = 2048;   // sequences whose lengths / tile offsets are cached in LDS
constexpr int PLAN_LDS_MASK = 16384; // head-mask entries cached in LDS

__global__ __launch_bounds__(PLAN_THREADS) void plan_kernel(
    SeqGeom geo, int batch, int n_kv_heads, const int32_t* __restrict__ head_mask, Pattern pat,
    int BT, int BK, int64_t max_items, int32_t* __restrict__ tile_prefix,
    WorkItem* __restrict__ items, int32_t* __restrict__ n_items) {
  __shared__ int hist[PLAN_BUCKETS];
  __shared__ int cursor[PLAN_BUCKETS];
  __shared__ int scan_tmp[PLAN_THREADS];
  __shared__ int s_prefix[PLAN_LDS_SEQ + 1];
  __shared__ int s_len[PLAN_LDS_SEQ];   // query rows
  __shared__ int s_klen[PLAN_LDS_SEQ];  // key rows
  __shared__ unsigned char s_full[PLAN_LDS_MASK];
  __shared__ int carry;
  const int tid = threadIdx.x;
  const bool seq_cached = batch <= PLAN_LDS_SEQ;
  const bool mask_cached = (int64_t)batch * n_kv_heads <= PLAN_LDS_MASK;

  auto seq_len = [&](int b) -> int {
    return geo.cu_q ? geo.cu_q[b + 1] - geo.cu_q[b] : (int)geo.total_q;
  };
  auto key_len = [&](int b) -> int {
    return geo.cu_k ? geo.cu_k[b + 1] - geo.cu_k[b] : (int)geo.total_k;
  };

  // 1. tile_prefix[b] = query tiles of the sequences before b (block-wide scan in chunks).
  if (tid == 0) carry = 0;
  for (int i = tid; i < PLAN_BUCKETS; i += PLAN_THREADS) {
    hist[i] = 0;
    cursor[i] = 0;
  }
  if (mask_cached) {
    for (int i = tid; i < batch * n_kv_heads; i += PLAN_THREADS)
      s_full[i] = head_mask == nullptr || head_mask[i] != 0;
  }
  __syncthreads();
  for (int base = 0; base < batch; base += PLAN_THREADS) {
    const int b = base + tid;
    const int len = b < batch ? seq_len(b) : 0;
    const int nt = (len + BT - 1) / BT;
    scan_tmp[tid] = nt;
    __syncthreads();
    for (int off = 1; off < PLAN_THREADS; off <<= 1) {
      const int add = tid >= off ? scan_tmp[tid - off] : 0;
      __syncthreads();
      scan_tmp[tid] += add;
      __syncthreads();
    }
    if (b < batch) {
      const int pre = carry + scan_tmp[tid] - nt;
      tile_prefix[b] = pre;
      if (seq_cached) {
        s_prefix[b] = pre;
        s_len[b] = len;
        s_klen[b] = key_len(b);
      }
    }
    __syncthreads();
    if (tid == PLAN_THREADS - 1) carry += scan_tmp[tid];
    __syncthreads();
  }
  const int total_tiles = carry;
  if (tid == 0) {
    tile_prefix[batch] = total_tiles;
    if (seq_cached) s_prefix[batch] = total_tiles;
  }
  __syncthreads();
  int64_t count = (int64_t)total_tiles * n_kv_heads;
  if (count > max_items) count = max_items;  // cannot happen for consistent cu_seqlens
  const int nitem = (int)count;

  // 2. Items u = tile * n_kv_heads + g: locate, cost and histogram them.
  auto describe = [&](int u, WorkItem& it) {
    const int tile = u / n_kv_heads;
    const int g = u - tile * n_kv_heads;
    int lo = 0, hi = batch - 1;  // last b with prefix[b] <= tile
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      const int pm = seq_cached ? s_prefix[mid] : tile_prefix[mid];
      if (pm <= tile) lo = mid; else hi = mid - 1;
    }
    const int b = lo;
    const int qt = tile - (seq_cached ? s_prefix[b] : tile_prefix[b]);
    const int n = seq_cached ? s_len[b] : seq_len(b);
    const int nk = seq_cached ? s_klen[b] : key_len(b);
    const int qp = geo.q_pos >= 0 ? geo.q_pos : geo.k_pos + nk - n;  // absolute position of row 0
    const int t0 = qt * BT;
    const int t1 = min(t0 + BT, n) - 1;
    const int mi = b * n_kv_heads + g;
    const bool full = mask_cached ? s_full[mi] != 0 : (head_mask == nullptr || head_mask[mi] != 0);
    it.seq = b;
    it.group = g;
    it.qtile = qt;
    if (!full && pat.kind == ELASTIC_SPARSE_BLOCK_LIST) {
      // block lists: listed blocks of the item's query blocks (an upper bound of the union)
      const int a0 = qp + t0, a1 = qp + t1;
      int c = 0;
      if (a1 >= 0)
        for (int qb = a0 > 0 ? a0 / pat.block : 0; qb <= a1 / pat.block && qb < pat.qblocks; ++qb) {
          const int64_t r = ((int64_t)b * n_kv_heads + g) * pat.qblocks + qb;
          c += pat.row_ptr[r + 1] - pat.row_ptr[r];
        }
      it.cost = c * (pat.block / BK);
    } else {
      const KeyTiles kt(full ? MODE_FULL : pat.kind, pat, qp + t0, qp + t1, BK, geo.k_pos, geo.k_pos + nk);
      it.cost = kt.count();
    }
  };
  for (int u = tid; u < nitem; u += PLAN_THREADS) {
    WorkItem it;
    describe(u, it);
    atomicAdd(&hist[min(it.cost, PLAN_BUCKETS - 1)], 1);
  }
  __syncthreads();

  // 3. Exclusive scan in decreasing-cost order: offset[c] = items with a larger bucket.
  {
    constexpr int PER = PLAN_BUCKETS / PLAN_THREADS;
    int local[PER];
    int sum = 0;
#pragma unroll
    for (int r = 0; r < PER; ++r) {  // thread tid owns buckets counted from the top
      local[r] = hist[PLAN_BUCKETS - 1 - (tid * PER + r)];
      sum += local[r];
    }
    scan_tmp[tid] = sum;
    __syncthreads();
    for (int off = 1; off < PLAN_THREADS; off <<= 1) {
      const int add = tid >= off ? scan_tmp[tid - off] : 0;
      __syncthreads();
      scan_tmp[tid] += add;
      __syncthreads();
    }
    int run = scan_tmp[tid] - sum;
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      hist[PLAN_BUCKETS - 1 - (tid * PER + r)] = run;
      run += local[r];
    }
  }
  __syncthreads();

  // 4. Scatter.  Order inside a bucket is arbitrary; every item writes disjoint outputs with
  //    a fixed reduction order, so results do not depend on it.
  for (int u = tid; u < nitem; u += PLAN_THREADS) {
    WorkItem it;
    describe(u, it);
    const int bucket = min(it.cost, PLAN_BUCKETS - 1);
    items[hist[bucket] + atomicAdd(&cursor[bucket], 1)] = it;
  }
  if (tid == 0) *n_items = nitem;
}

}  // namespace

hipError_t launch_plan(const SeqGeom& geo, int batch, int n_kv_heads, const int32_t* head_mask,
                       const Pattern& pat, int BT, int BK, int64_t max_items, int32_t* tile_prefix,
                       WorkItem* items, int32_t* n_items, hipStream_t stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(PLAN_THREADS), 0, stream, geo, batch, n_kv_heads,
                     head_mask, pat, BT, BK, max_items, tile_prefix, items, n_items);
  return hipGetLastError();
}

}  // namespace elastic
