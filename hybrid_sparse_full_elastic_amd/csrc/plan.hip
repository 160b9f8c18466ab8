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
// streaming ones), cuts the groups (sequence, KV head) into one cost-balanced queue per XCD,
// and counting-sorts each queue by decreasing cost (longest processing time first): the
// workgroups of an XCD take the long causal items of their groups first, the short sparse
// items fill the tail, and XCDs that run ahead take items from the other queues.
#include "elastic_internal.hpp"

namespace elastic {
namespace {

constexpr int PLAN_THREADS = 1024;
constexpr int PLAN_BUCKETS = 1024;   // cost buckets per queue (see bucket_of)
constexpr int PLAN_LDS_SEQ = 1024;   // sequences whose lengths / tile offsets are cached in LDS
constexpr int PLAN_LDS_MASK = 16384; // head-mask entries cached in LDS
constexpr int PLAN_LDS_COST = 16384; // items whose costs are cached in LDS (else cost_tmp)
constexpr int PLAN_MEMO_TILES = 4096; // query tiles whose full / sparse costs are tabulated in LDS
constexpr int ITEM_OVERHEAD = 2;     // per-item cost (prologue, epilogue) in key tiles, for the cut

// Cost bucket: exact below 768 key tiles, then 16 tiles wide; 1023 holds everything above.
__device__ inline int bucket_of(int cost) {
  return cost < 768 ? cost : min(768 + ((cost - 768) >> 4), PLAN_BUCKETS - 1);
}

// x of the lane that the DPP control CTRL names (0 where it names none, and in the rows that
// ROWS leaves out), both 32-bit halves moved alike.
template <int CTRL, int ROWS>
__device__ inline long long dpp_take(long long x) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)x, CTRL, ROWS, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(x >> 32), CTRL, ROWS, 0xf, false);
  return (long long)(((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo);
}
// Inclusive scan over the 64 lanes of a wave: Kogge-Stone inside each 16-lane row (row_shr 1,
// 2, 4, 8), then the total of row 0 into rows 1 and 3 (row_bcast:15) and of rows 0-1 into
// rows 2 and 3 (row_bcast:31).  DPP moves are VALU operations, where a shuffle is an LDS
// round trip; the scheduler's single workgroup runs a chain of these scans.
__device__ inline long long wave_scan(long long x) {
  x += dpp_take<0x111, 0xf>(x);
  x += dpp_take<0x112, 0xf>(x);
  x += dpp_take<0x114, 0xf>(x);
  x += dpp_take<0x118, 0xf>(x);
  x += dpp_take<0x142, 0xa>(x);
  x += dpp_take<0x143, 0xc>(x);
  return x;
}

// Block-wide inclusive scan of one value per thread (64-bit): wave scans, then a scan of the
// wave totals.  Returns the thread's inclusive prefix and leaves the block total in *total.
// Every thread must call it; tmp holds PLAN_THREADS / 64 values.
constexpr int PLAN_WAVES = PLAN_THREADS / 64;
__device__ inline long long block_scan(long long x, long long* tmp, long long* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  x = wave_scan(x);
  if (lane == 63) tmp[w] = x;
  __syncthreads();
  if (w == 0) {
    const long long t = wave_scan(lane < PLAN_WAVES ? tmp[lane] : 0);
    if (lane < PLAN_WAVES) tmp[lane] = t;
  }
  __syncthreads();
  const long long r = x + (w > 0 ? tmp[w - 1] : 0);
  *total = tmp[PLAN_WAVES - 1];
  __syncthreads();  // tmp is reused by the next call
  return r;
}

// One slot of a shared LDS counter per lane: `key` (any value where active is false) is
// incremented by one for every active lane, and each active lane gets the counter's value
// before its own increment.  When every active lane of the wave has the same key (items of
// equal cost in one queue, the common case for sparse heads) one atomic adds them all, which
// spares the LDS from serialising 64 atomics on one address.  Every lane of the wave calls it.
__device__ inline int lds_count(int* counters, int key, bool active) {
  const int lane = threadIdx.x & 63;
  const uint64_t act = __ballot(active);
  if (act == 0) return 0;
  const int leader = __ffsll((unsigned long long)act) - 1;  // wave-uniform
  const int k0 = __builtin_amdgcn_readlane(key, leader);
  if (__ballot(active && key == k0) == act) {
    int base = 0;
    if (lane == leader) base = atomicAdd(&counters[k0], (int)__popcll(act));
    base = __builtin_amdgcn_readlane(base, leader);
    return base + (int)__popcll(act & ((1ull << lane) - 1ull));
  }
  return active ? atomicAdd(&counters[key], 1) : 0;
}

// BK (key tile width) is a template argument so that the tile arithmetic of the cost model
// divides by a constant.  SMALL (the host's choice: the sequences, the head mask and the item
// bound all fit the LDS caches) makes every cached read an LDS instruction; with the caches
// chosen at run time the compiler merges the two sources into generic (flat) loads.
template <int BK, bool SMALL>
__global__ __launch_bounds__(PLAN_THREADS) void plan_kernel(
    SeqGeom geo, int batch, int n_kv_heads, const int32_t* __restrict__ head_mask, Pattern pat,
    int BT, int64_t max_items, int32_t* __restrict__ tile_prefix,
    int32_t* __restrict__ cost_tmp, WorkItem* __restrict__ items, int32_t* __restrict__ sched) {
  __shared__ int hist[SCHED_NX * PLAN_BUCKETS];
  __shared__ long long scan_tmp[PLAN_WAVES];
  __shared__ int s_prefix[PLAN_LDS_SEQ + 1];
  __shared__ int s_len[PLAN_LDS_SEQ];   // query rows
  __shared__ int s_klen[PLAN_LDS_SEQ];  // key rows
  __shared__ unsigned char s_full[PLAN_LDS_MASK];
  __shared__ int s_cost[PLAN_LDS_COST];
  __shared__ int s_memo[2][PLAN_MEMO_TILES];  // cost of a query tile: [0] sparse heads, [1] full
  const int tid = threadIdx.x;
  const bool seq_cached = SMALL || batch <= PLAN_LDS_SEQ;
  const bool mask_cached = SMALL || (int64_t)batch * n_kv_heads <= PLAN_LDS_MASK;

  auto seq_len = [&](int b) -> int {
    return geo.cu_q ? geo.cu_q[b + 1] - geo.cu_q[b] : (int)geo.total_q;
  };
  auto key_len = [&](int b) -> int {
    return geo.cu_k ? geo.cu_k[b + 1] - geo.cu_k[b] : (int)geo.total_k;
  };

  // 1. tile_prefix[b] = query tiles of the sequences before b (block-wide scan in chunks).
  for (int i = tid; i < SCHED_NX * PLAN_BUCKETS; i += PLAN_THREADS) hist[i] = 0;
  if (mask_cached) {
    for (int i = tid; i < batch * n_kv_heads; i += PLAN_THREADS)
      s_full[i] = head_mask == nullptr || head_mask[i] != 0;
  }
  long long carry = 0, total;
  for (int base = 0; base < batch; base += PLAN_THREADS) {
    const int b = base + tid;
    const int len = b < batch ? seq_len(b) : 0;
    const int nt = (len + BT - 1) / BT;
    const long long inc = block_scan(nt, scan_tmp, &total);
    if (b < batch) {
      const int pre = (int)(carry + inc - nt);
      tile_prefix[b] = pre;
      if (seq_cached) {
        s_prefix[b] = pre;
        s_len[b] = len;
        s_klen[b] = key_len(b);
      }
    }
    carry += total;
  }
  const int total_tiles = (int)carry;
  if (tid == 0) {
    tile_prefix[batch] = total_tiles;
    if (seq_cached) s_prefix[batch] = total_tiles;
  }
  __syncthreads();
  int64_t count = (int64_t)total_tiles * n_kv_heads;
  if (count > max_items) count = max_items;  // cannot happen for consistent cu_seqlens
  if (SMALL && count > PLAN_LDS_COST) count = PLAN_LDS_COST;  // max_items bounds it
  const int nitem = (int)count;

  // Item u = tile * n_kv_heads + g, tile = tile_prefix[b] + qtile.
  auto seq_of_tile = [&](int tile) {  // last b with prefix[b] <= tile
    int lo = 0, hi = batch - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      const int pm = seq_cached ? s_prefix[mid] : tile_prefix[mid];
      if (pm <= tile) lo = mid; else hi = mid - 1;
    }
    return lo;
  };
  auto prefix_of = [&](int b) { return seq_cached ? s_prefix[b] : tile_prefix[b]; };
  // u / n_kv_heads: a shift for the usual power-of-two head counts (a runtime division costs
  // tens of instructions, and this one workgroup is bound by its own VALU work per item)
  const int hkv_shift = (n_kv_heads & (n_kv_heads - 1)) == 0 ? __builtin_ctz(n_kv_heads) : -1;
  auto tile_of = [&](int u) { return hkv_shift >= 0 ? u >> hkv_shift : u / n_kv_heads; };
  auto locate = [&](int u, WorkItem& it) {
    const int tile = tile_of(u);
    it.group = u - tile * n_kv_heads;
    it.seq = seq_of_tile(tile);
    it.qtile = tile - prefix_of(it.seq);
  };
  auto full_of = [&](const WorkItem& it) -> bool {
    const int mi = it.seq * n_kv_heads + it.group;
    return mask_cached ? s_full[mi] != 0 : (head_mask == nullptr || head_mask[mi] != 0);
  };
  // cost: key tiles of the sequence's key range that the item's queries may see
  auto cost_of_mode = [&](const WorkItem& it, bool full) -> int {
    const int b = it.seq, g = it.group;
    const int n = seq_cached ? s_len[b] : seq_len(b);
    const int nk = seq_cached ? s_klen[b] : key_len(b);
    const int qp = geo.q_pos >= 0 ? geo.q_pos : geo.k_pos + nk - n;  // absolute position of row 0
    const int t0 = it.qtile * BT;
    const int t1 = min(t0 + BT, n) - 1;
    if (!full && pat.kind == ELASTIC_SPARSE_BLOCK_LIST) {
      // block lists: listed blocks of the item's query blocks (an upper bound of the union)
      const int a0 = qp + t0, a1 = qp + t1;
      int c = 0;
      if (a1 >= 0)
        for (int qb = a0 > 0 ? a0 / pat.block : 0; qb <= a1 / pat.block && qb < pat.qblocks; ++qb) {
          const int64_t r = ((int64_t)b * n_kv_heads + g) * pat.qblocks + qb;
          c += pat.row_ptr[r + 1] - pat.row_ptr[r];
        }
      return c * (pat.block / BK);
    }
    const KeyTiles kt(full ? MODE_FULL : pat.kind, pat, qp + t0, qp + t1, BK, geo.k_pos, geo.k_pos + nk);
    return kt.count();
  };
  auto cost_of = [&](const WorkItem& it) -> int { return cost_of_mode(it, full_of(it)); };

  // per-item cost (then cost | XCD << 28): in LDS when it fits, else in the workspace
  int* const cost = SMALL || nitem <= PLAN_LDS_COST ? s_cost : cost_tmp;

  // 2. Costs, and their total weight for the cut.  Every KV head of a query tile shares its
  //    tile's cost for its mode (except with block lists, which differ per head), so the
  //    closed forms are evaluated once per (tile, mode) into an LDS table when it fits.
  const bool memo = pat.kind != ELASTIC_SPARSE_BLOCK_LIST && total_tiles <= PLAN_MEMO_TILES &&
                    nitem > 2 * PLAN_THREADS;  // below that the extra pass costs what it saves
  if (memo) {
    for (int t = tid; t < 2 * total_tiles; t += PLAN_THREADS) {
      const int tile = t >> 1;
      WorkItem it;
      it.seq = seq_of_tile(tile);
      it.qtile = tile - prefix_of(it.seq);
      it.group = 0;
      s_memo[t & 1][tile] = cost_of_mode(it, (t & 1) != 0);
    }
    __syncthreads();
  }
  long long wsum = 0;
  for (int u = tid; u < nitem; u += PLAN_THREADS) {
    WorkItem it;
    locate(u, it);
    const int c = memo ? s_memo[full_of(it) ? 1 : 0][tile_of(u)] : cost_of(it);
    cost[u] = c;
    wsum += c + ITEM_OVERHEAD;
  }
  block_scan(wsum, scan_tmp, &total);
  const long long W = total > 0 ? total : 1;
  const double inv_2w = (double)SCHED_NX / (2.0 * (double)W);

  // 3. Cut: lay the groups (sequence, KV head) end to end and give item L of that line to XCD
  //    floor(8 * (weight before L + half its own) / W).  Line index L: sequence b owns
  //    [tile_prefix[b] * Hkv, tile_prefix[b + 1] * Hkv), KV head major inside it, and a
  //    group's query tiles alternate from both ends (0, last, 1, last - 1, ...), so that any
  //    stretch of the line -- a queue -- holds long and short items alike (causal costs grow
  //    with the query tile) and every queue ends on short items.  The XCD goes into the top
  //    bits of cost[u].
  //    Each thread takes CUT_PT consecutive line positions per round, so a round needs one
  //    block-wide scan; the thread locates its first position with divisions and steps to the
  //    next ones (query tile, then KV head, then sequence).
  constexpr int CUT_PT = 4;
  carry = 0;
  for (int base = 0; base < nitem; base += PLAN_THREADS * CUT_PT) {
    int uu[CUT_PT], cc[CUT_PT];
    long long wt = 0;  // this thread's weight in the round
    const int L0 = base + tid * CUT_PT;
    int b = 0, p0 = 0, nt = 1, g = 0, j = 0;
    if (L0 < nitem) {
      b = seq_of_tile(tile_of(L0));
      p0 = prefix_of(b);
      nt = prefix_of(b + 1) - p0;  // >= 1: b holds position L0
      const int rr = L0 - p0 * n_kv_heads;
      g = rr / nt;
      j = rr - g * nt;
    }
#pragma unroll
    for (int r = 0; r < CUT_PT; ++r) {
      uu[r] = -1;
      cc[r] = 0;
      if (L0 + r < nitem) {
        if (r > 0 && ++j == nt) {  // next group, or the next sequence that has query tiles
          j = 0;
          if (++g == n_kv_heads) {
            g = 0;
            do {
              p0 += nt;
              nt = prefix_of(++b + 1) - p0;
            } while (nt == 0);
          }
        }
        const int qt = (j & 1) ? nt - 1 - (j >> 1) : (j >> 1);  // 0, nt-1, 1, nt-2, ...
        uu[r] = (p0 + qt) * n_kv_heads + g;
        cc[r] = cost[uu[r]];
        wt += cc[r] + ITEM_OVERHEAD;
      }
    }
    const long long inc = block_scan(wt, scan_tmp, &total);
    long long before = carry + inc - wt;  // line weight before this thread's first position
#pragma unroll
    for (int r = 0; r < CUT_PT; ++r) {
      const bool active = uu[r] >= 0;
      int key = 0;
      if (active) {
        const long long w = cc[r] + ITEM_OVERHEAD;
        const long long mid2 = 2 * before + w;  // twice the item's midpoint
        before += w;
        // floor(8 * midpoint / W) in fp64 (a 64-bit integer division costs far more; a
        // boundary rounded the other way only moves one item to the neighbouring queue)
        const int x = (int)min((double)(SCHED_NX - 1), floor((double)mid2 * inv_2w));
        cost[uu[r]] = cc[r] | (x << 28);
        key = x * PLAN_BUCKETS + (PLAN_BUCKETS - 1 - bucket_of(cc[r]));
      }
      lds_count(hist, key, active);
    }
    carry += total;
  }
  __syncthreads();

  // 4. Exclusive scan over (queue, decreasing cost): hist[key] becomes the key's first slot.
  {
    constexpr int PER = SCHED_NX * PLAN_BUCKETS / PLAN_THREADS;
    int local[PER];
    int sum = 0;
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      local[r] = hist[tid * PER + r];
      sum += local[r];
    }
    const long long inc = block_scan(sum, scan_tmp, &total);
    int run = (int)(inc - sum);
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int key = tid * PER + r;
      if (key % PLAN_BUCKETS == 0) sched[1 + key / PLAN_BUCKETS] = run;  // queue start
      hist[key] = run;
      run += local[r];
    }
  }
  __syncthreads();

  // 5. Scatter.  Order inside a bucket is arbitrary; every item writes disjoint outputs with
  //    a fixed reduction order, so results do not depend on it.
  for (int base = 0; base < nitem; base += PLAN_THREADS) {  // whole waves call lds_count
    const int u = base + tid;
    const bool active = u < nitem;
    WorkItem it;
    int key = 0;
    if (active) {
      locate(u, it);
      const int packed = cost[u];
      const int c = packed & 0x0fffffff;
      const int x = (int)((unsigned)packed >> 28);
      it.full = full_of(it) ? 1 : 0;
      key = x * PLAN_BUCKETS + (PLAN_BUCKETS - 1 - bucket_of(c));
    }
    const int slot = lds_count(hist, key, active);
    if (active) items[slot] = it;
  }
  if (tid == 0) {
    sched[0] = nitem;
    sched[1 + SCHED_NX] = nitem;
  }
  for (int x = tid; x < SCHED_NX; x += PLAN_THREADS) sched[SCHED_CTR * (1 + x)] = 0;
}

}  // namespace

hipError_t launch_plan(const SeqGeom& geo, int batch, int n_kv_heads, const int32_t* head_mask,
                       const Pattern& pat, int BT, int BK, int64_t max_items, int32_t* tile_prefix,
                       int32_t* cost_tmp, WorkItem* items, int32_t* sched, hipStream_t stream) {
  auto launch = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(1), dim3(PLAN_THREADS), 0, stream, geo, batch, n_kv_heads,
                       head_mask, pat, BT, max_items, tile_prefix, cost_tmp, items, sched);
  };
  const bool small = batch <= PLAN_LDS_SEQ && (int64_t)batch * n_kv_heads <= PLAN_LDS_MASK &&
                     max_items <= PLAN_LDS_COST;
  if (BK == BF16_BK)
    small ? launch(plan_kernel<BF16_BK, true>) : launch(plan_kernel<BF16_BK, false>);
  else if (BK == F32_BK)
    small ? launch(plan_kernel<F32_BK, true>) : launch(plan_kernel<F32_BK, false>);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace elastic
