// Hybrid-head GQA prefill attention in true fp32 (inputs, products, softmax and output).
//
// Same semantics and work list as the bf16 MFMA kernel ("Elastic Attention", arXiv
// 2601.17367; paperlayer summary section 2 "Hybrid Head Mechanism", appendix D.1 "Sparse
// Inference"), for callers that need fp32 accuracy.  One thread owns one query row
// (token, head) of the item and keeps q and the output accumulator in registers; the
// workgroup's rows are the G heads of BT tokens, so every K/V tile staged in LDS is read by
// all G heads of the group with broadcast (conflict-free) LDS reads.  Scores of a 32-key
// tile are formed first, then one online-softmax update per tile (exp2 domain).
#include <type_traits>

#include "elastic_internal.hpp"

namespace elastic {
namespace {

constexpr float LN2 = 0.69314718055994530942f;

template <int D>
__global__ __launch_bounds__(F32_ROWS, 1) void attn_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, float* __restrict__ lse, SeqGeom geo, int Hq, int Hkv, int G, int BT,
    float scale_log2, Pattern pat,
    const WorkItem* __restrict__ items, int32_t* sched) {
  constexpr int BK = F32_BK, NT = F32_ROWS;
  constexpr int CH = BK * D / 4;  // float4 chunks per tile
  __shared__ __attribute__((aligned(16))) float k_lds[BK * D];
  __shared__ __attribute__((aligned(16))) float v_lds[BK * D];
  __shared__ uint32_t list_vis[LIST_MAX_KB];  // block lists: visibility of each key block

  // one item per workgroup, claimed from the XCD's queue (or another); the grid has at least
  // as many workgroups as items, so every item is claimed
  __shared__ int s_claim;
  if (threadIdx.x == 0) s_claim = claim_item(sched);
  __syncthreads();
  if (s_claim < 0) return;
  const WorkItem it = items[s_claim];
  // queries at absolute positions sp.qp + t, keys at k_pos + j
  const SeqSpan sp = seq_span(geo, it.seq);
  const int64_t seq0 = sp.q0;
  const int n = sp.nq;
  const int t0 = it.qtile * BT;
  const int t1 = min(t0 + BT, n) - 1;
  const int g = it.group;
  const bool full = it.full != 0;
  const int mode = full ? MODE_FULL : pat.kind;
  const int k_end = geo.k_pos + sp.nk;

  const int tid = threadIdx.x;
  const int tl = tid / G, hh = tid - (tid / G) * G;
  const int qi = t0 + tl;
  const int qabs = sp.qp + qi;
  const int head = g * G + hh;
  const bool valid = tl < BT && qi <= t1;
  const int64_t kv_row = (int64_t)Hkv * D;

  float qr[D], acc[D];
  if (valid) {
    const float4* src = reinterpret_cast<const float4*>(q + ((seq0 + qi) * Hq + head) * (int64_t)D);
#pragma unroll
    for (int c = 0; c < D / 4; ++c) {
      const float4 x = src[c];
      qr[4 * c] = x.x; qr[4 * c + 1] = x.y; qr[4 * c + 2] = x.z; qr[4 * c + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int d = 0; d < D; ++d) qr[d] = 0.f;
  }
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = 0.f;
  float m_run = -1.0e30f, l_run = 0.f;

  const int blk_shift = 31 - __clz(pat.block);  // block sizes are powers of two
  // key tiles: closed forms, or the block lists marked in LDS (one loop for both)
  const bool LIST = mode == MODE_LIST;
  struct {
    bool list;
    KeyTiles kt;
    ListTiles lt;
    __device__ int next(int x) const { return list ? lt.next(x) : kt.next(x); }
    __device__ bool needs_mask(int x) const { return list ? lt.needs_mask(x) : kt.needs_mask(x); }
  } tiles{LIST, KeyTiles(LIST ? MODE_FULL : mode, pat, sp.qp + t0, sp.qp + t1, BK, geo.k_pos, k_end),
          LIST ? list_tiles(list_vis, pat, it.seq, g, Hkv, sp.qp + t0, sp.qp + t1, geo.k_pos, k_end, BK, tid, NT)
               : ListTiles{}};
  for (int kt = tiles.next(0); kt >= 0; kt = tiles.next(kt + 1)) {
    __syncthreads();  // previous tile fully consumed
    for (int c = tid; c < CH; c += NT) {
      const int row = c / (D / 4), c4 = c % (D / 4);
      const int key = kt * BK + row;  // absolute; row key - k_pos of the sequence's keys
      float4 kx = make_float4(0.f, 0.f, 0.f, 0.f), vx = kx;
      if (key < k_end) {
        const int64_t kr = sp.k0 + (key - geo.k_pos);
        kx = *reinterpret_cast<const float4*>(k + kr * kv_row + (int64_t)g * D + c4 * 4);
        vx = *reinterpret_cast<const float4*>(v + kr * kv_row + (int64_t)g * D + c4 * 4);
      }
      *reinterpret_cast<float4*>(&k_lds[row * D + c4 * 4]) = kx;
      *reinterpret_cast<float4*>(&v_lds[row * D + c4 * 4]) = vx;
    }
    __syncthreads();

    const bool masked = tiles.needs_mask(kt);
    bool row_sees_block = true;  // block lists: does this row's query block list the tile's block?
    if (LIST) {
      const int bit = (qabs >> blk_shift) - tiles.lt.qb0;
      row_sees_block = bit >= 0 && bit < LIST_MAX_QB && ((tiles.lt.vis_of(kt) >> bit) & 1u);
    }
    float s[BK];
    float mt = -__builtin_huge_valf();
#pragma unroll
    for (int j = 0; j < BK; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) dot = fmaf(qr[d], k_lds[j * D + d], dot);
      float x = dot * scale_log2;
      const int kj = kt * BK + j;
      const bool ok = LIST ? (row_sees_block && kj <= qabs) : key_allowed(mode, pat, qabs, kj);
      if (masked && (!valid || kj >= k_end || !ok)) x = -__builtin_huge_valf();
      s[j] = x;
      mt = fmaxf(mt, x);
    }
    const float m_new = fmaxf(m_run, mt);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] *= alpha;
#pragma unroll
    for (int j = 0; j < BK; ++j) {
      const float p = __builtin_amdgcn_exp2f(s[j] - m_new);
      l_run += p;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = fmaf(p, v_lds[j * D + d], acc[d]);
    }
  }

  if (!valid) return;
  const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
  float4* dst = reinterpret_cast<float4*>(o + ((seq0 + qi) * Hq + head) * (int64_t)D);
#pragma unroll
  for (int c = 0; c < D / 4; ++c)
    dst[c] = make_float4(acc[4 * c] * inv, acc[4 * c + 1] * inv, acc[4 * c + 2] * inv, acc[4 * c + 3] * inv);
  if (lse != nullptr)  // log of an empty sum is -inf
    lse[(int64_t)head * geo.total_q + seq0 + qi] = (m_run + __log2f(l_run)) * LN2;
}

}  // namespace

hipError_t launch_attn_f32(int head_dim, const void* q, const void* k, const void* v, void* o,
                           float* lse, const SeqGeom& geo, int n_q_heads, int n_kv_heads, int BT,
                           float scale, const Pattern& pat,
                           const WorkItem* items, int32_t* sched, int64_t grid,
                           hipStream_t stream) {
  const float scale_log2 = scale * 1.4426950408889634f;
  const int G = n_q_heads / n_kv_heads;
  if (grid <= 0) return hipSuccess;
  if (head_dim == 128) {
    hipLaunchKernelGGL(attn_f32_kernel<128>, dim3((unsigned)grid), dim3(F32_ROWS), 0, stream,
                       (const float*)q, (const float*)k, (const float*)v, (float*)o, lse, geo,
                       n_q_heads, n_kv_heads, G, BT, scale_log2, pat, items, sched);
  } else {
    hipLaunchKernelGGL(attn_f32_kernel<64>, dim3((unsigned)grid), dim3(F32_ROWS), 0, stream,
                       (const float*)q, (const float*)k, (const float*)v, (float*)o, lse, geo,
                       n_q_heads, n_kv_heads, G, BT, scale_log2, pat, items, sched);
  }
  return hipGetLastError();
}

}  // namespace elastic
