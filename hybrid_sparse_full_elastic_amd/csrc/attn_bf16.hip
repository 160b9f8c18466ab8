// Hybrid-head GQA prefill attention, bf16 in/out, on gfx950 MFMA.
//
// Method ("Elastic Attention", arXiv 2601.17367; paperlayer summary section 2 "Hybrid Head
// Mechanism", section 3 "Efficient Deployment", appendix D.1 "Sparse Inference"): every KV
// head runs either causal full attention or a sparse pattern (sink + local window streaming,
// or a fixed block pattern), in one launch fed by the routing mask; head outputs are
// concatenated into o[T, Hq, D].
//
// Design for CDNA4:
//  * One workgroup = one work item: a query tile of BT tokens times all G query heads of one
//    KV head (rows r = token * G + head, so the K/V tile staged in LDS serves the whole GQA
//    group), 4 waves, each wave owning 2 blocks of 32 query rows.
//  * S^T = K . Q^T with v_mfma_f32_32x32x16_bf16: every lane holds one query column, so the
//    softmax row statistics are per-lane; only one cross-half swap (v_permlane32_swap) per
//    tile is needed for the maximum.  Q stays in registers for the whole item.
//  * O^T = V^T . P^T: P^T comes straight from the S^T accumulators (bf16) with a fixed
//    key-slot permutation; V is stored transposed in LDS with the same permutation, so the
//    rescale of O by the running maximum is a per-lane multiply.
//  * Online softmax in the exp2 domain with the softmax scale and log2(e) folded into one
//    multiply; fp32 accumulation throughout; masks are evaluated only on tiles that cross a
//    causal, sink, window or block boundary, and tiles no query of the item may see are
//    never loaded (streaming items cost O(sink + window), not O(n)).
//  * K/V tiles are double-buffered in LDS; the next tile's global loads are in flight while
//    the current tile is multiplied.
#include "elastic_internal.hpp"

namespace elastic {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float LN2 = 0.69314718055994530942f;

// x[lane] combined with x[lane ^ 32] by `op`; the swap returns both halves' values.
__device__ inline float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D>
__global__ __launch_bounds__(BF16_NW * 64, 1) void attn_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, float* __restrict__ lse, const int32_t* __restrict__ cu_seqlens,
    int64_t total_tokens, int Hq, int Hkv, int G, int BT, float scale_log2,
    const int32_t* __restrict__ head_mask, Pattern pat, const WorkItem* __restrict__ items,
    const int32_t* __restrict__ n_items) {
  constexpr int NW = BF16_NW, NB = BF16_NB, BK = BF16_BK, NT = NW * 64;
  constexpr int DC = D / 16;   // 16-wide d chunks of Q.K^T
  constexpr int DB = D / 32;   // 32-row d blocks of O^T
  constexpr int KST = D + 8;   // K tile row stride in LDS (elements), breaks bank conflicts
  constexpr int VST = BK + 4;  // V^T tile row stride in LDS (elements)
  constexpr int KCH = BK * D / 8 / NT;                  // 16-byte K chunks per thread
  constexpr int VUNITS = (BK / 4) * (D / 8);            // (4 keys x 8 d) V units per tile
  constexpr int VPT = (VUNITS + NT - 1) / NT;           // V units per thread
  static_assert(KCH * NT * 8 == BK * D, "K tile split");

  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][BK * KST];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][D * VST];

  if ((int)blockIdx.x >= *n_items) return;
  const WorkItem it = items[blockIdx.x];
  const int64_t seq0 = cu_seqlens ? cu_seqlens[it.seq] : 0;
  const int n = cu_seqlens ? cu_seqlens[it.seq + 1] - (int)seq0 : (int)total_tokens;
  const int t0 = it.qtile * BT;
  const int t1 = min(t0 + BT, n) - 1;
  const int g = it.group;
  const bool full = head_mask == nullptr || head_mask[it.seq * Hkv + g] != 0;
  const int mode = full ? MODE_FULL : pat.kind;
  const KeyTiles tiles(mode, pat, t0, t1, BK);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int64_t kv_row = (int64_t)Hkv * D;  // elements between consecutive tokens of k / v
  const uint16_t* kbase = k + seq0 * kv_row + (int64_t)g * D;
  const uint16_t* vbase = v + seq0 * kv_row + (int64_t)g * D;

  // ---- this lane's query rows: r = token * G + head inside the item
  int qi[NB], qhead[NB];
  bool qvalid[NB];
  bf16x8 qreg[NB][DC];
#pragma unroll
  for (int qb = 0; qb < NB; ++qb) {
    const int r = (wave * NB + qb) * 32 + l32;
    const int tl = r / G;
    const int hh = r - tl * G;
    qi[qb] = t0 + tl;
    qhead[qb] = g * G + hh;
    qvalid[qb] = tl < BT && qi[qb] <= t1;
    if (qvalid[qb]) {
      const u32x4* src = reinterpret_cast<const u32x4*>(
          q + ((seq0 + qi[qb]) * Hq + qhead[qb]) * (int64_t)D + half * 8);
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) qreg[qb][dc] = __builtin_bit_cast(bf16x8, src[dc * 2]);
    } else {
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) qreg[qb][dc] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
    }
  }

  // ---- K/V tile staging (global -> registers -> LDS; V transposed to V^T)
  u32x4 kreg[KCH];
  u32x4 vreg[VPT][4];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      const int idx = tid + c * NT;
      const int row = idx / (D / 8), col8 = idx % (D / 8);
      const int key = kt * BK + row;
      kreg[c] = key < n ? *reinterpret_cast<const u32x4*>(kbase + key * kv_row + col8 * 8)
                        : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int idx = tid + u * NT;
      const int kq = idx / (D / 8), d8 = idx % (D / 8);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = kt * BK + kq * 4 + r;
        vreg[u][r] = (idx < VUNITS && key < n)
                         ? *reinterpret_cast<const u32x4*>(vbase + key * kv_row + d8 * 8)
                         : u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      const int idx = tid + c * NT;
      const int row = idx / (D / 8), col8 = idx % (D / 8);
      *reinterpret_cast<u32x4*>(&k_lds[buf][row * KST + col8 * 8]) = kreg[c];
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int idx = tid + u * NT;
      if (idx < VUNITS) {
        const int kq = idx / (D / 8), d8 = idx % (D / 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int w = e >> 1, sh = (e & 1) * 16;
          const uint32_t x0 = (vreg[u][0][w] >> sh) & 0xffffu, x1 = (vreg[u][1][w] >> sh) & 0xffffu;
          const uint32_t x2 = (vreg[u][2][w] >> sh) & 0xffffu, x3 = (vreg[u][3][w] >> sh) & 0xffffu;
          *reinterpret_cast<u32x2*>(&v_lds[buf][(d8 * 8 + e) * VST + kq * 4]) =
              u32x2{x0 | (x1 << 16), x2 | (x3 << 16)};
        }
      }
    }
  };

  // ---- running state
  f32x16 oacc[DB][NB];
  float m_run[NB], l_run[NB];
#pragma unroll
  for (int qb = 0; qb < NB; ++qb) {
    m_run[qb] = -1.0e30f;  // finite: a fully masked first tile leaves alpha = 1, p = 0
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[db][qb][e] = 0.f;
  }

  int kt = tiles.next(0);
  int buf = 0;
  if (kt >= 0) {
    load_tile(kt);
    store_tile(0);
  }
  while (kt >= 0) {
    const int nkt = tiles.next(kt + 1);
    if (nkt >= 0) load_tile(nkt);
    __syncthreads();

    // S^T[key, query] for two 32-key blocks x NB 32-query blocks
    f32x16 sacc[2][NB];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < NB; ++qb)
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[kb][qb][e] = 0.f;
    const uint16_t* ks = &k_lds[buf][0];
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      bf16x8 a[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        a[kb] = *reinterpret_cast<const bf16x8*>(ks + (kb * 32 + l32) * KST + dc * 16 + half * 8);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < NB; ++qb)
          sacc[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kb], qreg[qb][dc], sacc[kb][qb], 0, 0, 0);
    }

    // online softmax (exp2 domain); P^T packed to bf16 in MFMA B-operand order
    const bool masked = tiles.needs_mask(kt);
    bf16x8 pop[2][2][NB];
#pragma unroll
    for (int qb = 0; qb < NB; ++qb) {
      float mt = -__builtin_huge_valf();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float x = sacc[kb][qb][e] * scale_log2;
          if (masked) {
            const int j = kt * BK + kb * 32 + (e >> 2) * 8 + half * 4 + (e & 3);
            if (!qvalid[qb] || !key_allowed(mode, pat, qi[qb], j)) x = -__builtin_huge_valf();
          }
          sacc[kb][qb][e] = x;
          mt = fmaxf(mt, x);
        }
      mt = half_max(mt);
      const float m_new = fmaxf(m_run[qb], mt);
      const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_new);
      m_run[qb] = m_new;
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = __builtin_amdgcn_exp2f(sacc[kb][qb][e] - m_new);
          ls += p;
          pop[kb][e >> 3][qb][e & 7] = (__bf16)p;
        }
      l_run[qb] = l_run[qb] * alpha + ls;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][qb][e] *= alpha;
    }

    // O^T[d, query] += V^T[d, key] . P^T[key, query]
    const uint16_t* vs = &v_lds[buf][0];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const uint16_t* row = vs + (db * 32 + l32) * VST + kb * 32 + c * 16 + half * 4;
          const u32x2 lo = *reinterpret_cast<const u32x2*>(row);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(row + 8);
          const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
          for (int qb = 0; qb < NB; ++qb)
            oacc[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pop[kb][c][qb], oacc[db][qb], 0, 0, 0);
        }

    if (nkt >= 0) store_tile(buf ^ 1);
    buf ^= 1;
    kt = nkt;
  }

  // ---- epilogue: normalise, store bf16 O (and the natural-log LSE)
#pragma unroll
  for (int qb = 0; qb < NB; ++qb) {
    const float lt = half_sum(l_run[qb]);
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    if (!qvalid[qb]) continue;
    uint16_t* dst = o + ((seq0 + qi[qb]) * Hq + qhead[qb]) * (int64_t)D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int ig = 0; ig < 4; ++ig) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (__bf16)(oacc[db][qb][ig * 4 + e] * inv);
        *reinterpret_cast<u32x2*>(dst + db * 32 + ig * 8 + half * 4) = __builtin_bit_cast(u32x2, w);
      }
    if (lse != nullptr && half == 0)
      lse[(int64_t)qhead[qb] * total_tokens + seq0 + qi[qb]] = (m_run[qb] + __log2f(lt)) * LN2;
  }
}

}  // namespace

hipError_t launch_attn_bf16(int head_dim, const void* q, const void* k, const void* v, void* o,
                            float* lse, const int32_t* cu_seqlens, int64_t total_tokens,
                            int n_q_heads, int n_kv_heads, int BT, float scale,
                            const int32_t* head_mask, const Pattern& pat, const WorkItem* items,
                            const int32_t* n_items, int64_t grid, hipStream_t stream) {
  const float scale_log2 = scale * 1.4426950408889634f;
  const int G = n_q_heads / n_kv_heads;
  const dim3 block(BF16_NW * 64);
  if (grid <= 0) return hipSuccess;
  if (head_dim == 128) {
    hipLaunchKernelGGL(attn_bf16_kernel<128>, dim3((unsigned)grid), block, 0, stream,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, lse,
                       cu_seqlens, total_tokens, n_q_heads, n_kv_heads, G, BT, scale_log2,
                       head_mask, pat, items, n_items);
  } else {
    hipLaunchKernelGGL(attn_bf16_kernel<64>, dim3((unsigned)grid), block, 0, stream,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, lse,
                       cu_seqlens, total_tokens, n_q_heads, n_kv_heads, G, BT, scale_log2,
                       head_mask, pat, items, n_items);
  }
  return hipGetLastError();
}

}  // namespace elastic
