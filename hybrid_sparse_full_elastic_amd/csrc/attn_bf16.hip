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
//    group), NW waves each owning NB blocks of 32 query rows.  The shipped configuration is
//    8 waves x 1 block (256 rows): every wave fits in 256 VGPRs, so two waves share a SIMD and
//    one wave's MFMAs overlap the other's softmax.
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
//  * Software pipeline per tile j: Q.K^T of tile j+1 is issued while exp2 of tile j runs,
//    and P.V of tile j while tile j+1 is masked and reduced to its maximum.  The running
//    maximum is raised lazily (only when a tile exceeds it by 2^8), so O is almost never
//    rescaled.  K is staged two tiles ahead and V one tile ahead in double-buffered LDS
//    slots; global loads run one more tile ahead in registers; one barrier per tile.
#include "elastic_internal.hpp"

namespace elastic {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

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
struct LdsTiles {
  // Row strides in elements.  K rows: +8 spreads a wave's 16-byte row reads over all banks.
  // V rows: +32 makes the four key rows of one transposing read start 16 banks apart, so
  // each half-wave of ds_read_b64_tr_b16 touches every bank exactly once.
  static constexpr int KST = D + 8;
  static constexpr int VST = D + 32;
  uint16_t k[2][BF16_BK * KST];
  uint16_t v[2][BF16_BK * VST];
};

// max of three floats in one instruction (the inputs are never NaN here)
__device__ inline float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// One work item with its mode known at compile time.
template <int D, int NW, int NB, int MODE>
__device__ __forceinline__ void attn_item(
    const WorkItem& it, LdsTiles<D>& lds, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
    float* __restrict__ lse, const int32_t* __restrict__ cu_seqlens, int64_t total_tokens, int Hq,
    int Hkv, int G, int BT, float scale_log2, const Pattern& pat) {
  constexpr int BK = BF16_BK, NT = NW * 64;
  constexpr int DC = D / 16;   // 16-wide d chunks of Q.K^T
  constexpr int DB = D / 32;   // 32-row d blocks of O^T
  constexpr int KST = LdsTiles<D>::KST, VST = LdsTiles<D>::VST;
  constexpr int KCH = (BK * D / 8 + NT - 1) / NT;       // 16-byte K chunks per thread
  // Lazy rescaling: the running maximum is only raised when a tile's maximum exceeds it by
  // more than 2^SLACK, so p = exp2(s - m) stays <= 2^SLACK and O is rarely rescaled.
  constexpr float SLACK = 8.0f;
  static_assert((BK * D / 8) % NT == 0 || NT > BK * D / 8, "K tile split");

  auto& k_lds = lds.k;
  auto& v_lds = lds.v;
  const int64_t seq0 = cu_seqlens ? cu_seqlens[it.seq] : 0;
  const int n = cu_seqlens ? cu_seqlens[it.seq + 1] - (int)seq0 : (int)total_tokens;
  const int t0 = it.qtile * BT;
  const int t1 = min(t0 + BT, n) - 1;
  const int g = it.group;
  constexpr int mode = MODE;
  const KeyTilesT<MODE> tiles(MODE, pat, t0, t1, BK);
  const int blk_shift = 31 - __clz(pat.block);  // block sizes are powers of two

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int64_t kv_row = (int64_t)Hkv * D;  // elements between consecutive tokens of k / v
  const uint16_t* kbase = k + seq0 * kv_row + (int64_t)g * D;
  const uint16_t* vbase = v + seq0 * kv_row + (int64_t)g * D;
  const float c = scale_log2;
  // source address of this lane in a transposing V read: key (l/4) + 4*half of the 16-key
  // chunk, columns (group parity)*16 + 4*(l%4) of the 32-column d block
  const int v_lane_off = ((lane & 15) / 4 + 4 * half) * VST + ((lane >> 4) & 1) * 16 + 4 * (lane & 3);

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

  // ---- K/V tile staging: global -> registers -> LDS, both row-major [key][d]
  u32x4 kreg[KCH];
  u32x4 vreg[KCH];
  // Raw buffer loads: a per-tile descriptor covers only the tile's rows that exist in the
  // sequence, so rows past its end read as zero without branches.
  auto tile_rsrc = [&](const uint16_t* base, int kt) {
    const int rows = min(n - kt * BK, BK);
    return __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(base + (int64_t)kt * BK * kv_row), (short)0,
        rows * (int)kv_row * 2, 0x00020000);
  };
  auto load_tile = [&](const uint16_t* base, int kt, u32x4 (&reg)[KCH]) {
    const auto rs = tile_rsrc(base, kt);
#pragma unroll
    for (int cc = 0; cc < KCH; ++cc) {
      const int idx = tid + cc * NT;
      const int row = idx / (D / 8), col8 = idx % (D / 8);
      if (idx < BK * D / 8)
        reg[cc] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (row * (int)kv_row + col8 * 8) * 2, 0, 0));
    }
  };
  auto load_k = [&](int kt) { load_tile(kbase, kt, kreg); };
  auto load_v = [&](int kt) { load_tile(vbase, kt, vreg); };
  auto store_tile = [&](uint16_t* dst, int stride, const u32x4 (&reg)[KCH]) {
#pragma unroll
    for (int cc = 0; cc < KCH; ++cc) {
      const int idx = tid + cc * NT;
      const int row = idx / (D / 8), col8 = idx % (D / 8);
      if (idx < BK * D / 8) *reinterpret_cast<u32x4*>(dst + row * stride + col8 * 8) = reg[cc];
    }
  };
  auto store_k = [&](int buf) { store_tile(&k_lds[buf][0], KST, kreg); };
  auto store_v = [&](int buf) { store_tile(&v_lds[buf][0], VST, vreg); };

  // ---- S^T[key, query] = K . Q^T for the two 32-key halves of a tile
  auto qk = [&](int buf, f32x16 (&s)[2][NB]) {
    const uint16_t* ks = &k_lds[buf][0];
    const f32x16 zero = {};
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
          s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kb], qreg[qb][dc],
                                                             dc == 0 ? zero : s[kb][qb], 0, 0, 0);
    }
  };

  // ---- masks: allowed(j) = j <= hi && (j < a || j >= b), exact per (query, key)
  int qblk[NB];
#pragma unroll
  for (int qb = 0; qb < NB; ++qb) qblk[qb] = qi[qb] >> blk_shift;
  auto apply_mask = [&](f32x16 (&s)[2][NB], int kt) {
    const int kblk = (kt * BK) >> blk_shift;  // one key block per tile (block % BK == 0)
    const bool kvis_static = kblk < pat.sink_blocks ||
                             (pat.stride_blocks > 0 && kblk % pat.stride_blocks == 0);
#pragma unroll
    for (int qb = 0; qb < NB; ++qb) {
      const int i = qi[qb];
      const int hi = qvalid[qb] ? i : -1;
      int a = 0, b = 0;
      if (mode == MODE_STREAM) {
        a = pat.sink;
        b = i - pat.window + 1;
      } else if (mode == MODE_BLOCK) {
        b = (kvis_static || qblk[qb] - kblk <= pat.local_blocks) ? 0 : 0x7fffffff;
      }
      const int base = kt * BK + half * 4;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int j = base + kb * 32 + (e >> 2) * 8 + (e & 3);
          const bool ok = j <= hi && (j < a || j >= b);
          if (!ok) s[kb][qb][e] = -__builtin_huge_valf();
        }
    }
  };
  auto tile_max = [&](f32x16 (&s)[2][NB], float (&mt)[NB]) {
#pragma unroll
    for (int qb = 0; qb < NB; ++qb) {
      float m0 = max3f(s[0][qb][0], s[1][qb][0], s[0][qb][1]);
      float m1 = max3f(s[1][qb][1], s[0][qb][2], s[1][qb][2]);
#pragma unroll
      for (int e = 3; e < 15; e += 2) {
        m0 = max3f(m0, s[0][qb][e], s[1][qb][e]);
        m1 = max3f(m1, s[0][qb][e + 1], s[1][qb][e + 1]);
      }
      mt[qb] = half_max(max3f(m0, m1, max3f(s[0][qb][15], s[1][qb][15], m0)));
    }
  };

  // ---- running state (m in the scaled log2 domain)
  f32x16 oacc[DB][NB];
  float m_sc[NB], l_run[NB], alpha[NB];
#pragma unroll
  for (int qb = 0; qb < NB; ++qb) {
    m_sc[qb] = -1.0e30f;  // finite: fully masked tiles give p = 0 and never raise it
    l_run[qb] = 0.f;
    alpha[qb] = 1.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[db][qb][e] = 0.f;
  }
  bool pending = false;  // wave-uniform: O and l wait for a multiply by alpha

  // Raise the running maximum for the scores in s (raw, masked); decide the rescale.
  auto update_max = [&](f32x16 (&s)[2][NB]) {
    float mt[NB];
    tile_max(s, mt);
    bool need = false;
    float mn[NB];
#pragma unroll
    for (int qb = 0; qb < NB; ++qb) {
      const float ms = mt[qb] * c;
      need |= ms > m_sc[qb] + SLACK;
      mn[qb] = fmaxf(m_sc[qb], ms);
    }
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
      for (int qb = 0; qb < NB; ++qb) {
        alpha[qb] = __builtin_amdgcn_exp2f(m_sc[qb] - mn[qb]);
        m_sc[qb] = mn[qb];
      }
      pending = true;
    }
  };

  // ---- tile schedule: kt_cur = tile j, kt_n1 = j+1, kt_n2 = j+2
  int kt_cur = tiles.next(0);
  if (kt_cur < 0) return;  // cannot happen: the diagonal tile is always visited
  int kt_n1 = tiles.next(kt_cur + 1);
  int kt_n2 = kt_n1 >= 0 ? tiles.next(kt_n1 + 1) : -1;

  // prologue: tile 0 (K and V) and K of tile 1 into LDS; registers hold K_2 and V_1
  load_k(kt_cur);
  load_v(kt_cur);
  store_k(0);
  store_v(0);
  if (kt_n1 >= 0) {
    load_k(kt_n1);
    load_v(kt_n1);
    store_k(1);
  }
  if (kt_n2 >= 0) load_k(kt_n2);
  __syncthreads();
  f32x16 s0[2][NB], s1[2][NB];
  qk(0, s0);
  __syncthreads();  // every wave is done with K slot 0 before it is refilled
  if (tiles.needs_mask(kt_cur)) apply_mask(s0, kt_cur);
  update_max(s0);
  pending = false;  // O and l are still zero
  int slot = 0;

  // One pipelined step on tile j: Q.K^T of tile j+1 and exp of tile j, then P.V of tile j
  // and the mask / maximum of tile j+1; LDS refills of K_{j+2} and V_{j+1}; global loads of
  // K_{j+3} and V_{j+2}; one barrier.
  auto step = [&](f32x16 (&sc)[2][NB], f32x16 (&sn)[2][NB]) {
    if (pending) {
#pragma unroll
      for (int qb = 0; qb < NB; ++qb) {
        l_run[qb] *= alpha[qb];
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) oacc[db][qb][e] *= alpha[qb];
      }
      pending = false;
    }
    const bool has_next = kt_n1 >= 0;
    // phase A: S_{j+1} (MFMA) while p_j = exp2(c s_j - m) (VALU)
    qk(slot ^ 1, sn);
    bf16x8 pop[2][2][NB];
    float lsum4[NB][4];
#pragma unroll
    for (int qb = 0; qb < NB; ++qb) {
      lsum4[qb][0] = lsum4[qb][1] = lsum4[qb][2] = lsum4[qb][3] = 0.f;
      const float nm = -m_sc[qb];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sc[kb][qb][e], c, nm));
          lsum4[qb][e & 3] += p;
          pop[kb][e >> 3][qb][e & 7] = (__bf16)p;
        }
    }
    // phase B: O^T += V^T P^T (MFMA) while l += sum p and the next tile's max (VALU)
    // V^T A-operands straight from the row-major V tile: ds_read_b64_tr_b16 hands lane
    // (16-lane group gr, index l) V[key_i][dbase + l] for the four keys key_i its group's
    // source lanes point at; two reads give the 8 key slots of the MFMA lane.
    const uint16_t* vs = &v_lds[slot][0] + v_lane_off;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const uint16_t* src = vs + (kb * 32 + cc * 16) * VST + db * 32;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(src));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(src + 8 * VST));
          const bf16x8 a = __builtin_bit_cast(
              bf16x8, s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
#pragma unroll
          for (int qb = 0; qb < NB; ++qb)
            oacc[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pop[kb][cc][qb], oacc[db][qb], 0, 0, 0);
        }
#pragma unroll
    for (int qb = 0; qb < NB; ++qb)
      l_run[qb] += (lsum4[qb][0] + lsum4[qb][1]) + (lsum4[qb][2] + lsum4[qb][3]);
    if (has_next) {
      if (tiles.needs_mask(kt_n1)) apply_mask(sn, kt_n1);
      update_max(sn);
    }
    if (kt_n2 >= 0) store_k(slot);
    if (has_next) store_v(slot ^ 1);
    const int kt_n3 = kt_n2 >= 0 ? tiles.next(kt_n2 + 1) : -1;
    if (kt_n3 >= 0) load_k(kt_n3);
    if (kt_n2 >= 0) load_v(kt_n2);
    __syncthreads();
    kt_cur = kt_n1;
    kt_n1 = kt_n2;
    kt_n2 = kt_n3;
    slot ^= 1;
  };

  while (true) {
    step(s0, s1);
    if (kt_cur < 0) break;
    step(s1, s0);
    if (kt_cur < 0) break;
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
      lse[(int64_t)qhead[qb] * total_tokens + seq0 + qi[qb]] = (m_sc[qb] + __log2f(lt)) * LN2;
  }
}

template <int D, int NW, int NB>
__global__ __launch_bounds__(NW * 64, 1) void attn_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, float* __restrict__ lse, const int32_t* __restrict__ cu_seqlens,
    int64_t total_tokens, int Hq, int Hkv, int G, int BT, float scale_log2,
    const int32_t* __restrict__ head_mask, Pattern pat, const WorkItem* __restrict__ items,
    const int32_t* __restrict__ n_items) {
  __shared__ __attribute__((aligned(16))) LdsTiles<D> lds;
  if ((int)blockIdx.x >= *n_items) return;
  const WorkItem it = items[blockIdx.x];
  const bool full = head_mask == nullptr || head_mask[it.seq * Hkv + it.group] != 0;
  if (full)
    attn_item<D, NW, NB, MODE_FULL>(it, lds, q, k, v, o, lse, cu_seqlens, total_tokens, Hq, Hkv, G,
                                    BT, scale_log2, pat);
  else if (pat.kind == ELASTIC_SPARSE_STREAMING)
    attn_item<D, NW, NB, MODE_STREAM>(it, lds, q, k, v, o, lse, cu_seqlens, total_tokens, Hq, Hkv,
                                      G, BT, scale_log2, pat);
  else
    attn_item<D, NW, NB, MODE_BLOCK>(it, lds, q, k, v, o, lse, cu_seqlens, total_tokens, Hq, Hkv,
                                     G, BT, scale_log2, pat);
}

}  // namespace

template <int D, int NW, int NB>
static void launch_cfg(int64_t grid, hipStream_t stream, const void* q, const void* k, const void* v,
                       void* o, float* lse, const int32_t* cu_seqlens, int64_t total_tokens,
                       int n_q_heads, int n_kv_heads, int G, int BT, float scale_log2,
                       const int32_t* head_mask, const Pattern& pat, const WorkItem* items,
                       const int32_t* n_items) {
  hipLaunchKernelGGL((attn_bf16_kernel<D, NW, NB>), dim3((unsigned)grid), dim3(NW * 64), 0, stream,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, lse,
                     cu_seqlens, total_tokens, n_q_heads, n_kv_heads, G, BT, scale_log2, head_mask,
                     pat, items, n_items);
}

hipError_t launch_attn_bf16(int head_dim, const void* q, const void* k, const void* v, void* o,
                            float* lse, const int32_t* cu_seqlens, int64_t total_tokens,
                            int n_q_heads, int n_kv_heads, int BT, float scale,
                            const int32_t* head_mask, const Pattern& pat, const WorkItem* items,
                            const int32_t* n_items, int64_t grid, hipStream_t stream) {
  const float scale_log2 = scale * 1.4426950408889634f;
  const int G = n_q_heads / n_kv_heads;
  if (grid <= 0) return hipSuccess;
  if (head_dim == 128)
    launch_cfg<128, BF16_NW, BF16_NB>(grid, stream, q, k, v, o, lse, cu_seqlens, total_tokens,
                                      n_q_heads, n_kv_heads, G, BT, scale_log2, head_mask, pat,
                                      items, n_items);
  else
    launch_cfg<64, BF16_NW, BF16_NB>(grid, stream, q, k, v, o, lse, cu_seqlens, total_tokens,
                                     n_q_heads, n_kv_heads, G, BT, scale_log2, head_mask, pat,
                                     items, n_items);
  return hipGetLastError();
}

}  // namespace elastic
