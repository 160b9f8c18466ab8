// Static retrieval-score head assignment ("Elastic Attention", arXiv 2601.17367; paperlayer
// summary, appendix C.1 "Retrieval Score Calculation" and "Sparsity Assignment"): the pages'
// static baseline ranks heads by how much attention the last token of a probing sequence
// puts on an inserted needle, and keeps the top-ranked heads on full attention.
//
// retrieval_partial: HBM-bound pass over the keys.  Workgroup (key chunk c, KV head g, head
//   slice, sequence b) streams RET_CHUNK keys of head g once: a lane owns a key row and issues
//   all of the row's 16-byte loads at once, then scores it against the last query of up to
//   8 query heads of the group (bf16: dot2 with exact products and fp32 sums; fp32: FMAs),
//   reading the query from LDS as broadcasts.  The chunk's scores go to LDS; then one wave
//   per query head forms the chunk's softmax state in the exp2 domain: maximum m, sum of
//   weights l over all keys, and over the needle keys ln.
// retrieval_combine: one workgroup per (sequence, KV head) merges the chunks of each query
//   head (lanes over chunks, a fixed butterfly across lanes), S = ln / l, and averages the G
//   query heads in head order for the KV head.
// assign_kernel: ranks the N units (scores, staged in LDS by every workgroup) by counting, one
//   wave per unit: unit i is full when fewer than k units rank above it (higher score; equal
//   score and lower index; NaN below every number).
#include <algorithm>
#include <type_traits>

#include "elastic_internal.hpp"

namespace elastic {
namespace {

constexpr int RET_THREADS = 256;
constexpr float RET_LOG2E = 1.4426950408889634f;

struct ChunkState {
  float m, l, ln;
};

__device__ inline ChunkState merge(ChunkState a, ChunkState b) {
  const float m = fmaxf(a.m, b.m);
  if (m == -__builtin_huge_valf()) return a;  // both empty
  const float wa = exp2f(a.m - m), wb = exp2f(b.m - m);
  return ChunkState{m, a.l * wa + b.l * wb, a.ln * wa + b.ln * wb};
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// grid: (chunks, n_kv_heads * slices, batch).  Pass 1: each thread scores one key row (the
// row's 16-byte loads all in flight, the NH query heads read from LDS as broadcasts) into
// LDS; pass 2 reduces each head's scores to (m, l, ln), one wave per head.
template <typename T, int D, int NH>
__global__ __launch_bounds__(RET_THREADS) void retrieval_partial(
    const T* __restrict__ q, const T* __restrict__ k, const int32_t* __restrict__ cu,
    int64_t total, int Hq, int Hkv, float scale_log2, const int32_t* __restrict__ needle,
    int chunks, float* __restrict__ part) {
  constexpr bool BF = sizeof(T) == 2;
  constexpr int SEG = D / 8;             // 8-value segments of a row
  __shared__ __attribute__((aligned(16))) T qs[NH][D];  // the last query, input precision
  __shared__ float sc[NH][RET_CHUNK];   // scores of the chunk, log2 domain

  const int G = Hq / Hkv;
  const int slices = (G + NH - 1) / NH;
  const int g = blockIdx.y / slices, slice = blockIdx.y - g * slices;
  const int h0 = g * G + slice * NH;
  const int nh = min(NH, G - slice * NH);
  const int b = blockIdx.z, c = blockIdx.x;
  const int64_t lo = cu ? cu[b] : 0;
  const int n = (int)((cu ? cu[b + 1] : total) - lo);
  const int j0 = c * RET_CHUNK, j1 = min(n, j0 + RET_CHUNK);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // pass 1: one key row per thread (the chunk is one row per thread).  The row's loads are
  // issued first, so they are in flight while the query is staged.
  static_assert(RET_CHUNK == RET_THREADS, "one key row per thread");
  const int j = j0 + tid;
  uint4 kr[BF ? SEG : 2 * SEG];
  if (j < j1) {
    const uint4* row = reinterpret_cast<const uint4*>(k + ((lo + j) * Hkv + g) * (int64_t)D);
#pragma unroll
    for (int s = 0; s < (BF ? SEG : 2 * SEG); ++s) kr[s] = row[s];
  }
  // the last query of the sequence, heads h0 .. h0 + nh - 1 (zero past nh)
  for (int i = tid; i < NH * D; i += RET_THREADS) {
    const int h = i / D, d = i - h * D;
    T x = T(0);
    if (h < nh && n > 0) x = q[((lo + n - 1) * Hq + h0 + h) * (int64_t)D + d];
    qs[h][d] = x;
  }
  __syncthreads();
  if (j < j1) {
    float acc[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) acc[h] = 0.f;
#pragma unroll
    for (int s = 0; s < SEG; ++s) {
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        if constexpr (BF) {
          // 8 bf16 of the row against 8 bf16 of the query: four exact-product dot2 steps
          const uint4 qq = *reinterpret_cast<const uint4*>(&qs[h][s * 8]);
          const uint32_t kw[4] = {kr[s].x, kr[s].y, kr[s].z, kr[s].w};
          const uint32_t qw[4] = {qq.x, qq.y, qq.z, qq.w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[h] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, kw[e]),
                                                     __builtin_bit_cast(bf16x2_t, qw[e]), acc[h],
                                                     false);
        } else {
          const float4 q0 = *reinterpret_cast<const float4*>(&qs[h][s * 8]);
          const float4 q1 = *reinterpret_cast<const float4*>(&qs[h][s * 8 + 4]);
          const float4 k0 = __builtin_bit_cast(float4, kr[2 * s]);
          const float4 k1 = __builtin_bit_cast(float4, kr[2 * s + 1]);
          float a = acc[h];
          a = fmaf(q0.x, k0.x, a), a = fmaf(q0.y, k0.y, a), a = fmaf(q0.z, k0.z, a);
          a = fmaf(q0.w, k0.w, a), a = fmaf(q1.x, k1.x, a), a = fmaf(q1.y, k1.y, a);
          a = fmaf(q1.z, k1.z, a), a = fmaf(q1.w, k1.w, a);
          acc[h] = a;
        }
      }
    }
#pragma unroll
    for (int h = 0; h < NH; ++h) sc[h][j - j0] = acc[h] * scale_log2;
  }
  __syncthreads();

  // pass 2: per query head, m = max, l = sum 2^(s - m), ln = the same over the needle
  constexpr int NW = RET_THREADS / 64;
  const int a = needle ? max(0, needle[2 * b]) : 0, e = needle ? min(n, needle[2 * b + 1]) : 0;
  const int nk = j1 - j0;
  for (int h = wave; h < nh; h += NW) {
    float m = -__builtin_huge_valf();
    for (int i = lane; i < nk; i += 64) m = fmaxf(m, sc[h][i]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    float l = 0.f, ln = 0.f;
    if (nk > 0)
      for (int i = lane; i < nk; i += 64) {
        const float p = exp2f(sc[h][i] - m);
        l += p;
        const int j = j0 + i;
        if (j >= a && j < e) ln += p;
      }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      l += __shfl_xor(l, off, 64);
      ln += __shfl_xor(ln, off, 64);
    }
    if (lane == 0) {
      float* out = part + (((int64_t)b * Hq + h0 + h) * chunks + c) * 3;
      out[0] = m;
      out[1] = l;
      out[2] = ln;
    }
  }
}

// one workgroup per (sequence, KV head): wave per query head, lanes over chunks (merged in a
// fixed butterfly order), then the mean over the G query heads in head order
__global__ __launch_bounds__(RET_THREADS) void retrieval_combine(
    const int32_t* __restrict__ cu, int64_t total, int Hq, int Hkv, int chunks,
    const float* __restrict__ part, float* __restrict__ scores_q, float* __restrict__ scores_kv) {
  constexpr int NW = RET_THREADS / 64;
  __shared__ float s_head[RET_MAX_G];
  const int b = blockIdx.x / Hkv, g = blockIdx.x - b * Hkv;
  const int n = (int)(cu ? cu[b + 1] - cu[b] : total);
  const int nc = (n + RET_CHUNK - 1) / RET_CHUNK;
  const int G = Hq / Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = wave; i < G; i += NW) {
    const int h = g * G + i;
    ChunkState acc{-__builtin_huge_valf(), 0.f, 0.f};
    for (int c = lane; c < nc; c += 64) {
      const float* p = part + (((int64_t)b * Hq + h) * chunks + c) * 3;
      acc = merge(acc, ChunkState{p[0], p[1], p[2]});
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const ChunkState o{__shfl_xor(acc.m, off, 64), __shfl_xor(acc.l, off, 64),
                         __shfl_xor(acc.ln, off, 64)};
      acc = (lane & off) ? merge(o, acc) : merge(acc, o);  // same operand order on both lanes
    }
    if (lane == 0) {
      const float s = acc.l > 0.f ? acc.ln / acc.l : 0.f;  // an empty sequence scores 0
      if (scores_q) scores_q[(int64_t)b * Hq + h] = s;
      s_head[i] = s;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0 && scores_kv) {
    float sum = 0.f;
    for (int i = 0; i < G; ++i) sum += s_head[i];
    scores_kv[(int64_t)b * Hkv + g] = sum / (float)G;
  }
}

// Unit i is full iff fewer than k units rank above it.  Every workgroup stages all n scores
// in LDS; each wave ranks one unit at a time (the grid's waves stride over the units), its 64
// lanes splitting the n comparisons, and adds the counts across the wave.  (One workgroup
// doing all n^2 comparisons took 12.9 us for 256 units, bound by one CU's VALU.)
constexpr int ASSIGN_THREADS = 256;
__global__ __launch_bounds__(ASSIGN_THREADS) void assign_kernel(const float* __restrict__ scores,
                                                                int n, int k,
                                                                int32_t* __restrict__ mask) {
  __shared__ float s_sc[ELASTIC_ASSIGN_MAX_UNITS];
  for (int i = threadIdx.x; i < n; i += ASSIGN_THREADS) s_sc[i] = scores[i];
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int waves = (int)gridDim.x * (ASSIGN_THREADS / 64);
  for (int i = (int)blockIdx.x * (ASSIGN_THREADS / 64) + (int)(threadIdx.x >> 6); i < n; i += waves) {
    const float si = s_sc[i];
    const bool ni = si != si;
    int above = 0;
    for (int j = lane; j < n; j += 64) {
      const float sj = s_sc[j];
      const bool nj = sj != sj;
      // j ranks above i: a number above NaN; higher score; equal score and lower index
      const bool up = (!nj && ni) || (!nj && !ni && (sj > si || (sj == si && j < i))) ||
                      (nj && ni && j < i);
      above += up ? 1 : 0;
    }
    for (int off = 32; off >= 1; off >>= 1) above += __shfl_xor(above, off, 64);
    if (lane == 0) mask[i] = above < k ? 1 : 0;
  }
}

}  // namespace

int64_t retrieval_chunks(int32_t max_seqlen) {
  return max_seqlen > 0 ? (max_seqlen + RET_CHUNK - 1) / RET_CHUNK : 1;
}

hipError_t launch_retrieval(int dtype, int head_dim, const void* q, const void* k,
                            const int32_t* cu, int64_t total, int batch, int max_seqlen, int Hq,
                            int Hkv, float scale, const int32_t* needle, float* part,
                            float* scores_q, float* scores_kv, hipStream_t stream) {
  const int chunks = (int)retrieval_chunks(max_seqlen);
  const int G = Hq / Hkv;
  const int nh = G >= 8 ? 8 : (G >= 4 ? 4 : (G >= 2 ? 2 : 1));  // query heads per workgroup
  const int slices = (G + nh - 1) / nh;
  const dim3 grid((unsigned)chunks, (unsigned)(Hkv * slices), (unsigned)batch);
  const float sl2 = scale * RET_LOG2E;
  auto go = [&](auto kernel, auto* qp, auto* kp) {
    hipLaunchKernelGGL(kernel, grid, dim3(RET_THREADS), 0, stream, qp, kp, cu, total, Hq, Hkv, sl2,
                       needle, chunks, part);
  };
  auto by_heads = [&](auto tag, auto dtag) {
    using T = decltype(tag);
    constexpr int D = decltype(dtag)::value;
    const T* qp = static_cast<const T*>(q);
    const T* kp = static_cast<const T*>(k);
    if (nh == 8) go(retrieval_partial<T, D, 8>, qp, kp);
    else if (nh == 4) go(retrieval_partial<T, D, 4>, qp, kp);
    else if (nh == 2) go(retrieval_partial<T, D, 2>, qp, kp);
    else go(retrieval_partial<T, D, 1>, qp, kp);
  };
  using D128 = std::integral_constant<int, 128>;
  using D64 = std::integral_constant<int, 64>;
  if (dtype == ELASTIC_BF16) {
    if (head_dim == 128) by_heads(uint16_t{}, D128{});
    else by_heads(uint16_t{}, D64{});
  } else {
    if (head_dim == 128) by_heads(float{}, D128{});
    else by_heads(float{}, D64{});
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(retrieval_combine, dim3((unsigned)(batch * Hkv)), dim3(RET_THREADS), 0, stream,
                     cu, total, Hq, Hkv, chunks, part, scores_q, scores_kv);
  return hipGetLastError();
}

hipError_t launch_assign(const float* scores, int n, int k, int32_t* mask, hipStream_t stream) {
  const int units_per_wg = ASSIGN_THREADS / 64;
  const int grid = std::min((n + units_per_wg - 1) / units_per_wg, 1024);
  hipLaunchKernelGGL(assign_kernel, dim3((unsigned)std::max(grid, 1)), dim3(ASSIGN_THREADS), 0, stream,
                     scores, n, k, mask);
  return hipGetLastError();
}

}  // namespace elastic
