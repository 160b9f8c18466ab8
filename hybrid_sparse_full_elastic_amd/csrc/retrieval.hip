// Static retrieval-score head assignment ("Elastic Attention", arXiv 2601.17367; paperlayer
// summary, appendix C.1 "Retrieval Score Calculation" and "Sparsity Assignment"): the pages'
// static baseline ranks heads by how much attention the last token of a probing sequence
// puts on an inserted needle, and keeps the top-ranked heads on full attention.
//
// retrieval_partial: HBM-bound pass over the keys.  Workgroup (key chunk c, KV head g, head
//   slice, sequence b) streams RET_CHUNK keys of head g once with 16-byte loads (a key row of
//   D bf16 values is read by D / 8 lanes) and scores them against the last query of up to
//   RET_HPW query heads of the group (held in LDS as fp32).  Per query head it keeps the
//   online softmax state of the chunk in the exp2 domain: maximum m, sum of weights l over
//   all keys, and over the needle keys ln.
// retrieval_combine: one thread per (sequence, KV head) merges the chunks of its query
//   heads in chunk order, S = ln / l, and averages the G query heads for the KV head.
// assign_kernel: one workgroup ranks the N units (scores) by counting: unit i is full when
//   fewer than k units rank above it (higher score; equal score and lower index; NaN below
//   every number).
#include "elastic_internal.hpp"

namespace elastic {
namespace {

constexpr int RET_THREADS = 256;
constexpr int RET_HPW = 8;  // query heads per workgroup
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

template <typename T, int D>
__device__ inline void load8(const T* p, float (&x)[8]) {
  if constexpr (sizeof(T) == 2) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __uint_as_float(w[e] << 16);
      x[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    x[0] = a.x, x[1] = a.y, x[2] = a.z, x[3] = a.w, x[4] = b.x, x[5] = b.y, x[6] = b.z, x[7] = b.w;
  }
}

// grid: (chunks, n_kv_heads * slices, batch)
template <typename T, int D>
__global__ __launch_bounds__(RET_THREADS) void retrieval_partial(
    const T* __restrict__ q, const T* __restrict__ k, const int32_t* __restrict__ cu,
    int64_t total, int Hq, int Hkv, float scale_log2, const int32_t* __restrict__ needle,
    int chunks, float* __restrict__ part) {
  constexpr int LPK = D / 8;             // lanes per key row
  constexpr int KPW = 64 / LPK;          // keys per wave and step
  constexpr int NW = RET_THREADS / 64;
  __shared__ float qs[RET_HPW][D];
  __shared__ ChunkState red[NW * KPW][RET_HPW];

  const int G = Hq / Hkv;
  const int slices = (G + RET_HPW - 1) / RET_HPW;
  const int g = blockIdx.y / slices, slice = blockIdx.y - g * slices;
  const int h0 = g * G + slice * RET_HPW;
  const int nh = min(RET_HPW, G - slice * RET_HPW);
  const int b = blockIdx.z, c = blockIdx.x;
  const int64_t lo = cu ? cu[b] : 0;
  const int n = (int)((cu ? cu[b + 1] : total) - lo);
  const int j0 = c * RET_CHUNK, j1 = min(n, j0 + RET_CHUNK);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // the last query of the sequence, heads h0 .. h0 + nh - 1, as fp32
  if (n > 0)
    for (int i = tid; i < RET_HPW * D; i += RET_THREADS) {
      const int h = i / D, d = i - h * D;
      float x = 0.f;
      if (h < nh) {
        const T* src = q + ((lo + n - 1) * Hq + h0 + h) * (int64_t)D + d;
        if constexpr (sizeof(T) == 2)
          x = __uint_as_float((uint32_t)(*reinterpret_cast<const uint16_t*>(src)) << 16);
        else
          x = *src;
      }
      qs[h][d] = x;
    }
  __syncthreads();

  const int a = needle ? max(0, needle[2 * b]) : 0, e = needle ? min(n, needle[2 * b + 1]) : 0;
  const int kg = lane / LPK, kl = lane - kg * LPK;  // key slot of the lane, its 8-value part
  ChunkState st[RET_HPW];
#pragma unroll
  for (int h = 0; h < RET_HPW; ++h) st[h] = ChunkState{-__builtin_huge_valf(), 0.f, 0.f};
  float qv[RET_HPW][8];
#pragma unroll
  for (int h = 0; h < RET_HPW; ++h)
#pragma unroll
    for (int t = 0; t < 8; ++t) qv[h][t] = qs[h][kl * 8 + t];

  for (int j = j0 + wave * KPW + kg; j < j1; j += NW * KPW) {
    float kx[8];
    load8<T, D>(k + ((lo + j) * Hkv + g) * (int64_t)D + kl * 8, kx);
    const bool in_needle = j >= a && j < e;
#pragma unroll
    for (int h = 0; h < RET_HPW; ++h) {
      float s = 0.f;
#pragma unroll
      for (int t = 0; t < 8; ++t) s = fmaf(qv[h][t], kx[t], s);
#pragma unroll
      for (int off = LPK / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
      s *= scale_log2;
      // online update of (m, l, ln) with one key
      if (s > st[h].m) {
        const float w = exp2f(st[h].m - s);
        st[h].l *= w;
        st[h].ln *= w;
        st[h].m = s;
      }
      const float p = exp2f(s - st[h].m);
      st[h].l += p;
      if (in_needle) st[h].ln += p;
    }
  }
  // combine the key slots of the workgroup (every lane of a slot holds the same state)
  if (kl == 0)
#pragma unroll
    for (int h = 0; h < RET_HPW; ++h) red[wave * KPW + kg][h] = st[h];
  __syncthreads();
  if (tid < nh) {
    ChunkState acc{-__builtin_huge_valf(), 0.f, 0.f};
    for (int r = 0; r < NW * KPW; ++r) acc = merge(acc, red[r][tid]);
    float* out = part + (((int64_t)b * Hq + h0 + tid) * chunks + c) * 3;
    out[0] = acc.m;
    out[1] = acc.l;
    out[2] = acc.ln;
  }
}

// one thread per (sequence, KV head)
__global__ __launch_bounds__(256) void retrieval_combine(
    const int32_t* __restrict__ cu, int64_t total, int batch, int Hq, int Hkv, int chunks,
    const float* __restrict__ part, float* __restrict__ scores_q, float* __restrict__ scores_kv) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= batch * Hkv) return;
  const int b = t / Hkv, g = t - b * Hkv;
  const int n = (int)(cu ? cu[b + 1] - cu[b] : total);
  const int nc = (n + RET_CHUNK - 1) / RET_CHUNK;
  const int G = Hq / Hkv;
  float sum = 0.f;
  for (int i = 0; i < G; ++i) {
    const int h = g * G + i;
    ChunkState acc{-__builtin_huge_valf(), 0.f, 0.f};
    for (int c = 0; c < nc; ++c) {
      const float* p = part + (((int64_t)b * Hq + h) * chunks + c) * 3;
      acc = merge(acc, ChunkState{p[0], p[1], p[2]});
    }
    const float s = acc.l > 0.f ? acc.ln / acc.l : 0.f;  // an empty sequence scores 0
    if (scores_q) scores_q[(int64_t)b * Hq + h] = s;
    sum += s;
  }
  if (scores_kv) scores_kv[(int64_t)b * Hkv + g] = sum / (float)G;
}

// one workgroup; unit i is full iff fewer than k units rank above it
__global__ __launch_bounds__(1024) void assign_kernel(const float* __restrict__ scores, int n,
                                                      int k, int32_t* __restrict__ mask) {
  for (int i = threadIdx.x; i < n; i += 1024) {
    const float si = scores[i];
    const bool ni = si != si;
    int above = 0;
    for (int j = 0; j < n && above < k; ++j) {
      const float sj = scores[j];
      const bool nj = sj != sj;
      // j ranks above i: a number above NaN; higher score; equal score and lower index
      const bool up = (!nj && ni) || (!nj && !ni && (sj > si || (sj == si && j < i))) ||
                      (nj && ni && j < i);
      above += up ? 1 : 0;
    }
    mask[i] = above < k ? 1 : 0;
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
  const int slices = (G + RET_HPW - 1) / RET_HPW;
  const dim3 grid((unsigned)chunks, (unsigned)(Hkv * slices), (unsigned)batch);
  const float sl2 = scale * RET_LOG2E;
  if (dtype == ELASTIC_BF16) {
    if (head_dim == 128)
      hipLaunchKernelGGL((retrieval_partial<uint16_t, 128>), grid, dim3(RET_THREADS), 0, stream,
                         (const uint16_t*)q, (const uint16_t*)k, cu, total, Hq, Hkv, sl2, needle,
                         chunks, part);
    else
      hipLaunchKernelGGL((retrieval_partial<uint16_t, 64>), grid, dim3(RET_THREADS), 0, stream,
                         (const uint16_t*)q, (const uint16_t*)k, cu, total, Hq, Hkv, sl2, needle,
                         chunks, part);
  } else {
    if (head_dim == 128)
      hipLaunchKernelGGL((retrieval_partial<float, 128>), grid, dim3(RET_THREADS), 0, stream,
                         (const float*)q, (const float*)k, cu, total, Hq, Hkv, sl2, needle, chunks,
                         part);
    else
      hipLaunchKernelGGL((retrieval_partial<float, 64>), grid, dim3(RET_THREADS), 0, stream,
                         (const float*)q, (const float*)k, cu, total, Hq, Hkv, sl2, needle, chunks,
                         part);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int units = batch * Hkv;
  hipLaunchKernelGGL(retrieval_combine, dim3((unsigned)((units + 255) / 256)), dim3(256), 0,
                     stream, cu, total, batch, Hq, Hkv, chunks, part, scores_q, scores_kv);
  return hipGetLastError();
}

hipError_t launch_assign(const float* scores, int n, int k, int32_t* mask, hipStream_t stream) {
  hipLaunchKernelGGL(assign_kernel, dim3(1), dim3(1024), 0, stream, scores, n, k, mask);
  return hipGetLastError();
}

}  // namespace elastic
