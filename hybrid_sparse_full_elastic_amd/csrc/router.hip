// Attention Router forward on gfx950.
//
// "Elastic Attention" (arXiv 2601.17367; paperlayer summary section 1: the router reads the
// layer's input hidden states and routes head by head; section 3 "Attention Router": pooled
// states pass a task MLP and a router MLP that give one logit per key/value head, and the
// head runs full or sparse attention; appendix H.4 "Router Input Length": boundary pooling
// over the first and last tokens).  Here: h = mean of the pooled rows, z = W1 h,
// logit = W2 relu(z), mask = logit > threshold.
//
// Pooling streams hidden[T, d] once from HBM and dominates the router's time, so it is
// written for bandwidth: many workgroups, each summing a slab of up to ROUTE_SLAB rows of a
// 512-column strip with 16-byte loads (4 waves interleave rows), then fixed-order
// reductions.  No floating-point atomics anywhere: results are bitwise reproducible.
#include "elastic_internal.hpp"

namespace elastic {
namespace {

constexpr int RT = 256;          // threads per workgroup
constexpr int RCOLS = 512;       // columns per pooling workgroup: 64 lanes x 8
constexpr int FIN_COLS = 64;     // columns per finishing workgroup

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct SeqPool {
  int64_t start;  // first token of the sequence
  int n;          // tokens
  int m;          // pooled rows
  int head;       // pooled rows taken from the front (rest from the back)
};

__device__ inline SeqPool seq_pool(const int32_t* cu, int b, int64_t total, int pool_head,
                                   int pool_tail) {
  SeqPool s;
  s.start = cu ? cu[b] : 0;
  s.n = cu ? cu[b + 1] - cu[b] : (int)total;
  if ((pool_head > 0 || pool_tail > 0) && s.n > pool_head + pool_tail) {
    s.m = pool_head + pool_tail;
    s.head = pool_head;
  } else {
    s.m = s.n;
    s.head = s.n;
  }
  return s;
}

// Local row of pooled index p.
__device__ inline int pooled_row(const SeqPool& s, int p) {
  return p < s.head ? p : s.n - s.m + p;
}

// 8 consecutive hidden values as fp32.
__device__ inline void load8(const void* hidden, int dtype, int64_t off, float* x) {
  if (dtype == ELASTIC_BF16) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(hidden) + off);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __uint_as_float(w[e] << 16);
      x[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(hidden) + off);
    const float4 a = p[0], b = p[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

// Partial column sums of one slab: partials[slab, col].
__global__ __launch_bounds__(RT) void route_pool_partial(
    const void* __restrict__ hidden, int dtype, const int32_t* __restrict__ cu, int batch,
    int64_t total, int d, int pool_head, int pool_tail, float* __restrict__ partials) {
  __shared__ float red[3][64][8 + 1];
  const int slab = blockIdx.x;
  int b = -1, slab_in = 0, acc = 0;
  SeqPool s{};
  for (int bb = 0; bb < batch; ++bb) {
    s = seq_pool(cu, bb, total, pool_head, pool_tail);
    const int ns = (s.m + ROUTE_SLAB - 1) / ROUTE_SLAB;
    if (slab < acc + ns) {
      b = bb;
      slab_in = slab - acc;
      break;
    }
    acc += ns;
  }
  if (b < 0) return;  // past the last slab of the batch
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = blockIdx.y * RCOLS + lane * 8;
  const int p0 = slab_in * ROUTE_SLAB;
  const int p1 = min(s.m, p0 + ROUTE_SLAB);
  float sum[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (col < d) {
    int p = p0 + wave;
    for (; p + 12 < p1; p += 16) {  // four rows in flight per lane
      float x[4][8];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        load8(hidden, dtype, (s.start + pooled_row(s, p + 4 * r)) * (int64_t)d + col, x[r]);
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) sum[e] += x[r][e];
    }
    for (; p < p1; p += 4) {
      float x[8];
      load8(hidden, dtype, (s.start + pooled_row(s, p)) * (int64_t)d + col, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) sum[e] += x[e];
    }
  }
  if (wave > 0)
#pragma unroll
    for (int e = 0; e < 8; ++e) red[wave - 1][lane][e] = sum[e];
  __syncthreads();
  if (wave == 0 && col < d) {
#pragma unroll
    for (int w = 0; w < 3; ++w)
#pragma unroll
      for (int e = 0; e < 8; ++e) sum[e] += red[w][lane][e];
    float4* dst = reinterpret_cast<float4*>(partials + (int64_t)slab * d + col);
    dst[0] = make_float4(sum[0], sum[1], sum[2], sum[3]);
    dst[1] = make_float4(sum[4], sum[5], sum[6], sum[7]);
  }
}

// pooled[b, col] = (sum over the slabs of sequence b) / pooled rows.
__global__ __launch_bounds__(RT) void route_pool_finish(
    const float* __restrict__ partials, const int32_t* __restrict__ cu, int batch, int64_t total,
    int d, int pool_head, int pool_tail, float* __restrict__ pooled) {
  __shared__ float red[4][FIN_COLS];
  const int b = blockIdx.x;
  int first = 0;
  for (int bb = 0; bb < b; ++bb) {
    const SeqPool s = seq_pool(cu, bb, total, pool_head, pool_tail);
    first += (s.m + ROUTE_SLAB - 1) / ROUTE_SLAB;
  }
  const SeqPool s = seq_pool(cu, b, total, pool_head, pool_tail);
  const int ns = (s.m + ROUTE_SLAB - 1) / ROUTE_SLAB;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = blockIdx.y * FIN_COLS + lane;
  float sum = 0.f;
  if (col < d) {
    int i = wave;
    for (; i + 12 < ns; i += 16) {
      float x[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = partials[(int64_t)(first + i + 4 * r) * d + col];
#pragma unroll
      for (int r = 0; r < 4; ++r) sum += x[r];
    }
    for (; i < ns; i += 4) sum += partials[(int64_t)(first + i) * d + col];
  }
  red[wave][lane] = sum;
  __syncthreads();
  if (wave == 0 && col < d) {
    const float t = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
    pooled[(int64_t)b * d + col] = s.m > 0 ? t / (float)s.m : 0.f;
  }
}

// z[b, r] = <W1[r, :], pooled[b, :]> for 4 rows r per workgroup.
__global__ __launch_bounds__(RT) void route_mlp1(const float* __restrict__ pooled,
                                                 const float* __restrict__ w1, int d, int d_router,
                                                 float* __restrict__ z) {
  __shared__ float red[4][4];
  const int b = blockIdx.x;
  const int r0 = blockIdx.y * 4;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* h = pooled + (int64_t)b * d;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int c = tid * 4; c < d; c += RT * 4) {  // d is a multiple of 8
    const float4 hv = *reinterpret_cast<const float4*>(h + c);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (r0 + r < d_router) {
        const float4 wv = *reinterpret_cast<const float4*>(w1 + (int64_t)(r0 + r) * d + c);
        acc[r] += wv.x * hv.x + wv.y * hv.y + wv.z * hv.z + wv.w * hv.w;
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float x = acc[r];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    if (lane == 0) red[wave][r] = x;
  }
  __syncthreads();
  if (tid < 4 && r0 + tid < d_router)
    z[(int64_t)b * d_router + r0 + tid] = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
}

// logit[b, g] = <W2[g, :], relu(z[b, :])>; mask = logit > threshold.
__global__ __launch_bounds__(RT) void route_mlp2(const float* __restrict__ z,
                                                 const float* __restrict__ w2, int d_router,
                                                 int n_kv_heads, float threshold,
                                                 float* __restrict__ logits,
                                                 int32_t* __restrict__ mask) {
  const int b = blockIdx.x, g = threadIdx.x;
  if (g >= n_kv_heads) return;
  const float* zb = z + (int64_t)b * d_router;
  const float* wg = w2 + (int64_t)g * d_router;
  float acc = 0.f;
  for (int r = 0; r < d_router; ++r) acc = fmaf(wg[r], fmaxf(zb[r], 0.f), acc);
  if (logits) logits[(int64_t)b * n_kv_heads + g] = acc;
  mask[(int64_t)b * n_kv_heads + g] = acc > threshold ? 1 : 0;
}

}  // namespace

hipError_t launch_route(const void* hidden, int hidden_dtype, const int32_t* cu_seqlens, int batch,
                        int64_t total_tokens, int d_model, int pool_head, int pool_tail,
                        const float* w1, int d_router, const float* w2, int n_kv_heads,
                        float threshold, float* logits_out, int32_t* mask_out, float* partials,
                        int64_t max_slabs, float* pooled, float* zbuf, hipStream_t stream) {
  const int chunks = (d_model + RCOLS - 1) / RCOLS;
  if (max_slabs > 0) {
    hipLaunchKernelGGL(route_pool_partial, dim3((unsigned)max_slabs, chunks), dim3(RT), 0, stream,
                       hidden, hidden_dtype, cu_seqlens, batch, total_tokens, d_model, pool_head,
                       pool_tail, partials);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(route_pool_finish, dim3(batch, (d_model + FIN_COLS - 1) / FIN_COLS), dim3(RT),
                     0, stream, partials, cu_seqlens, batch, total_tokens, d_model, pool_head,
                     pool_tail, pooled);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(route_mlp1, dim3(batch, (d_router + 3) / 4), dim3(RT), 0, stream, pooled, w1,
                     d_model, d_router, zbuf);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(route_mlp2, dim3(batch), dim3(RT), 0, stream, zbuf, w2, d_router, n_kv_heads,
                     threshold, logits_out, mask_out);
  return hipGetLastError();
}

}  // namespace elastic
