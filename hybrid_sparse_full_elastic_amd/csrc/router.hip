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
// 512-column strip with 16-byte loads (4 waves interleave rows, 4 rows in flight per lane).
// Two small kernels finish the mean, the MLP and the threshold.  No floating-point atomics
// anywhere: every sum runs in a fixed order, so results are bitwise reproducible.
#include "elastic_internal.hpp"

namespace elastic {
namespace {

constexpr int RT = 256;          // threads per workgroup
constexpr int RCOLS = 512;       // columns per pooling workgroup: 64 lanes x 8

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

// 8 consecutive hidden values as fp32.  Non-temporal loads: the hidden states are read once,
// so they should not displace cached lines (8% faster pooling at 32K x 4096).
__device__ inline void load8(const void* hidden, int dtype, int64_t off, float* x) {
  if (dtype == ELASTIC_BF16) {
    const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(hidden) + off));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __uint_as_float(w[e] << 16);
      x[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
  } else {
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const float*>(hidden) + off);
    const u32x4 a = __builtin_nontemporal_load(p), b = __builtin_nontemporal_load(p + 1);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = __uint_as_float(a[e]);
      x[4 + e] = __uint_as_float(b[e]);
    }
  }
}

// Partial column sums of one slab: partials[slab, col].
__global__ __launch_bounds__(RT) void route_pool_partial(
    const void* __restrict__ hidden, int dtype, const int32_t* __restrict__ cu, int batch,
    int64_t total, int d, int pool_head, int pool_tail, int slab_rows, float* __restrict__ partials) {
  __shared__ float red[3][64][8 + 1];
  const int slab = blockIdx.x;
  int b = -1, slab_in = 0, acc = 0;
  SeqPool s{};
  for (int bb = 0; bb < batch; ++bb) {
    s = seq_pool(cu, bb, total, pool_head, pool_tail);
    const int ns = (s.m + slab_rows - 1) / slab_rows;
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
  const int p0 = slab_in * slab_rows;
  const int p1 = min(s.m, p0 + slab_rows);
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

// route_strip: workgroup (b, ch) finishes the mean of sequence b over HCOLS columns (the
// sequence's slab partials summed in slab order) and multiplies that strip into every row of
// W1 (partial z).  route_finish (one workgroup per sequence) sums the partial z in strip order,
// applies ReLU and W2 and thresholds the logits.  The kernel boundary makes the partial z
// visible: a completion counter inside one kernel needs a device-scope fence per workgroup,
// which writes back the L2 and measured about 17 us.  All floating-point sums run in a fixed
// order.
constexpr int HCOLS = ROUTE_HCOLS;
constexpr int HT = 1024;          // threads of route_strip: 16 waves split a sequence's slabs
constexpr int HW = HT / 64;

__global__ __launch_bounds__(HT) void route_strip(
    const float* __restrict__ partials, const int32_t* __restrict__ cu, int batch, int64_t total,
    int d, int pool_head, int pool_tail, int slab_rows, const float* __restrict__ w1, int d_router,
    float* __restrict__ zpart) {
  __shared__ float red[HW][HCOLS];
  __shared__ float hbar[HCOLS];
  const int b = blockIdx.x, ch = blockIdx.y, nch = gridDim.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int first = 0;
  for (int bb = 0; bb < b; ++bb) {
    const SeqPool s = seq_pool(cu, bb, total, pool_head, pool_tail);
    first += (s.m + slab_rows - 1) / slab_rows;
  }
  const SeqPool sp = seq_pool(cu, b, total, pool_head, pool_tail);
  const int ns = (sp.m + slab_rows - 1) / slab_rows;
  const int c0 = ch * HCOLS;

  // W1 strip of this workgroup, fetched first so its latency overlaps the partial sums:
  // 4 threads per W1 row, 16 columns each
  const int ncol = min(HCOLS, d - c0);
  const int jrow = tid / 4, q4 = tid & 3;
  float w1r[16];
  if (jrow < d_router) {
    const float* wr = w1 + (int64_t)jrow * d + c0 + q4 * 16;
#pragma unroll
    for (int e = 0; e < 16; ++e) w1r[e] = (q4 * 16 + e < ncol) ? wr[e] : 0.f;
  }

  // 1. mean over the pooled rows for columns [c0, c0 + HCOLS): waves split the slabs, up to
  //    16 slab rows in flight per lane, each wave summing its slabs in increasing order
  const int col = c0 + lane;
  float sum = 0.f;
  if (col < d) {
    for (int i0 = wave; i0 < ns; i0 += 16 * HW) {
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = i0 + HW * r;
        x[r] = i < ns ? partials[(int64_t)(first + i) * d + col] : 0.f;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sum += x[r];
    }
  }
  red[wave][lane] = sum;
  __syncthreads();
  if (wave == 0) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < HW; ++w) t += red[w][lane];
    hbar[lane] = (col < d && sp.m > 0) ? t / (float)sp.m : 0.f;
  }
  __syncthreads();

  // 2. partial z[j] over this strip
  static_assert(HT / 4 >= ROUTE_MAX_DR, "one pass over the W1 rows");
  {
    float acc = 0.f;
    if (jrow < d_router) {
#pragma unroll
      for (int e = 0; e < 16; ++e) acc = fmaf(w1r[e], hbar[q4 * 16 + e], acc);
    }
    acc += __shfl_xor(acc, 1);
    acc += __shfl_xor(acc, 2);
    if (jrow < d_router && q4 == 0) zpart[((int64_t)b * nch + ch) * ROUTE_MAX_DR + jrow] = acc;
  }
}

constexpr int FT = 256;  // threads of route_finish

__global__ __launch_bounds__(FT) void route_finish(const float* __restrict__ zpart, int nch,
                                                   int d_router, const float* __restrict__ w2,
                                                   int n_kv_heads, float threshold,
                                                   float* __restrict__ logits,
                                                   int32_t* __restrict__ mask) {
  __shared__ float zq[4][ROUTE_MAX_DR];
  __shared__ float zs[ROUTE_MAX_DR];
  const int b = blockIdx.x, tid = threadIdx.x;
  // z[j]: 4 threads per row each sum a quarter of the strips in order, then the quarters
  {
    const int q4 = tid & 3, per = (nch + 3) / 4;
    for (int j = tid / 4; j < d_router; j += FT / 4) {
      float z = 0.f;
      const int c1 = min(nch, (q4 + 1) * per);
      for (int cs0 = q4 * per; cs0 < c1; cs0 += 16) {
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r)
          x[r] = cs0 + r < c1 ? zpart[((int64_t)b * nch + cs0 + r) * ROUTE_MAX_DR + j] : 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) z += x[r];
      }
      zq[q4][j] = z;
    }
  }
  __syncthreads();
  for (int j = tid; j < d_router; j += FT) zs[j] = fmaxf(((zq[0][j] + zq[1][j]) + zq[2][j]) + zq[3][j], 0.f);
  __syncthreads();
  for (int gh = tid; gh < n_kv_heads; gh += FT) {
    const float* wg = w2 + (int64_t)gh * d_router;
    float acc = 0.f;
    for (int r = 0; r < d_router; ++r) acc = fmaf(wg[r], zs[r], acc);
    if (logits) logits[(int64_t)b * n_kv_heads + gh] = acc;
    mask[(int64_t)b * n_kv_heads + gh] = acc > threshold ? 1 : 0;
  }
}

}  // namespace

hipError_t launch_route(const void* hidden, int hidden_dtype, const int32_t* cu_seqlens, int batch,
                        int64_t total_tokens, int d_model, int pool_head, int pool_tail,
                        const float* w1, int d_router, const float* w2, int n_kv_heads,
                        float threshold, float* logits_out, int32_t* mask_out, float* partials,
                        int64_t max_slabs, float* zpart, hipStream_t stream) {
  const int chunks = (d_model + RCOLS - 1) / RCOLS;
  // Boundary pooling reads at most pool_head + pool_tail rows per sequence.  Few rows give
  // few slabs, and a 128-row slab is eight dependent load rounds for its workgroup, so such
  // calls use 16-row slabs (one round) whenever the workspace, sized for 128-row slabs of
  // every token, holds them; the grid covers the pooled slabs only.
  int slab_rows = ROUTE_SLAB;
  if (pool_head > 0 || pool_tail > 0) {
    const int64_t pooled = (int64_t)pool_head + pool_tail;
    const int64_t small = (int64_t)batch * ((pooled + 15) / 16);
    if (small <= max_slabs) {
      slab_rows = 16;
      max_slabs = small;
    } else {
      const int64_t per = (pooled + ROUTE_SLAB - 1) / ROUTE_SLAB;
      if ((int64_t)batch * per < max_slabs) max_slabs = (int64_t)batch * per;
    }
  }
  hipLaunchKernelGGL(route_pool_partial, dim3((unsigned)(max_slabs > 0 ? max_slabs : 1), chunks),
                     dim3(RT), 0, stream, hidden, hidden_dtype, cu_seqlens, batch, total_tokens,
                     d_model, pool_head, pool_tail, slab_rows, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nch = (d_model + HCOLS - 1) / HCOLS;
  hipLaunchKernelGGL(route_strip, dim3(batch, nch), dim3(HT), 0, stream, partials, cu_seqlens, batch,
                     total_tokens, d_model, pool_head, pool_tail, slab_rows, w1, d_router, zpart);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(route_finish, dim3(batch), dim3(FT), 0, stream, zpart, nch, d_router, w2,
                     n_kv_heads, threshold, logits_out, mask_out);
  return hipGetLastError();
}

}  // namespace elastic
