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
// 512-column strip with 16-byte loads, waves interleaving rows; the workgroup shape follows
// the number of slabs (launch_route).  One small kernel finishes the mean, the MLP and the
// threshold.  No floating-point atomics anywhere: every sum runs in a fixed order, so results
// are bitwise reproducible.
#include "elastic_internal.hpp"

namespace elastic {
namespace {

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

// Slabs of slab_rows pooled rows in sequence b.
__device__ inline int seq_slabs(const int32_t* cu, int b, int64_t total, int pool_head,
                                int pool_tail, int slab_rows) {
  const SeqPool s = seq_pool(cu, b, total, pool_head, pool_tail);
  return (s.m + slab_rows - 1) / slab_rows;
}

// The sequence holding global slab `slab` and the slab's index inside it (mode 0), or the
// first global slab of sequence `slab` (mode 1).  Up to 64 sequences: a plain walk.  Larger
// packed batches: 64 sequences per step across the lanes of each wave (every wave computes the
// same, so no LDS is involved), O(batch / 64) steps instead of one per sequence.
__device__ inline void find_slab(const int32_t* cu, int batch, int64_t total, int pool_head,
                                 int pool_tail, int slab_rows, int slab, bool first_of_seq,
                                 int* seq_out, int* idx_out) {
  if (batch <= 64) {
    int acc = 0;
    for (int bb = 0; bb < batch; ++bb) {
      const int ns = seq_slabs(cu, bb, total, pool_head, pool_tail, slab_rows);
      if (first_of_seq ? bb == slab : slab < acc + ns) {
        *seq_out = bb;
        *idx_out = first_of_seq ? acc : slab - acc;
        return;
      }
      acc += ns;
    }
    *seq_out = -1;
    *idx_out = 0;
    return;
  }
  const int lane = threadIdx.x & 63;
  int acc = 0;
  for (int base = 0; base < batch; base += 64) {
    const int bb = base + lane;
    const int ns = bb < batch ? seq_slabs(cu, bb, total, pool_head, pool_tail, slab_rows) : 0;
    int incl = ns;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    const int excl = incl - ns;
    if (first_of_seq) {
      if (slab >= base && slab < base + 64) {
        *seq_out = slab;
        *idx_out = __builtin_amdgcn_readfirstlane(acc + __shfl(excl, slab - base, 64));
        return;
      }
    } else {
      const uint64_t hit = __ballot(bb < batch && slab >= acc + excl && slab < acc + incl);
      if (hit != 0) {
        const int l = __ffsll((unsigned long long)hit) - 1;
        *seq_out = base + l;
        *idx_out = __builtin_amdgcn_readfirstlane(slab - acc - __shfl(excl, l, 64));
        return;
      }
    }
    acc += __builtin_amdgcn_readfirstlane(__shfl(incl, 63, 64));
  }
  *seq_out = -1;
  *idx_out = 0;
}

// Adds 8 consecutive hidden values, held as loaded (bf16: one 16-byte word; fp32: two), to
// sum.  The loads are non-temporal: the hidden states are read once, so they should not
// displace cached lines (8% faster pooling at 32K x 4096).
__device__ inline u32x4 load16(const void* base, int64_t byte_off) {
  return __builtin_nontemporal_load(
      reinterpret_cast<const u32x4*>(static_cast<const char*>(base) + byte_off));
}
__device__ inline void add_bf16x8(float* sum, const u32x4 w) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    sum[2 * e] += __uint_as_float(w[e] << 16);
    sum[2 * e + 1] += __uint_as_float(w[e] & 0xffff0000u);
  }
}
__device__ inline void add_f32x4(float* sum, const u32x4 w) {
#pragma unroll
  for (int e = 0; e < 4; ++e) sum[e] += __uint_as_float(w[e]);
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

// Partial column sums of one slab: partials[slab, col], 4 waves interleaving the slab's rows
// with four rows in flight per lane (many slabs: about eight such workgroups per CU stream).
__global__ __launch_bounds__(256) void route_pool_partial(
    const void* __restrict__ hidden, int dtype, const int32_t* __restrict__ cu, int batch,
    int64_t total, int d, int pool_head, int pool_tail, int slab_rows, float* __restrict__ partials,
    int32_t* __restrict__ done) {
  __shared__ float red[3][64][8 + 1];
  if (blockIdx.x == 0 && blockIdx.y == 0)  // route_strip's completion counters
    for (int i = threadIdx.x; i < batch; i += blockDim.x) done[i] = 0;
  const int slab = blockIdx.x;
  int b, slab_in;
  find_slab(cu, batch, total, pool_head, pool_tail, slab_rows, slab, false, &b, &slab_in);
  if (b < 0) return;  // past the last slab of the batch (uniform)
  const SeqPool s = seq_pool(cu, b, total, pool_head, pool_tail);
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

// The same sums with 8 waves, every lane issuing the loads of all its rows of the slab (up to
// 16) before adding any, so a slab is one round of loads (few slabs: one or two workgroups per
// CU, whose rounds would otherwise each wait a full memory latency).  DT: the hidden dtype.
template <int DT>
__global__ __launch_bounds__(512) void route_pool_partial_1r(
    const void* __restrict__ hidden, const int32_t* __restrict__ cu, int batch, int64_t total,
    int d, int pool_head, int pool_tail, int slab_rows, float* __restrict__ partials,
    int32_t* __restrict__ done) {
  constexpr int RW = 8, RIF = 16;
  constexpr bool BF = DT == ELASTIC_BF16;
  constexpr int esz = BF ? 2 : 4;
  __shared__ float red[RW - 1][64][8 + 1];
  if (blockIdx.x == 0 && blockIdx.y == 0)  // route_strip's completion counters
    for (int i = threadIdx.x; i < batch; i += blockDim.x) done[i] = 0;
  const int slab = blockIdx.x;
  int b, slab_in;
  find_slab(cu, batch, total, pool_head, pool_tail, slab_rows, slab, false, &b, &slab_in);
  if (b < 0) return;  // past the last slab of the batch (uniform)
  const SeqPool s = seq_pool(cu, b, total, pool_head, pool_tail);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = blockIdx.y * RCOLS + lane * 8;
  const int p0 = slab_in * slab_rows;
  const int p1 = min(s.m, p0 + slab_rows);
  float sum[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto row_off = [&](int p) { return ((s.start + pooled_row(s, p)) * (int64_t)d + col) * esz; };
  if (col < d) {
    // rows p0 + wave, + RW, + 2 RW, ...: the raw words of all the lane's rows in flight at once
    // (rows past the slab read nothing and add zero), added in increasing order
    for (int pb = p0 + wave; pb < p1; pb += RIF * RW) {
      if constexpr (BF) {
        u32x4 x[RIF];
#pragma unroll
        for (int r = 0; r < RIF; ++r) {
          const int p = pb + RW * r;
          x[r] = p < p1 ? load16(hidden, row_off(p)) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int r = 0; r < RIF; ++r) add_bf16x8(sum, x[r]);
      } else {
        u32x4 x[RIF / 2][2];  // fp32 rows are twice as wide: half as many per round
        for (int ph = pb; ph < pb + RIF * RW && ph < p1; ph += RIF / 2 * RW) {
#pragma unroll
          for (int r = 0; r < RIF / 2; ++r) {
            const int p = ph + RW * r;
            x[r][0] = p < p1 ? load16(hidden, row_off(p)) : u32x4{0u, 0u, 0u, 0u};
            x[r][1] = p < p1 ? load16(hidden, row_off(p) + 16) : u32x4{0u, 0u, 0u, 0u};
          }
#pragma unroll
          for (int r = 0; r < RIF / 2; ++r) {
            add_f32x4(sum, x[r][0]);
            add_f32x4(sum + 4, x[r][1]);
          }
        }
      }
    }
  }
  if (wave > 0)
#pragma unroll
    for (int e = 0; e < 8; ++e) red[wave - 1][lane][e] = sum[e];
  __syncthreads();
  if (wave == 0 && col < d) {
#pragma unroll
    for (int w = 0; w < RW - 1; ++w)
#pragma unroll
      for (int e = 0; e < 8; ++e) sum[e] += red[w][lane][e];
    float4* dst = reinterpret_cast<float4*>(partials + (int64_t)slab * d + col);
    dst[0] = make_float4(sum[0], sum[1], sum[2], sum[3]);
    dst[1] = make_float4(sum[4], sum[5], sum[6], sum[7]);
  }
}

// route_strip: workgroup (b, ch) finishes the mean of sequence b over HCOLS columns (the
// sequence's slab partials summed in slab order) and multiplies that strip into every row of
// W1 (partial z).  The last of the sequence's nch workgroups to finish -- a completion count
// per sequence, zeroed by the pooling kernel -- then sums the partial z in strip order, applies
// ReLU and W2 and thresholds the logits.  One device-scope release per workgroup makes its
// partial z visible (64 workgroups per sequence at d = 4096, each with 256 bytes to write
// back; a count over the pooling kernel's workgroups, each with a slab of partial sums, cost
// about 17 us).  All floating-point sums run in a fixed order.
constexpr int HCOLS = ROUTE_HCOLS;
constexpr int HT = 1024;          // threads of route_strip: 16 waves split a sequence's slabs
constexpr int HW = HT / 64;

// Sequence b's logits and mask from its partial z: z[j] as 4 fixed quarters of the strips,
// each summed in strip order, then the quarters in order; ReLU, W2, threshold.  The whole
// workgroup (NT threads) calls it.
template <int NT>
__device__ void finish_seq(const float* __restrict__ zpart, int b, int nch, int d_router,
                           const float* __restrict__ w2, int n_kv_heads, float threshold,
                           float* __restrict__ logits, int32_t* __restrict__ mask,
                           float (&zq)[4][ROUTE_MAX_DR], float (&zs)[ROUTE_MAX_DR]) {
  const int tid = threadIdx.x;
  {
    const int q4 = tid & 3, per = (nch + 3) / 4;
    for (int j = tid / 4; j < d_router; j += NT / 4) {
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
  for (int j = tid; j < d_router; j += NT) zs[j] = fmaxf(((zq[0][j] + zq[1][j]) + zq[2][j]) + zq[3][j], 0.f);
  __syncthreads();
  for (int gh = tid; gh < n_kv_heads; gh += NT) {
    const float* wg = w2 + (int64_t)gh * d_router;
    float acc = 0.f;
    for (int r = 0; r < d_router; ++r) acc = fmaf(wg[r], zs[r], acc);
    if (logits) logits[(int64_t)b * n_kv_heads + gh] = acc;
    mask[(int64_t)b * n_kv_heads + gh] = acc > threshold ? 1 : 0;
  }
}

__global__ __launch_bounds__(HT) void route_strip(
    const float* __restrict__ partials, const int32_t* __restrict__ cu, int batch, int64_t total,
    int d, int pool_head, int pool_tail, int slab_rows, const float* __restrict__ w1, int d_router,
    float* __restrict__ zpart, int32_t* __restrict__ done, const float* __restrict__ w2,
    int n_kv_heads, float threshold, float* __restrict__ logits, int32_t* __restrict__ mask) {
  __shared__ float red[HW][HCOLS];
  __shared__ float hbar[HCOLS];
  __shared__ float zq[4][ROUTE_MAX_DR];
  __shared__ float zs[ROUTE_MAX_DR];
  __shared__ int last;
  const int b = blockIdx.x, ch = blockIdx.y, nch = gridDim.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int first, seq;
  find_slab(cu, batch, total, pool_head, pool_tail, slab_rows, b, true, &seq, &first);
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

  // 3. the sequence's last workgroup finishes it.  The barrier orders every wave's partial z
  //    before thread 0's device-scope release; the acquire after the count orders the other
  //    workgroups' partial z before this workgroup's reads.
  __syncthreads();
  if (tid == 0) {
    __threadfence();
    const int prior = atomicAdd(done + b, 1);
    if (prior == nch - 1) __threadfence();
    last = prior == nch - 1;
  }
  __syncthreads();
  if (!last) return;  // uniform
  finish_seq<HT>(zpart, b, nch, d_router, w2, n_kv_heads, threshold, logits, mask, zq, zs);
}

}  // namespace

hipError_t launch_route(const void* hidden, int hidden_dtype, const int32_t* cu_seqlens, int batch,
                        int64_t total_tokens, int d_model, int pool_head, int pool_tail,
                        const float* w1, int d_router, const float* w2, int n_kv_heads,
                        float threshold, float* logits_out, int32_t* mask_out, float* partials,
                        int64_t max_slabs, float* zpart, int32_t* done, hipStream_t stream) {
  const int chunks = (d_model + RCOLS - 1) / RCOLS;
  // Boundary pooling reads at most pool_head + pool_tail rows per sequence: the grid covers
  // those slabs only.
  int slab_rows = ROUTE_SLAB;
  if (pool_head > 0 || pool_tail > 0) {
    const int64_t per = ((int64_t)pool_head + pool_tail + ROUTE_SLAB - 1) / ROUTE_SLAB;
    if ((int64_t)batch * per < max_slabs) max_slabs = (int64_t)batch * per;
  }
  // Pooling shape: few slabs (a short batch, boundary pooling) leave most CUs one or two
  // workgroups, so each reads its whole slab in one round (8 waves x 16 rows in flight per
  // lane: 8K x 4096 pools in 13 us instead of 22); many slabs keep about eight small
  // workgroups per CU streaming (4 waves x 4 rows in flight: 6.4 TB/s at 32K x 4096, where the
  // one-round shape measured 20% slower).
  const unsigned nslab = (unsigned)(max_slabs > 0 ? max_slabs : 1);
  if ((int64_t)nslab * chunks <= 1024) {
    auto pool = [&](auto kernel) {
      hipLaunchKernelGGL(kernel, dim3(nslab, chunks), dim3(512), 0, stream, hidden, cu_seqlens,
                         batch, total_tokens, d_model, pool_head, pool_tail, slab_rows, partials, done);
    };
    if (hidden_dtype == ELASTIC_BF16) pool(route_pool_partial_1r<ELASTIC_BF16>);
    else pool(route_pool_partial_1r<ELASTIC_FP32>);
  } else {
    hipLaunchKernelGGL(route_pool_partial, dim3(nslab, chunks), dim3(256), 0, stream, hidden,
                       hidden_dtype, cu_seqlens, batch, total_tokens, d_model, pool_head, pool_tail,
                       slab_rows, partials, done);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nch = (d_model + HCOLS - 1) / HCOLS;
  hipLaunchKernelGGL(route_strip, dim3(batch, nch), dim3(HT), 0, stream, partials, cu_seqlens, batch,
                     total_tokens, d_model, pool_head, pool_tail, slab_rows, w1, d_router, zpart,
                     done, w2, n_kv_heads, threshold, logits_out, mask_out);
  return hipGetLastError();
}

}  // namespace elastic
