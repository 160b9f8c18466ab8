// Merge of two partial attention results over disjoint key sets, by their log-sum-exp.
//
// Prefill in query chunks and key ranges ("Elastic Attention", arXiv 2601.17367; paperlayer
// summary, appendix D.1 "Sparse Inference": prefill chunks of 16,384 queries) splits one
// softmax over several calls.  For a row with partial results (o_a, lse_a) and (o_b, lse_b):
//   lse = log(e^lse_a + e^lse_b),   o = e^(lse_a - lse) o_a + e^(lse_b - lse) o_b,
// and a row that saw no key at all (lse = -inf on both sides) stays o = 0, lse = -inf.
//
// HBM-bound elementwise pass: each lane owns 8 consecutive values of one (row, head) pair, so
// a wave reads and writes whole rows with 16-byte accesses (bf16) and the pair's two lse
// values are broadcast loads.  Every pair is handled by the lanes of one wave only, which
// read both lse values before any of them writes, so the outputs may alias the inputs.
#include "elastic_internal.hpp"

namespace elastic {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int MT = 256;  // threads per workgroup

__device__ inline void weights(float a, float b, float& wa, float& wb, float& lse) {
  const float m = fmaxf(a, b);
  if (m == -__builtin_huge_valf()) {  // neither side saw a key (NaN inputs fall through)
    wa = wb = 0.f;
    lse = m;
    return;
  }
  const float ea = expf(a - m), eb = expf(b - m);
  const float s = ea + eb;
  wa = ea / s;
  wb = eb / s;
  lse = m + logf(s);
}

// bf16: one lane = 8 values (16 bytes) of one (row, head) pair.
__global__ __launch_bounds__(MT) void lse_merge_bf16(
    const uint16_t* oa, const float* la, const uint16_t* ob,
    const float* lb, uint16_t* oo, float* lo, int64_t rows, int heads, int D) {
  const int cpr = D / 8;  // lanes per pair
  const int64_t t = (int64_t)blockIdx.x * MT + threadIdx.x;
  const int64_t pair = t / cpr;
  if (pair >= rows * heads) return;
  const int c = (int)(t - pair * cpr);
  const int64_t row = pair / heads;
  const int head = (int)(pair - row * heads);
  const int64_t li = (int64_t)head * rows + row;
  float wa, wb, lse;
  weights(la[li], lb[li], wa, wb, lse);
  // the partial results are read once: non-temporal loads (5% faster at 32K x 32 heads)
  const u32x4 xa = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(oa + pair * D + c * 8));
  const u32x4 xb = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ob + pair * D + c * 8));
  u32x4 y;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a0 = __uint_as_float(xa[e] << 16), a1 = __uint_as_float(xa[e] & 0xffff0000u);
    const float b0 = __uint_as_float(xb[e] << 16), b1 = __uint_as_float(xb[e] & 0xffff0000u);
    const float r0 = fmaf(wa, a0, wb * b0), r1 = fmaf(wa, a1, wb * b1);
    const __bf16 h0 = (__bf16)r0, h1 = (__bf16)r1;  // round to nearest even
    y[e] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
  }
  *reinterpret_cast<u32x4*>(oo + pair * D + c * 8) = y;
  if (c == 0) lo[li] = lse;
}

// fp32: one lane = 4 values (16 bytes) of one (row, head) pair.
__global__ __launch_bounds__(MT) void lse_merge_f32(
    const float* oa, const float* la, const float* ob,
    const float* lb, float* oo, float* lo, int64_t rows, int heads, int D) {
  const int cpr = D / 4;
  const int64_t t = (int64_t)blockIdx.x * MT + threadIdx.x;
  const int64_t pair = t / cpr;
  if (pair >= rows * heads) return;
  const int c = (int)(t - pair * cpr);
  const int64_t row = pair / heads;
  const int head = (int)(pair - row * heads);
  const int64_t li = (int64_t)head * rows + row;
  float wa, wb, lse;
  weights(la[li], lb[li], wa, wb, lse);
  const u32x4 xa = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(oa + pair * D + c * 4));
  const u32x4 xb = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ob + pair * D + c * 4));
  float4 y;
  y.x = fmaf(wa, __uint_as_float(xa[0]), wb * __uint_as_float(xb[0]));
  y.y = fmaf(wa, __uint_as_float(xa[1]), wb * __uint_as_float(xb[1]));
  y.z = fmaf(wa, __uint_as_float(xa[2]), wb * __uint_as_float(xb[2]));
  y.w = fmaf(wa, __uint_as_float(xa[3]), wb * __uint_as_float(xb[3]));
  *reinterpret_cast<float4*>(oo + pair * D + c * 4) = y;
  if (c == 0) lo[li] = lse;
}

}  // namespace

hipError_t launch_lse_merge(int dtype, const void* o_a, const float* lse_a, const void* o_b,
                            const float* lse_b, void* o_out, float* lse_out, int64_t rows,
                            int heads, int head_dim, hipStream_t stream) {
  const int per = dtype == ELASTIC_BF16 ? 8 : 4;
  const int64_t lanes = rows * heads * (head_dim / per);
  if (lanes <= 0) return hipSuccess;
  const dim3 grid((unsigned)((lanes + MT - 1) / MT));
  if (dtype == ELASTIC_BF16)
    hipLaunchKernelGGL(lse_merge_bf16, grid, dim3(MT), 0, stream, (const uint16_t*)o_a, lse_a,
                       (const uint16_t*)o_b, lse_b, (uint16_t*)o_out, lse_out, rows, heads, head_dim);
  else
    hipLaunchKernelGGL(lse_merge_f32, grid, dim3(MT), 0, stream, (const float*)o_a, lse_a,
                       (const float*)o_b, lse_b, (float*)o_out, lse_out, rows, heads, head_dim);
  return hipGetLastError();
}

}  // namespace elastic
