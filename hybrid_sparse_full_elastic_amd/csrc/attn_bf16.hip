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
//    group), 8 waves of 32 query rows.  Every wave fits in 256 VGPRs, so two waves share a
//    SIMD.
//  * S^T = K . Q^T with v_mfma_f32_32x32x16_bf16: every lane holds one query column, so the
//    softmax row statistics are per-lane (a v_permlane32_swap joins the two halves of a
//    column).  Q stays in registers for the whole item.
//  * O^T = V^T . P^T: P^T comes straight from the S^T accumulators (bf16) with a fixed
//    key-slot permutation, and ds_read_b64_tr_b16 builds the matching V^T operand from the
//    row-major V tile.  The rescale of O by the running maximum is a per-lane multiply.
//  * Online softmax in the exp2 domain with the softmax scale and log2(e) folded into one
//    FMA; fp32 accumulation throughout; the row sum adds the bf16 weights the P.V product
//    uses (v_dot2) so numerator and denominator agree.  The running maximum m comes from the
//    first tile and is raised only when a tile's weights 2^(s - m) grow past 2^64, which the
//    row sums reveal for free (a partial sum above 2^70): such a tile is redone with its own
//    maximum and O rescaled.  No per-tile maximum is computed; fp32 holds the weights and
//    sums with room to spare, and the result is exact in exact arithmetic for any m.
//  * Masks are evaluated only on tiles that cross a causal, sink, window or block boundary,
//    and tiles no query of the item may see are never loaded (streaming items cost
//    O(sink + window), not O(n)).  Each item runs a loop compiled for its mode.  A lane turns
//    its kept keys of an edge tile into two 32-bit words, so an element costs one bit
//    extract and one select.
//  * K/V tiles travel global -> LDS by buffer_load ... lds (no register staging): four K
//    slots (K four tiles ahead) and four V slots (V two tiles ahead), so a load has two tile
//    steps to land; tile j sits in K and V slot j mod 4, a compile-time constant in every
//    step (steps run four per loop iteration), so the fragment addresses fold into the LDS
//    read offsets (four V slots rather than three: 1.4% faster on full heads).  Rows past the sequence end read as zero through the buffer descriptor's
//    range.  Tiles are unpadded with XOR swizzles of the 16-byte chunks chosen so the K row
//    reads and the transposing V reads are free of LDS bank conflicts.
//  * Per tile step j, two instruction regions fenced with sched_barrier so the issue order is
//    the written one: the Q.K^T MFMAs of tile j+1 with the second half of tile j's exp2 /
//    bf16 packing / row sums between them (K fragments read five MFMAs ahead, the step's DMA
//    issued halfway, the first V fragments read during the last MFMAs), then the P.V MFMAs of
//    tile j with the transposing V reads (four ahead) and the first half of tile j+1's
//    weights between them and, after them, the first K fragments of tile j+2 (it landed one
//    barrier early), so the next step starts on MFMAs.  Both regions carry half of the
//    softmax work, and the two waves sharing a SIMD fill each other's gaps.  The mask of an
//    edge tile sits between the regions; one barrier per step.
//  * Persistent grid: each workgroup claims items from its XCD's queue; the next item is
//    claimed in the current item's prologue and its descriptor copied to LDS meanwhile.
//  * Epilogue: each wave stages its 32 normalised rows in the idle tile slots (same swizzle) and
//    writes whole O rows with 16-byte non-temporal stores, so the G heads of a token leave as
//    one contiguous run instead of scattered 8-byte pieces.
#include <type_traits>

#include "elastic_internal.hpp"

namespace elastic {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr float LN2 = 0.69314718055994530942f;
constexpr int NSK = 4;   // LDS slots for K tiles
constexpr int NSV = 4;   // LDS slots for V tiles
static_assert(NSK == 4 && NSV == NSK, "tile j sits in slot j mod 4 for K and V");
constexpr int NPRE = 2;  // K fragments of the next step read before its barrier
constexpr int NVPRE = 2; // V fragments of a step read during its Q.K^T MFMAs

// x[lane] combined with x[lane ^ 32]; the swap returns both halves' values.
__device__ inline float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// max of three floats in one instruction (the inputs are never NaN here)
__device__ inline float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// An empty statement that takes the values in registers: the computations producing them stay
// above it.
__device__ __forceinline__ void keep_here(const bf16x8 (&p0)[2], const bf16x8 (&p1)[2], const float l) {
  asm volatile("" ::"v"(p0[0]), "v"(p0[1]), "v"(p1[0]), "v"(p1[1]), "v"(l));
}
__device__ __forceinline__ void lds_wait_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Opaque copy: the value is the same, but the compiler cannot treat it as loop-invariant.
__device__ __forceinline__ void launder_lane(int& x) { asm volatile("" : "+v"(x)); }

// s_waitcnt vmcnt(n) leaving the other counters alone (gfx9 encoding)
#define WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | 0x70 | 0xF00 | ((((n) >> 4) & 3) << 14))

template <int D>
struct LdsTiles {
  uint16_t k[NSK][BF16_BK * D];
  uint16_t v[NSV][BF16_BK * D];
};

// XOR swizzles of the 16-byte chunk index within a tile row (D/8 chunks per row).  K is read
// 16 rows x one chunk at a time: consecutive rows must land in distinct 16-byte bank groups
// of a 256-byte window.  V is read by ds_read_b64_tr_b16 as 4 rows x 4 chunks: each of the
// 4 rows must shift the chunk group by 4 chunks.
template <int D>
__device__ __host__ constexpr int k_swizzle(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D>
__device__ __host__ constexpr int v_swizzle(int row) {
  return D == 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2);
}

// The workgroup's claim of its next item, in LDS.  Thread 0 claims the next item during the
// current item's prologue (the queue counter's atomic travels with the first K/V copies) and
// loads its descriptor while the tile steps run, so no global round trip sits between two
// items.
struct NextClaim {
  int idx;        // claimed item, or -1 when every queue is empty
  int q0, len;    // this workgroup's own queue: first item and length (read once)
  WorkItem next;  // the claimed item's descriptor
};

// The Q fragments of one item: lane (l32, half) of wave w holds row r = w*32 + l32 (token
// r / G, head r % G of the item's KV group), elements dc*16 + half*8 .. +7 in qreg[dc]; rows
// past the item's tokens are zero.
template <int D>
__device__ __forceinline__ void load_q(bf16x8 (&qreg)[D / 16], const uint16_t* __restrict__ q,
                                       const SeqGeom& geo, const WorkItem& it, int tid, int Hq, int G,
                                       int BT) {
  const SeqSpan sp = seq_span(geo, it.seq);
  const int lane = tid & 63, r = (tid >> 6) * 32 + (lane & 31), half = lane >> 5;
  const int tl = r / G;
  const int t0 = it.qtile * BT;
  const int qi = t0 + tl;
  if (tl < BT && qi <= min(t0 + BT, sp.nq) - 1) {
    const int qhead = it.group * G + (r - tl * G);
    const u32x4* src = reinterpret_cast<const u32x4*>(q + ((sp.q0 + qi) * Hq + qhead) * (int64_t)D + half * 8);
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc) qreg[dc] = __builtin_bit_cast(bf16x8, src[dc * 2]);
  } else {
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc) qreg[dc] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
  }
}

// One work item with its mode known at compile time.  KIND is the sparse kind of the launch:
// each kernel instantiates its own copies of the item loops.
template <int D, int MODE, int KIND>
__device__ __forceinline__ void attn_item(
    const WorkItem& it, const int tid, LdsTiles<D>& lds, uint32_t* list_vis, NextClaim& cl,
    int32_t* sched, const WorkItem* __restrict__ items, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
    float* __restrict__ lse, const SeqGeom& geo, int Hq, int Hkv, int G, int BT, float scale_log2,
    const Pattern& pat) {
  constexpr int NW = BF16_NW, BK = BF16_BK, NT = NW * 64;
  constexpr int DC = D / 16;          // 16-wide d chunks of Q.K^T
  constexpr int DB = D / 32;          // 32-row d blocks of O^T
  constexpr int CPR = D / 8;          // 16-byte chunks per tile row
  constexpr int CPT = BK * CPR / NT;  // DMA chunks per thread per tile and operand
  static_assert(CPT >= 1 && CPT * NT == BK * CPR, "tile split");
  static_assert(NW * 32 * D * 2 <= sizeof(LdsTiles<D>), "O staging fits in the tile slots");
  constexpr int SLOT = BK * D;        // elements per LDS slot

  // rows of this sequence: queries at absolute positions sp.qp + t, keys at k_pos + j
  const SeqSpan sp = seq_span(geo, it.seq);
  const int64_t seq0 = sp.q0;
  const int n = sp.nq;
  const int t0 = it.qtile * BT;
  const int t1 = min(t0 + BT, n) - 1;
  const int g = it.group;
  const int k_end = geo.k_pos + sp.nk;  // one past the last key (absolute)
  // the item's key tiles: closed forms, or the block lists marked in LDS (whole workgroup)
  const auto tiles = [&] {
    if constexpr (MODE == MODE_LIST)
      return list_tiles(list_vis, pat, it.seq, g, Hkv, sp.qp + t0, sp.qp + t1, geo.k_pos, k_end, BK,
                        tid, NT);
    else
      return KeyTilesT<MODE>(MODE, pat, sp.qp + t0, sp.qp + t1, BK, geo.k_pos, k_end);
  }();
  const int blk_shift = 31 - __clz(pat.block);  // block sizes are powers of two

  const int lane = tid & 63, wave = tid >> 6;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);  // uniform: LDS DMA bases in scalar registers
  const int l32 = lane & 31, half = lane >> 5;
  const int64_t kv_row = (int64_t)Hkv * D;  // elements between consecutive tokens of k / v
  const uint16_t* kbase = k + sp.k0 * kv_row + (int64_t)g * D;
  const uint16_t* vbase = v + sp.k0 * kv_row + (int64_t)g * D;
  const float c = scale_log2;

  // ---- this lane's query row: r = token * G + head inside the item
  const int r = wave * 32 + l32;
  const int tl = r / G;
  const int qi = t0 + tl;          // query row within the sequence
  const int qabs = sp.qp + qi;     // its absolute position
  const int qhead = g * G + (r - tl * G);
  const bool qvalid = tl < BT && qi <= t1;
  const int qblk = qabs >> blk_shift;
  bf16x8 qreg[DC];
  load_q<D>(qreg, q, geo, it, tid, Hq, G, BT);

  // ---- DMA staging.  Instruction m of wave w fills LDS chunks [(w*CPT+m)*64, +64) of a tile;
  // lane i's chunk P holds row P/CPR, logical chunk (P%CPR) ^ swizzle(row).
  int k_voff[CPT], v_voff[CPT];
#pragma unroll
  for (int m = 0; m < CPT; ++m) {
    const int P = (wave * CPT + m) * 64 + lane;
    const int row = P / CPR, pc = P % CPR;
    k_voff[m] = (row * (int)kv_row + (pc ^ k_swizzle<D>(row)) * 8) * 2;
    v_voff[m] = (row * (int)kv_row + (pc ^ v_swizzle<D>(row)) * 8) * 2;
  }
  // tile kt (absolute) holds key rows [kt * BK - k_pos, +BK) of the sequence; rows past the
  // key range read as zero through the descriptor's range
  auto tile_rsrc = [&](const uint16_t* base, int kt) {
    const int rows = min(k_end - kt * BK, BK);  // >= 1: the general step loads tiles <= last only
    return __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(base + (int64_t)(kt * BK - geo.k_pos) * kv_row), (short)0,
        rows * (int)kv_row * 2, 0x00020000);
  };
  // a tile whole inside the key range: constant descriptor range
  auto dma_full = [&](const uint16_t* base, int kt, uint16_t* slot, const int (&voff)[CPT]) {
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(base + (int64_t)(kt * BK - geo.k_pos) * kv_row), (short)0,
        BK * (int)kv_row * 2, 0x00020000);
#pragma unroll
    for (int m = 0; m < CPT; ++m)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(slot + (wave_s * CPT + m) * 512), 16,
                                               voff[m], 0, 0, 0);
  };
  auto dma = [&](const uint16_t* base, int kt, uint16_t* slot, const int (&voff)[CPT]) {
    const auto rs = tile_rsrc(base, kt);
#pragma unroll
    for (int m = 0; m < CPT; ++m)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(slot + (wave_s * CPT + m) * 512), 16,
                                               voff[m], 0, 0, 0);
  };

  // ---- LDS read offsets (elements), loop-invariant per lane
  // K: row kb*32 + l32, logical chunk dc*2 + half
  int k_roff[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) k_roff[dc] = l32 * D + (((dc * 2 + half) ^ k_swizzle<D>(l32)) * 8);
  // V (transposing read): source row 4*half + (lane&15)/4 of a 16-key chunk, columns
  // db*32 + ((lane>>4)&1)*16 + 4*(lane&3) .. +3
  int v_roff[DB];
  {
    const int s = lane & 15;
    const int row0 = 4 * half + (s >> 2);
    const int cl = ((lane >> 4) & 1) * 2 + ((s & 3) >> 1);
#pragma unroll
    for (int db = 0; db < DB; ++db)
      v_roff[db] = row0 * D + (((db * 4 + cl) ^ v_swizzle<D>(row0)) * 8) + (s & 1) * 4;
  }

  // ---- S^T[key, query] = K . Q^T for the two 32-key halves of a tile
  auto qk = [&](const uint16_t* ks, f32x16 (&s)[2]) {
    const f32x16 zero = {};
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      bf16x8 a[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        a[kb] = *reinterpret_cast<const bf16x8*>(ks + kb * 32 * D + k_roff[dc]);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kb], qreg[dc], dc == 0 ? zero : s[kb], 0, 0, 0);
    }
  };

  // ---- exact masks on edge tiles: allowed(j) = j <= hi && (j < a || j >= b)
  auto apply_mask = [&](f32x16 (&s)[2], int kt) {
    const int hi = qvalid ? min(qabs, k_end - 1) : -1;
    int a = 0, b = 0;
    if (MODE == MODE_STREAM) {
      a = pat.sink;
      b = qabs - pat.window + 1;
    } else if (MODE == MODE_BLOCK) {
      const int kblk = (kt * BK) >> blk_shift;  // one key block per tile (block % BK == 0)
      const bool vis = kblk < pat.sink_blocks || qblk - kblk <= pat.local_blocks ||
                       (pat.stride_blocks > 0 && kblk % pat.stride_blocks == 0);
      b = vis ? 0 : 0x7fffffff;
    } else if (MODE == MODE_LIST) {
      b = tiles.lists(kt, qblk) ? 0 : 0x7fffffff;
    }
    // This lane's keys of the tile as bits (offset o = j - kt*BK): [0, hi] minus [a, b), one 32-bit
    // word per 32-key half, shifted so that element (kb, e) sits at bit (e/4)*8 + e%4.  Each
    // element then takes one sign-extending bit extract and one bitwise select (no compares,
    // no branches).
    const int base = kt * BK;
    auto low_bits = [](int n) -> uint32_t { return n >= 32 ? 0xffffffffu : (n <= 0 ? 0u : (1u << n) - 1u); };
    // interval ends, exclusive; keys are >= 0, so b <= 0 means no gap (and no overflow below)
    const int A = a - base, B = (b > 0 ? b : 0) - base, H = hi + 1 - base;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int o = kb * 32;
      const uint32_t w = (low_bits(H - o) & (low_bits(A - o) | ~low_bits(B - o))) >> (half * 4);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const uint32_t keep = (uint32_t)__builtin_amdgcn_sbfe((int)w, (e >> 2) * 8 + (e & 3), 1);
        const uint32_t x = __float_as_uint(s[kb][e]);
        s[kb][e] = __uint_as_float((x & keep) | (0xff800000u & ~keep));  // -inf where masked
      }
    }
  };

  // ---- running state (m in the scaled log2 domain)
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
  float m_sc = -1.0e30f;  // finite: fully masked tiles give p = 0 and never raise it
  float l_run = 0.f;

  // m from the first tile (O and l are still zero, so nothing is rescaled)
  auto first_max = [&](f32x16 (&s)[2]) {
    float m0 = max3f(s[0][0], s[1][0], s[0][1]);
    float m1 = max3f(s[1][1], s[0][2], s[1][2]);
#pragma unroll
    for (int e = 3; e < 15; e += 2) {
      m0 = max3f(m0, s[0][e], s[1][e]);
      m1 = max3f(m1, s[0][e + 1], s[1][e + 1]);
    }
    m_sc = fmaxf(m_sc, half_max(max3f(m0, m1, max3f(s[0][15], s[1][15], m0))) * c);
  };

  bool claimed = false;  // uniform: the next item was claimed in the prologue

  // ---- tile schedule: kt_cur = tile j, kt_n1..kt_n4 = tiles j+1..j+4 (-1 when absent)
  // An item whose queries see no key of the range (a query chunk placed before its key
  // range) skips straight to the epilogue and writes O = 0, lse = -inf.
  int kt_cur = tiles.next(0);
  if (kt_cur >= 0) {
    int kt_n1 = tiles.next(kt_cur + 1);
    int kt_n2 = kt_n1 >= 0 ? tiles.next(kt_n1 + 1) : -1;
    int kt_n3 = kt_n2 >= 0 ? tiles.next(kt_n2 + 1) : -1;
    int kt_n4 = kt_n3 >= 0 ? tiles.next(kt_n3 + 1) : -1;

    // prologue: K_0..K_3 and V_0, V_1 land; S_0 computed and reduced.  K tile j lives in K
    // slot j mod 4, V tile j in V slot j mod 4.  Only Q and K_0 are waited for before S_0;
    // the other copies land while it is computed.
    uint16_t* kslot = &lds.k[0][0];
    uint16_t* vslot = &lds.v[0][0];
    // the next item: the queue counter's atomic goes first and lands with K_0
    int k_next = 0;
    if (tid == 0) k_next = atomicAdd(sched + SCHED_CTR * (1 + (int)(blockIdx.x % SCHED_NX)), 1);
    dma(kbase, kt_cur, kslot, k_voff);
    if (kt_n1 >= 0) dma(kbase, kt_n1, kslot + SLOT, k_voff);
    dma(vbase, kt_cur, vslot, v_voff);
    if (kt_n2 >= 0) dma(kbase, kt_n2, kslot + 2 * SLOT, k_voff);
    if (kt_n1 >= 0) dma(vbase, kt_n1, vslot + SLOT, v_voff);
    if (kt_n3 >= 0) dma(kbase, kt_n3, kslot + 3 * SLOT, k_voff);
    // copies issued after K_0 (each CPT instructions): V_0, and K_1, V_1, K_2, K_3 if present
    const int n_after = 1 + (kt_n1 >= 0 ? 2 : 0) + (kt_n2 >= 0 ? 1 : 0) + (kt_n3 >= 0 ? 1 : 0);
    if (n_after == 5) WAIT_VMCNT(5 * CPT);
    else if (n_after == 4) WAIT_VMCNT(4 * CPT);
    else if (n_after == 3) WAIT_VMCNT(3 * CPT);
    else WAIT_VMCNT(CPT);
    // K_0 is in LDS, and every wave has read this item's claim: the slot is free.  An LDS-only
    // barrier: __syncthreads would also wait for every copy still in flight
    lds_wait_barrier();
    int next_idx = 0;  // thread 0
    if (tid == 0) {
      next_idx = k_next < cl.len ? cl.q0 + k_next : claim_item(sched);
      cl.idx = next_idx;
    }
    claimed = true;
    f32x16 s0[2], s1[2];
    qk(kslot, s0);
    // every copy but V_1 and K_3 (first read in step 1; step 0's closing wait retires them) has
    // landed, and every wave is done with K slot 0 before step 0 refills it
    if (kt_n3 >= 0) WAIT_VMCNT(2 * CPT);
    else if (kt_n1 >= 0) WAIT_VMCNT(CPT);
    else WAIT_VMCNT(0);
    lds_wait_barrier();
    if (wave == 0) {
      // the next item's descriptor goes global -> LDS by DMA (4 lanes x 4 bytes) and lands
      // during the tile steps, whose copy waits retire it
      const int idx = __builtin_amdgcn_readfirstlane(next_idx);
      if (idx >= 0 && lane < 4) {
        const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<WorkItem*>(items + idx), (short)0,
                                                          (int)sizeof(WorkItem), 0x00020000);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)&cl.next, 4, lane * 4, 0, 0, 0);
      }
    }
    if (tiles.needs_mask(kt_cur)) apply_mask(s0, kt_cur);
    first_max(s0);
    // The weights of a tile are made in two halves: pairs 0-7 (keys 0-31) during the P.V
    // MFMAs of the step before, pairs 8-15 (keys 32-63) during its own Q.K^T MFMAs, so both
    // MFMA regions carry half of the softmax VALU work (measured 0.8% faster on full heads
    // than all of it in the Q.K^T region, where the P.V region left the VALU idle).
    // phalf: the first half (P fragments of keys 0-31), ls_half its row sum.
    bf16x8 phalf[2];
    float ls_half;
    auto weight_pair = [&](const f32x16 (&s)[2], int pair, float nm, bf16x8 (&ph)[2], bf16x8 (&p1)[2]) {
      const int kb = pair >> 3, e = (pair & 7) * 2;
      const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][e], c, nm));
      const float pq = __builtin_amdgcn_exp2f(fmaf(s[kb][e + 1], c, nm));
      const bf16x2 pp = {(__bf16)p0, (__bf16)pq};
      bf16x8& dst = kb == 0 ? ph[e >> 3] : p1[e >> 3];
      dst[e & 7] = pp[0];
      dst[(e & 7) + 1] = pp[1];
      return pp;
    };
    {
      const float nm = -m_sc;
      const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
      bf16x8 unused[2];
#pragma unroll
      for (int pair = 0; pair < 8; ++pair) {
        const bf16x2 pp = weight_pair(s0, pair, nm, phalf, unused);
        ls_half = pair == 0 ? __builtin_amdgcn_fdot2_f32_bf16(pp, ones, 0.f, false)
                            : __builtin_amdgcn_fdot2_f32_bf16(pp, ones, ls_half, false);
      }
    }
    // the first K fragments of step 0 (tile 1)
    bf16x8 kpre[NPRE];
#pragma unroll
    for (int i = 0; i < NPRE; ++i)
      kpre[i] = *reinterpret_cast<const bf16x8*>(kslot + SLOT + (i & 1) * 32 * D + k_roff[i >> 1]);

    // One step on tile j: DMA K_{j+4} and V_{j+2}; S_{j+1} = K_{j+1} Q^T; p_j = exp2(c s_j - m);
    // O += V_j^T P_j^T; the first K fragments of tile j+2; mask of S_{j+1}; wait for the
    // previous step's DMA; barrier.
    // Slots: K_{j+4} refills the slot of K_j (read last step), V_{j+2} that of V_{j-2} (read
    // two steps ago).  K_{j+2} landed before the previous barrier (it was copied two steps ago), so
    // its first fragments are read before this step's barrier and the next step's first
    // MFMAs wait for no LDS read.
    // STEADY: a step inside a run of consecutive whole tiles where tile j+1 needs no mask (the
    // key-tile schedule's steady_pair), so no bound, mask or DMA-count decisions are taken:
    // the scalar work of a step shrinks to the DMA descriptors and one loop test.  Used for
    // full items, whose tiles below the diagonal form one such run; for the shorter runs of
    // sparse items the extra loop copy costs more than it saves.
    auto step = [&](auto steady_tag, f32x16 (&sc)[2], f32x16 (&sn)[2], auto slot_tag) {
      constexpr bool STEADY = decltype(steady_tag)::value;
      constexpr int skj_ = decltype(slot_tag)::value;  // K_j's and V_j's slot: steps run in slot order
      static_assert(skj_ >= 0 && skj_ < NSK, "K slot");
      constexpr int sk1 = (skj_ + 1) & (NSK - 1), sk2 = (skj_ + 2) & (NSK - 1);
      constexpr int sv2 = (skj_ + 2) & (NSV - 1);  // V_{j+2}'s slot
      const int n_dma = STEADY ? 2 * CPT : (kt_n4 >= 0 ? CPT : 0) + (kt_n2 >= 0 ? CPT : 0);
      const bool has_next = STEADY || kt_n1 >= 0;
      // Region 1: Q.K^T of tile j+1 (NQK MFMAs; K fragments read five ahead) with the second
      // half of tile j's exp2 / bf16 packing / row sums (pairs 8-15) placed between them; the
      // DMA is issued halfway (measured: 1.6% faster on full heads than right after the first
      // MFMAs), and the first V fragments of region 2 are read during the last MFMAs.
      constexpr int NQK = 2 * DC, NPV = 4 * DB;
      constexpr int QPP = NQK / 8;   // Q.K^T MFMAs per weight pair of the second half
      constexpr int AHEAD = 5;
      bf16x8 pop1[2];  // P fragments of keys 32-63 of tile j
      // row sum of the tile's weights: one dependent chain on from the first half's sum
      float ls = ls_half;
      // transposing reads of V_j (landed before the last barrier)
      const uint16_t* vs = vslot + skj_ * SLOT;
      bf16x8 av[NPV];
      // P.V fragment i: O block db = i % DB, weights (kb, cc) = i / DB, so that consecutive
      // MFMAs accumulate into different O blocks (measured 0.5% faster on full heads than four
      // in a row into one block)
      auto vread = [&](int i) {
        const int db = i % DB, kb = (i / DB) >> 1, cc = (i / DB) & 1;
        const uint16_t* src = vs + v_roff[db] + (kb * 32 + cc * 16) * D;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(src));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(src + 8 * D));
        av[i] = __builtin_bit_cast(bf16x8, s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
      };
      const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
      {
        const uint16_t* ks = kslot + sk1 * SLOT;
        const float nm = -m_sc;
        const f32x16 zero = {};
        bf16x8 a[NQK];
#pragma unroll
        for (int i = 0; i < NPRE; ++i) a[i] = kpre[i];
#pragma unroll
        for (int i = NPRE; i < AHEAD; ++i)
          a[i] = *reinterpret_cast<const bf16x8*>(ks + (i & 1) * 32 * D + k_roff[i >> 1]);
#pragma unroll
        for (int i = 0; i < NQK; ++i) {
          if (i + AHEAD < NQK)
            a[i + AHEAD] = *reinterpret_cast<const bf16x8*>(ks + ((i + AHEAD) & 1) * 32 * D + k_roff[(i + AHEAD) >> 1]);
          sn[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], qreg[i >> 1], i < 2 ? zero : sn[i & 1], 0, 0, 0);
          if (i % QPP == QPP - 1) {
            const bf16x2 pp = weight_pair(sc, 8 + i / QPP, nm, phalf, pop1);
            ls = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, ls, false);
          }
          // the first V fragments of region 2, during the last MFMAs
          if (i >= NQK - NVPRE) vread(i - (NQK - NVPRE));
          if (i == NQK / 2) {
            if (STEADY) {
              dma_full(kbase, kt_n4, kslot + skj_ * SLOT, k_voff);
              dma_full(vbase, kt_n2, vslot + sv2 * SLOT, v_voff);
            } else {
              if (kt_n4 >= 0) dma(kbase, kt_n4, kslot + skj_ * SLOT, k_voff);
              if (kt_n2 >= 0) dma(vbase, kt_n2, vslot + sv2 * SLOT, v_voff);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // keep tile j's weights in this region (no sinking past the mask branch)
      keep_here(phalf, pop1, ls);
      // The weights of tile j used the running maximum m.  A row whose partial sum passes
      // 2^70 (some weight above 2^64: the first tiles of a row, or a sharp rise of its scores)
      // is redone with the tile's own maximum; inf and NaN sums take the same path.
      if (__builtin_amdgcn_ballot_w64(!(ls <= 0x1p70f)) != 0) {
        float m0 = max3f(sc[0][0], sc[1][0], sc[0][1]);
        float m1 = max3f(sc[1][1], sc[0][2], sc[1][2]);
#pragma unroll
        for (int e = 3; e < 15; e += 2) {
          m0 = max3f(m0, sc[0][e], sc[1][e]);
          m1 = max3f(m1, sc[0][e + 1], sc[1][e + 1]);
        }
        const float ms = half_max(max3f(m0, m1, max3f(sc[0][15], sc[1][15], m0))) * c;
        const float mn = fmaxf(m_sc, ms);
        const float al = __builtin_amdgcn_exp2f(m_sc - mn);
        m_sc = mn;
        l_run *= al;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) oacc[db][e] *= al;
        const float nm = -m_sc;
        ls = 0.f;
#pragma unroll
        for (int pair = 0; pair < 16; ++pair) {
          const bf16x2 pp = weight_pair(sc, pair, nm, phalf, pop1);
          ls = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, ls, false);
        }
      }
      if (!STEADY && has_next && tiles.needs_mask(kt_n1)) apply_mask(sn, kt_n1);
      // Region 2: P.V of tile j (NPV MFMAs; transposing V reads four fragments ahead) with the
      // first half of tile j+1's weights (pairs 0-7) between them: a pair goes into phalf once
      // the MFMAs that read tile j's fragment there are issued (fragment cc of the first half
      // is read by MFMAs cc*DB .. cc*DB + DB - 1).  After the last step these are made from a
      // tile that does not exist and are never used.
      {
        const uint16_t* kn = kslot + sk2 * SLOT;
        const float nm = -m_sc;
        float lsn = 0.f;
        auto slot_of = [](int p) {  // the P.V MFMA after which pair p of the next tile is made
          return p < 4 ? DB - 1 + p : 2 * DB - 1 + (p - 4) * ((NPV - 2 * DB) / 4);
        };
#pragma unroll
        for (int i = NVPRE; i < 4; ++i) vread(i);
#pragma unroll
        for (int i = 0; i < NPV; ++i) {
          if (i + 4 < NPV) vread(i + 4);
          const int db = i % DB, kb = (i / DB) >> 1, cc = (i / DB) & 1;
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], kb == 0 ? phalf[cc] : pop1[cc], oacc[db], 0, 0, 0);
#pragma unroll
          for (int p = 0; p < 8; ++p) {
            if (slot_of(p) == i) {
              bf16x8 unused[2];
              const bf16x2 pp = weight_pair(sn, p, nm, phalf, unused);
              lsn = p == 0 ? __builtin_amdgcn_fdot2_f32_bf16(pp, ones, 0.f, false)
                           : __builtin_amdgcn_fdot2_f32_bf16(pp, ones, lsn, false);
            }
          }
          // the first K fragments of tile j+2, after the last V reads
          if (i >= NPV - NPRE)
            kpre[i - (NPV - NPRE)] =
                *reinterpret_cast<const bf16x8*>(kn + ((i - (NPV - NPRE)) & 1) * 32 * D + k_roff[(i - (NPV - NPRE)) >> 1]);
          __builtin_amdgcn_sched_barrier(0);
        }
        l_run += ls;
        ls_half = lsn;
      }
      const int kt_n5 = STEADY ? kt_n4 + 1 : (kt_n4 >= 0 ? tiles.next(kt_n4 + 1) : -1);
      // this step's DMA may stay in flight; the previous step's (K_{j+3}, V_{j+1}) must land
      if (n_dma == 2 * CPT) WAIT_VMCNT(2 * CPT);
      else if (n_dma == CPT) WAIT_VMCNT(CPT);
      else WAIT_VMCNT(0);
      // LDS reads of this step done, then the barrier.  (__syncthreads would also wait for the
      // DMA issued this step, which must stay in flight.)
      lds_wait_barrier();
      kt_cur = kt_n1;
      kt_n1 = kt_n2;
      kt_n2 = kt_n3;
      kt_n3 = kt_n4;
      kt_n4 = kt_n5;
    };

    using SteadyT = std::integral_constant<bool, true>;
    using GeneralT = std::integral_constant<bool, false>;
    if (MODE == MODE_FULL) {
      // Full items visit consecutive tiles.  A pair of steady steps from tile j loads tiles up
      // to j+5 (whole inside the key range), advances the schedule to j+6 (a visited tile) and
      // computes S of tiles j+1, j+2 (below the diagonal and the key range's end: no mask).
      // Two pairs per iteration keep the K slot indices compile-time constants, so the K
      // fragment addresses fold into the LDS read offsets (9 fewer VALU per step, -0.7%).
      using K0 = std::integral_constant<int, 0>;
      using K1 = std::integral_constant<int, 1>;
      using K2 = std::integral_constant<int, 2>;
      using K3 = std::integral_constant<int, 3>;
      // the steady loop starts right after the prologue (K slot 0) and keeps the slot period
      while (tiles.steady_pair(kt_cur) && tiles.steady_pair(kt_cur + 2)) {
        step(SteadyT{}, s0, s1, K0{});
        step(SteadyT{}, s1, s0, K1{});
        step(SteadyT{}, s0, s1, K2{});
        step(SteadyT{}, s1, s0, K3{});
      }
    }
    // The general steps start on K slot 0 too (after the prologue, or after whole steady
    // iterations), so four of them per iteration also keep the K slot a compile-time constant
    // (block-pattern heads -1.9%, streaming -0.5 to -1.4% against a runtime slot).
    {
      using K0 = std::integral_constant<int, 0>;
      using K1 = std::integral_constant<int, 1>;
      using K2 = std::integral_constant<int, 2>;
      using K3 = std::integral_constant<int, 3>;
      while (true) {
        step(GeneralT{}, s0, s1, K0{});
        if (kt_cur < 0) break;
        step(GeneralT{}, s1, s0, K1{});
        if (kt_cur < 0) break;
        step(GeneralT{}, s0, s1, K2{});
        if (kt_cur < 0) break;
        step(GeneralT{}, s1, s0, K3{});
        if (kt_cur < 0) break;
      }
    }
  }

  // ---- the next item, for an item without keys (no prologue ran): claim it now, once every
  // wave has read this item's claim
  if (!claimed) {
    __syncthreads();
    if (tid == 0) {
      const int idx = claim_item(sched);
      cl.idx = idx;
      if (idx >= 0) cl.next = items[idx];
    }
  }

  // ---- epilogue: normalise, stage the wave's 32 rows in LDS (every wave passed the last
  // barrier, so the tile slots are idle), then write whole O rows with 16-byte stores (O is
  // written once: non-temporal stores, 1-2% faster on sparse heads)
  const float lt = half_sum(l_run);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  uint16_t* stage = reinterpret_cast<uint16_t*>(&lds) + wave * 32 * D;  // 32 rows x D, swizzled
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int ig = 0; ig < 4; ++ig) {
      bf16x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = (__bf16)(oacc[db][ig * 4 + e] * inv);
      const int chunk = db * 4 + ig;  // d = chunk * 8 + half * 4 + e
      *reinterpret_cast<u32x2*>(stage + l32 * D + ((chunk ^ k_swizzle<D>(l32)) * 8) + half * 4) =
          __builtin_bit_cast(u32x2, w);
    }
  lds_wait();  // the wave reads back its own rows
  constexpr int RPI = 64 / CPR;                        // rows per store instruction
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int rr = i * RPI + lane / CPR, cc = lane % CPR;
    const u32x4 val = *reinterpret_cast<const u32x4*>(stage + rr * D + ((cc ^ k_swizzle<D>(rr)) * 8));
    const int row = wave * 32 + rr;
    const int rt = row / G;
    if (rt < BT && t0 + rt <= t1)
      __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(o + ((seq0 + t0 + rt) * Hq + g * G + (row - rt * G)) * (int64_t)D + cc * 8));
  }
  if (lse != nullptr && half == 0 && qvalid)  // log of an empty sum is -inf
    lse[(int64_t)qhead * geo.total_q + seq0 + qi] = (m_sc + __log2f(lt)) * LN2;
}

// Kernel arguments, in one struct (the only kernel argument) so that the item loop can
// re-read them from the kernel argument segment for every item (see the loop below).
struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  SeqGeom geo;
  int Hq, Hkv, G, BT;
  float scale_log2;
  Pattern pat;
  const WorkItem* items;
  int32_t* sched;
};
typedef __attribute__((address_space(4))) const AttnArgs ConstArgs;
__device__ __forceinline__ void launder(ConstArgs*& p) { asm volatile("" : "+s"(p)); }

// All of a workgroup's LDS in one object.  With several LDS variables the compiler tags LDS
// accesses with per-variable alias scopes and then makes every LDS read wait for all K/V
// copies still in flight, which serialises the tile pipeline.
template <int D, bool LISTS>
struct __attribute__((aligned(1024))) KernelLds {
  LdsTiles<D> tiles;
  uint32_t list_vis[LISTS ? LIST_MAX_KB : 1];  // block lists: visibility per key block
  NextClaim claim;                              // the workgroup's next item
};

// One kernel per sparse pattern kind: every launch holds full items and items of one sparse
// kind, so each instantiation carries two item loops only (less code and fewer live scalar
// registers than one kernel for every mode).  The grid is persistent (one workgroup per
// CU): each workgroup claims items from its XCD's queue, then from the others, until none
// is left.
template <int D, int KIND>
__global__ __launch_bounds__(BF16_NW * 64, 1) void attn_bf16_kernel(AttnArgs args) {
  __shared__ KernelLds<D, KIND == ELASTIC_SPARSE_BLOCK_LIST> shm;
  // The arguments are read afresh for each item through an opaque pointer to the kernel
  // argument segment, where the only explicit argument sits at offset 0: values derived from
  // them are then computed inside the item instead of being held in registers across the
  // whole loop (which spills).  (Taking the address of `args` would copy it to scratch.)
  // The library build reads every instance's code-object metadata and stops unless `args` is
  // its one explicit argument, by value at offset 0 of the segment.
  ConstArgs* const base = (ConstArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  (void)args;
  if (threadIdx.x == 0) {  // the first claim; later ones come from each item's prologue
    const int x = (int)(blockIdx.x % SCHED_NX);
    shm.claim.q0 = base->sched[1 + x];
    shm.claim.len = base->sched[2 + x] - shm.claim.q0;
    const int idx = claim_item(base->sched);
    shm.claim.idx = idx;
    if (idx >= 0) shm.claim.next = base->items[idx];
  }
  for (;;) {
    ConstArgs* a = base;
    launder(a);
    // the claim is in LDS, and every wave is done with the previous item's LDS (O staging)
    lds_wait_barrier();
    // uniform, and in scalar registers
    const int idx = __builtin_amdgcn_readfirstlane(shm.claim.idx);
    if (idx < 0) return;  // every queue is empty
    WorkItem it;
    it.seq = __builtin_amdgcn_readfirstlane(shm.claim.next.seq);
    it.group = __builtin_amdgcn_readfirstlane(shm.claim.next.group);
    it.qtile = __builtin_amdgcn_readfirstlane(shm.claim.next.qtile);
    it.full = __builtin_amdgcn_readfirstlane(shm.claim.next.full);
    int tid = threadIdx.x;
    launder_lane(tid);
    const bool full = it.full != 0;
    SeqGeom geo;
    geo.cu_q = a->geo.cu_q, geo.cu_k = a->geo.cu_k, geo.total_q = a->geo.total_q;
    geo.total_k = a->geo.total_k, geo.q_pos = a->geo.q_pos, geo.k_pos = a->geo.k_pos;
    Pattern pat;
    pat.kind = a->pat.kind, pat.sink = a->pat.sink, pat.window = a->pat.window;
    pat.block = a->pat.block, pat.sink_blocks = a->pat.sink_blocks;
    pat.local_blocks = a->pat.local_blocks, pat.stride_blocks = a->pat.stride_blocks;
    pat.qblocks = a->pat.qblocks, pat.row_ptr = a->pat.row_ptr, pat.col_idx = a->pat.col_idx;
#define ELASTIC_ITEM_ARGS it, tid, shm.tiles, shm.list_vis, shm.claim, a->sched, a->items, a->q, \
                          a->k, a->v, a->o, a->lse, geo, \
                          a->Hq, a->Hkv, a->G, a->BT, a->scale_log2, pat
    if (full)
      attn_item<D, MODE_FULL, KIND>(ELASTIC_ITEM_ARGS);
    else if constexpr (KIND == ELASTIC_SPARSE_STREAMING)
      attn_item<D, MODE_STREAM, KIND>(ELASTIC_ITEM_ARGS);
    else if constexpr (KIND == ELASTIC_SPARSE_BLOCK)
      attn_item<D, MODE_BLOCK, KIND>(ELASTIC_ITEM_ARGS);
    else
      attn_item<D, MODE_LIST, KIND>(ELASTIC_ITEM_ARGS);
#undef ELASTIC_ITEM_ARGS
  }
}

}  // namespace

hipError_t launch_attn_bf16(int head_dim, const void* q, const void* k, const void* v, void* o,
                            float* lse, const SeqGeom& geo, int n_q_heads, int n_kv_heads, int BT,
                            float scale, const int32_t* head_mask, const Pattern& pat,
                            const WorkItem* items, int32_t* sched, int64_t max_items,
                            hipStream_t stream) {
  const float scale_log2 = scale * 1.4426950408889634f;
  const int G = n_q_heads / n_kv_heads;
  if (max_items <= 0) return hipSuccess;
  hipError_t err = hipSuccess;
  auto launch = [&](auto kernel) {
    int64_t grid = 0;
    err = resident_grid(reinterpret_cast<const void*>(kernel), BF16_NW * 64, &grid);
    if (err != hipSuccess) return;
    grid = grid < max_items ? grid : max_items;
    const AttnArgs args{(const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, lse,
                        geo, n_q_heads, n_kv_heads, G, BT, scale_log2, pat, items, sched};
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(BF16_NW * 64), 0, stream, args);
  };
  // without a head mask every item is full: any instantiation serves
  const int kind = head_mask == nullptr ? ELASTIC_SPARSE_STREAMING : pat.kind;
  if (head_dim == 128) {
    if (kind == ELASTIC_SPARSE_STREAMING) launch(attn_bf16_kernel<128, ELASTIC_SPARSE_STREAMING>);
    else if (kind == ELASTIC_SPARSE_BLOCK) launch(attn_bf16_kernel<128, ELASTIC_SPARSE_BLOCK>);
    else launch(attn_bf16_kernel<128, ELASTIC_SPARSE_BLOCK_LIST>);
  } else {
    if (kind == ELASTIC_SPARSE_STREAMING) launch(attn_bf16_kernel<64, ELASTIC_SPARSE_STREAMING>);
    else if (kind == ELASTIC_SPARSE_BLOCK) launch(attn_bf16_kernel<64, ELASTIC_SPARSE_BLOCK>);
    else launch(attn_bf16_kernel<64, ELASTIC_SPARSE_BLOCK_LIST>);
  }
  if (err != hipSuccess) return err;
  return hipGetLastError();
}

}  // namespace elastic
