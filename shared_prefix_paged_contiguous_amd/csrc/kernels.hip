// Decode-attention kernels for MI355X (gfx950, CDNA4, wave64).
//
// What is computed (GraniKV pages, paperlayer.ai summary §2 "Prefix-suffix
// attention" and §3 "Dual attention backends"): the attention of each decode
// query over its shared HOT prefix and over its own COLD suffix, each as a
// partial softmax (normalised output + log-sum-exp), joined by a log-sum-exp
// merge.  Scores are q.k / sqrt(d); query head h reads KV head h / G.
//
// Matrix-core mapping (shared by all attention kernels).  A wave works on a
// block of 16 "columns" (query rows: the G heads of one request in the suffix
// kernel, 16 rows of a prefix class in the prefix kernels) and 32 tokens at a
// time, with two MFMA products per tile:
//   S^T[token][col] = K[token][:] . Q[col][:]    (A = K rows, B = Q^T)
//   O^T[d][col]    += V^T[d][token] P^T[token][col]  (A = V^T, B = P^T)
// The 16x16 accumulator layout puts, in lane l (col n = l%16, group g = l/16),
// rows 4g..4g+3 of column n.  Computing S^T rather than S leaves each lane
// holding scores of ONE column for 8 tokens (two 16-token halves), which is
// exactly the B-operand slice of P^T the second product needs: no shuffles
// between the softmax and the PV product.  The softmax max over a column is
// a max over the lane's 8 values and across the 4 lane groups (two xor
// shuffles); the running sum stays per lane and is reduced once at the end.
// The A operand V^T is built without LDS transposes: a lane loads, for each
// of its 8 tokens, the D/16 consecutive elements d = (D/16)*n .. +D/16, and
// output row r of block j is taken to be d = (D/16)*r + j, so that block j's
// A operand is element j of each loaded vector (an 8x(D/16) register
// transpose of 16-bit values, done with v_perm).  The K-dimension of the
// first product is permuted the same way on both operands.
//
// Kernels
//   step_kernel     all attention of one decode step in one launch.  Blocks
//                   [0, prefix_blocks) are prefix workgroups, one per (class,
//                   KV head, M-tile, L split): they stream the split's HOT
//                   blocks into an LDS ring with direct global->LDS loads and
//                   run the MFMA tile for RB 16-row blocks per wave (RB = 1
//                   with many L splits: cascade backend, each slab byte read
//                   once per step; RB = 2: dense backend, HydraGen-style
//                   batched GEMM of M_eff rows).  The rest are suffix
//                   workgroups, one per (slot-table part, KV head): they
//                   gather COLD rows through the slot table (software-
//                   pipelined one tile ahead) and join their waves' pieces
//                   in LDS.  Partials are joined by log-sum-exp inside the
//                   same launch (see StepArgs).
//   hot_write_kernel  scatter of token rows into the blocked HOT layout.
//   append_kernel   byte copy of new token rows into COLD slots.
//   zero_kernel     clears the join counters of a newly bound workspace.
//
// Partials keep lse in base 2 of the scaled scores (s * log2(e)/sqrt(d));
// the join converts the final lse to natural log.

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <algorithm>
#include <cstring>
#include <cstdint>
#include <mutex>
#include <type_traits>

#include "kernels.h"

// Scratch of the allocation-free step (gkv_decode_step_static): status word,
// join counters and partial results in a static array of every device the
// library runs on, held until the process ends.  Host code never uses the
// array's name as an address (it names a host-side stand-in): the device
// address comes from hipGetSymbolAddress, once per device (scratch_region).
static __device__ __align__(256) uint8_t scratch[gkv::kStaticScratchBytes];

namespace gkv {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLazy = 8.f;   // rescale threshold of the online softmax (log2 units)

// Token of k-slot (lane group g, element e) in a 32-token tile: the tokens
// whose scores lane group g holds, in the order the S^T accumulators give.
__device__ __forceinline__ int tau(int g, int e) {
  return e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4);
}

// Entry i of a 4-byte-aligned int16 / int8 table in the kernel arguments,
// read through its aligned 32-bit word: there are no 8- or 16-bit scalar
// loads, so a wave-uniform i then stays a scalar-cache read instead of a
// vector memory round trip.
template <typename I>
__device__ __forceinline__ int table_at(const I* t, int i) {
  constexpr int kBits = 8 * static_cast<int>(sizeof(I));
  constexpr int kPer = 4 / static_cast<int>(sizeof(I));
  const uint32_t w = reinterpret_cast<const uint32_t*>(t)[i / kPer];
  return static_cast<int32_t>(w << (32 - kBits - (i % kPer) * kBits)) >> (32 - kBits);
}

__device__ __forceinline__ float wave_max_groups(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}

__device__ __forceinline__ float wave_sum_groups(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

// ------------------------------------------------------------------ traits
template <typename T, int D>
struct Traits;

// bf16: v_mfma_f32_16x16x32_bf16, 8 elements per lane per k-step.
template <int D>
struct Traits<__bf16, D> {
  static constexpr int KS = D / 32;      // k-steps of S^T = K Q^T
  static constexpr int EPB = D / 16;     // V elements per lane per token = output blocks
  static constexpr int VW = EPB / 2;     // 32-bit words per V vector
  using KOp = u32x4;
  struct VVec { uint32_t w[VW]; };

  // Q or K operand of one row: k-step s, lane group g -> d = 8g + 32s .. +8
  __device__ static void load_row(KOp (&op)[KS], const __bf16* row, int g) {
#pragma unroll
    for (int s = 0; s < KS; ++s) op[s] = *reinterpret_cast<const u32x4*>(row + 8 * g + 32 * s);
  }
  __device__ static void zero_row(KOp (&op)[KS]) {
#pragma unroll
    for (int s = 0; s < KS; ++s) op[s] = u32x4{0u, 0u, 0u, 0u};
  }
  __device__ static VVec load_v(const __bf16* p) {
    VVec v;
    if constexpr (VW == 4) {
      u32x4 x = *reinterpret_cast<const u32x4*>(p);
      v.w[0] = x[0]; v.w[1] = x[1]; v.w[2] = x[2]; v.w[3] = x[3];
    } else {
      u32x2 x = *reinterpret_cast<const u32x2*>(p);
      v.w[0] = x[0]; v.w[1] = x[1];
    }
    return v;
  }
  __device__ static f32x4 qk(const KOp (&k)[KS], const KOp (&q)[KS]) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k[s]),
                                                    __builtin_bit_cast(bf16x8, q[s]), acc, 0, 0, 0);
    return acc;
  }
  // A operands of the PV product: a[j] = element j of the 8 token vectors.
  struct VOp { u32x4 a[EPB]; };
  __device__ static void make_vop(VOp& o, const VVec (&v)[8]) {
#pragma unroll
    for (int k = 0; k < VW; ++k)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        o.a[2 * k][j] = __builtin_amdgcn_perm(v[2 * j + 1].w[k], v[2 * j].w[k], 0x05040100u);
        o.a[2 * k + 1][j] = __builtin_amdgcn_perm(v[2 * j + 1].w[k], v[2 * j].w[k], 0x07060302u);
      }
  }
  // Operands from a HOT block image (see the layout note above hot_write_kernel)
  __device__ static void load_k_img(KOp (&k)[KS], const uint8_t* img, int h, int lane) {
#pragma unroll
    for (int s = 0; s < KS; ++s) k[s] = reinterpret_cast<const u32x4*>(img)[(h * KS + s) * 64 + lane];
  }
  __device__ static void load_v_img(VOp& o, const uint8_t* img, int lane) {
#pragma unroll
    for (int j = 0; j < EPB; ++j) o.a[j] = reinterpret_cast<const u32x4*>(img)[j * 64 + lane];
  }
  // zero the V operand elements of tokens >= valid (element e <-> token tau(g, e))
  __device__ static void mask_v(VOp& o, int valid, int g) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t m = (tau(g, 2 * w) < valid ? 0x0000ffffu : 0u) | (tau(g, 2 * w + 1) < valid ? 0xffff0000u : 0u);
#pragma unroll
      for (int j = 0; j < EPB; ++j) o.a[j][w] &= m;
    }
  }
  // (The softmax denominators are summed on the VALU in fp32 from the
  // unrounded weights: a sum of the bf16-rounded weights on the matrix cores,
  // an all-ones block of this product, would cost up to 2^-9 of relative
  // precision in lse.)
  __device__ static void pv(f32x4 (&acc)[EPB], const VOp& vo, const f32x4& p0, const f32x4& p1) {
    bf16x8 pb = {(__bf16)p0[0], (__bf16)p0[1], (__bf16)p0[2], (__bf16)p0[3],
                 (__bf16)p1[0], (__bf16)p1[1], (__bf16)p1[2], (__bf16)p1[3]};
#pragma unroll
    for (int j = 0; j < EPB; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vo.a[j]), pb,
                                                       acc[j], 0, 0, 0);
  }
};

// fp32: v_mfma_f32_16x16x4_f32, one element per lane per k-step.
template <int D>
struct Traits<float, D> {
  static constexpr int KS = D / 4;
  static constexpr int EPB = D / 16;
  using KOp = float;
  struct VVec { float x[EPB]; };

  // k-step s, lane group g -> d = (D/4) g + s: a lane reads D/4 consecutive floats
  __device__ static void load_row(KOp (&op)[KS], const float* row, int g) {
    const f32x4* p = reinterpret_cast<const f32x4*>(row + (D / 4) * g);
#pragma unroll
    for (int s4 = 0; s4 < KS / 4; ++s4) {
      f32x4 x = p[s4];
      op[4 * s4] = x[0]; op[4 * s4 + 1] = x[1]; op[4 * s4 + 2] = x[2]; op[4 * s4 + 3] = x[3];
    }
  }
  __device__ static void zero_row(KOp (&op)[KS]) {
#pragma unroll
    for (int s = 0; s < KS; ++s) op[s] = 0.f;
  }
  __device__ static VVec load_v(const float* p) {
    VVec v;
    const f32x4* q = reinterpret_cast<const f32x4*>(p);
#pragma unroll
    for (int s4 = 0; s4 < EPB / 4; ++s4) {
      f32x4 x = q[s4];
      v.x[4 * s4] = x[0]; v.x[4 * s4 + 1] = x[1]; v.x[4 * s4 + 2] = x[2]; v.x[4 * s4 + 3] = x[3];
    }
    return v;
  }
  __device__ static f32x4 qk(const KOp (&k)[KS], const KOp (&q)[KS]) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(k[s], q[s], acc, 0, 0, 0);
    return acc;
  }
  struct VOp { VVec v[8]; };
  __device__ static void make_vop(VOp& o, const VVec (&v)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) o.v[e] = v[e];
  }
  __device__ static void load_k_img(KOp (&k)[KS], const uint8_t* img, int h, int lane) {
#pragma unroll
    for (int s4 = 0; s4 < D / 16; ++s4) {
      const f32x4 x = reinterpret_cast<const f32x4*>(img)[(h * (D / 16) + s4) * 64 + lane];
      k[4 * s4] = x[0]; k[4 * s4 + 1] = x[1]; k[4 * s4 + 2] = x[2]; k[4 * s4 + 3] = x[3];
    }
  }
  __device__ static void load_v_img(VOp& o, const uint8_t* img, int lane) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      o.v[e] = load_v(reinterpret_cast<const float*>(img) + (e * 64 + lane) * EPB);
  }
  __device__ static void mask_v(VOp& o, int valid, int g) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (tau(g, e) >= valid)
#pragma unroll
        for (int j = 0; j < EPB; ++j) o.v[e].x[j] = 0.f;
  }
  // step e contracts the 4 tokens tau(g, e) of the four lane groups
  __device__ static void pv(f32x4 (&acc)[EPB], const VOp& vo, const f32x4& p0, const f32x4& p1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float b = e < 4 ? p0[e] : p1[e - 4];
#pragma unroll
      for (int j = 0; j < EPB; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(vo.v[e].x[j], b, acc[j], 0, 0, 0);
    }
  }
};

// ------------------------------------------------------- online softmax core
template <typename T, int D>
struct ColState {
  using TR = Traits<T, D>;
  typename TR::KOp q[TR::KS];
  f32x4 acc[TR::EPB];
  float m;   // running max of scaled scores (base-2 units), per column
  float l;   // this lane's share of the running sum

  __device__ void init() {
    m = kNegInf;
    l = 0.f;
#pragma unroll
    for (int j = 0; j < TR::EPB; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // rescales the running state when the reference point moves by log2(alpha)
  __device__ void rescale(float alpha) {
    l *= alpha;
#pragma unroll
    for (int j = 0; j < TR::EPB; ++j) acc[j] *= alpha;
  }
  // adds this block's weights (this lane's 8) to the running sum
  __device__ void add_sum(const f32x4& p0, const f32x4& p1) {
    l += (p0[0] + p0[1]) + (p0[2] + p0[3]) + (p1[0] + p1[1]) + (p1[2] + p1[3]);
  }

  // One 32-token tile: K operands of the two 16-token halves, V operands, the
  // number of valid tokens (tokens >= valid are masked) and the score scale.
  __device__ void tile(const typename TR::KOp (&k0)[TR::KS], const typename TR::KOp (&k1)[TR::KS],
                       const typename TR::VOp& vo, int valid, int g, float c) {
    f32x4 s0 = TR::qk(k0, q);
    f32x4 s1 = TR::qk(k1, q);
    if (valid < 32) {
      // partial tile (the last of a range): the compares stay behind the
      // branch (opaque bound), off the path of full tiles
      int v = __builtin_amdgcn_readfirstlane(valid);
      asm volatile("" : "+s"(v));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (4 * g + i >= v) s0[i] = kNegInf;
        if (16 + 4 * g + i >= v) s1[i] = kNegInf;
      }
    }
    // Lazy rescaling: the reference point m of a column only moves when one
    // of its scores exceeds it by more than kLazy (log2 units), so
    // p = 2^(s*c - m) < 2^kLazy and the accumulators are rescaled rarely (the
    // first tile and genuine jumps).  The common path needs no cross-lane
    // reduction: a wave vote on the lane-local maxima decides; only then is
    // the column maximum formed (across the four lane groups) and m moved.
    // Numerator and denominator share m, so the result does not change.
    const float lmx = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])),
                            fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3]))) * c;
    if (__any(lmx > m + kLazy)) {
      const float m_new = fmaxf(m, wave_max_groups(lmx));
      rescale(__builtin_amdgcn_exp2f(m - m_new));
      m = m_new;
    }
    f32x4 p0, p1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p0[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[i], c, -m));
      p1[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[i], c, -m));
    }
    add_sum(p0, p1);
    TR::pv(acc, vo, p0, p1);
  }

  // Normalised output slice of this lane (D/4 values for d = (D/4) g ..) and
  // the base-2 lse of the column.  out[EPB*i + j] = acc[j][i] / l_total.
  __device__ float finish(float (&o)[D / 4]) {
    const float lt = wave_sum_groups(l);
    const float inv = 1.f / lt;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < TR::EPB; ++j) o[TR::EPB * i + j] = acc[j][i] * inv;
    return m + __log2f(lt);
  }
};

// One 32-token tile for RB row blocks that share the K/V operands, in
// phases: all QK^T products, then all softmax updates, then all PV
// products.  The row blocks' dependency chains are independent, so each
// phase's work for one row block overlaps the latency of another's.  Same
// arithmetic, per row block, as ColState::tile.
template <typename T, int D, int RB>
__device__ __forceinline__ void tile_rows(ColState<T, D> (&st)[RB], const typename Traits<T, D>::KOp (&k0)[Traits<T, D>::KS],
                                          const typename Traits<T, D>::KOp (&k1)[Traits<T, D>::KS],
                                          const typename Traits<T, D>::VOp& vo, int valid, int g, float c) {
  using TR = Traits<T, D>;
  f32x4 s0[RB], s1[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    s0[rb] = TR::qk(k0, st[rb].q);
    s1[rb] = TR::qk(k1, st[rb].q);
  }
  if (valid < 32) {
    int v = __builtin_amdgcn_readfirstlane(valid);
    asm volatile("" : "+s"(v));
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (4 * g + i >= v) s0[rb][i] = kNegInf;
        if (16 + 4 * g + i >= v) s1[rb][i] = kNegInf;
      }
  }
  f32x4 p0[RB], p1[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    ColState<T, D>& cs = st[rb];
    const float lmx = fmaxf(fmaxf(fmaxf(s0[rb][0], s0[rb][1]), fmaxf(s0[rb][2], s0[rb][3])),
                            fmaxf(fmaxf(s1[rb][0], s1[rb][1]), fmaxf(s1[rb][2], s1[rb][3]))) * c;
    if (__any(lmx > cs.m + kLazy)) {
      const float m_new = fmaxf(cs.m, wave_max_groups(lmx));
      cs.rescale(__builtin_amdgcn_exp2f(cs.m - m_new));
      cs.m = m_new;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p0[rb][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[rb][i], c, -cs.m));
      p1[rb][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[rb][i], c, -cs.m));
    }
    cs.add_sum(p0[rb], p1[rb]);
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) TR::pv(st[rb].acc, vo, p0[rb], p1[rb]);
}

// The same per-block arithmetic as tile_rows, in pieces for a software
// pipeline that overlaps the QK^T products of the next block (matrix cores)
// with the softmax of the current one (VALU).
// S^T tiles of one block for the RB row blocks.
template <typename T, int D, int RB>
__device__ __forceinline__ void qk_rows(const ColState<T, D> (&st)[RB], const typename Traits<T, D>::KOp (&k0)[Traits<T, D>::KS],
                                        const typename Traits<T, D>::KOp (&k1)[Traits<T, D>::KS], f32x4 (&s0)[RB],
                                        f32x4 (&s1)[RB]) {
  using TR = Traits<T, D>;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    s0[rb] = TR::qk(k0, st[rb].q);
    s1[rb] = TR::qk(k1, st[rb].q);
  }
}
// Masks tokens >= valid and moves the reference points (lazy rescaling, one
// wave vote for all row blocks; rare).
template <typename T, int D, int RB>
__device__ __forceinline__ void softmax_ref(ColState<T, D> (&st)[RB], f32x4 (&s0)[RB], f32x4 (&s1)[RB], int valid, int g,
                                            float c) {
  if (valid < 32) {
    int v = __builtin_amdgcn_readfirstlane(valid);
    asm volatile("" : "+s"(v));
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (4 * g + i >= v) s0[rb][i] = kNegInf;
        if (16 + 4 * g + i >= v) s1[rb][i] = kNegInf;
      }
  }
  float lmx[RB];
  bool jump = false;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    lmx[rb] = fmaxf(fmaxf(fmaxf(s0[rb][0], s0[rb][1]), fmaxf(s0[rb][2], s0[rb][3])),
                    fmaxf(fmaxf(s1[rb][0], s1[rb][1]), fmaxf(s1[rb][2], s1[rb][3]))) * c;
    jump = jump || lmx[rb] > st[rb].m + kLazy;
  }
  if (__any(jump)) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      ColState<T, D>& cs = st[rb];
      const float m_new = fmaxf(cs.m, wave_max_groups(lmx[rb]));
      cs.rescale(__builtin_amdgcn_exp2f(cs.m - m_new));
      cs.m = m_new;
    }
  }
}
// The pipelined prefix loop keeps a block's scores as y = s*c - m, formed
// when the block's QK^T product is done (beside the PV products of the block
// before), so that the weights exp2(y) cost the VALU no scale and subtract
// beside the next QK^T products.  softmax_ref_y masks tokens >= valid, forms
// y against the current reference points and moves them lazily (a column's y
// above kLazy: rare), shifting the state and this block's y with them; the
// reference points must be set (the first block of a split goes through
// softmax_ref and shift_scores).
template <int RB>
__device__ __forceinline__ void shift_scores(f32x4 (&s0)[RB], f32x4 (&s1)[RB], const float (&m)[RB], float c) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s0[rb][i] = __builtin_fmaf(s0[rb][i], c, -m[rb]);
      s1[rb][i] = __builtin_fmaf(s1[rb][i], c, -m[rb]);
    }
}
template <typename T, int D, int RB>
__device__ __forceinline__ void softmax_ref_y(ColState<T, D> (&st)[RB], f32x4 (&s0)[RB], f32x4 (&s1)[RB], int valid,
                                              int g, float c) {
  if (valid < 32) {
    int v = __builtin_amdgcn_readfirstlane(valid);
    asm volatile("" : "+s"(v));
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (4 * g + i >= v) s0[rb][i] = kNegInf;
        if (16 + 4 * g + i >= v) s1[rb][i] = kNegInf;
      }
  }
  float m[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) m[rb] = st[rb].m;
  shift_scores<RB>(s0, s1, m, c);
  float lmx[RB];
  bool jump = false;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    lmx[rb] = fmaxf(fmaxf(fmaxf(s0[rb][0], s0[rb][1]), fmaxf(s0[rb][2], s0[rb][3])),
                    fmaxf(fmaxf(s1[rb][0], s1[rb][1]), fmaxf(s1[rb][2], s1[rb][3])));
    jump = jump || lmx[rb] > kLazy;
  }
  if (__any(jump)) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      ColState<T, D>& cs = st[rb];
      const float d = fmaxf(wave_max_groups(lmx[rb]), 0.f);
      cs.rescale(__builtin_amdgcn_exp2f(-d));
      cs.m += d;
      s0[rb] -= d;
      s1[rb] -= d;
    }
  }
}
// Weights exp2(y) of one block (no row sums: those go beside the PV
// products).
template <int RB>
__device__ __forceinline__ void softmax_py(const f32x4 (&y0)[RB], const f32x4 (&y1)[RB], f32x4 (&p0)[RB],
                                           f32x4 (&p1)[RB]) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p0[rb][i] = __builtin_amdgcn_exp2f(y0[rb][i]);
      p1[rb][i] = __builtin_amdgcn_exp2f(y1[rb][i]);
    }
}

// Partials cross workgroups (and XCDs, whose L2 caches are not coherent
// with one another) inside one launch, so they are written and read with
// agent-scope relaxed atomic accesses: these bypass the non-coherent cache
// state instead of needing cache-wide write-back / invalidate.  A writer
// waits for its stores to complete before the arrival that publishes them.
__device__ __forceinline__ void store_partial(float* dst, float v) {
  __hip_atomic_store(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// n consecutive floats from o to dst (n even, dst 8-byte aligned)
__device__ __forceinline__ void store_partial_row(float* dst, const float* o, int n) {
  for (int k = 0; k < n; k += 2) {
    const uint64_t w = static_cast<uint64_t>(__builtin_bit_cast(uint32_t, o[k])) |
                       (static_cast<uint64_t>(__builtin_bit_cast(uint32_t, o[k + 1])) << 32);
    __hip_atomic_store(reinterpret_cast<uint64_t*>(dst + k), w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}
__device__ __forceinline__ float load_partial(const float* src) {
  return __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <int PER>
__device__ __forceinline__ void load_partial_row(const float* src, float (&v)[PER]) {
  if constexpr (PER == 2) {
    const uint64_t w = __hip_atomic_load(reinterpret_cast<const uint64_t*>(src), __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    v[0] = __builtin_bit_cast(float, static_cast<uint32_t>(w));
    v[1] = __builtin_bit_cast(float, static_cast<uint32_t>(w >> 32));
  } else {
#pragma unroll
    for (int j = 0; j < PER; ++j) v[j] = load_partial(src + j);
  }
}
// PER consecutive values of a partial row in the input dtype T (PER even
// or T = float): 32-bit (two bf16) or 64-bit (two fp32) agent-scope accesses
template <typename T, int PER>
__device__ __forceinline__ void store_partial_vals(T* dst, const float (&v)[PER]) {
  if constexpr (sizeof(T) == 2 && PER == 1) {
    __hip_atomic_store(reinterpret_cast<uint16_t*>(dst), __builtin_bit_cast(uint16_t, static_cast<__bf16>(v[0])),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else if constexpr (sizeof(T) == 2) {
    static_assert(PER % 2 == 0, "bf16 partial slices: one or an even number");
#pragma unroll
    for (int k = 0; k < PER; k += 2) {
      const uint32_t w = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(v[k]))) |
                         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(v[k + 1]))) << 16);
      __hip_atomic_store(reinterpret_cast<uint32_t*>(dst + k), w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  } else if constexpr (PER % 2 == 0) {
    store_partial_row(reinterpret_cast<float*>(dst), v, PER);
  } else {
#pragma unroll
    for (int k = 0; k < PER; ++k) store_partial(reinterpret_cast<float*>(dst) + k, v[k]);
  }
}
template <typename T, int PER>
__device__ __forceinline__ void load_partial_vals(const T* src, float (&v)[PER]) {
  if constexpr (sizeof(T) == 2 && PER == 1) {
    const uint16_t w = __hip_atomic_load(reinterpret_cast<const uint16_t*>(src), __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    v[0] = static_cast<float>(__builtin_bit_cast(__bf16, w));
  } else if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int k = 0; k < PER; k += 2) {
      const uint32_t w = __hip_atomic_load(reinterpret_cast<const uint32_t*>(src + k), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
      v[k] = static_cast<float>(__builtin_bit_cast(__bf16, static_cast<uint16_t>(w)));
      v[k + 1] = static_cast<float>(__builtin_bit_cast(__bf16, static_cast<uint16_t>(w >> 16)));
    }
  } else {
    load_partial_row<PER>(reinterpret_cast<const float*>(src), v);
  }
}

// all of this wave's partial stores have completed
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// cache-policy operand of the buffer intrinsics: sc1, the bit the compiler
// sets for agent-scope atomic stores (write through to every XCD's view)
constexpr int kCachePolicySc1 = 16;

// One 16-byte piece of a partial row, written through to where every XCD
// reads it (sc1), by compiler-emitted stores: a store of more than 8 bytes
// reads its data registers after issue, and only the compiler's hazard
// tracking keeps the next instructions from overwriting them (an inline-asm
// 16-byte store lost the last lanes' data that way).  With `narrow` (the
// host's word that the whole workspace spans less than 2 GB) it is one
// buffer store at a 32-bit offset from the first active lane's address,
// which must be the lowest; otherwise two agent-scope 64-bit stores.
__device__ __forceinline__ void store_chunk(void* dst, const u32x4& v, bool narrow) {
  if (narrow) {
    const uint64_t a64 = reinterpret_cast<uint64_t>(dst);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a64));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a64 >> 32));
    const uint64_t b64 = (static_cast<uint64_t>(hi) << 32) | lo;
    // untyped 32-bit buffer format; no bound check needed beyond 2 GB
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(b64), static_cast<short>(0), 0x7fffffff, 0x00020000);
    __builtin_amdgcn_raw_buffer_store_b128(v, r, static_cast<uint32_t>(a64 - b64), 0, kCachePolicySc1);
    return;
  }
  uint64_t* p = static_cast<uint64_t*>(dst);
  const uint64_t lo = static_cast<uint64_t>(v[0]) | (static_cast<uint64_t>(v[1]) << 32);
  const uint64_t hi = static_cast<uint64_t>(v[2]) | (static_cast<uint64_t>(v[3]) << 32);
  __hip_atomic_store(p, lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(p + 1, hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16 bytes of a row from 16 / sizeof(T) floats (LDS), in the dtype T
template <typename T>
__device__ __forceinline__ u32x4 pack_chunk(const float* src) {
  if constexpr (sizeof(T) == 2) {
    const f32x4 x0 = reinterpret_cast<const f32x4*>(src)[0], x1 = reinterpret_cast<const f32x4*>(src)[1];
    auto two = [](float lo, float hi) {
      return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(lo))) |
             (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(hi))) << 16);
    };
    return u32x4{two(x0[0], x0[1]), two(x0[2], x0[3]), two(x1[0], x1[1]), two(x1[2], x1[3])};
  } else {
    // the whole vector at once (a bit_cast of one element of an ext_vector
    // lvalue reads element 0 with this compiler)
    return __builtin_bit_cast(u32x4, reinterpret_cast<const f32x4*>(src)[0]);
  }
}


// Joins the partial softmax results of one query head: np parts, part p has
// base-2 lse lse_of(p) and normalised output row whose PER elements at
// PER*lane load_o(p, v) fetches.  All loads of a batch of MB parts are
// issued before any is used.  Leaves the joined row slice in acc and
// returns the joined base-2 lse.
template <int PER, int MB, typename LseF, typename RowF>
__device__ __forceinline__ float join_parts(int np, int lane, LseF lse_of, RowF load_o, float (&acc)[PER]) {
  auto wave_max = [](float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
  };
  float mx = kNegInf;
  if (np > MB) {
    for (int base = 0; base < np; base += 64) mx = fmaxf(mx, base + lane < np ? lse_of(base + lane) : kNegInf);
    mx = wave_max(mx);
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) acc[j] = 0.f;
  float wsum = 0.f;
  for (int base = 0; base < np; base += MB) {
    const int cnt = min(MB, np - base);
    const float lp = lane < cnt ? lse_of(base + lane) : kNegInf;
    float v[MB][PER];
#pragma unroll
    for (int k = 0; k < MB; ++k)
      if (k < cnt) load_o(base + k, v[k]);
    if (np <= MB) mx = wave_max(lp);
    const float wl = lane < cnt && lp != kNegInf ? __builtin_amdgcn_exp2f(lp - mx) : 0.f;
    wsum += wl;
#pragma unroll
    for (int k = 0; k < MB; ++k)
      if (k < cnt) {
        const float wk = __shfl(wl, k);
#pragma unroll
        for (int j = 0; j < PER; ++j) acc[j] += wk * v[k][j];
      }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) wsum += __shfl_xor(wsum, off);
  // no tokens in any part (e.g. the suffix pieces of a prefix-only
  // request): an empty result, o = 0 and lse = -inf, so it weighs nothing
  if (!(wsum > 0.f)) {
#pragma unroll
    for (int j = 0; j < PER; ++j) acc[j] = 0.f;
    return kNegInf;
  }
  const float inv = 1.f / wsum;
#pragma unroll
  for (int j = 0; j < PER; ++j) acc[j] *= inv;
  return mx + __log2f(wsum);
}

// ------------------------------------------------------- in-kernel join
// Where the partials of request b come from: its HOT class's n_splits prefix
// splits (rows (b * max_splits + s) * n_q + h of p_o / p_lse) and its
// n_parts suffix parts from part c0 on (rows part * n_q + h of s_o / s_lse).
// suffix parts of a ranked request: at least one
__device__ __forceinline__ int parts_of(const RankDesc& rd) {
  return max(1, static_cast<int>((static_cast<int64_t>(rd.tok1) - rd.tok0 + kSuffixPart - 1) / kSuffixPart));
}
struct JoinSrc {
  int ns, c0, n_parts;
};
template <class A>
__device__ __forceinline__ JoinSrc join_src(const A& a, int b) {
  const RankDesc rd = a.ranks[table_at(a.rank_of, b)];
  const int cls = table_at(a.req_class, b);
  JoinSrc s;
  s.ns = cls >= 0 ? a.classes[cls].n_splits : 0;
  s.c0 = rd.part0;
  s.n_parts = parts_of(rd);
  return s;
}

// 16 bytes of a partial row with two agent-scope 64-bit loads
__device__ __forceinline__ u32x4 load_partial_chunk(const void* src) {
  const uint64_t* p = static_cast<const uint64_t*>(src);
  const uint64_t lo = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t hi = __hip_atomic_load(p + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return u32x4{static_cast<uint32_t>(lo), static_cast<uint32_t>(lo >> 32), static_cast<uint32_t>(hi),
               static_cast<uint32_t>(hi >> 32)};
}
// the 16 / sizeof(T) values of a 16-byte chunk
template <typename T>
__device__ __forceinline__ void unpack_chunk(const u32x4& w, float (&v)[16 / sizeof(T)]) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = __builtin_bit_cast(float, w[k] << 16);
      v[2 * k + 1] = __builtin_bit_cast(float, w[k] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t x = w[k];   // a scalar copy: bit_cast of a vector-element lvalue reads element 0
      v[k] = __builtin_bit_cast(float, x);
    }
  }
}

// One wave joins the partials of request b for query head h by log-sum-exp
// and writes out[b][h] (input dtype) and lse[b][h] (natural log).  Lane l
// reads 16-byte chunk l % CH of partial rows l / CH, l / CH + 64 / CH, ...,
// so one wave-wide access covers 64 / CH rows and a batch of up to 32
// partials is a handful of independent loads issued back to back (indices
// past the last partial repeat it and weigh zero).  The lane groups then sum
// their chunks with cross-lane adds.
template <typename T, int D, typename P, class A>
__device__ __forceinline__ void join_row(const A& a, const JoinSrc& src, int b, int h, int lane) {
  constexpr int CH = D * static_cast<int>(sizeof(P)) / 16;   // 16-byte chunks per partial row
  constexpr int RPI = 64 / CH;                                 // rows per wave-wide access
  constexpr int EPC = 16 / static_cast<int>(sizeof(P));      // values per chunk
  constexpr int NB = 32;                                       // partials per batch
  constexpr int NL = NB / RPI;                                 // chunk loads per lane per batch
  static_assert(CH <= 64 && 64 % CH == 0, "row chunks must tile the wave");
  const int ns = src.ns, c0 = src.c0, np = ns + src.n_parts;
  const int ch = lane % CH, rg = lane / CH;
  const size_t prow0 = static_cast<size_t>(b) * a.max_splits * a.n_q + h;
  auto row_of = [&](int p) -> size_t {   // row of partial p in p_o / p_lse (p < ns) or s_o / s_lse
    return p < ns ? prow0 + static_cast<size_t>(p) * a.n_q : static_cast<size_t>(c0 + p - ns) * a.n_q + h;
  };
  auto lse_of = [&](int p) { return load_partial((p < ns ? a.p_lse : a.s_lse) + row_of(p)); };
  auto chunk_of = [&](int p) {
    const P* base = static_cast<const P*>(p < ns ? a.p_o : a.s_o);
    return load_partial_chunk(base + row_of(p) * D + EPC * ch);
  };
  auto wave_max = [](float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
  };

  float mx = kNegInf;
  if (np > NB) {   // more partials than one batch: the common reference point first
    for (int base = 0; base < np; base += 64) mx = fmaxf(mx, base + lane < np ? lse_of(base + lane) : kNegInf);
    mx = wave_max(mx);
  }
  float acc[EPC];
#pragma unroll
  for (int j = 0; j < EPC; ++j) acc[j] = 0.f;
  float wsum = 0.f;
  for (int base = 0; base < np; base += NB) {
    const int cnt = min(NB, np - base);
    const float lp = lane < cnt ? lse_of(base + lane) : kNegInf;
    u32x4 raw[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) raw[i] = chunk_of(base + min(i * RPI + rg, cnt - 1));
    if (np <= NB) mx = wave_max(lp);
    const float wl = lane < cnt && lp != kNegInf ? __builtin_amdgcn_exp2f(lp - mx) : 0.f;
    wsum += wl;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const float w = __shfl(wl, i * RPI + rg);   // zero for rows past cnt
      float v[EPC];
      unpack_chunk<P>(raw[i], v);
#pragma unroll
      for (int j = 0; j < EPC; ++j) acc[j] += w * v[j];
    }
  }
#pragma unroll
  for (int off = CH; off < 64; off <<= 1)
#pragma unroll
    for (int j = 0; j < EPC; ++j) acc[j] += __shfl_xor(acc[j], off);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) wsum += __shfl_xor(wsum, off);
  // no tokens in any part: an empty result, o = 0 and lse = -inf
  const bool empty = !(wsum > 0.f);
  const float inv = empty ? 0.f : 1.f / wsum;
  if (rg == 0) {
    T* dst = static_cast<T*>(a.out) + (static_cast<size_t>(b) * a.n_q + h) * D + EPC * ch;
#pragma unroll
    for (int k = 0; k < EPC; ++k) dst[k] = static_cast<T>(acc[k] * inv);
  }
  if (lane == 0)
    a.lse[static_cast<size_t>(b) * a.n_q + h] = empty ? kNegInf : (mx + __log2f(wsum)) * 0.69314718055994531f;
}

// One wave joins request b's ns prefix partials for query head h with NL
// partials held in LDS (a suffix part joined in the workgroup that attended
// it: row p at loc_o + p * o_stride, D fp32 values, base-2 lse at
// loc_lse[p * l_stride]) and writes out[b][h] and lse[b][h].  Same
// arithmetic and load pattern as join_row; the LDS partials enter the
// reference point from the start and their weighted rows are added by lane
// group 0 before the cross-lane sum.
template <typename T, int D, typename P, int NL_LOC, class A>
__device__ __forceinline__ void join_local(const A& a, int ns, int b, int h, const float* loc_o, int o_stride,
                                           const float* loc_lse, int l_stride, int lane) {
  constexpr int CH = D * static_cast<int>(sizeof(P)) / 16;   // 16-byte chunks per partial row
  constexpr int RPI = 64 / CH;                                 // rows per wave-wide access
  constexpr int EPC = 16 / static_cast<int>(sizeof(P));      // values per chunk
  constexpr int NB = 32;                                       // partials per batch
  constexpr int NL = NB / RPI;                                 // chunk loads per lane per batch
  static_assert(CH <= 64 && 64 % CH == 0, "row chunks must tile the wave");
  const int ch = lane % CH, rg = lane / CH;
  const size_t prow0 = static_cast<size_t>(b) * a.max_splits * a.n_q + h;
  auto lse_of = [&](int p) { return load_partial(a.p_lse + prow0 + static_cast<size_t>(p) * a.n_q); };
  auto chunk_of = [&](int p) {
    return load_partial_chunk(static_cast<const P*>(a.p_o) + (prow0 + static_cast<size_t>(p) * a.n_q) * D + EPC * ch);
  };
  auto wave_max = [](float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
  };
  float llse[NL_LOC];
  float lmx = kNegInf;
#pragma unroll
  for (int p = 0; p < NL_LOC; ++p) {
    llse[p] = loc_lse[p * l_stride];
    lmx = fmaxf(lmx, llse[p]);
  }
  float mx = lmx;
  if (ns > NB) {
    float x = kNegInf;
    for (int base = 0; base < ns; base += 64) x = fmaxf(x, base + lane < ns ? lse_of(base + lane) : kNegInf);
    mx = fmaxf(lmx, wave_max(x));
  }
  float acc[EPC];
#pragma unroll
  for (int j = 0; j < EPC; ++j) acc[j] = 0.f;
  float wsum = 0.f;
  for (int base = 0; base < ns; base += NB) {
    const int cnt = min(NB, ns - base);
    const float lp = lane < cnt ? lse_of(base + lane) : kNegInf;
    u32x4 raw[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) raw[i] = chunk_of(base + min(i * RPI + rg, cnt - 1));
    if (ns <= NB) mx = fmaxf(lmx, wave_max(lp));
    const float wl = lane < cnt && lp != kNegInf ? __builtin_amdgcn_exp2f(lp - mx) : 0.f;
    wsum += wl;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const float w = __shfl(wl, i * RPI + rg);   // zero for rows past cnt
      float v[EPC];
      unpack_chunk<P>(raw[i], v);
#pragma unroll
      for (int j = 0; j < EPC; ++j) acc[j] += w * v[j];
    }
  }
  // the LDS partials (once: lane group 0; their weights join the sum once)
  float wloc = 0.f;
#pragma unroll
  for (int p = 0; p < NL_LOC; ++p) {
    const float w = llse[p] != kNegInf ? __builtin_amdgcn_exp2f(llse[p] - mx) : 0.f;
    wloc += w;
    if (rg == 0)
#pragma unroll
      for (int j = 0; j < EPC; ++j) acc[j] += w * loc_o[p * o_stride + EPC * ch + j];
  }
#pragma unroll
  for (int off = CH; off < 64; off <<= 1)
#pragma unroll
    for (int j = 0; j < EPC; ++j) acc[j] += __shfl_xor(acc[j], off);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) wsum += __shfl_xor(wsum, off);
  wsum += wloc;
  // no tokens in any part: an empty result, o = 0 and lse = -inf
  const bool empty = !(wsum > 0.f);
  const float inv = empty ? 0.f : 1.f / wsum;
  if (rg == 0) {
    T* dst = static_cast<T*>(a.out) + (static_cast<size_t>(b) * a.n_q + h) * D + EPC * ch;
#pragma unroll
    for (int k = 0; k < EPC; ++k) dst[k] = static_cast<T>(acc[k] * inv);
  }
  if (lane == 0)
    a.lse[static_cast<size_t>(b) * a.n_q + h] = empty ? kNegInf : (mx + __log2f(wsum)) * 0.69314718055994531f;
}

// join_local in two halves for up to 32 prefix partials, so that a wave can
// issue the loads of two joins before it waits for either: local_loads issues
// the lse and row-chunk loads, local_finish weighs them with the LDS
// partials and writes the output (same arithmetic as join_local).
template <int NL>
struct LocalLoads {
  float lp;
  u32x4 raw[NL];
};
template <typename T, int D, typename P, class A>
__device__ __forceinline__ LocalLoads<32 / (64 / (D * static_cast<int>(sizeof(P)) / 16))> local_loads(
    const A& a, int ns, int b, int h, int lane) {
  constexpr int CH = D * static_cast<int>(sizeof(P)) / 16;
  constexpr int RPI = 64 / CH;
  constexpr int EPC = 16 / static_cast<int>(sizeof(P));
  constexpr int NL = 32 / RPI;
  const int ch = lane % CH, rg = lane / CH;
  const size_t prow0 = static_cast<size_t>(b) * a.max_splits * a.n_q + h;
  LocalLoads<NL> r;
  r.lp = lane < ns ? load_partial(a.p_lse + prow0 + static_cast<size_t>(lane) * a.n_q) : kNegInf;
#pragma unroll
  for (int i = 0; i < NL; ++i)
    r.raw[i] = load_partial_chunk(static_cast<const P*>(a.p_o) +
                                  (prow0 + static_cast<size_t>(min(i * RPI + rg, ns - 1)) * a.n_q) * D + EPC * ch);
  return r;
}
template <typename T, int D, typename P, int NL_LOC, int NL, class A>
__device__ __forceinline__ void local_finish(const A& a, const LocalLoads<NL>& r, int ns, int b, int h,
                                             const float* loc_o, int o_stride, const float* loc_lse, int l_stride,
                                             int lane) {
  constexpr int CH = D * static_cast<int>(sizeof(P)) / 16;
  constexpr int RPI = 64 / CH;
  constexpr int EPC = 16 / static_cast<int>(sizeof(P));
  const int ch = lane % CH, rg = lane / CH;
  float llse[NL_LOC];
  float mx = r.lp;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
#pragma unroll
  for (int p = 0; p < NL_LOC; ++p) {
    llse[p] = loc_lse[p * l_stride];
    mx = fmaxf(mx, llse[p]);
  }
  const float wl = lane < ns && r.lp != kNegInf ? __builtin_amdgcn_exp2f(r.lp - mx) : 0.f;
  float acc[EPC];
#pragma unroll
  for (int j = 0; j < EPC; ++j) acc[j] = 0.f;
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const float w = __shfl(wl, i * RPI + rg);   // zero for rows past ns
    float v[EPC];
    unpack_chunk<P>(r.raw[i], v);
#pragma unroll
    for (int j = 0; j < EPC; ++j) acc[j] += w * v[j];
  }
  float wloc = 0.f;
#pragma unroll
  for (int p = 0; p < NL_LOC; ++p) {
    const float w = llse[p] != kNegInf ? __builtin_amdgcn_exp2f(llse[p] - mx) : 0.f;
    wloc += w;
    if (rg == 0)
#pragma unroll
      for (int j = 0; j < EPC; ++j) acc[j] += w * loc_o[p * o_stride + EPC * ch + j];
  }
#pragma unroll
  for (int off = CH; off < 64; off <<= 1)
#pragma unroll
    for (int j = 0; j < EPC; ++j) acc[j] += __shfl_xor(acc[j], off);
  float wsum = wl;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) wsum += __shfl_xor(wsum, off);
  wsum += wloc;
  const bool empty = !(wsum > 0.f);
  const float inv = empty ? 0.f : 1.f / wsum;
  if (rg == 0) {
    T* dst = static_cast<T*>(a.out) + (static_cast<size_t>(b) * a.n_q + h) * D + EPC * ch;
#pragma unroll
    for (int k = 0; k < EPC; ++k) dst[k] = static_cast<T>(acc[k] * inv);
  }
  if (lane == 0)
    a.lse[static_cast<size_t>(b) * a.n_q + h] = empty ? kNegInf : (mx + __log2f(wsum)) * 0.69314718055994531f;
}

// One wave's joins of request b (ns <= 32 prefix partials) for the query
// heads h0 + c, c = c0, c0 + cstep, ... < G, with NL_LOC partials in LDS per
// head (head c's at loc_o + c * D and loc_lse + c, the NL_LOC of one head
// o_stride and l_stride apart): three joins' loads are issued before any of
// them is finished.
template <typename T, int D, typename P, int NL_LOC, class A>
__device__ __forceinline__ void local_joins(const A& a, int ns, int b, int h0, int c0, int cstep, int G,
                                            const float* loc_o, int o_stride, const float* loc_lse, int l_stride,
                                            int lane) {
  constexpr int kInFlight = 3;
  for (int c = c0; c < G; c += kInFlight * cstep) {
    decltype(local_loads<T, D, P>(a, 1, 0, 0, lane)) r[kInFlight];
#pragma unroll
    for (int k = 0; k < kInFlight; ++k)
      if (c + k * cstep < G) r[k] = local_loads<T, D, P>(a, ns, b, h0 + c + k * cstep, lane);
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) {
      const int col = c + k * cstep;
      if (col < G)
        local_finish<T, D, P, NL_LOC>(a, r[k], ns, b, h0 + col, loc_o + col * D, o_stride, loc_lse + col, l_stride,
                                      lane);
    }
  }
}

// Joins the partials of request b for the G query heads of KV head gk, 64 /
// CH heads per pass: lane l takes 16-byte chunk l % CH of query head
// gk * G + l / CH and walks the partials itself, NB at a time with all their
// lse and chunk loads issued together, against a running reference point.
// One round trip per NB partials for a whole KV head (short requests have
// few partials per head: their prefix splits and their tile); a batch loads
// only its partials (the count is uniform across the wave).
template <typename T, int D, typename P, class A>
__device__ __forceinline__ void join_group(const A& a, const JoinSrc& src, int b, int gk, int lane) {
  constexpr int CH = D * static_cast<int>(sizeof(P)) / 16;   // 16-byte chunks per partial row
  constexpr int HP = 64 / CH;                                  // query heads per pass
  constexpr int EPC = 16 / static_cast<int>(sizeof(P));      // values per chunk
  constexpr int NB = 32;                                       // partials per batch
  static_assert(CH <= 64 && 64 % CH == 0, "row chunks must tile the wave");
  const int ns = src.ns, np = ns + src.n_parts, G = a.group;
  const int ch = lane % CH;
  for (int h0 = 0; h0 < G; h0 += HP) {
    const int col = h0 + lane / CH;
    const int h = gk * G + min(col, G - 1);
    const size_t prow0 = static_cast<size_t>(b) * a.max_splits * a.n_q + h;
    auto row_of = [&](int p) -> size_t {
      return p < ns ? prow0 + static_cast<size_t>(p) * a.n_q : static_cast<size_t>(src.c0 + p - ns) * a.n_q + h;
    };
    float m = kNegInf, wsum = 0.f;
    float acc[EPC];
#pragma unroll
    for (int j = 0; j < EPC; ++j) acc[j] = 0.f;
    for (int base = 0; base < np; base += NB) {
      const int cnt = min(NB, np - base);
      float lp[NB];
      u32x4 raw[NB];
#pragma unroll
      for (int k = 0; k < NB; ++k) {   // slots past the last partial weigh zero
        lp[k] = kNegInf;
        raw[k] = u32x4{0u, 0u, 0u, 0u};
        if (k < cnt) {
          const int p = base + k;
          lp[k] = load_partial((p < ns ? a.p_lse : a.s_lse) + row_of(p));
          raw[k] = load_partial_chunk(static_cast<const P*>(p < ns ? a.p_o : a.s_o) + row_of(p) * D + EPC * ch);
        }
      }
      float mb = m;
#pragma unroll
      for (int k = 0; k < NB; ++k) mb = fmaxf(mb, lp[k]);
      if (mb == kNegInf) continue;   // no tokens in any partial so far
      const float sc = __builtin_amdgcn_exp2f(m - mb);   // 0 while m is -inf
      wsum *= sc;
#pragma unroll
      for (int j = 0; j < EPC; ++j) acc[j] *= sc;
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const float wk = lp[k] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(lp[k] - mb);
        wsum += wk;
        float v[EPC];
        unpack_chunk<P>(raw[k], v);
#pragma unroll
        for (int j = 0; j < EPC; ++j) acc[j] += wk * v[j];
      }
      m = mb;
    }
    // no tokens in any partial: an empty result, o = 0 and lse = -inf
    const bool empty = !(wsum > 0.f);
    const float inv = empty ? 0.f : 1.f / wsum;
    if (col < G) {
      T* dst = static_cast<T*>(a.out) + (static_cast<size_t>(b) * a.n_q + h) * D + EPC * ch;
#pragma unroll
      for (int k = 0; k < EPC; ++k) dst[k] = static_cast<T>(acc[k] * inv);
      if (ch == 0)
        a.lse[static_cast<size_t>(b) * a.n_q + h] = empty ? kNegInf : (m + __log2f(wsum)) * 0.69314718055994531f;
    }
  }
}

// Joins up to NU units, unit u being the pass h0[u] (query heads
// gk[u] * G + h0[u] .. + 64 / CH) of KV head gk[u] of request b[u] with
// partials src[u], when every unit has at most NB partials: the lse and
// chunk loads of all the units are issued before any is used, so the set
// costs one round trip (join_group takes one per KV head).  Same arithmetic
// as join_group; units u >= nu are skipped.
template <typename T, int D, typename P, int NB, int NU, class A>
__device__ __forceinline__ void join_units(const A& a, const JoinSrc (&src)[NU], const int (&b)[NU],
                                           const int (&gk)[NU], const int (&h0)[NU], int nu, int lane) {
  constexpr int CH = D * static_cast<int>(sizeof(P)) / 16;   // 16-byte chunks per partial row
  constexpr int EPC = 16 / static_cast<int>(sizeof(P));      // values per chunk
  const int G = a.group;
  const int ch = lane % CH;
  float lp[NU][NB];
  u32x4 raw[NU][NB];
  int h[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    h[u] = gk[u] * G + min(h0[u] + lane / CH, G - 1);
    const int ns = src[u].ns, np = ns + src[u].n_parts;
    const size_t prow0 = static_cast<size_t>(b[u]) * a.max_splits * a.n_q + h[u];
#pragma unroll
    for (int k = 0; k < NB; ++k) {   // slots past the last partial weigh zero
      lp[u][k] = kNegInf;
      raw[u][k] = u32x4{0u, 0u, 0u, 0u};
      if (u < nu && k < np) {
        const size_t row = k < ns ? prow0 + static_cast<size_t>(k) * a.n_q
                                  : static_cast<size_t>(src[u].c0 + k - ns) * a.n_q + h[u];
        lp[u][k] = load_partial((k < ns ? a.p_lse : a.s_lse) + row);
        raw[u][k] = load_partial_chunk(static_cast<const P*>(k < ns ? a.p_o : a.s_o) + row * D + EPC * ch);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    if (u >= nu) break;
    float m = kNegInf;
#pragma unroll
    for (int k = 0; k < NB; ++k) m = fmaxf(m, lp[u][k]);
    float wsum = 0.f, acc[EPC];
#pragma unroll
    for (int j = 0; j < EPC; ++j) acc[j] = 0.f;
    if (m != kNegInf) {
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const float wk = lp[u][k] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(lp[u][k] - m);
        wsum += wk;
        float v[EPC];
        unpack_chunk<P>(raw[u][k], v);
#pragma unroll
        for (int j = 0; j < EPC; ++j) acc[j] += wk * v[j];
      }
    }
    // no tokens in any partial: an empty result, o = 0 and lse = -inf
    const bool empty = !(wsum > 0.f);
    const float inv = empty ? 0.f : 1.f / wsum;
    if (h0[u] + lane / CH < G) {
      T* dst = static_cast<T*>(a.out) + (static_cast<size_t>(b[u]) * a.n_q + h[u]) * D + EPC * ch;
#pragma unroll
      for (int k = 0; k < EPC; ++k) dst[k] = static_cast<T>(acc[k] * inv);
      if (ch == 0)
        a.lse[static_cast<size_t>(b[u]) * a.n_q + h[u]] = empty ? kNegInf : (m + __log2f(wsum)) * 0.69314718055994531f;
    }
  }
}

// Counts the arrival of one partial of (request b, KV head g).  Protocol:
// every wave of the arriving workgroup has stored its partial rows with
// agent-scope accesses and waited for them to complete, then the workgroup
// barrier; only then is the arrival counted, so a count seen by the join
// workgroup means the partial is in place.
template <class A>
__device__ __forceinline__ void arrive(const A& a, int b, int g) {
  __hip_atomic_fetch_add(a.counters + static_cast<size_t>(b) * a.n_kv + g, 1, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
}

// Waits until all n partials of (request b, KV head g) have arrived, then
// takes n off the counter for the next call.  One thread calls it.
//
// The wait is bounded by a.spin_limit polls (an agent-scope load plus a short
// sleep each; the default bound, about 0.1 s, is far beyond any step), so the
// kernel ends even if a count were never to arrive.  A join that stops
// waiting adds one to the workspace's status word (read by the host with
// gkv_step_status) and joins whatever the partials hold; its output is not
// valid.  Taking n off (instead of storing zero) keeps the counters exact
// for the next call in that case too: the late arrivals of this call still
// land before the kernel ends, and bring the counter back to zero.
template <class A>
__device__ __forceinline__ void wait_arrivals(const A& a, int b, int g, int n) {
  int32_t* cnt = a.counters + static_cast<size_t>(b) * a.n_kv + g;
  bool arrived = false;
  for (int it = 0; it < a.spin_limit; ++it) {
    if (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= n) {
      arrived = true;
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  if (!arrived) {
    arrived = __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= n;
    if (!arrived) __hip_atomic_fetch_add(a.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __hip_atomic_fetch_add(cnt, -n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// wait_arrivals for two (request, KV head g) counters at once (b2 < 0: one):
// each poll loads both, so the two waits cost one round trip, not two.
template <class A>
__device__ __forceinline__ void wait_arrivals2(const A& a, int b1, int n1, int b2, int n2, int g) {
  if (b2 < 0) {
    wait_arrivals(a, b1, g, n1);
    return;
  }
  int32_t* c1 = a.counters + static_cast<size_t>(b1) * a.n_kv + g;
  int32_t* c2 = a.counters + static_cast<size_t>(b2) * a.n_kv + g;
  bool ok1 = false, ok2 = false;
  for (int it = 0; it < a.spin_limit && !(ok1 && ok2); ++it) {
    const int32_t v1 = __hip_atomic_load(c1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int32_t v2 = __hip_atomic_load(c2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    ok1 = ok1 || v1 >= n1;
    ok2 = ok2 || v2 >= n2;
    if (!(ok1 && ok2)) __builtin_amdgcn_s_sleep(1);
  }
  if (!ok1) ok1 = __hip_atomic_load(c1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= n1;
  if (!ok2) ok2 = __hip_atomic_load(c2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= n2;
  if (!ok1) __hip_atomic_fetch_add(a.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (!ok2) __hip_atomic_fetch_add(a.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_fetch_add(c1, -n1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_fetch_add(c2, -n2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------ timeline
// Records of gkv_step_trace (see kTraceWords): one thread per workgroup
// writes its start, its marks and its end.
template <class A>
__device__ __forceinline__ void trace_start(const A& a, int blk, uint32_t kind) {
  // HW_ID (hardware register 4) and XCC_ID (20), whole 32-bit fields
  const uint32_t hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);
  const uint32_t xcc = __builtin_amdgcn_s_getreg((31 << 11) | 20) & 0xf;
  uint64_t* r = a.trace + static_cast<size_t>(blk) * kTraceWords;
  r[kTraceStart] = __builtin_amdgcn_s_memrealtime();
  r[kTraceMark] = 0;
  r[kTraceMark2] = 0;
  r[kTraceMark3] = 0;
  r[kTraceKind] = (static_cast<uint64_t>(kind) << 32) | (xcc << 16) | (hw & 0xffff);
}
template <class A>
__device__ __forceinline__ void trace_mark(const A& a, int blk, int word = kTraceMark) {
  if (a.trace && threadIdx.x == 0)
    a.trace[static_cast<size_t>(blk) * kTraceWords + word] = __builtin_amdgcn_s_memrealtime();
}

// ------------------------------------------------------------ suffix blocks
// One (suffix part, KV head) per call; see StepArgs.  Each wave runs the
// online softmax over its quarter of the part through the slot table and the
// four results meet in LDS.  A request without a HOT prefix whose slot table
// is one part is finished here; otherwise the part's partial is written for
// the request's join workgroup.
template <typename T, int D>
struct SuffixSmem {
  int32_t ids[kWaves][kWaveTokens];
  float o[kWaves][16][D];
  float lse[kWaves][16];
  // the merged result of a folded pair's first part, joined at the end of
  // the pair (suffix joins)
  float keep_o[16][D];
  float keep_lse[16];
};

// What a suffix part does with its four wave results: publish them (the
// part's partial, counted for its join workgroup, or the request's output),
// keep their merge in LDS for the workgroup's join at the end of a folded
// pair (first part), or leave them in LDS for that join (last part).  A
// request without a HOT prefix is always finished in place.
enum class PartEnd { kPublish, kKeep, kLeave };

// A wave's piece of one suffix part: the part's request b, the end tb1 of
// its slot-table range, and the wave's quarter [w0, w0 + len) of the part
// (quarters are whole 32-token tiles, `piece` tokens long but the last).
struct SuffixPiece {
  int b, w0, len, tb1, piece;
  bool single;   // the request's slot table is this one part
};
template <class A>
__device__ __forceinline__ SuffixPiece suffix_piece(const A& a, int part, int wave) {
  // rank: the last r with ranks[r].part0 <= part, which is the part itself
  // when every request has one part
  int lo = part;
  if (a.multi_part) {
    lo = 0;
    int hi = a.batch - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.ranks[mid].part0 <= part) lo = mid; else hi = mid - 1;
    }
  }
  const RankDesc rd = a.ranks[lo];
  const int j = part - rd.part0;
  const int tb0 = rd.tok0, tb1 = rd.tok1;
  const int p0 = min(tb1, tb0 + j * kSuffixPart), p1 = min(tb1, p0 + kSuffixPart);
  SuffixPiece pc;
  pc.b = rd.req;
  pc.tb1 = tb1;
  pc.single = parts_of(rd) == 1;
  pc.piece = (((p1 - p0 + kWaves - 1) / kWaves) + kSuffixTile - 1) / kSuffixTile * kSuffixTile;
  pc.w0 = min(p1, p0 + wave * pc.piece);
  pc.len = min(p1, pc.w0 + pc.piece) - pc.w0;
  return pc;
}

// The four wave results of one part meet in LDS (slot w = wave w's piece):
// wave w joins columns w, w+4, ... and writes the request's output (a
// request without a HOT prefix whose slot table is this one part) or the
// part's partial.  Returns true for the former.
template <typename T, int D, typename P, class A>
__device__ __forceinline__ bool suffix_publish(const A& a, SuffixSmem<T, D>& sm, int part, int b,
                                               bool single, int gk, int wave, int lane) {
  constexpr int PER = D / 64;
  const int G = a.group;
  const bool final_here = single && table_at(a.req_class, b) < 0;
  for (int col = wave; col < G; col += kWaves) {
    const int hc = gk * G + col;
    float acc[PER];
    const float l2 = join_parts<PER, 4>(
        kWaves, lane, [&](int p) { return sm.lse[p][col]; },
        [&](int p, float (&v)[PER]) {
#pragma unroll
          for (int j = 0; j < PER; ++j) v[j] = sm.o[p][col][PER * lane + j];
        },
        acc);
    if (final_here) {
      T* dst = static_cast<T*>(a.out) + (static_cast<size_t>(b) * a.n_q + hc) * D + PER * lane;
#pragma unroll
      for (int k = 0; k < PER; ++k) dst[k] = static_cast<T>(acc[k]);
      if (lane == 0) a.lse[static_cast<size_t>(b) * a.n_q + hc] = l2 * 0.69314718055994531f;
    } else {
      const size_t row = static_cast<size_t>(part) * a.n_q + hc;
      store_partial_vals<P, PER>(static_cast<P*>(a.s_o) + row * D + PER * lane, acc);
      if (lane == 0) store_partial(a.s_lse + row, l2);
    }
  }
  return final_here;
}

// A wave's result for one part into its LDS slot (column n, lane group g).
template <typename T, int D>
__device__ __forceinline__ void suffix_to_lds(SuffixSmem<T, D>& sm, int wave, int n, int g, bool col_ok,
                                              const float (&o)[D / 4], float lse2) {
  if (col_ok) {
#pragma unroll
    for (int k = 0; k < D / 16; ++k)
      *reinterpret_cast<f32x4*>(&sm.o[wave][n][(D / 4) * g + 4 * k]) =
          f32x4{o[4 * k], o[4 * k + 1], o[4 * k + 2], o[4 * k + 3]};
    if (g == 0) sm.lse[wave][n] = lse2;
  }
}

// Fused decode step: copies KV head gk's share of request b's new token
// (k_new/v_new row) into its COLD slot; slots outside the pool are skipped.
// The eight KV-head workgroups of the part write the whole row; nothing else
// reads that slot in the step.
template <typename T, int D, class A>
__device__ __forceinline__ void suffix_copy_new(const A& a, int b, int gk, int lane) {
  constexpr int CH = D * static_cast<int>(sizeof(T)) / 16;   // 16-byte chunks per row
  static_assert(CH <= 32, "a row copy takes at most half a wave");
  const int slot = a.new_slots[b];
  if (slot >= 0 && slot < a.cold_cap) {
    const size_t new_row = (static_cast<size_t>(b) * a.n_kv + gk) * D;
    const size_t dst = (static_cast<size_t>(slot) * a.n_kv + cold_row_pos(gk, slot, a.cold_mask)) * D;
    const int ch = lane & 31;
    const T* src = static_cast<const T*>(lane < 32 ? a.k_new : a.v_new) + new_row;
    T* to = static_cast<T*>(const_cast<void*>(lane < 32 ? a.k_cold : a.v_cold)) + dst;
    if (ch < CH) reinterpret_cast<u32x4*>(to)[ch] = reinterpret_cast<const u32x4*>(src)[ch];
  }
}

template <typename T, int D, typename P, class A>
__device__ __forceinline__ void suffix_part(const A& a, int part, int gk, uint8_t* smem_raw, PartEnd end) {
  using TR = Traits<T, D>;
  using KOp = typename TR::KOp;
  using VVec = typename TR::VVec;
  SuffixSmem<T, D>& sm = *reinterpret_cast<SuffixSmem<T, D>*>(smem_raw);
  auto& lds_ids = sm.ids;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: so are the loop bounds
  const SuffixPiece pc = suffix_piece(a, part, wave);
  const int b = pc.b, w0 = pc.w0, len = pc.len, tb1 = pc.tb1;
  const bool single = pc.single;

  const int n = lane & 15, g = lane >> 4;
  const int G = a.group;
  const bool col_ok = n < G;
  const int h = gk * G + (col_ok ? n : 0);
  const float c = a.scale_log2;

  float lse2 = kNegInf;
  float o[D / 4];
#pragma unroll
  for (int k = 0; k < D / 4; ++k) o[k] = 0.f;
  if (len > 0) {
    const size_t stride = static_cast<size_t>(a.n_kv) * D;
    const T* kc = static_cast<const T*>(a.k_cold);
    const T* vc = static_cast<const T*>(a.v_cold) + TR::EPB * n;
    const int mask = a.cold_mask;
    const int n_tiles = (len + kSuffixTile - 1) / kSuffixTile;
    const int cap1 = a.cold_cap - 1;
    // Fused decode step: the wave whose piece ends the slot table reads the
    // table's last token (the request's new one) from k_new/v_new, and
    // copies this KV head's share of it into the new slot.
    const bool fresh = a.k_new != nullptr && w0 + len == tb1;
    const size_t new_row = (static_cast<size_t>(b) * a.n_kv + gk) * D;
    const T* knew = static_cast<const T*>(a.k_new) + new_row;
    const T* vnew = static_cast<const T*>(a.v_new) + new_row + TR::EPB * n;
    if (fresh) suffix_copy_new<T, D>(a, b, gk, lane);

    // the piece's slot ids, clamped into the pool, staged in this wave's
    // LDS row once: no tile waits on a slot-id load.  The loads of 256 ids
    // are issued before the first is used (one round trip per 256 ids).
    int32_t* ids = lds_ids[wave];
    for (int base = 0; base < len; base += 256) {
      int32_t raw[4];
#pragma unroll
      for (int ck = 0; ck < 4; ++ck) raw[ck] = a.cold_indices[w0 + min(base + 64 * ck + lane, len - 1)];
#pragma unroll
      for (int ck = 0; ck < 4; ++ck)
        if (base + 64 * ck + lane < len) ids[base + 64 * ck + lane] = min(max(raw[ck], 0), cap1);
    }
    // a fresh wave's last position is the new token: id -1 sends its loads to
    // k_new / v_new (the same wave wrote the position above, in order)
    if (fresh && lane == 0) ids[len - 1] = -1;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // the query row after the slot ids: the ids' wait does not cover it
    ColState<T, D> st;
    st.init();
    if (col_ok) TR::load_row(st.q, static_cast<const T*>(a.q) + (static_cast<size_t>(b) * a.n_q + h) * D, g);
    else TR::zero_row(st.q);

    // Slot id -1 (the new token) reads k_new / v_new.  One branch-free load
    // sequence serves every tile: with a separate sequence for the fresh
    // tile the compiler merged the two, and a V load common to both then sank
    // below the QK^T of the tile, which waits for K, so each tile cost two
    // memory round trips.
    auto row = [&](const T* pool, const T* fresh_row, int id) {
      const int s = max(id, 0);
      const T* p = pool + static_cast<size_t>(s) * stride + cold_row_pos(gk, s, mask) * D;
      return id < 0 ? fresh_row : p;
    };
    auto load_kv = [&](int i, KOp (&k0)[TR::KS], KOp (&k1)[TR::KS], VVec (&v)[8]) {
      const int base = kSuffixTile * i, last = len - 1;
      TR::load_row(k0, row(kc, knew, ids[min(base + n, last)]), g);
      TR::load_row(k1, row(kc, knew, ids[min(base + 16 + n, last)]), g);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = TR::load_v(row(vc, vnew, ids[min(base + tau(g, e), last)]));
    };
    auto run_tile = [&](const KOp (&k0)[TR::KS], const KOp (&k1)[TR::KS], const VVec (&v)[8], int i) {
      typename TR::VOp vo;
      TR::make_vop(vo, v);
      st.tile(k0, k1, vo, min(kSuffixTile, len - kSuffixTile * i), g, c);
    };

    // bf16: two register sets, so tile i + 1's loads are in flight while
    // tile i is computed.  Every load sits outside any branch (the loop is
    // peeled), so each tile waits only for its own loads, never for the
    // younger set.  fp32 operands are twice the registers: one set.
    KOp ka0[TR::KS], ka1[TR::KS];
    VVec va[8];
    load_kv(0, ka0, ka1, va);
    int i = 0;
    if constexpr (sizeof(T) == 2) {
      KOp kb0[TR::KS], kb1[TR::KS];
      VVec vb[8];
      for (; i + 2 < n_tiles; i += 2) {
        load_kv(i + 1, kb0, kb1, vb);
        __builtin_amdgcn_sched_barrier(0);
        run_tile(ka0, ka1, va, i);
        __builtin_amdgcn_sched_barrier(0);
        load_kv(i + 2, ka0, ka1, va);
        __builtin_amdgcn_sched_barrier(0);
        run_tile(kb0, kb1, vb, i + 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (i + 1 < n_tiles) {
        load_kv(i + 1, kb0, kb1, vb);
        __builtin_amdgcn_sched_barrier(0);
        run_tile(ka0, ka1, va, i);
        __builtin_amdgcn_sched_barrier(0);
        run_tile(kb0, kb1, vb, i + 1);
        i = n_tiles;
      }
    } else {
      for (; i + 1 < n_tiles; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        run_tile(ka0, ka1, va, i);
        __builtin_amdgcn_sched_barrier(0);
        load_kv(i + 1, ka0, ka1, va);
      }
    }
    if (i < n_tiles) {
      __builtin_amdgcn_sched_barrier(0);
      run_tile(ka0, ka1, va, i);
    }
    lse2 = st.finish(o);
  }

  // the wave pieces meet in LDS
  suffix_to_lds<T, D>(sm, wave, n, g, col_ok, o, lse2);
  __syncthreads();
  if (end != PartEnd::kPublish && table_at(a.req_class, b) >= 0) {
    if (end == PartEnd::kKeep) {
      constexpr int PER = D / 64;
      for (int col = wave; col < G; col += kWaves) {
        float acc[PER];
        const float l2 = join_parts<PER, 4>(
            kWaves, lane, [&](int p) { return sm.lse[p][col]; },
            [&](int p, float (&v)[PER]) {
#pragma unroll
              for (int j = 0; j < PER; ++j) v[j] = sm.o[p][col][PER * lane + j];
            },
            acc);
#pragma unroll
        for (int j = 0; j < PER; ++j) sm.keep_o[col][PER * lane + j] = acc[j];
        if (lane == 0) sm.keep_lse[col] = l2;
      }
    }
    return;
  }
  if (suffix_publish<T, D, P>(a, sm, part, b, single, gk, wave, lane)) return;

  // this part's partial is written: count it for the request's join
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0) arrive(a, b, gk);
}

// Suffix block i: part q = i / n_kv for KV head i % n_kv, or, folded, part
// n_parts-1-q (the shorter) and then part q; the barrier between the two
// frees the LDS.  Folded, blocks q >= ceil(n_parts / 2) are grid padding.
//
// Suffix joins (every request's slot table is one part): the workgroup
// joins its parts' requests itself, for its KV head, once the requests'
// prefix splits have arrived (a request without a HOT prefix is finished by
// its part): the first part's merged result waits in LDS, the last part's
// four wave results are joined directly, and no part partial or join
// workgroup is needed.  The prefix splits never wait and precede every
// suffix block in each XCD's in-order dispatch, so the wait ends.
template <typename T, int D, typename P, class A>
__device__ __forceinline__ void suffix_block(const A& a, int blk, uint8_t* smem_raw) {
  const int q = blk / a.n_kv;
  const int gk = blk - q * a.n_kv;
  if (q >= (a.fold ? (a.n_parts + 1) / 2 : a.n_parts)) return;   // grid padding
  const int first = a.fold ? a.n_parts - 1 - q : q;
  const bool joins = a.suffix_joins != 0;
  if (first > q) {
    suffix_part<T, D, P>(a, first, gk, smem_raw, joins ? PartEnd::kKeep : PartEnd::kPublish);
    __syncthreads();
    trace_mark(a, a.prefix_blocks + blk);
  }
  suffix_part<T, D, P>(a, q, gk, smem_raw, joins ? PartEnd::kLeave : PartEnd::kPublish);
  if (!joins) return;
  trace_mark(a, a.prefix_blocks + blk, kTraceMark2);

  // the parts' requests and their prefix splits (-1: no HOT prefix, done)
  auto req_of = [&](int part) {
    const int b = a.ranks[part].req;   // one part per request: part = rank
    return table_at(a.req_class, b) >= 0 ? b : -1;
  };
  const int b_last = req_of(q), b_first = first > q ? req_of(first) : -1;
  if (b_last < 0 && b_first < 0) return;
  auto splits_of = [&](int b) { return a.classes[table_at(a.req_class, b)].n_splits; };
  if (threadIdx.x == 0) {
    if (b_last >= 0)
      wait_arrivals2(a, b_last, splits_of(b_last), b_first, b_first >= 0 ? splits_of(b_first) : 0, gk);
    else
      wait_arrivals(a, b_first, gk, splits_of(b_first));
  }
  __syncthreads();
  trace_mark(a, a.prefix_blocks + blk, kTraceMark3);
  SuffixSmem<T, D>& sm = *reinterpret_cast<SuffixSmem<T, D>*>(smem_raw);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = a.group;
  const int ns_last = b_last >= 0 ? splits_of(b_last) : 0, ns_first = b_first >= 0 ? splits_of(b_first) : 0;
  if (sizeof(P) == 2 && ns_last <= 32 && ns_first <= 32) {
    // The G (query head, request) joins of each request are dealt to the
    // waves in turn; with two requests the even waves take the last part's
    // and the odd waves the first part's, so a wave's joins are of one kind.
    // A wave keeps up to three joins' loads in flight (one round trip for
    // G <= 6; bf16 partials only: fp32 rows would not fit the registers).
    const bool two = b_last >= 0 && b_first >= 0;
    const bool of_first = two ? (wave & 1) != 0 : b_last < 0;
    const int cstep = two ? kWaves / 2 : kWaves;
    const int c0 = two ? wave >> 1 : wave;
    if (of_first)
      local_joins<T, D, P, 1>(a, ns_first, b_first, gk * G, c0, cstep, G, &sm.keep_o[0][0], D, &sm.keep_lse[0], 1,
                              lane);
    else
      local_joins<T, D, P, kWaves>(a, ns_last, b_last, gk * G, c0, cstep, G, &sm.o[0][0][0], 16 * D, &sm.lse[0][0],
                                   16, lane);
    return;
  }
  for (int col = wave; col < G; col += kWaves) {
    const int h = gk * G + col;
    if (b_last >= 0)
      join_local<T, D, P, kWaves>(a, ns_last, b_last, h, &sm.o[0][col][0], 16 * D, &sm.lse[0][col], 16, lane);
    if (b_first >= 0)
      join_local<T, D, P, 1>(a, ns_first, b_first, h, &sm.keep_o[col][0], D, &sm.keep_lse[col], 1, lane);
  }
}

// ------------------------------------------------------------ prefix kernel
// HOT block images.  A HOT pool stores, per KV head, blocks of kHotBlock = 32
// tokens; each block is kept as the exact register image of the MFMA
// operands the attention tile needs, in the order the lanes load them, so a
// wave fetches every operand with one contiguous 1 KB access:
//   K image: for half h (tokens 16h..16h+15), k-group s, lane l = n + 16g,
//            16 bytes = K[16h + n][d of k-group s, lane group g]
//            (bf16: d = 8g + 32s .. +8; fp32: d = (D/4)g + 4s .. +4);
//   V image: bf16: for block j < D/16, lane l, the 8 values
//            V[tau(g, e)][(D/16) n + j], e = 0..7 (V transposed per lane);
//            fp32: for e < 8, lane l, the D/16 values V[tau(g, e)][(D/16) n ..].
// gkv_hot_write scatters token rows into this layout.
template <typename T, int D>
__device__ __forceinline__ void hot_offsets(int tt, int d, int& ko, int& vo) {
  constexpr int EPB = D / 16;
  const int h = tt >> 4, nk = tt & 15;
  const int gl = tt < 16 ? tt >> 2 : (tt - 16) >> 2;     // inverse of tau
  const int e = tt < 16 ? tt & 3 : 4 + ((tt - 16) & 3);
  const int nv = d / EPB, j = d % EPB;
  if constexpr (sizeof(T) == 2) {
    const int s = d >> 5, dd = d & 31;
    ko = ((h * (D / 32) + s) * 64 + nk + 16 * (dd >> 3)) * 8 + (dd & 7);
    vo = (j * 64 + nv + 16 * gl) * 8 + e;
  } else {
    const int gk = d / (D / 4), w = d % (D / 4);
    ko = ((h * (D / 16) + (w >> 2)) * 64 + nk + 16 * gk) * 4 + (w & 3);
    vo = (e * 64 + nv + 16 * gl) * EPB + j;
  }
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void hot_write_kernel(const T* k_rows, const T* v_rows, int32_t n,
                                                             int64_t tok0, int32_t n_kv, int64_t hot_blocks,
                                                             T* k_hot, T* v_hot) {
  const int64_t total = static_cast<int64_t>(n) * n_kv * D;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t t = i / (static_cast<int64_t>(n_kv) * D);
    const int rem = static_cast<int>(i - t * n_kv * D);
    const int g = rem / D, d = rem % D;
    const int64_t tok = tok0 + t;
    const int64_t img = (static_cast<int64_t>(g) * hot_blocks + tok / kHotBlock) * (kHotBlock * D);
    int ko, vo;
    hot_offsets<T, D>(static_cast<int>(tok % kHotBlock), d, ko, vo);
    k_hot[img + ko] = k_rows[i];
    v_hot[img + vo] = v_rows[i];
  }
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Waits until at most n blocks of C direct-to-LDS loads each (issued after
// the block waited for) are still in flight, 0 <= n <= NMAX; loads retire in
// issue order, so older blocks have then landed.
template <int C, int NMAX>
__device__ __forceinline__ void wait_blocks_after(int n) {
  if constexpr (NMAX > 0) {
    if (n >= NMAX) {
      wait_vmcnt<NMAX * C>();
      return;
    }
    wait_blocks_after<C, NMAX - 1>(n);
  } else {
    wait_vmcnt<0>();
  }
}

// Direct global->LDS copy of 1 KB per wave: lane l moves the 16 bytes at
// base + voff (voff = 16 l + a per-wave constant) to LDS address lds + 16 l
// (base and lds wave-uniform).  Counted by vmcnt like any vector load.
// Issued as inline assembly so that the compiler's own wait-count
// bookkeeping does not see these transfers: the kernel orders them with
// explicit vmcnt waits, and the compiler's conservative view of them would
// otherwise drain the whole ring at some loop barriers.  The compiler's
// waits for other loads stay correct, only more conservative: vector loads
// retire in issue order.  The copy takes its LDS address from M0, a
// register the compiler may hold a value in (it cannot be declared
// clobbered): the asm saves M0 in a scratch SGPR and restores it, and the
// trailing s_nop covers the wait state an M0 write needs before an
// instruction that reads it.
__device__ __forceinline__ void load_lds_1k(uint32_t voff, const uint8_t* base, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0"
      : "=&s"(saved)
      : "v"(voff), "s"(base), "s"(lds)
      : "memory");
}

// LDS byte address of a pointer into __shared__ memory
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const uint8_t*)(p)));
}

// One prefix workgroup per (class, KV head, M-tile, L split).  The workgroup
// streams the split's HOT blocks into an LDS ring with direct global->LDS
// loads (16 bytes per lane, each block image copied as is), several blocks
// ahead; every wave reads its MFMA operands from the ring with contiguous
// 16-byte LDS reads and runs the attention tile for its RB blocks of 16 query
// rows.  One tile spans 64*RB rows, so a class of up to that many rows per
// KV head reads each slab byte from HBM exactly once per step.  RB = 1 with
// many L splits is the cascade backend; RB = 2 is the dense backend
// (HydraGen-style batched GEMM over M_eff rows with 128-row tiles, tiles of
// one split sharing it through their XCD's L2).
template <typename T, int D>
struct PrefixSmem {
  static constexpr int kImg = kHotBlock * D * static_cast<int>(sizeof(T));   // bytes of one K or V image
  // ring depth: what kRingBytes holds, at least 3 (fp32 rows of 128 take
  // more LDS) and at most 8
  static constexpr int kFit = kRingBytes / (2 * kImg);
  static constexpr int kStages = kFit > 8 ? 8 : (kFit < 3 ? 3 : kFit);
  // a block's K and V images are 2*kImg bytes, copied in 1 KB pieces spread
  // evenly over the waves
  static constexpr int kCopies = 2 * kImg / 1024 / kWaves;
  static_assert(kStages >= 3, "LDS ring too shallow");
  static_assert(kCopies >= 1 && kCopies * kWaves * 1024 == 2 * kImg, "block images must split evenly over waves");
  uint8_t ring[kStages][2 * kImg];
};

template <typename T, int D, int RB, typename P, class A>
__device__ __forceinline__ void prefix_block(const A& a, int blk, uint8_t* smem_raw) {
  using TR = Traits<T, D>;
  using KOp = typename TR::KOp;
  using SM = PrefixSmem<T, D>;
  constexpr int kImg = SM::kImg, kStages = SM::kStages, kCopies = SM::kCopies;
  auto& ring = reinterpret_cast<SM*>(smem_raw)->ring;

  // block -> class, KV head, split, M-tile (see ClassDesc)
  // the last class whose first block is <= blk (block_base increases)
  int ci = 0;
  for (int hi = a.n_classes - 1; ci < hi;) {
    const int mid = (ci + hi + 1) >> 1;
    if (a.classes[mid].block_base <= blk) ci = mid; else hi = mid - 1;
  }
  const ClassDesc& cl = a.classes[ci];
  const int local = blk - cl.block_base;
  const int xcds = a.xcds;
  const int r8 = local / xcds;
  const int m_tile = r8 % cl.m_tiles;
  const int grp = (r8 / cl.m_tiles) * xcds + local % xcds;
  if (grp >= cl.n_groups) return;   // XCD padding: whole workgroup leaves before any barrier
  const int kv_head = grp / cl.n_splits, split = grp % cl.n_splits;
  const int t0 = split * cl.chunk;
  const int t1 = min(cl.len, t0 + cl.chunk);
  const int nb = (t1 - t0 + kHotBlock - 1) / kHotBlock;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int n = lane & 15, g = lane >> 4;
  const int G = a.group;
  // the tile's requests: members [mem0, mem0 + n_mem) of the class, rows
  // r = i * G + j (member mem0 + i, query head kv_head * G + j)
  const int tm = tile_members(G, RB);
  const int mem0 = m_tile * tm;
  const int n_mem = min(tm, cl.n_members - mem0);
  const int rows = n_mem * G;
  const float c = a.scale_log2;
  const int wrow0 = wave * 16 * RB;
  const bool wave_active = wrow0 < rows;

  // K image at ring[slot][0, kImg), V image at ring[slot][kImg, 2 kImg).  A
  // block's images are kImg bytes each in the separate K and V pools; copy
  // cp of a wave moves the 1 KB piece at offset (cp * kWaves + wave) KB of
  // the pair.  Sources and LDS targets are wave-uniform (scalar) addresses;
  // the per-lane 16-byte offset is the same for every copy.
  const size_t img0 = (static_cast<size_t>(kv_head) * a.hot_blocks + (cl.slab_off + t0) / kHotBlock) * kImg;
  const uint8_t* src0[kCopies];
  uint32_t dst0[kCopies];
  const uint32_t ring_lds = lds_addr(&ring[0][0]);
#pragma unroll
  for (int cp = 0; cp < kCopies; ++cp) {
    const int off = (cp * kWaves + wave) * 1024;
    src0[cp] = off < kImg ? static_cast<const uint8_t*>(a.k_hot) + img0 + off
                          : static_cast<const uint8_t*>(a.v_hot) + img0 + (off - kImg);
    dst0[cp] = ring_lds + off;
  }
  const uint32_t voff = static_cast<uint32_t>(lane) * 16;
  // copies block i into ring slot `slot`
  auto copy = [&](int i, int slot) {
#pragma unroll
    for (int cp = 0; cp < kCopies; ++cp)
      load_lds_1k(voff, src0[cp] + static_cast<size_t>(i) * kImg, dst0[cp] + slot * (2 * kImg));
  };
  // the tile's request ids, one per lane (tile_members <= 128), loaded once
  // without a branch: query rows and partial rows find theirs by lane reads
  static_assert(kWaves * 16 * 2 <= 128, "tile members exceed two lanes' worth");
  const int mb0 = a.members[cl.member_off + mem0 + min(lane, n_mem - 1)];
  const int mb1 = a.members[cl.member_off + mem0 + min(lane + 64, n_mem - 1)];
  ColState<T, D> st[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    st[rb].init();
    const int r = wrow0 + 16 * rb + n;
    const int k = r / G;
    const int b0 = __shfl(mb0, k & 63), b1 = __shfl(mb1, k & 63);
    if (r < rows) {
      const int b = k < 64 ? b0 : b1;
      const int h = kv_head * G + r % G;
      TR::load_row(st[rb].q, static_cast<const T*>(a.q) + (static_cast<size_t>(b) * a.n_q + h) * D, g);
    } else {
      TR::zero_row(st[rb].q);
    }
  }
  // The first kStages - 1 copies fly while the query rows land.  Their
  // number is fixed (slots past the last block get a spare copy of it, never
  // read), and the query registers are claimed right after them: the
  // compiler's wait for the query loads is then placed here with an exact
  // count and none remains inside the loop, where it would drain the ring.
#pragma unroll
  for (int i = 0; i < kStages - 1; ++i) copy(min(i, nb - 1), i);
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int s2 = 0; s2 < TR::KS; ++s2) asm volatile("" : "+v"(st[rb].q[s2]));

  // Where registers allow (kPipeK: K operands, the block's score tiles for
  // two blocks and the V operands beside the state), the block loop is
  // software-pipelined (below); fp32 rows of 128 read and compute each
  // block in place.
  constexpr int kKRegs = 2 * TR::KS * static_cast<int>(sizeof(KOp)) / 4;
  constexpr int kVRegs = static_cast<int>(sizeof(typename TR::VOp)) / 4;
  constexpr int kStateRegs = RB * static_cast<int>(sizeof(ColState<T, D>)) / 4;
  constexpr bool kPipeK = kStateRegs + kKRegs + kVRegs + 8 * RB <= 200;
  struct KOps { KOp k0[TR::KS], k1[TR::KS]; };
  struct Ops {
    KOps k;
    typename TR::VOp vo;
  };
  auto read_k = [&](KOps& o, int i) {
    const uint8_t* ki = ring[i % kStages];
    TR::load_k_img(o.k0, ki, 0, lane);
    TR::load_k_img(o.k1, ki, 1, lane);
  };
  auto read_v = [&](typename TR::VOp& vo, int i) { TR::load_v_img(vo, ring[i % kStages] + kImg, lane); };
  // wait until block j's copies have landed in every wave; `issued` is the
  // last block whose copies this wave has issued
  auto wait_block = [&](int j, int issued) {
    wait_blocks_after<kCopies, kStages - 2>(issued - j);
    __syncthreads();
  };
  // Only the last block of a split can be partial: its V operands past the
  // slab end are zeroed (pool memory there is arbitrary) and its scores
  // masked (inside the tile).
  auto compute = [&](const KOps& k, typename TR::VOp& vo, int i) {
    const int valid = min(kHotBlock, t1 - t0 - kHotBlock * i);
    if (valid < kHotBlock) {
      int v = __builtin_amdgcn_readfirstlane(valid);
      asm volatile("" : "+s"(v));
      TR::mask_v(vo, v, g);
    }
    tile_rows<T, D, RB>(st, k.k0, k.k1, vo, valid, g, c);
  };

  if constexpr (kPipeK) {
    // Software pipeline over blocks.  S(i) = QK^T of block i is computed in
    // iteration i - 1, then shifted to y = s*c - m with its reference points
    // moved (rare branch).  Iteration i waits for block i + 1 and passes the
    // barrier (block i - 1's slot is then free: its K was read in iteration
    // i - 2, its V in i - 1), issues the copy of block i + kStages - 1, reads
    // K(i+1) and V(i), then runs one branch-free region: the QK^T of block
    // i + 1 on the matrix cores interleaved with the weights exp2(y(i)) on
    // the VALU, then PV(i) beside the row sums; last, the shift of S(i + 1)
    // (the scale and subtract out of the exp2 region: 1-2% on dense steps).
    // Only the last block can be partial; it is masked when its scores are
    // formed and done after the loop.  The loop is unrolled by two so that
    // the score tiles of consecutive blocks alternate between two register
    // sets (no copies).
    auto valid_of = [&](int j) { return min(kHotBlock, t1 - t0 - kHotBlock * j); };
    f32x4 s0[RB], s1[RB], n0[RB], n1[RB];
    wait_block(0, min(nb - 1, kStages - 2));
    if (wave_active) {
      KOps k;
      read_k(k, 0);
      qk_rows<T, D, RB>(st, k.k0, k.k1, s0, s1);
      softmax_ref<T, D, RB>(st, s0, s1, valid_of(0), g, c);
      float m[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) m[rb] = st[rb].m;
      shift_scores<RB>(s0, s1, m, c);
    }
    // iteration i: S(i) in (c0, c1), S(i + 1) into (x0, x1)
    auto iteration = [&](int i, f32x4 (&c0)[RB], f32x4 (&c1)[RB], f32x4 (&x0)[RB], f32x4 (&x1)[RB]) {
      wait_block(i + 1, min(nb - 1, i + kStages - 2));
      if (i + kStages - 1 < nb) copy(i + kStages - 1, (i + kStages - 1) % kStages);
      if (wave_active) {
        typename TR::VOp vo;
        KOps k;
        read_k(k, i + 1);
        read_v(vo, i);
        f32x4 p0[RB], p1[RB];
        qk_rows<T, D, RB>(st, k.k0, k.k1, x0, x1);
        softmax_py<RB>(c0, c1, p0, p1);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) TR::pv(st[rb].acc, vo, p0[rb], p1[rb]);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) st[rb].add_sum(p0[rb], p1[rb]);
        // kLead VALU instructions of the weights first (the first QK^T(i + 1)
        // product waits for K(i + 1) from LDS, and issue is in order: work
        // placed behind it would wait too), then one MFMA of QK^T(i + 1) and
        // one VALU instruction (the exp2 are quarter rate), repeated; the PV
        // products follow, beside the row sums and the shift of S(i + 1)
        constexpr int kLead = 8;
        __builtin_amdgcn_sched_group_barrier(0x002, kLead, 0);
#pragma unroll
        for (int x = 0; x < 2 * RB * TR::KS; ++x) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);
        }
        softmax_ref_y<T, D, RB>(st, x0, x1, valid_of(i + 1), g, c);
      }
    };
    int i = 0;
    for (; i + 2 < nb; i += 2) {
      iteration(i, s0, s1, n0, n1);
      iteration(i + 1, n0, n1, s0, s1);
    }
    if (i + 1 < nb) {
      iteration(i, s0, s1, n0, n1);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {   // once per split: the last block's scores to (s0, s1)
        s0[rb] = n0[rb];
        s1[rb] = n1[rb];
      }
    }
    if (wave_active) {
      const int i = nb - 1;
      typename TR::VOp vo;
      read_v(vo, i);
      const int valid = valid_of(i);
      if (valid < kHotBlock) {
        int v = __builtin_amdgcn_readfirstlane(valid);
        asm volatile("" : "+s"(v));
        TR::mask_v(vo, v, g);
      }
      f32x4 p0[RB], p1[RB];
      softmax_py<RB>(s0, s1, p0, p1);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        st[rb].add_sum(p0[rb], p1[rb]);
        TR::pv(st[rb].acc, vo, p0[rb], p1[rb]);
      }
    }
  } else {
    for (int i = 0; i < nb; ++i) {
      wait_block(i, min(nb - 1, i + kStages - 2));
      if (i + kStages - 1 < nb) copy(i + kStages - 1, (i + kStages - 1) % kStages);
      if (wave_active) {
        Ops o;
        read_k(o.k, i);
        read_v(o.vo, i);
        compute(o.k, o.vo, i);
      }
    }
  }

  // Partial rows go out whole: each wave stages its 16 x D tile in its own
  // part of the (now idle) ring, then writes every row as one contiguous
  // run across the lanes (the partial stores write through the caches, so
  // scattered pieces would cost partial-line writes).
  __syncthreads();   // every wave is done reading the ring
  trace_mark(a, blk);
  constexpr int kStride = D + 4;   // padded row stride of the staging tile (floats)
  static_assert(kWaves * 16 * kStride * 4 <= kStages * 2 * kImg, "staging tile exceeds the ring");
  float* stage = reinterpret_cast<float*>(&ring[0][0]) + wave * 16 * kStride;
  if (wave_active) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float o[D / 4];
      const float lse2 = st[rb].finish(o);
#pragma unroll
      for (int k = 0; k < D / 16; ++k)
        *reinterpret_cast<f32x4*>(stage + n * kStride + (D / 4) * g + 4 * k) =
            f32x4{o[4 * k], o[4 * k + 1], o[4 * k + 2], o[4 * k + 3]};
      // partial row index of tile row wrow0 + 16 rb + l, computed once by
      // lane l (< 16, one division by G for all rows); the lse of row n
      // moves to lane n and lanes < 16 store it
      const float lse_n = __shfl(lse2, n);
      const int r = wrow0 + 16 * rb + n;
      const int kr = r / G;
      const int bl0 = __shfl(mb0, kr & 63), bl1 = __shfl(mb1, kr & 63);
      const int bl = kr < 64 ? bl0 : bl1;
      const int prow = (bl * a.max_splits + split) * a.n_q + kv_head * G + (r - kr * G);
      if (lane < 16 && r < rows) store_partial(a.p_lse + prow, lse_n);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // 16-byte stores: lane l writes chunk l % CH of row l / CH of each
      // group of RPI rows, so one instruction covers RPI whole rows.  All
      // chunks leave LDS before the first store (one LDS wait).
      constexpr int CH = D * static_cast<int>(sizeof(P)) / 16;
      constexpr int RPI = 64 / CH;
      static_assert(CH <= 64 && 64 % CH == 0, "row chunks must tile the wave");
      const int ch = lane % CH, rsub = lane / CH;
      u32x4 pk[16 / RPI];
      int prow_of[16 / RPI];
#pragma unroll
      for (int s = 0; s < 16 / RPI; ++s) {
        const int rr = s * RPI + rsub;
        pk[s] = pack_chunk<P>(stage + rr * kStride + (16 / sizeof(P)) * ch);
        prow_of[s] = __shfl(prow, rr);
      }
#pragma unroll
      for (int s = 0; s < 16 / RPI; ++s)
        if (wrow0 + 16 * rb + s * RPI + rsub < rows)
          store_chunk(static_cast<P*>(a.p_o) + static_cast<size_t>(prow_of[s]) * D + (16 / sizeof(P)) * ch, pk[s],
                      a.narrow_ws != 0);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }

  // this split's partials are written: count one arrival per request of the
  // tile (its G rows for this KV head) for the requests' joins
  wait_stores();
  __syncthreads();
  trace_mark(a, blk, kTraceMark2);
  if (wave == 0) {
    if (lane < n_mem) arrive(a, mb0, kv_head);
    if (lane + 64 < n_mem) arrive(a, mb1, kv_head);
  }
}

// -------------------------------------------------------------- step kernel
// Prefix and suffix workgroups of one decode step in one launch: blocks
// [0, prefix_blocks) are prefix work (longest-running first), the rest
// suffix work, longest slot tables first.  Workgroups are handed to the 8
// XCDs round-robin by index and, within an XCD, to its shader engines in
// turn, so any periodic interleave of the two kinds can pin one kind to a
// subset of the engines; keeping each kind contiguous spreads both over all
// CUs.  A prefix block keeps blockIdx % 8 = its index % 8, i.e. its XCD.
template <typename T, int D>
constexpr size_t step_smem_bytes() {
  return sizeof(PrefixSmem<T, D>) > sizeof(SuffixSmem<T, D>) ? sizeof(PrefixSmem<T, D>) : sizeof(SuffixSmem<T, D>);
}

// Join of short requests (ranks r0 .. r0 + nr - 1 >= inline_rank0: each a
// HOT prefix and at most kInlineTokens slot-table tokens, no suffix part),
// in three phases.  Tiles: for each request, wave w takes KV heads w, w + 4,
// ... and attends the request's slot-table tile for each (one 32-token tile
// through the slot ids; in a fused step the last entry is the new token,
// read from its input row and copied into its slot, as a suffix part does),
// writing the normalised rows and lse to the request's own partial rows
// (part0).  Wait: once these stores are complete, one thread per (request,
// KV head) waits for the head's prefix splits.  Join: for each request, wave
// w joins KV heads w, w + 4, ...  The tiles need no prefix result, so with
// free slots they run beside it.
template <typename T, int D, typename P, class A>
__device__ __forceinline__ void short_join(const A& a, int r0, int nr, int blk) {
  using TR = Traits<T, D>;
  using KOp = typename TR::KOp;
  using VVec = typename TR::VVec;
  constexpr int EPC = 16 / static_cast<int>(sizeof(P));   // values per 16-byte chunk of a partial row
  constexpr int HP = 64 / (D * static_cast<int>(sizeof(P)) / 16);   // query heads per join pass
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int G = a.group;
  const bool col_ok = n < G;
  const float c = a.scale_log2;
  const size_t stride = static_cast<size_t>(a.n_kv) * D;

  // Tiles, per (request, KV head) unit of this wave.  The slot ids of up to
  // kIdRegs requests are loaded once, up front.  (Issuing two units' operand
  // loads before computing either measured no better: dense prefix-only
  // steps 1% faster, cascade ones 1.5% slower, 12 more registers.)
  constexpr int kIdRegs = 4;
  auto load_id = [&](int ri) {
    const RankDesc rd = a.ranks[r0 + ri];
    const int len = rd.tok1 - rd.tok0;
    int id = 0;
    if (lane < len) id = min(max(a.cold_indices[rd.tok0 + lane], 0), a.cold_cap - 1);
    // the new token of a fused step: -1
    if (a.k_new != nullptr && len > 0 && lane == len - 1) id = -1;
    return id;
  };
  int idv[kIdRegs];
#pragma unroll
  for (int ri = 0; ri < kIdRegs; ++ri) idv[ri] = ri < nr ? load_id(ri) : 0;
  struct Ops {
    KOp q[TR::KS], k0[TR::KS], k1[TR::KS];
    VVec v[8];
  };
  const int heads = (a.n_kv - wave + kWaves - 1) / kWaves;   // KV heads of this wave
  const int units = nr * heads;
  auto unit_of = [&](int u, int& ri, int& gk) {
    ri = u / max(heads, 1);
    gk = wave + (u - ri * heads) * kWaves;
  };
  auto load_unit = [&](int u, Ops& op) {
    int ri, gk;
    unit_of(u, ri, gk);
    const RankDesc rd = a.ranks[r0 + ri];
    const int b = rd.req, len = rd.tok1 - rd.tok0;
    if (a.k_new != nullptr && len > 0) suffix_copy_new<T, D>(a, b, gk, lane);
    if (len == 0) return;
    int id = ri < kIdRegs ? idv[0] : load_id(ri);
#pragma unroll
    for (int j = 1; j < kIdRegs; ++j)
      if (ri == j) id = idv[j];
    const int h = gk * G + (col_ok ? n : 0);
    if (col_ok) TR::load_row(op.q, static_cast<const T*>(a.q) + (static_cast<size_t>(b) * a.n_q + h) * D, g);
    else TR::zero_row(op.q);
    const T* kc = static_cast<const T*>(a.k_cold);
    const T* vc = static_cast<const T*>(a.v_cold) + TR::EPB * n;
    const size_t new_row = (static_cast<size_t>(b) * a.n_kv + gk) * D;
    const T* knew = static_cast<const T*>(a.k_new) + new_row;
    const T* vnew = static_cast<const T*>(a.v_new) + new_row + TR::EPB * n;
    // row of tile position i (positions past the table repeat its last
    // entry; the tile masks them)
    auto row = [&](const T* pool, const T* fresh_row, int i) {
      const int t = __shfl(id, min(i, len - 1));
      return t < 0 ? fresh_row : pool + static_cast<size_t>(t) * stride + cold_row_pos(gk, t, a.cold_mask) * D;
    };
    TR::load_row(op.k0, row(kc, knew, n), g);
    TR::load_row(op.k1, row(kc, knew, 16 + n), g);
#pragma unroll
    for (int e = 0; e < 8; ++e) op.v[e] = TR::load_v(row(vc, vnew, tau(g, e)));
  };
  auto run_unit = [&](int u, const Ops& op) {
    int ri, gk;
    unit_of(u, ri, gk);
    const RankDesc rd = a.ranks[r0 + ri];
    const int len = rd.tok1 - rd.tok0;
    float lse2 = kNegInf;
    float o[D / 4];
#pragma unroll
    for (int k = 0; k < D / 4; ++k) o[k] = 0.f;
    if (len > 0) {
      ColState<T, D> st;
      st.init();
#pragma unroll
      for (int s2 = 0; s2 < TR::KS; ++s2) st.q[s2] = op.q[s2];
      typename TR::VOp vo;
      TR::make_vop(vo, op.v);
      st.tile(op.k0, op.k1, vo, len, g, c);
      lse2 = st.finish(o);
    }
    // lane (n, g) holds d = (D/4) g .. of query head h: whole 16-byte chunks
    if (col_ok) {
      const size_t prow = static_cast<size_t>(rd.part0) * a.n_q + gk * G + n;
      P* dst = static_cast<P*>(a.s_o) + prow * D + (D / 4) * g;
#pragma unroll
      for (int k = 0; k < D / 4; k += EPC) {
        float x[EPC];
#pragma unroll
        for (int j = 0; j < EPC; ++j) x[j] = o[k + j];
        store_chunk(dst + k, pack_chunk<P>(x), false);
      }
      if (g == 0) store_partial(a.s_lse + prow, lse2);
    }
  };
  auto tiles = [&]() {
    for (int u = 0; u < units; ++u) {
      Ops op;
      load_unit(u, op);
      run_unit(u, op);
    }
  };
  // Join, per request: this wave's units (KV head, pass of HP query heads),
  // two at a time with their loads together when the partials (the class's
  // prefix splits and the request's tile) are few, else one KV head at a
  // time (join_group).
  auto join = [&](int ri) {
    const RankDesc rd = a.ranks[r0 + ri];
    const JoinSrc src = {a.classes[table_at(a.req_class, rd.req)].n_splits, rd.part0, 1};
    const int b = rd.req;
    if (src.ns + src.n_parts <= 8) {
      const int passes = (G + HP - 1) / HP;
      const int nu = heads * passes;
      for (int i = 0; i < nu; i += 2) {
        const JoinSrc srcs[2] = {src, src};
        const int bs[2] = {b, b};
        int gk[2], h0[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int u = min(i + j, nu - 1);
          gk[j] = wave + (u / passes) * kWaves;
          h0[j] = (u % passes) * HP;
        }
        join_units<T, D, P, 8, 2>(a, srcs, bs, gk, h0, min(2, nu - i), lane);
      }
    } else {
      for (int gk = wave; gk < a.n_kv; gk += kWaves) join_group<T, D, P>(a, src, b, gk, lane);
    }
  };

  tiles();
  wait_stores();
  __syncthreads();
  for (int t = threadIdx.x; t < nr * a.n_kv; t += kThreads) {
    const int ri = t / a.n_kv;
    const int b = a.ranks[r0 + ri].req;
    wait_arrivals(a, b, t - ri * a.n_kv, a.classes[table_at(a.req_class, b)].n_splits);
  }
  __syncthreads();
  trace_mark(a, blk);
  for (int ri = 0; ri < nr; ++ri) join(ri);
}

// Join j: for j < inline_rank0 * n_kv, (ranked request, KV head g) with the
// ranks taken shortest slot table first (their partials arrive first): waits
// for the arrival of all partials, then wave w joins the request's query
// heads g*G + w, g*G + w + 4, ...  Where the partials lie is read before the
// wait, so after it only the partials themselves are loaded.  The rest:
// short_per_block consecutive short requests each (the last: what remains).
template <typename T, int D, typename P, class A>
__device__ __forceinline__ void join_block(const A& a, int j) {
  const int blk = a.prefix_blocks + a.suffix_blocks + j;
  const int nj = a.suffix_joins ? 0 : a.inline_rank0 * a.n_kv;
  if (j >= nj) {
    const int r0 = a.inline_rank0 + (j - nj) * a.short_per_block;
    short_join<T, D, P>(a, r0, min(a.short_per_block, a.batch - r0), blk);
    return;
  }
  const int q = j / a.n_kv, g = j - q * a.n_kv;
  const int b = a.ranks[a.inline_rank0 - 1 - q].req;
  const JoinSrc src = join_src(a, b);
  const int n = src.ns + src.n_parts;
  if (n == 1) return;   // finished by its only suffix part
  if (threadIdx.x == 0) wait_arrivals(a, b, g, n);
  __syncthreads();
  trace_mark(a, blk);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int col = wave; col < a.group; col += kWaves) join_row<T, D, P>(a, src, b, g * a.group + col, lane);
}

// Two workgroups per CU; fp32 rows of 128 take 96 KB of LDS per prefix
// workgroup, so one.
template <typename T, int D, int RB, typename P, class A>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(sizeof(T) == 4 && D == 128 ? 1 : 2))) void step_kernel(A a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[step_smem_bytes<T, D>()];
  if (a.tail != kArgsTail) return;   // the work description did not arrive whole
  const int blk = blockIdx.x;
  const int work = a.prefix_blocks + a.suffix_blocks;
  const uint32_t kind = blk >= work ? kTraceJoin : blk < a.prefix_blocks ? kTracePrefix : kTraceSuffix;
  if (a.trace && threadIdx.x == 0) trace_start(a, blk, kind);
  if (blk >= work) join_block<T, D, P>(a, blk - work);
  else if (blk < a.prefix_blocks) prefix_block<T, D, RB, P>(a, blk, smem);
  else suffix_block<T, D, P>(a, blk - a.prefix_blocks, smem);
  if (a.trace) {
    __syncthreads();
    if (threadIdx.x == 0) a.trace[static_cast<size_t>(blk) * kTraceWords + kTraceEnd] = __builtin_amdgcn_s_memrealtime();
  }
}

// Chunk ch of input row tok (head ch / head_chunks) goes to the same chunk
// of that head's position in slot slots[tok].
__global__ __launch_bounds__(kThreads) void append_kernel(const u32x4* k_new, const u32x4* v_new,
                                                          const int32_t* slots, int32_t n,
                                                          u32x4* k_cold, u32x4* v_cold,
                                                          int32_t head_chunks, int32_t n_kv,
                                                          int32_t cold_cap) {
  const int64_t row_chunks = static_cast<int64_t>(head_chunks) * n_kv;
  const int32_t mask = cold_mask_for(n_kv);
  const int64_t total = static_cast<int64_t>(n) * row_chunks;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t tok = i / row_chunks;
    const int32_t ch = static_cast<int32_t>(i - tok * row_chunks);
    const int32_t s = slots[tok];
    if (s < 0 || s >= cold_cap) continue;
    const int32_t g = ch / head_chunks;
    const int64_t dst = static_cast<int64_t>(s) * row_chunks +
                        static_cast<int64_t>(cold_row_pos(g, s, mask)) * head_chunks + (ch - g * head_chunks);
    k_cold[dst] = k_new[i];
    v_cold[dst] = v_new[i];
  }
}

template <typename T, int D, class A>
hipError_t launch_typed(const A& a, int32_t backend, hipStream_t stream, hipEvent_t* ev) {
  // With timing events, the kernel is launched through hipExtLaunchKernelGGL,
  // which stamps the events with the kernel's own start and end.
  hipEvent_t e0 = ev ? ev[0] : nullptr, e1 = ev ? ev[1] : nullptr;
  const int blocks = a.prefix_blocks + a.suffix_blocks + a.join_blocks;
  (void)backend;
  if constexpr (sizeof(T) == 2) {
    // bf16 inputs: partial rows in fp32 or in bf16, 64- or 128-row prefix tiles
    if (a.partial_f32) {
      if (a.rb == 2)
        hipExtLaunchKernelGGL(step_kernel<T, D, 2, float, A>, dim3(blocks), dim3(kThreads), 0, stream, e0, e1, 0, a);
      else
        hipExtLaunchKernelGGL(step_kernel<T, D, 1, float, A>, dim3(blocks), dim3(kThreads), 0, stream, e0, e1, 0, a);
    } else {
      if (a.rb == 2)
        hipExtLaunchKernelGGL(step_kernel<T, D, 2, T, A>, dim3(blocks), dim3(kThreads), 0, stream, e0, e1, 0, a);
      else
        hipExtLaunchKernelGGL(step_kernel<T, D, 1, T, A>, dim3(blocks), dim3(kThreads), 0, stream, e0, e1, 0, a);
    }
  } else {
    // fp32 inputs: fp32 partials, 64-row tiles
    if (a.rb != 1 || !a.partial_f32) return hipErrorInvalidValue;
    hipExtLaunchKernelGGL(step_kernel<T, D, 1, T, A>, dim3(blocks), dim3(kThreads), 0, stream, e0, e1, 0, a);
  }
  return hipGetLastError();
}

// Streaming read of n16 16-byte vectors (the measured read ceiling of the
// device).  Each wave reads 8 KB chunks (eight 1 KB loads, consecutive lanes
// on consecutive vectors, all in flight at once) with non-temporal loads,
// the waves striding over the chunks; the fastest plain read pattern found on
// gfx950 (grid-stride loads of single vectors reach about 12% less).  The
// data only feeds an xor whose (practically never taken) store to `sink`
// keeps the loads alive.
__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4* p, int64_t n16, uint32_t* sink) {
  constexpr int kChunk = 8 * 64;   // vectors per wave chunk
  uint32_t acc = 0;
  const int lane = threadIdx.x & 63;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  const int64_t waves = static_cast<int64_t>(gridDim.x) * kWaves;
  const int64_t full = n16 / kChunk;
  for (int64_t c = wave; c < full; c += waves) {
    const u32x4* q = p + c * kChunk + lane;
    u32x4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = __builtin_nontemporal_load(q + 64 * k);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
  }
  // the last partial chunk, one vector per lane of the grid
  for (int64_t i = full * kChunk + static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const u32x4 v = p[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x9e3779b9u) *sink = acc;
}

__global__ __launch_bounds__(kThreads) void zero_kernel(int32_t* p, size_t n) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = 0;
}

}  // namespace

hipError_t scratch_region(int device, uint8_t** ptr, bool* first_use) {
  static std::mutex mu;
  static uint8_t* addr[kMaxDevices] = {};
  static bool used[kMaxDevices] = {};
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[device]) {
    void* p = nullptr;
    // the caller made `device` current
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p || reinterpret_cast<uintptr_t>(p) % 256 != 0) return hipErrorInvalidSymbol;
    addr[device] = static_cast<uint8_t*>(p);
  }
  *ptr = addr[device];
  *first_use = !used[device];
  used[device] = true;
  return hipSuccess;
}

hipError_t launch_zero_i32(int32_t* p, size_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int grid = static_cast<int>(std::min<size_t>((n + kThreads - 1) / kThreads, 1024));
  zero_kernel<<<grid, kThreads, 0, stream>>>(p, n);
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* p, size_t bytes, int32_t workgroups, uint32_t* sink, hipStream_t stream) {
  const int64_t n16 = static_cast<int64_t>(bytes / 16);
  if (n16 == 0) return hipSuccess;
  read_kernel<<<workgroups, kThreads, 0, stream>>>(static_cast<const u32x4*>(p), n16, sink);
  return hipGetLastError();
}

hipError_t launch_cold_append(const void* k_new, const void* v_new, const int32_t* slots, int32_t n,
                              void* k_cold, void* v_cold, int32_t n_kv, int64_t head_bytes, int32_t cold_cap,
                              hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  if (n_kv <= 0 || head_bytes <= 0 || head_bytes % 16) return hipErrorInvalidValue;
  const int32_t head_chunks = static_cast<int32_t>(head_bytes / 16);
  const int64_t row_chunks = static_cast<int64_t>(head_chunks) * n_kv;
  const int64_t total = static_cast<int64_t>(n) * row_chunks;
  const int64_t blocks = (total + kThreads - 1) / kThreads;
  const int grid = static_cast<int>(blocks < 4096 ? blocks : 4096);
  append_kernel<<<grid, kThreads, 0, stream>>>(
      static_cast<const u32x4*>(k_new), static_cast<const u32x4*>(v_new), slots, n,
      static_cast<u32x4*>(k_cold), static_cast<u32x4*>(v_cold), head_chunks, n_kv, cold_cap);
  return hipGetLastError();
}

hipError_t launch_hot_write(const void* k_rows, const void* v_rows, int32_t n, int64_t tok0, int32_t n_kv,
                           int32_t head_dim, int32_t dtype, int64_t hot_blocks, void* k_hot, void* v_hot,
                           hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t total = static_cast<int64_t>(n) * n_kv * head_dim;
  const int grid = static_cast<int>(std::min<int64_t>((total + kThreads - 1) / kThreads, 8192));
#define GKV_HW(T, D)                                                                                     \
  hot_write_kernel<T, D><<<grid, kThreads, 0, stream>>>(static_cast<const T*>(k_rows),                  \
                                                        static_cast<const T*>(v_rows), n, tok0, n_kv,   \
                                                        hot_blocks, static_cast<T*>(k_hot), static_cast<T*>(v_hot))
  if (dtype == 1) {
    if (head_dim == 128) GKV_HW(__bf16, 128); else GKV_HW(__bf16, 64);
  } else {
    if (head_dim == 128) GKV_HW(float, 128); else GKV_HW(float, 64);
  }
#undef GKV_HW
  return hipGetLastError();
}

namespace {
template <class A>
hipError_t launch_sized(const A& a, int32_t dtype, int32_t backend, hipStream_t stream, hipEvent_t* ev) {
  if (dtype == 1) {
    return a.head_dim == 128 ? launch_typed<__bf16, 128>(a, backend, stream, ev)
                             : launch_typed<__bf16, 64>(a, backend, stream, ev);
  }
  return a.head_dim == 128 ? launch_typed<float, 128>(a, backend, stream, ev)
                           : launch_typed<float, 64>(a, backend, stream, ev);
}
}  // namespace

hipError_t launch_step(const StepArgs& a, int32_t dtype, int32_t backend, hipStream_t stream,
                       hipEvent_t* ev) {
  if (a.batch > kSmallBatch) return launch_sized(a, dtype, backend, stream, ev);
  // the small form: the head and the first kSmallBatch entries of each table
  StepArgsSmall s;
  static_cast<StepHead&>(s) = static_cast<const StepHead&>(a);
  std::memcpy(s.ranks, a.ranks, sizeof(s.ranks));
  std::memcpy(s.rank_of, a.rank_of, sizeof(s.rank_of));
  std::memcpy(s.members, a.members, sizeof(s.members));
  std::memcpy(s.req_class, a.req_class, sizeof(s.req_class));
  s.tail = a.tail;
  return launch_sized(s, dtype, backend, stream, ev);
}

}  // namespace gkv
