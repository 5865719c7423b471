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
//   suffix_kernel   one wave per (request, KV head, slot-table chunk): gathers
//                   K/V rows through the slot table (one 16-byte load per
//                   lane per token row piece, software-pipelined one tile
//                   ahead), writes a partial per query head.
//   prefix_kernel   one workgroup per (class, KV head, M-tile, L split):
//                   streams 64-token K/V tiles of the contiguous slab into
//                   LDS (double-buffered, 16-byte coalesced loads) and runs
//                   the MFMA tile for RB 16-row blocks per wave.  RB = 1 with
//                   many L splits is the cascade backend (each slab byte
//                   read once per step); RB = 2 with larger M tiles is the
//                   dense backend (HydraGen-style batched GEMM of M_eff rows).
//   merge_kernel    one wave per (request, query head): log-sum-exp merge of
//                   all prefix splits and suffix chunks, writes out and lse.
//   append_kernel   byte copy of new token rows into COLD slots.
//
// Partials keep lse in base 2 of the scaled scores (s * log2(e)/sqrt(d));
// the merge converts the final lse to natural log.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "kernels.h"

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

  // One 32-token tile: K operands of the two 16-token halves, V operands, the
  // number of valid tokens (tokens >= valid are masked) and the score scale.
  __device__ void tile(const typename TR::KOp (&k0)[TR::KS], const typename TR::KOp (&k1)[TR::KS],
                       const typename TR::VOp& vo, int valid, int g, float c) {
    f32x4 s0 = TR::qk(k0, q);
    f32x4 s1 = TR::qk(k1, q);
    if (valid < 32) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (4 * g + i >= valid) s0[i] = kNegInf;
        if (16 + 4 * g + i >= valid) s1[i] = kNegInf;
      }
    }
    float mx = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])),
                     fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
    mx = wave_max_groups(mx) * c;
    // Lazy rescaling: the reference point m only moves when a column's max
    // exceeds it by more than kLazy (log2 units), so p = 2^(s*c - m) stays
    // below 2^kLazy and the accumulators are rescaled rarely (the first tile
    // and genuine jumps), not on every new maximum.  The result is the same:
    // numerator and denominator share m.
    if (__any(mx > m + kLazy)) {
      const float m_new = fmaxf(m, mx);
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);
      l *= alpha;
#pragma unroll
      for (int j = 0; j < TR::EPB; ++j) acc[j] *= alpha;
      m = m_new;
    }
    f32x4 p0, p1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p0[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[i], c, -m));
      p1[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[i], c, -m));
    }
    l += (p0[0] + p0[1]) + (p0[2] + p0[3]) + (p1[0] + p1[1]) + (p1[2] + p1[3]);
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

__device__ __forceinline__ void store_row_slice(float* dst, const float* o, int n4) {
  for (int k = 0; k < n4; ++k)
    reinterpret_cast<f32x4*>(dst)[k] = f32x4{o[4 * k], o[4 * k + 1], o[4 * k + 2], o[4 * k + 3]};
}

// Joins the partial softmax results of one query head: np parts, part p has
// base-2 lse lse_of(p) and normalised output row o_of(p) (PER elements per
// lane at PER*lane).  All loads are issued before any is used.  Writes the
// joined row through put(acc_scaled) and returns the joined base-2 lse.
template <int PER, int MB, typename LseF, typename RowF>
__device__ __forceinline__ float join_parts(int np, int lane, LseF lse_of, RowF o_of, float (&acc)[PER]) {
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
      if (k < cnt) {
        const float* src = o_of(base + k);
#pragma unroll
        for (int j = 0; j < PER; ++j) v[k][j] = src[j];
      }
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
  const float inv = 1.f / wsum;
#pragma unroll
  for (int j = 0; j < PER; ++j) acc[j] *= inv;
  return mx + __log2f(wsum);
}

// ------------------------------------------------------------ suffix kernel
// One workgroup per (suffix part, KV head); see StepArgs.  Each wave runs
// the online softmax over its quarter of the part through the slot table,
// the four results meet in LDS, and the epilogue joins them (and, for a
// request with a single part, the request's prefix splits) into the output.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void suffix_kernel(StepArgs a) {
  using TR = Traits<T, D>;
  using KOp = typename TR::KOp;
  using VVec = typename TR::VVec;
  constexpr int PER = D / 64;
  __shared__ int32_t lds_ids[kWaves][kWaveTokens];
  __shared__ __attribute__((aligned(16))) float lds_o[kWaves][16][D];
  __shared__ float lds_lse[kWaves][16];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int part = blockIdx.x / a.n_kv;
  const int gk = blockIdx.x - part * a.n_kv;
  int lo = 0, hi = a.batch - 1;     // rank: last r with part_start[r] <= part
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.part_start[mid] <= part) lo = mid; else hi = mid - 1;
  }
  const int b = a.order[lo];
  const int j = part - a.part_start[lo];
  const bool single = a.part_start[lo + 1] - a.part_start[lo] == 1;
  const int tb0 = a.indptr[b], tb1 = a.indptr[b + 1];
  const int p0 = min(tb1, tb0 + j * kSuffixPart), p1 = min(tb1, p0 + kSuffixPart);
  const int quarter = (((p1 - p0 + kWaves - 1) / kWaves) + kSuffixTile - 1) / kSuffixTile * kSuffixTile;
  const int w0 = min(p1, p0 + wave * quarter), w1 = min(p1, w0 + quarter);
  const int len = w1 - w0;

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
    ColState<T, D> st;
    st.init();
    if (col_ok) TR::load_row(st.q, static_cast<const T*>(a.q) + (static_cast<size_t>(b) * a.n_q + h) * D, g);
    else TR::zero_row(st.q);

    const size_t stride = static_cast<size_t>(a.n_kv) * D;
    const T* kc = static_cast<const T*>(a.k_cold) + gk * D;
    const T* vc = static_cast<const T*>(a.v_cold) + gk * D + TR::EPB * n;
    const int n_tiles = (len + kSuffixTile - 1) / kSuffixTile;
    const int cap1 = a.cold_cap - 1;

    // the quarter's slot ids, clamped into the pool, staged in this wave's
    // LDS row once: no tile waits on a slot-id load
    int32_t* ids = lds_ids[wave];
    for (int k = lane; k < len; k += 64) ids[k] = min(max(a.cold_indices[w0 + k], 0), cap1);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    auto load_kv = [&](int i, KOp (&k0)[TR::KS], KOp (&k1)[TR::KS], VVec (&v)[8]) {
      const int base = kSuffixTile * i, last = len - 1;
      const int s0 = ids[min(base + n, last)], s1 = ids[min(base + 16 + n, last)];
      TR::load_row(k0, kc + static_cast<size_t>(s0) * stride, g);
      TR::load_row(k1, kc + static_cast<size_t>(s1) * stride, g);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int se = ids[min(base + tau(g, e), last)];
        v[e] = TR::load_v(vc + static_cast<size_t>(se) * stride);
      }
    };
    auto run_tile = [&](const KOp (&k0)[TR::KS], const KOp (&k1)[TR::KS], const VVec (&v)[8], int i) {
      typename TR::VOp vo;
      TR::make_vop(vo, v);
      st.tile(k0, k1, vo, min(kSuffixTile, len - kSuffixTile * i), g, c);
    };

    // two register sets, alternating: tile i+1 loads while tile i computes
    KOp ka0[TR::KS], ka1[TR::KS], kb0[TR::KS], kb1[TR::KS];
    VVec va[8], vb[8];
    load_kv(0, ka0, ka1, va);
    for (int i = 0; i < n_tiles; i += 2) {
      if (i + 1 < n_tiles) load_kv(i + 1, kb0, kb1, vb);
      run_tile(ka0, ka1, va, i);
      if (i + 1 >= n_tiles) break;
      if (i + 2 < n_tiles) load_kv(i + 2, ka0, ka1, va);
      run_tile(kb0, kb1, vb, i + 1);
    }
    lse2 = st.finish(o);
  }

  // the four quarters meet in LDS
  if (col_ok) {
#pragma unroll
    for (int k = 0; k < D / 16; ++k)
      *reinterpret_cast<f32x4*>(&lds_o[wave][n][(D / 4) * g + 4 * k]) =
          f32x4{o[4 * k], o[4 * k + 1], o[4 * k + 2], o[4 * k + 3]};
    if (g == 0) lds_lse[wave][n] = lse2;
  }
  __syncthreads();

  // epilogue: wave w joins columns w, w+4, ...
  const int cls = a.req_class[b];
  const int ns = single && cls >= 0 ? a.classes[cls].n_splits : 0;
  for (int col = wave; col < G; col += kWaves) {
    const int hc = gk * G + col;
    const size_t prow0 = static_cast<size_t>(b) * a.max_splits * a.n_q + hc;
    float acc[PER];
    const float l2 = join_parts<PER, 16>(
        kWaves + ns, lane,
        [&](int p) { return p < kWaves ? lds_lse[p][col] : a.p_lse[prow0 + static_cast<size_t>(p - kWaves) * a.n_q]; },
        [&](int p) -> const float* {
          return p < kWaves ? &lds_o[p][col][PER * lane]
                            : a.p_o + (prow0 + static_cast<size_t>(p - kWaves) * a.n_q) * D + PER * lane;
        },
        acc);
    if (single) {
      T* dst = static_cast<T*>(a.out) + (static_cast<size_t>(b) * a.n_q + hc) * D + PER * lane;
#pragma unroll
      for (int k = 0; k < PER; ++k) dst[k] = static_cast<T>(acc[k]);
      if (lane == 0) a.lse[static_cast<size_t>(b) * a.n_q + hc] = l2 * 0.69314718055994531f;
    } else {
      const size_t row = static_cast<size_t>(part) * a.n_q + hc;
      float* dst = a.s_o + row * D + PER * lane;
#pragma unroll
      for (int k = 0; k < PER; ++k) dst[k] = acc[k];
      if (lane == 0) a.s_lse[row] = l2;
    }
  }
}

// ------------------------------------------------------------ prefix kernel
// LDS staging of one 64-token K/V tile.  Threads 0..127 copy K rows as they
// are; threads 128..255 stage V.  For bf16, a V thread owns lane slot
// (n, g) of one 32-token half: it loads the 8 token rows tau(g, 0..7) at
// elements (D/16)*n .., transposes them in registers and writes the D/16
// A-operand vectors of that lane slot, so the computing waves read their PV
// operands with one 16-byte LDS read each and no further shuffling.
template <typename T, int D>
struct PrefixTileIO {
  using TR = Traits<T, D>;
  static constexpr int kKStride = D + 16 / static_cast<int>(sizeof(T));   // padded K row (elements)
  static constexpr int kChunksPerRow = D * static_cast<int>(sizeof(T)) / 16;
  static constexpr int kKChunks = kPrefixTile * kChunksPerRow / 128;      // per K thread
  static constexpr bool kVT = sizeof(T) == 2;                              // V pre-transposed
  static constexpr int kVBytes = kVT ? 2 * TR::EPB * 64 * 16 : kPrefixTile * kKStride * 4;
  static constexpr int kKBytes = kPrefixTile * kKStride * static_cast<int>(sizeof(T));
  static constexpr int kVRegs = kVT ? 8 : kKChunks;   // staged vectors per V thread

  using VStage = typename std::conditional<kVT, typename TR::VVec, u32x4>::type;
  u32x4 k[kKChunks];
  VStage v[kVRegs];

  // Thread's first K row and column chunk; its j-th chunk is row
  // krow + kRowStep * j of the same column (kRowStep = 128 / chunks per row).
  static constexpr int kRowStep = 128 / kChunksPerRow;
  static constexpr int kElemsPerChunk = 16 / static_cast<int>(sizeof(T));

  // Global -> registers for the tile starting at token tt.  Rows past t1
  // (only in the last tile) are clamped to t1 - 1: duplicates, masked later.
  __device__ void load(const T* kb, const T* vb, int tt, int t1) {
    const int tid = threadIdx.x;
    const bool full = tt + kPrefixTile <= t1;
    if (tid < 128) {
      const int krow = tid / kChunksPerRow, kcol = tid % kChunksPerRow;
      if (full) {
        const T* src = kb + static_cast<size_t>(tt + krow) * D + kcol * kElemsPerChunk;
#pragma unroll
        for (int j = 0; j < kKChunks; ++j) k[j] = *reinterpret_cast<const u32x4*>(src + j * kRowStep * D);
      } else {
#pragma unroll
        for (int j = 0; j < kKChunks; ++j)
          k[j] = *reinterpret_cast<const u32x4*>(
              kb + static_cast<size_t>(min(tt + krow + j * kRowStep, t1 - 1)) * D + kcol * kElemsPerChunk);
      }
    } else if constexpr (kVT) {
      const int vt = tid - 128, hh = vt >> 6, ls = vt & 63, n = ls & 15, g = ls >> 4;
      const int r0 = tt + 32 * hh + 4 * g;   // tau(g, e) = 4g + e, or 4g + 12 + e for e >= 4
      if (full) {
        const T* src = vb + static_cast<size_t>(r0) * D + TR::EPB * n;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = TR::load_v(src + (e < 4 ? e : 12 + e) * D);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          v[e] = TR::load_v(vb + static_cast<size_t>(min(r0 + (e < 4 ? e : 12 + e), t1 - 1)) * D + TR::EPB * n);
      }
    } else {
      const int krow = (tid - 128) / kChunksPerRow, kcol = (tid - 128) % kChunksPerRow;
#pragma unroll
      for (int j = 0; j < kKChunks; ++j)
        v[j] = *reinterpret_cast<const u32x4*>(
            vb + static_cast<size_t>(min(tt + krow + j * kRowStep, t1 - 1)) * D + kcol * kElemsPerChunk);
    }
  }

  __device__ void store(T* lk, uint8_t* lv) {
    const int tid = threadIdx.x;
    if (tid < 128) {
      const int krow = tid / kChunksPerRow, kcol = tid % kChunksPerRow;
#pragma unroll
      for (int j = 0; j < kKChunks; ++j)
        *reinterpret_cast<u32x4*>(lk + (krow + j * kRowStep) * kKStride + kcol * kElemsPerChunk) = k[j];
    } else if constexpr (kVT) {
      const int vt = tid - 128, hh = vt >> 6, ls = vt & 63;
      typename TR::VOp vo;
      TR::make_vop(vo, v);
#pragma unroll
      for (int j = 0; j < TR::EPB; ++j)
        reinterpret_cast<u32x4*>(lv)[(hh * TR::EPB + j) * 64 + ls] = vo.a[j];
    } else {
      const int krow = (tid - 128) / kChunksPerRow, kcol = (tid - 128) % kChunksPerRow;
#pragma unroll
      for (int j = 0; j < kKChunks; ++j)
        *reinterpret_cast<u32x4*>(reinterpret_cast<float*>(lv) + (krow + j * kRowStep) * kKStride + kcol * 4) = v[j];
    }
  }

  // PV operands of half hh for this lane
  __device__ static void read_vop(typename TR::VOp& vo, const uint8_t* lv, int hh, int lane, int n, int g) {
    if constexpr (kVT) {
#pragma unroll
      for (int j = 0; j < TR::EPB; ++j) vo.a[j] = reinterpret_cast<const u32x4*>(lv)[(hh * TR::EPB + j) * 64 + lane];
    } else {
      typename TR::VVec v[8];
      const float* base = reinterpret_cast<const float*>(lv) + (32 * hh) * kKStride;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = TR::load_v(reinterpret_cast<const T*>(base + tau(g, e) * kKStride + TR::EPB * n));
      TR::make_vop(vo, v);
    }
  }
};

template <typename T, int D, int RB>
__global__ __launch_bounds__(kThreads) void prefix_kernel(StepArgs a) {
  using TR = Traits<T, D>;
  using KOp = typename TR::KOp;
  using IO = PrefixTileIO<T, D>;
  __shared__ __attribute__((aligned(16))) T lds_k[2][IO::kKBytes / sizeof(T)];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v[2][IO::kVBytes];

  // block -> class, KV head, split, M-tile (see ClassDesc)
  const int blk = blockIdx.x;
  int ci = 0;
  while (ci + 1 < a.n_classes && blk >= a.classes[ci + 1].block_base) ++ci;
  const ClassDesc& cl = a.classes[ci];
  const int local = blk - cl.block_base;
  const int r8 = local / kXcds;
  const int m_tile = r8 % cl.m_tiles;
  const int grp = (r8 / cl.m_tiles) * kXcds + local % kXcds;
  if (grp >= cl.n_groups) return;   // XCD padding: whole workgroup leaves before any barrier
  const int kv_head = grp / cl.n_splits, split = grp % cl.n_splits;
  const int t0 = split * cl.chunk;
  const int t1 = min(cl.len, t0 + cl.chunk);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int G = a.group;
  const int rows = cl.n_members * G;
  const float c = a.scale_log2;
  const int wrow0 = m_tile * 64 * RB + wave * 16 * RB;
  const bool wave_active = wrow0 < rows;

  ColState<T, D> st[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    st[rb].init();
    const int r = wrow0 + 16 * rb + n;
    if (r < rows) {
      const int b = a.members[cl.member_off + r / G];
      const int h = kv_head * G + r % G;
      TR::load_row(st[rb].q, static_cast<const T*>(a.q) + (static_cast<size_t>(b) * a.n_q + h) * D, g);
    } else {
      TR::zero_row(st[rb].q);
    }
  }

  const size_t slab = (static_cast<size_t>(kv_head) * a.hot_cap + cl.slab_off) * D;
  const T* kb = static_cast<const T*>(a.k_hot) + slab;
  const T* vb = static_cast<const T*>(a.v_hot) + slab;
  const int n_tiles = (t1 - t0 + kPrefixTile - 1) / kPrefixTile;

  IO io;
  io.load(kb, vb, t0, t1);
  io.store(lds_k[0], lds_v[0]);
  __syncthreads();
  for (int i = 0; i < n_tiles; ++i) {
    const int buf = i & 1;
    if (i + 1 < n_tiles) io.load(kb, vb, t0 + kPrefixTile * (i + 1), t1);
    if (wave_active) {
      const int valid64 = t1 - (t0 + kPrefixTile * i);
#pragma unroll
      for (int hh = 0; hh < kPrefixTile / 32; ++hh) {
        const int valid = valid64 - 32 * hh;
        if (valid <= 0) break;
        const T* lk = &lds_k[buf][(32 * hh) * IO::kKStride];
        KOp k0[TR::KS], k1[TR::KS];
        TR::load_row(k0, lk + n * IO::kKStride, g);
        TR::load_row(k1, lk + (16 + n) * IO::kKStride, g);
        typename TR::VOp vo;
        IO::read_vop(vo, lds_v[buf], hh, lane, n, g);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) st[rb].tile(k0, k1, vo, min(valid, 32), g, c);
      }
    }
    if (i + 1 < n_tiles) io.store(lds_k[buf ^ 1], lds_v[buf ^ 1]);
    __syncthreads();
  }

  if (!wave_active) return;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float o[D / 4];
    const float lse2 = st[rb].finish(o);
    const int r = wrow0 + 16 * rb + n;
    if (r < rows) {
      const int b = a.members[cl.member_off + r / G];
      const int h = kv_head * G + r % G;
      const size_t row = (static_cast<size_t>(b) * a.max_splits + split) * a.n_q + h;
      store_row_slice(a.p_o + row * D + (D / 4) * g, o, D / 16);
      if (g == 0) a.p_lse[row] = lse2;
    }
  }
}

// ------------------------------------------------------------- merge kernel
// Requests whose slot table spans several suffix parts: one wave per
// (request, query head) joins the prefix splits and the part partials.
// Waves of single-part requests (finished by the suffix kernel) return.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void merge_kernel(StepArgs a) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  const int idx = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (idx >= a.batch * a.n_q) return;
  const int b = idx / a.n_q, h = idx % a.n_q;
  const int r = a.rank_of[b];
  const int c0 = a.part_start[r];
  const int nparts = a.part_start[r + 1] - c0;
  if (nparts == 1) return;
  const int cls = a.req_class[b];
  const int ns = cls >= 0 ? a.classes[cls].n_splits : 0;
  const size_t prow0 = static_cast<size_t>(b) * a.max_splits * a.n_q + h;
  float acc[PER];
  const float l2 = join_parts<PER, 32>(
      ns + nparts, lane,
      [&](int p) {
        return p < ns ? a.p_lse[prow0 + static_cast<size_t>(p) * a.n_q]
                      : a.s_lse[static_cast<size_t>(c0 + p - ns) * a.n_q + h];
      },
      [&](int p) -> const float* {
        return p < ns ? a.p_o + (prow0 + static_cast<size_t>(p) * a.n_q) * D + PER * lane
                      : a.s_o + (static_cast<size_t>(c0 + p - ns) * a.n_q + h) * D + PER * lane;
      },
      acc);
  T* dst = static_cast<T*>(a.out) + (static_cast<size_t>(b) * a.n_q + h) * D + PER * lane;
#pragma unroll
  for (int k = 0; k < PER; ++k) dst[k] = static_cast<T>(acc[k]);
  if (lane == 0) a.lse[idx] = l2 * 0.69314718055994531f;
}

// ------------------------------------------------------------ append kernel
__global__ __launch_bounds__(kThreads) void append_kernel(const u32x4* k_new, const u32x4* v_new,
                                                          const int32_t* slots, int32_t n,
                                                          u32x4* k_cold, u32x4* v_cold,
                                                          int64_t row_chunks, int32_t cold_cap) {
  const int64_t total = static_cast<int64_t>(n) * row_chunks;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t tok = i / row_chunks, ch = i % row_chunks;
    const int32_t s = slots[tok];
    if (s < 0 || s >= cold_cap) continue;
    k_cold[static_cast<int64_t>(s) * row_chunks + ch] = k_new[i];
    v_cold[static_cast<int64_t>(s) * row_chunks + ch] = v_new[i];
  }
}

template <typename T, int D>
hipError_t launch_typed(const StepArgs& a, int32_t backend, hipStream_t stream, hipEvent_t* ev) {
  if (ev) hipEventRecord(ev[0], stream);
  if (a.prefix_blocks > 0) {
    if (backend == 2) {
      if constexpr (sizeof(T) == 2) {
        prefix_kernel<T, D, kDenseRB><<<a.prefix_blocks, kThreads, 0, stream>>>(a);
      } else {
        return hipErrorInvalidValue;
      }
    } else {
      prefix_kernel<T, D, kCascadeRB><<<a.prefix_blocks, kThreads, 0, stream>>>(a);
    }
  }
  if (ev) hipEventRecord(ev[1], stream);
  suffix_kernel<T, D><<<a.suffix_blocks, kThreads, 0, stream>>>(a);
  if (ev) hipEventRecord(ev[2], stream);
  if (a.multi_part) {
    const int pairs = a.batch * a.n_q;
    merge_kernel<T, D><<<(pairs + kWaves - 1) / kWaves, kThreads, 0, stream>>>(a);
  }
  if (ev) hipEventRecord(ev[3], stream);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_cold_append(const void* k_new, const void* v_new, const int32_t* slots, int32_t n,
                              void* k_cold, void* v_cold, int64_t row_bytes, int32_t cold_cap,
                              hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t row_chunks = row_bytes / 16;
  const int64_t total = static_cast<int64_t>(n) * row_chunks;
  const int64_t blocks = (total + kThreads - 1) / kThreads;
  const int grid = static_cast<int>(blocks < 4096 ? blocks : 4096);
  append_kernel<<<grid, kThreads, 0, stream>>>(
      static_cast<const u32x4*>(k_new), static_cast<const u32x4*>(v_new), slots, n,
      static_cast<u32x4*>(k_cold), static_cast<u32x4*>(v_cold), row_chunks, cold_cap);
  return hipGetLastError();
}

hipError_t launch_step(const StepArgs& a, int32_t dtype, int32_t backend, hipStream_t stream,
                       hipEvent_t* ev) {
  if (dtype == 1) {
    return a.head_dim == 128 ? launch_typed<__bf16, 128>(a, backend, stream, ev)
                             : launch_typed<__bf16, 64>(a, backend, stream, ev);
  }
  return a.head_dim == 128 ? launch_typed<float, 128>(a, backend, stream, ev)
                           : launch_typed<float, 64>(a, backend, stream, ev);
}

}  // namespace gkv
