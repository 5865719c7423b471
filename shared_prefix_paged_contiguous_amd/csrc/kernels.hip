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

#include "kernels.h"

namespace gkv {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));

constexpr float kNegInf = -__builtin_inff();

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
    const float m_new = fmaxf(m, mx);
    if (__any(m_new > m)) {   // rescale only when some column's max moved
      const float alpha = exp2f(m - m_new);
      l *= alpha;
#pragma unroll
      for (int j = 0; j < TR::EPB; ++j) acc[j] *= alpha;
      m = m_new;
    }
    f32x4 p0, p1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p0[i] = exp2f(__builtin_fmaf(s0[i], c, -m));
      p1[i] = exp2f(__builtin_fmaf(s1[i], c, -m));
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

// ------------------------------------------------------------ suffix kernel
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void suffix_kernel(StepArgs a) {
  using TR = Traits<T, D>;
  using KOp = typename TR::KOp;
  using VVec = typename TR::VVec;
  const int lane = threadIdx.x & 63;
  const int item_id = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (item_id >= a.n_suffix_items) return;   // no barriers in this kernel
  const SuffixItem it = a.suffix_items[item_id];
  const int n = lane & 15, g = lane >> 4;
  const bool col_ok = n < a.group;
  const int h = it.kv_head * a.group + (col_ok ? n : 0);
  const float c = a.scale_log2;

  ColState<T, D> st;
  st.init();
  if (col_ok) TR::load_row(st.q, static_cast<const T*>(a.q) + (static_cast<size_t>(it.b) * a.n_q + h) * D, g);
  else TR::zero_row(st.q);

  const size_t stride = static_cast<size_t>(a.n_kv) * D;
  const T* kc = static_cast<const T*>(a.k_cold) + it.kv_head * D;
  const T* vc = static_cast<const T*>(a.v_cold) + it.kv_head * D + TR::EPB * n;
  const int n_tiles = (it.t1 - it.t0 + kSuffixTile - 1) / kSuffixTile;
  const int cap1 = a.cold_cap - 1;

  // slot id of token (lane % 32) of tile i (clamped into the tile and the pool)
  auto load_slot = [&](int i) {
    const int t = it.t0 + kSuffixTile * i;
    const int last = min(kSuffixTile, it.t1 - t) - 1;
    const int s = a.cold_indices[t + min(lane & 31, last)];
    return min(max(s, 0), cap1);
  };
  auto load_kv = [&](int slot, KOp (&k0)[TR::KS], KOp (&k1)[TR::KS], VVec (&v)[8]) {
    const int s0 = __shfl(slot, n), s1 = __shfl(slot, 16 + n);
    TR::load_row(k0, kc + static_cast<size_t>(s0) * stride, g);
    TR::load_row(k1, kc + static_cast<size_t>(s1) * stride, g);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int se = __shfl(slot, tau(g, e));
      v[e] = TR::load_v(vc + static_cast<size_t>(se) * stride);
    }
  };

  KOp k0[TR::KS], k1[TR::KS];
  VVec v[8];
  load_kv(load_slot(0), k0, k1, v);
  int slot_next = n_tiles > 1 ? load_slot(1) : 0;
  for (int i = 0; i < n_tiles; ++i) {
    KOp nk0[TR::KS], nk1[TR::KS];
    VVec nv[8];
    if (i + 1 < n_tiles) load_kv(slot_next, nk0, nk1, nv);
    if (i + 2 < n_tiles) slot_next = load_slot(i + 2);
    typename TR::VOp vo;
    TR::make_vop(vo, v);
    st.tile(k0, k1, vo, min(kSuffixTile, it.t1 - it.t0 - kSuffixTile * i), g, c);
    if (i + 1 < n_tiles) {
#pragma unroll
      for (int s = 0; s < TR::KS; ++s) { k0[s] = nk0[s]; k1[s] = nk1[s]; }
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = nv[e];
    }
  }

  float o[D / 4];
  const float lse2 = st.finish(o);
  if (col_ok) {
    const size_t row = static_cast<size_t>(it.part) * a.n_q + h;
    store_row_slice(a.s_o + row * D + (D / 4) * g, o, D / 16);
    if (g == 0) a.s_lse[row] = lse2;
  }
}

// ------------------------------------------------------------ prefix kernel
template <typename T, int D, int RB>
__global__ __launch_bounds__(kThreads) void prefix_kernel(StepArgs a) {
  using TR = Traits<T, D>;
  using KOp = typename TR::KOp;
  using VVec = typename TR::VVec;
  constexpr int kStride = D + 16 / static_cast<int>(sizeof(T));   // padded LDS row (elements)
  constexpr int kChunksPerRow = D * static_cast<int>(sizeof(T)) / 16;
  constexpr int kChunks = kPrefixTile * kChunksPerRow / kThreads;  // 16-byte chunks per thread
  constexpr int kElemsPerChunk = 16 / static_cast<int>(sizeof(T));
  __shared__ __attribute__((aligned(16))) T lds_k[2][kPrefixTile * kStride];
  __shared__ __attribute__((aligned(16))) T lds_v[2][kPrefixTile * kStride];

  const PrefixItem it = a.prefix_items[blockIdx.x];
  if (it.cls < 0) return;   // whole workgroup leaves before any barrier
  const PrefixClass cl = a.classes[it.cls];
  const int t0 = it.split * cl.chunk;
  const int t1 = min(cl.len, t0 + cl.chunk);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int G = a.group;
  const int rows = cl.n_members * G;
  const float c = a.scale_log2;
  const int wrow0 = it.row0 + wave * 16 * RB;
  const bool wave_active = wrow0 < rows;

  ColState<T, D> st[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    st[rb].init();
    const int r = wrow0 + 16 * rb + n;
    if (r < rows) {
      const int b = a.members[cl.member_off + r / G];
      const int h = it.kv_head * G + r % G;
      TR::load_row(st[rb].q, static_cast<const T*>(a.q) + (static_cast<size_t>(b) * a.n_q + h) * D, g);
    } else {
      TR::zero_row(st[rb].q);
    }
  }

  const size_t slab = (static_cast<size_t>(it.kv_head) * a.hot_cap + cl.slab_off) * D;
  const T* kb = static_cast<const T*>(a.k_hot) + slab;
  const T* vb = static_cast<const T*>(a.v_hot) + slab;
  const int n_tiles = (t1 - t0 + kPrefixTile - 1) / kPrefixTile;

  u32x4 stk[kChunks], stv[kChunks];
  auto stage = [&](int i) {   // global -> registers, rows clamped into [t0, t1)
    const int tt = t0 + kPrefixTile * i;
#pragma unroll
    for (int j = 0; j < kChunks; ++j) {
      const int ch = threadIdx.x + kThreads * j;
      const int row = ch / kChunksPerRow, col = ch % kChunksPerRow;
      const size_t off = static_cast<size_t>(min(tt + row, t1 - 1)) * D + col * kElemsPerChunk;
      stk[j] = *reinterpret_cast<const u32x4*>(kb + off);
      stv[j] = *reinterpret_cast<const u32x4*>(vb + off);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int j = 0; j < kChunks; ++j) {
      const int ch = threadIdx.x + kThreads * j;
      const int row = ch / kChunksPerRow, col = ch % kChunksPerRow;
      *reinterpret_cast<u32x4*>(&lds_k[buf][row * kStride + col * kElemsPerChunk]) = stk[j];
      *reinterpret_cast<u32x4*>(&lds_v[buf][row * kStride + col * kElemsPerChunk]) = stv[j];
    }
  };

  stage(0);
  store(0);
  __syncthreads();
  for (int i = 0; i < n_tiles; ++i) {
    const int buf = i & 1;
    if (i + 1 < n_tiles) stage(i + 1);
    if (wave_active) {
      const int valid64 = t1 - (t0 + kPrefixTile * i);
#pragma unroll
      for (int hh = 0; hh < kPrefixTile / 32; ++hh) {
        const int valid = valid64 - 32 * hh;
        if (valid <= 0) break;
        const T* lk = &lds_k[buf][(32 * hh) * kStride];
        const T* lv = &lds_v[buf][(32 * hh) * kStride];
        KOp k0[TR::KS], k1[TR::KS];
        TR::load_row(k0, lk + n * kStride, g);
        TR::load_row(k1, lk + (16 + n) * kStride, g);
        VVec v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = TR::load_v(lv + tau(g, e) * kStride + TR::EPB * n);
        typename TR::VOp vo;
        TR::make_vop(vo, v);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) st[rb].tile(k0, k1, vo, min(valid, 32), g, c);
      }
    }
    if (i + 1 < n_tiles) store(buf ^ 1);
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
      const int h = it.kv_head * G + r % G;
      const size_t row = static_cast<size_t>(a.reqs[b].prefix_base) + static_cast<size_t>(it.split) * a.n_q + h;
      store_row_slice(a.p_o + row * D + (D / 4) * g, o, D / 16);
      if (g == 0) a.p_lse[row] = lse2;
    }
  }
}

// ------------------------------------------------------------- merge kernel
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void merge_kernel(StepArgs a) {
  const int lane = threadIdx.x & 63;
  const int idx = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (idx >= a.batch * a.n_q) return;
  const int b = idx / a.n_q, h = idx % a.n_q;
  const ReqInfo r = a.reqs[b];
  const int np = r.n_splits + r.n_chunks;
  auto lse_of = [&](int p) -> float {
    return p < r.n_splits ? a.p_lse[r.prefix_base + p * a.n_q + h]
                          : a.s_lse[(r.chunk_base + p - r.n_splits) * a.n_q + h];
  };
  auto o_of = [&](int p) -> const float* {
    const size_t row = p < r.n_splits ? static_cast<size_t>(r.prefix_base) + static_cast<size_t>(p) * a.n_q + h
                                      : static_cast<size_t>(r.chunk_base + p - r.n_splits) * a.n_q + h;
    return (p < r.n_splits ? a.p_o : a.s_o) + row * D;
  };
  float mx = kNegInf;
  for (int p = lane; p < np; p += 64) mx = fmaxf(mx, lse_of(p));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  constexpr int PER = D / 64;   // output elements per lane
  float acc[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) acc[j] = 0.f;
  float wsum = 0.f;
  for (int p = 0; p < np; ++p) {
    const float w = exp2f(lse_of(p) - mx);
    wsum += w;
    const float* src = o_of(p) + PER * lane;
#pragma unroll
    for (int j = 0; j < PER; ++j) acc[j] += w * src[j];
  }
  const float inv = 1.f / wsum;
  T* dst = static_cast<T*>(a.out) + (static_cast<size_t>(b) * a.n_q + h) * D + PER * lane;
#pragma unroll
  for (int j = 0; j < PER; ++j) dst[j] = static_cast<T>(acc[j] * inv);
  if (lane == 0) a.lse[idx] = (mx + __log2f(wsum)) * 0.69314718055994531f;
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
hipError_t launch_typed(const StepArgs& a, int32_t backend, hipStream_t stream) {
  if (a.n_prefix_items > 0) {
    if (backend == 2) {
      if constexpr (sizeof(T) == 2) {
        prefix_kernel<T, D, kDenseRB><<<a.n_prefix_items, kThreads, 0, stream>>>(a);
      } else {
        return hipErrorInvalidValue;
      }
    } else {
      prefix_kernel<T, D, kCascadeRB><<<a.n_prefix_items, kThreads, 0, stream>>>(a);
    }
  }
  if (a.n_suffix_items > 0)
    suffix_kernel<T, D><<<(a.n_suffix_items + kWaves - 1) / kWaves, kThreads, 0, stream>>>(a);
  const int pairs = a.batch * a.n_q;
  merge_kernel<T, D><<<(pairs + kWaves - 1) / kWaves, kThreads, 0, stream>>>(a);
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

hipError_t launch_step(const StepArgs& a, int32_t dtype, int32_t backend, hipStream_t stream) {
  if (dtype == 1) {
    return a.head_dim == 128 ? launch_typed<__bf16, 128>(a, backend, stream)
                             : launch_typed<__bf16, 64>(a, backend, stream);
  }
  return a.head_dim == 128 ? launch_typed<float, 128>(a, backend, stream)
                           : launch_typed<float, 64>(a, backend, stream);
}

}  // namespace gkv
