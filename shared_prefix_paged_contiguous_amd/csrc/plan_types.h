// Work descriptors of one decode step, shared by the host planner and the
// device kernels.  Plain structs: the planner writes them into a pinned host
// buffer, one async copy moves them into the device workspace.
#pragma once

#include <cstdint>

namespace gkv {

// Prefix kernel tiling.  A workgroup is 4 waves; each wave owns RB blocks of
// 16 query rows (one MFMA column block each), so a workgroup tile covers
// 64*RB rows of one class and one KV head.  K/V tiles of kPrefixTile tokens
// are staged through LDS.
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kPrefixTile = 64;
constexpr int kCascadeRB = 1;     // cascade backend: 64-row tiles, many L splits
constexpr int kDenseRB = 2;       // dense backend: 128-row tiles (batched GEMM)
constexpr int kSuffixTile = 32;   // suffix kernel token tile (per wave)
constexpr int kMaxSplits = 64;    // L splits per prefix class

// One distinct HOT prefix in the step ("class": every request that starts
// with this slab).
struct PrefixClass {
  int64_t slab_off;     // token offset of the slab in the HOT pool
  int32_t len;          // slab length L_c (tokens)
  int32_t n_members;    // requests of the class
  int32_t member_off;   // first entry in the member list
  int32_t n_splits;     // L splits S_c
  int32_t chunk;        // tokens per split (the last split may be shorter)
  int32_t pad_;
};

// One prefix workgroup: rows [row0, row0 + 64*RB) of class `cls` (row r is
// member r / G, query head kv_head*G + r % G) against tokens
// [split*chunk, min(len, (split+1)*chunk)) of the slab.  cls < 0: idle
// (padding of the XCD-aware block order).
struct PrefixItem {
  int32_t cls;
  int32_t kv_head;
  int32_t row0;
  int32_t split;
};

// One suffix wave: request b, KV head kv_head, slot-table positions [t0, t1).
// Its G query heads write partial rows (part * n_q + h).
struct SuffixItem {
  int32_t b;
  int32_t kv_head;
  int32_t t0;
  int32_t t1;
  int32_t part;
  int32_t pad_[3];
};

// Per request: where its partials are, for the merge.
struct ReqInfo {
  int32_t cls;          // prefix class, -1 = none
  int32_t prefix_base;  // prefix partial row of split s, head h: prefix_base + s*n_q + h
  int32_t n_splits;     // 0 if no prefix
  int32_t chunk_base;   // first suffix part id
  int32_t n_chunks;     // suffix parts (0 if the slot table is empty)
  int32_t pad_[3];
};

// Everything a step's kernels read, passed by value.
struct StepArgs {
  int32_t batch, n_q, n_kv, group, head_dim;
  float scale_log2;            // log2(e) / sqrt(head_dim)
  const void* q;
  void* out;
  float* lse;
  const void* k_hot;
  const void* v_hot;
  int64_t hot_cap;
  const void* k_cold;
  const void* v_cold;
  int32_t cold_cap;
  const int32_t* cold_indices;
  const PrefixClass* classes;
  const int32_t* members;
  const PrefixItem* prefix_items;
  int32_t n_prefix_items;
  const SuffixItem* suffix_items;
  int32_t n_suffix_items;
  const ReqInfo* reqs;
  float* p_o;                  // prefix partials [rows][head_dim], normalised
  float* p_lse;                // prefix partial log2-sum-exp2 of scaled scores
  float* s_o;                  // suffix partials
  float* s_lse;
};

}  // namespace gkv
