// Host planner of one decode step: class grouping, the per-step backend rule
// and the work lists of the prefix, suffix and merge kernels.  Pure C++.
//
// Class grouping: paperlayer.ai summary of the GraniKV paper, Appendix B.8
// (each distinct prefix is batched against its own slab, "class-local"
// batching).  Backend rule: §3 "Per-step dispatch" and Appendix B.4 (dense
// iff M_eff = B * n_q/n_kv >= M_sat, decided on the realised batch).
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "plan_types.h"
#include "pools.h"

namespace gkv {

struct PlanShape {
  int32_t n_q, n_kv, head_dim;
};

struct Plan {
  int32_t backend = 0;          // GKV_BACKEND_CASCADE / _DENSE
  int32_t m_eff = 0;
  int32_t n_classes = 0;
  int32_t n_prefix_items = 0;   // prefix workgroups (including idle padding)
  int32_t n_suffix_items = 0;   // suffix waves
  int32_t n_chunks = 0;         // suffix parts
  int32_t suffix_chunk = 0;     // tokens per suffix part
  int64_t prefix_rows = 0;      // prefix partial rows
  int64_t suffix_rows = 0;      // suffix partial rows
  // byte offsets inside the plan blob (each 256-byte aligned)
  size_t off_classes = 0, off_members = 0, off_prefix = 0, off_suffix = 0, off_reqs = 0;
  size_t blob_bytes = 0;
};

// Rule alone: dense iff batch * group >= m_sat.
int32_t choose_backend(int32_t batch, int32_t group, int32_t m_sat, int32_t force);

// Fills `blob` and `plan`.  Returns 0 or -1 (message in err).  hot lookups go
// through `hot`.  `backend` is GKV_BACKEND_CASCADE or GKV_BACKEND_DENSE.
int build_plan(const PlanShape& shape, const HotPool& hot, int32_t batch,
               const int32_t* hot_prefix_ids, const int32_t* indptr, int32_t backend,
               std::vector<uint8_t>& blob, Plan& plan, std::string& err);

// Upper bounds used to size the workspace.
size_t plan_blob_bound(const PlanShape& shape, int32_t max_batch, int64_t max_suffix_tokens);
int64_t prefix_rows_bound(const PlanShape& shape, int32_t max_batch);
int64_t suffix_rows_bound(const PlanShape& shape, int32_t max_batch, int64_t max_suffix_tokens);

inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

}  // namespace gkv
