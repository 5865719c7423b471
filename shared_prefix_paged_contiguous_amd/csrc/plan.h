// Host planner of one decode step: class grouping, the per-step backend rule
// and the work decomposition of the step kernel (prefix splits, suffix parts,
// joins), all written into the kernel-argument block (StepArgs).  Pure C++.
//
// Class grouping: paperlayer.ai summary of the GraniKV paper, Appendix B.8
// (each distinct prefix is batched against its own slab, "class-local"
// batching).  Backend rule: §3 "Per-step dispatch" and Appendix B.4 (dense
// iff M_eff = B * n_q/n_kv >= M_sat, decided on the realised batch).
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

#include "plan_types.h"
#include "pools.h"

namespace gkv {

struct PlanShape {
  int32_t n_q, n_kv, head_dim;
  bool bf16;
  int32_t xcds = kDefaultCus / kCusPerXcd;   // XCDs of the device
  int32_t cus = kDefaultCus;                  // compute units of the device
};

struct Plan {
  int32_t backend = 0;          // GKV_BACKEND_CASCADE / _DENSE
  int32_t m_eff = 0;
  int32_t n_classes = 0;
  int32_t prefix_blocks = 0;    // prefix workgroups (including idle XCD padding)
  int32_t suffix_blocks = 0;    // suffix workgroups (incl. padding)
  int32_t join_blocks = 0;      // join workgroups
  int32_t n_parts = 0;          // suffix parts (>= one per request but the short ones)
  int32_t multi_part = 0;       // some request's output is joined from several partials
  int64_t prefix_rows = 0;      // prefix partial rows (B * max_splits * n_q)
  int64_t suffix_rows = 0;      // suffix partial rows
  int32_t part_tokens = 0;      // slot-table tokens per suffix part
  int32_t rb = 1;               // row blocks per wave of the prefix tiles
  int32_t fold = 0;             // suffix workgroups run folded pairs of parts
  int32_t n_short = 0;          // short requests, attended by their own join workgroups
};

// Rule alone: dense iff batch * group >= m_sat (unless forced).
int32_t choose_backend(int32_t batch, int32_t group, int32_t m_sat, int32_t force);

// Validates the step and fills the work-description part of `a` (classes,
// members, chunk starts, counts).  Returns 0, or -1 with a message in err.
int build_plan(const PlanShape& shape, const HotPool& hot, int32_t batch,
               const int32_t* hot_prefix_ids, const int32_t* indptr, int32_t backend,
               StepArgs& a, Plan& plan, std::string& err);

// Upper bounds used to size the workspace.
int64_t prefix_rows_bound(const PlanShape& shape, int32_t max_batch);
int64_t suffix_rows_bound(const PlanShape& shape, int32_t max_batch, int64_t max_suffix_tokens);

inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

}  // namespace gkv
