#include "plan.h"

#include <algorithm>

#include "../../include/gkv.h"

namespace gkv {

namespace {

constexpr int32_t kMinSplitTokens = 256;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

}  // namespace

int32_t choose_backend(int32_t batch, int32_t group, int32_t m_sat, int32_t force) {
  if (force == GKV_BACKEND_CASCADE || force == GKV_BACKEND_DENSE) return force;
  const int64_t m_eff = static_cast<int64_t>(batch) * group;
  return m_eff >= m_sat ? GKV_BACKEND_DENSE : GKV_BACKEND_CASCADE;
}

int64_t prefix_rows_bound(const PlanShape& s, int32_t max_batch) {
  return static_cast<int64_t>(max_batch) * kMaxSplits * s.n_q;
}

int64_t suffix_rows_bound(const PlanShape& s, int32_t max_batch, int64_t max_suffix_tokens) {
  return (max_suffix_tokens / kSuffixPart + max_batch) * s.n_q;
}

int build_plan(const PlanShape& shape, const HotPool& hot, int32_t batch, const int32_t* ids,
               const int32_t* indptr, int32_t backend, StepArgs& a, Plan& plan, std::string& err) {
  const int32_t n_q = shape.n_q, n_kv = shape.n_kv, group = n_q / n_kv;
  const int32_t xcds = std::max(1, shape.xcds);
  const int64_t step_slots = static_cast<int64_t>(kWgsPerCu) * std::max(1, shape.cus);
  const int64_t pad = static_cast<int64_t>(kGroupPerXcd) * xcds;   // padding unit of the grid ranges
  plan = Plan();
  plan.backend = backend;
  plan.m_eff = batch * group;
  if (batch > kMaxBatch) {
    err = "batch " + std::to_string(batch) + " exceeds the per-call limit " + std::to_string(kMaxBatch);
    return -1;
  }
  if (indptr[0] < 0) {
    err = "cold_indptr[0] is negative";
    return -1;
  }

  // ---- validation and class grouping (order of first appearance)
  int32_t class_id[kMaxClasses];
  int32_t class_size[kMaxClasses];
  int32_t n_classes = 0;
  int32_t last_id = -1, last_cls = -1;
  for (int32_t b = 0; b < batch; ++b) {
    const int32_t s_b = indptr[b + 1] - indptr[b];
    if (s_b < 0) {
      err = "cold_indptr decreases at request " + std::to_string(b);
      return -1;
    }
    const int32_t id = ids[b];
    if (id < -1) {
      err = "hot_prefix_ids[" + std::to_string(b) + "] < -1";
      return -1;
    }
    if (id == -1) {
      if (s_b == 0) {
        err = "request " + std::to_string(b) + " has neither a prefix nor a suffix";
        return -1;
      }
      a.req_class[b] = -1;
      continue;
    }
    int32_t c = -1;
    if (id == last_id) {
      c = last_cls;
    } else {
      for (int32_t i = 0; i < n_classes; ++i)
        if (class_id[i] == id) { c = i; break; }
      if (c < 0) {
        int64_t off;
        int32_t len;
        if (!hot.lookup(id, &off, &len)) {
          err = "hot prefix id " + std::to_string(id) + " is not live";
          return -1;
        }
        if (n_classes == kMaxClasses) {
          err = "more than " + std::to_string(kMaxClasses) + " distinct HOT prefixes in one step";
          return -1;
        }
        c = n_classes++;
        class_id[c] = id;
        class_size[c] = 0;
        a.classes[c].slab_off = off;
        a.classes[c].len = len;
      }
      last_id = id;
      last_cls = c;
    }
    a.req_class[b] = static_cast<int8_t>(c);
    class_size[c]++;
  }
  plan.n_classes = n_classes;
  a.n_classes = n_classes;

  // ---- members grouped by class
  {
    int32_t off = 0;
    for (int32_t c = 0; c < n_classes; ++c) {
      a.classes[c].member_off = off;
      a.classes[c].n_members = 0;
      off += class_size[c];
    }
    for (int32_t b = 0; b < batch; ++b) {
      const int32_t c = a.req_class[b];
      if (c < 0) continue;
      ClassDesc& cd = a.classes[c];
      a.members[cd.member_off + cd.n_members++] = static_cast<int16_t>(b);
    }
  }

  // ---- prefix splits: one split length for all classes so that the total
  // work (KV heads x M-tiles x tokens) spreads over about kTargetBlocks
  // workgroups, with at least kMinSplitTokens tokens per split.
  int32_t max_rows = 0;
  for (int32_t c = 0; c < n_classes; ++c) max_rows = std::max(max_rows, class_size[c] * group);
  const int32_t rb = shape.bf16 && (backend == GKV_BACKEND_DENSE || max_rows > kSmallTileRows) ? 2 : 1;
  a.rb = rb;
  plan.rb = rb;
  const int32_t target = backend == GKV_BACKEND_DENSE ? kDenseTarget : kCascadeTarget;
  const int32_t tm = tile_members(group, rb);
  if (tm < 1) {
    err = "query group of " + std::to_string(group) + " heads exceeds one prefix tile";
    return -1;
  }
  int64_t units = 0;
  for (int32_t c = 0; c < n_classes; ++c)
    units += static_cast<int64_t>(n_kv) * ceil_div(class_size[c], tm) * a.classes[c].len;
  // one split length for every class; returns the prefix blocks it makes
  auto split_classes = [&](int64_t split_tokens) {
    int32_t nb = 0;
    for (int32_t c = 0; c < n_classes; ++c) {
      ClassDesc& cd = a.classes[c];
      const int64_t len = cd.len;
      int64_t s = std::min<int64_t>(kMaxSplits, std::max<int64_t>(1, ceil_div(len, split_tokens)));
      const int64_t chunk = round_up(ceil_div(len, s), kPrefixTile);
      s = ceil_div(len, chunk);
      cd.n_splits = static_cast<int32_t>(s);
      cd.chunk = static_cast<int32_t>(chunk);
      cd.m_tiles = static_cast<int32_t>(ceil_div(cd.n_members, tm));
      cd.n_groups = n_kv * cd.n_splits;
      cd.block_base = nb;
      cd.n_blocks = xcds * static_cast<int32_t>(ceil_div(cd.n_groups, xcds)) * cd.m_tiles;
      cd.pad_ = 0;
      nb += cd.n_blocks;
    }
    return static_cast<int32_t>(round_up(nb, pad));
  };
  const int64_t split0 = std::max<int64_t>(
      kMinSplitTokens, round_up(ceil_div(std::max<int64_t>(units, 1), target), kPrefixTile));
  int32_t blocks = split_classes(split0);
  if (backend == GKV_BACKEND_DENSE && n_classes > 0) {
    // Dense steps give every slot to prefix work, and the busiest CU sets the
    // time: k = ceil(blocks / CUs) workgroups of one split length each, two
    // at a time (a CU with two resident prefix workgroups does about 1.25x
    // the work per unit time of a CU with one; measured) and the odd last one
    // alone, plus a fixed cost per workgroup (query rows, ring fill, partial
    // rows: about eight blocks' worth).  Take the split length with the least
    // such time; ties go to the fewer workgroups.
    int64_t lmax = 0;
    for (int32_t c = 0; c < n_classes; ++c) lmax = std::max<int64_t>(lmax, a.classes[c].len);
    const int64_t cus = std::max(1, shape.cus);
    double best = 0.0;
    int64_t best_st = split0;
    int32_t best_blocks = 0;
    for (int64_t ns = 1; ns <= kMaxSplits; ++ns) {
      const int64_t st = std::max<int64_t>(kMinSplitTokens, round_up(ceil_div(lmax, ns), kPrefixTile));
      const int32_t nb = split_classes(st);
      const int64_t k = ceil_div(nb, cus);
      const double per = static_cast<double>(std::min(st, lmax)) + 8.0 * kHotBlock;   // one workgroup
      const double t = (k / 2) * 2 * per / 1.25 + (k % 2) * per;
      if (best_blocks == 0 || t < best || (t == best && nb < best_blocks)) {
        best = t;
        best_st = st;
        best_blocks = nb;
      }
    }
    blocks = split_classes(best_st);
  }
  // Cascade: when folded suffix pairs (see below) would not fit beside this
  // prefix grid but would beside a somewhat smaller one, lengthen the splits
  // (up to twice) until they fit.
  if (backend == GKV_BACKEND_CASCADE && n_classes > 0) {
    int64_t parts = 0;
    for (int32_t b = 0; b < batch; ++b)
      if (indptr[b + 1] - indptr[b] > kInlineTokens || a.req_class[b] < 0)   // short requests have none
        parts += std::max<int64_t>(1, ceil_div(indptr[b + 1] - indptr[b], kSuffixPart));
    const int64_t pairs = ceil_div(parts, 2) * n_kv;
    if (parts > 1 && parts * n_kv > step_slots - blocks && pairs > step_slots - blocks &&
        pairs <= step_slots - pad) {
      int64_t st = split0 + kPrefixTile;
      while (st <= 2 * split0 && split_classes(st) > step_slots - pairs) st += kPrefixTile;
      blocks = split_classes(st <= 2 * split0 ? st : split0);   // the classes keep the last call's splits
    }
  }
  int32_t max_splits = 0;
  for (int32_t c = 0; c < n_classes; ++c) max_splits = std::max(max_splits, a.classes[c].n_splits);
  a.prefix_blocks = static_cast<int32_t>(round_up(blocks, pad));
  a.max_splits = max_splits;
  plan.prefix_blocks = a.prefix_blocks;
  plan.prefix_rows = static_cast<int64_t>(batch) * max_splits * n_q;

  // ---- suffix parts, longest slot table first (so the longest workgroups
  // start first and the kernel's tail is short); short requests (a HOT
  // prefix and at most kInlineTokens slot-table tokens) last, without parts:
  // their join workgroups attend their tables
  auto is_short = [&](int32_t b) {
    return a.req_class[b] >= 0 && indptr[b + 1] - indptr[b] <= kInlineTokens;
  };
  int32_t order[kMaxBatch];
  for (int32_t b = 0; b < batch; ++b) order[b] = b;
  std::stable_sort(order, order + batch, [&](int32_t x, int32_t y) {
    const bool sx = is_short(x), sy = is_short(y);
    if (sx != sy) return sy;
    return indptr[x + 1] - indptr[x] > indptr[y + 1] - indptr[y];
  });
  int64_t parts = 0;
  int32_t multi = 0;
  int32_t inline_rank0 = batch;
  for (int32_t r = 0; r < batch; ++r) {
    const int32_t b = order[r];
    a.rank_of[b] = static_cast<int16_t>(r);
    a.ranks[r] = RankDesc{indptr[b], indptr[b + 1], static_cast<int32_t>(parts), b};
    if (is_short(b)) {
      inline_rank0 = std::min(inline_rank0, r);
      continue;
    }
    const int64_t np = std::max<int64_t>(1, ceil_div(indptr[b + 1] - indptr[b], kSuffixPart));
    if (np > 1) multi = 1;
    parts += np;
  }
  if ((parts + pad) * n_kv + static_cast<int64_t>(batch) * n_kv + blocks > 0x7fffffffLL) {
    err = "too many suffix parts";
    return -1;
  }
  a.n_parts = static_cast<int32_t>(parts);
  a.tail = kArgsTail;
  // fold pairs of parts when the parts' workgroups overflow the slots the
  // prefix leaves and the folded ones fit (cascade steps only: dense fills
  // every slot with prefix work).  Folding into a second round of paired
  // workgroups is slower than not folding.
  const int64_t free_slots = step_slots - static_cast<int64_t>(a.prefix_blocks);
  const bool fold = backend == GKV_BACKEND_CASCADE && parts > 1 && parts * n_kv > free_slots &&
                    ceil_div(parts, 2) * n_kv <= free_slots;
  a.fold = fold ? 1 : 0;
  a.xcds = xcds;
  a.suffix_blocks = static_cast<int32_t>(round_up((fold ? ceil_div(parts, 2) : parts) * n_kv, pad));
  plan.fold = a.fold;
  a.multi_part = multi;
  a.need_merge = multi || n_classes > 0;
  a.inline_rank0 = inline_rank0;
  // each short request's tiles go to a partial row set of its own, after
  // the suffix parts' rows
  for (int32_t r = inline_rank0; r < batch; ++r) a.ranks[r].part0 = static_cast<int32_t>(parts) + (r - inline_rank0);
  // short requests: one join workgroup each, or several when there are more
  // of them than workgroup slots (a second round of workgroups would start
  // only as the first round ends)
  const int32_t n_short = batch - inline_rank0;
  const int32_t short_per = n_short > step_slots ? static_cast<int32_t>(ceil_div(n_short, step_slots)) : 1;
  a.short_per_block = short_per;
  // every slot table is one part: the suffix workgroups join their requests
  // (see StepArgs), and only the short requests have join workgroups.  A
  // suffix workgroup that joins waits for its requests' prefix splits and
  // holds its slot meanwhile, so a cascade step does this only when its
  // prefix and suffix workgroups are all resident at once (a suffix
  // workgroup waiting on a long prefix would otherwise keep the next round
  // of suffix work from starting: Llama-3.1-8B shape B = 256, 2048 suffix
  // workgroups in 7 rounds, 164 -> 196 us).  Dense steps start their
  // suffix workgroups as the prefix splits end, so their waits are short.
  a.suffix_joins = (multi == 0 && parts > 0 &&
                    (backend == GKV_BACKEND_DENSE ||
                     static_cast<int64_t>(a.prefix_blocks) + a.suffix_blocks <= step_slots))
                       ? 1
                       : 0;
  const int32_t ranked_joins = a.suffix_joins ? 0 : inline_rank0 * n_kv;
  a.join_blocks = a.need_merge ? ranked_joins + static_cast<int32_t>(ceil_div(n_short, short_per)) : 0;
  plan.n_short = n_short;
  plan.n_parts = static_cast<int32_t>(parts);
  plan.part_tokens = kSuffixPart;
  plan.suffix_blocks = a.suffix_blocks;
  plan.join_blocks = a.join_blocks;
  plan.multi_part = a.need_merge;
  plan.suffix_rows = a.need_merge ? (parts + (batch - inline_rank0)) * n_q : 0;
  return 0;
}

}  // namespace gkv
