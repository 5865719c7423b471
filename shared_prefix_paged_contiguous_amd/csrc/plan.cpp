#include "plan.h"

#include <algorithm>
#include <cstring>

#include "../../include/gkv.h"

namespace gkv {

namespace {

constexpr int32_t kCascadeTargetBlocks = 512;  // prefix workgroups to aim for
constexpr int32_t kDenseTargetBlocks = 512;
constexpr int32_t kMinSplitTokens = 256;
constexpr int32_t kSuffixTargetWaves = 2048;
constexpr int32_t kMinSuffixChunk = 32;
constexpr int kXcds = 8;  // MI355X: workgroups go to the 8 XCDs round-robin

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

int64_t suffix_waves(const int32_t* indptr, int32_t batch, int32_t n_kv, int32_t chunk) {
  int64_t w = 0;
  for (int32_t b = 0; b < batch; ++b) w += ceil_div(indptr[b + 1] - indptr[b], chunk);
  return w * n_kv;
}

}  // namespace

int32_t choose_backend(int32_t batch, int32_t group, int32_t m_sat, int32_t force) {
  if (force == GKV_BACKEND_CASCADE || force == GKV_BACKEND_DENSE) return force;
  const int64_t m_eff = static_cast<int64_t>(batch) * group;
  return m_eff >= m_sat ? GKV_BACKEND_DENSE : GKV_BACKEND_CASCADE;
}

size_t plan_blob_bound(const PlanShape& s, int32_t max_batch, int64_t max_suffix_tokens) {
  const int64_t group = s.n_q / s.n_kv;
  const int64_t mt_sum = max_batch * group / 64 + max_batch;           // sum of M-tiles over classes
  const int64_t prefix_items = static_cast<int64_t>(s.n_kv) * kMaxSplits * mt_sum +
                               kXcds * (max_batch * group / 64 + 1) + kXcds;
  const int64_t suffix_items =
      static_cast<int64_t>(s.n_kv) * (max_suffix_tokens / kMinSuffixChunk + max_batch);
  return align256(sizeof(PrefixClass) * max_batch) + align256(sizeof(int32_t) * max_batch) +
         align256(sizeof(PrefixItem) * prefix_items) +
         align256(sizeof(SuffixItem) * suffix_items) + align256(sizeof(ReqInfo) * max_batch);
}

int64_t prefix_rows_bound(const PlanShape& s, int32_t max_batch) {
  return static_cast<int64_t>(max_batch) * kMaxSplits * s.n_q;
}

int64_t suffix_rows_bound(const PlanShape& s, int32_t max_batch, int64_t max_suffix_tokens) {
  return (max_suffix_tokens / kMinSuffixChunk + max_batch) * s.n_q;
}

int build_plan(const PlanShape& shape, const HotPool& hot, int32_t batch,
               const int32_t* ids, const int32_t* indptr, int32_t backend,
               std::vector<uint8_t>& blob, Plan& plan, std::string& err) {
  const int32_t n_q = shape.n_q, n_kv = shape.n_kv, group = n_q / n_kv;
  plan = Plan();
  plan.backend = backend;
  plan.m_eff = batch * group;

  // ---- validation and class grouping (order of first appearance)
  std::vector<int32_t> class_ids;            // prefix id per class
  std::vector<int32_t> req_class(batch, -1);
  std::vector<int32_t> class_size;
  int32_t last_id = -1, last_cls = -1;
  if (indptr[0] < 0) {
    err = "cold_indptr[0] is negative";
    return -1;
  }
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
      continue;
    }
    int32_t c = -1;
    if (id == last_id) {
      c = last_cls;
    } else {
      for (size_t i = 0; i < class_ids.size(); ++i)
        if (class_ids[i] == id) { c = static_cast<int32_t>(i); break; }
      if (c < 0) {
        int64_t off;
        int32_t len;
        if (!hot.lookup(id, &off, &len)) {
          err = "hot prefix id " + std::to_string(id) + " is not live";
          return -1;
        }
        c = static_cast<int32_t>(class_ids.size());
        class_ids.push_back(id);
        class_size.push_back(0);
      }
      last_id = id;
      last_cls = c;
    }
    req_class[b] = c;
    class_size[c]++;
  }
  const int32_t n_classes = static_cast<int32_t>(class_ids.size());
  plan.n_classes = n_classes;

  // ---- classes, members and prefix splits
  std::vector<PrefixClass> classes(n_classes);
  std::vector<int32_t> members(batch);
  {
    int32_t off = 0;
    for (int32_t c = 0; c < n_classes; ++c) {
      int64_t slab_off;
      int32_t len;
      hot.lookup(class_ids[c], &slab_off, &len);
      classes[c].slab_off = slab_off;
      classes[c].len = len;
      classes[c].n_members = 0;
      classes[c].member_off = off;
      off += class_size[c];
    }
    for (int32_t b = 0; b < batch; ++b) {
      const int32_t c = req_class[b];
      if (c < 0) continue;
      members[classes[c].member_off + classes[c].n_members++] = b;
    }
  }
  const int32_t rb = backend == GKV_BACKEND_DENSE ? kDenseRB : kCascadeRB;
  const int32_t m_tile = 64 * rb;
  int64_t units = 0;
  for (int32_t c = 0; c < n_classes; ++c)
    units += static_cast<int64_t>(n_kv) * ceil_div(classes[c].n_members * group, m_tile) *
             classes[c].len;
  const int32_t target = backend == GKV_BACKEND_DENSE ? kDenseTargetBlocks : kCascadeTargetBlocks;
  const int64_t split_tokens =
      std::max<int64_t>(kMinSplitTokens, round_up(ceil_div(std::max<int64_t>(units, 1), target), kPrefixTile));
  for (int32_t c = 0; c < n_classes; ++c) {
    const int64_t len = classes[c].len;
    int64_t s = std::min<int64_t>(kMaxSplits, std::max<int64_t>(1, ceil_div(len, split_tokens)));
    const int64_t chunk = round_up(ceil_div(len, s), kPrefixTile);
    s = ceil_div(len, chunk);
    classes[c].n_splits = static_cast<int32_t>(s);
    classes[c].chunk = static_cast<int32_t>(chunk);
  }

  // ---- prefix items, XCD-aware: the M-tiles that share a (class, head,
  // split) K/V chunk go to the same XCD (block index congruent mod 8) and
  // are dispatched close together, so the chunk is read from HBM once and
  // served to the other tiles from that XCD's L2.
  std::vector<PrefixItem> items;
  {
    std::vector<std::vector<PrefixItem>> queue(kXcds);
    std::vector<int64_t> load(kXcds, 0);
    for (int32_t c = 0; c < n_classes; ++c) {
      const int32_t rows = classes[c].n_members * group;
      const int32_t mt = static_cast<int32_t>(ceil_div(rows, m_tile));
      for (int32_t g = 0; g < n_kv; ++g)
        for (int32_t s = 0; s < classes[c].n_splits; ++s) {
          const int x = static_cast<int>(std::min_element(load.begin(), load.end()) - load.begin());
          for (int32_t m = 0; m < mt; ++m) queue[x].push_back(PrefixItem{c, g, m * m_tile, s});
          load[x] += mt;
        }
    }
    size_t depth = 0;
    for (const auto& q : queue) depth = std::max(depth, q.size());
    items.assign(depth * kXcds, PrefixItem{-1, 0, 0, 0});
    for (int x = 0; x < kXcds; ++x)
      for (size_t i = 0; i < queue[x].size(); ++i) items[i * kXcds + x] = queue[x][i];
  }
  plan.n_prefix_items = static_cast<int32_t>(items.size());

  // ---- suffix parts
  int32_t chunk = 256;
  const int64_t w256 = suffix_waves(indptr, batch, n_kv, 256);
  if (w256 > 8 * kSuffixTargetWaves) {
    chunk = 512;
  } else {
    while (chunk > kMinSuffixChunk && suffix_waves(indptr, batch, n_kv, chunk) < kSuffixTargetWaves)
      chunk /= 2;
  }
  plan.suffix_chunk = chunk;
  std::vector<ReqInfo> reqs(batch);
  std::vector<SuffixItem> sitems;
  int32_t parts = 0;
  int64_t prefix_rows = 0;
  for (int32_t b = 0; b < batch; ++b) {
    ReqInfo& r = reqs[b];
    std::memset(&r, 0, sizeof(r));
    r.cls = req_class[b];
    if (r.cls >= 0) {
      r.n_splits = classes[r.cls].n_splits;
      r.prefix_base = static_cast<int32_t>(prefix_rows);
      prefix_rows += static_cast<int64_t>(r.n_splits) * n_q;
    }
    const int32_t t_begin = indptr[b], t_end = indptr[b + 1];
    r.chunk_base = parts;
    r.n_chunks = static_cast<int32_t>(ceil_div(t_end - t_begin, chunk));
    for (int32_t j = 0; j < r.n_chunks; ++j) {
      const int32_t t0 = t_begin + j * chunk;
      const int32_t t1 = std::min(t_end, t0 + chunk);
      for (int32_t g = 0; g < n_kv; ++g) {
        SuffixItem it;
        std::memset(&it, 0, sizeof(it));
        it.b = b;
        it.kv_head = g;
        it.t0 = t0;
        it.t1 = t1;
        it.part = parts + j;
        sitems.push_back(it);
      }
    }
    parts += r.n_chunks;
  }
  plan.n_suffix_items = static_cast<int32_t>(sitems.size());
  plan.n_chunks = parts;
  plan.prefix_rows = prefix_rows;
  plan.suffix_rows = static_cast<int64_t>(parts) * n_q;

  // ---- serialise
  size_t off = 0;
  plan.off_classes = off;
  off += align256(sizeof(PrefixClass) * classes.size());
  plan.off_members = off;
  off += align256(sizeof(int32_t) * members.size());
  plan.off_prefix = off;
  off += align256(sizeof(PrefixItem) * items.size());
  plan.off_suffix = off;
  off += align256(sizeof(SuffixItem) * sitems.size());
  plan.off_reqs = off;
  off += align256(sizeof(ReqInfo) * reqs.size());
  plan.blob_bytes = off;
  blob.resize(off);
  auto put = [&](size_t at, const void* src, size_t n) {
    if (n) std::memcpy(blob.data() + at, src, n);
  };
  put(plan.off_classes, classes.data(), sizeof(PrefixClass) * classes.size());
  put(plan.off_members, members.data(), sizeof(int32_t) * members.size());
  put(plan.off_prefix, items.data(), sizeof(PrefixItem) * items.size());
  put(plan.off_suffix, sitems.data(), sizeof(SuffixItem) * sitems.size());
  put(plan.off_reqs, reqs.data(), sizeof(ReqInfo) * reqs.size());
  return 0;
}

}  // namespace gkv
