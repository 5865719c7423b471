// Shared-prefix registry: reference counts and the admission policy of the
// two pools.  Pure C++ (no HIP).
//
// paperlayer.ai Appendix B.10 "Cross-pool admission and promotion policy":
// a prefix is admitted to the contiguous HOT pool first and goes to COLD
// when no contiguous HOT extent fits it (full pool or too-short fragments);
// prefixes in HOT are never demoted.  paperlayer.ai §1 "Design": admission
// and eviction belong to the engine; Appendix B.8: every distinct prefix is
// tagged and gets a slab of its own.
//
// Readings where the pages are silent: prefixes are identified by a caller
// key and reference-counted.  A prefix whose count reaches zero stays
// resident (cached) and may be evicted, least recently released first, when
// an admission needs its space or on request.  HOT capacity for an admission
// includes the slabs of cached HOT prefixes: the fewest of them, in eviction
// order, that make a contiguous extent appear are evicted and the prefix
// goes to HOT; else COLD, likewise with cached COLD prefixes; else the call
// fails with nothing changed.  Referenced prefixes never move.
#pragma once

#include <cstdint>
#include <map>
#include <string>
#include <unordered_map>
#include <vector>

#include "pools.h"

namespace gkv {

struct PrefixEntry {
  int32_t pool = 0;        // 0 HOT, 1 COLD
  int32_t n = 0;           // tokens
  int32_t refs = 0;
  int32_t hot_id = -1;     // HOT: the slab's prefix id
  int64_t offset = -1;     // HOT: token offset of the slab
  std::vector<int32_t> slots;   // COLD: slots in context order
  uint64_t tick = 0;       // release stamp while cached
};

struct RegistryCounts {
  int32_t resident_hot = 0, resident_cold = 0, referenced = 0, cached = 0;
  int64_t hits = 0, hot_admits = 0, cold_admits = 0, evictions = 0;
};

class Registry {
 public:
  Registry(HotPool& hot, ColdPool& cold);

  // Status codes of include/gkv.h (0, -1 invalid, -2 no space, -3 not found).
  int acquire(uint64_t key, int32_t n, const PrefixEntry** entry, bool* fresh, std::string& err);
  int release(uint64_t key, std::string& err);
  int evict(uint64_t key, std::string& err);
  int reclaim_cold(int64_t n_free, std::string& err);

  const PrefixEntry* find(uint64_t key) const;
  bool owns_hot(int32_t prefix_id) const { return hot_owner_.count(prefix_id) != 0; }
  bool owns_cold_slot(int32_t slot) const;
  RegistryCounts counts() const;

 private:
  void drop(uint64_t key);
  // cached prefixes of one pool, eviction order
  std::vector<uint64_t> cached(int32_t pool) const;
  int32_t cold_evictions_needed(int64_t n) const;   // -1 if impossible

  HotPool& hot_;
  ColdPool& cold_;
  std::unordered_map<uint64_t, PrefixEntry> entries_;
  std::map<uint64_t, uint64_t> cached_[2];   // per pool: release stamp -> key
  std::unordered_map<int32_t, uint64_t> hot_owner_;
  std::vector<uint8_t> cold_owned_;
  uint64_t clock_ = 0;
  RegistryCounts stats_;
};

}  // namespace gkv
