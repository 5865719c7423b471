#include "registry.h"

namespace gkv {

namespace {
constexpr int kHot = 0, kCold = 1;
}

Registry::Registry(HotPool& hot, ColdPool& cold)
    : hot_(hot), cold_(cold), cold_owned_(static_cast<size_t>(cold.capacity()), 0) {}

const PrefixEntry* Registry::find(uint64_t key) const {
  auto it = entries_.find(key);
  return it == entries_.end() ? nullptr : &it->second;
}

bool Registry::owns_cold_slot(int32_t slot) const {
  return slot >= 0 && static_cast<size_t>(slot) < cold_owned_.size() && cold_owned_[slot] != 0;
}

std::vector<uint64_t> Registry::cached(int32_t pool) const {
  std::vector<uint64_t> keys;
  keys.reserve(cached_[pool].size());
  for (const auto& kv : cached_[pool]) keys.push_back(kv.second);
  return keys;
}

int32_t Registry::cold_evictions_needed(int64_t n) const {
  int64_t free = cold_.free_count();
  int32_t j = 0;
  for (const auto& kv : cached_[kCold]) {
    if (free >= n) return j;
    free += entries_.at(kv.second).n;
    ++j;
  }
  return free >= n ? j : -1;
}

void Registry::drop(uint64_t key) {
  auto it = entries_.find(key);
  PrefixEntry& e = it->second;
  cached_[e.pool].erase(e.tick);
  if (e.pool == kHot) {
    hot_.release(e.hot_id);
    hot_owner_.erase(e.hot_id);
  } else {
    cold_.release(e.slots.data(), static_cast<int32_t>(e.slots.size()));
    for (int32_t s : e.slots) cold_owned_[s] = 0;
  }
  entries_.erase(it);
  ++stats_.evictions;
}

int Registry::acquire(uint64_t key, int32_t n, const PrefixEntry** entry, bool* fresh, std::string& err) {
  if (n < 1) {
    err = "prefix length must be >= 1";
    return -1;
  }
  auto it = entries_.find(key);
  if (it != entries_.end()) {
    PrefixEntry& e = it->second;
    if (e.n != n) {
      err = "prefix key is resident with " + std::to_string(e.n) + " tokens, not " + std::to_string(n);
      return -1;
    }
    if (e.refs == 0) cached_[e.pool].erase(e.tick);
    ++e.refs;
    ++stats_.hits;
    *entry = &e;
    *fresh = false;
    return 0;
  }
  PrefixEntry e;
  e.n = n;
  e.refs = 1;
  // HOT first, counting the slabs of cached HOT prefixes (eviction order)
  const std::vector<uint64_t> hot_cached = cached(kHot);
  std::vector<int32_t> ids;
  ids.reserve(hot_cached.size());
  for (uint64_t k : hot_cached) ids.push_back(entries_.at(k).hot_id);
  const int32_t jh = hot_.releases_to_fit(n, ids);
  if (jh >= 0) {
    for (int32_t j = 0; j < jh; ++j) drop(hot_cached[j]);
    int32_t id;
    int64_t off;
    if (hot_.alloc(n, &id, &off) != 0) {
      err = "internal: HOT admission found room that the allocator did not";
      return -1;
    }
    e.pool = kHot;
    e.hot_id = id;
    e.offset = off;
    hot_owner_.emplace(id, key);
    ++stats_.hot_admits;
  } else {
    const int32_t jc = cold_evictions_needed(n);
    if (jc < 0) {
      err = "no room for a prefix of " + std::to_string(n) + " tokens: no contiguous HOT extent and too few COLD slots";
      return -2;
    }
    const std::vector<uint64_t> cold_cached = cached(kCold);
    for (int32_t j = 0; j < jc; ++j) drop(cold_cached[j]);
    e.pool = kCold;
    e.slots.resize(n);
    if (cold_.alloc(n, e.slots.data()) != 0) {
      err = "internal: COLD admission found room that the allocator did not";
      return -1;
    }
    for (int32_t s : e.slots) cold_owned_[s] = 1;
    ++stats_.cold_admits;
  }
  auto ins = entries_.emplace(key, std::move(e)).first;
  *entry = &ins->second;
  *fresh = true;
  return 0;
}

int Registry::release(uint64_t key, std::string& err) {
  auto it = entries_.find(key);
  if (it == entries_.end()) {
    err = "prefix key is not resident";
    return -3;
  }
  PrefixEntry& e = it->second;
  if (e.refs == 0) {
    err = "prefix key holds no reference";
    return -1;
  }
  if (--e.refs == 0) {
    e.tick = ++clock_;
    cached_[e.pool].emplace(e.tick, key);
  }
  return 0;
}

int Registry::evict(uint64_t key, std::string& err) {
  auto it = entries_.find(key);
  if (it == entries_.end()) {
    err = "prefix key is not resident";
    return -3;
  }
  if (it->second.refs > 0) {
    err = "prefix key is referenced";
    return -1;
  }
  drop(key);
  return 0;
}

int Registry::reclaim_cold(int64_t n_free, std::string& err) {
  if (n_free < 0) {
    err = "n_free must be >= 0";
    return -1;
  }
  const int32_t jc = cold_evictions_needed(n_free);
  if (jc < 0) {
    err = "cannot free " + std::to_string(n_free) + " COLD slots";
    return -2;
  }
  const std::vector<uint64_t> cold_cached = cached(kCold);
  for (int32_t j = 0; j < jc; ++j) drop(cold_cached[j]);
  return 0;
}

RegistryCounts Registry::counts() const {
  RegistryCounts c = stats_;
  for (const auto& kv : entries_) {
    const PrefixEntry& e = kv.second;
    (e.pool == kHot ? c.resident_hot : c.resident_cold)++;
    (e.refs > 0 ? c.referenced : c.cached)++;
  }
  return c;
}

}  // namespace gkv
