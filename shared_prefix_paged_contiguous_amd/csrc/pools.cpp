#include "pools.h"

#include <algorithm>

namespace gkv {

HotPool::HotPool(int64_t capacity_tokens, int32_t block)
    : capacity_(capacity_tokens / block), block_(block) {
  if (capacity_ > 0) free_.emplace(0, capacity_);
}

int HotPool::alloc(int32_t n, int32_t* id, int64_t* offset) {
  const int64_t need = (static_cast<int64_t>(n) + block_ - 1) / block_;
  for (auto it = free_.begin(); it != free_.end(); ++it) {   // lowest address first
    if (it->second < need) continue;
    const int64_t off = it->first;
    const int64_t rest = it->second - need;
    free_.erase(it);
    if (rest > 0) free_.emplace(off + need, rest);
    int32_t pid;
    if (!released_ids_.empty()) {
      pid = *released_ids_.begin();
      released_ids_.erase(released_ids_.begin());
    } else {
      pid = next_id_++;
    }
    live_.emplace(pid, Slab{off, n});
    *id = pid;
    *offset = off * block_;
    return 0;
  }
  return -2;
}

int HotPool::release(int32_t id) {
  auto it = live_.find(id);
  if (it == live_.end()) return -3;
  int64_t off = it->second.offset;
  int64_t len = (static_cast<int64_t>(it->second.len) + block_ - 1) / block_;
  live_.erase(it);
  released_ids_.insert(id);
  // merge with the free extent that ends where this one starts
  auto next = free_.lower_bound(off);
  if (next != free_.begin()) {
    auto prev = std::prev(next);
    if (prev->first + prev->second == off) {
      off = prev->first;
      len += prev->second;
      free_.erase(prev);
    }
  }
  // ... and with the one that starts where it ends
  next = free_.find(off + len);
  if (next != free_.end()) {
    len += next->second;
    free_.erase(next);
  }
  free_.emplace(off, len);
  return 0;
}

bool HotPool::lookup(int32_t id, int64_t* offset, int32_t* len) const {
  auto it = live_.find(id);
  if (it == live_.end()) return false;
  *offset = it->second.offset * block_;
  *len = it->second.len;
  return true;
}

int32_t HotPool::releases_to_fit(int32_t n, const std::vector<int32_t>& ids) const {
  const int64_t need = (static_cast<int64_t>(n) + block_ - 1) / block_;
  std::map<int64_t, int64_t> trial = free_;
  int64_t longest = 0;
  for (const auto& e : trial) longest = std::max(longest, e.second);
  for (size_t j = 0;; ++j) {
    if (longest >= need) return static_cast<int32_t>(j);
    if (j == ids.size()) return -1;
    auto it = live_.find(ids[j]);
    if (it == live_.end()) return -1;
    int64_t off = it->second.offset;
    int64_t len = (static_cast<int64_t>(it->second.len) + block_ - 1) / block_;
    auto next = trial.lower_bound(off);
    if (next != trial.begin()) {
      auto prev = std::prev(next);
      if (prev->first + prev->second == off) {
        off = prev->first;
        len += prev->second;
        trial.erase(prev);
      }
    }
    next = trial.find(off + len);
    if (next != trial.end()) {
      len += next->second;
      trial.erase(next);
    }
    trial.emplace(off, len);
    longest = std::max(longest, len);
  }
}

int64_t HotPool::free_tokens() const {
  int64_t t = 0;
  for (const auto& e : free_) t += e.second;
  return t * block_;
}

int64_t HotPool::largest_hole() const {
  int64_t m = 0;
  for (const auto& e : free_) m = std::max(m, e.second);
  return m * block_;
}

ColdPool::ColdPool(int32_t capacity)
    : capacity_(capacity), allocated_(capacity, 0), mark_(capacity, 0) {
  stack_.reserve(capacity);
  for (int32_t s = capacity - 1; s >= 0; --s) stack_.push_back(s);
}

int ColdPool::alloc(int32_t n, int32_t* out) {
  if (static_cast<int64_t>(n) > static_cast<int64_t>(stack_.size())) return -2;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t s = stack_.back();
    stack_.pop_back();
    allocated_[s] = 1;
    out[i] = s;
  }
  return 0;
}

int ColdPool::release(const int32_t* slots, int32_t n) {
  if (++stamp_ == 0) {   // stamp wrapped: clear the marks once
    std::fill(mark_.begin(), mark_.end(), 0u);
    stamp_ = 1;
  }
  for (int32_t i = 0; i < n; ++i) {
    const int32_t s = slots[i];
    if (s < 0 || s >= capacity_ || !allocated_[s] || mark_[s] == stamp_) return -3;
    mark_[s] = stamp_;
  }
  for (int32_t i = 0; i < n; ++i) {
    allocated_[slots[i]] = 0;
    stack_.push_back(slots[i]);
  }
  return 0;
}

}  // namespace gkv
