// Host-side bookkeeping of the two KV pools.  Pure C++ (no HIP): it builds
// and runs without a GPU.
//
// HOT pool: paperlayer.ai summary of the GraniKV paper, §3 "Asymmetric
// KV-cache paging" (contiguous shared-prefix storage); reading card "Key
// ideas" (one bump-pointer slab per prefix node); Appendix B.8 (first-fit
// packing of mixed slab sizes); Appendix B.10 (admission fails when no
// contiguous extent fits, even if the free total would; live slabs are never
// demoted).  Free space is a set of address-ordered extents; the last one is
// the bump region.  Allocation takes the lowest-address extent that fits and
// carves from its start; freeing merges with free neighbours.  Space is
// counted in blocks of `block` tokens (the attention kernels' K/V block): a
// prefix of n tokens takes ceil(n / block) blocks and starts on a block
// boundary; a pool of C tokens holds floor(C / block) blocks.
//
// COLD pool: paperlayer.ai §3 (page size one token); reading card (token-level
// free list).  A LIFO stack of free slots; a fresh pool hands out 0, 1, 2, ...
#pragma once

#include <cstdint>
#include <map>
#include <set>
#include <vector>

namespace gkv {

struct HotPool {
  HotPool(int64_t capacity_tokens, int32_t block);

  // 0 on success; -2 when no extent of n tokens exists (state unchanged).
  int alloc(int32_t n, int32_t* id, int64_t* offset);
  // 0 on success; -3 when id is not live.
  int release(int32_t id);
  bool lookup(int32_t id, int64_t* offset, int32_t* len) const;
  // Fewest slabs of `ids`, taken in that order, whose release would leave a
  // free extent for n tokens (0 if one exists now); -1 if releasing all of
  // them would not.  Nothing changes.
  int32_t releases_to_fit(int32_t n, const std::vector<int32_t>& ids) const;

  int64_t capacity_blocks() const { return capacity_; }
  int64_t free_tokens() const;      // free blocks x block
  int64_t largest_hole() const;     // tokens of the longest free extent
  int32_t live_count() const { return static_cast<int32_t>(live_.size()); }
  int32_t extent_count() const { return static_cast<int32_t>(free_.size()); }

 private:
  struct Slab {
    int64_t offset;
    int32_t len;
  };
  int64_t capacity_;                  // in blocks
  int32_t block_;
  std::map<int64_t, int64_t> free_;   // block offset -> blocks, address order
  std::map<int32_t, Slab> live_;      // id -> slab (block offset, tokens)
  std::set<int32_t> released_ids_;    // ids below next_id_ that are free again
  int32_t next_id_ = 0;
};

struct ColdPool {
  explicit ColdPool(int32_t capacity);

  // All or nothing; -2 when fewer than n slots are free.
  int alloc(int32_t n, int32_t* out);
  // -3 (nothing changed) if a slot is out of range, not allocated or repeated.
  int release(const int32_t* slots, int32_t n);

  int32_t capacity() const { return capacity_; }
  int64_t free_count() const { return static_cast<int64_t>(stack_.size()); }

 private:
  int32_t capacity_;
  std::vector<int32_t> stack_;        // back() is the next slot handed out
  std::vector<uint8_t> allocated_;    // per slot: 1 while handed out
  std::vector<uint32_t> mark_;        // per slot: call stamp for duplicate checks
  uint32_t stamp_ = 0;
};

}  // namespace gkv
