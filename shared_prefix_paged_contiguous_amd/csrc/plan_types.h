// Work description of one decode step, shared by the host planner and the
// device kernels.  The whole description travels in the kernel arguments
// (about 24 KB, or 6 KB for a batch of at most 128), so a step needs no
// host-to-device copy before its kernels.
#pragma once

#include <cstddef>
#include <cstdint>

namespace gkv {

// Step kernel tiling.  A workgroup is 4 waves (one per SIMD); two
// workgroups share a CU, each with its own barriers, so one's MFMA and
// softmax work overlaps the other's waits.  In a prefix workgroup each wave
// owns RB blocks of 16 query rows (one MFMA column block each), so a
// workgroup tile covers 64*RB rows of one class and one KV head and every
// HOT block it streams through LDS feeds all of them.
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kPrefixTile = 64;
// Row blocks per wave of a prefix tile (RB): 2 (128-row tiles, each LDS read
// of a block feeds two row blocks) when some class has more than 64 rows
// per KV head and the dtype is bf16, else 1 (64-row tiles).
constexpr int kSmallTileRows = 64;
// Prefix workgroups a step aims for: the cascade backend (memory-bound
// regime) leaves half of the chip's workgroup slots to the suffix gather,
// which runs alongside; the dense backend (compute-bound regime) spreads
// the prefix GEMM over all of them.
constexpr int kCascadeTarget = 256;
constexpr int kDenseTarget = 512;
constexpr int kSuffixTile = 32;   // suffix kernel token tile (per wave)
constexpr int kWaveTokens = 1024; // most slot-table tokens one suffix wave covers (ids staged in LDS)
constexpr int kSuffixPart = kWaves * kWaveTokens;   // tokens per suffix workgroup
constexpr int kMaxSplits = 64;    // L splits per prefix class
constexpr int kHotBlock = 32;     // tokens per HOT block; slabs start on block boundaries
constexpr int kRingBytes = 64 * 1024;   // LDS ring of a prefix workgroup (K+V images of 3..8 blocks)
// Chip topology the planner works with (read from the device when a step is
// planned; these are the gfx950 values used when no device answers, so that
// host-side validation runs without a GPU).  Workgroups are dealt to the
// XCDs round-robin by index; each CU holds two step workgroups.
constexpr int kCusPerXcd = 32;          // gfx950: compute units per XCD
constexpr int kDefaultCus = 256;        // MI355X: 8 XCDs x 32 CUs
constexpr int kWgsPerCu = 2;            // resident step workgroups per CU

// Requests per prefix M-tile: a tile holds whole requests (all G query
// heads of a member for the tile's KV head), at most 64 * RB rows.
constexpr int tile_members(int group, int rb) { return kWaves * 16 * rb / group; }

// Limits of one step (the description must fit the kernel arguments).
constexpr int kMaxBatch = 1024;
constexpr int kMaxClasses = 64;

// One distinct HOT prefix in the step ("class": every request that starts
// with this slab).  Its prefix blocks are [block_base, block_base+n_blocks):
// local block i -> XCD slot x = i % X, r = i / X, M-tile r % m_tiles, group
// (r / m_tiles) * X + x (X = the device's XCDs), group = kv_head * n_splits
// + split.  The M-tiles of one group thus share an XCD (and its L2) and are
// dispatched together.
struct ClassDesc {
  int64_t slab_off;     // token offset of the slab in the HOT pool
  int32_t len;          // slab length L_c (tokens)
  int32_t n_members;    // requests of the class
  int32_t member_off;   // first entry in members[]
  int32_t n_splits;     // L splits S_c
  int32_t chunk;        // tokens per split (the last split may be shorter)
  int32_t m_tiles;      // ceil(n_members / tile_members(G, RB)): M-tiles hold whole requests
  int32_t n_groups;     // n_kv * n_splits
  int32_t block_base;   // first prefix block
  int32_t n_blocks;     // X * ceil(n_groups / X) * m_tiles
  int32_t pad_;
};

// Suffix work: one workgroup per (suffix part, KV head).  Requests are
// ranked longest slot table first (short requests last, see below); rank r
// owns parts [ranks[r].part0,
// ranks[r].part0 + n) with n = max(1, ceil(table length / kSuffixPart))
// (at least one, so every request gets a merge epilogue); part j covers its
// table positions [j * kSuffixPart, (j+1) * kSuffixPart) and the 4 waves
// take consecutive quarters of it.  Block i -> part i / n_kv, KV head
// i % n_kv.  A request with no HOT prefix and one part is finished in the
// suffix workgroup's epilogue.  Otherwise every prefix split writes a
// partial per (request, query head) and counts its arrival on the (request,
// KV head) counter.  When every slot table is one part (suffix_joins), the
// suffix workgroup that attended a request's part waits for that count and
// joins the prefix partials with its own result, kept in LDS, into the
// output.  Otherwise the suffix parts write partials and count arrivals too,
// and a join workgroup per (request, KV head), placed after all prefix and
// suffix work in the grid, waits for the count and joins the partials.
//
// Folding (cascade steps): when the parts' workgroups would not all fit in
// the workgroup slots the prefix leaves but half as many would, suffix block
// i runs two parts for its KV head, the short part n_parts-1-q first and then
// the long part q (q = i / n_kv).  Ranked longest first, the pairs carry
// about equal work, so all suffix work is resident from the start instead of
// a second round of short workgroups, each bound by its fixed round trips,
// running after the prefix ends; and each workgroup finishes on a long part,
// which keeps many loads in flight to the end.
//
// Short requests: a request with a HOT prefix whose slot table holds at
// most kInlineTokens tokens (one tile) gets no suffix part.  Ranked after all
// other requests, it has a join workgroup (its own, or shared with the next
// short requests when they outnumber the workgroup slots) that attends every
// KV head's slot-table tile itself (wave w takes KV heads w, w + 4, ...)
// into a partial row set of its own (rows after the suffix parts';
// ranks[r].part0 names it), waits once for the prefix splits of all its KV
// heads and joins them.  Steps whose requests carry a token or a few each
// (prefix-bound steps) thus launch one workgroup per request or fewer,
// instead of two per (request, KV head), and the tiles overlap the prefix
// when slots are free.
constexpr int kInlineTokens = 32;
//
// Grid: prefix blocks, then suffix blocks, then the joins: one per (ranked
// request, KV head) for the requests ranked before inline_rank0, shortest
// slot table first, then one per short request (or per short_per_block
// consecutive short requests, when there are more of them than workgroup
// slots).  Prefix and suffix blocks
// never wait, and every join block follows all of them in each XCD's
// (in-order) dispatch, so the joins' waits end.  The prefix and suffix
// ranges of the grid are padded to 4 * xcds blocks.
constexpr int kGroupPerXcd = 4;

// A ranked request's suffix work in one 16-byte record (one scalar load).
struct RankDesc {
  int32_t tok0, tok1;   // its slot-table range [tok0, tok1) in cold_indices
  int32_t part0;        // its first suffix part (short requests: its tile rows, >= n_parts)
  int32_t req;          // the request (batch index)
};

// The work description, in two parts: StepHead (sizes, pointers, classes)
// and the per-request tables sized for MB requests.  The kernel arguments
// carry the whole of it; a step of at most kSmallBatch requests is
// launched with the small form (about 6 KB instead of 24 KB), which takes
// less host time per launch and less time to reach the device.
struct StepHead {
  int32_t batch, n_q, n_kv, group, head_dim;
  float scale_log2;            // log2(e) / sqrt(head_dim)
  int32_t xcds;                // XCDs of the device (prefix blocks of one group share one)
  int32_t spin_limit;          // most polls of a join's wait before it gives up (and reports it)
  int32_t n_classes;
  int32_t rb;                  // row blocks per wave of the prefix tiles (1 or 2)
  int32_t prefix_blocks;       // sum of class n_blocks, padded to a multiple of 4 * xcds
  int32_t suffix_blocks;       // n_parts * n_kv (or folded pairs), padded to a multiple of 4 * xcds
  int32_t join_blocks;         // batch * n_kv when some output is joined, else 0
  int32_t max_splits;          // prefix partial row (b, s, h) = (b * max_splits + s) * n_q + h
  int32_t multi_part;          // some request has more than one suffix part
  int32_t n_parts;             // suffix parts of the step
  int32_t need_merge;          // some request is joined from several partials (HOT prefix or parts)
  int32_t narrow_ws;           // the step's workspace spans less than 2 GB (32-bit store offsets)
  int32_t fold;                // suffix block i runs parts n_parts-1-i/n_kv and i/n_kv (see above)
  int32_t partial_f32;         // partial rows are fp32 (else the input dtype)
  int32_t inline_rank0;        // ranks [inline_rank0, batch) are short requests (no suffix part)
  int32_t short_per_block;     // short requests per join workgroup (consecutive ranks)
  int32_t suffix_joins;        // every slot table is one part: suffix workgroups join their requests
  const void* q;
  void* out;
  float* lse;
  const void* k_hot;           // blocked HOT layout (see gkv_hot_write)
  const void* v_hot;
  int64_t hot_blocks;          // HOT blocks per KV head
  const void* k_cold;
  const void* v_cold;
  int32_t cold_cap;
  int32_t cold_mask;           // in-slot placement of KV-head rows: cold_row_pos
  const int32_t* cold_indices; // dev
  // fused decode step (null otherwise): request b's new token, the last
  // entry of its slot table, is read from k_new/v_new [B][n_kv][head_dim]
  // and copied into COLD slot new_slots[b] inside the launch
  const void* k_new;
  const void* v_new;
  const int32_t* new_slots;    // dev [B]
  void* p_o;                   // prefix partials [rows][head_dim], normalised (fp32 or the input dtype)
  float* p_lse;                // prefix partial log2-sum-exp2 of scaled scores
  void* s_o;                   // suffix-part partials, row = part * n_q + h (same dtype as p_o)
  float* s_lse;
  int32_t* counters;           // [kMaxBatch][n_kv] partial arrivals (zero between calls)
  int32_t* status;             // status word: joins that gave up waiting (gkv_step_status)
  uint64_t* trace;             // per-workgroup timeline records (kTraceWords each), null: off
  ClassDesc classes[kMaxClasses];
};

template <int MB>
struct StepArgsT : StepHead {
  alignas(16) RankDesc ranks[MB];   // by rank
  // small-int tables, 4-byte aligned so entries can be read with 32-bit loads
  alignas(4) int16_t rank_of[MB];   // rank of request b
  alignas(4) int16_t members[MB];   // requests grouped by class
  alignas(4) int8_t req_class[MB];  // class of request b, -1 = none
  // last word: the kernels do nothing unless it holds kArgsTail, so a work
  // description that did not arrive whole is never acted on
  int32_t tail;
};
constexpr int kSmallBatch = 128;
using StepArgs = StepArgsT<kMaxBatch>;
using StepArgsSmall = StepArgsT<kSmallBatch>;
constexpr int32_t kArgsTail = 0x47'4b'56'31;

// COLD in-slot layout: slot s holds the row of KV head g at position
// g ^ (s & mask), mask = (largest power of two dividing n_kv) - 1.  A KV
// head's rows thus sit at every position of their aligned group, not at one
// fixed offset: gathering 256-byte head rows that all lie 256 bytes past a
// 1 KB boundary ran measurably slower than the other offsets on gfx950, and
// with a fixed position every request's joins waited for those heads.
constexpr int32_t cold_mask_for(int32_t n_kv) { return (n_kv & -n_kv) - 1; }
// (constexpr functions serve host and device code alike)
constexpr int32_t cold_row_pos(int32_t g, int32_t slot, int32_t mask) { return g ^ (slot & mask); }

// Status word of a workspace (one 256-byte line after the counters): the
// number of joins that stopped waiting for their partials at the spin limit
// (their outputs are not valid).  Zero while every step is well formed.
constexpr int kDefaultSpinLimit = 1 << 16;

// Timeline record of one workgroup (gkv_step_trace), s_memrealtime ticks
// (100 MHz) unless noted: start; a mid-point mark (prefix: end of the block
// loop; suffix: end of the first part of a folded pair; join: end of its
// wait); end; (kind << 32) | the XCC id << 16 | the low 16 bits of HW_ID
// (wave, SIMD, CU, SH, SE); a second mark (prefix: its partial rows stored,
// before the arrivals; suffix with suffix joins: end of its tiles); a third
// mark (suffix with suffix joins: end of the wait for its requests' prefix
// splits); two unused words.  Marks a workgroup does not reach stay 0.
constexpr int kTraceWords = 8;
enum TraceWord : int {
  kTraceStart = 0, kTraceMark = 1, kTraceEnd = 2, kTraceKind = 3, kTraceMark2 = 4, kTraceMark3 = 5
};
enum TraceKind : uint32_t { kTracePrefix = 0, kTraceSuffix = 1, kTraceJoin = 2 };

// Static scratch of the allocation-free step, per device: a 256-byte status
// line, the join counters of up to kMaxBatch requests x 256 KV heads, then
// the step's partial results.
constexpr size_t kStaticScratchBytes = size_t{32} << 20;
constexpr size_t kStaticCounterOffset = 256;
constexpr size_t kStaticControlBytes = kStaticCounterOffset + size_t{kMaxBatch} * 256 * 4;
constexpr int kMaxDevices = 64;

}  // namespace gkv
