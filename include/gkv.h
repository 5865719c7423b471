/*
 * gkv.h - C ABI of libgkv: shared-prefix decode attention over a contiguous
 * HOT prefix pool and a token-level COLD suffix pool, for AMD Instinct
 * MI355X (gfx950).
 *
 * The operations follow the GraniKV pages ("GraniKV: Asymmetric Granularity
 * KV-Cache Paging for Multi-Agent Systems with Long Shared Prefix"):
 *   - paperlayer.ai summary §3 "Asymmetric KV-cache paging": shared prefixes
 *     live contiguously in a HOT pool, suffix and decoded tokens one token per
 *     slot in a COLD pool;
 *   - reading card (observer.broadside.tech) "Key ideas": one bump-pointer
 *     slab per prefix node in HOT, a token-level free list in COLD;
 *   - paperlayer.ai Appendix B.8 (first-fit packing of mixed slab sizes) and
 *     B.10 (HOT-first admission, failure when no contiguous extent fits, no
 *     demotion);
 *   - paperlayer.ai §2 "Prefix-suffix attention": prefix attention and suffix
 *     attention are computed apart and joined by log-sum-exp;
 *   - paperlayer.ai §3 "Per-step dispatch" and Appendix B.4: each step picks
 *     the dense (batched GEMM) or the cascade prefix backend from
 *     M_eff = B * n_q / n_kv against a measured threshold M_sat.
 *
 * Conventions
 *   - Every function returns a gkv_status (0 = success) except gkv_destroy and
 *     gkv_last_error.  No C++ exception crosses this boundary.  On failure the
 *     context keeps a message readable with gkv_last_error.
 *   - Device memory is owned by the caller (allocated by any means, e.g.
 *     torch); the library never frees it.  "dev" marks device pointers,
 *     "host" host pointers.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Device calls enqueue work and return without synchronising.
 *   - Pool bookkeeping calls are host-only and synchronous.  A context is not
 *     thread-safe; callers serialise calls on one context.  Device calls that
 *     share a context's workspace must be issued on one stream (or otherwise
 *     ordered): each call reuses the workspace, and the workgroups of one
 *     call coordinate through counters kept in it.
 *   - Element types: GKV_F32 (float) or GKV_BF16 (bfloat16, round to nearest
 *     even on output).  All arithmetic accumulates in fp32.
 *   - Device: the kernels are built for gfx950 (CDNA4) only.  The first
 *     device call of a context reads the current device's compute units
 *     (and from them its XCDs, 32 compute units each) and refuses any other
 *     architecture with GKV_ERR_DEVICE; a context then stays on that device.
 */
#ifndef GKV_H
#define GKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GKV_OK = 0,
  GKV_ERR_INVALID = -1,   /* bad argument, shape, id or state */
  GKV_ERR_NOSPACE = -2,   /* pool has no room; nothing changed */
  GKV_ERR_NOTFOUND = -3,  /* unknown prefix id or unallocated slot; nothing changed */
  GKV_ERR_DEVICE = -4     /* a HIP call failed (message names it) */
} gkv_status;

enum { GKV_F32 = 0, GKV_BF16 = 1 };

/* Element type of the partial results a step keeps in its workspace (prefix
 * splits, suffix parts) before their log-sum-exp join. */
enum {
  GKV_PARTIALS_INPUT = 0,   /* the input dtype (bf16 inputs: bf16 partials) */
  GKV_PARTIALS_F32 = 1      /* fp32 */
};

enum {
  GKV_BACKEND_AUTO = 0,     /* per step: dense iff M_eff >= m_sat */
  GKV_BACKEND_CASCADE = 1,  /* split-K prefix kernel reading each slab once */
  GKV_BACKEND_DENSE = 2     /* M-tiled batched-GEMM prefix kernel (bf16 only) */
};

typedef struct {
  int32_t n_q_heads;             /* query heads (<= 256); a multiple of n_kv_heads */
  int32_t n_kv_heads;            /* KV heads; n_q/n_kv (the group G) in 1..16 */
  int32_t head_dim;              /* 64 or 128 */
  int32_t dtype;                 /* GKV_F32 or GKV_BF16: q, K, V and out */
  int32_t n_layers;              /* number of bindable layers, >= 1 */
  int64_t hot_capacity_tokens;   /* C_hot >= 0 */
  int64_t cold_capacity_tokens;  /* C_cold >= 0, < 2^31 */
  int32_t m_sat;                 /* dense threshold on M_eff; <= 0 = library default */
  int32_t force_backend;         /* GKV_BACKEND_*; AUTO for the per-step rule */
  int32_t partials;              /* GKV_PARTIALS_INPUT (default) or GKV_PARTIALS_F32 */
} gkv_config;

typedef struct {
  int64_t hot_free_tokens;     /* sum of free HOT extents (whole blocks) */
  int64_t hot_largest_hole;    /* longest free HOT extent, tokens */
  int32_t hot_live_prefixes;   /* live HOT slabs */
  int32_t hot_free_extents;    /* number of free HOT extents */
  int64_t cold_free_slots;     /* free COLD slots */
} gkv_stats;

typedef struct gkv_ctx gkv_ctx;

/* Library default for m_sat (4096), fit on MI355X over full decode steps:
 * cascade was at least as fast as dense for every M_eff up to 3840. */
int32_t gkv_default_m_sat(void);

/* Create a context.  Validates the config (GKV_ERR_INVALID otherwise; *out is
 * set to NULL).  Makes no HIP call: pool bookkeeping works without a GPU. */
int gkv_create(const gkv_config* cfg, gkv_ctx** out);
void gkv_destroy(gkv_ctx* ctx);
/* Last error message of this context ("" if none).  Valid until the next call. */
const char* gkv_last_error(const gkv_ctx* ctx);

/* Pools of one layer, all dev, element type cfg.dtype, 16-byte aligned:
 *   k_hot, v_hot   gkv_hot_pool_bytes() bytes each, in the library's blocked
 *                  layout: per KV head, C_hot / 32 blocks of 32 tokens, each
 *                  block stored as the register image of the attention
 *                  kernels' matrix-core operands (V transposed per lane).
 *                  Head-major, so one (head, prefix) slab is one linear run
 *                  of whole blocks.  Write rows with gkv_hot_write.
 *   k_cold, v_cold [C_cold][n_kv][head_dim]  token-major: one slot holds one
 *                  token of every KV head, the row of head g at position
 *                  g ^ (slot & m), m = (largest power of two dividing n_kv)
 *                  - 1 (heads permuted within aligned groups of m + 1, so a
 *                  head's rows are spread over the in-slot offsets); written
 *                  with gkv_cold_append.  Odd n_kv: position g.
 * Prefix ids, HOT offsets and COLD slots are shared by all layers.  NULL is
 * allowed for a pool that holds no block / slot. */
int gkv_bind_layer(gkv_ctx* ctx, int32_t layer, void* k_hot, void* v_hot,
                   void* k_cold, void* v_cold);

/* Workspace bytes needed by gkv_attn_decode for steps of at most max_batch
 * requests and at most max_suffix_tokens slot-table entries in total. */
int gkv_workspace_size(const gkv_ctx* ctx, int32_t max_batch, int64_t max_suffix_tokens,
                       size_t* bytes);
/* Bind caller-owned device workspace (dev, >= 256-byte aligned).  Host-only:
 * the first gkv_attn_decode after a bind also enqueues, on its stream, a
 * small kernel that zeroes the workspace's counter area (partial-join
 * counters of the step kernel); later calls leave it consistent. */
int gkv_bind_workspace(gkv_ctx* ctx, void* dev, size_t bytes);

/* Bytes of one HOT pool buffer (k_hot or v_hot) of one layer. */
int gkv_hot_pool_bytes(const gkv_ctx* ctx, size_t* bytes);

/* Write rows [token_begin, token_begin + n) of a live slab (the caller's
 * prefill of a shared prefix).  k_rows, v_rows: dev [n][n_kv][head_dim].
 * GKV_ERR_NOTFOUND for a dead id, GKV_ERR_INVALID for rows outside the slab.
 * Asynchronous on `stream`; byte copies into the blocked layout. */
int gkv_hot_write(gkv_ctx* ctx, int32_t layer, int32_t prefix_id, int32_t token_begin, int32_t n,
                  const void* k_rows, const void* v_rows, void* stream);

/* HOT pool (paperlayer.ai §3, reading card "Key ideas", Appendix B.8/B.10).
 * Space is counted in blocks of 32 tokens (the kernels' K/V block): a slab
 * of n tokens takes ceil(n/32) blocks and starts on a block boundary.
 * First fit over address-ordered free extents; the slab is carved from the
 * start of the lowest-address extent that fits.  Returns the new
 * prefix id (smallest unused non-negative integer) and the slab's token
 * offset.  GKV_ERR_NOSPACE when no single free extent fits - also when the
 * total free space would - with no change to the pool and no demotion of
 * live slabs; the caller then places the prefix in COLD. */
int gkv_hot_pool_alloc(gkv_ctx* ctx, int32_t n_tokens, int32_t* prefix_id,
                       int64_t* token_offset);
/* Return a slab; it merges with free neighbours.  GKV_ERR_NOTFOUND for an
 * unknown or already-freed id. */
int gkv_hot_pool_free(gkv_ctx* ctx, int32_t prefix_id);
/* Offset and length of a live slab (GKV_ERR_NOTFOUND otherwise). */
int gkv_hot_prefix_info(const gkv_ctx* ctx, int32_t prefix_id, int64_t* token_offset,
                        int32_t* n_tokens);

/* COLD pool (paperlayer.ai §3: page size one token; reading card: token-level
 * free list).  LIFO free list: a fresh pool hands out 0, 1, 2, ...; alloc pops
 * n slots into slots_out (host, n entries) in pop order, all or nothing
 * (GKV_ERR_NOSPACE when fewer than n are free, nothing changed). */
int gkv_cold_pool_alloc(gkv_ctx* ctx, int32_t n, int32_t* slots_out);
/* Push slots (host) back in the order given; the last one becomes the next
 * handed out.  GKV_ERR_NOTFOUND, with nothing changed, if any slot is out of
 * range, not allocated, or repeated in the call. */
int gkv_cold_pool_free(gkv_ctx* ctx, const int32_t* slots, int32_t n);

int gkv_pool_stats(const gkv_ctx* ctx, gkv_stats* out);

/* ---------------------------------------------------------------- prefixes
 * Shared-prefix registry: reference-counted prefixes and the admission policy
 * of the two pools (paperlayer.ai Appendix B.10 "Cross-pool admission and
 * promotion policy": HOT first, COLD when no contiguous HOT extent fits the
 * prefix - a full pool or only shorter fragments - and prefixes in HOT are
 * never demoted; Appendix B.8: every distinct prefix gets a slab of its own;
 * §1 "Design": admission and eviction are part of the engine).
 *
 * A prefix is named by a caller key (e.g. a hash of its tokens).  A prefix
 * whose last reference is released stays resident as a cached prefix; cached
 * prefixes are evicted least recently released first, only when an admission
 * needs their space or on request.  Evicting frees a prefix's slab or slots;
 * referenced prefixes never move or change pool.  Host-only calls, no GPU.
 * Slabs and slots owned by the registry are refused by gkv_hot_pool_free and
 * gkv_cold_pool_free (GKV_ERR_INVALID). */

/* HOT and COLD token capacities for a KV budget of total_tokens tokens per
 * layer, the HOT pool taking the fraction f_p, fixed at start-up (paperlayer.ai
 * "Limitations": static HOT/COLD pool fraction, 0.2 by default), rounded down
 * to whole 32-token blocks: hot = floor(floor(f_p * total) / 32) * 32, cold =
 * total - hot.  GKV_ERR_INVALID if total < 0, f_p is outside [0, 1] or cold
 * exceeds 2^31 - 1 slots.  Needs no context. */
int gkv_partition_capacity(int64_t total_tokens, double f_p, int64_t* hot_tokens,
                           int64_t* cold_tokens);

enum { GKV_POOL_HOT = 0, GKV_POOL_COLD = 1 };

typedef struct {
  int32_t pool;         /* GKV_POOL_HOT or GKV_POOL_COLD */
  int32_t prefix_id;    /* HOT: the slab's prefix id (for hot_prefix_ids); COLD: -1 */
  int64_t hot_offset;   /* HOT: token offset of the slab; COLD: -1 */
  int32_t n_tokens;     /* prefix length */
  int32_t fresh;        /* 1 if this call admitted the prefix: the caller writes its
                           K/V (gkv_hot_write, or gkv_cold_append on its slots) */
  int32_t refs;         /* references held after the call */
  int32_t reserved;
} gkv_prefix_ref;

/* Take a reference to prefix `key` of n_tokens tokens.  If it is resident the
 * reference count grows and its placement is returned (fresh = 0; n_tokens
 * must equal its length, else GKV_ERR_INVALID).  Otherwise it is admitted:
 *   1. HOT, if a free extent fits it, or if evicting cached HOT prefixes in
 *      eviction order makes one appear (the fewest such are evicted); the
 *      slab is placed first-fit as by gkv_hot_pool_alloc;
 *   2. else COLD, if the free slots - plus those of cached COLD prefixes,
 *      evicted in order as needed - number n_tokens; popped as by
 *      gkv_cold_pool_alloc (read them with gkv_prefix_cold_slots);
 *   3. else GKV_ERR_NOSPACE with nothing changed (no eviction).
 * out: host, written on success. */
int gkv_prefix_acquire(gkv_ctx* ctx, uint64_t key, int32_t n_tokens, gkv_prefix_ref* out);
/* Placement of a resident prefix without changing its count (fresh = 0);
 * GKV_ERR_NOTFOUND if not resident. */
int gkv_prefix_lookup(const gkv_ctx* ctx, uint64_t key, gkv_prefix_ref* out);
/* The COLD slots (host, >= n_tokens entries) of a COLD-resident prefix, in
 * context order.  GKV_ERR_NOTFOUND if not resident, GKV_ERR_INVALID if it is
 * in HOT or max_slots < n_tokens. */
int gkv_prefix_cold_slots(const gkv_ctx* ctx, uint64_t key, int32_t* slots_out, int32_t max_slots);
/* Drop one reference; at zero the prefix is cached (still resident).
 * GKV_ERR_NOTFOUND if not resident, GKV_ERR_INVALID if it holds no reference. */
int gkv_prefix_release(gkv_ctx* ctx, uint64_t key);
/* Evict a cached prefix now.  GKV_ERR_NOTFOUND if not resident,
 * GKV_ERR_INVALID if it is referenced. */
int gkv_prefix_evict(gkv_ctx* ctx, uint64_t key);
/* Evict cached COLD prefixes, in eviction order, until at least n_free_slots
 * COLD slots are free (e.g. before allocating a batch's suffix slots).
 * GKV_ERR_NOSPACE with nothing changed if even all of them would not do. */
int gkv_prefix_reclaim_cold(gkv_ctx* ctx, int32_t n_free_slots);

typedef struct {
  int32_t resident_hot;    /* resident prefixes in HOT */
  int32_t resident_cold;   /* resident prefixes in COLD */
  int32_t referenced;      /* resident with refs > 0 */
  int32_t cached;          /* resident with refs == 0 */
  int64_t hits;            /* acquires of a resident prefix, since create */
  int64_t hot_admits;      /* admissions to HOT */
  int64_t cold_admits;     /* admissions to COLD (HOT could not hold the prefix) */
  int64_t evictions;       /* cached prefixes evicted */
} gkv_registry_counts;
int gkv_registry_stats(const gkv_ctx* ctx, gkv_registry_counts* out);

/* Append decoded tokens into COLD (paperlayer.ai §1 "Design": COLD holds
 * suffix and decoded tokens).  k_new, v_new: dev [n][n_kv][head_dim];
 * slots_dev: dev int32 [n].  Slot slots[i] of layer `layer`'s k_cold/v_cold
 * becomes a byte copy of row i, its KV heads at their in-slot positions
 * (gkv_bind_layer); other slots are untouched.  Slots outside
 * [0, C_cold) are skipped on the device (the host cannot read them); repeated
 * slots in one call leave one of the rows, unspecified which.  Asynchronous
 * on `stream`. */
int gkv_cold_append(gkv_ctx* ctx, int32_t layer, const void* k_new, const void* v_new,
                    const int32_t* slots_dev, int32_t n, void* stream);

/* One decode step of one layer (paperlayer.ai §2 "Prefix-suffix attention",
 * §3 "Dual attention backends", §3 "Per-step dispatch").
 *   q              dev  [B][n_q][head_dim], cfg.dtype
 *   hot_prefix_ids host [B]: live prefix id whose HOT slab starts request b's
 *                  context, or -1 for none (paged fallback: the whole
 *                  context is in the slot table)
 *   cold_indptr_h  host [B+1]: CSR row pointers (non-decreasing); request
 *                  b's slot table is cold_indices_d[indptr[b] .. indptr[b+1]).
 *                  The kernels receive this host copy in their arguments.
 *   cold_indptr_d  dev [B+1], nullable: a device copy of the same pointers,
 *                  kept for callers that hold one; not read
 *   cold_indices_d dev int32: COLD slots in context order (the current token
 *                  last).  Slots outside [0, C_cold) are clamped on the device.
 *   out            dev  [B][n_q][head_dim], cfg.dtype
 *   lse            dev  float [B][n_q]: natural log of the softmax
 *                  denominator over the whole context (scores scaled by
 *                  1/sqrt(head_dim))
 *   backend_out    host, nullable: the prefix backend used this step
 * Context of request b = its HOT slab's tokens, then its slot-table tokens.
 * Query head h attends KV head h / (n_q / n_kv).  GKV_ERR_INVALID (nothing
 * enqueued, nothing written) if B < 1, a request has neither a prefix nor a
 * suffix, an id is not live, indptr decreases, the layer is not bound, the
 * workspace is missing or too small, or cfg.force_backend/override is DENSE
 * with dtype F32.  Asynchronous on `stream`. */
int gkv_attn_decode(gkv_ctx* ctx, int32_t layer, const void* q, int32_t batch,
                    const int32_t* hot_prefix_ids, const int32_t* cold_indptr_h,
                    const int32_t* cold_indptr_d, const int32_t* cold_indices_d,
                    void* out, float* lse, void* stream, int32_t* backend_out);

/* One whole decode step in one launch: the batch's new tokens are appended to
 * COLD and every request attends its context including its new token
 * (paperlayer.ai §1 "Design": decoded tokens go to COLD; §2 "Prefix-suffix
 * attention").  Same result as gkv_cold_append(ctx, layer, k_new, v_new,
 * new_slots_d, B, stream) followed by gkv_attn_decode(...) with the same
 * other arguments, provided that for every request b new_slots_d[b] is the
 * last entry of b's slot table (its decode token); otherwise the result is
 * unspecified.
 *   k_new, v_new  dev [B][n_kv][head_dim], cfg.dtype, 16-byte aligned: the
 *                 new token of request b
 *   new_slots_d   dev int32 [B]; slots outside [0, C_cold) are not written
 *   other arguments as gkv_attn_decode (cold_indices_d already holds the
 *   new slots at the ends of the tables)
 * Inside the launch the new token's K/V are read from k_new/v_new, so no part
 * of the step waits for the append, and the workgroups that attend it copy it
 * into its slot.  Errors as gkv_attn_decode, and GKV_ERR_INVALID (nothing
 * enqueued) if a pointer is null or misaligned or a request's slot table is
 * empty.  Asynchronous on `stream`; the plan diagnostics and kernel timing
 * are those of gkv_attn_decode. */
int gkv_decode_step(gkv_ctx* ctx, int32_t layer, const void* q, const void* k_new, const void* v_new,
                    const int32_t* new_slots_d, int32_t batch, const int32_t* hot_prefix_ids,
                    const int32_t* cold_indptr_h, const int32_t* cold_indices_d, void* out, float* lse,
                    void* stream, int32_t* backend_out);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * step as gkv_decode_step, with the same arguments and result, whose scratch
 * (join counters, status word, partial results) lives in a static device
 * array of the library - 32 MiB on every device the library runs on, held
 * until the process ends - instead of the context's bound workspace, so no
 * workspace needs to be bound.  Allocates nothing: no hipMalloc, hipFree or
 * allocating library call.  The first call on a device clears the array's
 * counters and status word with a small fill kernel on `stream`; every call
 * leaves the counters at zero again.  GKV_ERR_INVALID (nothing enqueued) if
 * the step's partial results do not fit the array, besides the errors of
 * gkv_decode_step.  All calls on one device share its array, whatever their
 * context: calls that overlap in time on one device (other streams, other
 * threads) race on it and give undefined results; issue them on one stream.
 * gkv_step_status also reports joins of these calls that gave up waiting,
 * from the current device's array. */
int gkv_decode_step_static(gkv_ctx* ctx, int32_t layer, const void* q, const void* k_new, const void* v_new,
                           const int32_t* new_slots_d, int32_t batch, const int32_t* hot_prefix_ids,
                           const int32_t* cold_indptr_h, const int32_t* cold_indices_d, void* out, float* lse,
                           void* stream, int32_t* backend_out);

/* Per-step rule alone (host, no GPU): backend for a batch of `batch` requests
 * under the context's threshold and override (paperlayer.ai §3 "Per-step
 * dispatch": dense iff M_eff = B * n_q/n_kv >= M_sat). */
int gkv_select_backend(const gkv_ctx* ctx, int32_t batch, int32_t* backend);
/* Change the backend override (GKV_BACKEND_*) and/or threshold (> 0) of a
 * context; m_sat <= 0 keeps the current threshold. */
int gkv_set_dispatch(gkv_ctx* ctx, int32_t force_backend, int32_t m_sat);

/* What the last successful gkv_attn_decode of this context planned (host
 * diagnostics: no GPU needed to read it). */
typedef struct {
  int32_t backend;            /* GKV_BACKEND_CASCADE or GKV_BACKEND_DENSE */
  int32_t m_eff;              /* B * n_q / n_kv of the step */
  int32_t n_classes;          /* distinct HOT prefixes in the step */
  int32_t n_prefix_blocks;    /* prefix workgroups launched (incl. idle padding) */
  int32_t n_suffix_blocks;    /* suffix workgroups (parts x KV-head groups) */
  int32_t n_suffix_parts;     /* slot-table parts (>= one per request, short requests aside) */
  int32_t joins_partials;     /* 1 if some output is joined from several partials (a HOT
                                 prefix or a multi-part slot table), inside the step kernel */
  int32_t suffix_part_tokens; /* slot-table tokens per suffix part this step */
  int32_t folded_parts;       /* 1 if each suffix workgroup ran two parts (a short one, then a
                                 long one): chosen for cascade steps whose parts' workgroups
                                 overflow the workgroup slots beside the prefix while half as
                                 many fit */
  int32_t n_join_blocks;      /* join workgroups (when some output is joined from several
                                 partials: one per request and KV head when some slot table
                                 spans several suffix parts, none for the others when every
                                 table is one part (the suffix workgroups then join their
                                 requests themselves); one per short request, or per k
                                 consecutive short requests when they outnumber the
                                 workgroup slots; else 0) */
  int32_t n_short_requests;   /* short requests: a HOT prefix and at most 32 slot-table tokens.
                                 They get no suffix part; their join workgroup (one per
                                 request, or per k requests) attends each KV head's
                                 slot-table tile itself and joins it with the prefix splits */
  int64_t workspace_bytes;    /* workspace bytes the step used */
  double host_plan_us;        /* host time spent validating and planning */
  double host_call_us;        /* host time of the whole call: validation, planning and the
                                 kernel launch (the call returns right after the launch) */
} gkv_plan_info;
int gkv_last_plan(const gkv_ctx* ctx, gkv_plan_info* out);

/* Plans a step without running it: the request grouping, backend rule and
 * work decomposition that gkv_attn_decode / gkv_decode_step would use for
 * these requests (hot_prefix_ids and cold_indptr_h as there; same shape
 * checks), written to *out (workspace_bytes: what the bound workspace must
 * hold; host_call_us 0).  Host only: no launch and no device memory access
 * (the device's compute-unit count is read when a device is present; without
 * one, gfx950's 256).  The plan is the same as the step's for the same
 * arguments, context settings (gkv_set_dispatch) and pools.  Errors: those
 * of gkv_attn_decode's host checks on these arguments. */
int gkv_plan_step(gkv_ctx* ctx, int32_t batch, const int32_t* hot_prefix_ids, const int32_t* cold_indptr_h,
                  gkv_plan_info* out);

/* Status of the steps run on the bound workspace since it was bound or last
 * read: *joins_timed_out = the number of (request, KV head) joins that gave
 * up waiting for their partial results at the spin limit (their outputs are
 * not valid).  The join of a step's partials runs inside the step kernel and
 * waits for the partials' arrival counts with a bounded wait, so that the
 * kernel always ends; a well-formed step never reaches the bound.  Enqueues
 * a 4-byte copy on `stream` and synchronises it.  After a nonzero status the
 * next step first clears the workspace's counters and status word.
 * GKV_ERR_INVALID without a bound workspace. */
int gkv_step_status(gkv_ctx* ctx, void* stream, int32_t* joins_timed_out);

/* Bound of the join's wait, in polls (each an agent-scope load and a short
 * sleep; default 65536, about 0.1 s): polls >= 0 sets it, -1 restores the
 * default.  For tests of the give-up path (e.g. 0: a join that finds its
 * partials missing gives up at once, and the kernel still ends normally). */
int gkv_set_join_spin_limit(gkv_ctx* ctx, int32_t polls);

/* Measurement: per-workgroup timeline of the following step launches of this
 * context.  With trace_dev non-null (dev, 8-byte aligned, `bytes` long) every
 * step whose grid fits (64 bytes per workgroup; the grid is n_prefix_blocks +
 * n_suffix_blocks + n_join_blocks of gkv_last_plan) writes, per workgroup b,
 * eight uint64 at trace_dev[8 b]: [0] its start; [1] a mid-point mark
 * (prefix split: end of its block loop; suffix workgroup: end of its first
 * part when it runs two, else 0; join: end of its wait); [2] its end;
 * [3] (kind << 32) | (XCC id << 16) | (low 16 bits of the wave's HW_ID
 * register), kind 0 = prefix, 1 = suffix, 2 = join; [4] a second mark
 * (prefix split: its partial rows stored, before it counts its arrivals;
 * suffix workgroup joining its own requests: end of its tiles; else 0);
 * [5] a third mark (suffix workgroup joining its own requests: end of its
 * wait for their prefix splits; else 0); [6], [7] unused.  Times are
 * s_memrealtime ticks of the 100 MHz clock common to the device.  A step
 * whose grid does not fit is not traced.  trace_dev NULL turns tracing off.
 * Host-only. */
int gkv_step_trace(gkv_ctx* ctx, void* trace_dev, size_t bytes);

/* Measurement: a plain streaming read of `bytes` (a multiple of 16) at dev
 * (16-byte aligned) by `workgroups` workgroups of 256 lanes: each wave reads
 * 8 KB chunks with non-temporal loads (eight 16-byte loads in flight per
 * lane), the waves striding over the buffer; the data is discarded (sink_dev: 4 bytes of
 * device memory that the kernel practically never writes).  Timed by the
 * caller on `stream`, it gives the device's achievable read bandwidth, the
 * ceiling the attention kernels are compared with beside the data-sheet
 * peak.  Needs no context.  Asynchronous. */
int gkv_stream_read(const void* dev, size_t bytes, int32_t workgroups, uint32_t* sink_dev, void* stream);

/* Kernel timing, for measurement.  With capacity > 0, each following
 * gkv_attn_decode launches its step kernel (prefix splits, suffix parts and
 * the join of partials, all in one launch) with HIP events that the runtime
 * stamps with the kernel's own start and end, for up to `capacity` calls
 * (then recording stops until read).  capacity 0 disables it and releases
 * the events.  Creating the events is a HIP call. */
int gkv_kernel_timing(gkv_ctx* ctx, int32_t capacity);
/* Waits for the recorded calls and writes the milliseconds of call i's step
 * kernel into ms[i]; *n = number of calls written (<= max_calls).  Clears
 * the record. */
int gkv_kernel_timing_read(gkv_ctx* ctx, float* ms, int32_t max_calls, int32_t* n);

#ifdef __cplusplus
}
#endif

#endif /* GKV_H */
