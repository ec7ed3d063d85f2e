/*
 * kv_hier.h - C ABI of libkvhier.so: one speculative verification step of
 * sparse attention over a hierarchical KV cache, on one AMD Instinct MI355X
 * (gfx950).
 *
 * The operation follows "Adaptive DHiSparse: Speculative Decoding over a
 * Load-Adaptive KV Hierarchy" (arXiv 2610.13708):
 *   - §2.1 eq. (1): each query attends over the rows its top-k selected;
 *     eq. (2): ready rows R_t and the host-recovery set D_t = S_t \ R_t.
 *   - §2.2 "Fixed-cache offloading": per request and KV source a bounded
 *     GPU cache of B rows, hit detection, protection of selected rows, LRU
 *     victims, one fetch per missing row from pinned host memory.
 *   - §3.2 / Figure 2: resolution order (1) ready optional history,
 *     (2) hot cache, (3) host copy; locations returned in selection order.
 *   - §3.3 eqs. (5)-(7): the K_r queries of a request keep their own causal
 *     boundary; the union U_r of their selections is resolved once and each
 *     distinct missing row is copied once (Figure 3 callout 2); overflow
 *     rows beyond the hot cache are staged; acceptance commits the anchor
 *     and A_r drafts, n' = n + 1 + A.
 *   - §3.4 eqs. (9)-(10) and the staging paragraph: window-bounded ring of
 *     R_d = p*ceil((W+p-1+K_max)/p) rows per request addressed
 *     phi(i,t) = i*R_d + (t mod R_d); chi staging arenas of N*K_max*k rows
 *     reused across layer groups after their readers finish and promoted rows
 *     are copied back to their hot-cache slots.
 *   - §3.5 eqs. (11)-(12): every list entry gets a location l with
 *     KV[l] = c_{r,s}; a row held in two tiers resolves to one of them.
 *   - §3.1 eqs. (3)-(4) ("Load-Adaptive Residency"): optional history in
 *     reclaimable pages of the device pool; admission reclaims whole requests
 *     in the runtime's reclaim order until their pages cover the deficit;
 *     bounded round-robin repopulation; locations are published as ready
 *     only after their copies complete (kv_hier_opt_*).
 *
 * Conventions
 *   - Every call returns KV_OK (0) or a negative KV_E* code; no exception
 *     crosses the ABI.  kv_hier_last_error() gives a message for the handle.
 *   - Every argument is checked before a call changes anything: a call that
 *     returns KV_EINVAL, KV_ESTATE, KV_EUNSUPPORTED or KV_EWAIT has changed
 *     nothing.  If a call that changes state fails after its checks (a HIP
 *     runtime error, a failed pinned allocation), the handle's device state
 *     may be partly updated: the handle is then latched, and every later call
 *     that changes state or enqueues device work returns KV_ESTATE (its
 *     message names the first failure).  Calls that only read (stats, lists,
 *     info, hist_len, sync, last_error) and kv_hier_destroy still work.
 *   - Streams: steps, Reuse layers and commits may be issued on different
 *     caller streams of the handle's device; the library orders its own work
 *     between them with events (each layer's plan after every earlier reader
 *     of the plan state it rewrites, a Reuse after the step whose selection it
 *     reads, every launch using the shared split-key partials after the
 *     previous one).  The caller orders its own buffers.
 *   - "device" pointers are HIP device allocations owned by the caller that
 *     must stay valid until the stream passes the step; "host" pointers are
 *     ordinary host memory read or written before the call returns.
 *   - Rows are bf16 (stored as uint16 bit patterns), row_elems per row.
 *   - Out-of-range values inside device arrays (a top-k entry outside
 *     [0, n_r), for instance) are not errors: they are counted and skipped.
 *   - Location code (int32): tier in bits 30..29, index in bits 28..0,
 *     -1 = none.  Tier 0: hot slot r*B + slot; tier 1: staged row
 *     r*K_max*k + i of the group's arena; tier 2: resident pool index;
 *     tier 3: ring row r*R_d + (pos mod R_d) (a selected row still in the
 *     request's tail, Figure 2 callout 1).
 */
#ifndef KV_HIER_H
#define KV_HIER_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  KV_OK = 0,
  KV_EINVAL = -1,        /* bad argument or size                        */
  KV_ENOMEM = -2,        /* device or pinned host allocation failed      */
  KV_EHIP = -3,          /* a HIP runtime call failed                    */
  KV_ESTATE = -4,        /* call not valid in the current state          */
  KV_EUNSUPPORTED = -5,  /* shape outside what the kernels are built for */
  KV_EWAIT = -6          /* admission must wait (eq. 4): nothing changed  */
};

enum { KV_TIER_HOT = 0, KV_TIER_STAGED = 1, KV_TIER_RESIDENT = 2, KV_TIER_RING = 3 };

enum {
  KV_FLAG_TIMING = 1,    /* time every kernel with HIP events (kv_hier_stats ms_*) */
  KV_FLAG_POISON = 2,    /* debug: fill a staging-arena chunk with NaN between its last readers
                            and its next fetch (and a dynamic pool at create)            */
  KV_FLAG_TIMING_ATTN = 4, /* time only the attention (and split-combine) launches, with
                              events bound to the launches (no marker on any stream)   */
  KV_FLAG_SERIAL = 8,     /* measurement: the step's attention starts only after its whole
                             host fetch, so it runs alone on the GPU (slower steps)     */
  KV_FLAG_SYNC_BACKUP = 16, /* measurement: commit's host backup runs on the caller's stream,
                             ahead of the next step, instead of beside it             */
  KV_FLAG_TEST_FAIL_ATTN = 32 /* test hook: every attention launch reports a HIP error without
                             launching anything (exercises the failure latch below)   */
};

typedef struct kv_hier kv_hier_t;  /* opaque, owned by the library */

typedef struct {
  int32_t n_req;            /* N request slots                                          */
  int32_t n_groups;         /* G layer groups (payload sources), each with its own cache */
  int32_t n_arenas;         /* chi staging arenas; group g stages into arena g % chi     */
  int32_t hist_cap;         /* L: history rows per request (host backing, maps)          */
  int32_t n_prefix;         /* shared host prefixes; 0 = every request owns rows [0, L)  */
  int32_t prefix_len;       /* rows [0, prefix_len) of request r live in prefix r % n_prefix */
  int32_t row_elems;        /* bf16 elements per row (d_KV = 2*row_elems bytes)          */
  int32_t d_qk;             /* key: K = row[0 : d_qk]                                    */
  int32_t v_off;            /* value: V = row[v_off : v_off + d_v]                       */
  int32_t d_v;              /* layouts with kernels (row_elems, d_qk, v_off, d_v):
                               (576, 576, 0, 512) absorbed MLA (512 latent + 64 rope);
                               (144, 144, 0, 128) the 288-B rows of Table 3
                               (128 latent + 16 rope); (256, 128, 128, 128) K || V.
                               Others: KV_EUNSUPPORTED                                   */
  int32_t n_heads;          /* query heads sharing each row                              */
  int32_t q_max;            /* K_max verification queries per request (<= 32)           */
  int32_t topk;             /* k >= 1 selections per query (a query with nothing selected
                               passes a list of -1 pads).  The resolution keeps the
                               q_max*topk location codes of a request in LDS beside the
                               hot-slot bitmap: above about 40,000 entries create returns
                               KV_EUNSUPPORTED                                           */
  int32_t hot_slots;        /* B (<= 16384)                                              */
  int32_t ring_window;      /* W                                                         */
  int32_t ring_page;        /* p                                                         */
  int32_t ring_block_only;  /* 1: ring branch limited to positions >= n_r (eq. 5 literal) */
  int32_t n_chunks;         /* request chunks pipelined fetch -> attention.  0 = auto:
                               for N >= 64 four quarters of the requests, the last one
                               halved when each half still has >= 256 attention workgroups
                               (N/8 x q_max x head groups); below 64 requests two chunks
                               (one under 16).  A chunk under 256 attention workgroups
                               splits each query's keys (merged by a combine pass)       */
  int64_t resident_cap;     /* rows of the resident pool per group (0 = no resident tier) */
  float softmax_scale;      /* <= 0 selects 1/sqrt(d_qk)                                 */
  int32_t flags;            /* KV_FLAG_*                                                 */
  int32_t fetch_cus;        /* >0: CUs reserved for the host fetch (CU-masked streams: the
                               fetch runs on those CUs, the rest of the step on the others);
                               0: every stream may use every CU                          */
  int32_t fetch_wgs;        /* one-wave workgroups of a chunk's host fetch, at least one per
                               request (0 = 128): enough PCIe reads in flight to fill the
                               link; more only queue in the memory system and slow the
                               attention running beside them                             */
  int32_t plan_share;       /* > 1: groups come in consecutive sets of plan_share payload
                               layers fed by one index producer (one selection).  The first
                               group of a set resolves the selection once and starts the
                               host fetch of every layer of the set (each into its own
                               arena: n_arenas >= plan_share); the others reuse its plan
                               and their verify_step only attends and copies back.  Groups
                               of a set must be given identical set_hot / set_resident
                               contents (their own payload rows).  0 or 1: one plan per
                               group.                                                    */
  int32_t opt_page_rows;    /* > 0: dynamic optional residency (kv_hier_opt_*): the resident
                               pool of every group is resident_cap / opt_page_rows pages of
                               this many rows (resident_cap a multiple of it); one page index
                               addresses the same page in every group's pool.  Static
                               resident sets (kv_hier_set_resident) are then refused.
                               0: static resident sets only.                             */
  int32_t opt_reserve;      /* M_res of eq. (3), in pages (dynamic residency)            */
} kv_hier_config;

/* Counters of one layer group (kv_hier_stats).  "union_*" count distinct rows
 * of U_r, "sel_*" count list entries (selections). */
typedef struct {
  int64_t calls;
  int64_t active_requests;
  int64_t active_queries;   /* verified query tokens                                     */
  int64_t selections;       /* valid list entries                                        */
  int64_t pads;
  int64_t invalid;
  int64_t union_rows;
  int64_t union_resident;
  int64_t union_hot;
  int64_t union_miss;       /* = rows fetched from host, once each                       */
  int64_t fetched_bytes;
  int64_t promoted;         /* missing rows given a hot-cache slot                       */
  int64_t overflow;         /* missing rows staged only                                  */
  int64_t sel_resident;
  int64_t sel_hot;
  int64_t sel_miss;         /* missing selections (sum over queries)                     */
  /* kernel time in ms summed over timed calls (KV_FLAG_TIMING), and launch counts
     (a leader's ring write runs inside its plan and is counted there)          */
  double ms_ring, ms_plan, ms_gather, ms_attn, ms_combine, ms_promote, ms_victims;
  int64_t n_ring, n_plan, n_gather, n_attn, n_combine, n_promote, n_victims;
  int64_t union_tail;       /* distinct rows resolved from the tail (the ring)           */
  int64_t sel_tail;         /* selections resolved from the tail                         */
  double ms_order;          /* the row-ordered lists (timed as the kernels above)        */
  int64_t n_order;
} kv_hier_counters;

/* Per-request lists of the last verify_step of a group (kv_hier_last_lists).
 * Every array is caller-owned host memory of q_max*topk elements. */
typedef struct {
  int32_t *union_rows;      /* U_r ascending                                             */
  int32_t *union_loc;       /* location code of each union row                           */
  int32_t *miss_rows;       /* D_r ascending = staging order                             */
  int32_t *victims;         /* hot slot taken by miss i, i < n_promote                   */
  int32_t *loc;             /* [q_max][topk] location of every list entry                */
  int32_t n_union, n_miss, n_promote, n_active;
} kv_hier_lists;

typedef struct {
  int32_t ring_rows;        /* R_d of eq. (9)                                            */
  int32_t n_chunks;
  int64_t bytes_hot, bytes_staging, bytes_ring, bytes_maps, bytes_resident, bytes_host;
  int32_t attn_splits;      /* the largest key split count of a chunk (1: none)          */
  int32_t attn_head_groups; /* attention workgroups per query of a request-chunk launch
                               (the largest over the chunks): 32, 64 or 128 heads each   */
  int32_t plan_rows_per_pass; /* history rows the resolution's LDS row bitmap covers at once:
                               a longer history is resolved in ceil(n_r / this) passes
                               over row ranges (the q_max*topk location codes share the
                               bitmap's LDS)                                             */
  int32_t attn_reuse_head_groups; /* the same for a launch over every request (Reuse)      */
  int32_t attn_row_order;   /* 1: the attention of every request chunk but a leader's
                               first (and of Reuse layers) walks each query's rows in
                               ascending row order, written after the resolution beside the
                               first fetch from its selection-order locations (a query that
                               repeats a row keeps its selection order); 0: selection order
                               everywhere (one request chunk, lists of fewer than 1024
                               entries, or the per-query bitmaps do not fit one
                               workgroup's LDS)                                          */
} kv_hier_info;

/* Creates a handle ("Adaptive DHiSparse" §2.2 fixed-cache offloading and
 * §3.4: per request and source a bounded hot cache of B rows, the draft ring
 * of eq. (9), chi staging arenas shared by the layer groups, host copies of the
 * history): allocates hot caches, slot tables, maps, rings, staging
 * arenas, plan buffers, a side stream and events on the current HIP device,
 * and pinned host history for every group.  Every later call on the handle
 * runs on that device whatever device is current when it is made (the
 * caller's current device is restored before it returns); streams passed to
 * it must belong to that device.  Returns KV_EINVAL for
 * inconsistent sizes, KV_EUNSUPPORTED for a row layout without kernels,
 * KV_ENOMEM when an allocation fails. */
int kv_hier_create(const kv_hier_config *cfg, kv_hier_t **out);

/* Frees everything; waits for outstanding work first.  NULL is accepted. */
void kv_hier_destroy(kv_hier_t *h);

/* Message of the last failing call on h (never NULL); with h == NULL, the
 * message of the last failed kv_hier_create on the calling thread. */
const char *kv_hier_last_error(const kv_hier_t *h);

/* Sizes of what create allocated.  Host out-pointer. */
int kv_hier_info_get(kv_hier_t *h, kv_hier_info *out);

/* Pinned host rows of group g that the caller fills before the first step:
 * kind 0 = prefix `index` (prefix_len rows), kind 1 = tail of request `index`
 * (rows prefix_len .. hist_cap-1, i.e. hist_cap - prefix_len rows).  The
 * pointer stays owned by the library (valid until destroy). */
int kv_hier_host_rows(kv_hier_t *h, int g, int kind, int index, void **rows, int64_t *n_rows);

/* Committed frontier n_r of every request (host int32[n_req]); also marks the
 * ring of every group empty below n_r.  Eq. (5): query j sits at n_r + j. */
int kv_hier_set_hist_len(kv_hier_t *h, const int32_t *hist_len);

/* Hot-cache contents of (g, r) ("Adaptive DHiSparse" §2.2: the bounded GPU
 * cache of one request and source, whose LRU stamps order the victims): n <= B
 * host rows (-1 = empty slot) with their
 * last-used stamps (>= 0); rows must be distinct and < hist_cap.  Row bytes
 * are copied from the host backing.  Synchronous. */
int kv_hier_set_hot(kv_hier_t *h, int g, int r, const int32_t *rows, const int32_t *last_used, int n);

/* Static ready optional history of (g, r) (§3.1): host uint8[hist_cap] bitmap; rows
 * below the frontier with a non-zero byte become resident, receiving
 * consecutive pool indices in ascending row order after those already handed
 * out in this group.  Once per (g, r) until kv_hier_clear_resident(g).
 * KV_ENOMEM when the pool (resident_cap rows) is full.  Synchronous. */
int kv_hier_set_resident(kv_hier_t *h, int g, int r, const uint8_t *bitmap);
int kv_hier_clear_resident(kv_hier_t *h, int g);

/* Loads committed positions first_pos .. n_r-1 (n rows, host bf16
 * [n][row_elems]) into the ring of (g, r) at the addresses of
 * "Adaptive DHiSparse" §3.4 eq. (10), phi(r, t) = r*R_d + (t mod R_d); first_pos + n must equal n_r and
 * n <= R_d.  Synchronous. */
int kv_hier_ring_load(kv_hier_t *h, int g, int r, int32_t first_pos, const void *rows, int n);

/* One verification step of layer group g, asynchronous on `stream`
 * (hipStream_t; NULL = default stream):
 *   queries    device bf16 [N][q_max][n_heads][d_qk]
 *   topk_idx   device int32 [N][q_max][topk]; -1 = pad
 *   causal_pos device int32 [N][q_max]: n_r + j for active queries, -1 for an
 *              inactive suffix (request inactive when causal_pos[r][0] < 0)
 *   ring_rows  device bf16 [N][q_max][row_elems]: new KV row of each query's
 *              position, written to the ring at phi(r, p_j) (eq. 10); NULL for a
 *              Reindex consumer of a shared source, whose producer already wrote
 *              this step's rows (the ring is left as it is)
 *   out        device bf16 [N][q_max][n_heads][d_v]; zero for inactive queries
 * Resolves the union of each request's selections, probes the tail (rows the
 * request's ring still holds: positions >= max(first ring position,
 * n_r + q_max - R_d)) and the resident map, then the hot cache, fetches every
 * distinct missing row once from pinned host memory
 * into the group's staging arena (the first request chunk on `stream` after
 * the resolution, the others on a side stream, overlapped with attention of
 * earlier request chunks), runs exact sparse attention of every query over
 * its own list plus its ring window, and copies promoted rows into their
 * victim slots.  Caller contract (not checked on the device): causal_pos[r][0]
 * equals the frontier set by kv_hier_set_hist_len / kv_hier_commit.
 * With plan_share > 1 ("Adaptive DHiSparse" §3.2: one index producer announcing
 * positions for several payload layers): the first group of a set resolves
 * topk_idx and starts the host fetch of every layer of the set; a follower
 * group's step (after its leader's, once per step, else KV_ESTATE) ignores
 * topk_idx (may be NULL), attends over its own payload through the leader's
 * locations and copies back into its own hot cache.
 * Shared KV sources ("Adaptive DHiSparse" §2 physical-source sharing, §3.2):
 * a group is one physical source; a Reindex consumer is another verify_step
 * on the same group within the step (fresh topk_idx, ring_rows NULL): it
 * resolves against the cache state the earlier consumers left, so only rows
 * absent from it are fetched.  A Reuse consumer is kv_hier_verify_reuse. */
int kv_hier_verify_step(kv_hier_t *h, int g, const void *queries, const int32_t *topk_idx,
                        const int32_t *causal_pos, const void *ring_rows, void *out,
                        void *stream);

/* kv_hier_verify_step for callers that cannot allocate device memory during
 * a call (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same step, same arguments and same results, but the
 * attention's split-key partials live in a file-scope device array of the
 * library (32 MiB, one copy per GPU, held until the process ends) instead of
 * the handle's buffer, and the call allocates nothing: no device or host
 * memory, no events (KV_FLAG_TIMING and KV_FLAG_TIMING_ATTN are not honoured
 * here), and optional-history pages are not published here (kv_hier_opt_publish
 * and kv_hier_verify_step publish them).  The caller still passes every input
 * and output.  Returns KV_EINVAL, before any device work, when the handle's
 * split-key partials (blocks x heads per workgroup x (d_v + 2) floats) exceed
 * the array.  Calls on one handle are ordered by the library; calls of two
 * handles on one GPU that overlap in time share the array and race. */
int kv_hier_verify_step_static(kv_hier_t *h, int g, const void *queries, const int32_t *topk_idx,
                               const int32_t *causal_pos, const void *ring_rows, void *out, void *stream);

/* A Reuse consumer of source g ("Adaptive DHiSparse" §2, §3.2): new queries
 * (device bf16 [N][q_max][n_heads][d_qk]) attend, exactly as in verify_step,
 * over the latest selection of g through its location vector and the payload
 * it materialized (hot cache, staged rows, resident pool, ring): no
 * resolution, fetch or cache update.  causal_pos must equal the one given to
 * that selection's verify_step (caller contract); out as in verify_step.
 * Asynchronous on `stream`.  KV_ESTATE when g has no selection in this step
 * (none yet, or a commit since) or when a later fetch of another group has
 * replaced its staged rows (arena g mod n_arenas). */
int kv_hier_verify_reuse(kv_hier_t *h, int g, const void *queries, const int32_t *causal_pos, void *out,
                         void *stream);

/* Acceptance (eq. 7) for every request: accepted[r] = A_r in [0, q_max-1], or
 * -1 for no commit.  Copies the ring rows of positions n_r .. n_r+A_r of every
 * group into the pinned host backing and advances n_r by 1 + A_r; rejected
 * rows are never published.  The host backup runs after `stream`'s work on a
 * library stream, beside the next step (when R_d >= 2 q_max; else on
 * `stream`): the rows it writes stay in the tail through the next step, which
 * therefore never fetches them, and each step waits for the backup of the
 * commit before the last.  accepted is host memory read before return.
 * Caller contract: A_r < K_r of the last step. */
int kv_hier_commit(kv_hier_t *h, const int32_t *accepted, void *stream);

/* Compressed sources ("Adaptive DHiSparse" §3.3 eq. 8): group g stores one
 * row per m consecutive token positions.  Its history rows (host rows,
 * set_hot / set_resident indexes, topk_idx entries) are stored-row indexes;
 * an entry s is a valid selection iff 0 <= s < floor(n_r / m): the
 * incomplete group stays in the tail as positions, reached by the ring
 * branch, whose rows (ring_rows, ring_load) stay per position.  Selections of
 * such a group never resolve from the ring.  Call before the group's first
 * step; m = 1 restores an uncompressed source.  KV_ESTATE with dynamic
 * residency or plan-sharing sets (both assume uncompressed sources). */
int kv_hier_set_compression(kv_hier_t *h, int g, int32_t m);

/* kv_hier_commit for handles with compressed sources: src_rows is a host
 * array of n_groups device pointers; for a group with m > 1 it points to bf16
 * [N][ceil(q_max/m)][row_elems], row i of request r being the stored row
 * floor(n_r/m) + i completed by the commit (eq. 8: floor(n_r/m) <= s <
 * floor(n_r'/m)); entries of uncompressed groups are ignored (may be NULL).
 * The completed rows get their host copy in `stream`'s order (before the next
 * step can fetch them); the caller's buffers must stay valid until `stream`
 * passes the commit.  kv_hier_commit on a handle with a compressed group is
 * KV_EINVAL. */
int kv_hier_commit_src(kv_hier_t *h, const int32_t *accepted, const void *const *src_rows, void *stream);

/* Waits for all work of the handle, then returns group g's counters:
 * cumulative over all steps and of the last step.  Either pointer may be NULL.
 * They are the quantities "Adaptive DHiSparse" §4.3.1-4.3.2 measures: the
 * share of selected rows fetched from the host (sel_miss / selections, Table
 * A1), distinct fetched rows and bytes (the resolver's unique host-miss
 * payload, Figure 8a), and missing selections per fetched row. */
int kv_hier_stats(kv_hier_t *h, int g, kv_hier_counters *cumulative, kv_hier_counters *last);
int kv_hier_reset_stats(kv_hier_t *h);

/* Waits, then copies request r's lists of the last step of group g (a
 * follower's are its leader's): the union U_r of eq. (6), the host-recovery
 * set D_r of eq. (2) in staging order, and the location of every list entry
 * in selection order, eq. (12). */
int kv_hier_last_lists(kv_hier_t *h, int g, int r, kv_hier_lists *out);

/* Waits, then copies the slot table of (g, r): host int32[B] rows and stamps
 * (a follower's is its leader's: the plan's table). */
int kv_hier_slot_table(kv_hier_t *h, int g, int r, int32_t *rows, int32_t *last_used);

/* Waits, then copies the rows at n location codes (host int32) of group g
 * into host bf16 [n][row_elems]; codes of -1 produce zero rows. */
int kv_hier_read_rows(kv_hier_t *h, int g, const int32_t *locs, int n, void *rows);

/* Committed frontier per request (host int32[n_req]). */
int kv_hier_hist_len(kv_hier_t *h, int32_t *hist_len);

/* Waits for every stream the handle uses. */
int kv_hier_sync(kv_hier_t *h);

/* Replaces the KV_FLAG_* bits set at create (takes effect for later calls). */
int kv_hier_set_flags(kv_hier_t *h, int32_t flags);

/* ---------------------------------------------------------------------------
 * Dynamic optional residency ("Adaptive DHiSparse" §3.1, eqs. 3-4; Figure 2).
 * Needs opt_page_rows > 0.  The pool holds M = resident_cap / opt_page_rows
 * pages of P = opt_page_rows rows in every group.  An admitted request's
 * required allocations are charged against M in pages (they live in the
 * request's own hot cache, ring and staging, not in the pool); its optional
 * history is the complete pages of its imported history, floor(n_r / P)
 * pages for the frontier n_r at admission.  Eq. (3) holds at all times:
 * sum(required) + sum(held) + opt_reserve <= M.  A page is "held" once
 * population reserves it and "ready" once its copy has completed and it has
 * been published to the map that resolution probes first; rows of a pending
 * page resolve through the hot cache or the host.  Every row keeps its host
 * copy, so reclaiming never needs a backup copy here.  All of these calls
 * are host-side decisions plus asynchronous device work: they never wait for
 * the GPU (except kv_hier_opt_publish with wait = 1).
 * ------------------------------------------------------------------------- */

typedef struct {
  int32_t pool_pages;          /* M                                                     */
  int32_t page_rows;           /* P                                                     */
  int32_t reserve;             /* M_res                                                 */
  int32_t cursor;              /* next request slot the round-robin population visits   */
  int64_t admitted;            /* admitted requests                                     */
  int64_t required_pages;      /* sum of required pages of admitted requests            */
  int64_t held_pages;          /* optional pages held (pending + ready)                 */
  int64_t ready_pages;         /* optional pages published as ready                     */
  int64_t pending_pages;       /* held, copy not yet published                          */
  int64_t free_pages;          /* pool pages held by nobody                             */
  int64_t eligible_pages;      /* complete imported pages of admitted requests          */
  int64_t pages_populated;     /* cumulative: pages reserved and copied                 */
  int64_t pages_published;     /* cumulative                                            */
  int64_t pages_reclaimed;     /* cumulative: pages dropped by reclaim or completion    */
  int64_t requests_reclaimed;  /* cumulative: requests taken by eq. (4)                 */
  int64_t admissions_waited;   /* cumulative: admissions refused with KV_EWAIT          */
  int64_t bytes_populated;     /* cumulative host bytes copied into the pool (all groups) */
} kv_hier_opt_info;

/* Admission of request r with `required_pages` pages of required allocations
 * (eq. 3).  When the admission leaves a deficit
 *   Delta = sum(required) + required_pages + sum(held) + reserve - M > 0,
 * the requests of `order` (host int32[n_order], distinct admitted requests:
 * the runtime's reclaim order r_1, r_2, ...) are walked and the first q with
 * a_{r_1} + ... + a_{r_q} >= Delta lose all of their optional pages (eq. 4;
 * a_r counts held pages, pending or ready); the other requests keep theirs.
 * Reclaimed pages are unpublished before any later step resolves, and reused
 * only after the attention of earlier steps has read them.  A reclaimed request
 * stays admitted and resolves through its hot cache and the host.  If the
 * whole order cannot cover Delta, returns KV_EWAIT and changes nothing.
 * *n_reclaimed (may be NULL) receives q.  KV_ESTATE: no dynamic residency, or
 * r already admitted. */
int kv_hier_opt_admit(kv_hier_t *h, int r, int32_t required_pages, const int32_t *order, int n_order,
                      int32_t *n_reclaimed);

/* Completion of request r: its required and optional pages are released
 * (optional pages unpublished and reused as after a reclaim).  KV_ESTATE if r
 * is not admitted. */
int kv_hier_opt_complete(kv_hier_t *h, int r);

/* One bounded round-robin population attempt: request slots are visited
 * cyclically from the cursor; each visit to an admitted request holding fewer
 * than its eligible pages reserves its next page (ascending page index) in
 * the lowest free pool page.  Stops after max_pages pages, when the eq. (3)
 * budget is used up, or after a whole cycle without a reservation; the cursor
 * then points past the last visited slot.  The rows of the reserved pages are
 * copied from pinned host memory into every group's pool on the library's
 * population stream, concurrently with steps; the pages become ready when
 * published after the copy.  *n_assigned (may be NULL) receives the count. */
int kv_hier_opt_populate(kv_hier_t *h, int32_t max_pages, int32_t *n_assigned);

/* Publishes the pages whose copies have completed (wait = 0: those already
 * complete; wait = 1: waits for every pending copy first).  Publication is
 * ordered before the next step's resolution.  The first group's verify_step
 * (g = 0) publishes completed copies by itself, without waiting. */
int kv_hier_opt_publish(kv_hier_t *h, int wait);

/* Host view of the residency state: totals (info, may be NULL) and, for
 * request r when r >= 0, the pool page held for each of its first n_pages
 * page indexes (held, host int32[n_pages], -1 = none) and whether it is
 * published (ready, host uint8[n_pages]); either array may be NULL. */
int kv_hier_opt_query(kv_hier_t *h, int r, int32_t n_pages, int32_t *held, uint8_t *ready,
                      kv_hier_opt_info *info);

/* Cache-state snapshot of group g: op 0 saves the hot rows, slot tables,
 * row->slot map and step counter into library-owned device memory (allocated
 * on the first save); op 1 restores them, so a following step with the same
 * inputs resolves exactly as the step after the save did.  Waits for
 * outstanding work.  KV_ESTATE when restoring without a save. */
int kv_hier_cache_snapshot(kv_hier_t *h, int g, int op);

#ifdef __cplusplus
}
#endif
#endif /* KV_HIER_H */
