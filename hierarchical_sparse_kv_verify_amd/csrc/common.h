// Internal declarations shared by the HIP sources of libkvhier.so (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvh {

// ---------------------------------------------------------------- location codes
// tier in bits 30..29, index in bits 28..0, -1 = none (see include/kv_hier.h)
constexpr int kTierShift = 29;
constexpr int32_t kIndexMask = (1 << kTierShift) - 1;
constexpr int32_t kTierHot = 0, kTierStaged = 1, kTierResident = 2, kTierRing = 3;
__host__ __device__ inline int32_t make_loc(int32_t tier, int32_t idx) { return (tier << kTierShift) | idx; }
__host__ __device__ inline int32_t loc_tier(int32_t code) { return code >> kTierShift; }
__host__ __device__ inline int32_t loc_index(int32_t code) { return code & kIndexMask; }

// ---------------------------------------------------------------- counters
// Per-request last-step counters and the per-group cumulative counters use
// the same order as the counter fields of kv_hier_stats.
enum Counter {
  C_ACTIVE_REQ = 0, C_ACTIVE_Q, C_SEL, C_PAD, C_INVALID, C_UNION, C_U_RES, C_U_HOT, C_U_MISS,
  C_PROMOTED, C_OVERFLOW, C_S_RES, C_S_HOT, C_S_MISS, C_U_TAIL, C_S_TAIL, C_NUM
};

// per-request info written by the plan kernel
enum ReqInfo { I_NUNION = 0, I_NMISS, I_NPROMOTE, I_NACTIVE, I_NR, I_NUM = 8 };

// ---------------------------------------------------------------- plan
struct PlanArgs {
  const int32_t* topk;       // [N][Q][k]
  const int32_t* causal;     // [N][Q]
  const int32_t* res_map;    // [N][L] row -> resident pool index or -1
  const int32_t* ring_lo;    // [N] first position the ring has held
  int32_t* slot_map;         // [N][L] row -> hot slot or -1
  int32_t* slot_row;         // [N][B]
  int32_t* slot_lu;          // [N][B]
  int32_t* union_rows;       // [N][Q*k]
  int32_t* union_loc;        // [N][Q*k]
  int32_t* miss_rows;        // [N][Q*k]
  int32_t* victims;          // [N][Q*k]
  uint32_t* protect;         // [N][ceil(B/32)] slots holding a selected row (resolve -> victims)
  int32_t* loc;              // [N][Q][k]
  // [N][Q][k] the same codes with each query's valid entries in ascending row
  // order, then -1 (a query with a repeated row keeps its selection order;
  // written by the order kernel)
  int32_t* sloc;
  int32_t* req_info;         // [N][I_NUM]
  int64_t* req_counts;       // [N][C_NUM] last step
  unsigned long long* cum;   // [C_NUM] cumulative
  int N, Q, k, B, L, t;
  int Rd;                    // ring rows per request (the tail: positions >= max(ring_lo, n_r + Q - Rd))
  int m;                     // positions per stored row (compressed source when > 1: no tail)
  int has_resident;          // 0: the resident map holds no row (its lookups are skipped)
  int chunk_words;           // bitmap words per row chunk (rows per chunk = 32 * chunk_words)
  int sort_cap;              // power of two >= B
  // the step's own ring write (eq. 10), done by the plan's workgroups: row j of
  // request r goes to ring slot r*Rd + causal[r][j] % Rd for causal >= 0
  // (ring_rows null: nothing written)
  const uint4* ring_rows;    // [N][Q][row16]
  uint4* ring;               // [N*Rd][row16]
  int row16;
};
size_t plan_lds_bytes(int Q, int k, int B, int chunk_words, int sort_cap);
// LDS of the order kernel (row-ordered lists)
size_t plan_order_lds_bytes(int Q, int k, int chunk_words);
// union, probe, staging positions, locations (everything the fetch needs);
// ev_start / ev_stop as for launch_miss_gather
hipError_t launch_plan(const PlanArgs& a, size_t lds, hipStream_t s, hipEvent_t ev_start = nullptr,
                       hipEvent_t ev_stop = nullptr);
// dynamic-LDS limits of the plan and attention kernels, on the current device
hipError_t plan_init_attributes();
hipError_t attn_init_attributes();
// LRU victims, promotions and slot-table updates (after launch_plan)
hipError_t launch_plan_victims(const PlanArgs& a, size_t lds, hipStream_t s);
// each query's location codes in ascending row order (a.sloc), after the
// plan; ev_start / ev_stop as for launch_plan
hipError_t launch_plan_order(const PlanArgs& a, size_t lds, hipStream_t s, hipEvent_t ev_start = nullptr,
                             hipEvent_t ev_stop = nullptr);

// ---------------------------------------------------------------- copies
struct HostRowSrc {
  const uint4* const* prefix;   // device array [n_prefix] of host-mapped prefix bases
  const uint4* tails;           // host-mapped base of [N][tail_rows][row]
  int n_prefix, prefix_len, tail_rows, row16;   // row16 = 16-byte chunks per row
};

// miss gather: for r in [r0, r1), i < req_info[r][I_NMISS]:
//   staging[(r*QK + i)] = host row miss_rows[r][i]
// (ev_start / ev_stop, when given, are bound to the launch itself: they complete
// with it and time its own start and end, with no marker of their own)
hipError_t launch_miss_gather(const HostRowSrc& src, const int32_t* miss_rows, const int32_t* req_info,
                              uint4* staging, int QK, int r0, int r1, int wg_per_req, hipStream_t s,
                              hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);
// promote: hot[(r*B + victims[r][i])] = staging[r*QK + i], i < req_info[r][I_NPROMOTE]
hipError_t launch_promote(const uint4* staging, const int32_t* victims, const int32_t* req_info,
                          uint4* hot, int QK, int B, int row16, int r0, int r1, hipStream_t s);
// ring write: ring[r*Rd + causal[r][j] % Rd] = rows[r][j] for active j
hipError_t launch_ring_write(const uint4* rows, const int32_t* causal, uint4* ring, int N, int Q,
                             int Rd, int row16, hipStream_t s);
// setup gather from host: dst[dst_idx[i]] = host row (req[i], row[i]), i < n
hipError_t launch_host_rows_to_dev(const HostRowSrc& src, const int32_t* req, const int32_t* rows,
                                   const int64_t* dst_idx, int n, uint4* dst, hipStream_t s);
// commit: for r with acc[r] >= 0, n = nbefore[r], n' = n + 1 + acc[r]:
//   a group with m == 1: host tail row (pos - prefix_len) = ring row of pos, n <= pos < n';
//   a group with m > 1 (eq. 8): host tail row (s - prefix_len) = src[g][r*cmax + s - n/m],
//   n/m <= s < n'/m.  compressed = 0 handles the m == 1 groups, 1 the others.
struct CommitGroup { const uint4* ring; uint4* tails; int m, cmax; };
hipError_t launch_commit(const CommitGroup* groups, int G, const int32_t* nbefore, const int32_t* acc,
                         const uint4* const* src, int compressed, int N, int Qmax, int Rd, int prefix_len,
                         int tail_rows, int row16, hipStream_t s);
// read rows at location codes into dst [n][row]
struct PoolView { const uint4* hot; const uint4* staging; const uint4* resident; const uint4* ring; };
hipError_t launch_read_rows(const PoolView& pv, const int32_t* locs, int n, uint4* dst, int row16,
                            hipStream_t s);
// a follower layer's counters: dst[r][c] = src[r][c]; cum[c] += sum_r src[r][c]
hipError_t launch_counts_follow(const int64_t* src, int64_t* dst, unsigned long long* cum, int N, hipStream_t s);
// dynamic optional residency: one descriptor per group; a page list holds
// (request, page index, pool page) triples
struct OptGroup { HostRowSrc src; uint4* pool; int32_t* res_map; };
// pool rows of every listed page in every group <- host rows idx*P .. idx*P+P-1 of the request
hipError_t launch_opt_copy(const OptGroup* groups, int G, const int32_t* list, int n, int P, int row16, int wgs,
                           hipStream_t s);
// res_map of every group: rows of every listed page -> pool*P + i (publish) or -1 (withdraw)
hipError_t launch_opt_map(const OptGroup* groups, int G, const int32_t* list, int n, int P, int L, int publish,
                          hipStream_t s);
// fill 32-bit words with a value (used instead of memset inside the step)
hipError_t launch_fill32(uint32_t* p, uint32_t v, size_t n, hipStream_t s);

// ---------------------------------------------------------------- attention
struct AttnArgs {
  const uint16_t* q;          // [N][Q][H][d_qk]
  const int32_t* loc;         // [N][Q][k]
  const int32_t* causal;      // [N][Q]
  const int32_t* ring_lo;     // [N]
  const uint16_t* hot;        // hot pool of the group
  const uint16_t* staging;    // arena of the group
  const uint16_t* resident;   // resident pool (may be null)
  const uint16_t* ring;       // ring of the group
  const uint16_t* zero;       // one all-zero row (masked positions read it)
  uint16_t* out;              // [N][Q][H][d_v]
  float* part_o;              // [(chunk requests)*Q*HG*S][32*HB][d_v] partial numerators (splits > 1)
  float* part_ml;             // [(chunk requests)*Q*HG*S][32*HB][2]
  int N, Q, k, H, W, Rd, block_only;
  int r0, r1;                 // request range of this launch
  int splits, head_groups;
  int hpw;                    // heads per workgroup of this launch: 32, 64 or 128 (attn_heads_per_wg)
  float scale_log2;           // softmax scale * log2(e)
};
// supported layouts; returns hipErrorInvalidValue for others
bool attn_layout_supported(int row_elems, int d_qk, int v_off, int d_v);
// heads per attention workgroup for a launch over `queries` queries
int attn_heads_per_wg(int H, int row_elems, int64_t queries);
// ev_start / ev_stop as for launch_miss_gather
hipError_t launch_attn(const AttnArgs& a, int row_elems, int d_qk, int v_off, int d_v, hipStream_t s,
                       hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);
hipError_t launch_attn_combine(const AttnArgs& a, int d_v, hipStream_t s, hipEvent_t ev_start = nullptr,
                               hipEvent_t ev_stop = nullptr);

}  // namespace kvh
