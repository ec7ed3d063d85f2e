// Resolution plan of one verification step, one 1024-thread workgroup per
// request in each of its two kernels.
//
// "Adaptive DHiSparse" (arXiv 2610.13708):
//  - §3.3 eq. (6): the retrieval union U_r of the K_r queries' selections and
//    the missing set D_r = U_r \ R_r; each distinct missing row is fetched once.
//  - §3.2 / Figure 2: probe order (1) the tail (rows the request's ring
//    still holds) or the ready optional-history map, (2) hot cache,
//    (3) host; locations emitted in selection order (eq. 12).
//  - §2.2 "Fixed-cache offloading": selected rows in the cache are protected,
//    unselected rows are LRU victims.
//  - §3.3 (overflow paragraph) and §3.4: missing rows are staged in the
//    request's K_max*k segment of the arena; rows that get a victim slot are
//    promoted (copied back) after attention, the rest overflow.
//
// Union and dedup use an LDS bitmap over a chunk of row ids: marking is one
// LDS atomicOr per selection, and compaction of the bitmap (popcount + block
// prefix sum) yields U_r already in ascending order together with a per-word
// prefix table, so the rank of any row in U_r is a prefix lookup plus one
// popcount.  Histories longer than a chunk are processed chunk by chunk.
// LRU victims run in a second kernel, off the path to the host fetch (the
// fetch needs only the missing rows): the unselected slots' (last_used, slot)
// keys are compacted in LDS and bitonic-sorted; keys are unique, so the order
// is deterministic.  A third kernel, beside the first fetch, writes each
// query's location codes in ascending row order (the order the attention
// walks, so that a request's queries meet their shared rows close together in
// time and re-read them from the L2).
#include "common.h"

#include <hip/hip_ext.h>

#include <algorithm>

namespace kvh {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
// a union row found nowhere on the device is held as -2 - row until it gets
// its staging position (every other code is >= 0)
__device__ __forceinline__ int32_t miss_mark(int row) { return -2 - row; }
constexpr int kBatch = 16;         // independent loads issued together

__host__ __device__ inline size_t align16(size_t x) { return (x + 15) & ~size_t(15); }

__host__ __device__ inline size_t region_a_bytes(int QK, int cw) {
  return align16(size_t(cw) * 4) + align16(size_t(cw) * 2) + align16(size_t(QK) * 4);
}

// Exclusive scan over the block of one int per thread; *total gets the sum.
__device__ int block_exclusive_scan(int v, int* scratch, int* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) scratch[wid] = x;
  __syncthreads();
  if (wid == 0) {
    int w = lane < kWaves ? scratch[lane] : 0;
    int ws = w;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      int y = __shfl_up(ws, d, 64);
      if (lane >= d) ws += y;
    }
    if (lane < kWaves) scratch[lane] = ws - w;
    if (lane == kWaves - 1) scratch[kWaves] = ws;
  }
  __syncthreads();
  const int res = scratch[wid] + x - v;
  *total = scratch[kWaves];
  __syncthreads();
  return res;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}

__global__ __launch_bounds__(kThreads) void plan_resolve_kernel(PlanArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int Q = a.Q, k = a.k, QK = Q * k, B = a.B, L = a.L;
  const int CW = a.chunk_words, CB = CW * 32;

  uint32_t* bitmap = reinterpret_cast<uint32_t*>(lds);
  uint16_t* wpre = reinterpret_cast<uint16_t*>(lds + align16(size_t(CW) * 4));
  int32_t* uloc = reinterpret_cast<int32_t*>(lds + align16(size_t(CW) * 4) + align16(size_t(CW) * 2));
  const size_t ra = region_a_bytes(QK, CW);
  const int pwords = (B + 31) / 32;
  uint32_t* protect = reinterpret_cast<uint32_t*>(lds + ra);
  int* scratch = reinterpret_cast<int*>(lds + ra + align16(size_t(pwords) * 4));
  int* cnt = scratch + 32;          // C_NUM counters

  const int32_t* cp = a.causal + size_t(r) * Q;
  const int32_t* tk = a.topk + size_t(r) * QK;
  int32_t* loc = a.loc + size_t(r) * QK;
  // this step's ring rows (nothing in the plan reads them: no barrier)
  if (a.ring_rows) {
    for (int i = tid; i < Q * a.row16; i += kThreads) {
      const int j = i / a.row16, c = i - j * a.row16;
      const int pos = cp[j];
      if (pos >= 0)
        a.ring[(size_t(r) * a.Rd + pos % a.Rd) * a.row16 + c] = a.ring_rows[(size_t(r) * Q + j) * a.row16 + c];
    }
  }
  const int n_raw = cp[0];
  if (n_raw < 0) {  // inactive request: no selections, nothing resolved
    for (int i = tid; i < QK; i += kThreads) loc[i] = -1;
    if (tid < I_NUM && tid != I_NPROMOTE) a.req_info[r * I_NUM + tid] = 0;   // the victim kernel sets I_NPROMOTE
    if (tid < C_NUM) a.req_counts[size_t(r) * C_NUM + tid] = 0;
    return;
  }
  // stored rows: complete groups of m positions (eq. 8)
  const int n_src = n_raw / a.m;
  const int n_r = n_src < L ? n_src : L;
  // the ring still holds positions >= tail_lo: this step's block (n_r ..
  // n_r+Q-1) takes the slots of the positions below (eq. 10).  A compressed
  // source's ring holds positions, not stored rows: no tail.
  const int tail_lo = a.m == 1 ? max(a.ring_lo[r], n_r + Q - a.Rd) : n_r;
  uint32_t amask = 0;
  for (int j = 0; j < Q; ++j) amask |= (cp[j] >= 0 ? 1u : 0u) << j;

  // When a thread's entries fit one batch (QK <= kBatch * kThreads, the usual
  // case) they are loaded once and held in registers through the marking and
  // location passes of every row chunk.
  const bool held = QK <= kBatch * kThreads;
  int hv[kBatch];
  if (held) {
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int i = tid + b * kThreads;
      hv[b] = i < QK ? tk[i] : -1;
    }
  }
  for (int w = tid; w < pwords; w += kThreads) protect[w] = 0;
  if (tid < 32) cnt[tid] = 0;
  for (int w = tid; w < CW; w += kThreads) bitmap[w] = 0;   // the first row chunk's bitmap
  // the zeroing is complete in every wave before any wave adds to the
  // counters, marks a slot or marks a row (also when the row loop below runs
  // no chunk)
  __syncthreads();

  int c_sel = 0, c_pad = 0, c_bad = 0, c_sres = 0, c_shot = 0, c_smiss = 0, c_stail = 0;
  int c_ures = 0, c_uhot = 0, c_umiss = 0, c_utail = 0;
  int union_base = 0, miss_base = 0;
  const int WPT = (CW + kThreads - 1) / kThreads;

  for (int c0 = 0; c0 < n_r; c0 += CB) {
    const int c1 = min(c0 + CB, n_r);
    if (c0 > 0) {
      for (int w = tid; w < CW; w += kThreads) bitmap[w] = 0;
      __syncthreads();
    }
    // mark the selections of this row chunk (loads issued kBatch at a time)
    for (int i0 = tid; i0 < QK; i0 += kBatch * kThreads) {
      int ev[kBatch];
      bool on[kBatch];
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int i = i0 + b * kThreads;
        on[b] = i < QK && ((amask >> (i / k)) & 1u);
        ev[b] = on[b] ? (held ? hv[b] : tk[i]) : -1;
      }
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        if (!on[b]) continue;                    // past the list or an inactive query
        const int e = ev[b];
        if (c0 == 0) {
          if (e == -1) ++c_pad;
          else if (e >= 0 && e < n_r) ++c_sel;
          else ++c_bad;
        }
        if (e >= c0 && e < c1) {
          const int o = e - c0;
          atomicOr(&bitmap[o >> 5], 1u << (o & 31));
        }
      }
    }
    __syncthreads();
    // compaction: each thread owns WPT consecutive words
    const int wb = tid * WPT, we = min(wb + WPT, CW);
    int mine = 0;
    for (int w = wb; w < we; ++w) mine += __popc(bitmap[w]);
    int chunk_union;
    const int ubase = block_exclusive_scan(mine, scratch, &chunk_union);
    // union rows of the chunk in ascending order, with the per-word rank table;
    // the rows also go to uloc, which the probe below reads and overwrites
    // with their codes
    int run = ubase;
    for (int w = wb; w < we; ++w) {
      wpre[w] = static_cast<uint16_t>(run);
      uint32_t bits = bitmap[w];
      while (bits) {
        const int b = __ffs(bits) - 1;
        bits &= bits - 1;
        const int row = c0 + w * 32 + b;
        a.union_rows[size_t(r) * QK + union_base + run] = row;
        uloc[run] = row;
        ++run;
      }
    }
    __syncthreads();
    // probe every union row (strided, so each thread's map loads are
    // independent): the tail and the resident map first, then the hot cache
    // (Figure 2)
    for (int x0 = tid; x0 < chunk_union; x0 += kBatch * kThreads) {
      int uv[kBatch], rmv[kBatch], smv[kBatch];
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int x = x0 + b * kThreads;
        uv[b] = x < chunk_union ? uloc[x] : -1;
      }
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        rmv[b] = a.has_resident && uv[b] >= 0 ? a.res_map[size_t(r) * L + uv[b]] : -1;
        smv[b] = uv[b] >= 0 ? a.slot_map[size_t(r) * L + uv[b]] : -1;
      }
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int x = x0 + b * kThreads;
        if (x >= chunk_union) continue;
        const int rm = rmv[b], sm = smv[b];
        if (sm >= 0) atomicOr(&protect[sm >> 5], 1u << (sm & 31));
        int code;
        if (uv[b] >= tail_lo) {
          code = make_loc(kTierRing, r * a.Rd + uv[b] % a.Rd);
          ++c_utail;
        } else if (rm >= 0) {
          code = make_loc(kTierResident, rm);
          ++c_ures;
        } else if (sm >= 0) {
          code = make_loc(kTierHot, r * B + sm);
          a.slot_lu[size_t(r) * B + sm] = a.t;
          ++c_uhot;
        } else {
          code = miss_mark(uv[b]);
          ++c_umiss;
        }
        uloc[x] = code;
      }
    }
    __syncthreads();
    // staging positions: misses in ascending row order (contiguous ranges of the union)
    const int upt = (chunk_union + kThreads - 1) / kThreads;
    const int xb = min(tid * upt, chunk_union), xe = min(xb + upt, chunk_union);
    int my_miss = 0;
    for (int x = xb; x < xe; ++x) my_miss += uloc[x] < 0;
    int chunk_miss;
    const int mbase = block_exclusive_scan(my_miss, scratch, &chunk_miss);
    int mi = miss_base + mbase;
    for (int x = xb; x < xe; ++x) {
      int code = uloc[x];
      if (code < 0) {
        a.miss_rows[size_t(r) * QK + mi] = -2 - code;
        code = make_loc(kTierStaged, r * QK + mi);
        uloc[x] = code;
        ++mi;
      }
      a.union_loc[size_t(r) * QK + union_base + x] = code;
    }
    __syncthreads();
    // one location per list entry, in selection order (eq. 12)
    for (int i0 = tid; i0 < QK; i0 += kBatch * kThreads) {
      int ev[kBatch];
#pragma unroll
      for (int q = 0; q < kBatch; ++q) ev[q] = i0 + q * kThreads < QK ? (held ? hv[q] : tk[i0 + q * kThreads]) : -1;
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        const int i = i0 + q * kThreads;
        if (i >= QK) continue;
        const bool act = (amask >> (i / k)) & 1u;
        const int e = ev[q];
        const bool valid = act && e >= 0 && e < n_r;
        if (c0 == 0 && !valid) loc[i] = -1;
        if (valid && e >= c0 && e < c1) {
          const int o = e - c0, w = o >> 5, b = o & 31;
          const int rank = wpre[w] + __popc(bitmap[w] & ((1u << b) - 1u));
          const int code = uloc[rank];
          loc[i] = code;
          const int tier = loc_tier(code);
          c_sres += tier == kTierResident;
          c_shot += tier == kTierHot;
          c_smiss += tier == kTierStaged;
          c_stail += tier == kTierRing;
        }
      }
    }
    union_base += chunk_union;
    miss_base += chunk_miss;
    __syncthreads();
  }
  if (n_r <= 0) {  // no history: every active entry is a pad or invalid
    for (int i = tid; i < QK; i += kThreads) {
      loc[i] = -1;
      if ((amask >> (i / k)) & 1u) {
        if (tk[i] == -1) ++c_pad;
        else ++c_bad;
      }
    }
  }

  // block totals of the per-thread counters: wave sums, one LDS atomic per wave
  {
    const int v[11] = {c_sel, c_pad, c_bad, c_sres, c_shot, c_smiss, c_ures, c_uhot, c_umiss, c_utail, c_stail};
    const int slot[11] = {C_SEL, C_PAD, C_INVALID, C_S_RES, C_S_HOT, C_S_MISS, C_U_RES, C_U_HOT, C_U_MISS,
                          C_U_TAIL, C_S_TAIL};
#pragma unroll
    for (int q = 0; q < 11; ++q) {
      const int tot = wave_sum(v[q]);
      if ((tid & 63) == 0 && tot) atomicAdd(&cnt[slot[q]], tot);
    }
  }

  // hits protect their slots from eviction: handed to the victim kernel
  for (int w = tid; w < pwords; w += kThreads) a.protect[size_t(r) * pwords + w] = protect[w];
  __syncthreads();
  if (tid == 0) {
    cnt[C_ACTIVE_REQ] = 1;
    cnt[C_ACTIVE_Q] = __popc(amask);
    cnt[C_UNION] = union_base;
    int32_t* info = a.req_info + r * I_NUM;
    info[I_NUNION] = union_base;
    info[I_NMISS] = miss_base;
    info[I_NACTIVE] = __popc(amask);
    info[I_NR] = n_r;
  }
  __syncthreads();
  // promoted / overflow are counted by the victim kernel
  if (tid < C_NUM && tid != C_PROMOTED && tid != C_OVERFLOW) {
    a.req_counts[size_t(r) * C_NUM + tid] = cnt[tid];
    if (cnt[tid]) atomicAdd(&a.cum[tid], static_cast<unsigned long long>(cnt[tid]));
  }
}

// LRU victims of one request: the i-th missing row (ascending) takes the i-th
// unprotected slot in (last_used, slot) order, empty slots first; the rest
// overflow.  Updates the slot tables and the row -> slot map.
__global__ __launch_bounds__(kThreads) void plan_victims_kernel(PlanArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int QK = a.Q * a.k, B = a.B, L = a.L;
  const int pwords = (B + 31) / 32;
  unsigned long long* keys = reinterpret_cast<unsigned long long*>(lds);
  uint32_t* protect = reinterpret_cast<uint32_t*>(lds + size_t(a.sort_cap) * 8);
  int* misc = reinterpret_cast<int*>(lds + size_t(a.sort_cap) * 8 + align16(size_t(pwords) * 4));
  const int n_miss = a.req_info[r * I_NUM + I_NMISS];
  int n_prom = 0;
  if (n_miss > 0) {
    for (int w = tid; w < pwords; w += kThreads) protect[w] = a.protect[size_t(r) * pwords + w];
    if (tid == 0) misc[0] = 0;
    __syncthreads();
    // unselected slots' keys, compacted with one LDS atomic per wave (the
    // order is fixed by the sort below)
    const int lane = tid & 63;
    for (int s0 = 0, ms = 0; s0 < B; s0 += kThreads, ++ms) {
      const int s = s0 + tid;
      bool take = false;
      unsigned long long key = 0;
      if (s < B && !((protect[s >> 5] >> (s & 31)) & 1u)) {
        const int row = a.slot_row[size_t(r) * B + s];
        const int lu = a.slot_lu[size_t(r) * B + s];
        const unsigned hi = row < 0 ? 0u : unsigned(lu) + 1u;
        key = (static_cast<unsigned long long>(hi) << 32) | unsigned(s);
        take = true;
      }
      const unsigned long long m = __builtin_amdgcn_ballot_w64(take);
      int base = 0;
      if (lane == 0 && m) base = atomicAdd(&misc[0], static_cast<int>(__popcll(m)));
      base = __shfl(base, 0, 64);
      if (take) keys[base + static_cast<int>(__popcll(m & ((1ull << lane) - 1ull)))] = key;
    }
    __syncthreads();
    const int n_unprot = misc[0];
    n_prom = min(n_miss, n_unprot);
    int sort_n = 1;
    while (sort_n < n_unprot) sort_n <<= 1;
    if (n_prom > 0) {
      for (int i = n_unprot + tid; i < sort_n; i += kThreads) keys[i] = ~0ull;
      __syncthreads();
      // bitonic network; a wave's 64 pairs of a stage with stride <= 64 lie in
      // its own 128 keys, so between two such stages the wave's own ordering
      // suffices; a workgroup barrier separates every other pair of stages
      for (int size = 2; size <= sort_n; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
          for (int i = tid; i < sort_n / 2; i += kThreads) {
            const int lo = 2 * stride * (i / stride) + (i % stride);
            const int hi = lo + stride;
            const bool asc = (lo & size) == 0;
            const unsigned long long x = keys[lo], y = keys[hi];
            if ((x > y) == asc) { keys[lo] = y; keys[hi] = x; }
          }
          const int next_stride = stride > 1 ? stride >> 1 : size;
          if (stride > 64 || next_stride > 64 || sort_n / 2 > kThreads || (stride == 1 && size == sort_n)) {
            __syncthreads();
          } else {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          }
        }
      }
      // the i-th missing row (ascending) takes the i-th victim
      for (int i = tid; i < n_prom; i += kThreads) {
        const int s = static_cast<int>(keys[i] & 0xffffffffull);
        const int old = a.slot_row[size_t(r) * B + s];
        if (old >= 0) a.slot_map[size_t(r) * L + old] = -1;
        const int nu = a.miss_rows[size_t(r) * QK + i];
        a.slot_row[size_t(r) * B + s] = nu;
        a.slot_lu[size_t(r) * B + s] = a.t;
        a.slot_map[size_t(r) * L + nu] = s;
        a.victims[size_t(r) * QK + i] = s;
      }
    }
  }
  if (tid == 0) {
    a.req_info[r * I_NUM + I_NPROMOTE] = n_prom;
    a.req_counts[size_t(r) * C_NUM + C_PROMOTED] = n_prom;
    a.req_counts[size_t(r) * C_NUM + C_OVERFLOW] = n_miss - n_prom;
    if (n_prom) atomicAdd(&a.cum[C_PROMOTED], static_cast<unsigned long long>(n_prom));
    if (n_miss - n_prom) atomicAdd(&a.cum[C_OVERFLOW], static_cast<unsigned long long>(n_miss - n_prom));
  }
}

// Row order of every query's list: the valid entries' location codes sorted
// by row id, then -1; a query that repeats a row keeps its selection order
// (each repeat is its own term, and distinct rows alone would drop it).  One
// 1024-thread workgroup per request.  Per row chunk (as in the resolution):
// the union bitmap and its word prefix table give each entry's rank in the
// union; each query marks its ranks in a bitmap of its own, whose prefix
// table places its rows; the codes (the union's, in rank order) go to an LDS
// staging copy of the request's lists, written out once, coalesced.
__global__ __launch_bounds__(kThreads) void plan_order_kernel(PlanArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int Q = a.Q, k = a.k, QK = Q * k, L = a.L;
  const int CW = a.chunk_words, CB = CW * 32;
  const int QW = (min(QK, CB) + 31) / 32;

  uint32_t* bitmap = reinterpret_cast<uint32_t*>(lds);
  uint16_t* wpre = reinterpret_cast<uint16_t*>(lds + align16(size_t(CW) * 4));
  int32_t* stage = reinterpret_cast<int32_t*>(lds + align16(size_t(CW) * 4) + align16(size_t(CW) * 2));
  unsigned char* q0 = lds + region_a_bytes(QK, CW);
  uint32_t* qbits = reinterpret_cast<uint32_t*>(q0);
  uint16_t* qpre = reinterpret_cast<uint16_t*>(q0 + align16(size_t(Q) * QW * 4));
  int* qbase = reinterpret_cast<int*>(q0 + align16(size_t(Q) * QW * 4) + align16(size_t(Q) * QW * 2));
  int* qcnt = qbase + Q;            // entries of the current chunk
  int* qflag = qcnt + Q;            // 1: the query repeats a row
  int* scratch = qflag + Q;         // block scan (kWaves + 1)

  const int32_t* cp = a.causal + size_t(r) * Q;
  const int32_t* tk = a.topk + size_t(r) * QK;
  const int32_t* loc = a.loc + size_t(r) * QK;
  const int32_t* uloc = a.union_loc + size_t(r) * QK;
  int32_t* sloc = a.sloc + size_t(r) * QK;
  const int n_raw = cp[0];
  if (n_raw < 0) {  // inactive request
    for (int i = tid; i < QK; i += kThreads) sloc[i] = -1;
    return;
  }
  const int n_src = n_raw / a.m;
  const int n_r = n_src < L ? n_src : L;
  uint32_t amask = 0;
  for (int j = 0; j < Q; ++j) amask |= (cp[j] >= 0 ? 1u : 0u) << j;
  const bool held = QK <= kBatch * kThreads;
  int hv[kBatch];
  if (held) {
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int i = tid + b * kThreads;
      hv[b] = i < QK ? tk[i] : -1;
    }
  }
  if (tid < Q) qbase[tid] = qflag[tid] = 0;
  const int WPT = (CW + kThreads - 1) / kThreads;
  int union_base = 0;
  for (int c0 = 0; c0 < n_r; c0 += CB) {
    const int c1 = min(c0 + CB, n_r);
    for (int w = tid; w < CW; w += kThreads) bitmap[w] = 0;
    if (tid < Q) qcnt[tid] = 0;
    __syncthreads();
    // the chunk's union: one bit per selected row
    for (int i0 = tid; i0 < QK; i0 += kBatch * kThreads) {
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int i = i0 + b * kThreads;
        if (i >= QK || !((amask >> (i / k)) & 1u)) continue;
        const int e = held ? hv[b] : tk[i];
        if (e >= c0 && e < c1) atomicOr(&bitmap[(e - c0) >> 5], 1u << ((e - c0) & 31));
      }
    }
    __syncthreads();
    // word prefix table: the rank of a row in the chunk's union
    const int wb = tid * WPT, we = min(wb + WPT, CW);
    int mine = 0;
    for (int w = wb; w < we; ++w) mine += __popc(bitmap[w]);
    int chunk_union;
    int run = block_exclusive_scan(mine, scratch, &chunk_union);
    for (int w = wb; w < we; ++w) {
      wpre[w] = static_cast<uint16_t>(run);
      run += __popc(bitmap[w]);
    }
    const int qw = (chunk_union + 31) / 32;
    for (int x = tid; x < Q * qw; x += kThreads) qbits[(x / qw) * QW + x % qw] = 0;
    __syncthreads();
    // each query's ranks, and its entries in the chunk (one ballot per wave
    // and batch when the wave's entries belong to one query)
    for (int i0 = tid; i0 < QK; i0 += kBatch * kThreads) {
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int i = i0 + b * kThreads;
        if (i >= QK) continue;
        const int j = i / k;
        const int e = held ? hv[b] : tk[i];
        const bool in = ((amask >> j) & 1u) && e >= c0 && e < c1;
        if (in) {
          const int o = e - c0, w = o >> 5;
          const int rank = wpre[w] + __popc(bitmap[w] & ((1u << (o & 31)) - 1u));
          atomicOr(&qbits[j * QW + (rank >> 5)], 1u << (rank & 31));
        }
        const int i_w = i - lane;
        const int j0 = i_w / k, j1 = min(i_w + 63, QK - 1) / k;
        if (j0 == j1) {
          const int n = __popcll(__builtin_amdgcn_ballot_w64(in));
          if (lane == 0 && n) atomicAdd(&qcnt[j0], n);
        } else if (in) {
          atomicAdd(&qcnt[j], 1);
        }
      }
    }
    __syncthreads();
    // each query's word prefix table (one wave per query); more entries than
    // distinct rows: a repeated row
    for (int j = wv; j < Q; j += kWaves) {
      int carry = 0;
      for (int w0 = 0; w0 < qw; w0 += 64) {
        const int w = w0 + lane;
        const int c = w < qw ? __popc(qbits[j * QW + w]) : 0;
        int x = c;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const int y = __shfl_up(x, d, 64);
          if (lane >= d) x += y;
        }
        if (w < qw) qpre[j * QW + w] = static_cast<uint16_t>(carry + x - c);
        carry += __shfl(x, 63, 64);
      }
      if (lane == 0) {
        if (qcnt[j] > carry) qflag[j] = 1;
        qcnt[j] = carry;           // the chunk's distinct rows of the query
      }
    }
    __syncthreads();
    // each query's rows of the chunk at its next positions in rank (= row)
    // order, codes from the union's list (rank order)
    for (int x = tid; x < Q * qw; x += kThreads) {
      const int j = x / qw, w = x - j * qw;
      uint32_t bits = qbits[j * QW + w];
      int32_t* dst = stage + j * k + qbase[j] + qpre[j * QW + w];
      const int32_t* src = uloc + union_base + w * 32;
      while (bits) {
        const int b = __ffs(bits) - 1;
        bits &= bits - 1;
        *dst++ = src[b];
      }
    }
    __syncthreads();
    if (tid < Q) qbase[tid] += qcnt[tid];
    union_base += chunk_union;
  }
  __syncthreads();
  for (int i = tid; i < QK; i += kThreads) {
    const int j = i / k;
    sloc[i] = qflag[j] ? loc[i] : (i - j * k < qbase[j] ? stage[i] : -1);
  }
}

}  // namespace

size_t plan_order_lds_bytes(int Q, int k, int chunk_words) {
  const int QW = (std::min(Q * k, chunk_words * 32) + 31) / 32;
  return region_a_bytes(Q * k, chunk_words) + align16(size_t(Q) * QW * 4) + align16(size_t(Q) * QW * 2) +
         size_t(Q) * 3 * 4 + size_t(kWaves + 1) * 4;
}

size_t plan_lds_bytes(int Q, int k, int B, int chunk_words, int sort_cap) {
  const int pwords = (B + 31) / 32;
  const size_t resolve = region_a_bytes(Q * k, chunk_words) + align16(size_t(pwords) * 4) + 128 * 4;
  const size_t victims = size_t(sort_cap) * 8 + align16(size_t(pwords) * 4) + 16;
  return resolve > victims ? resolve : victims;
}

hipError_t plan_init_attributes() {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(plan_resolve_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(plan_victims_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(plan_order_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  return e;
}

hipError_t launch_plan(const PlanArgs& a, size_t lds, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
  if (ev_start || ev_stop) {
    hipExtLaunchKernelGGL(plan_resolve_kernel, dim3(a.N), dim3(kThreads), uint32_t(lds), s, ev_start, ev_stop, 0, a);
  } else {
    hipLaunchKernelGGL(plan_resolve_kernel, dim3(a.N), dim3(kThreads), lds, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_plan_order(const PlanArgs& a, size_t lds, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
  if (ev_start || ev_stop) {
    hipExtLaunchKernelGGL(plan_order_kernel, dim3(a.N), dim3(kThreads), uint32_t(lds), s, ev_start, ev_stop, 0, a);
  } else {
    hipLaunchKernelGGL(plan_order_kernel, dim3(a.N), dim3(kThreads), lds, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_plan_victims(const PlanArgs& a, size_t lds, hipStream_t s) {
  hipLaunchKernelGGL(plan_victims_kernel, dim3(a.N), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

}  // namespace kvh
