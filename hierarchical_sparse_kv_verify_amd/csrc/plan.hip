// Resolution plan of one verification step, one 1024-thread workgroup per request.
//
// "Adaptive DHiSparse" (arXiv 2610.13708):
//  - §3.3 eq. (6): the retrieval union U_r of the K_r queries' selections and
//    the missing set D_r = U_r \ R_r; each distinct missing row is fetched once.
//  - §3.2 / Figure 2: probe order (1) ready optional-history map,
//    (2) hot cache, (3) host; locations emitted in selection order (eq. 12).
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
// LRU victims: the unselected slots' (last_used, slot) keys are compacted in
// LDS and bitonic-sorted; keys are unique, so the order is deterministic.
#include "common.h"

namespace kvh {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kMissMark = -2;

__host__ __device__ inline size_t align16(size_t x) { return (x + 15) & ~size_t(15); }

__host__ __device__ inline size_t region_a_bytes(int QK, int cw, int sort_cap) {
  size_t chunk = align16(size_t(cw) * 4) + align16(size_t(cw) * 2) + align16(size_t(QK) * 4);
  size_t sort = size_t(sort_cap) * 8;
  return align16(chunk > sort ? chunk : sort);
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

__global__ __launch_bounds__(kThreads) void plan_kernel(PlanArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int Q = a.Q, k = a.k, QK = Q * k, B = a.B, L = a.L;
  const int CW = a.chunk_words, CB = CW * 32;

  uint32_t* bitmap = reinterpret_cast<uint32_t*>(lds);
  uint16_t* wpre = reinterpret_cast<uint16_t*>(lds + align16(size_t(CW) * 4));
  int32_t* uloc = reinterpret_cast<int32_t*>(lds + align16(size_t(CW) * 4) + align16(size_t(CW) * 2));
  unsigned long long* keys = reinterpret_cast<unsigned long long*>(lds);
  const size_t ra = region_a_bytes(QK, CW, a.sort_cap);
  const int pwords = (B + 31) / 32;
  uint32_t* protect = reinterpret_cast<uint32_t*>(lds + ra);
  int* scratch = reinterpret_cast<int*>(lds + ra + align16(size_t(pwords) * 4));
  int* cnt = scratch + 32;          // C_NUM counters
  int* misc = cnt + 32;             // misc[0] = number of unprotected slots

  const int32_t* cp = a.causal + size_t(r) * Q;
  const int32_t* tk = a.topk + size_t(r) * QK;
  int32_t* loc = a.loc + size_t(r) * QK;
  const int n_raw = cp[0];
  if (n_raw < 0) {  // inactive request: no selections, nothing resolved
    for (int i = tid; i < QK; i += kThreads) loc[i] = -1;
    if (tid < I_NUM) a.req_info[r * I_NUM + tid] = 0;
    if (tid < C_NUM) a.req_counts[size_t(r) * C_NUM + tid] = 0;
    return;
  }
  const int n_r = n_raw < L ? n_raw : L;
  uint32_t amask = 0;
  for (int j = 0; j < Q; ++j) amask |= (cp[j] >= 0 ? 1u : 0u) << j;

  for (int w = tid; w < pwords; w += kThreads) protect[w] = 0;
  if (tid < 32) cnt[tid] = 0;
  if (tid == 0) misc[0] = 0;

  int c_sel = 0, c_pad = 0, c_bad = 0, c_sres = 0, c_shot = 0, c_smiss = 0;
  int c_ures = 0, c_uhot = 0, c_umiss = 0;
  int union_base = 0, miss_base = 0;
  const int WPT = (CW + kThreads - 1) / kThreads;

  for (int c0 = 0; c0 < n_r; c0 += CB) {
    const int c1 = min(c0 + CB, n_r);
    for (int w = tid; w < CW; w += kThreads) bitmap[w] = 0;
    __syncthreads();
    // mark the selections of this row chunk
    for (int i = tid; i < QK; i += kThreads) {
      if (!((amask >> (i / k)) & 1u)) continue;
      const int e = tk[i];
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
    __syncthreads();
    // compaction: each thread owns WPT consecutive words
    const int wb = tid * WPT, we = min(wb + WPT, CW);
    int mine = 0;
    for (int w = wb; w < we; ++w) mine += __popc(bitmap[w]);
    int chunk_union;
    const int ubase = block_exclusive_scan(mine, scratch, &chunk_union);
    // union rows in ascending order; probe resident map, then hot cache
    int run = ubase, my_miss = 0;
    for (int w = wb; w < we; ++w) {
      wpre[w] = static_cast<uint16_t>(run);
      uint32_t bits = bitmap[w];
      while (bits) {
        const int b = __ffs(bits) - 1;
        bits &= bits - 1;
        const int u = c0 + w * 32 + b;
        a.union_rows[size_t(r) * QK + union_base + run] = u;
        const int rm = a.res_map[size_t(r) * L + u];
        const int sm = a.slot_map[size_t(r) * L + u];
        if (sm >= 0) atomicOr(&protect[sm >> 5], 1u << (sm & 31));
        int code;
        if (rm >= 0) {
          code = make_loc(kTierResident, rm);
          ++c_ures;
        } else if (sm >= 0) {
          code = make_loc(kTierHot, r * B + sm);
          a.slot_lu[size_t(r) * B + sm] = a.t;
          ++c_uhot;
        } else {
          code = kMissMark;
          ++my_miss;
          ++c_umiss;
        }
        uloc[run] = code;
        ++run;
      }
    }
    int chunk_miss;
    const int mbase = block_exclusive_scan(my_miss, scratch, &chunk_miss);
    // staging positions: misses in ascending row order
    int mi = miss_base + mbase;
    for (int x = ubase; x < ubase + mine; ++x) {
      int code = uloc[x];
      if (code == kMissMark) {
        a.miss_rows[size_t(r) * QK + mi] = a.union_rows[size_t(r) * QK + union_base + x];
        code = make_loc(kTierStaged, r * QK + mi);
        uloc[x] = code;
        ++mi;
      }
      a.union_loc[size_t(r) * QK + union_base + x] = code;
    }
    __syncthreads();
    // one location per list entry, in selection order (eq. 12)
    for (int i = tid; i < QK; i += kThreads) {
      const bool act = (amask >> (i / k)) & 1u;
      const int e = tk[i];
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

  // block totals of the per-thread counters
  if (c_sel) atomicAdd(&cnt[C_SEL], c_sel);
  if (c_pad) atomicAdd(&cnt[C_PAD], c_pad);
  if (c_bad) atomicAdd(&cnt[C_INVALID], c_bad);
  if (c_sres) atomicAdd(&cnt[C_S_RES], c_sres);
  if (c_shot) atomicAdd(&cnt[C_S_HOT], c_shot);
  if (c_smiss) atomicAdd(&cnt[C_S_MISS], c_smiss);
  if (c_ures) atomicAdd(&cnt[C_U_RES], c_ures);
  if (c_uhot) atomicAdd(&cnt[C_U_HOT], c_uhot);
  if (c_umiss) atomicAdd(&cnt[C_U_MISS], c_umiss);

  // LRU victims among unselected slots, ordered by (last_used, slot), empty slots first
  for (int s = tid; s < B; s += kThreads) {
    if ((protect[s >> 5] >> (s & 31)) & 1u) continue;
    const int row = a.slot_row[size_t(r) * B + s];
    const unsigned hi = row < 0 ? 0u : unsigned(a.slot_lu[size_t(r) * B + s]) + 1u;
    const int pos = atomicAdd(&misc[0], 1);
    keys[pos] = (static_cast<unsigned long long>(hi) << 32) | unsigned(s);
  }
  __syncthreads();
  const int n_unprot = misc[0];
  const int n_miss = miss_base;
  const int n_prom = min(n_miss, n_unprot);
  int sort_n = 1;
  while (sort_n < n_unprot) sort_n <<= 1;
  if (n_prom > 0) {
    for (int i = n_unprot + tid; i < sort_n; i += kThreads) keys[i] = ~0ull;
    __syncthreads();
    for (int size = 2; size <= sort_n; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int i = tid; i < sort_n / 2; i += kThreads) {
          const int lo = 2 * stride * (i / stride) + (i % stride);
          const int hi = lo + stride;
          const bool asc = (lo & size) == 0;
          const unsigned long long x = keys[lo], y = keys[hi];
          if ((x > y) == asc) { keys[lo] = y; keys[hi] = x; }
        }
        __syncthreads();
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
  __syncthreads();
  if (tid == 0) {
    cnt[C_ACTIVE_REQ] = 1;
    cnt[C_ACTIVE_Q] = __popc(amask);
    cnt[C_UNION] = union_base;
    cnt[C_PROMOTED] = n_prom;
    cnt[C_OVERFLOW] = n_miss - n_prom;
    int32_t* info = a.req_info + r * I_NUM;
    info[I_NUNION] = union_base;
    info[I_NMISS] = n_miss;
    info[I_NPROMOTE] = n_prom;
    info[I_NACTIVE] = __popc(amask);
    info[I_NR] = n_r;
  }
  __syncthreads();
  if (tid < C_NUM) {
    a.req_counts[size_t(r) * C_NUM + tid] = cnt[tid];
    if (cnt[tid]) atomicAdd(&a.cum[tid], static_cast<unsigned long long>(cnt[tid]));
  }
}

}  // namespace

size_t plan_lds_bytes(int Q, int k, int B, int chunk_words, int sort_cap) {
  const int pwords = (B + 31) / 32;
  return region_a_bytes(Q * k, chunk_words, sort_cap) + align16(size_t(pwords) * 4) + 128 * 4;
}

hipError_t launch_plan(const PlanArgs& a, size_t lds, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(plan_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(plan_kernel, dim3(a.N), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

}  // namespace kvh
