// Row movement kernels of the verification step (gfx950).
//
//  - miss gather: each distinct missing row is read once from pinned host
//    memory (mapped into the GPU address space) and written to its staging
//    row ("Adaptive DHiSparse", §3.3 and Figure 3 callout 2; the pages'
//    resolver copies over a grid that scales with the batch, §3.2).  Reads
//    are whole 1152-byte (or 512-byte) rows split in 16-byte lanes, so every
//    PCIe read request covers full 64/128-byte lines; the host side of the
//    link measured the same rate for this pattern as for a bulk copy.
//  - promote: staged rows that took a victim slot are copied back to their
//    stable hot-cache address after the step's readers finish (§3.4).
//  - ring write: the new KV row of every active query goes to
//    phi(r, p) = r*R_d + (p mod R_d) (eq. 10; Figure 3 callout 4).
//  - commit: committed ring rows get their host copy (eq. 7 and the text
//    after eq. 8: host backup of committed rows follows verification).
//  - optional-history population and its publication in the resident map
//    (§3.1: reserve pages, copy their rows, publish after the copy).
// Loop bounds come from device-side counts, so no host round trip is needed
// between resolution and movement.
#include "common.h"

#include <hip/hip_ext.h>

namespace kvh {
namespace {

__device__ inline const uint4* host_row(const HostRowSrc& s, int r, int row) {
  if (row < s.prefix_len)
    return s.prefix[r % s.n_prefix] + size_t(row) * s.row16;
  return s.tails + (size_t(r) * s.tail_rows + (row - s.prefix_len)) * s.row16;
}

// One 16-byte chunk in flight per lane with 32-bit incremental (row, chunk)
// indices: the kernel needs few registers, so its waves fit on CUs that also
// run attention workgroups (a fetch that must wait for free CUs loses most of
// its host-link rate).  One wave per workgroup spreads the host reads thinly
// over many CUs: the attention workgroups sharing a CU with them slow down
// less than under a few CUs each holding four fetch waves.
__global__ __launch_bounds__(64) void miss_gather_kernel(HostRowSrc src, const int32_t* __restrict__ miss_rows,
                                                          const int32_t* __restrict__ req_info,
                                                          uint4* __restrict__ staging, int QK, int r0) {
  const int r = r0 + blockIdx.y;
  const int n = req_info[r * I_NUM + I_NMISS];
  const int row16 = src.row16;
  const int32_t* mr = miss_rows + size_t(r) * QK;
  uint4* dst = staging + size_t(r) * QK * row16;
  const int stride = gridDim.x * blockDim.x;
  const int drow = stride / row16, dc = stride - drow * row16;
  const int i0 = blockIdx.x * blockDim.x + threadIdx.x;
  int row = i0 / row16, c = i0 - row * row16;
  while (row < n) {
    dst[size_t(row) * row16 + c] = host_row(src, r, mr[row])[c];
    row += drow;
    c += dc;
    if (c >= row16) { c -= row16; ++row; }
  }
}

// Staged rows copied into their victim slots with the fetch's 32-bit
// incremental indices: the kernel stays within 16 VGPRs, so a promote wave and
// a fetch wave together fit beside two attention waves on one SIMD.  (Each
// attention wave holds 240 of the SIMD's 512 registers; with a wider promote
// wave, a CU whose SIMD already carries a fetch wave cannot take its attention
// workgroup until the promote ends, and the whole launch waits for it.)
__global__ __launch_bounds__(256) void promote_kernel(const uint4* __restrict__ staging,
                                                      const int32_t* __restrict__ victims,
                                                      const int32_t* __restrict__ req_info,
                                                      uint4* __restrict__ hot, int QK, int B, int row16, int r0) {
  const int r = r0 + blockIdx.y;
  const int n = req_info[r * I_NUM + I_NPROMOTE];
  const int32_t* vic = victims + size_t(r) * QK;
  const uint4* src = staging + size_t(r) * QK * row16;
  uint4* dst = hot + size_t(r) * B * row16;
  const int stride = gridDim.x * blockDim.x;
  const int drow = stride / row16, dc = stride - drow * row16;
  const int i0 = blockIdx.x * blockDim.x + threadIdx.x;
  int row = i0 / row16, c = i0 - row * row16;
  while (row < n) {
    dst[size_t(vic[row]) * row16 + c] = src[size_t(row) * row16 + c];
    row += drow;
    c += dc;
    if (c >= row16) { c -= row16; ++row; }
  }
}

__global__ __launch_bounds__(256) void ring_write_kernel(const uint4* __restrict__ rows,
                                                         const int32_t* __restrict__ causal,
                                                         uint4* __restrict__ ring, int N, int Q, int Rd, int row16) {
  const size_t total = size_t(N) * Q * row16;
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < total; i += stride) {
    const size_t rj = i / row16;
    const int c = static_cast<int>(i % row16);
    const int pos = causal[rj];
    if (pos < 0) continue;
    const size_t r = rj / Q;
    ring[(r * Rd + size_t(pos % Rd)) * row16 + c] = rows[i];
  }
}

__global__ __launch_bounds__(256) void host_rows_to_dev_kernel(HostRowSrc src, const int32_t* __restrict__ req,
                                                               const int32_t* __restrict__ rows,
                                                               const int64_t* __restrict__ dst_idx, int n,
                                                               uint4* __restrict__ dst) {
  const int row16 = src.row16;
  const size_t total = size_t(n) * row16;
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int x = static_cast<int>(i / row16), c = static_cast<int>(i % row16);
    dst[size_t(dst_idx[x]) * row16 + c] = host_row(src, req[x], rows[x])[c];
  }
}

__global__ __launch_bounds__(256) void commit_kernel(const CommitGroup* __restrict__ groups,
                                                     const int32_t* __restrict__ nbefore,
                                                     const int32_t* __restrict__ acc,
                                                     const uint4* const* __restrict__ src, int compressed,
                                                     int Qmax, int Rd, int prefix_len, int tail_rows, int row16) {
  const int r = blockIdx.y, g = blockIdx.z;
  const int a = acc[r];
  const int m = groups[g].m;
  if (a < 0 || (m > 1) != (compressed != 0)) return;
  const int n0 = nbefore[r];
  uint4* tails = groups[g].tails;
  if (m == 1) {
    const int total = (a + 1) * row16;
    const uint4* ring = groups[g].ring;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < total; i += gridDim.x * blockDim.x) {
      const int d = i / row16, c = i % row16;
      const int pos = n0 + d;
      tails[(size_t(r) * tail_rows + (pos - prefix_len)) * row16 + c] =
          ring[(size_t(r) * Rd + size_t(pos % Rd)) * row16 + c];
    }
  } else {
    // eq. (8): the stored rows completed by the new frontier
    const int s0 = n0 / m, s1 = (n0 + a + 1) / m;
    const int total = (s1 - s0) * row16;
    const uint4* rows = src[g] + size_t(r) * groups[g].cmax * row16;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < total; i += gridDim.x * blockDim.x) {
      const int d = i / row16, c = i % row16;
      tails[(size_t(r) * tail_rows + (s0 + d - prefix_len)) * row16 + c] = rows[size_t(d) * row16 + c];
    }
  }
  // no fence: later readers of these host rows are kernels ordered after this
  // one by stream events (its completion makes the writes visible) or the host
  // after a synchronisation
}

__global__ __launch_bounds__(256) void read_rows_kernel(PoolView pv, const int32_t* __restrict__ locs, int n,
                                                        uint4* __restrict__ dst, int row16) {
  const size_t total = size_t(n) * row16;
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int x = static_cast<int>(i / row16), c = static_cast<int>(i % row16);
    const int code = locs[x];
    uint4 v = make_uint4(0, 0, 0, 0);
    if (code >= 0) {
      const int tier = loc_tier(code);
      const size_t idx = size_t(loc_index(code));
      const uint4* base = tier == kTierHot ? pv.hot : tier == kTierStaged ? pv.staging
                          : tier == kTierResident ? pv.resident : pv.ring;
      if (base) v = base[idx * row16 + c];
    }
    dst[i] = v;
  }
}

// A follower layer's counters: the leader's last-step per-request counts,
// copied and added to the follower's cumulative counters.
__global__ __launch_bounds__(256) void counts_follow_kernel(const int64_t* __restrict__ src, int64_t* __restrict__ dst,
                                                            unsigned long long* __restrict__ cum, int N) {
  for (int c = 0; c < C_NUM; ++c) {
    int64_t part = 0;
    for (int r = threadIdx.x; r < N; r += blockDim.x) {
      const int64_t v = src[size_t(r) * C_NUM + c];
      dst[size_t(r) * C_NUM + c] = v;
      part += v;
    }
    if (part) atomicAdd(&cum[c], static_cast<unsigned long long>(part));
  }
}

// Population of optional history ("Adaptive DHiSparse" §3.1): the rows of
// each listed page, for every group, from pinned host memory into the group's
// pool page.  Flattened over (page, group, row, 16-byte chunk) so consecutive
// lanes read consecutive chunks of one host row; one-wave workgroups, as for
// the miss fetch, keep the reads spread thinly beside concurrent steps.
__global__ __launch_bounds__(64) void opt_copy_kernel(const OptGroup* __restrict__ groups,
                                                      const int32_t* __restrict__ list, int n, int G, int P,
                                                      int row16) {
  const size_t per_page = size_t(P) * row16;
  const size_t total = size_t(n) * G * per_page;
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < total; i += stride) {
    const size_t eg = i / per_page;
    const int w = static_cast<int>(i - eg * per_page);
    const int e = static_cast<int>(eg / G), g = static_cast<int>(eg - size_t(e) * G);
    const int row = w / row16, c = w - row * row16;
    const int r = list[3 * e], idx = list[3 * e + 1], page = list[3 * e + 2];
    const OptGroup& og = groups[g];
    og.pool[(size_t(page) * P + row) * row16 + c] = host_row(og.src, r, idx * P + row)[c];
  }
}

// Publication (or withdrawal) of listed pages in every group's resident map.
__global__ __launch_bounds__(256) void opt_map_kernel(const OptGroup* __restrict__ groups,
                                                     const int32_t* __restrict__ list, int n, int G, int P, int L,
                                                     int publish) {
  const size_t total = size_t(n) * G * P;
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < total; i += stride) {
    const size_t eg = i / P;
    const int row = static_cast<int>(i - eg * P);
    const int e = static_cast<int>(eg / G), g = static_cast<int>(eg - size_t(e) * G);
    const int r = list[3 * e], idx = list[3 * e + 1], page = list[3 * e + 2];
    groups[g].res_map[size_t(r) * L + size_t(idx) * P + row] = publish ? page * P + row : -1;
  }
}

__global__ __launch_bounds__(256) void fill32_kernel(uint32_t* p, uint32_t v, size_t n) {
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = v;
}

inline unsigned grid_for(size_t work, unsigned cap) {
  size_t g = (work + 255) / 256;
  if (g < 1) g = 1;
  return static_cast<unsigned>(g < cap ? g : cap);
}

}  // namespace

hipError_t launch_miss_gather(const HostRowSrc& src, const int32_t* miss_rows, const int32_t* req_info,
                              uint4* staging, int QK, int r0, int r1, int wg_per_req, hipStream_t s,
                              hipEvent_t ev_start, hipEvent_t ev_stop) {
  if (r1 <= r0) {
    // nothing to launch: the events still mark this point of the stream
    if (ev_start) (void)hipEventRecord(ev_start, s);
    if (ev_stop) return hipEventRecord(ev_stop, s);
    return hipSuccess;
  }
  if (ev_start || ev_stop) {
    hipExtLaunchKernelGGL(miss_gather_kernel, dim3(wg_per_req, r1 - r0), dim3(64), 0, s, ev_start, ev_stop, 0, src,
                          miss_rows, req_info, staging, QK, r0);
  } else {
    hipLaunchKernelGGL(miss_gather_kernel, dim3(wg_per_req, r1 - r0), dim3(64), 0, s, src, miss_rows, req_info,
                       staging, QK, r0);
  }
  return hipGetLastError();
}

hipError_t launch_promote(const uint4* staging, const int32_t* victims, const int32_t* req_info, uint4* hot,
                          int QK, int B, int row16, int r0, int r1, hipStream_t s) {
  if (r1 <= r0) return hipSuccess;
  hipLaunchKernelGGL(promote_kernel, dim3(4, r1 - r0), dim3(256), 0, s, staging, victims, req_info, hot, QK,
                     B, row16, r0);
  return hipGetLastError();
}

hipError_t launch_ring_write(const uint4* rows, const int32_t* causal, uint4* ring, int N, int Q, int Rd,
                             int row16, hipStream_t s) {
  const size_t work = size_t(N) * Q * row16;
  hipLaunchKernelGGL(ring_write_kernel, dim3(grid_for(work, 2048)), dim3(256), 0, s, rows, causal, ring, N, Q,
                     Rd, row16);
  return hipGetLastError();
}

hipError_t launch_host_rows_to_dev(const HostRowSrc& src, const int32_t* req, const int32_t* rows,
                                   const int64_t* dst_idx, int n, uint4* dst, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(host_rows_to_dev_kernel, dim3(grid_for(size_t(n) * src.row16, 128)), dim3(256), 0, s,
                     src, req, rows, dst_idx, n, dst);
  return hipGetLastError();
}

hipError_t launch_commit(const CommitGroup* groups, int G, const int32_t* nbefore, const int32_t* acc,
                         const uint4* const* src, int compressed, int N, int Qmax, int Rd, int prefix_len,
                         int tail_rows, int row16, hipStream_t s) {
  // one workgroup per (request, group): at most K_max rows of row16 chunks each
  hipLaunchKernelGGL(commit_kernel, dim3(1, N, G), dim3(256), 0, s, groups, nbefore, acc, src, compressed, Qmax,
                     Rd, prefix_len, tail_rows, row16);
  return hipGetLastError();
}

hipError_t launch_read_rows(const PoolView& pv, const int32_t* locs, int n, uint4* dst, int row16,
                            hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(read_rows_kernel, dim3(grid_for(size_t(n) * row16, 1024)), dim3(256), 0, s, pv, locs, n,
                     dst, row16);
  return hipGetLastError();
}

hipError_t launch_counts_follow(const int64_t* src, int64_t* dst, unsigned long long* cum, int N, hipStream_t s) {
  hipLaunchKernelGGL(counts_follow_kernel, dim3(1), dim3(256), 0, s, src, dst, cum, N);
  return hipGetLastError();
}

hipError_t launch_opt_copy(const OptGroup* groups, int G, const int32_t* list, int n, int P, int row16, int wgs,
                           hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const size_t work = size_t(n) * G * P * row16;
  size_t grid = (work + 63) / 64;
  if (grid > size_t(wgs)) grid = size_t(wgs);
  hipLaunchKernelGGL(opt_copy_kernel, dim3(static_cast<unsigned>(grid)), dim3(64), 0, s, groups, list, n, G, P,
                     row16);
  return hipGetLastError();
}

hipError_t launch_opt_map(const OptGroup* groups, int G, const int32_t* list, int n, int P, int L, int publish,
                          hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(opt_map_kernel, dim3(grid_for(size_t(n) * G * P, 1024)), dim3(256), 0, s, groups, list, n, G,
                     P, L, publish);
  return hipGetLastError();
}

hipError_t launch_fill32(uint32_t* p, uint32_t v, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fill32_kernel, dim3(grid_for(n, 4096)), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}

}  // namespace kvh
