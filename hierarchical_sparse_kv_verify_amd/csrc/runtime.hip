// Host runtime of libkvhier.so: the C ABI declared in include/kv_hier.h.
//
// One handle holds, per layer group (payload source), the hot caches, slot
// tables, row->slot and row->resident maps, the draft ring and the pinned host
// backing, plus chi staging arenas shared by all groups ("Adaptive
// DHiSparse", §3.4: arenas are reused across layer groups once readers and
// copy-back finish).  A step runs on three streams ordered by events:
//  - side stream (after the caller's prior work): resolution plan, the host
//    fetch of each request chunk, then the LRU victim choice (only the
//    copy-back and the group's next plan, on this same stream, need it);
//  - caller's stream: ring write (beside the plan), then per chunk the
//    attention once the chunk's fetch is done;
//  - copy-back stream: promotion of staged rows into their victim slots
//    (slots no list of the step names, so it need not wait for the
//    attention).
// The fetch of chunk c+1 overlaps the attention of chunk c; an arena chunk is
// released once both its attention and its copy-back are done; the group's
// next attention waits for this step's copy-backs.
// No host synchronisation happens inside a step.
//
// Dynamic optional residency (§3.1, eqs. 3-4) keeps its bookkeeping on the
// host: admission, reclaim and round-robin population are host decisions; the
// page copies run on a fourth stream beside the steps, and the resident maps
// change only through small map kernels on the side stream, so every plan
// sees the maps as of its own place in that stream.  A page is published
// once its copy's event has completed (checked without waiting at the first
// group's step); a reclaimed page is withdrawn at once and rewritten only
// after the attention of every earlier step.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <deque>
#include <mutex>
#include <set>
#include <string>
#include <new>
#include <vector>

#include "common.h"
#include "kv_hier.h"

using namespace kvh;

namespace {

constexpr int kCommitBufs = 4;

// Scratch of kv_hier_verify_step_static: the split-key partial numerators and
// (max, sum) pairs of its attention launches, in a file-scope device array
// instead of memory the handle allocated, for callers that cannot allocate.
// Every GPU the library runs on holds its own copy until the process ends; in
// host code the array's name is not a device address, so every use goes
// through the address hipGetSymbolAddress returns on that device
// (scratch_on_device).
constexpr size_t kStaticScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

// Device address of `scratch` on the current device, looked up once per device
// (at handle creation) and kept; nullptr on failure.
unsigned char* scratch_on_device(int device, hipError_t* err) {
  static std::mutex mu;
  static std::vector<unsigned char*> addr;
  std::lock_guard<std::mutex> lock(mu);
  *err = hipSuccess;
  if (device < 0) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  if (size_t(device) >= addr.size()) addr.resize(size_t(device) + 1, nullptr);
  if (!addr[device]) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    addr[device] = static_cast<unsigned char*>(p);
  }
  return addr[device];
}

enum TimedKind { K_RING = 0, K_PLAN, K_GATHER, K_ATTN, K_COMBINE, K_PROMOTE, K_VICTIMS, K_ORDER, K_NUM };

struct Group {
  int leader = 0;                   // group whose plan this group uses (itself unless a follower)
  int member = 0;                   // index within its plan-sharing set (0 = the leader)
  uint16_t* hot = nullptr;
  int32_t* slot_row = nullptr;
  int32_t* slot_lu = nullptr;
  int32_t* slot_map = nullptr;
  int32_t* res_map = nullptr;
  uint16_t* resident = nullptr;
  int64_t res_cursor = 0;
  std::vector<char> res_set;
  uint16_t* ring = nullptr;
  int32_t* ring_lo = nullptr;
  int32_t *union_rows = nullptr, *union_loc = nullptr, *miss_rows = nullptr, *victims = nullptr;
  int32_t *loc = nullptr, *req_info = nullptr;
  int32_t* sloc = nullptr;          // the codes in each query's row order (row_order handles)
  uint32_t* protect = nullptr;      // [N][ceil(B/32)] slots protected by this step's hits
  hipEvent_t ev_done = nullptr;     // copy-backs of the group's last step finished
  bool done_recorded = false;
  hipEvent_t ev_sel = nullptr;      // the group's last step wrote its ring rows and ran its attention
  bool sel_recorded = false;
  bool sel_valid = false;           // this step's selection may be reused (until commit)
  bool map_wait = false;            // the resident maps changed on the side stream since its last plan
  int m = 1;                        // positions per stored row (compressed source when > 1)
  int64_t* req_counts = nullptr;
  unsigned long long* cum = nullptr;
  std::vector<void*> prefix_host;
  void* tails_host = nullptr;
  const uint4** prefix_table = nullptr;   // device array of host-mapped prefix bases
  const uint4* tails_dev = nullptr;       // host-mapped tails
  int t = 0;
  int64_t calls = 0;
  // cache-state snapshot (kv_hier_cache_snapshot)
  uint16_t* snap_hot = nullptr;
  int32_t *snap_row = nullptr, *snap_lu = nullptr, *snap_map = nullptr;
  int snap_t = -1;
  double ms[K_NUM] = {0};
  int64_t nt[K_NUM] = {0};
};

struct Timed {
  int kind, g;
  hipEvent_t a, b;
};

// pinned host page list handed to a stream (reusable once its event completes)
struct ListBuf {
  int32_t* host = nullptr;
  size_t cap = 0;
  hipEvent_t ev = nullptr;
  bool busy = false;
};

enum PageState : char { PG_FREE = 0, PG_PENDING = 1, PG_READY = 2 };

// Host bookkeeping of dynamic optional residency (one per handle: a page index
// addresses the same page in every group's pool).
struct Opt {
  bool on = false;
  int P = 0, M = 0, reserve = 0, cursor = 0;
  int64_t sum_req = 0, sum_held = 0, n_published = 0;
  std::vector<char> admitted;
  std::vector<int32_t> required, eligible, n_held, n_ready;
  std::vector<std::vector<int32_t>> held;     // [r][page index] -> pool page (pages fill ascending)
  std::vector<char> state, needs_wait;        // per pool page
  std::vector<uint32_t> gen;                  // per pool page: bumped at every reservation
  std::set<int32_t> free;                     // lowest first
  struct Batch {
    hipEvent_t ev;
    std::vector<int32_t> ent;                 // (request, page index, pool page, gen) per page
  };
  std::deque<Batch> pending;
  hipStream_t stream = nullptr;               // population copies
  hipEvent_t ev_unpub = nullptr;              // last withdrawal from the maps (side stream)
  bool unpub_recorded = false;
  int32_t* d_list_side = nullptr;             // page lists on the device, one per stream
  int32_t* d_list_copy = nullptr;
  OptGroup* d_groups = nullptr;
  std::vector<ListBuf> bufs;
  std::vector<hipEvent_t> ev_pool;
  int64_t pages_populated = 0, pages_published = 0, pages_reclaimed = 0, requests_reclaimed = 0,
          admissions_waited = 0, bytes_populated = 0;
};

}  // namespace

struct kv_hier {
  kv_hier_config cfg{};
  int device = 0;
  int Rd = 0, QK = 0, row16 = 0, plen = 0, n_prefix = 0, tail_rows = 0, L = 0;
  size_t row_bytes = 0;
  std::vector<Group> grp;
  std::vector<uint16_t*> arena;
  float* part_o = nullptr;
  uint16_t* zero_row = nullptr;   // one all-zero row: target of masked attention reads
  float* part_ml = nullptr;
  size_t step_part_heads = 0;       // split-key partial slots (blocks x heads per block) of the largest chunk launch of a step
  unsigned char* scratch_dev = nullptr;   // this device's copy of the static scratch array
  bool no_alloc_call = false;       // inside kv_hier_verify_step_static: take no events, allocate nothing
  int splits = 1, head_groups = 1, n_chunks = 1;   // the largest of chunk_splits / of the chunks' head groups
  // key splits and heads per workgroup of one launch over every request (Reuse layers)
  int all_splits = 1, all_hpw = 64;
  std::vector<int> chunk_lo, chunk_splits, chunk_hpw;
  int chunk_words = 0, sort_cap = 1;
  bool row_order = false;           // the order kernel writes row-ordered lists, which the attention walks
  size_t order_lds = 0;
  size_t plan_lds = 0;
  hipStream_t side = nullptr;       // host fetch
  hipStream_t work = nullptr;       // the rest of the step when CUs are partitioned (else null)
  hipStream_t aux = nullptr;        // copy-back of promoted rows
  hipEvent_t ev_planned = nullptr;  // the last plan is complete (its launch's own end)
  hipEvent_t ev_map = nullptr;      // last resident-map update on the side stream
  hipEvent_t ev_in = nullptr, ev_out = nullptr;
  int share = 1;                    // groups per plan-sharing set (leader + followers)
  std::vector<std::vector<hipEvent_t>> ev_fetched;   // [set member][chunk]
  std::vector<hipEvent_t> ev_free;  // [arena]: the arena's last readers are done (every chunk at once)
  std::vector<char> free_recorded;
  std::vector<int> arena_owner;     // group whose payload the arena holds (-1 none)
  std::vector<int> arena_step;      // that group's step counter when it was fetched
  std::vector<int32_t> hist_len;
  int32_t* d_commit = nullptr;
  const uint4** d_src = nullptr;    // per group: the caller's completed stored rows of a commit
  // pinned staging of a commit's frontiers, acceptances and row pointers: a
  // ring of kCommitBufs buffers, each reused once the copy that read it is done
  // (the host waits only when that many commits are still ahead of the GPU)
  int32_t* h_commit[kCommitBufs] = {};
  const uint4** h_src[kCommitBufs] = {};
  hipEvent_t ev_commit[kCommitBufs] = {};
  bool commit_pending[kCommitBufs] = {};
  // split-key partials (part_o / part_ml) are one buffer for every launch of
  // the handle: each launch that uses them waits for the previous one
  hipEvent_t ev_part = nullptr;
  bool part_recorded = false;
  // a call failed after it had started to change device state: every later
  // call that changes state is refused (KV_ESTATE)
  bool began = false;
  bool broken = false;
  std::string broken_msg;
  // host backup of committed rows (eq. 7) on its own stream, after verification
  hipStream_t backup = nullptr;     // the copy-back stream, or null: backups run on the caller's stream
  hipEvent_t ev_verified = nullptr; // the step's ring rows are written (caller's stream)
  hipEvent_t ev_backup[2] = {nullptr, nullptr};
  int64_t n_commits = 0;
  CommitGroup* d_commit_groups = nullptr;
  std::vector<Timed> pending;
  std::vector<hipEvent_t> pool;
  Opt opt;
  std::string err;
  int64_t bytes_hot = 0, bytes_staging = 0, bytes_ring = 0, bytes_maps = 0, bytes_res = 0, bytes_host = 0;
};

// Entry points run on the handle's device (its memory, streams and events
// belong to the device that was current at create); the caller's current
// device is restored on return.
struct DeviceGuard {
  int prev = -1;
  explicit DeviceGuard(const kv_hier* h) {
    int cur = -1;
    if (h && hipGetDevice(&cur) == hipSuccess && cur != h->device && hipSetDevice(h->device) == hipSuccess)
      prev = cur;
  }
  ~DeviceGuard() {
    if (prev >= 0) (void)hipSetDevice(prev);
  }
  DeviceGuard(const DeviceGuard&) = delete;
  DeviceGuard& operator=(const DeviceGuard&) = delete;
};

namespace {

int fail(kv_hier* h, int code, const char* fmt, ...) {
  if (h) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    h->err = buf;
  }
  return code;
}

#define HIPCHK(h, call)                                                                          \
  do {                                                                                           \
    hipError_t e_ = (call);                                                                      \
    if (e_ != hipSuccess) return fail((h), KV_EHIP, "%s failed: %s", #call, hipGetErrorString(e_)); \
  } while (0)

template <class T>
int dev_alloc(kv_hier* h, T** p, size_t count, int64_t* acct) {
  *p = nullptr;
  if (count == 0) return KV_OK;
  void* v = nullptr;
  if (hipMalloc(&v, count * sizeof(T)) != hipSuccess) {
    (void)hipGetLastError();
    return fail(h, KV_ENOMEM, "hipMalloc of %zu bytes failed", count * sizeof(T));
  }
  *p = static_cast<T*>(v);
  if (acct) *acct += int64_t(count * sizeof(T));
  return KV_OK;
}

int host_alloc(kv_hier* h, void** p, size_t bytes) {
  *p = nullptr;
  if (bytes == 0) return KV_OK;
  if (hipHostMalloc(p, bytes, hipHostMallocDefault) != hipSuccess) {
    (void)hipGetLastError();
    *p = nullptr;
    return fail(h, KV_ENOMEM, "hipHostMalloc of %zu bytes failed", bytes);
  }
  h->bytes_host += int64_t(bytes);
  return KV_OK;
}

HostRowSrc host_src(const kv_hier* h, const Group& G) {
  HostRowSrc s;
  s.prefix = G.prefix_table;
  s.tails = G.tails_dev;
  s.n_prefix = h->n_prefix > 0 ? h->n_prefix : 1;
  s.prefix_len = h->plen;
  s.tail_rows = h->tail_rows;
  s.row16 = h->row16;
  return s;
}

hipEvent_t take_event(kv_hier* h) {
  if (!h->pool.empty()) {
    hipEvent_t e = h->pool.back();
    h->pool.pop_back();
    return e;
  }
  // timing events serve hipEventElapsedTime only (read after a device-wide
  // synchronisation): without the system-scope fence a launch-bound pair adds
  // about 1 us to its launch instead of about 4
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

// Records a start event when timing is on; returns the pending index or -1.
int time_begin(kv_hier* h, int kind, int g, hipStream_t s) {
  if (h->no_alloc_call) return -1;   // the pool may have to create events
  const bool on = (h->cfg.flags & KV_FLAG_TIMING) ||
                  ((h->cfg.flags & KV_FLAG_TIMING_ATTN) && (kind == K_ATTN || kind == K_COMBINE));
  if (!on) return -1;
  Timed t{kind, g, take_event(h), take_event(h)};
  if (!t.a || !t.b || hipEventRecord(t.a, s) != hipSuccess) return -1;
  h->pending.push_back(t);
  return int(h->pending.size()) - 1;
}

void time_end(kv_hier* h, int idx, hipStream_t s) {
  if (idx < 0) return;
  (void)hipEventRecord(h->pending[idx].b, s);
}

// Events bound to one launch (hipExtLaunchKernel): with timing on, the pair
// that times the launch itself (no markers around it) and `done` to be
// recorded after it; else `done` itself is the launch's end event.
struct LaunchEv {
  hipEvent_t start = nullptr, stop = nullptr, after = nullptr;
};
LaunchEv launch_events(kv_hier* h, int kind, int g, hipEvent_t done) {
  LaunchEv le;
  le.stop = done;
  const bool on = !h->no_alloc_call &&
                  ((h->cfg.flags & KV_FLAG_TIMING) ||
                   ((h->cfg.flags & KV_FLAG_TIMING_ATTN) && (kind == K_ATTN || kind == K_COMBINE)));
  if (!on) return le;
  Timed t{kind, g, take_event(h), take_event(h)};
  if (!t.a || !t.b) {
    if (t.a) h->pool.push_back(t.a);
    if (t.b) h->pool.push_back(t.b);
    return le;
  }
  h->pending.push_back(t);
  le.start = t.a;
  le.stop = t.b;
  le.after = done;
  return le;
}

int drain_timing(kv_hier* h) {
  for (const Timed& t : h->pending) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, t.a, t.b) == hipSuccess) {
      h->grp[t.g].ms[t.kind] += ms;
      h->grp[t.g].nt[t.kind] += 1;
    } else {
      (void)hipGetLastError();
    }
    h->pool.push_back(t.a);
    h->pool.push_back(t.b);
  }
  h->pending.clear();
  return KV_OK;
}

int sync_all(kv_hier* h) {
  HIPCHK(h, hipDeviceSynchronize());
  return drain_timing(h);
}

int check_group(kv_hier* h, int g) {
  if (!h) return KV_EINVAL;
  if (g < 0 || g >= h->cfg.n_groups) return fail(h, KV_EINVAL, "group %d outside [0, %d)", g, h->cfg.n_groups);
  return KV_OK;
}

int check_req(kv_hier* h, int r) {
  if (r < 0 || r >= h->cfg.n_req) return fail(h, KV_EINVAL, "request %d outside [0, %d)", r, h->cfg.n_req);
  return KV_OK;
}

// A call that changes state marks the point where its checks end and its
// device work (or bookkeeping that must match the device) begins; an error
// after that point leaves the handle inconsistent, so the handle is latched
// and every later state-changing call returns KV_ESTATE.
void begin_work(kv_hier* h) { h->began = true; }

int refuse_if_broken(kv_hier* h) {
  if (h && h->broken) return fail(h, KV_ESTATE, "handle unusable after a failed call: %s", h->broken_msg.c_str());
  return KV_OK;
}

int finish(kv_hier* h, int rc) {
  if (!h) return rc;
  if (rc != KV_OK && h->began && !h->broken) {
    h->broken = true;
    h->broken_msg = h->err;
  }
  h->began = false;
  return rc;
}


int upload(kv_hier* h, void* dst, const void* src, size_t bytes) {
  if (bytes == 0) return KV_OK;
  HIPCHK(h, hipMemcpy(dst, src, bytes, hipMemcpyHostToDevice));
  return KV_OK;
}

int download(kv_hier* h, void* dst, const void* src, size_t bytes) {
  if (bytes == 0) return KV_OK;
  HIPCHK(h, hipMemcpy(dst, src, bytes, hipMemcpyDeviceToHost));
  return KV_OK;
}

// Scatters values into an int32 device array: base[idx[i]] = val[i] (set-up path).
__global__ void scatter32_kernel(int32_t* base, const int64_t* idx, const int32_t* val, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) base[idx[i]] = val[i];
}

int scatter32(kv_hier* h, int32_t* base, const std::vector<int64_t>& idx, const std::vector<int32_t>& val) {
  const int n = int(idx.size());
  if (n == 0) return KV_OK;
  int64_t* di = nullptr;
  int32_t* dv = nullptr;
  int rc = dev_alloc(h, &di, size_t(n), nullptr);
  if (rc) return rc;
  rc = dev_alloc(h, &dv, size_t(n), nullptr);
  if (rc) { (void)hipFree(di); return rc; }
  rc = upload(h, di, idx.data(), size_t(n) * 8);
  if (!rc) rc = upload(h, dv, val.data(), size_t(n) * 4);
  if (!rc) {
    hipLaunchKernelGGL(scatter32_kernel, dim3(std::min(1024, (n + 255) / 256)), dim3(256), 0, nullptr, base, di,
                       dv, n);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) rc = fail(h, KV_EHIP, "scatter: %s", hipGetErrorString(e));
  }
  (void)hipFree(di);
  (void)hipFree(dv);
  return rc;
}

// Copies host-backing rows (req[i], rows[i]) to dst rows dst_idx[i] (set-up path).
int rows_from_host(kv_hier* h, const Group& G, const std::vector<int32_t>& req, const std::vector<int32_t>& rows,
                   const std::vector<int64_t>& dst_idx, uint16_t* dst) {
  const int n = int(rows.size());
  if (n == 0) return KV_OK;
  int32_t *dq = nullptr, *dr = nullptr;
  int64_t* di = nullptr;
  int rc = dev_alloc(h, &dq, size_t(n), nullptr);
  if (!rc) rc = dev_alloc(h, &dr, size_t(n), nullptr);
  if (!rc) rc = dev_alloc(h, &di, size_t(n), nullptr);
  if (!rc) rc = upload(h, dq, req.data(), size_t(n) * 4);
  if (!rc) rc = upload(h, dr, rows.data(), size_t(n) * 4);
  if (!rc) rc = upload(h, di, dst_idx.data(), size_t(n) * 8);
  if (!rc) {
    hipError_t e = launch_host_rows_to_dev(host_src(h, G), dq, dr, di, n, reinterpret_cast<uint4*>(dst), nullptr);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) rc = fail(h, KV_EHIP, "host row copy: %s", hipGetErrorString(e));
  }
  (void)hipFree(dq);
  (void)hipFree(dr);
  (void)hipFree(di);
  return rc;
}

void free_all(kv_hier* h) {
  for (Group& G : h->grp) {
    (void)hipFree(G.hot);
    (void)hipFree(G.slot_row);
    (void)hipFree(G.slot_lu);
    (void)hipFree(G.slot_map);
    (void)hipFree(G.res_map);
    (void)hipFree(G.resident);
    (void)hipFree(G.ring);
    (void)hipFree(G.ring_lo);
    (void)hipFree(G.union_rows);
    (void)hipFree(G.union_loc);
    (void)hipFree(G.miss_rows);
    (void)hipFree(G.victims);
    (void)hipFree(G.protect);
    if (G.ev_done) (void)hipEventDestroy(G.ev_done);
    if (G.ev_sel) (void)hipEventDestroy(G.ev_sel);
    (void)hipFree(G.loc);
    (void)hipFree(G.sloc);
    (void)hipFree(G.req_info);
    (void)hipFree(G.req_counts);
    (void)hipFree(G.cum);
    (void)hipFree(G.snap_hot);
    (void)hipFree(G.snap_row);
    (void)hipFree(G.snap_lu);
    (void)hipFree(G.snap_map);
    (void)hipFree(const_cast<uint4**>(G.prefix_table));
    for (void* p : G.prefix_host) if (p) (void)hipHostFree(p);
    if (G.tails_host) (void)hipHostFree(G.tails_host);
  }
  for (uint16_t* a : h->arena) (void)hipFree(a);
  (void)hipFree(h->part_o);
  (void)hipFree(h->zero_row);
  (void)hipFree(h->part_ml);
  (void)hipFree(h->d_commit);
  (void)hipFree(h->d_commit_groups);
  (void)hipFree(const_cast<uint4**>(h->d_src));
  for (int i = 0; i < kCommitBufs; ++i) {
    if (h->h_commit[i]) (void)hipHostFree(h->h_commit[i]);
    if (h->h_src[i]) (void)hipHostFree(const_cast<uint4**>(h->h_src[i]));
    if (h->ev_commit[i]) (void)hipEventDestroy(h->ev_commit[i]);
  }
  if (h->ev_part) (void)hipEventDestroy(h->ev_part);
  for (auto& t : h->pending) { (void)hipEventDestroy(t.a); (void)hipEventDestroy(t.b); }
  for (hipEvent_t e : h->pool) (void)hipEventDestroy(e);
  if (h->ev_in) (void)hipEventDestroy(h->ev_in);
  if (h->ev_out) (void)hipEventDestroy(h->ev_out);
  if (h->work) (void)hipStreamDestroy(h->work);
  if (h->ev_verified) (void)hipEventDestroy(h->ev_verified);
  for (hipEvent_t e : h->ev_backup)
    if (e) (void)hipEventDestroy(e);
  for (auto& v : h->ev_fetched) for (hipEvent_t e : v) (void)hipEventDestroy(e);
  for (hipEvent_t e : h->ev_free) (void)hipEventDestroy(e);
  if (h->ev_map) (void)hipEventDestroy(h->ev_map);
  if (h->ev_planned) (void)hipEventDestroy(h->ev_planned);
  if (h->side) (void)hipStreamDestroy(h->side);
  if (h->aux) (void)hipStreamDestroy(h->aux);
  Opt& o = h->opt;
  for (auto& b : o.pending) (void)hipEventDestroy(b.ev);
  for (hipEvent_t e : o.ev_pool) (void)hipEventDestroy(e);
  for (ListBuf& b : o.bufs) {
    if (b.host) (void)hipHostFree(b.host);
    if (b.ev) (void)hipEventDestroy(b.ev);
  }
  (void)hipFree(o.d_list_side);
  (void)hipFree(o.d_list_copy);
  (void)hipFree(o.d_groups);
  if (o.ev_unpub) (void)hipEventDestroy(o.ev_unpub);
  if (o.stream) (void)hipStreamDestroy(o.stream);
}

// Ring size of "Adaptive DHiSparse" §3.4 eq. (9): page-rounded window plus block.
int ring_size(int W, int p, int kmax) { return p * ((W + p - 1 + kmax + p - 1) / p); }

int validate(kv_hier* h, const kv_hier_config& c) {
  if (c.n_req <= 0 || c.n_groups <= 0 || c.n_arenas <= 0 || c.hist_cap <= 0 || c.row_elems <= 0 ||
      c.d_qk <= 0 || c.d_v <= 0 || c.v_off < 0 || c.n_heads <= 0 || c.q_max <= 0 || c.topk <= 0 ||
      c.hot_slots <= 0 || c.ring_window <= 0 || c.ring_page <= 0 || c.n_prefix < 0 || c.prefix_len < 0 ||
      c.n_chunks < 0 || c.resident_cap < 0 || c.fetch_cus < 0 || c.fetch_wgs < 0 || c.plan_share < 0 ||
      c.opt_page_rows < 0 || c.opt_reserve < 0)
    return fail(h, KV_EINVAL, "non-positive size in config");
  if (c.q_max > 32) return fail(h, KV_EUNSUPPORTED, "q_max %d > 32", c.q_max);
  if (int64_t(c.q_max) * c.topk > 65535) return fail(h, KV_EUNSUPPORTED, "q_max*topk > 65535");
  if (c.d_qk > c.row_elems || c.v_off + c.d_v > c.row_elems) return fail(h, KV_EINVAL, "K/V outside the row");
  if (c.n_prefix > 0 && (c.prefix_len <= 0 || c.prefix_len > c.hist_cap))
    return fail(h, KV_EINVAL, "prefix_len must be in (0, hist_cap] with shared prefixes");
  if (c.n_prefix == 0 && c.prefix_len != 0) return fail(h, KV_EINVAL, "prefix_len without prefixes");
  if (!attn_layout_supported(c.row_elems, c.d_qk, c.v_off, c.d_v))
    return fail(h, KV_EUNSUPPORTED, "row layout (%d, %d, %d, %d) has no attention kernel", c.row_elems, c.d_qk,
                c.v_off, c.d_v);
  const int64_t lim = int64_t(1) << kTierShift;
  if (int64_t(c.n_req) * c.hot_slots >= lim || int64_t(c.n_req) * c.q_max * c.topk >= lim ||
      c.resident_cap >= lim || int64_t(c.hist_cap) >= lim ||
      int64_t(c.n_req) * ring_size(c.ring_window, c.ring_page, c.q_max) >= lim)
    return fail(h, KV_EUNSUPPORTED, "an index space exceeds 2^29 rows");
  if (c.hot_slots > 16384) return fail(h, KV_EUNSUPPORTED, "hot_slots > 16384");
  if (c.plan_share > 1 && c.n_groups % c.plan_share != 0)
    return fail(h, KV_EINVAL, "n_groups %d is not a multiple of plan_share %d", c.n_groups, c.plan_share);
  if (c.plan_share > 1 && c.n_arenas < c.plan_share)
    return fail(h, KV_EINVAL, "plan_share %d needs as many arenas (n_arenas %d)", c.plan_share, c.n_arenas);
  if (c.opt_page_rows > 0 &&
      (c.resident_cap <= 0 || c.resident_cap % c.opt_page_rows != 0 || c.opt_page_rows > c.hist_cap))
    return fail(h, KV_EINVAL, "dynamic residency needs resident_cap a positive multiple of opt_page_rows <= hist_cap");
  return KV_OK;
}

// ---------------------------------------------------------------- optional residency helpers

// A pinned page list of n int32 for one stream use; *out receives its index.
int take_list(kv_hier* h, size_t n, int* out) {
  Opt& o = h->opt;
  for (size_t i = 0; i < o.bufs.size(); ++i) {
    ListBuf& b = o.bufs[i];
    if (b.busy) {
      const hipError_t q = hipEventQuery(b.ev);
      if (q == hipErrorNotReady) continue;
      if (q != hipSuccess) return fail(h, KV_EHIP, "list event: %s", hipGetErrorString(q));
      b.busy = false;
    }
    if (b.cap >= n) {
      *out = int(i);
      return KV_OK;
    }
  }
  ListBuf b;
  b.cap = std::max<size_t>(n, 4096);
  void* p = nullptr;
  if (hipHostMalloc(&p, b.cap * 4, hipHostMallocDefault) != hipSuccess) {
    (void)hipGetLastError();
    return fail(h, KV_ENOMEM, "pinned page list of %zu entries", b.cap);
  }
  b.host = static_cast<int32_t*>(p);
  if (hipEventCreateWithFlags(&b.ev, hipEventDisableTiming) != hipSuccess) {
    (void)hipHostFree(p);
    return fail(h, KV_EHIP, "event create failed");
  }
  o.bufs.push_back(b);
  *out = int(o.bufs.size()) - 1;
  return KV_OK;
}

// Moves a (request, page, pool page) list to the stream's device list buffer.
int stage_list(kv_hier* h, const std::vector<int32_t>& ent, int32_t* dev, hipStream_t s) {
  int bi = -1;
  int rc = take_list(h, ent.size(), &bi);
  if (rc) return rc;
  ListBuf& b = h->opt.bufs[bi];
  std::memcpy(b.host, ent.data(), ent.size() * 4);
  HIPCHK(h, hipMemcpyAsync(dev, b.host, ent.size() * 4, hipMemcpyHostToDevice, s));
  HIPCHK(h, hipEventRecord(b.ev, s));
  b.busy = true;
  return KV_OK;
}

// Publication (publish = 1) or withdrawal of pages in every group's resident
// map, on the side stream, between the plans issued before it and those
// issued after it: it waits for every group's last step (its plan ran before
// its attention), and every group's next plan waits for it (map_wait).
int opt_map(kv_hier* h, const std::vector<int32_t>& ent, int publish) {
  if (ent.empty()) return KV_OK;
  Opt& o = h->opt;
  for (const Group& G : h->grp)
    if (G.member == 0 && G.sel_recorded) HIPCHK(h, hipStreamWaitEvent(h->side, G.ev_sel, 0));
  int rc = stage_list(h, ent, o.d_list_side, h->side);
  if (rc) return rc;
  HIPCHK(h, launch_opt_map(o.d_groups, h->cfg.n_groups, o.d_list_side, int(ent.size() / 3), o.P, h->L, publish,
                           h->side));
  HIPCHK(h, hipEventRecord(h->ev_map, h->side));
  for (Group& G : h->grp) G.map_wait = true;
  if (!publish) {
    HIPCHK(h, hipEventRecord(o.ev_unpub, h->side));
    o.unpub_recorded = true;
  }
  return KV_OK;
}

// Publishes every pending page whose copy has completed (all of them, waiting,
// when wait is set).  Batches complete in order: they share one stream.
int opt_publish_impl(kv_hier* h, bool wait) {
  Opt& o = h->opt;
  std::vector<int32_t> pub;
  while (!o.pending.empty()) {
    Opt::Batch& b = o.pending.front();
    if (wait) {
      HIPCHK(h, hipEventSynchronize(b.ev));
    } else {
      const hipError_t q = hipEventQuery(b.ev);
      if (q == hipErrorNotReady) break;
      if (q != hipSuccess) return fail(h, KV_EHIP, "population event: %s", hipGetErrorString(q));
    }
    for (size_t i = 0; i + 4 <= b.ent.size(); i += 4) {
      const int32_t r = b.ent[i], idx = b.ent[i + 1], pg = b.ent[i + 2];
      const uint32_t gen = uint32_t(b.ent[i + 3]);
      // a page reclaimed while its copy ran is not published (its owner changed)
      if (o.gen[pg] != gen || o.state[pg] != PG_PENDING) continue;
      o.state[pg] = PG_READY;
      o.n_ready[r] += 1;
      pub.push_back(r);
      pub.push_back(idx);
      pub.push_back(pg);
    }
    o.ev_pool.push_back(b.ev);
    o.pending.pop_front();
  }
  if (pub.empty()) return KV_OK;
  o.n_published += int64_t(pub.size() / 3);
  o.pages_published += int64_t(pub.size() / 3);
  return opt_map(h, pub, 1);
}

// Drops every optional page of request r (reclaim or completion): ready pages
// are withdrawn from the maps now and marked to be rewritten only after the
// readers of earlier steps; pending pages are simply never published.
int opt_drop(kv_hier* h, int r) {
  Opt& o = h->opt;
  std::vector<int32_t> wd;
  for (int idx = 0; idx < o.n_held[r]; ++idx) {
    const int32_t pg = o.held[r][idx];
    if (o.state[pg] == PG_READY) {
      wd.push_back(r);
      wd.push_back(idx);
      wd.push_back(pg);
      o.needs_wait[pg] = 1;
      o.n_published -= 1;
    }
    o.state[pg] = PG_FREE;
    o.free.insert(pg);
    o.held[r][idx] = -1;
  }
  o.pages_reclaimed += o.n_held[r];
  o.sum_held -= o.n_held[r];
  o.n_held[r] = 0;
  o.n_ready[r] = 0;
  return opt_map(h, wd, 0);
}

// Attention of one request range (+ the merge of its key splits) on stream
// s.  Split partials live in one buffer of the handle: a launch that uses
// them waits for the previous user, wherever that ran.
int attend(kv_hier* h, int g, const AttnArgs& at, hipStream_t s) {
  const kv_hier_config& c = h->cfg;
  if (at.splits > 1 && h->part_recorded) HIPCHK(h, hipStreamWaitEvent(s, h->ev_part, 0));
  LaunchEv le = launch_events(h, K_ATTN, g, nullptr);
  // test hook: the launch reports an error without launching anything
  HIPCHK(h, (c.flags & KV_FLAG_TEST_FAIL_ATTN)
                ? hipErrorLaunchFailure
                : launch_attn(at, c.row_elems, c.d_qk, c.v_off, c.d_v, s, le.start, le.stop));
  if (at.splits > 1) {
    // the partials' release is the merge's own end event unless timing holds it
    le = launch_events(h, K_COMBINE, g, h->ev_part);
    HIPCHK(h, launch_attn_combine(at, c.d_v, s, le.start, le.stop));
    if (le.after) HIPCHK(h, hipEventRecord(le.after, s));
    h->part_recorded = true;
  }
  return KV_OK;
}

}  // namespace

extern "C" {

// message of the last failed kv_hier_create on this thread (no handle exists then)
static thread_local std::string g_create_error = "null handle";

const char* kv_hier_last_error(const kv_hier_t* h) { return h ? h->err.c_str() : g_create_error.c_str(); }

void kv_hier_destroy(kv_hier_t* h) {
  DeviceGuard dg(h);
  if (!h) return;
  (void)hipDeviceSynchronize();
  free_all(h);
  delete h;
}

static int create_impl(kv_hier* h) {
  int rc = KV_OK;
  const kv_hier_config& c = h->cfg;
  (void)hipGetDevice(&h->device);
  const int N = c.n_req, B = c.hot_slots, L = c.hist_cap;
  h->L = L;
  h->QK = c.q_max * c.topk;
  h->row_bytes = size_t(c.row_elems) * 2;
  h->row16 = c.row_elems / 8;
  h->Rd = ring_size(c.ring_window, c.ring_page, c.q_max);
  h->n_prefix = c.n_prefix;
  h->plen = c.n_prefix > 0 ? c.prefix_len : 0;
  h->tail_rows = L - h->plen;
  h->hist_len.assign(N, 0);

  // plan kernel shared memory: row-chunk bitmap, word prefixes and union codes
  int sc = 1;
  while (sc < B) sc <<= 1;
  h->sort_cap = sc;
  {
    const size_t budget = 160 * 1024 - 1024 - ((size_t(B + 31) / 32) * 4 + 16);
    const size_t qk_bytes = (size_t(h->QK) * 4 + 15) & ~size_t(15);
    if (qk_bytes + 64 > budget || size_t(sc) * 8 > budget) return fail(h, KV_EUNSUPPORTED, "plan LDS");
    size_t cw_max = (budget - qk_bytes - 32) / 6;
    size_t cw = (size_t(L) + 31) / 32;
    if (cw > cw_max) cw = cw_max;
    h->chunk_words = int(cw);
    h->plan_lds = plan_lds_bytes(c.q_max, c.topk, B, h->chunk_words, sc);
    if (h->plan_lds > 160 * 1024) return fail(h, KV_EUNSUPPORTED, "plan LDS %zu", h->plan_lds);
    // the row-ordered lists (the order kernel's per-query bitmaps beside the
    // resolution's row chunk); without them the attention walks the
    // selection order
    // (they are ordered before the attention through the fetches on the fetch
    // stream, so a handle with one request chunk has none)
    h->order_lds = plan_order_lds_bytes(c.q_max, c.topk, h->chunk_words);
    h->row_order = h->order_lds <= 160 * 1024;
  }
  // the plan and attention kernels take more than 64 KB of dynamic LDS (set
  // per device: every handle sets it on its own)
  HIPCHK(h, plan_init_attributes());
  HIPCHK(h, attn_init_attributes());
  {
    hipError_t e = hipSuccess;
    h->scratch_dev = scratch_on_device(h->device, &e);
    if (!h->scratch_dev) return fail(h, KV_EHIP, "static scratch address: %s", hipGetErrorString(e));
  }
  // request chunks for the fetch/attention pipeline
  // Automatic layout for N >= 64: four quarters, the last one halved when each
  // half still fills the GPU with attention workgroups (N/8 x Q x head groups
  // >= 256).  The halving shortens the attention left after the last fetch
  // (nothing overlaps it); below a full wave a chunk needs key splits and a
  // merge, which cost more than the shorter tail saves.
  if (c.n_chunks == 0 && N >= 64) {
    const int hpw = attn_heads_per_wg(c.n_heads, c.row_elems, int64_t(N / 8) * c.q_max);
    const int64_t hgroups = (c.n_heads + hpw - 1) / hpw;
    const bool halve = int64_t(N / 8) * c.q_max * hgroups >= 256;
    const std::vector<int> eighths = halve ? std::vector<int>{0, 2, 4, 6, 7, 8} : std::vector<int>{0, 2, 4, 6, 8};
    for (int x : eighths) h->chunk_lo.push_back(int(int64_t(N) * x / 8));
  } else {
    const int nch = c.n_chunks > 0 ? std::min(c.n_chunks, N) : (N >= 16 ? 2 : 1);
    for (int i = 0; i <= nch; ++i) h->chunk_lo.push_back(int(int64_t(N) * i / nch));
  }
  h->n_chunks = int(h->chunk_lo.size()) - 1;
  // lists shorter than 1024 entries keep the selection order: there the order
  // kernel, beside a short first fetch, costs more than the walk saves
  // (measured on 288-B rows at k = 512)
  if (h->n_chunks < 2 || c.topk < 1024) h->row_order = false;
  {
    // heads per workgroup and key splits per launch: about 256 workgroups
    // per launch (the combine pass merges the splits); partials are indexed
    // from the launch's first request, 32*HB heads per block
    const int tiles = (c.topk + c.ring_window + 31) / 32;
    size_t slots = 0;
    h->splits = 1;
    h->head_groups = 1;
    auto split_for = [&](int64_t wgs) {
      int s = wgs < 256 ? int(std::min<int64_t>(8, std::max<int64_t>(1, 256 / std::max<int64_t>(1, wgs)))) : 1;
      return std::max(1, std::min(s, tiles / 4));
    };
    for (int ch = 0; ch < h->n_chunks; ++ch) {
      const int64_t queries = int64_t(h->chunk_lo[ch + 1] - h->chunk_lo[ch]) * c.q_max;
      const int hpw = attn_heads_per_wg(c.n_heads, c.row_elems, queries);
      const int hg = (c.n_heads + hpw - 1) / hpw;
      const int64_t wgs = queries * hg;
      const int s = split_for(wgs);
      h->chunk_splits.push_back(s);
      h->chunk_hpw.push_back(hpw);
      h->splits = std::max(h->splits, s);
      h->head_groups = std::max(h->head_groups, hg);
      if (s > 1) slots = std::max(slots, size_t(wgs) * s * hpw);
    }
    h->step_part_heads = slots;
    {
      // a Reuse layer has no fetch to overlap: one launch over every request
      const int64_t queries = int64_t(N) * c.q_max;
      h->all_hpw = attn_heads_per_wg(c.n_heads, c.row_elems, queries);
      const int64_t wgs = queries * ((c.n_heads + h->all_hpw - 1) / h->all_hpw);
      h->all_splits = split_for(wgs);
      h->splits = std::max(h->splits, h->all_splits);
      if (h->all_splits > 1) slots = std::max(slots, size_t(wgs) * h->all_splits * h->all_hpw);
    }
    if (slots > 0) {
      rc = dev_alloc(h, &h->part_o, slots * c.d_v, &h->bytes_maps);
      if (!rc) rc = dev_alloc(h, &h->part_ml, slots * 2, &h->bytes_maps);
      if (rc) return rc;
    }
  }
  h->share = c.plan_share > 1 ? c.plan_share : 1;
  h->grp.resize(c.n_groups);
  for (int g = 0; g < c.n_groups; ++g) {
    Group& G = h->grp[g];
    G.member = g % h->share;
    G.leader = g - G.member;
    G.res_set.assign(N, 0);
    const size_t NB = size_t(N) * B, NL = size_t(N) * L, NQK = size_t(N) * h->QK;
    if ((rc = dev_alloc(h, &G.hot, NB * c.row_elems, &h->bytes_hot))) return rc;
    if ((rc = dev_alloc(h, &G.slot_row, NB, &h->bytes_maps))) return rc;
    if ((rc = dev_alloc(h, &G.slot_lu, NB, &h->bytes_maps))) return rc;
    if ((rc = dev_alloc(h, &G.slot_map, NL, &h->bytes_maps))) return rc;
    if ((rc = dev_alloc(h, &G.res_map, NL, &h->bytes_maps))) return rc;
    if (c.resident_cap > 0 && (rc = dev_alloc(h, &G.resident, size_t(c.resident_cap) * c.row_elems, &h->bytes_res)))
      return rc;
    if ((rc = dev_alloc(h, &G.ring, size_t(N) * h->Rd * c.row_elems, &h->bytes_ring))) return rc;
    if ((rc = dev_alloc(h, &G.ring_lo, size_t(N), &h->bytes_maps))) return rc;
    if ((rc = dev_alloc(h, &G.union_rows, NQK, &h->bytes_maps))) return rc;
    if ((rc = dev_alloc(h, &G.union_loc, NQK, &h->bytes_maps))) return rc;
    if ((rc = dev_alloc(h, &G.miss_rows, NQK, &h->bytes_maps))) return rc;
    if ((rc = dev_alloc(h, &G.victims, NQK, &h->bytes_maps))) return rc;
    if ((rc = dev_alloc(h, &G.protect, size_t(N) * ((c.hot_slots + 31) / 32), &h->bytes_maps))) return rc;
    if ((rc = dev_alloc(h, &G.loc, NQK, &h->bytes_maps))) return rc;
    if (h->row_order && (rc = dev_alloc(h, &G.sloc, NQK, &h->bytes_maps))) return rc;
    if ((rc = dev_alloc(h, &G.req_info, size_t(N) * I_NUM, &h->bytes_maps))) return rc;
    if ((rc = dev_alloc(h, &G.req_counts, size_t(N) * C_NUM, &h->bytes_maps))) return rc;
    if ((rc = dev_alloc(h, &G.cum, size_t(C_NUM), &h->bytes_maps))) return rc;
    const uint32_t neg = 0xffffffffu;
    if (launch_fill32(reinterpret_cast<uint32_t*>(G.slot_row), neg, NB, nullptr) != hipSuccess ||
        launch_fill32(reinterpret_cast<uint32_t*>(G.slot_lu), 0, NB, nullptr) != hipSuccess ||
        launch_fill32(reinterpret_cast<uint32_t*>(G.slot_map), neg, NL, nullptr) != hipSuccess ||
        launch_fill32(reinterpret_cast<uint32_t*>(G.res_map), neg, NL, nullptr) != hipSuccess ||
        launch_fill32(reinterpret_cast<uint32_t*>(G.ring), 0, size_t(N) * h->Rd * c.row_elems / 2, nullptr) !=
            hipSuccess ||
        launch_fill32(reinterpret_cast<uint32_t*>(G.ring_lo), 0, size_t(N), nullptr) != hipSuccess ||
        launch_fill32(reinterpret_cast<uint32_t*>(G.req_info), 0, size_t(N) * I_NUM, nullptr) != hipSuccess ||
        launch_fill32(reinterpret_cast<uint32_t*>(G.req_counts), 0, size_t(N) * C_NUM * 2, nullptr) !=
            hipSuccess ||
        launch_fill32(reinterpret_cast<uint32_t*>(G.cum), 0, size_t(C_NUM) * 2, nullptr) != hipSuccess) {
      return fail(h, KV_EHIP, "initial fill failed");
    }
    // pinned host backing, mapped into the device address space
    const int np = c.n_prefix;
    G.prefix_host.assign(np > 0 ? np : 0, nullptr);
    std::vector<const uint4*> table(np > 0 ? np : 1, nullptr);
    for (int p = 0; p < np; ++p) {
      if ((rc = host_alloc(h, &G.prefix_host[p], size_t(h->plen) * h->row_bytes))) return rc;
      std::memset(G.prefix_host[p], 0, size_t(h->plen) * h->row_bytes);
      void* dp = nullptr;
      HIPCHK(h, hipHostGetDevicePointer(&dp, G.prefix_host[p], 0));
      table[p] = static_cast<const uint4*>(dp);
    }
    if ((rc = host_alloc(h, &G.tails_host, size_t(N) * h->tail_rows * h->row_bytes))) return rc;
    std::memset(G.tails_host, 0, size_t(N) * h->tail_rows * h->row_bytes);
    {
      void* dp = nullptr;
      HIPCHK(h, hipHostGetDevicePointer(&dp, G.tails_host, 0));
      G.tails_dev = static_cast<const uint4*>(dp);
    }
    const uint4** dt = nullptr;
    if ((rc = dev_alloc(h, &dt, table.size(), nullptr))) return rc;
    G.prefix_table = dt;
    if ((rc = upload(h, dt, table.data(), table.size() * sizeof(void*)))) return rc;
  }
  h->arena.assign(c.n_arenas, nullptr);
  for (int a = 0; a < c.n_arenas; ++a)
    if ((rc = dev_alloc(h, &h->arena[a], size_t(N) * h->QK * c.row_elems, &h->bytes_staging))) return rc;
  if ((rc = dev_alloc(h, &h->zero_row, size_t(c.row_elems), &h->bytes_maps))) return rc;
  if (launch_fill32(reinterpret_cast<uint32_t*>(h->zero_row), 0, size_t(c.row_elems) / 2, nullptr) != hipSuccess)
    return fail(h, KV_EHIP, "zero row fill failed");
  if (c.opt_page_rows > 0) {
    Opt& o = h->opt;
    o.on = true;
    o.P = c.opt_page_rows;
    o.M = int(c.resident_cap / c.opt_page_rows);
    o.reserve = c.opt_reserve;
    o.admitted.assign(N, 0);
    o.required.assign(N, 0);
    o.eligible.assign(N, 0);
    o.n_held.assign(N, 0);
    o.n_ready.assign(N, 0);
    o.held.assign(N, {});
    o.state.assign(o.M, PG_FREE);
    o.needs_wait.assign(o.M, 0);
    o.gen.assign(o.M, 0);
    for (int i = 0; i < o.M; ++i) o.free.insert(o.free.end(), i);
    std::vector<OptGroup> og(c.n_groups);
    for (int g = 0; g < c.n_groups; ++g) {
      og[g].src = host_src(h, h->grp[g]);
      og[g].pool = reinterpret_cast<uint4*>(h->grp[g].resident);
      og[g].res_map = h->grp[g].res_map;
      // debug: a page read before its copy completes shows up as NaN
      if ((c.flags & KV_FLAG_POISON) &&
          launch_fill32(reinterpret_cast<uint32_t*>(h->grp[g].resident), 0x7fc07fc0u,
                        size_t(c.resident_cap) * c.row_elems / 2, nullptr) != hipSuccess)
        return fail(h, KV_EHIP, "pool poison fill failed");
    }
    if ((rc = dev_alloc(h, &o.d_groups, og.size(), nullptr))) return rc;
    if ((rc = upload(h, o.d_groups, og.data(), og.size() * sizeof(OptGroup)))) return rc;
    if ((rc = dev_alloc(h, &o.d_list_side, size_t(o.M) * 3, &h->bytes_maps))) return rc;
    if ((rc = dev_alloc(h, &o.d_list_copy, size_t(o.M) * 3, &h->bytes_maps))) return rc;
    HIPCHK(h, hipStreamCreateWithFlags(&o.stream, hipStreamNonBlocking));
    HIPCHK(h, hipEventCreateWithFlags(&o.ev_unpub, hipEventDisableTiming));
  }
  {
    std::vector<CommitGroup> cg(c.n_groups);
    for (int g = 0; g < c.n_groups; ++g) {
      cg[g].ring = reinterpret_cast<const uint4*>(h->grp[g].ring);
      cg[g].tails = const_cast<uint4*>(h->grp[g].tails_dev);
      cg[g].m = 1;
      cg[g].cmax = c.q_max;
    }
    if ((rc = dev_alloc(h, &h->d_commit_groups, cg.size(), nullptr))) return rc;
    if ((rc = upload(h, h->d_commit_groups, cg.data(), cg.size() * sizeof(CommitGroup)))) return rc;
    if ((rc = dev_alloc(h, &h->d_commit, size_t(2) * N, nullptr))) return rc;
    const uint4** ds = nullptr;
    if ((rc = dev_alloc(h, &ds, size_t(c.n_groups), nullptr))) return rc;
    h->d_src = ds;
    for (int i = 0; i < kCommitBufs; ++i) {
      void* hc = nullptr;
      if (hipHostMalloc(&hc, size_t(2) * N * 4, hipHostMallocDefault) != hipSuccess) {
        (void)hipGetLastError();
        return fail(h, KV_ENOMEM, "pinned commit buffer");
      }
      h->h_commit[i] = static_cast<int32_t*>(hc);
      void* hs = nullptr;
      if (hipHostMalloc(&hs, size_t(c.n_groups) * sizeof(void*), hipHostMallocDefault) != hipSuccess) {
        (void)hipGetLastError();
        return fail(h, KV_ENOMEM, "pinned commit buffer");
      }
      h->h_src[i] = static_cast<const uint4**>(hs);
      HIPCHK(h, hipEventCreateWithFlags(&h->ev_commit[i], hipEventDisableTiming));
    }
  }
  if (c.fetch_cus > 0) {
    // partition the CUs: a few for the PCIe-latency-bound fetch, the rest for the step
    hipDeviceProp_t prop;
    HIPCHK(h, hipGetDeviceProperties(&prop, h->device));
    const int ncu = prop.multiProcessorCount;
    if (c.fetch_cus >= ncu) return fail(h, KV_EINVAL, "fetch_cus %d >= %d CUs", c.fetch_cus, ncu);
    const int words = (ncu + 31) / 32;
    std::vector<uint32_t> fm(words, 0), wm(words, 0);
    // mask bit i belongs to XCD i mod 8 and every stream needs CUs on every XCD:
    // the first fetch_cus bits give the fetch the same share of each XCD
    if (c.fetch_cus % 8 != 0) return fail(h, KV_EINVAL, "fetch_cus %d is not a multiple of 8", c.fetch_cus);
    for (int cu = 0; cu < c.fetch_cus; ++cu) fm[cu / 32] |= 1u << (cu % 32);
    for (int cu = 0; cu < ncu; ++cu)
      if (!((fm[cu / 32] >> (cu % 32)) & 1u)) wm[cu / 32] |= 1u << (cu % 32);
    HIPCHK(h, hipExtStreamCreateWithCUMask(&h->side, uint32_t(words), fm.data()));
    HIPCHK(h, hipExtStreamCreateWithCUMask(&h->work, uint32_t(words), wm.data()));
  } else {
    HIPCHK(h, hipStreamCreateWithFlags(&h->side, hipStreamNonBlocking));
  }
  HIPCHK(h, hipStreamCreateWithFlags(&h->aux, hipStreamNonBlocking));
  for (Group& G : h->grp) {
    HIPCHK(h, hipEventCreateWithFlags(&G.ev_done, hipEventDisableTiming));
    HIPCHK(h, hipEventCreateWithFlags(&G.ev_sel, hipEventDisableTiming));
  }
  HIPCHK(h, hipEventCreateWithFlags(&h->ev_planned, hipEventDisableTiming));
  HIPCHK(h, hipEventCreateWithFlags(&h->ev_in, hipEventDisableTiming));
  HIPCHK(h, hipEventCreateWithFlags(&h->ev_out, hipEventDisableTiming));
  HIPCHK(h, hipEventCreateWithFlags(&h->ev_part, hipEventDisableTiming));
  // Asynchronous host backup needs every row of the last commit to stay in the
  // ring's tail through the next step (R_d >= 2 K_max); otherwise the backup
  // runs on the caller's stream, ahead of the next step.
  // It shares the copy-back stream: one more stream would share a hardware
  // queue with another and add false dependencies.
  if (h->Rd >= 2 * c.q_max) {
    h->backup = h->aux;
    HIPCHK(h, hipEventCreateWithFlags(&h->ev_verified, hipEventDisableTiming));
    for (hipEvent_t& e : h->ev_backup) HIPCHK(h, hipEventCreateWithFlags(&e, hipEventDisableTiming));
  }
  h->ev_fetched.assign(h->share, std::vector<hipEvent_t>(h->n_chunks, nullptr));
  for (auto& v : h->ev_fetched)
    for (auto& e : v) HIPCHK(h, hipEventCreateWithFlags(&e, hipEventDisableTiming));
  h->ev_free.assign(c.n_arenas, nullptr);
  h->free_recorded.assign(c.n_arenas, 0);
  h->arena_owner.assign(c.n_arenas, -1);
  h->arena_step.assign(c.n_arenas, 0);
  for (auto& e : h->ev_free) HIPCHK(h, hipEventCreateWithFlags(&e, hipEventDisableTiming));
  HIPCHK(h, hipEventCreateWithFlags(&h->ev_map, hipEventDisableTiming));
  HIPCHK(h, hipDeviceSynchronize());
  return rc;
}

int kv_hier_create(const kv_hier_config* cfg, kv_hier_t** out) {
  if (!cfg || !out) return KV_EINVAL;
  *out = nullptr;
  kv_hier* h = new (std::nothrow) kv_hier();
  if (!h) {
    g_create_error = "kv_hier_create: out of host memory";
    return KV_ENOMEM;
  }
  h->cfg = *cfg;
  int rc = validate(h, *cfg);
  if (!rc) rc = create_impl(h);
  if (rc) {
    g_create_error = h->err.empty() ? "kv_hier_create failed" : h->err;
    (void)hipDeviceSynchronize();
    free_all(h);
    delete h;
    return rc;
  }
  *out = h;
  return KV_OK;
}


int kv_hier_info_get(kv_hier_t* h, kv_hier_info* out) {
  if (!h || !out) return KV_EINVAL;
  out->ring_rows = h->Rd;
  out->n_chunks = h->n_chunks;
  out->bytes_hot = h->bytes_hot;
  out->bytes_staging = h->bytes_staging;
  out->bytes_ring = h->bytes_ring;
  out->bytes_maps = h->bytes_maps;
  out->bytes_resident = h->bytes_res;
  out->bytes_host = h->bytes_host;
  out->attn_splits = h->splits;
  out->attn_head_groups = h->head_groups;
  out->attn_reuse_head_groups = (h->cfg.n_heads + h->all_hpw - 1) / h->all_hpw;
  out->attn_row_order = h->row_order ? 1 : 0;
  out->plan_rows_per_pass = h->chunk_words * 32;
  return KV_OK;
}

int kv_hier_host_rows(kv_hier_t* h, int g, int kind, int index, void** rows, int64_t* n_rows) {
  DeviceGuard dg(h);
  int rc = check_group(h, g);
  if (rc) return rc;
  if (!rows || !n_rows) return fail(h, KV_EINVAL, "null output");
  Group& G = h->grp[g];
  if (kind == 0) {
    if (index < 0 || index >= h->n_prefix) return fail(h, KV_EINVAL, "prefix %d outside [0, %d)", index, h->n_prefix);
    *rows = G.prefix_host[index];
    *n_rows = h->plen;
  } else if (kind == 1) {
    if ((rc = check_req(h, index))) return rc;
    *rows = static_cast<char*>(G.tails_host) + size_t(index) * h->tail_rows * h->row_bytes;
    *n_rows = h->tail_rows;
  } else {
    return fail(h, KV_EINVAL, "kind %d", kind);
  }
  return KV_OK;
}

static int set_hist_len_impl(kv_hier_t* h, const int32_t* hist_len) {
  if (!h || !hist_len) return KV_EINVAL;
  for (int r = 0; r < h->cfg.n_req; ++r)
    if (hist_len[r] < 0 || hist_len[r] > h->cfg.hist_cap)
      return fail(h, KV_EINVAL, "hist_len[%d] = %d outside [0, %d]", r, hist_len[r], h->cfg.hist_cap);
  if (h->opt.on)
    for (int r = 0; r < h->cfg.n_req; ++r)
      if (h->opt.admitted[r])
        return fail(h, KV_ESTATE, "request %d is admitted: its imported history is fixed until completion", r);
  begin_work(h);
  int rc = sync_all(h);
  if (rc) return rc;
  h->hist_len.assign(hist_len, hist_len + h->cfg.n_req);
  for (Group& G : h->grp)
    if ((rc = upload(h, G.ring_lo, hist_len, size_t(h->cfg.n_req) * 4))) return rc;
  return KV_OK;
}

int kv_hier_set_hist_len(kv_hier_t* h, const int32_t* hist_len) {
  DeviceGuard dg(h);
  if (int rc = refuse_if_broken(h)) return rc;
  return finish(h, set_hist_len_impl(h, hist_len));
}

int kv_hier_hist_len(kv_hier_t* h, int32_t* hist_len) {
  DeviceGuard dg(h);
  if (!h || !hist_len) return KV_EINVAL;
  std::copy(h->hist_len.begin(), h->hist_len.end(), hist_len);
  return KV_OK;
}

static int set_hot_impl(kv_hier_t* h, int g, int r, const int32_t* rows, const int32_t* last_used, int n) {
  int rc = check_group(h, g);
  if (rc) return rc;
  if ((rc = check_req(h, r))) return rc;
  const int B = h->cfg.hot_slots, L = h->L;
  if (n < 0 || n > B || (n > 0 && (!rows || !last_used))) return fail(h, KV_EINVAL, "bad hot set size %d", n);
  std::vector<int32_t> nrow(B, -1), nlu(B, 0);
  std::vector<char> seen(size_t(L), 0);
  int maxlu = 0;
  for (int s = 0; s < n; ++s) {
    if (rows[s] < -1 || rows[s] >= L) return fail(h, KV_EINVAL, "hot row %d outside [-1, %d)", rows[s], L);
    if (last_used[s] < 0) return fail(h, KV_EINVAL, "negative last_used");
    if (rows[s] >= 0) {
      if (seen[rows[s]]) return fail(h, KV_EINVAL, "hot row %d repeated", rows[s]);
      seen[rows[s]] = 1;
    }
    nrow[s] = rows[s];
    nlu[s] = last_used[s];
    maxlu = std::max(maxlu, last_used[s]);
  }
  begin_work(h);
  if ((rc = sync_all(h))) return rc;
  Group& G = h->grp[g];
  std::vector<int32_t> old(B);
  if ((rc = download(h, old.data(), G.slot_row + size_t(r) * B, size_t(B) * 4))) return rc;
  std::vector<int64_t> idx;
  std::vector<int32_t> val;
  for (int s = 0; s < B; ++s)
    if (old[s] >= 0) { idx.push_back(int64_t(r) * L + old[s]); val.push_back(-1); }
  if ((rc = scatter32(h, G.slot_map, idx, val))) return rc;
  idx.clear();
  val.clear();
  std::vector<int32_t> req, src;
  std::vector<int64_t> dst;
  for (int s = 0; s < B; ++s)
    if (nrow[s] >= 0) {
      idx.push_back(int64_t(r) * L + nrow[s]);
      val.push_back(s);
      req.push_back(r);
      src.push_back(nrow[s]);
      dst.push_back(int64_t(r) * B + s);
    }
  if ((rc = scatter32(h, G.slot_map, idx, val))) return rc;
  if ((rc = upload(h, G.slot_row + size_t(r) * B, nrow.data(), size_t(B) * 4))) return rc;
  if ((rc = upload(h, G.slot_lu + size_t(r) * B, nlu.data(), size_t(B) * 4))) return rc;
  if ((rc = rows_from_host(h, G, req, src, dst, G.hot))) return rc;
  G.t = std::max(G.t, maxlu);
  return KV_OK;
}

int kv_hier_set_hot(kv_hier_t* h, int g, int r, const int32_t* rows, const int32_t* last_used, int n) {
  DeviceGuard dg(h);
  if (int rc = refuse_if_broken(h)) return rc;
  return finish(h, set_hot_impl(h, g, r, rows, last_used, n));
}

static int set_resident_impl(kv_hier_t* h, int g, int r, const uint8_t* bitmap) {
  int rc = check_group(h, g);
  if (rc) return rc;
  if ((rc = check_req(h, r))) return rc;
  if (!bitmap) return fail(h, KV_EINVAL, "null bitmap");
  if (h->opt.on) return fail(h, KV_ESTATE, "static resident sets are not used with dynamic residency");
  Group& G = h->grp[g];
  if (G.res_set[r]) return fail(h, KV_ESTATE, "resident set of request %d already given", r);
  const int lim = std::min(h->hist_len[r] / G.m, h->L);
  std::vector<int64_t> idx, dst;
  std::vector<int32_t> val, req, src;
  for (int s = 0; s < lim; ++s)
    if (bitmap[s]) {
      idx.push_back(int64_t(r) * h->L + s);
      val.push_back(int32_t(G.res_cursor + int64_t(val.size())));
      req.push_back(r);
      src.push_back(s);
      dst.push_back(G.res_cursor + int64_t(dst.size()));
    }
  if (G.res_cursor + int64_t(val.size()) > h->cfg.resident_cap)
    return fail(h, KV_ENOMEM, "resident pool full (%lld of %lld rows)", (long long)(G.res_cursor + val.size()),
                (long long)h->cfg.resident_cap);
  begin_work(h);
  if ((rc = sync_all(h))) return rc;
  if ((rc = scatter32(h, G.res_map, idx, val))) return rc;
  if ((rc = rows_from_host(h, G, req, src, dst, G.resident))) return rc;
  G.res_cursor += int64_t(val.size());
  G.res_set[r] = 1;
  return KV_OK;
}

int kv_hier_set_resident(kv_hier_t* h, int g, int r, const uint8_t* bitmap) {
  DeviceGuard dg(h);
  if (int rc = refuse_if_broken(h)) return rc;
  return finish(h, set_resident_impl(h, g, r, bitmap));
}

static int clear_resident_impl(kv_hier_t* h, int g) {
  int rc = check_group(h, g);
  if (rc) return rc;
  if (h->opt.on) return fail(h, KV_ESTATE, "static resident sets are not used with dynamic residency");
  begin_work(h);
  if ((rc = sync_all(h))) return rc;
  Group& G = h->grp[g];
  HIPCHK(h, launch_fill32(reinterpret_cast<uint32_t*>(G.res_map), 0xffffffffu, size_t(h->cfg.n_req) * h->L, nullptr));
  HIPCHK(h, hipDeviceSynchronize());
  G.res_cursor = 0;
  std::fill(G.res_set.begin(), G.res_set.end(), 0);
  return KV_OK;
}

int kv_hier_clear_resident(kv_hier_t* h, int g) {
  DeviceGuard dg(h);
  if (int rc = refuse_if_broken(h)) return rc;
  return finish(h, clear_resident_impl(h, g));
}

static int ring_load_impl(kv_hier_t* h, int g, int r, int32_t first_pos, const void* rows, int n) {
  int rc = check_group(h, g);
  if (rc) return rc;
  if ((rc = check_req(h, r))) return rc;
  if (n < 0 || first_pos < 0 || n > h->Rd || (n > 0 && !rows) || int64_t(first_pos) + n != h->hist_len[r])
    return fail(h, KV_EINVAL, "ring_load must cover [first_pos, n_r) with at most R_d=%d rows", h->Rd);
  begin_work(h);
  if ((rc = sync_all(h))) return rc;
  Group& G = h->grp[g];
  const char* src = static_cast<const char*>(rows);
  int done = 0;
  while (done < n) {
    const int pos = first_pos + done;
    const int slot = pos % h->Rd;
    const int run = std::min(n - done, h->Rd - slot);
    char* dst = reinterpret_cast<char*>(G.ring) + (size_t(r) * h->Rd + slot) * h->row_bytes;
    if ((rc = upload(h, dst, src + size_t(done) * h->row_bytes, size_t(run) * h->row_bytes))) return rc;
    done += run;
  }
  const int32_t lo = first_pos;
  return upload(h, G.ring_lo + r, &lo, 4);
}

int kv_hier_ring_load(kv_hier_t* h, int g, int r, int32_t first_pos, const void* rows, int n) {
  DeviceGuard dg(h);
  if (int rc = refuse_if_broken(h)) return rc;
  return finish(h, ring_load_impl(h, g, r, first_pos, rows, n));
}

static int verify_step_impl(kv_hier_t* h, int g, const void* queries, const int32_t* topk_idx,
                        const int32_t* causal_pos, const void* ring_rows, void* out, void* stream) {
  int rc = check_group(h, g);
  if (rc) return rc;
  if (!queries || !causal_pos || !out) return fail(h, KV_EINVAL, "null device pointer");
  {
    const Group& G0 = h->grp[g];
    if (G0.member == 0 && !topk_idx) return fail(h, KV_EINVAL, "null device pointer");
    if (G0.member != 0 && h->grp[G0.leader].t != G0.t + 1)
      return fail(h, KV_ESTATE, "group %d uses the plan of group %d: call that group's step first, once per step",
                  g, G0.leader);
  }
  begin_work(h);
  const kv_hier_config& c = h->cfg;
  hipStream_t caller = static_cast<hipStream_t>(stream);
  hipStream_t s = caller;
  if (h->work) {           // the step runs on the partitioned stream, ordered after the caller's work
    HIPCHK(h, hipEventRecord(h->ev_in, caller));
    HIPCHK(h, hipStreamWaitEvent(h->work, h->ev_in, 0));
    s = h->work;
  }
  Group& G = h->grp[g];
  Group& P = h->grp[G.leader];      // owner of the plan state (G itself unless a follower)
  const bool lead = G.member == 0;
  // rows of the last commit are still in the tail (resolved from the ring);
  // those of the commit before may be fetched from the host or have their ring
  // slots rewritten by this step: its backup must be complete (the side
  // stream's fetches of this step follow the first fetch on this stream)
  if (h->backup && h->n_commits >= 2) HIPCHK(h, hipStreamWaitEvent(s, h->ev_backup[h->n_commits % 2], 0));
  const int N = c.n_req;
  const int a = g % c.n_arenas;
  if (lead) {
    G.t += 1;
  } else {
    G.t = P.t;
  }
  G.calls += 1;

  int ti = -1;
  // null ring_rows: the source's producer already wrote this step's rows (a
  // Reindex consumer); a leader's plan writes them itself (below)
  if (ring_rows && !lead) {
    ti = time_begin(h, K_RING, g, s);
    HIPCHK(h, launch_ring_write(static_cast<const uint4*>(ring_rows), causal_pos, reinterpret_cast<uint4*>(G.ring),
                                N, c.q_max, h->Rd, h->row16, s));
    time_end(h, ti, s);
  }
  if (lead) {
    // The resolution plan and the first chunk's host fetch run on this stream,
    // after the caller's prior work: no hop between streams lies between the
    // caller's work, the plan, the first fetch and the first attention (each
    // hop costs about as much as a short kernel).  The side stream fetches the
    // other chunks once the first fetch is done, so after the plan.
    // The plan rewrites the set's lists, counts and (through the victims) its
    // slot tables: every group of the set must have finished reading the
    // previous ones (its attention, copy-back and counters, all before its
    // ev_done), whatever stream its step was issued on.
    for (int m = 0; m < h->share; ++m)
      if (h->grp[g + m].done_recorded) HIPCHK(h, hipStreamWaitEvent(s, h->grp[g + m].ev_done, 0));
    // optional-history pages whose copies have completed become ready for
    // this step's resolution (the first group's step is the step boundary)
    if (g == 0 && h->opt.on && !h->no_alloc_call && (rc = opt_publish_impl(h, false))) return rc;
    // resident-map updates issued since this group's last plan
    if (G.map_wait) {
      HIPCHK(h, hipStreamWaitEvent(s, h->ev_map, 0));
      G.map_wait = false;
    }

    PlanArgs pa;
    pa.topk = topk_idx;
    pa.causal = causal_pos;
    pa.res_map = G.res_map;
    pa.ring_lo = G.ring_lo;
    pa.Rd = h->Rd;
    pa.m = G.m;
    pa.has_resident = (h->opt.on ? h->opt.n_published > 0 : G.res_cursor > 0) ? 1 : 0;
    pa.slot_map = G.slot_map;
    pa.slot_row = G.slot_row;
    pa.slot_lu = G.slot_lu;
    pa.union_rows = G.union_rows;
    pa.union_loc = G.union_loc;
    pa.miss_rows = G.miss_rows;
    pa.victims = G.victims;
    pa.protect = G.protect;
    pa.loc = G.loc;
    pa.sloc = h->row_order ? G.sloc : nullptr;
    pa.req_info = G.req_info;
    pa.req_counts = G.req_counts;
    pa.cum = G.cum;
    pa.N = N;
    pa.Q = c.q_max;
    pa.k = c.topk;
    pa.B = c.hot_slots;
    pa.L = h->L;
    pa.t = G.t;
    pa.chunk_words = h->chunk_words;
    pa.sort_cap = h->sort_cap;
    pa.ring_rows = static_cast<const uint4*>(ring_rows);
    pa.ring = reinterpret_cast<uint4*>(G.ring);
    pa.row16 = h->row16;
    {
      const LaunchEv le = launch_events(h, K_PLAN, g, h->ev_planned);
      HIPCHK(h, launch_plan(pa, h->plan_lds, s, le.start, le.stop));
      if (le.after) HIPCHK(h, hipEventRecord(le.after, s));
    }
    // LRU victims on the copy-back stream right after the plan: they run
    // while the first chunk is fetched, when few other kernels hold CUs (each
    // of their workgroups excludes an attention workgroup from its CU), and
    // the copy-backs that need them follow on the same stream.  The group's
    // next plan sees the updated slot tables through its ev_done.
    HIPCHK(h, hipStreamWaitEvent(h->aux, h->ev_planned, 0));
    ti = time_begin(h, K_VICTIMS, g, h->aux);
    HIPCHK(h, launch_plan_victims(pa, h->plan_lds, h->aux));
    time_end(h, ti, h->aux);
    // the row-ordered lists on the fetch stream, ahead of every fetch issued
    // there: they run beside the first chunk's fetch, and the attention of
    // every chunk fetched there (all but the leader's first) is ordered after
    // them through its fetch.  A wait of the caller's stream for a kernel on
    // the copy-back stream instead slowed every later attention launch by a
    // quarter (127 -> 159 us at the 128-request shape).
    if (h->row_order) {
      HIPCHK(h, hipStreamWaitEvent(h->side, h->ev_planned, 0));
      ti = time_begin(h, K_ORDER, g, h->side);
      HIPCHK(h, launch_plan_order(pa, h->order_lds, h->side));
      time_end(h, ti, h->side);
    }

    // host fetch of every chunk, for this group and then for every follower
    // layer of its plan (one selection starts the transfers of all of them;
    // each layer fetches its own bytes into its own arena)
    for (int m = 0; m < h->share; ++m) {
      const int gm = g + m, am = gm % c.n_arenas;
      const HostRowSrc src = host_src(h, h->grp[gm]);
      for (int ch = 0; ch < h->n_chunks; ++ch) {
        const int r0 = h->chunk_lo[ch], r1 = h->chunk_lo[ch + 1];
        const bool here = m == 0 && ch == 0;      // the leader's first chunk: this stream
        hipStream_t fs = here ? s : h->side;
        // every chunk of an arena is released at once (after the arena's last
        // readers); later chunks follow this wait on the same stream or, for
        // the leader's arena, the first fetch
        if (ch == 0 && h->free_recorded[am]) HIPCHK(h, hipStreamWaitEvent(fs, h->ev_free[am], 0));
        if (c.flags & KV_FLAG_POISON) {
          // debug: between the chunk's last readers and its next fetch the arena
          // holds NaN, so a read outside that order shows in the outputs
          const size_t words = size_t(r1 - r0) * h->QK * c.row_elems / 2;
          HIPCHK(h, launch_fill32(reinterpret_cast<uint32_t*>(h->arena[am] + size_t(r0) * h->QK * c.row_elems),
                                  0x7fc07fc0u, words, fs));
        }
        // 128 one-wave workgroups: enough host reads in flight to fill the link;
        // more only queue in the memory system and slow the attention beside them
        const int wgs = c.fetch_wgs > 0 ? c.fetch_wgs : 128;
        const int wpr = std::max(1, wgs / std::max(1, r1 - r0));
        // the chunk's fetched event is the launch's own end (no marker) unless timing holds it
        const LaunchEv le = launch_events(h, K_GATHER, gm, h->ev_fetched[m][ch]);
        HIPCHK(h, launch_miss_gather(src, G.miss_rows, G.req_info, reinterpret_cast<uint4*>(h->arena[am]), h->QK,
                                     r0, r1, wpr, fs, le.start, le.stop));
        if (le.after) HIPCHK(h, hipEventRecord(le.after, fs));
        if (here) HIPCHK(h, hipStreamWaitEvent(h->side, h->ev_fetched[0][0], 0));
      }
      h->arena_owner[am] = gm;
      h->arena_step[am] = G.t;
    }
  }
  // attention per chunk on the caller's stream, copy-back on the copy-back stream
  AttnArgs at;
  at.q = static_cast<const uint16_t*>(queries);
  at.loc = P.loc;
  at.causal = causal_pos;
  at.ring_lo = G.ring_lo;
  at.hot = G.hot;
  at.staging = h->arena[a];
  at.resident = G.resident;
  at.ring = G.ring;
  at.zero = h->zero_row;
  at.out = static_cast<uint16_t*>(out);
  at.part_o = h->part_o;
  at.part_ml = h->part_ml;
  if (h->no_alloc_call) {
    // the same partials, in this device's static scratch (size checked before any work)
    at.part_o = reinterpret_cast<float*>(h->scratch_dev);
    at.part_ml = at.part_o + h->step_part_heads * size_t(c.d_v);
  }
  at.N = N;
  at.Q = c.q_max;
  at.k = c.topk;
  at.H = c.n_heads;
  at.W = c.ring_window;
  at.Rd = h->Rd;
  at.block_only = c.ring_block_only ? 1 : 0;
  const float scale = c.softmax_scale > 0.f ? c.softmax_scale : 1.0f / std::sqrt(float(c.d_qk));
  at.scale_log2 = scale * 1.4426950408889634f;
  // The hot slots promoted by this group's previous step are complete before
  // any chunk's attention: the leader's plan (this stream, or the leader's
  // for a follower) waited for every set member's ev_done before the first
  // fetch, and every chunk's attention follows a fetch of this step.
  if (c.flags & KV_FLAG_SERIAL) HIPCHK(h, hipStreamWaitEvent(s, h->ev_fetched[G.member][h->n_chunks - 1], 0));
  for (int ch = 0; ch < h->n_chunks; ++ch) {
    at.r0 = h->chunk_lo[ch];
    at.r1 = h->chunk_lo[ch + 1];
    at.splits = h->chunk_splits[ch];
    at.hpw = h->chunk_hpw[ch];
    at.head_groups = (c.n_heads + at.hpw - 1) / at.hpw;
    // the row-ordered lists, for every chunk fetched on the fetch stream
    // (after them); the leader's first chunk, fetched here right after the
    // plan, walks the selection order
    at.loc = h->row_order && !(lead && ch == 0) ? P.sloc : P.loc;
    // the leader's first chunk was fetched on this stream
    if (!(lead && ch == 0)) HIPCHK(h, hipStreamWaitEvent(s, h->ev_fetched[G.member][ch], 0));
    if ((rc = attend(h, g, at, s))) return rc;
    // copy-back on the aux stream, after the victims (issued there by the
    // leader's step) and the chunk's fetch, concurrent with the attention
    // (victim slots are not read by the step)
    // a follower's counters are its plan's: copy the leader's last-step counts
    if (ch == 0 && !lead) HIPCHK(h, launch_counts_follow(P.req_counts, G.req_counts, G.cum, N, h->aux));
    HIPCHK(h, hipStreamWaitEvent(h->aux, h->ev_fetched[G.member][ch], 0));
    ti = time_begin(h, K_PROMOTE, g, h->aux);
    HIPCHK(h, launch_promote(reinterpret_cast<const uint4*>(h->arena[a]), P.victims, P.req_info,
                             reinterpret_cast<uint4*>(G.hot), h->QK, c.hot_slots, h->row16, at.r0, at.r1, h->aux));
    time_end(h, ti, h->aux);
  }
  // One event after the group's last attention chunk (an event record costs
  // the stream a few microseconds, so there is none per chunk): a Reuse of
  // this selection waits for it, and the arena is released after it and the
  // copy-backs (a later fetch into any chunk then waits for every chunk's
  // readers, which it does anyway when it belongs to a later step of the
  // caller's stream).
  HIPCHK(h, hipEventRecord(G.ev_sel, s));
  G.sel_recorded = true;
  G.sel_valid = true;
  HIPCHK(h, hipStreamWaitEvent(h->aux, G.ev_sel, 0));
  HIPCHK(h, hipEventRecord(h->ev_free[a], h->aux));
  h->free_recorded[a] = 1;
  // the group's hot cache is complete after its copy-backs: the group's next
  // attention waits for this
  HIPCHK(h, hipEventRecord(G.ev_done, h->aux));
  G.done_recorded = true;
  if (h->work) {
    HIPCHK(h, hipEventRecord(h->ev_out, s));
    HIPCHK(h, hipStreamWaitEvent(caller, h->ev_out, 0));
  }
  return KV_OK;
}

int kv_hier_verify_step(kv_hier_t* h, int g, const void* queries, const int32_t* topk_idx,
                        const int32_t* causal_pos, const void* ring_rows, void* out, void* stream) {
  DeviceGuard dg(h);
  if (int rc = refuse_if_broken(h)) return rc;
  return finish(h, verify_step_impl(h, g, queries, topk_idx, causal_pos, ring_rows, out, stream));
}

int kv_hier_verify_step_static(kv_hier_t* h, int g, const void* queries, const int32_t* topk_idx,
                               const int32_t* causal_pos, const void* ring_rows, void* out, void* stream) {
  DeviceGuard dg(h);
  if (!h) return KV_EINVAL;
  if (int rc = refuse_if_broken(h)) return rc;
  const size_t need = h->step_part_heads * (size_t(h->cfg.d_v) + 2) * sizeof(float);
  if (need > kStaticScratchBytes)
    return fail(h, KV_EINVAL,
                "split-key partials of this handle's steps take %zu bytes, over the %zu-byte static scratch", need,
                kStaticScratchBytes);
  h->no_alloc_call = true;
  const int rc = finish(h, verify_step_impl(h, g, queries, topk_idx, causal_pos, ring_rows, out, stream));
  h->no_alloc_call = false;
  return rc;
}

static int verify_reuse_impl(kv_hier_t* h, int g, const void* queries, const int32_t* causal_pos, void* out,
                         void* stream) {
  int rc = check_group(h, g);
  if (rc) return rc;
  if (!queries || !causal_pos || !out) return fail(h, KV_EINVAL, "null device pointer");
  const kv_hier_config& c = h->cfg;
  Group& G = h->grp[g];
  const Group& P = h->grp[G.leader];
  const int a = g % c.n_arenas;
  if (!G.sel_valid) return fail(h, KV_ESTATE, "group %d has no selection of this step to reuse", g);
  if (h->arena_owner[a] != g || h->arena_step[a] != G.t)
    return fail(h, KV_ESTATE, "the staged payload of group %d was replaced by a later fetch into arena %d", g, a);
  begin_work(h);
  hipStream_t caller = static_cast<hipStream_t>(stream);
  hipStream_t s = caller;
  if (h->work) {
    HIPCHK(h, hipEventRecord(h->ev_in, caller));
    HIPCHK(h, hipStreamWaitEvent(h->work, h->ev_in, 0));
    s = h->work;
  }
  // the latest selection's locations and payload, read by the new queries
  AttnArgs at;
  at.q = static_cast<const uint16_t*>(queries);
  at.loc = P.loc;
  at.causal = causal_pos;
  at.ring_lo = G.ring_lo;
  at.hot = G.hot;
  at.staging = h->arena[a];
  at.resident = G.resident;
  at.ring = G.ring;
  at.zero = h->zero_row;
  at.out = static_cast<uint16_t*>(out);
  at.part_o = h->part_o;
  at.part_ml = h->part_ml;
  at.N = c.n_req;
  at.Q = c.q_max;
  at.k = c.topk;
  at.H = c.n_heads;
  at.W = c.ring_window;
  at.Rd = h->Rd;
  at.block_only = c.ring_block_only ? 1 : 0;
  const float scale = c.softmax_scale > 0.f ? c.softmax_scale : 1.0f / std::sqrt(float(c.d_qk));
  at.scale_log2 = scale * 1.4426950408889634f;
  // the selection's ring rows, staged rows and lists are complete once its
  // step's attention ran (that step waited for every fetch chunk)
  if (G.sel_recorded) HIPCHK(h, hipStreamWaitEvent(s, G.ev_sel, 0));
  at.r0 = 0;
  at.r1 = c.n_req;
  at.splits = h->all_splits;
  at.hpw = h->all_hpw;
  at.head_groups = (c.n_heads + at.hpw - 1) / at.hpw;
  int rc2 = attend(h, g, at, s);
  if (rc2) return rc2;
  // the arena is released once this reader and the step's own readers and
  // copy-backs are done: the release events now follow all of them
  if (h->free_recorded[a]) HIPCHK(h, hipStreamWaitEvent(s, h->ev_free[a], 0));
  HIPCHK(h, hipEventRecord(h->ev_free[a], s));
  h->free_recorded[a] = 1;
  if (h->work) {
    HIPCHK(h, hipEventRecord(h->ev_out, s));
    HIPCHK(h, hipStreamWaitEvent(caller, h->ev_out, 0));
  }
  return KV_OK;
}

int kv_hier_verify_reuse(kv_hier_t* h, int g, const void* queries, const int32_t* causal_pos, void* out,
                         void* stream) {
  DeviceGuard dg(h);
  if (int rc = refuse_if_broken(h)) return rc;
  return finish(h, verify_reuse_impl(h, g, queries, causal_pos, out, stream));
}

static int commit_src_impl(kv_hier_t* h, const int32_t* accepted, const void* const* src_rows, void* stream) {
  if (!h || !accepted) return KV_EINVAL;
  const kv_hier_config& c = h->cfg;
  const int N = c.n_req, G = c.n_groups;
  bool any_compressed = false;
  for (int g = 0; g < G; ++g) {
    if (h->grp[g].m == 1) continue;
    any_compressed = true;
    if (!src_rows || !src_rows[g])
      return fail(h, KV_EINVAL, "group %d stores compressed rows: its completed rows are needed", g);
  }
  for (int r = 0; r < N; ++r) {
    const int a = accepted[r];
    if (a < -1 || a >= c.q_max) return fail(h, KV_EINVAL, "accepted[%d] = %d outside [-1, %d)", r, a, c.q_max);
    if (a >= 0) {
      if (int64_t(h->hist_len[r]) + 1 + a > c.hist_cap) return fail(h, KV_EINVAL, "request %d: history full", r);
      if (h->hist_len[r] < h->plen) return fail(h, KV_EINVAL, "request %d: frontier inside the shared prefix", r);
      for (int g = 0; g < G; ++g)
        if (h->grp[g].m > 1 && h->hist_len[r] / h->grp[g].m < h->plen)
          return fail(h, KV_EINVAL, "request %d: stored rows of group %d inside the shared prefix", r, g);
    }
  }
  begin_work(h);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // staging buffer of this commit: the one whose copy was issued kCommitBufs
  // commits ago (the host waits only if that copy has not run yet)
  const int cb = int(h->n_commits % kCommitBufs);
  if (h->commit_pending[cb]) {
    HIPCHK(h, hipEventSynchronize(h->ev_commit[cb]));
    h->commit_pending[cb] = false;
  }
  int32_t* hc = h->h_commit[cb];
  const uint4** hs = h->h_src[cb];
  for (int r = 0; r < N; ++r) {
    hc[r] = h->hist_len[r];
    hc[N + r] = accepted[r];
  }
  for (int g = 0; g < G; ++g)
    hs[g] = (src_rows && h->grp[g].m > 1) ? static_cast<const uint4*>(src_rows[g]) : nullptr;
  // the previous backup still reads the device commit buffers until it ends
  if (h->backup && h->n_commits >= 1) HIPCHK(h, hipStreamWaitEvent(s, h->ev_backup[(h->n_commits - 1) % 2], 0));
  HIPCHK(h, hipMemcpyAsync(h->d_commit, hc, size_t(2) * N * 4, hipMemcpyHostToDevice, s));
  HIPCHK(h, hipMemcpyAsync(const_cast<uint4**>(h->d_src), hs, size_t(G) * sizeof(void*), hipMemcpyHostToDevice, s));
  HIPCHK(h, hipEventRecord(h->ev_commit[cb], s));
  h->commit_pending[cb] = true;
  // compressed sources: the caller's rows are consumed in its stream order, so
  // their host copy exists before the next step fetches (they have no tail)
  if (any_compressed)
    HIPCHK(h, launch_commit(h->d_commit_groups, G, h->d_commit, h->d_commit + N, h->d_src, 1, N, c.q_max, h->Rd,
                            h->plen, h->tail_rows, h->row16, s));
  // the other groups' backup reads the ring rows the step wrote: after the
  // caller's work, on the backup stream when there is one
  hipStream_t b = s;
  const bool async = h->backup && !(c.flags & KV_FLAG_SYNC_BACKUP);
  if (async) {
    HIPCHK(h, hipEventRecord(h->ev_verified, s));
    HIPCHK(h, hipStreamWaitEvent(h->backup, h->ev_verified, 0));
    b = h->backup;
  }
  HIPCHK(h, launch_commit(h->d_commit_groups, G, h->d_commit, h->d_commit + N, h->d_src, 0, N, c.q_max, h->Rd,
                          h->plen, h->tail_rows, h->row16, b));
  if (h->backup) HIPCHK(h, hipEventRecord(h->ev_backup[h->n_commits % 2], b));
  h->n_commits += 1;
  for (int r = 0; r < N; ++r)
    if (accepted[r] >= 0) h->hist_len[r] += 1 + accepted[r];
  for (Group& G2 : h->grp) G2.sel_valid = false;     // the step's selections end with its commit
  return KV_OK;
}

int kv_hier_commit_src(kv_hier_t* h, const int32_t* accepted, const void* const* src_rows, void* stream) {
  DeviceGuard dg(h);
  if (int rc = refuse_if_broken(h)) return rc;
  return finish(h, commit_src_impl(h, accepted, src_rows, stream));
}

int kv_hier_commit(kv_hier_t* h, const int32_t* accepted, void* stream) {
  DeviceGuard dg(h);
  return kv_hier_commit_src(h, accepted, nullptr, stream);
}

static int set_compression_impl(kv_hier_t* h, int g, int32_t m) {
  int rc = check_group(h, g);
  if (rc) return rc;
  Group& G = h->grp[g];
  if (m < 1) return fail(h, KV_EINVAL, "positions per stored row must be >= 1");
  if (G.calls > 0) return fail(h, KV_ESTATE, "group %d has already run a step", g);
  if (m > 1 && h->opt.on) return fail(h, KV_ESTATE, "dynamic residency pages assume uncompressed sources");
  if (m > 1 && h->share > 1) return fail(h, KV_ESTATE, "plan-sharing sets assume uncompressed sources");
  begin_work(h);
  if ((rc = sync_all(h))) return rc;
  G.m = m;
  CommitGroup cg;
  cg.ring = reinterpret_cast<const uint4*>(G.ring);
  cg.tails = const_cast<uint4*>(G.tails_dev);
  cg.m = m;
  cg.cmax = (h->cfg.q_max + m - 1) / m;
  return upload(h, h->d_commit_groups + g, &cg, sizeof cg);
}

int kv_hier_set_compression(kv_hier_t* h, int g, int32_t m) {
  DeviceGuard dg(h);
  if (int rc = refuse_if_broken(h)) return rc;
  return finish(h, set_compression_impl(h, g, m));
}

int kv_hier_stats(kv_hier_t* h, int g, kv_hier_counters* cum, kv_hier_counters* last) {
  DeviceGuard dg(h);
  int rc = check_group(h, g);
  if (rc) return rc;
  if ((rc = sync_all(h))) return rc;
  Group& G = h->grp[g];
  const int N = h->cfg.n_req;
  unsigned long long cv[C_NUM];
  std::vector<int64_t> rq(size_t(N) * C_NUM);
  if ((rc = download(h, cv, G.cum, sizeof cv))) return rc;
  if ((rc = download(h, rq.data(), G.req_counts, rq.size() * 8))) return rc;
  auto fill = [&](kv_hier_counters* o, const int64_t* v, int64_t calls, bool timing) {
    std::memset(o, 0, sizeof *o);
    o->calls = calls;
    o->active_requests = v[C_ACTIVE_REQ];
    o->active_queries = v[C_ACTIVE_Q];
    o->selections = v[C_SEL];
    o->pads = v[C_PAD];
    o->invalid = v[C_INVALID];
    o->union_rows = v[C_UNION];
    o->union_resident = v[C_U_RES];
    o->union_hot = v[C_U_HOT];
    o->union_miss = v[C_U_MISS];
    o->fetched_bytes = v[C_U_MISS] * int64_t(h->row_bytes);
    o->promoted = v[C_PROMOTED];
    o->overflow = v[C_OVERFLOW];
    o->sel_resident = v[C_S_RES];
    o->sel_hot = v[C_S_HOT];
    o->sel_miss = v[C_S_MISS];
    o->union_tail = v[C_U_TAIL];
    o->sel_tail = v[C_S_TAIL];
    if (timing) {
      o->ms_ring = G.ms[K_RING];
      o->ms_plan = G.ms[K_PLAN];
      o->ms_gather = G.ms[K_GATHER];
      o->ms_attn = G.ms[K_ATTN];
      o->ms_combine = G.ms[K_COMBINE];
      o->ms_promote = G.ms[K_PROMOTE];
      o->ms_victims = G.ms[K_VICTIMS];
      o->n_ring = G.nt[K_RING];
      o->n_plan = G.nt[K_PLAN];
      o->n_gather = G.nt[K_GATHER];
      o->n_attn = G.nt[K_ATTN];
      o->n_combine = G.nt[K_COMBINE];
      o->n_promote = G.nt[K_PROMOTE];
      o->n_victims = G.nt[K_VICTIMS];
      o->ms_order = G.ms[K_ORDER];
      o->n_order = G.nt[K_ORDER];
    }
  };
  if (cum) {
    int64_t v[C_NUM];
    for (int i = 0; i < C_NUM; ++i) v[i] = int64_t(cv[i]);
    fill(cum, v, G.calls, true);
  }
  if (last) {
    int64_t v[C_NUM] = {0};
    for (int r = 0; r < N; ++r)
      for (int i = 0; i < C_NUM; ++i) v[i] += rq[size_t(r) * C_NUM + i];
    fill(last, v, G.calls > 0 ? 1 : 0, false);
  }
  return KV_OK;
}

int kv_hier_reset_stats(kv_hier_t* h) {
  DeviceGuard dg(h);
  if (!h) return KV_EINVAL;
  int rc = sync_all(h);
  if (rc) return rc;
  for (Group& G : h->grp) {
    HIPCHK(h, launch_fill32(reinterpret_cast<uint32_t*>(G.cum), 0, size_t(C_NUM) * 2, nullptr));
    G.calls = 0;
    for (int i = 0; i < K_NUM; ++i) { G.ms[i] = 0; G.nt[i] = 0; }
  }
  HIPCHK(h, hipDeviceSynchronize());
  return KV_OK;
}

int kv_hier_last_lists(kv_hier_t* h, int g, int r, kv_hier_lists* o) {
  DeviceGuard dg(h);
  int rc = check_group(h, g);
  if (rc) return rc;
  if ((rc = check_req(h, r))) return rc;
  if (!o || !o->union_rows || !o->union_loc || !o->miss_rows || !o->victims || !o->loc)
    return fail(h, KV_EINVAL, "null list buffer");
  if ((rc = sync_all(h))) return rc;
  Group& G = h->grp[h->grp[g].leader];   // lists belong to the plan (the leader's for a follower)
  int32_t info[I_NUM];
  if ((rc = download(h, info, G.req_info + size_t(r) * I_NUM, sizeof info))) return rc;
  const size_t base = size_t(r) * h->QK;
  o->n_union = info[I_NUNION];
  o->n_miss = info[I_NMISS];
  o->n_promote = info[I_NPROMOTE];
  o->n_active = info[I_NACTIVE];
  if ((rc = download(h, o->union_rows, G.union_rows + base, size_t(o->n_union) * 4))) return rc;
  if ((rc = download(h, o->union_loc, G.union_loc + base, size_t(o->n_union) * 4))) return rc;
  if ((rc = download(h, o->miss_rows, G.miss_rows + base, size_t(o->n_miss) * 4))) return rc;
  if ((rc = download(h, o->victims, G.victims + base, size_t(o->n_promote) * 4))) return rc;
  return download(h, o->loc, G.loc + base, size_t(h->QK) * 4);
}

int kv_hier_slot_table(kv_hier_t* h, int g, int r, int32_t* rows, int32_t* last_used) {
  DeviceGuard dg(h);
  int rc = check_group(h, g);
  if (rc) return rc;
  if ((rc = check_req(h, r))) return rc;
  if (!rows || !last_used) return fail(h, KV_EINVAL, "null output");
  if ((rc = sync_all(h))) return rc;
  const int B = h->cfg.hot_slots;
  const Group& G = h->grp[h->grp[g].leader];   // the plan's slot table (shared by its followers)
  if ((rc = download(h, rows, G.slot_row + size_t(r) * B, size_t(B) * 4))) return rc;
  return download(h, last_used, G.slot_lu + size_t(r) * B, size_t(B) * 4);
}

int kv_hier_read_rows(kv_hier_t* h, int g, const int32_t* locs, int n, void* rows) {
  DeviceGuard dg(h);
  int rc = check_group(h, g);
  if (rc) return rc;
  if (n < 0 || (n > 0 && (!locs || !rows))) return fail(h, KV_EINVAL, "bad read_rows arguments");
  if (n == 0) return KV_OK;
  const kv_hier_config& c = h->cfg;
  Group& G = h->grp[g];
  for (int i = 0; i < n; ++i) {
    const int32_t code = locs[i];
    if (code == -1) continue;
    if (code < 0) return fail(h, KV_EINVAL, "location code %d", code);
    const int tier = loc_tier(code);
    const int64_t idx = loc_index(code);
    const int64_t lim = tier == kTierHot ? int64_t(c.n_req) * c.hot_slots
                        : tier == kTierStaged ? int64_t(c.n_req) * h->QK
                        : tier == kTierResident ? c.resident_cap : int64_t(c.n_req) * h->Rd;
    if (idx >= lim) return fail(h, KV_EINVAL, "location %d beyond its pool", code);
  }
  if ((rc = sync_all(h))) return rc;
  int32_t* dl = nullptr;
  uint16_t* dr = nullptr;
  if ((rc = dev_alloc(h, &dl, size_t(n), nullptr))) return rc;
  if ((rc = dev_alloc(h, &dr, size_t(n) * c.row_elems, nullptr))) { (void)hipFree(dl); return rc; }
  PoolView pv;
  pv.hot = reinterpret_cast<const uint4*>(G.hot);
  pv.staging = reinterpret_cast<const uint4*>(h->arena[g % c.n_arenas]);
  pv.resident = reinterpret_cast<const uint4*>(G.resident);
  pv.ring = reinterpret_cast<const uint4*>(G.ring);
  rc = upload(h, dl, locs, size_t(n) * 4);
  if (!rc) {
    hipError_t e = launch_read_rows(pv, dl, n, reinterpret_cast<uint4*>(dr), h->row16, nullptr);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) rc = fail(h, KV_EHIP, "read_rows: %s", hipGetErrorString(e));
  }
  if (!rc) rc = download(h, rows, dr, size_t(n) * h->row_bytes);
  (void)hipFree(dl);
  (void)hipFree(dr);
  return rc;
}

int kv_hier_sync(kv_hier_t* h) {
  DeviceGuard dg(h);
  if (!h) return KV_EINVAL;
  return sync_all(h);
}

int kv_hier_set_flags(kv_hier_t* h, int32_t flags) {
  DeviceGuard dg(h);
  if (!h) return KV_EINVAL;
  if (flags & ~(KV_FLAG_TIMING | KV_FLAG_POISON | KV_FLAG_TIMING_ATTN | KV_FLAG_SERIAL | KV_FLAG_SYNC_BACKUP |
                KV_FLAG_TEST_FAIL_ATTN))
    return fail(h, KV_EINVAL, "unknown flags %d", flags);
  int rc = sync_all(h);
  if (rc) return rc;
  h->cfg.flags = flags;
  return KV_OK;
}

static int cache_snapshot_impl(kv_hier_t* h, int g, int op) {
  int rc = check_group(h, g);
  if (rc) return rc;
  if (op != 0 && op != 1) return fail(h, KV_EINVAL, "snapshot op %d", op);
  if (op == 1 && h->grp[g].snap_t < 0) return fail(h, KV_ESTATE, "no snapshot of group %d", g);
  begin_work(h);
  if ((rc = sync_all(h))) return rc;
  Group& G = h->grp[g];
  const size_t NB = size_t(h->cfg.n_req) * h->cfg.hot_slots, NL = size_t(h->cfg.n_req) * h->L;
  const size_t hot_bytes = NB * h->row_bytes;
  if (op == 0) {
    if (!G.snap_hot) {
      if ((rc = dev_alloc(h, &G.snap_hot, NB * h->cfg.row_elems, nullptr))) return rc;
      if ((rc = dev_alloc(h, &G.snap_row, NB, nullptr))) return rc;
      if ((rc = dev_alloc(h, &G.snap_lu, NB, nullptr))) return rc;
      if ((rc = dev_alloc(h, &G.snap_map, NL, nullptr))) return rc;
    }
    HIPCHK(h, hipMemcpy(G.snap_hot, G.hot, hot_bytes, hipMemcpyDeviceToDevice));
    HIPCHK(h, hipMemcpy(G.snap_row, G.slot_row, NB * 4, hipMemcpyDeviceToDevice));
    HIPCHK(h, hipMemcpy(G.snap_lu, G.slot_lu, NB * 4, hipMemcpyDeviceToDevice));
    HIPCHK(h, hipMemcpy(G.snap_map, G.slot_map, NL * 4, hipMemcpyDeviceToDevice));
    G.snap_t = G.t;
  } else {
    if (G.snap_t < 0) return fail(h, KV_ESTATE, "no snapshot of group %d", g);
    HIPCHK(h, hipMemcpy(G.hot, G.snap_hot, hot_bytes, hipMemcpyDeviceToDevice));
    HIPCHK(h, hipMemcpy(G.slot_row, G.snap_row, NB * 4, hipMemcpyDeviceToDevice));
    HIPCHK(h, hipMemcpy(G.slot_lu, G.snap_lu, NB * 4, hipMemcpyDeviceToDevice));
    HIPCHK(h, hipMemcpy(G.slot_map, G.snap_map, NL * 4, hipMemcpyDeviceToDevice));
    G.t = G.snap_t;
  }
  HIPCHK(h, hipDeviceSynchronize());
  return KV_OK;
}

int kv_hier_cache_snapshot(kv_hier_t* h, int g, int op) {
  DeviceGuard dg(h);
  if (int rc = refuse_if_broken(h)) return rc;
  return finish(h, cache_snapshot_impl(h, g, op));
}

// ---------------------------------------------------------------- dynamic optional residency

static int opt_admit_impl(kv_hier_t* h, int r, int32_t required_pages, const int32_t* order, int n_order,
                      int32_t* n_reclaimed) {
  if (!h) return KV_EINVAL;
  Opt& o = h->opt;
  if (!o.on) return fail(h, KV_ESTATE, "dynamic residency is off (opt_page_rows = 0)");
  int rc = check_req(h, r);
  if (rc) return rc;
  if (o.admitted[r]) return fail(h, KV_ESTATE, "request %d is already admitted", r);
  if (required_pages < 0 || n_order < 0 || (n_order > 0 && !order))
    return fail(h, KV_EINVAL, "bad admission arguments");
  std::vector<char> seen(h->cfg.n_req, 0);
  for (int i = 0; i < n_order; ++i) {
    const int x = order[i];
    if (x < 0 || x >= h->cfg.n_req || !o.admitted[x] || seen[x])
      return fail(h, KV_EINVAL, "reclaim order entry %d (%d) is not a distinct admitted request", i, x);
    seen[x] = 1;
  }
  // eq. (3): required + optional + reserve <= M; eq. (4): the first q of the
  // reclaim order whose optional pages cover the deficit
  const int64_t deficit = o.sum_req + required_pages + o.sum_held + o.reserve - int64_t(o.M);
  int q = 0;
  if (deficit > 0) {
    int64_t covered = 0;
    while (q < n_order && covered < deficit) covered += o.n_held[order[q++]];
    if (covered < deficit) {
      o.admissions_waited += 1;
      return fail(h, KV_EWAIT, "admission of request %d waits: deficit %lld pages, reclaimable %lld", r,
                  (long long)deficit, (long long)covered);
    }
  }
  begin_work(h);
  for (int i = 0; i < q; ++i)
    if ((rc = opt_drop(h, order[i]))) return rc;
  o.requests_reclaimed += q;
  o.admitted[r] = 1;
  o.required[r] = required_pages;
  o.sum_req += required_pages;
  o.eligible[r] = std::min(h->hist_len[r], h->L) / o.P;   // complete imported pages
  o.held[r].assign(o.eligible[r], -1);
  o.n_held[r] = 0;
  o.n_ready[r] = 0;
  if (n_reclaimed) *n_reclaimed = q;
  return KV_OK;
}

int kv_hier_opt_admit(kv_hier_t* h, int r, int32_t required_pages, const int32_t* order, int n_order,
                      int32_t* n_reclaimed) {
  DeviceGuard dg(h);
  if (int rc = refuse_if_broken(h)) return rc;
  return finish(h, opt_admit_impl(h, r, required_pages, order, n_order, n_reclaimed));
}

static int opt_complete_impl(kv_hier_t* h, int r) {
  if (!h) return KV_EINVAL;
  Opt& o = h->opt;
  if (!o.on) return fail(h, KV_ESTATE, "dynamic residency is off (opt_page_rows = 0)");
  int rc = check_req(h, r);
  if (rc) return rc;
  if (!o.admitted[r]) return fail(h, KV_ESTATE, "request %d is not admitted", r);
  begin_work(h);
  if ((rc = opt_drop(h, r))) return rc;
  o.admitted[r] = 0;
  o.sum_req -= o.required[r];
  o.required[r] = 0;
  o.eligible[r] = 0;
  o.held[r].clear();
  return KV_OK;
}

int kv_hier_opt_complete(kv_hier_t* h, int r) {
  DeviceGuard dg(h);
  if (int rc = refuse_if_broken(h)) return rc;
  return finish(h, opt_complete_impl(h, r));
}

static int opt_populate_impl(kv_hier_t* h, int32_t max_pages, int32_t* n_assigned) {
  if (!h) return KV_EINVAL;
  Opt& o = h->opt;
  if (!o.on) return fail(h, KV_ESTATE, "dynamic residency is off (opt_page_rows = 0)");
  if (max_pages < 0) return fail(h, KV_EINVAL, "negative page bound");
  begin_work(h);
  const int N = h->cfg.n_req;
  const int64_t budget = int64_t(o.M) - o.sum_req - o.reserve - o.sum_held;
  const int64_t limit = std::min<int64_t>(max_pages, std::max<int64_t>(0, budget));
  std::vector<int32_t> ent, copy;
  bool wait = false;
  int r = o.cursor, idle = 0;
  int64_t n = 0;
  while (n < limit && idle < N) {
    if (o.admitted[r] && o.n_held[r] < o.eligible[r]) {
      const int idx = o.n_held[r];          // held pages always form a prefix 0 .. n_held-1
      const int32_t pg = *o.free.begin();
      o.free.erase(o.free.begin());
      o.held[r][idx] = pg;
      o.n_held[r] += 1;
      o.state[pg] = PG_PENDING;
      o.gen[pg] += 1;
      if (o.needs_wait[pg]) { wait = true; o.needs_wait[pg] = 0; }
      ent.insert(ent.end(), {r, idx, pg, int32_t(o.gen[pg])});
      copy.insert(copy.end(), {r, idx, pg});
      ++n;
      idle = 0;
    } else {
      ++idle;
    }
    r = (r + 1) % N;
  }
  o.cursor = r;
  o.sum_held += n;
  if (n_assigned) *n_assigned = int32_t(n);
  if (n == 0) return KV_OK;
  if (wait) {
    // pages withdrawn from the maps: rewrite them only after the withdrawal and
    // after the attention of every step issued so far (their last readers)
    if (o.unpub_recorded) HIPCHK(h, hipStreamWaitEvent(o.stream, o.ev_unpub, 0));
    for (Group& G : h->grp)
      if (G.done_recorded) HIPCHK(h, hipStreamWaitEvent(o.stream, G.ev_done, 0));
  }
  int rc = stage_list(h, copy, o.d_list_copy, o.stream);
  if (rc) return rc;
  HIPCHK(h, launch_opt_copy(o.d_groups, h->cfg.n_groups, o.d_list_copy, int(n), o.P, h->row16, 128, o.stream));
  Opt::Batch b;
  if (!o.ev_pool.empty()) {
    b.ev = o.ev_pool.back();
    o.ev_pool.pop_back();
  } else {
    HIPCHK(h, hipEventCreateWithFlags(&b.ev, hipEventDisableTiming));
  }
  HIPCHK(h, hipEventRecord(b.ev, o.stream));
  b.ent = std::move(ent);
  o.pending.push_back(std::move(b));
  o.pages_populated += n;
  o.bytes_populated += n * o.P * int64_t(h->row_bytes) * h->cfg.n_groups;
  return KV_OK;
}

int kv_hier_opt_populate(kv_hier_t* h, int32_t max_pages, int32_t* n_assigned) {
  DeviceGuard dg(h);
  if (int rc = refuse_if_broken(h)) return rc;
  return finish(h, opt_populate_impl(h, max_pages, n_assigned));
}

static int opt_publish_entry(kv_hier_t* h, int wait) {
  if (!h) return KV_EINVAL;
  if (!h->opt.on) return fail(h, KV_ESTATE, "dynamic residency is off (opt_page_rows = 0)");
  if (wait != 0 && wait != 1) return fail(h, KV_EINVAL, "wait must be 0 or 1");
  begin_work(h);
  return opt_publish_impl(h, wait == 1);
}

int kv_hier_opt_publish(kv_hier_t* h, int wait) {
  DeviceGuard dg(h);
  if (int rc = refuse_if_broken(h)) return rc;
  return finish(h, opt_publish_entry(h, wait));
}

int kv_hier_opt_query(kv_hier_t* h, int r, int32_t n_pages, int32_t* held, uint8_t* ready,
                      kv_hier_opt_info* info) {
  DeviceGuard dg(h);
  if (!h) return KV_EINVAL;
  const Opt& o = h->opt;
  if (!o.on) return fail(h, KV_ESTATE, "dynamic residency is off (opt_page_rows = 0)");
  if (info) {
    std::memset(info, 0, sizeof *info);
    info->pool_pages = o.M;
    info->page_rows = o.P;
    info->reserve = o.reserve;
    info->cursor = o.cursor;
    for (int x = 0; x < h->cfg.n_req; ++x) {
      info->admitted += o.admitted[x] ? 1 : 0;
      info->ready_pages += o.n_ready[x];
      info->eligible_pages += o.admitted[x] ? o.eligible[x] : 0;
    }
    info->required_pages = o.sum_req;
    info->held_pages = o.sum_held;
    info->pending_pages = o.sum_held - info->ready_pages;
    info->free_pages = int64_t(o.free.size());
    info->pages_populated = o.pages_populated;
    info->pages_published = o.pages_published;
    info->pages_reclaimed = o.pages_reclaimed;
    info->requests_reclaimed = o.requests_reclaimed;
    info->admissions_waited = o.admissions_waited;
    info->bytes_populated = o.bytes_populated;
  }
  if (r >= 0) {
    int rc = check_req(h, r);
    if (rc) return rc;
    if (n_pages < 0) return fail(h, KV_EINVAL, "negative page count");
    for (int i = 0; i < n_pages; ++i) {
      const int32_t pg = (i < int(o.held[r].size())) ? o.held[r][i] : -1;
      if (held) held[i] = pg;
      if (ready) ready[i] = (pg >= 0 && o.state[pg] == PG_READY) ? 1 : 0;
    }
  }
  return KV_OK;
}

}  // extern "C"
