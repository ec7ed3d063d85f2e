// Exact sparse attention of every verification query over its own ordered
// list of selected rows plus its ring window, for gfx950.
//
// "Adaptive DHiSparse" (arXiv 2610.13708): eq. (1) u = Attn(h, {c_s}) over
// the query's selection; §3.3 (Figure 3 caption): each query attends over its
// own selection and keeps its own causal boundary; eq. (5) visible positions;
// §3.5 eqs. (11)-(12): rows are read through their resolved locations,
// KV[l] = c_{r,s}, so the result does not depend on which tier holds a row.
// The ring branch covers positions max(ring_lo, p_j-W+1) .. p_j.
//
// Layout and schedule (one workgroup = one query x up to 64 heads x one key split):
//  - rows are shared by all heads (MQA / absorbed MLA), so heads form the MFMA
//    N dimension and 32-row tiles form M: S^T = K Q^T with
//    v_mfma_f32_32x32x16_bf16, then O^T = V^T P^T with the probabilities as
//    the B operand.
//  - four waves per 32-head block split the key width for S^T (partial scores
//    meet in LDS) and the value width for O^T; each of the four then owns a
//    quarter of the tile's rows for the softmax (reduce-scatter), so every
//    score is exponentiated once; probabilities go to LDS as bf16 P^T.
//  - a tile lives in LDS once; K fragments are plain 16-byte reads and V^T
//    fragments come from the same rows through ds_read_b64_tr_b16, with the
//    value dims of an MFMA block interleaved (8 dims from each 32-dim group)
//    so that both read patterns hit every bank once per half-wave.
//  - rows of 72 16-byte chunks (absorbed MLA) go straight from memory to LDS
//    (global_load_lds, three tile buffers, tile t+2 issued while tile t
//    computes): chunks 0..63 of a row land in its head-region slot (1040-byte
//    stride, 4 banks apart), chunks 64..71 in a swizzled tail region; the
//    location codes travel the same way, two tiles ahead.  Other row widths
//    are gathered one tile ahead into registers and stored to a double
//    buffer with a 36-bank stride.  Either way each wave decodes the codes
//    of its own rows into wave-uniform addresses (readlane / lane permute),
//    and masked positions read a zero row, so no load depends on a per-lane
//    branch.
//  - two barriers per tile: after the partial scores (then the next tiles'
//    loads are issued and the softmax runs) and after the probabilities
//    (which also publishes the next tile); the next tile's K fragments are
//    read right after the second, one tile ahead of their products, and the
//    tile's V^T fragments right after the first.
//  - online softmax in fp32 with exp2 (scale folded with log2 e): the running
//    max of a head is raised only when a score exceeds it by more than 2^8,
//    detected per tile with one ballot; the rare raise takes a second pass
//    over the tile (tile max exchanged in LDS, O and l rescaled).
//  - the sum order depends only on the list order and the split boundaries,
//    never on where a row is cached, so outputs are bitwise identical across
//    cache states.
//  - block index -> (request, query, head group, split) keeps every workgroup
//    of one request on one XCD (dispatch is round-robin over the 8 XCDs), so
//    rows shared by a request's queries are re-read from that XCD's L2.
#include "common.h"

#include <hip/hip_ext.h>

#include <type_traits>

namespace kvh {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
// Global-address-space views: gathered rows and location codes are read with
// global (not flat) loads, so waiting on LDS never waits on the prefetch.
#define GLOBAL_AS __attribute__((address_space(1)))
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef const GLOBAL_AS u32x4 gu32x4;
typedef const GLOBAL_AS int32_t gint32;

__device__ __forceinline__ uint4 gload16(uintptr_t addr) {
  const u32x4 v = *reinterpret_cast<gu32x4*>(addr);
  return make_uint4(v.x, v.y, v.z, v.w);
}

constexpr int TILE = 32;
constexpr float kNegBig = -1.0e30f;
// A score may exceed its head's running max by up to this much (log2 units)
// before the max is raised: numerator and normaliser always share the same
// max, so the result is unchanged, and p stays below 2^8.
constexpr float kRescaleLog2 = 8.0f;

template <int D_QK_, int V_OFF_, int D_V_, int ROW_, int HB_>
struct Cfg {
  static constexpr int D_QK = D_QK_, V_OFF = V_OFF_, D_V = D_V_, ROW = ROW_, HB = HB_;
  static constexpr int NDP = 4;              // waves per 32-head block: key / value width split
  static constexpr int NW = NDP * HB;
  static constexpr int NT = NW * 64;
  static constexpr int KST = D_QK / 16;      // 16-wide k-steps over the key width
  // k-steps of one wave's key part (wave dq takes k-steps dq*KS .. dq*KS+KS-1
  // that exist: with a key width that is no multiple of 64 the last waves
  // take fewer, or none)
  static constexpr int KS = (KST + NDP - 1) / NDP;
  static constexpr bool KS_EVEN = KST % NDP == 0;
  static constexpr int DVB = D_V / NDP / 32; // 32-dim value blocks of this wave's value part
  static constexpr int RCH = ROW / 8;        // 16-byte chunks per row
  static constexpr int RPW = TILE / NW;      // rows of a tile gathered by one wave
  // gather instructions per wave and tile: with rows of >= 64 chunks, one
  // instruction per row for chunks 0..63 plus shared ones for the rest
  static constexpr bool WIDE = RCH >= 64;
  static constexpr int REST = WIDE ? RCH - 64 : 0;
  static constexpr int NU = WIDE ? RPW + (RPW * REST + 63) / 64 : (RPW * RCH + 63) / 64;
  static constexpr bool GATHER_EXACT = WIDE || (RPW * RCH) % 64 == 0;   // no idle lanes
  // row stride: 36 banks (dwords mod 64) apart
  static constexpr int ROW_DW = ROW / 2;
  static constexpr int KSTR = ROW + 2 * ((36 - ROW_DW % 64 + 64) % 64);
  static constexpr int KBUF = TILE * KSTR;   // elements per tile buffer
  static constexpr int PSTR = TILE + 8;      // P^T row stride (elements): 20 banks
  // LDS DMA layout (rows of 72 chunks): chunks 0..63 of tile row r at
  // r*HSTR (260 dwords: 16 consecutive rows hit distinct banks), chunks 64..71
  // at TAILO + r*64 in slot order c ^ tail_swz(r); three buffers, and per
  // wave three 64-entry slots of location codes.
  static constexpr bool DMA = WIDE && REST == 8;
  static constexpr int HSTR = 520;
  static constexpr int TAILO = TILE * HSTR;
  static constexpr int NBUF = DMA ? 3 : 2;
  static constexpr int BSTR = DMA ? TAILO + TILE * 64 : KBUF;   // elements per tile buffer
  static constexpr int RSTR = DMA ? HSTR : KSTR;                 // row stride of the K / V reads
  static constexpr int NVM = RPW + 2;      // DMA instructions per wave and tile (rows, tail, codes)
  static constexpr size_t LDS_K = size_t(NBUF) * BSTR * 2;
  static constexpr size_t LDS_S = size_t(NW) * 4 * 64 * 16;
  static constexpr size_t LDS_P = size_t(HB) * 32 * PSTR * 2;
  static constexpr size_t LDS_M = size_t(NW) * 32 * 4;
  static constexpr size_t LDS_C = DMA ? size_t(3) * NW * 64 * 4 : 0;
  static constexpr size_t LDS = LDS_K + LDS_S + LDS_P + LDS_M + LDS_C + 16;
  static_assert(D_QK % 16 == 0 && D_V % (NDP * 32) == 0 && ROW % 8 == 0, "shape");
  static_assert(V_OFF % 8 == 0 && V_OFF + D_V <= ROW && D_QK <= ROW, "row layout");
  static_assert(WIDE ? (REST <= 64 && 64 % REST == 0) : RCH <= 64, "gather");
  static_assert(LDS <= 160 * 1024, "LDS");
  static_assert(!DMA || (RPW * 8 <= 64 && NVM <= 15), "DMA tile");
};

struct RowCtx {
  gint32* loc;
  int k, n_total, Rd;
  int ring_row0;    // ring row of the window's first position: r*R_d + (lo mod R_d)
  int ring_end;     // (r+1)*R_d: ring rows wrap from here back to r*R_d
  uintptr_t hot, d_staging, d_resident, d_ring, zero;   // d_*: pool base minus hot base
};

// Raw code of list position idx, loaded one tile before it is decoded (the
// load is clamped into this query's list; positions past it are rewritten by
// final_code).
__device__ __forceinline__ int raw_code(const RowCtx& c, int idx) { return c.loc[min(idx, c.k - 1)]; }

// Positions past the list are the ring window (tier 3, index r*R_d + pos mod
// R_d) and, past its end, masked (-1).
__device__ __forceinline__ int final_code(const RowCtx& c, int idx, int raw) {
  int rrow = c.ring_row0 + (idx - c.k);             // consecutive positions, one wrap at most
  rrow -= rrow >= c.ring_end ? c.Rd : 0;
  const int rc = make_loc(kTierRing, rrow);
  return idx < c.k ? raw : (idx < c.n_total ? rc : -1);
}

// Address of the row a code names; masked codes read the zero row.
template <int ROW>
__device__ __forceinline__ uintptr_t row_addr(const RowCtx& c, int code) {
  const int tier = loc_tier(code);
  // pool offsets from the hot pool base, selected arithmetically (a select
  // chain becomes an indexed table in scratch memory)
  const uintptr_t off = (tier == kTierStaged ? c.d_staging : uintptr_t(0)) +
                        (tier == kTierResident ? c.d_resident : uintptr_t(0)) +
                        (tier == kTierRing ? c.d_ring : uintptr_t(0));
  return code < 0 ? c.zero : c.hot + off + size_t(loc_index(code)) * (size_t(ROW) * 2);
}

// (row within the wave's rows, chunk) of gather instruction u for a lane, and
// whether the lane's chunk is stored (the shared tail instruction may carry
// duplicates).
template <class C>
__device__ __forceinline__ void task_of(int u, int lane, int& rr, int& ch, bool& st) {
  if (C::WIDE) {
    if (u < C::RPW) { rr = u; ch = lane; st = true; return; }
    const int per = 64 / C::REST;                  // rows per tail instruction
    const int x = (u - C::RPW) * per + lane / C::REST;
    st = x < C::RPW;
    rr = st ? x : 0;
    ch = 64 + lane % C::REST;
  } else {
    // rows whose chunk count does not divide the wave: the last
    // instruction's idle lanes load a chunk of the wave's first row and store
    // nothing
    const int x = u * 64 + lane;
    st = C::GATHER_EXACT || x < C::RPW * C::RCH;
    rr = st ? x / C::RCH : 0;
    ch = st ? x % C::RCH : 0;
  }
}

template <class C>
struct Gather {
  uint4 v[C::NU];
};

// Issues the loads of one tile: lanes 0..31 (and their mirrors 32..63) hold
// the codes of the tile's 32 rows; each lane decodes its row's address, and a
// wave's instruction takes its row base from the owning lane (readlane for
// a whole-row instruction, a lane permute otherwise).  Loads are
// unconditional and their values are consumed one tile later, so the wave
// never waits for them here.  Returns the tile's live-row mask.
template <class C>
__device__ __forceinline__ uint32_t gather_issue(Gather<C>& g, const RowCtx& ctx, int code, int w, int lane) {
  const uint32_t live = static_cast<uint32_t>(__builtin_amdgcn_ballot_w64(code >= 0));
  const uintptr_t my = row_addr<C::ROW>(ctx, code);
  const int mlo = static_cast<int>(static_cast<uint32_t>(my));
  const int mhi = static_cast<int>(static_cast<uint32_t>(my >> 32));
#pragma unroll
  for (int u = 0; u < C::NU; ++u) {
    int rr, ch;
    bool st;
    task_of<C>(u, lane, rr, ch, st);
    uintptr_t base;
    if (C::WIDE && u < C::RPW) {
      const int src = w * C::RPW + u;
      base = (uintptr_t(uint32_t(__builtin_amdgcn_readlane(mhi, src))) << 32) |
             uint32_t(__builtin_amdgcn_readlane(mlo, src));
    } else {
      const int src = w * C::RPW + rr;
      base = (uintptr_t(uint32_t(__shfl(mhi, src, 64))) << 32) | uint32_t(__shfl(mlo, src, 64));
    }
    g.v[u] = gload16(base + size_t(ch) * 16);
  }
  return live;
}

template <class C>
__device__ __forceinline__ void gather_store(const Gather<C>& g, uint16_t* kb, int w, int lane) {
#pragma unroll
  for (int u = 0; u < C::NU; ++u) {
    int rr, ch;
    bool st;
    task_of<C>(u, lane, rr, ch, st);
    if (st) *reinterpret_cast<uint4*>(kb + (w * C::RPW + rr) * C::KSTR + ch * 8) = g.v[u];
  }
}

// LDS DMA: each lane's 16 (or 4) bytes land at the wave-uniform LDS address
// plus lane*16 (lane*4).  Issued as inline assembly so that the compiler
// neither counts these loads nor inserts waits for them: each wait is explicit
// (vmcnt before the barrier that publishes a tile).  Waiting with vmcnt(N)
// completes every vector-memory instruction older than the N most recent, so
// other loads interleaved by the compiler can only lengthen a wait.  The LDS
// offset is the low word of the generic address of dynamic shared memory.
__device__ __forceinline__ void dma16(uintptr_t gaddr, const void* lds_dst) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds_dst)));
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(gaddr), "{m0}"(m0) : "memory");
}
__device__ __forceinline__ void dma4(uintptr_t gaddr, const void* lds_dst) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds_dst)));
  asm volatile("global_load_lds_dword %0, off" ::"v"(gaddr), "{m0}"(m0) : "memory");
}

// Workgroup barrier after this wave's LDS writes completed; vector-memory
// loads (tile DMA) stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);                  // lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}
// The same after all but the N most recent vector-memory instructions
// completed (s_waitcnt encoding: vmcnt bits 3:0 and 15:14, lgkmcnt 0).
template <int N>
__device__ __forceinline__ void lds_vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70);
  asm volatile("s_barrier" ::: "memory");
}

// Tail-region slot swizzle of tile row r: chunk 64+c sits in slot c ^ tail_swz(r)
// (16 consecutive rows reading one chunk hit distinct banks).
__device__ __forceinline__ int tail_swz(int r) { return (r >> 1) & 7; }

// DMA of the raw codes of tile t into this wave's 64-entry slot (lanes l and
// l+32 load the code of row l; positions past the list are clamped into it
// and rewritten by final_code).  One instruction.
template <class C>
__device__ __forceinline__ void dma_codes(int32_t* slot, const RowCtx& c, int t, int w, int lane) {
  const int idx = min(t * TILE + (lane & 31), c.k - 1);
  dma4(reinterpret_cast<uintptr_t>(c.loc + idx), slot + w * 64);
}

// DMA of one tile: lanes l and l+32 hold the code of tile row l; wave w moves
// rows w*RPW .. w*RPW+RPW-1, one instruction per row for chunks 0..63 and one
// for the rows' chunks 64..71 (RPW*8 lanes).  RPW+1 instructions.  Returns
// the tile's live-row mask.
template <class C>
__device__ __forceinline__ uint32_t dma_tile(uint16_t* dst, const RowCtx& ctx, int code, int w, int lane) {
  const uint32_t live = static_cast<uint32_t>(__builtin_amdgcn_ballot_w64(code >= 0));
  const uintptr_t my = row_addr<C::ROW>(ctx, code);
  const int mlo = static_cast<int>(static_cast<uint32_t>(my));
  const int mhi = static_cast<int>(static_cast<uint32_t>(my >> 32));
  {
    const int row = w * C::RPW + ((lane >> 3) & (C::RPW - 1));
    const uintptr_t base = (uintptr_t(uint32_t(__shfl(mhi, row, 64))) << 32) | uint32_t(__shfl(mlo, row, 64));
    const int cp = (lane & 7) ^ tail_swz(row);
    if (C::RPW * 8 == 64 || lane < C::RPW * 8)
      dma16(base + size_t(64 + cp) * 16, dst + C::TAILO + w * C::RPW * 64);
  }
#pragma unroll
  for (int u = 0; u < C::RPW; ++u) {
    const int row = w * C::RPW + u;
    const uintptr_t base = (uintptr_t(uint32_t(__builtin_amdgcn_readlane(mhi, row))) << 32) |
                           uint32_t(__builtin_amdgcn_readlane(mlo, row));
    dma16(base + size_t(lane) * 16, dst + row * C::HSTR);
  }
  return live;
}

template <class C>
__global__ __launch_bounds__(C::NT, 1) void attn_kernel(AttnArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  uint16_t* Kb = reinterpret_cast<uint16_t*>(lds);
  float4* Sx = reinterpret_cast<float4*>(lds + C::LDS_K);
  uint16_t* Pb = reinterpret_cast<uint16_t*>(lds + C::LDS_K + C::LDS_S);
  float* Mx = reinterpret_cast<float*>(lds + C::LDS_K + C::LDS_S + C::LDS_P);
  int32_t* Cs = reinterpret_cast<int32_t*>(lds + C::LDS_K + C::LDS_S + C::LDS_P + C::LDS_M);   // DMA only
  uint8_t* flags = reinterpret_cast<uint8_t*>(lds + C::LDS_K + C::LDS_S + C::LDS_P + C::LDS_M + C::LDS_C);

  const int nreq = a.r1 - a.r0;
  const int per_req = a.Q * a.head_groups * a.splits;
  const int b = blockIdx.x;
  const int rr = ((b >> 3) / per_req) * 8 + (b & 7);
  if (rr >= nreq) return;
  const int sub = (b >> 3) % per_req;
  const int j = sub / (a.head_groups * a.splits);
  const int hg = (sub / a.splits) % a.head_groups;
  const int sp = sub % a.splits;
  const int r = a.r0 + rr;
  const int qi = r * a.Q + j;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);      // wave-uniform: held in SGPRs
  const int hb = w / C::NDP, dq = w % C::NDP;
  const int hl = hb * 32 + (lane & 31);               // head within the workgroup
  const int head = hg * 32 * C::HB + hl;
  const size_t blk = (size_t(qi - a.r0 * a.Q) * a.head_groups + hg) * a.splits + sp;   // from the chunk's start
  const int hi_half = lane >> 5;
  const int vq0 = dq * (C::D_V / C::NDP);             // first value dim of this wave

  const int p_j = a.causal[qi];
  if (p_j < 0) {  // inactive query: zero output (the combine pass does it when split)
    if (a.splits == 1 && head < a.H) {
      uint16_t* op = a.out + (size_t(qi) * a.H + head) * C::D_V + vq0;
      for (int d = hi_half; d < C::D_V / C::NDP / 4; d += 2)
        *reinterpret_cast<uint2*>(op + d * 4) = make_uint2(0, 0);
    }
    return;
  }
  const int n_r = a.causal[size_t(r) * a.Q];
  int lo = a.ring_lo[r];
  lo = max(lo, p_j - a.W + 1);
  lo = max(lo, 0);
  if (a.block_only) lo = max(lo, n_r);
  const int n_ring = p_j >= lo ? p_j - lo + 1 : 0;

  RowCtx ctx;
  ctx.loc = reinterpret_cast<gint32*>(reinterpret_cast<uintptr_t>(a.loc + size_t(qi) * a.k));
  ctx.k = a.k;
  ctx.n_total = a.k + n_ring;
  ctx.Rd = a.Rd;
  ctx.ring_row0 = r * a.Rd + lo % a.Rd;
  ctx.ring_end = (r + 1) * a.Rd;
  ctx.hot = reinterpret_cast<uintptr_t>(a.hot);
  ctx.d_staging = reinterpret_cast<uintptr_t>(a.staging) - ctx.hot;
  ctx.d_resident = reinterpret_cast<uintptr_t>(a.resident) - ctx.hot;
  ctx.d_ring = reinterpret_cast<uintptr_t>(a.ring) - ctx.hot;
  ctx.zero = reinterpret_cast<uintptr_t>(a.zero);

  const int n_tiles = (ctx.n_total + TILE - 1) / TILE;
  const int tb = int((long long)n_tiles * sp / a.splits);
  const int te = int((long long)n_tiles * (sp + 1) / a.splits);

  // Q fragment: B operand of S^T = K Q^T, head = lane%32, 8 dims per k-step
  bf16x8 qreg[C::KS];
  {
    const uint16_t* qp = a.q + (size_t(qi) * a.H + head) * C::D_QK + dq * (C::KS * 16) + hi_half * 8;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (head < a.H && (C::KS_EVEN || dq * C::KS + ks < C::KST)) v = gload16(reinterpret_cast<uintptr_t>(qp + ks * 16));
      qreg[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  f32x16 O[C::DVB];
#pragma unroll
  for (int d = 0; d < C::DVB; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) O[d][i] = 0.f;
  float m_run = kNegBig, l_run = 0.f;
  const float sl2 = a.scale_log2;
  const int crow = lane & 31;                          // tile row whose code this lane holds

  // tile t lives in buffer (t - tb) mod NBUF; with DMA its codes in slot (t - tb) mod 3
  auto kbuf = [&](int t) { return Kb + ((t - tb) % C::NBUF) * C::BSTR; };
  auto cslot = [&](int t) { return Cs + ((t - tb) % 3) * (C::NW * 64); };
  Gather<C> g;
  uint32_t live_cur, live_n1;
  int raw = 0;
  if constexpr (C::DMA) {
    // prologue: codes of tb and tb+1; DMA of tiles tb, tb+1 and of the codes
    // of tb+2, tb+3; tile tb landed in every wave before the first scores
    __builtin_amdgcn_s_waitcnt(0x0F70);              // vmcnt(0): Q fragments in registers
    dma_codes<C>(cslot(tb), ctx, tb, w, lane);
    dma_codes<C>(cslot(tb + 1), ctx, tb + 1, w, lane);
    __builtin_amdgcn_s_waitcnt(0x0F70);              // vmcnt(0)
    live_cur = dma_tile<C>(kbuf(tb), ctx, final_code(ctx, tb * TILE + crow, cslot(tb)[w * 64 + lane]), w, lane);
    dma_codes<C>(cslot(tb + 2), ctx, tb + 2, w, lane);
    const int code1 = tb + 1 < te ? final_code(ctx, (tb + 1) * TILE + crow, cslot(tb + 1)[w * 64 + lane]) : -1;
    live_n1 = dma_tile<C>(kbuf(tb + 1), ctx, code1, w, lane);
    dma_codes<C>(cslot(tb + 3), ctx, tb + 3, w, lane);
    lds_vm_barrier<C::NVM>();
  } else {
    // prologue: tile tb into LDS buffer 0, tile tb+1 in flight, codes of tb+2 in flight
    int code = final_code(ctx, tb * TILE + crow, raw_code(ctx, tb * TILE + crow));
    live_cur = gather_issue<C>(g, ctx, code, w, lane);
    raw = raw_code(ctx, (tb + 1) * TILE + crow);
    gather_store<C>(g, Kb, w, lane);
    live_n1 = gather_issue<C>(g, ctx, final_code(ctx, (tb + 1) * TILE + crow, raw), w, lane);
    raw = raw_code(ctx, (tb + 2) * TILE + crow);
    __syncthreads();
  }

  // per-lane LDS offsets (elements) inside a tile buffer: K fragment of k-step
  // ks = row crow, chunk of dims dq*D_QK/4 + 16ks + 8hi
  int koff[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    const int c = (dq * (C::KS * 16) + ks * 16 + hi_half * 8) / 8;
    koff[ks] = !C::DMA || c < 64 ? crow * C::RSTR + c * 8
                                 : C::TAILO + crow * 64 + (((c - 64) ^ tail_swz(crow)) * 8);
  }
  int v_off;
  {
    const int gq = (lane >> 4) & 3, s = lane & 15, aq = s & 3;
    const int row = (gq >> 1) * 8 + (s >> 2);
    const int dim = C::V_OFF + vq0 + ((gq & 1) * 2 + (aq >> 1)) * (8 * C::DVB) + (aq & 1) * 4;
    v_off = row * C::RSTR + dim;
  }
  float4* sx_own = Sx + size_t(w) * 4 * 64 + lane;
  const float4* sx_red = Sx + size_t(hb * C::NDP) * 4 * 64 + dq * 64 + lane;   // + q * 256
  uint16_t* p_own = Pb + (size_t(hb) * 32 + (lane & 31)) * C::PSTR + dq * 8 + hi_half * 4;
  const uint16_t* p_rd = Pb + (size_t(hb) * 32 + (lane & 31)) * C::PSTR + hi_half * 8;
  const int sbit0 = dq * 8 + hi_half * 4;              // first tile row of this lane's quarter

  // K fragments of tile tb (every later tile's are read right after the
  // barrier that publishes it, one tile ahead of their products)
  bf16x8 kfr[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks)
    kfr[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(kbuf(tb) + koff[ks]));

  // One tile; B = (t - tb) mod NBUF is a compile-time constant (the loop below
  // is unrolled NBUF times), so buffer and slot offsets fold into the LDS
  // instructions.
  auto tile = [&](int t, auto bconst) {
    constexpr int B = decltype(bconst)::value;
    const uint16_t* kb = Kb + B * C::BSTR;
    // codes of tile t+2 (landed before the last barrier; DMA path)
    if constexpr (C::DMA) raw = (Cs + ((B + 2) % 3) * (C::NW * 64))[w * 64 + lane];

    // partial scores over this wave's part of the key width
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
      if (C::KS_EVEN || dq * C::KS + ks < C::KST)     // wave-uniform: k-steps past the key width are skipped
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfr[ks], qreg[ks], acc, 0, 0, 0);
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4)
      sx_own[i4 * 64] = make_float4(acc[4 * i4], acc[4 * i4 + 1], acc[4 * i4 + 2], acc[4 * i4 + 3]);
    if constexpr (C::DMA)
      lds_barrier();
    else
      __syncthreads();

    // LDS reads first (this wave's partial scores, the tile's V^T fragments),
    // then the next tiles' loads while they land
    float4 sxv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) sxv[q] = sx_red[q * 256];
    bf16x8 vfr[2][C::DVB];
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
      for (int d = 0; d < C::DVB; ++d) {
        const uint16_t* vp = kb + v_off + ks2 * 16 * C::RSTR + d * 8;
        const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp));
        const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp + 4 * C::RSTR));
        vfr[ks2][d] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    uint32_t live_n2;
    if constexpr (C::DMA) {
      // DMA of tile t+2 into the buffer of tile t-1 (its last readers, the PV
      // products of t-1, finished before the barrier) and of the codes of
      // tile t+4 into the slot of t+1; issued unconditionally so that every
      // wave keeps NVM instructions per tile (tiles past the range read the
      // zero row and are never used)
      const int code = t + 2 < te ? final_code(ctx, (t + 2) * TILE + crow, raw) : -1;
      live_n2 = dma_tile<C>(Kb + ((B + 2) % 3) * C::BSTR, ctx, code, w, lane);
      dma_codes<C>(Cs + ((B + 1) % 3) * (C::NW * 64), ctx, t + 4, w, lane);
    } else {
      // tile t+1 into the other buffer (its last reader, PV of tile t-1, is done);
      // issue tile t+2 and the codes of tile t+3 (unconditional: positions past
      // the range read the zero row and are never used)
      gather_store<C>(g, Kb + ((B + 1) % C::NBUF) * C::BSTR, w, lane);
      live_n2 = gather_issue<C>(g, ctx, final_code(ctx, (t + 2) * TILE + crow, raw), w, lane);
      raw = raw_code(ctx, (t + 3) * TILE + crow);
    }

    // this wave's quarter of the rows: scores summed over the key parts in order
    float s[4];
    s[0] = ((sxv[0].x + sxv[1].x) + sxv[2].x) + sxv[3].x;
    s[1] = ((sxv[0].y + sxv[1].y) + sxv[2].y) + sxv[3].y;
    s[2] = ((sxv[0].z + sxv[1].z) + sxv[2].z) + sxv[3].z;
    s[3] = ((sxv[0].w + sxv[1].w) + sxv[2].w) + sxv[3].w;
    const uint32_t lb = live_cur >> sbit0;
    bool over = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[i] = (lb >> i) & 1u ? s[i] * sl2 : -INFINITY;
      over |= s[i] > m_run + kRescaleLog2;
    }
    float p[4];
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = __builtin_amdgcn_exp2f(s[i] - m_run);
      ps += p[i];
    }
    {
      uint2 pk;
      pk.x = uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(p[0]))) |
             (uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(p[1]))) << 16);
      pk.y = uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(p[2]))) |
             (uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(p[3]))) << 16);
      *reinterpret_cast<uint2*>(p_own) = pk;
    }
    const bool any_over = __builtin_amdgcn_ballot_w64(over) != 0;
    if (lane == 0) flags[w] = any_over ? 1 : 0;
    if constexpr (C::DMA)
      lds_vm_barrier<C::NVM>();                        // and tile t+1 landed in every wave
    else
      __syncthreads();

    // K fragments of tile t+1 (published by this barrier) for its scores
    // after this tile's PV products
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
      kfr[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(Kb + ((B + 1) % C::NBUF) * C::BSTR + koff[ks]));
    bf16x8 pbf[2];
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2)
      pbf[ks2] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p_rd + ks2 * 16));
    const bool slow = C::NW == 8 ? *reinterpret_cast<const uint64_t*>(flags) != 0
                                 : *reinterpret_cast<const uint32_t*>(flags) != 0;
    if (slow) {
      // some score of some head exceeds its running max by more than 2^8:
      // exchange the tile max, raise the max where needed, redo this tile's p
      float mq = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
      mq = fmaxf(mq, __shfl_xor(mq, 32, 64));
      if (lane < 32) Mx[w * 32 + lane] = mq;
      __syncthreads();
      float mt = Mx[(hb * C::NDP) * 32 + (lane & 31)];
#pragma unroll
      for (int q = 1; q < C::NDP; ++q) mt = fmaxf(mt, Mx[(hb * C::NDP + q) * 32 + (lane & 31)]);
      if (mt > m_run + kRescaleLog2) {
        const float alpha = __builtin_amdgcn_exp2f(m_run - mt);
        l_run *= alpha;
        m_run = mt;
#pragma unroll
        for (int d = 0; d < C::DVB; ++d)
#pragma unroll
          for (int i = 0; i < 16; ++i) O[d][i] *= alpha;
      }
      ps = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = __builtin_amdgcn_exp2f(s[i] - m_run);
        ps += p[i];
      }
      uint2 pk;
      pk.x = uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(p[0]))) |
             (uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(p[1]))) << 16);
      pk.y = uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(p[2]))) |
             (uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(p[3]))) << 16);
      *reinterpret_cast<uint2*>(p_own) = pk;
      __syncthreads();
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2)
        pbf[ks2] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p_rd + ks2 * 16));
    }
    l_run += ps;

    // O^T += V^T P^T over the tile's 32 rows (two 16-row k-steps)
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
      for (int d = 0; d < C::DVB; ++d) O[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfr[ks2][d], pbf[ks2], O[d], 0, 0, 0);
    live_cur = live_n1;
    live_n1 = live_n2;
  };
  for (int t = tb; t < te; t += C::NBUF) {
    tile(t, std::integral_constant<int, 0>{});
    if (t + 1 < te) tile(t + 1, std::integral_constant<int, 1>{});
    if constexpr (C::NBUF == 3)
      if (t + 2 < te) tile(t + 2, std::integral_constant<int, 2>{});
  }
  if constexpr (C::DMA) __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0): no DMA outlives the loop

  // normaliser: this wave's rows, both lane halves, then the four quarters in order
  float l2 = l_run + __shfl_xor(l_run, 32, 64);
  __syncthreads();
  if (lane < 32) Mx[w * 32 + lane] = l2;
  __syncthreads();
  float l_tot = Mx[(hb * C::NDP) * 32 + (lane & 31)];
#pragma unroll
  for (int q = 1; q < C::NDP; ++q) l_tot += Mx[(hb * C::NDP + q) * 32 + (lane & 31)];

  // O^T register i of block d holds value dim vq0 + (i/4)*8*DVB + d*8 + hi*4 + i%4
  if (a.splits == 1) {
    if (head < a.H) {
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      uint16_t* op = a.out + (size_t(qi) * a.H + head) * C::D_V + vq0 + hi_half * 4;
#pragma unroll
      for (int d = 0; d < C::DVB; ++d)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          uint16_t h4[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            h4[e] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(O[d][g4 * 4 + e] * inv));
          uint2 pk;
          pk.x = uint32_t(h4[0]) | (uint32_t(h4[1]) << 16);
          pk.y = uint32_t(h4[2]) | (uint32_t(h4[3]) << 16);
          *reinterpret_cast<uint2*>(op + g4 * 8 * C::DVB + d * 8) = pk;
        }
    }
  } else {
    float* po = a.part_o + (blk * 32 * C::HB + hl) * C::D_V + vq0 + hi_half * 4;
#pragma unroll
    for (int d = 0; d < C::DVB; ++d)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *reinterpret_cast<float4*>(po + g4 * 8 * C::DVB + d * 8) =
            make_float4(O[d][g4 * 4 + 0], O[d][g4 * 4 + 1], O[d][g4 * 4 + 2], O[d][g4 * 4 + 3]);
    if (dq == 0 && hi_half == 0) {
      float* pm = a.part_ml + (blk * 32 * C::HB + hl) * 2;
      pm[0] = m_run;
      pm[1] = l_tot;
    }
  }
}

// ---------------------------------------------------------------------------
// Rows of 72 16-byte chunks (absorbed MLA: K = all 576 elements, V = the
// first 512) at 64 heads per workgroup: a wave-specialised pipeline with one
// barrier per 32-row tile.
//  - four score waves own 16 heads each over the whole key width (their Q
//    fragments stay in registers): S^T = K Q^T with v_mfma_f32_16x16x32_bf16,
//    tile rows in M and heads in N, so the 32 scores of a head are complete
//    in four lanes of one wave and no partial scores cross waves.  The
//    online softmax runs there (per head; the max is raised lazily as
//    above), and the probabilities go to LDS as bf16 P^T together with each
//    head's rescale factor and a per-wave flag.
//  - four product waves own a quarter of the value width for all 64 heads:
//    O^T += V^T P^T with v_mfma_f32_32x32x16_bf16, V^T through
//    ds_read_b64_tr_b16 in the layout above.
//  - score waves work on tile t+1 while product waves fold tile t into O; a
//    wave of each kind sits on every SIMD, so the products of one overlap the
//    fragment reads and softmax of the other.
//  - tiles reach LDS by DMA in the head-region / swizzled-tail layout above,
//    four buffers: tile t+3 is issued while tiles t+1 (scores) and t
//    (products) are read, giving each tile two tile-times to land.  The first
//    product wave DMAs the location codes into a shared ring of slots, four
//    tiles ahead.
template <int D_QK_, int V_OFF_, int D_V_, int ROW_>
struct WCfg {
  static constexpr int D_QK = D_QK_, V_OFF = V_OFF_, D_V = D_V_, ROW = ROW_;
  static constexpr int NS = 4;                 // score waves (16 heads each)
  static constexpr int NP = 4;                 // product waves (a quarter of the value width each)
  static constexpr int NW = NS + NP;
  static constexpr int NT = NW * 64;
  static constexpr int KST = D_QK / 32;        // 32-dim k-steps of the score products
  static constexpr int DVB = D_V / NP / 32;    // 32-dim value blocks of one product wave
  static constexpr int RCH = ROW / 8;          // 16-byte chunks per row
  static constexpr int DPW = TILE / NP;        // tile rows DMA'd by one product wave
  static constexpr int HSTR = 520;             // head-region row stride (elements)
  static constexpr int TAILO = TILE * HSTR;    // tail region (chunks 64..71)
  static constexpr int BSTR = TAILO + TILE * 64;
  static constexpr int RSTR = HSTR;
  static constexpr int NBUF = 4;
  static constexpr int PSTR = TILE + 8;        // P^T row stride (elements): 20 banks
  static constexpr int NVM = DPW + 1;          // DMA instructions per product wave and tile
  static constexpr size_t LDS_K = size_t(NBUF) * BSTR * 2;
  static constexpr size_t LDS_P = size_t(2) * 64 * PSTR * 2;   // two P^T slots
  static constexpr size_t LDS_A = size_t(2) * 64 * 4;          // rescale factors per slot; (m, l) at the end
  static constexpr size_t LDS_F = 16;                          // rescale flags: a byte per score wave and slot
  static constexpr size_t LDS_C = size_t(4) * 64 * 4;          // code slots (lanes l, l+32: row l)
  static constexpr size_t LDS = LDS_K + LDS_P + LDS_A + LDS_F + LDS_C;
  static_assert(D_QK % 32 == 0 && D_V % (NP * 32) == 0 && RCH == 72 && DPW == 8, "shape");
  static_assert(V_OFF % 8 == 0 && V_OFF + D_V <= ROW && D_QK <= ROW, "row layout");
  static_assert(LDS <= 160 * 1024, "LDS");
};

// Score k-step ks of lane quarter g: first chunk of the k-step's head-region
// block, the quarter's chunk, and the row permutation of the A fragment.
__host__ __device__ constexpr int ws_base(int ks) { return 16 * (ks / 4) + 2 * (ks % 4); }
__device__ __forceinline__ int ws_chunk(int ks, int g) {
  return ks < 16 ? ws_base(ks) + ((g & 1) << 3) + (g >> 1) : 64 + 4 * (ks - 16) + g;
}
__device__ __forceinline__ int ws_row(int m) { return m ^ (((m >> 3) & 1) << 2); }

// max / sum over lanes l and l^16 (l^32) without LDS: the gfx950 lane swaps
// return (lower lane's value, upper lane's value) in every lane of the pair
__device__ __forceinline__ float max_x16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_x32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_x16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_x32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Tile DMA by a product wave wp: rows wp*DPW .. +DPW-1 of the tile, one
// instruction per row for chunks 0..63 and one for their chunks 64..71 (lane:
// row lane/8, slot lane%8).  Row bases are taken by readlane from the lanes
// holding the rows' codes; the tail instruction's base is selected from them.
template <class C>
struct WsDma {
  uintptr_t base[C::DPW];
  uintptr_t tail;
};
template <class C>
__device__ __forceinline__ void ws_dma_prepare(WsDma<C>& d, const RowCtx& ctx, int code, int wp, int lane) {
  const uintptr_t my = row_addr<C::ROW>(ctx, code);
  const int mlo = static_cast<int>(static_cast<uint32_t>(my));
  const int mhi = static_cast<int>(static_cast<uint32_t>(my >> 32));
#pragma unroll
  for (int u = 0; u < C::DPW; ++u)
    d.base[u] = (uintptr_t(uint32_t(__builtin_amdgcn_readlane(mhi, wp * C::DPW + u))) << 32) |
                uint32_t(__builtin_amdgcn_readlane(mlo, wp * C::DPW + u));
  const int rs = lane >> 3;
  uintptr_t tb = d.base[0];
#pragma unroll
  for (int u = 1; u < C::DPW; ++u) tb = rs == u ? d.base[u] : tb;
  d.tail = tb + size_t(64 + ((lane & 7) ^ tail_swz(wp * C::DPW + rs))) * 16;
}
template <class C>
__device__ __forceinline__ void ws_dma_row(const WsDma<C>& d, uint16_t* dst, int u, int wp, int lane) {
  dma16(d.base[u] + size_t(lane) * 16, dst + (wp * C::DPW + u) * C::HSTR);
}
template <class C>
__device__ __forceinline__ void ws_dma_tail(const WsDma<C>& d, uint16_t* dst, int wp) {
  dma16(d.tail, dst + C::TAILO + wp * C::DPW * 64);
}

template <class C>
__global__ __launch_bounds__(C::NT, 1) void attn_ws_kernel(AttnArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  uint16_t* Kb = reinterpret_cast<uint16_t*>(lds);
  uint16_t* Pb = reinterpret_cast<uint16_t*>(lds + C::LDS_K);
  float* Al = reinterpret_cast<float*>(lds + C::LDS_K + C::LDS_P);
  uint32_t* Fl = reinterpret_cast<uint32_t*>(lds + C::LDS_K + C::LDS_P + C::LDS_A);
  int32_t* Cs = reinterpret_cast<int32_t*>(lds + C::LDS_K + C::LDS_P + C::LDS_A + C::LDS_F);

  const int nreq = a.r1 - a.r0;
  const int per_req = a.Q * a.head_groups * a.splits;
  const int b = blockIdx.x;
  const int rr = ((b >> 3) / per_req) * 8 + (b & 7);
  if (rr >= nreq) return;
  const int sub = (b >> 3) % per_req;
  const int j = sub / (a.head_groups * a.splits);
  const int hg = (sub / a.splits) % a.head_groups;
  const int sp = sub % a.splits;
  const int r = a.r0 + rr;
  const int qi = r * a.Q + j;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);      // wave-uniform: held in SGPRs
  const bool score_wave = w < C::NS;
  const int hi_half = lane >> 5;
  const int dq = w - C::NS;                                    // product waves: value quarter
  const int vq0 = dq * (C::D_V / C::NP);
  const size_t blk = (size_t(qi - a.r0 * a.Q) * a.head_groups + hg) * a.splits + sp;   // from the chunk's start

  const int p_j = a.causal[qi];
  if (p_j < 0) {  // inactive query: zero output (the combine pass does it when split)
    if (!score_wave && a.splits == 1) {
      for (int hb = 0; hb < 2; ++hb) {
        const int head = hg * 64 + hb * 32 + (lane & 31);
        if (head < a.H) {
          uint16_t* op = a.out + (size_t(qi) * a.H + head) * C::D_V + vq0;
          for (int d = hi_half; d < C::D_V / C::NP / 4; d += 2)
            *reinterpret_cast<uint2*>(op + d * 4) = make_uint2(0, 0);
        }
      }
    }
    return;
  }
  const int n_r = a.causal[size_t(r) * a.Q];
  int lo = a.ring_lo[r];
  lo = max(lo, p_j - a.W + 1);
  lo = max(lo, 0);
  if (a.block_only) lo = max(lo, n_r);
  const int n_ring = p_j >= lo ? p_j - lo + 1 : 0;

  RowCtx ctx;
  ctx.loc = reinterpret_cast<gint32*>(reinterpret_cast<uintptr_t>(a.loc + size_t(qi) * a.k));
  ctx.k = a.k;
  ctx.n_total = a.k + n_ring;
  ctx.Rd = a.Rd;
  ctx.ring_row0 = r * a.Rd + lo % a.Rd;
  ctx.ring_end = (r + 1) * a.Rd;
  ctx.hot = reinterpret_cast<uintptr_t>(a.hot);
  ctx.d_staging = reinterpret_cast<uintptr_t>(a.staging) - ctx.hot;
  ctx.d_resident = reinterpret_cast<uintptr_t>(a.resident) - ctx.hot;
  ctx.d_ring = reinterpret_cast<uintptr_t>(a.ring) - ctx.hot;
  ctx.zero = reinterpret_cast<uintptr_t>(a.zero);

  const int n_tiles = (ctx.n_total + TILE - 1) / TILE;
  const int tb = int((long long)n_tiles * sp / a.splits);
  const int te = int((long long)n_tiles * (sp + 1) / a.splits);
  const int crow = lane & 31;                          // tile row whose code this lane holds
  const float sl2 = a.scale_log2;

  // tile t lives in buffer (t - tb) mod 4, its codes in slot (t - tb) mod 4,
  // its probabilities in P^T slot (t - tb) mod 2
  auto kbuf = [&](int t) { return Kb + ((t - tb) & 3) * C::BSTR; };
  auto cslot = [&](int t) { return Cs + ((t - tb) & 3) * 64; };
  // DMA of tile t (its codes landed): every wave moves RPW rows; tiles past
  // the range read the zero row, so every wave keeps NVM instructions per tile
  auto tile_code = [&](int t, int raw) { return t < te ? final_code(ctx, t * TILE + crow, raw) : -1; };

  if (score_wave) {
    // ---- score waves: heads hs of this wave.  A k-step's 32 dims are four
    // 16-byte chunks, one per lane quarter g = lane/16: chunk ws_chunk(ks, g)
    // (head region: 16(ks/4) + 2(ks%4) + {0, 8, 1, 9}[g]; tail: 64 + 4(ks-16)
    // + g).  The A fragment (K) of lane l holds tile row 16rb + ws_row(l%16),
    // where ws_row flips bit 2 of rows 8..15: with the chunk offsets this puts
    // the 16 lanes of every LDS service group of a 16-byte read (lanes of
    // equal bit 5 and equal parity of bits 2..4) on 16 distinct bank quads.
    // The B fragment (Q) takes the same chunks.
    const int g = lane >> 4;
    const int hs = hg * 64 + w * 16 + (lane & 15);
    bf16x8 qreg[C::KST];
    {
      const uint16_t* qp = a.q + (size_t(qi) * a.H + (hs < a.H ? hs : 0)) * C::D_QK;
#pragma unroll
      for (int ks = 0; ks < C::KST; ++ks) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (hs < a.H) v = gload16(reinterpret_cast<uintptr_t>(qp + ws_chunk(ks, g) * 8));
        qreg[ks] = __builtin_bit_cast(bf16x8, v);
      }
    }
    float m_run = kNegBig, l_run = 0.f;
    // A fragment offsets: the head region (plus 8 ws_base(ks) per k-step)
    // and the two tail k-steps
    int koff[2], ktail[2][2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int row = rb * 16 + ws_row(lane & 15);
      koff[rb] = row * C::HSTR + ws_chunk(0, g) * 8;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) ktail[rb][kt] = C::TAILO + row * 64 + (((kt * 4 + g) ^ tail_swz(row)) * 8);
    }
    // this lane's scores: D rows 4g + i of each 16-row block = tile rows
    // 16rb + ws_row(4g) + i; P^T written there (head 16w + lane%16)
    const int prow = ws_row(4 * g);
    const int pw_off = (w * 16 + (lane & 15)) * C::PSTR + prow;

    auto score_tile = [&](int t) {
      const uint16_t* kb = kbuf(t);
      const int ps = (t - tb) & 1;
      const int code = final_code(ctx, t * TILE + crow, cslot(t)[lane]);
      const uint32_t live = static_cast<uint32_t>(__builtin_amdgcn_ballot_w64(code >= 0));
      typedef float f32x4 __attribute__((ext_vector_type(4)));
      f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      // K fragments in batches of KB k-steps, the next batch's reads issued
      // before this batch's products (batches of 1, 2 or 3 k-steps measure
      // the same; 6 took 30 more registers and 5% longer, 9 another 10%)
      constexpr int KB = 3, NBT = C::KST / KB;
      static_assert(C::KST % KB == 0, "k-step batches");
      bf16x8 fr[2][2][KB];
      auto load = [&](int bt, bf16x8 (&dst)[2][KB]) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int jj = 0; jj < KB; ++jj) {
            const int ks = bt * KB + jj;
            const int off = ks < 16 ? koff[rb] + ws_base(ks) * 8 : ktail[rb][ks - 16];
            dst[rb][jj] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(kb + off));
          }
      };
      load(0, fr[0]);
#pragma unroll
      for (int bt = 0; bt < NBT; ++bt) {
        if (bt + 1 < NBT) load(bt + 1, fr[(bt + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int jj = 0; jj < KB; ++jj)
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
            acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr[bt & 1][rb][jj], qreg[bt * KB + jj], acc[rb], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      // tile max per head over the raw scores of live rows (the scale is
      // positive, so it is applied to the max once); p = exp2(s*scale - m)
      // with scale and max in one fma
      float r[8];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) r[rb * 4 + i] = acc[rb][i];
      if (__builtin_expect(live != 0xFFFFFFFFu, 0)) {   // wave-uniform: a tile with masked rows
        const uint32_t lmask = live >> prow;             // bits i and 16+i: rows prow+i, 16+prow+i
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (!((lmask >> (rb * 16 + i)) & 1u)) r[rb * 4 + i] = -INFINITY;
      }
      float mt = fmaxf(fmaxf(fmaxf(r[0], r[1]), fmaxf(r[2], r[3])), fmaxf(fmaxf(r[4], r[5]), fmaxf(r[6], r[7])));
      mt = max_x32(max_x16(mt)) * sl2;
      const bool raise = mt > m_run + kRescaleLog2;
      float alpha = 1.f;
      if (raise) {
        alpha = __builtin_amdgcn_exp2f(m_run - mt);
        m_run = mt;
        l_run *= alpha;
      }
      float ps_sum = 0.f;
      uint16_t* pw = Pb + ps * (64 * C::PSTR) + pw_off;
      typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
      typedef float f32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(r[rb * 4 + i], sl2, -m_run));
          ps_sum += p[i];
        }
        const bf16x2 b01 = __builtin_convertvector(f32x2{p[0], p[1]}, bf16x2);
        const bf16x2 b23 = __builtin_convertvector(f32x2{p[2], p[3]}, bf16x2);
        uint2 pk;
        pk.x = __builtin_bit_cast(uint32_t, b01);
        pk.y = __builtin_bit_cast(uint32_t, b23);
        *reinterpret_cast<uint2*>(pw + rb * 16) = pk;
      }
      l_run += ps_sum;
      if (lane < 16) Al[ps * 64 + w * 16 + lane] = alpha;
      const bool any = __builtin_amdgcn_ballot_w64(raise) != 0;
      if (lane == 0) reinterpret_cast<uint8_t*>(Fl + ps)[w] = any ? 1 : 0;
    };

    // prologue: Q in registers, codes of tb..tb+2 (first product wave), then
    // tiles tb..tb+2; scores of tile tb
    __builtin_amdgcn_s_waitcnt(0x0F70);              // vmcnt(0)
    lds_barrier();
    lds_barrier();                                   // tiles tb, tb+1 landed
    if (tb < te) score_tile(tb);
    lds_barrier();
    for (int t = tb; t < te; ++t) {
      if (t + 1 < te) score_tile(t + 1);
      lds_barrier();
    }
    __builtin_amdgcn_s_waitcnt(0x0070);              // vmcnt(0): no DMA outlives the loop
    __syncthreads();
    // (m, l) of this wave's heads: the four lanes of a head in a fixed order
    const float l2 = sum_x32(sum_x16(l_run));
    if (lane < 16) {
      Al[w * 16 + lane] = m_run;
      Al[64 + w * 16 + lane] = l2;
    }
    __syncthreads();
  } else {
    // ---- product waves: value dims vq0 .. vq0 + D_V/NP - 1 of all 64 heads
    f32x16 O[C::DVB][2];
#pragma unroll
    for (int d = 0; d < C::DVB; ++d)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int i = 0; i < 16; ++i) O[d][hb][i] = 0.f;
    int v_off;
    {
      const int gq = (lane >> 4) & 3, s4 = lane & 15, aq = s4 & 3;
      const int row = (gq >> 1) * 8 + (s4 >> 2);
      const int dim = C::V_OFF + vq0 + ((gq & 1) * 2 + (aq >> 1)) * (8 * C::DVB) + (aq & 1) * 4;
      v_off = row * C::RSTR + dim;
    }
    const int pr_off = (lane & 31) * C::PSTR + hi_half * 8;

    const int wp = dq;                               // product wave index: DMA rows wp*DPW ..
    auto issue_all = [&](int t, int raw) {
      WsDma<C> dm;
      ws_dma_prepare<C>(dm, ctx, tile_code(t, raw), wp, lane);
      uint16_t* dst = kbuf(t);
      ws_dma_tail<C>(dm, dst, wp);
#pragma unroll
      for (int u = 0; u < C::DPW; ++u) ws_dma_row<C>(dm, dst, u, wp, lane);
    };
    // products of tile t, with the DMA of tile t+3 (codes raw3) issued between
    // them, so that the address unit works while the matrix core does
    auto product_tile = [&](int t, int raw3) {
      const uint16_t* kb = kbuf(t);
      const int ps = (t - tb) & 1;
      WsDma<C> dm;
      ws_dma_prepare<C>(dm, ctx, tile_code(t + 3, raw3), wp, lane);
      uint16_t* dst = kbuf(t + 3);
      if (Fl[ps] != 0) {
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const float al = Al[ps * 64 + hb * 32 + (lane & 31)];
#pragma unroll
          for (int d = 0; d < C::DVB; ++d)
#pragma unroll
            for (int i = 0; i < 16; ++i) O[d][hb][i] *= al;
        }
      }
      const uint16_t* pr = Pb + ps * (64 * C::PSTR) + pr_off;
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        bf16x8 vfr[C::DVB];
#pragma unroll
        for (int d = 0; d < C::DVB; ++d) {
          const uint16_t* vp = kb + v_off + ks2 * 16 * C::RSTR + d * 8;
          const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp));
          const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp + 4 * C::RSTR));
          vfr[d] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
        }
        bf16x8 pbf[2];
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
          pbf[hb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(pr + hb * 32 * C::PSTR + ks2 * 16));
        // 8 products; DMA instructions after products 0..4 (k-step 0: the
        // tail and rows 0..3; k-step 1: rows 4..7)
#pragma unroll
        for (int x = 0; x < 2 * C::DVB; ++x) {
          const int d = x >> 1, hb = x & 1;
          O[d][hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfr[d], pbf[hb], O[d][hb], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
          if (ks2 == 0 && x == 0) ws_dma_tail<C>(dm, dst, wp);
          if (ks2 == 0 && x >= 1 && x <= 4) ws_dma_row<C>(dm, dst, x - 1, wp, lane);
          if (ks2 == 1 && x <= 3) ws_dma_row<C>(dm, dst, 4 + x, wp, lane);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };

    const bool coder = w == C::NS;                    // the wave that DMAs the codes
    if (coder) {
      dma_codes<C>(cslot(tb), ctx, tb, 0, lane);
      dma_codes<C>(cslot(tb + 1), ctx, tb + 1, 0, lane);
      dma_codes<C>(cslot(tb + 2), ctx, tb + 2, 0, lane);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);              // vmcnt(0)
    lds_barrier();
    issue_all(tb, cslot(tb)[lane]);
    issue_all(tb + 1, cslot(tb + 1)[lane]);
    if (coder) dma_codes<C>(cslot(tb + 3), ctx, tb + 3, 0, lane);
    issue_all(tb + 2, cslot(tb + 2)[lane]);
    lds_vm_barrier<C::NVM>();                        // tiles tb, tb+1 and the codes of tb+3 landed
    lds_barrier();                                   // scores of tile tb
    for (int t = tb; t < te; ++t) {
      const int raw3 = cslot(t + 3)[lane];
      if (coder) dma_codes<C>(cslot(t + 4), ctx, t + 4, 0, lane);
      product_tile(t, raw3);
      lds_vm_barrier<C::NVM>();                      // tile t+2 and the codes of t+4 landed
    }
    __builtin_amdgcn_s_waitcnt(0x0070);              // vmcnt(0): no DMA outlives the loop
    __syncthreads();
    __syncthreads();                                 // (m, l) of every head in LDS

    // O^T register i of block d holds value dim vq0 + (i/4)*8*DVB + d*8 + hi*4 + i%4
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int hl = hb * 32 + (lane & 31);
      const int head = hg * 64 + hl;
      const float l_tot = Al[64 + hl];
      if (a.splits == 1) {
        if (head < a.H) {
          const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
          uint16_t* op = a.out + (size_t(qi) * a.H + head) * C::D_V + vq0 + hi_half * 4;
#pragma unroll
          for (int d = 0; d < C::DVB; ++d)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              uint16_t h4[4];
#pragma unroll
              for (int e = 0; e < 4; ++e)
                h4[e] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(O[d][hb][g4 * 4 + e] * inv));
              uint2 pk;
              pk.x = uint32_t(h4[0]) | (uint32_t(h4[1]) << 16);
              pk.y = uint32_t(h4[2]) | (uint32_t(h4[3]) << 16);
              *reinterpret_cast<uint2*>(op + g4 * 8 * C::DVB + d * 8) = pk;
            }
        }
      } else {
        float* po = a.part_o + (blk * 64 + hl) * C::D_V + vq0 + hi_half * 4;
#pragma unroll
        for (int d = 0; d < C::DVB; ++d)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4)
            *reinterpret_cast<float4*>(po + g4 * 8 * C::DVB + d * 8) =
                make_float4(O[d][hb][g4 * 4 + 0], O[d][hb][g4 * 4 + 1], O[d][hb][g4 * 4 + 2], O[d][hb][g4 * 4 + 3]);
        if (dq == 0 && hi_half == 0) {
          float* pm = a.part_ml + (blk * 64 + hl) * 2;
          pm[0] = Al[hl];
          pm[1] = l_tot;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Narrow rows (144 elements: K = all 144, V = the first 128) above 32 heads.
// One workgroup = one query x HB 32-head blocks (2: 64 heads, or 4: 128
// heads, each row then gathered once per query) x one key split.  A wave
// takes one head block and RB of the two 32-row blocks of every 64-row tile
// (RB = 1: two waves per head block, one per row half, 4 waves at 64 heads;
// RB = 2: one wave per head block, 4 waves at 128 heads, two workgroups per
// CU) over the whole key width (its heads' Q fragments stay in registers),
// so its scores are complete in its own accumulators.  The softmax runs in registers (the
// 32 rows of a head sit in lanes l and l+32) and the probabilities go from
// the accumulators straight into the B operand of O^T = V^T P^T; the V^T
// fragments are read in the same row order (rows 4hi..4hi+3 and 8+4hi..+3 of
// each 16-row k-step).  Tiles go from memory to LDS by DMA, two tiles ahead,
// in a chunk-major layout: chunk c of tile row rho sits in 16-byte slot
// c*64 + ((rho + c) & 63), so that the K reads (32 rows of one chunk) and the
// transposed V reads (4 rows x 4 chunks per half-wave) hit every bank once.
// One barrier per tile.  With two waves per head block each half keeps its
// own (m, l, O) and half 1 hands them to half 0 through LDS at the end.  Sum
// order depends only on list order and split boundaries.
template <int D_QK_, int V_OFF_, int D_V_, int ROW_, int HB_, int RB_>
struct NCfg {
  static constexpr int D_QK = D_QK_, V_OFF = V_OFF_, D_V = D_V_, ROW = ROW_;
  static constexpr int HB = HB_;               // 32-head blocks
  static constexpr int RB = RB_;               // 32-row blocks of a tile per wave
  static constexpr int NH = 2 / RB;            // waves per head block
  static constexpr int NW = NH * HB;           // waves: head block w % HB, row half w / HB
  static constexpr int MINB = RB == 2 ? 2 : 1; // workgroups per CU the registers are sized for
  static constexpr int NT = NW * 64;
  static constexpr int T = 64;                 // rows per tile
  static constexpr int KST = D_QK / 16;        // 16-dim k-steps over the key width
  static constexpr int DVB = D_V / 32;         // 32-dim value blocks (a wave holds all value dims)
  static constexpr int RCH = ROW / 8;          // 16-byte chunks per row
  static constexpr int TBUF = RCH * T * 8;     // elements per tile buffer (chunk-major, unpadded)
  static constexpr int NBUF = 3;
  // DMA instructions per wave and tile: the chunk columns 16/NW of every row,
  // a 1/(NW/2) share of chunk column 16 or 17, the codes
  static constexpr int NCOL = 16 / NW;
  static constexpr int NVM = NCOL + 2;
  static constexpr size_t LDS_K = size_t(NBUF) * TBUF * 2;
  static constexpr size_t LDS_C = size_t(3) * NW * 64 * 4;      // per wave, three 64-entry code slots
  // value blocks of O handed over per merge phase (16 registers x 64 lanes x
  // 4 B per block and head block, in the tile buffers)
  static constexpr int DPH = size_t(HB) * DVB * 4096 <= LDS_K ? DVB : (size_t(HB) * 2 * 4096 <= LDS_K ? 2 : 1);
  static constexpr size_t LDS_ML = NH > 1 ? size_t(HB) * 32 * 2 * 4 : 0;
  static constexpr size_t LDS = LDS_K + LDS_C + LDS_ML;
  static_assert(RB == 1 || RB == 2, "row blocks");
  static_assert(D_QK % 16 == 0 && D_V % 32 == 0 && ROW % 8 == 0, "shape");
  static_assert(V_OFF % 8 == 0 && V_OFF + D_V <= ROW && D_QK <= ROW, "row layout");
  // the DMA split: chunk columns w, w+NW, .. below 16 per wave, columns 16
  // and 17 in shares of 64/(NW/2) rows
  static_assert((NW == 8 || NW == 4 || NW == 2) && RCH == 18, "DMA split");
  static_assert(DVB % DPH == 0, "merge");
  static_assert(LDS <= 160 * 1024, "LDS");
};

// Element offset of (tile row rho, chunk c) in a chunk-major tile buffer.
__device__ __forceinline__ int narrow_slot(int rho, int c) { return (c * 64 + ((rho + c) & 63)) * 8; }

// DMA of one 64-row tile into buffer dst.  Lane l holds the code of tile row
// l; the instruction for chunk c moves row (l - c) & 63 in lane l (its
// address taken from that lane), landing in slot c*64 + l.  Wave w of NW
// moves chunks w, w+NW, .. below 16 of every row and the slots
// 64/(NW/2) * (w/2) .. +64/(NW/2)-1 of chunk 16 + (w & 1): 16/NW + 1
// instructions.  Returns the tile's live-row mask.
template <class C>
__device__ __forceinline__ uint64_t dma_narrow_tile(uint16_t* dst, const RowCtx& ctx, int code, int w, int lane) {
  const uint64_t live = __builtin_amdgcn_ballot_w64(code >= 0);
  const uintptr_t my = row_addr<C::ROW>(ctx, code);
  const int mlo = static_cast<int>(static_cast<uint32_t>(my));
  const int mhi = static_cast<int>(static_cast<uint32_t>(my >> 32));
  auto src_row = [&](int c) {
    const int src = (lane - c) & 63;
    return (uintptr_t(uint32_t(__shfl(mhi, src, 64))) << 32) | uint32_t(__shfl(mlo, src, 64));
  };
#pragma unroll
  for (int u = 0; u < C::NCOL; ++u) {
    const int c = w + C::NW * u;
    dma16(src_row(c) + size_t(c) * 16, dst + c * 64 * 8);
  }
  const int c = 16 + (w & 1);
  const uintptr_t ga = src_row(c) + size_t(c) * 16;
  if (lane / (128 / C::NW) == (w >> 1)) dma16(ga, dst + c * 64 * 8);
  return live;
}

// DMA of the raw codes of tile t (64 rows) into this wave's slot.
__device__ __forceinline__ void dma_narrow_codes(int32_t* slot, const RowCtx& c, int t, int lane) {
  dma4(reinterpret_cast<uintptr_t>(c.loc + min(t * 64 + lane, c.k - 1)), slot);
}

template <class C>
__global__ __launch_bounds__(C::NT, C::MINB) void attn_narrow_kernel(AttnArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  uint16_t* Kb = reinterpret_cast<uint16_t*>(lds);
  float* Om = reinterpret_cast<float*>(lds);                     // merge area (tile buffers, after the loop)
  int32_t* Cs = reinterpret_cast<int32_t*>(lds + C::LDS_K);      // code slots
  float* Mm = reinterpret_cast<float*>(lds + C::LDS_K + C::LDS_C);   // [HB][32] running max of half 1
  float* Ml = Mm + C::HB * 32;                                   // [HB][32] normaliser of half 1

  const int nreq = a.r1 - a.r0;
  const int per_req = a.Q * a.head_groups * a.splits;
  const int b = blockIdx.x;
  const int rr = ((b >> 3) / per_req) * 8 + (b & 7);
  if (rr >= nreq) return;
  const int sub = (b >> 3) % per_req;
  const int j = sub / (a.head_groups * a.splits);
  const int hg = (sub / a.splits) % a.head_groups;
  const int sp = sub % a.splits;
  const int r = a.r0 + rr;
  const int qi = r * a.Q + j;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hb = w % C::HB, h = w / C::HB;
  const int hl = hb * 32 + (lane & 31);
  const int head = hg * 32 * C::HB + hl;
  const size_t blk = (size_t(qi - a.r0 * a.Q) * a.head_groups + hg) * a.splits + sp;
  const int hi_half = lane >> 5;

  const int p_j = a.causal[qi];
  if (p_j < 0) {  // inactive query: zero output (the combine pass does it when split)
    if (a.splits == 1 && h == 0 && head < a.H) {
      uint16_t* op = a.out + (size_t(qi) * a.H + head) * C::D_V;
      for (int d = hi_half; d < C::D_V / 4; d += 2) *reinterpret_cast<uint2*>(op + d * 4) = make_uint2(0, 0);
    }
    return;
  }
  const int n_r = a.causal[size_t(r) * a.Q];
  int lo = a.ring_lo[r];
  lo = max(lo, p_j - a.W + 1);
  lo = max(lo, 0);
  if (a.block_only) lo = max(lo, n_r);
  const int n_ring = p_j >= lo ? p_j - lo + 1 : 0;

  RowCtx ctx;
  ctx.loc = reinterpret_cast<gint32*>(reinterpret_cast<uintptr_t>(a.loc + size_t(qi) * a.k));
  ctx.k = a.k;
  ctx.n_total = a.k + n_ring;
  ctx.Rd = a.Rd;
  ctx.ring_row0 = r * a.Rd + lo % a.Rd;
  ctx.ring_end = (r + 1) * a.Rd;
  ctx.hot = reinterpret_cast<uintptr_t>(a.hot);
  ctx.d_staging = reinterpret_cast<uintptr_t>(a.staging) - ctx.hot;
  ctx.d_resident = reinterpret_cast<uintptr_t>(a.resident) - ctx.hot;
  ctx.d_ring = reinterpret_cast<uintptr_t>(a.ring) - ctx.hot;
  ctx.zero = reinterpret_cast<uintptr_t>(a.zero);

  const int n_tiles = (ctx.n_total + C::T - 1) / C::T;
  const int tb = int((long long)n_tiles * sp / a.splits);
  const int te = int((long long)n_tiles * (sp + 1) / a.splits);

  // Q fragments over the whole key width: B operand of S^T = K Q^T
  bf16x8 qreg[C::KST];
  {
    const uint16_t* qp = a.q + (size_t(qi) * a.H + head) * C::D_QK + hi_half * 8;
#pragma unroll
    for (int ks = 0; ks < C::KST; ++ks) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (head < a.H) v = gload16(reinterpret_cast<uintptr_t>(qp + ks * 16));
      qreg[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }
  f32x16 O[C::DVB];
#pragma unroll
  for (int d = 0; d < C::DVB; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) O[d][i] = 0.f;
  float m_run = kNegBig, l_run = 0.f;
  const float sl2 = a.scale_log2;

  // tile x lives in buffer (x - tb) mod 3, its codes in slot (x - tb) mod 3
  int32_t* cs_w = Cs + w * 64;
  auto cslot = [&](int x) { return cs_w + ((x - tb) % 3) * (C::NW * 64); };
  // prologue: the codes of tb, tb+1 loaded beside the Q fragments, one wait
  // for both (the Q registers are then complete for the whole loop); DMA of
  // tiles tb, tb+1 and of the codes of tb+2, tb+3; tile tb and the codes of
  // tb+2 landed before the first tile
  dma_narrow_codes(cslot(tb), ctx, tb, lane);
  dma_narrow_codes(cslot(tb + 1), ctx, tb + 1, lane);
  __builtin_amdgcn_s_waitcnt(0x0F70);              // vmcnt(0)
  uint64_t live_cur = dma_narrow_tile<C>(Kb, ctx, final_code(ctx, tb * C::T + lane, cslot(tb)[lane]), w, lane);
  dma_narrow_codes(cslot(tb + 2), ctx, tb + 2, lane);
  uint64_t live_n1 = dma_narrow_tile<C>(Kb + C::TBUF, ctx, final_code(ctx, (tb + 1) * C::T + lane, cslot(tb + 1)[lane]),
                                        w, lane);
  dma_narrow_codes(cslot(tb + 3), ctx, tb + 3, lane);
  lds_vm_barrier<C::NVM>();

  // per-lane parts of the LDS offsets in row block b = h*RB + rb: K fragment
  // rows 32b + lane%32, chunk 2ks + hi; V^T rows 32b + 16ks2 + 4(gq/2) + s/4
  // (+8), chunks c0 + d
  const int krow = lane & 31;
  int vrow, vc0, vsub;
  {
    const int gq = (lane >> 4) & 3, sl = lane & 15, aq = sl & 3;
    vrow = (gq >> 1) * 4 + (sl >> 2);
    vc0 = C::V_OFF / 8 + ((gq & 1) * 2 + (aq >> 1)) * C::DVB;
    vsub = (aq & 1) * 4;
  }
  uint64_t live_n2 = 0;

  auto tile = [&](int t, auto pconst) {
    constexpr int P = decltype(pconst)::value;       // (t - tb) mod 3: buffer of tile t
    const uint16_t* kb = Kb + P * C::TBUF;
    // the codes of tile t+2 (landed before the last barrier), then this
    // tile's K fragments: their LDS latency passes while the next DMA is
    // issued (LDS reads complete in order, so the codes come first)
    const int raw2 = (cs_w + ((P + 2) % 3) * (C::NW * 64))[lane];
    auto kfrag = [&](int rb, int ks) {
      return __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const uint4*>(kb + narrow_slot(32 * (h * C::RB + rb) + krow, 2 * ks + hi_half)));
    };
    bf16x8 kf[C::KST];
#pragma unroll
    for (int ks = 0; ks < C::KST; ++ks) kf[ks] = kfrag(0, ks);
    // DMA of tile t+2 into the buffer of tile t-1 (its readers passed the
    // last barrier) and of the codes of tile t+4 into the slot of t+1;
    // unconditional, so that every wave keeps NVM instructions per tile
    // (positions past the range read the zero row and are never used)
    {
      live_n2 = dma_narrow_tile<C>(Kb + ((P + 2) % 3) * C::TBUF, ctx, final_code(ctx, (t + 2) * C::T + lane, raw2), w,
                                   lane);
      dma_narrow_codes(cs_w + ((P + 1) % 3) * (C::NW * 64), ctx, t + 4, lane);
    }

    // scores of this wave's row blocks x 32 heads
    // (the second block's K fragments replace the first's as they are used)
    f32x16 acc[C::RB];
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[rb][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < C::KST; ++ks) {
        acc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qreg[ks], acc[rb], 0, 0, 0);
        if (rb + 1 < C::RB) kf[ks] = kfrag(rb + 1, ks);
      }
    }
    // V^T fragments, read while the scores are finished and exponentiated:
    // k-step ks2 covers rows 16ks2 + {4hi..4hi+3, 8+4hi..8+4hi+3} of the
    // block, the rows whose probabilities this lane holds
    auto vfrag = [&](int rb, int ks2, int d) {
      const int c = vc0 + d;
      const int row = 32 * (h * C::RB + rb) + vrow + 16 * ks2;
      const uint16_t* vp0 = kb + narrow_slot(row, c) + vsub;
      const uint16_t* vp1 = kb + narrow_slot(row + 8, c) + vsub;
      const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp0));
      const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp1));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    bf16x8 vfr[2][C::DVB];
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
      for (int d = 0; d < C::DVB; ++d) vfr[ks2][d] = vfrag(0, ks2, d);
    // register i of block b holds tile row 32b + 8(i/4) + 4hi + i%4 of head
    // lane%32; dead rows (pads, positions past the window) only in a tile
    // whose live mask says so (wave-uniform test)
    const uint64_t lvw = C::RB == 2 ? live_cur : (live_cur >> (32 * h)) & 0xFFFFFFFFull;
    float sc[C::RB][16];
    if (lvw == (C::RB == 2 ? ~0ull : 0xFFFFFFFFull)) {
#pragma unroll
      for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[rb][i] = acc[rb][i];
    } else {
#pragma unroll
      for (int rb = 0; rb < C::RB; ++rb) {
        const uint32_t lv = static_cast<uint32_t>(lvw >> (32 * rb)) >> (4 * hi_half);
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[rb][i] = (lv >> (8 * (i / 4) + i % 4)) & 1u ? acc[rb][i] : -INFINITY;
      }
    }
    // the scale is positive, so the lane's largest scaled score is its
    // largest raw score times the scale (rounding is monotone)
    float mx = sc[0][0];
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[rb][i]);
    if (__builtin_amdgcn_ballot_w64(mx * sl2 > m_run + kRescaleLog2) != 0) {
      // a score exceeds its head's running max by more than 2^8: raise the
      // max of that head (both lanes of the pair take the pair's tile max)
      const float mq = fmaxf(mx, __shfl_xor(mx, 32, 64)) * sl2;
      if (mq > m_run + kRescaleLog2) {
        const float alpha = __builtin_amdgcn_exp2f(m_run - mq);
        l_run *= alpha;
        m_run = mq;
#pragma unroll
        for (int d = 0; d < C::DVB; ++d)
#pragma unroll
          for (int i = 0; i < 16; ++i) O[d][i] *= alpha;
      }
    }
    float ps = 0.f;
    bf16x8 pb[C::RB][2];
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[rb][i], sl2, -m_run));
        ps += p;
        pb[rb][i / 8][i % 8] = static_cast<__bf16>(p);
      }
    l_run += ps;

    // O^T += V^T P^T (the second block's V^T fragments replace the first's
    // as they are used)
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
        for (int d = 0; d < C::DVB; ++d) {
          O[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfr[ks2][d], pb[rb][ks2], O[d], 0, 0, 0);
          if (rb + 1 < C::RB) vfr[ks2][d] = vfrag(rb + 1, ks2, d);
        }
    live_cur = live_n1;
    live_n1 = live_n2;
    // tile t+1 and the codes of t+3 landed in every wave (the NVM
    // instructions of this tile stay in flight); this tile's readers done
    lds_vm_barrier<C::NVM>();
  };
  for (int t = tb; t < te; t += 3) {
    tile(t, std::integral_constant<int, 0>{});
    if (t + 1 < te) tile(t + 1, std::integral_constant<int, 1>{});
    if (t + 2 < te) tile(t + 2, std::integral_constant<int, 2>{});
  }
  // no DMA outlives the loop, in any wave, before the tile buffers take the merge
  __builtin_amdgcn_s_waitcnt(0x0070);              // vmcnt(0)
  if constexpr (C::NH == 2) __syncthreads();

  const float l2 = l_run + __shfl_xor(l_run, 32, 64);
  float m_tot = m_run, l_tot = l2;
  if constexpr (C::NH == 2) {
    // merge the halves: half 1 hands (m, l, O) to half 0 through LDS
    if (h == 1 && lane < 32) {
      Mm[hb * 32 + lane] = m_run;
      Ml[hb * 32 + lane] = l2;
    }
    float a0 = 1.f, a1 = 0.f;
#pragma unroll
    for (int ph = 0; ph < C::DVB / C::DPH; ++ph) {
      if (h == 1) {
#pragma unroll
        for (int dd = 0; dd < C::DPH; ++dd)
#pragma unroll
          for (int i = 0; i < 16; ++i) Om[((hb * C::DPH + dd) * 16 + i) * 64 + lane] = O[ph * C::DPH + dd][i];
      }
      __syncthreads();
      if (h == 0) {
        if (ph == 0) {
          const float m1 = Mm[hb * 32 + (lane & 31)], l1 = Ml[hb * 32 + (lane & 31)];
          m_tot = fmaxf(m_run, m1);
          a0 = __builtin_amdgcn_exp2f(m_run - m_tot);
          a1 = __builtin_amdgcn_exp2f(m1 - m_tot);
          l_tot = l2 * a0 + l1 * a1;
        }
#pragma unroll
        for (int dd = 0; dd < C::DPH; ++dd)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            O[ph * C::DPH + dd][i] = O[ph * C::DPH + dd][i] * a0 + Om[((hb * C::DPH + dd) * 16 + i) * 64 + lane] * a1;
      }
      __syncthreads();
    }
    if (h != 0) return;
  }

  // O^T register i of block d holds value dim (i/4)*8*DVB + d*8 + hi*4 + i%4
  if (a.splits == 1) {
    if (head < a.H) {
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      uint16_t* op = a.out + (size_t(qi) * a.H + head) * C::D_V + hi_half * 4;
#pragma unroll
      for (int d = 0; d < C::DVB; ++d)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          uint16_t h4[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            h4[e] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(O[d][g4 * 4 + e] * inv));
          uint2 pk;
          pk.x = uint32_t(h4[0]) | (uint32_t(h4[1]) << 16);
          pk.y = uint32_t(h4[2]) | (uint32_t(h4[3]) << 16);
          *reinterpret_cast<uint2*>(op + g4 * 8 * C::DVB + d * 8) = pk;
        }
    }
  } else {
    float* po = a.part_o + (blk * 32 * C::HB + hl) * C::D_V + hi_half * 4;
#pragma unroll
    for (int d = 0; d < C::DVB; ++d)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *reinterpret_cast<float4*>(po + g4 * 8 * C::DVB + d * 8) =
            make_float4(O[d][g4 * 4 + 0], O[d][g4 * 4 + 1], O[d][g4 * 4 + 2], O[d][g4 * 4 + 3]);
    if (hi_half == 0) {
      float* pm = a.part_ml + (blk * 32 * C::HB + hl) * 2;
      pm[0] = m_tot;
      pm[1] = l_tot;
    }
  }
}

// Merge of key splits: out = sum_s 2^(m_s-m) O_s / sum_s 2^(m_s-m) l_s, the
// sums in split order.  One 256-thread block per (query, head group, 8 heads):
// 32 threads per head, each over float4 groups of value dims 128g + 4(t mod
// 32), so every load instruction reads 512 contiguous bytes.  Block index ->
// request as in the attention kernel, so the partials are read on the XCD
// (and from the L2) where they were written.
template <int D_V, int HB>
__global__ __launch_bounds__(256) void combine_kernel(AttnArgs a) {
  constexpr int HPW = 32 * HB, N8 = HPW / 8;
  const int nreq = a.r1 - a.r0;
  const int per_req = a.Q * a.head_groups * N8;
  const int b = blockIdx.x;
  const int rr = ((b >> 3) / per_req) * 8 + (b & 7);
  if (rr >= nreq) return;
  const int sub = (b >> 3) % per_req;
  const int j = sub / (a.head_groups * N8);
  const int hg = (sub / N8) % a.head_groups;
  const int hl = (sub % N8) * 8 + int(threadIdx.x >> 5);
  const int qi = (a.r0 + rr) * a.Q + j;
  const int head = hg * HPW + hl;
  if (head >= a.H) return;
  const int d0 = 4 * int(threadIdx.x & 31);
  uint16_t* op = a.out + (size_t(qi) * a.H + head) * D_V;
  if (a.causal[qi] < 0) {
    for (int d = d0; d < D_V; d += 128) *reinterpret_cast<uint2*>(op + d) = make_uint2(0, 0);
    return;
  }
  const size_t blk0 = (size_t(qi - a.r0 * a.Q) * a.head_groups + hg) * a.splits;
  float m = kNegBig;
  for (int s = 0; s < a.splits; ++s) m = fmaxf(m, a.part_ml[((blk0 + s) * HPW + hl) * 2]);
  float wsum[8];
  float den = 0.f;
  for (int s = 0; s < 8; ++s) {
    wsum[s] = 0.f;
    if (s < a.splits) {
      const float* pm = a.part_ml + ((blk0 + s) * HPW + hl) * 2;
      wsum[s] = exp2f(pm[0] - m);
      den += pm[1] * wsum[s];
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  for (int d = d0; d < D_V; d += 128) {
    float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < a.splits; ++s) {
      const float4 o = *reinterpret_cast<const float4*>(a.part_o + ((blk0 + s) * HPW + hl) * D_V + d);
      num.x += o.x * wsum[s];
      num.y += o.y * wsum[s];
      num.z += o.z * wsum[s];
      num.w += o.w * wsum[s];
    }
    uint2 pk;
    pk.x = uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(num.x * inv))) |
           (uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(num.y * inv))) << 16);
    pk.y = uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(num.z * inv))) |
           (uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(num.w * inv))) << 16);
    *reinterpret_cast<uint2*>(op + d) = pk;
  }
}

template <class C>
hipError_t set_lds_limit() {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(attn_kernel<C>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, int(C::LDS));
}

template <class C>
hipError_t set_ws_lds_limit() {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(attn_ws_kernel<C>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, int(C::LDS));
}

template <class C>
hipError_t set_narrow_lds_limit() {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(attn_narrow_kernel<C>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, int(C::LDS));
}

// Events, when given, are bound to the launch (they complete with it and time
// its own start and end); with nothing to launch they are recorded in place.
hipError_t no_launch(hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
  if (ev_start) (void)hipEventRecord(ev_start, s);
  if (ev_stop) return hipEventRecord(ev_stop, s);
  return hipSuccess;
}

template <class K, class... Args>
hipError_t launch_with(K kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s, hipEvent_t ev_start,
                       hipEvent_t ev_stop, Args... args) {
  if (ev_start || ev_stop) {
    hipExtLaunchKernelGGL(kernel, grid, block, uint32_t(lds), s, ev_start, ev_stop, 0, args...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
  }
  return hipGetLastError();
}

template <class C>
hipError_t launch_cfg(const AttnArgs& a, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
  const int nreq = a.r1 - a.r0;
  if (nreq <= 0) return no_launch(s, ev_start, ev_stop);
  const int per_req = a.Q * a.head_groups * a.splits;
  const long long blocks = (long long)((nreq + 7) / 8) * 8 * per_req;
  return launch_with(attn_kernel<C>, dim3(unsigned(blocks)), dim3(C::NT), C::LDS, s, ev_start, ev_stop, a);
}

template <class C>
hipError_t launch_ws(const AttnArgs& a, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
  const int nreq = a.r1 - a.r0;
  if (nreq <= 0) return no_launch(s, ev_start, ev_stop);
  const int per_req = a.Q * a.head_groups * a.splits;
  const long long blocks = (long long)((nreq + 7) / 8) * 8 * per_req;
  return launch_with(attn_ws_kernel<C>, dim3(unsigned(blocks)), dim3(C::NT), C::LDS, s, ev_start, ev_stop, a);
}

template <class C>
hipError_t launch_narrow(const AttnArgs& a, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
  const int nreq = a.r1 - a.r0;
  if (nreq <= 0) return no_launch(s, ev_start, ev_stop);
  const int per_req = a.Q * a.head_groups * a.splits;
  const long long blocks = (long long)((nreq + 7) / 8) * 8 * per_req;
  return launch_with(attn_narrow_kernel<C>, dim3(unsigned(blocks)), dim3(C::NT), C::LDS, s, ev_start, ev_stop, a);
}

}  // namespace

hipError_t attn_init_attributes() {
  hipError_t e = set_lds_limit<Cfg<576, 0, 512, 576, 1>>();
  if (e == hipSuccess) e = set_ws_lds_limit<WCfg<576, 0, 512, 576>>();
  if (e == hipSuccess) e = set_lds_limit<Cfg<128, 128, 128, 256, 1>>();
  if (e == hipSuccess) e = set_lds_limit<Cfg<128, 128, 128, 256, 2>>();
  if (e == hipSuccess) e = set_lds_limit<Cfg<144, 0, 128, 144, 1>>();
  if (e == hipSuccess) e = set_narrow_lds_limit<NCfg<144, 0, 128, 144, 2, 1>>();
  if (e == hipSuccess) e = set_narrow_lds_limit<NCfg<144, 0, 128, 144, 4, 2>>();
  return e;
}

bool attn_layout_supported(int row_elems, int d_qk, int v_off, int d_v) {
  return (row_elems == 576 && d_qk == 576 && v_off == 0 && d_v == 512) ||
         (row_elems == 256 && d_qk == 128 && v_off == 128 && d_v == 128) ||
         (row_elems == 144 && d_qk == 144 && v_off == 0 && d_v == 128);
}

// Heads of one workgroup: one 32-head block up to 32 heads, else two; rows of
// 144 elements take four blocks (two waves each) above 64 heads, so that each
// query's rows are gathered once.
// Heads of one workgroup: one 32-head block up to 32 heads, else two.  Rows
// of 144 elements above 64 heads take the narrow-row kernel with four blocks
// (each query's rows gathered once) when the launch still has at least 256
// workgroups; with fewer, two blocks per workgroup keep every CU busy (the
// 128-head workgroup is one per CU and would leave CUs idle).
int attn_heads_per_wg(int H, int row_elems, int64_t queries) {
  if (H <= 32) return 32;
  if (row_elems == 144 && H > 64 && queries * ((H + 127) / 128) >= 256) return 128;
  return 64;
}

hipError_t launch_attn(const AttnArgs& a, int row_elems, int d_qk, int v_off, int d_v, hipStream_t s,
                       hipEvent_t ev_start, hipEvent_t ev_stop) {
  const int hpw = a.hpw;
  if (row_elems == 576 && d_qk == 576 && v_off == 0 && d_v == 512) {
    if (hpw == 32) return launch_cfg<Cfg<576, 0, 512, 576, 1>>(a, s, ev_start, ev_stop);
    return launch_ws<WCfg<576, 0, 512, 576>>(a, s, ev_start, ev_stop);
  }
  if (row_elems == 256 && d_qk == 128 && v_off == 128 && d_v == 128) {
    if (hpw == 32) return launch_cfg<Cfg<128, 128, 128, 256, 1>>(a, s, ev_start, ev_stop);
    return launch_cfg<Cfg<128, 128, 128, 256, 2>>(a, s, ev_start, ev_stop);
  }
  if (row_elems == 144 && d_qk == 144 && v_off == 0 && d_v == 128) {
    if (hpw == 32) return launch_cfg<Cfg<144, 0, 128, 144, 1>>(a, s, ev_start, ev_stop);
    if (hpw == 128) return launch_narrow<NCfg<144, 0, 128, 144, 4, 2>>(a, s, ev_start, ev_stop);
    return launch_narrow<NCfg<144, 0, 128, 144, 2, 1>>(a, s, ev_start, ev_stop);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attn_combine(const AttnArgs& a, int d_v, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
  const int nreq = a.r1 - a.r0;
  if (nreq <= 0 || a.splits <= 1) return no_launch(s, ev_start, ev_stop);
  const int hpw = a.hpw;
  const dim3 grid(unsigned(((nreq + 7) / 8) * 8 * a.Q * a.head_groups * (hpw / 8)));
  if (d_v == 512) {
    if (hpw == 32) return launch_with(combine_kernel<512, 1>, grid, dim3(256), 0, s, ev_start, ev_stop, a);
    return launch_with(combine_kernel<512, 2>, grid, dim3(256), 0, s, ev_start, ev_stop, a);
  }
  if (d_v == 128) {
    if (hpw == 32) return launch_with(combine_kernel<128, 1>, grid, dim3(256), 0, s, ev_start, ev_stop, a);
    if (hpw == 128) return launch_with(combine_kernel<128, 4>, grid, dim3(256), 0, s, ev_start, ev_stop, a);
    return launch_with(combine_kernel<128, 2>, grid, dim3(256), 0, s, ev_start, ev_stop, a);
  }
  return hipErrorInvalidValue;
}

}  // namespace kvh
