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
//    N dimension and 32-row tiles of K form M: S^T = K Q^T with
//    v_mfma_f32_32x32x16_bf16; every lane then holds 16 scores of ONE head,
//    which makes the online softmax a per-lane update plus one cross-half
//    exchange, and the probabilities are already the B operand of
//    O^T = V^T P^T (no register transpose).
//  - waves come in pairs per 32-head block; the pair splits the key width for
//    QK^T (partial scores summed through LDS in a fixed order) and the value
//    width for PV, so Q fragments (registers) and O accumulators are halved.
//  - a tile is gathered from HBM through location codes into registers one
//    tile ahead (software prefetch), then written to LDS twice: row-major for
//    the K operand and transposed (4 rows per 8-byte write) for the V operand.
//  - softmax in fp32 with exp2 (scale folded with log2 e); P is rounded to bf16
//    for the PV contraction, the normaliser is accumulated from fp32 P.
//  - the sum order depends only on the list order and the split boundaries,
//    never on where a row is cached, so outputs are bitwise identical across
//    cache states.
//  - block index -> (request, query, head group, split) keeps every workgroup
//    of one request on one XCD (dispatch is round-robin over the 8 XCDs), so
//    rows shared by a request's queries are re-read from that XCD's L2.
#include "common.h"

namespace kvh {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
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
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;
// The running max of a head is raised only when a tile's max exceeds it by
// more than this (log2 units): numerator and normaliser always share the same
// max, so the result is unchanged, and p stays below 2^8.
constexpr float kRescaleLog2 = 8.0f;

template <int D_QK_, int V_OFF_, int D_V_, int ROW_, int HB_>
struct Cfg {
  static constexpr int D_QK = D_QK_, V_OFF = V_OFF_, D_V = D_V_, ROW = ROW_, HB = HB_;
  static constexpr int NDP = 4;              // waves per 32-head block: key / value width split
  static constexpr int NW = NDP * HB;
  static constexpr int NT = NW * 64;
  static constexpr int KS = D_QK / NDP / 16; // 16-wide k-steps over this wave's key part
  static constexpr int DVB = D_V / NDP / 32; // 32-wide value blocks of this wave's value part
  static constexpr int KCH = D_QK / 8;       // 16-byte chunks of the key
  static constexpr int V0 = V_OFF / 8, VCH = D_V / 8;
  static constexpr bool V_IN_K = (V_OFF == 0 && D_V <= D_QK);
  static constexpr int KO0 = V_IN_K ? VCH : 0;          // first key-only chunk
  static constexpr int NKO = V_IN_K ? (KCH - VCH) : KCH;
  static constexpr int KSTR = D_QK + 8;      // key tile row stride (elements): 16 B mod 128 B
  static constexpr int VSTR = TILE + 4;      // transposed value stride (elements)
  // (4-row group, value chunk) load tasks; consecutive tasks take consecutive
  // row groups, so a wave covers 8 row groups x 8 chunks: each load reads 8
  // whole 128-byte lines and the transposed 8-byte LDS writes hit every bank
  static constexpr int T1 = (TILE / 4) * VCH;
  static constexpr int T2 = TILE * NKO;         // (row, key-only chunk) load tasks
  static constexpr int T1PT = (T1 + NT - 1) / NT;
  static constexpr int T2PT = (T2 + NT - 1) / NT;
  static constexpr size_t LDS_K = size_t(TILE) * KSTR * 2;
  static constexpr size_t LDS_V = size_t(D_V) * VSTR * 2;
  static constexpr size_t LDS_S = size_t(NW) * 16 * 64 * 4;
  static constexpr size_t LDS = LDS_K + LDS_V + LDS_S + TILE * 4;
  static_assert(D_QK % (NDP * 16) == 0 && D_V % (NDP * 32) == 0 && ROW % 8 == 0, "shape");
  static_assert(V_IN_K || V_OFF >= D_QK, "value range must lie inside or after the key range");
  static_assert(LDS <= 160 * 1024, "LDS");
};

struct RowCtx {
  gint32* loc;
  int k, n_total, Rd;
  int ring_row0;    // ring row of the window's first position: r*R_d + (lo mod R_d)
  int ring_end;     // (r+1)*R_d: ring rows wrap from here back to r*R_d
  size_t ring_base;
  uintptr_t hot, d_staging, d_resident, d_ring;   // d_*: pool base minus hot base
};

// Location codes: a list entry's code is loaded raw (c.loc) one tile before
// its row is loaded and is only decoded when the row load is issued, so the
// wave never waits on a code load; positions past the list are the ring
// window (tier 3, index r*R_d + pos mod R_d) or, past its end, masked (-1).
__device__ __forceinline__ int raw_code(const RowCtx& c, int idx) {
  return c.loc[min(idx, c.k - 1)];                  // always inside this query's list
}

__device__ __forceinline__ int final_code(const RowCtx& c, int idx, int raw) {
  int rrow = c.ring_row0 + (idx - c.k);             // consecutive positions, one wrap at most
  rrow -= rrow >= c.ring_end ? c.Rd : 0;
  const int rc = make_loc(kTierRing, rrow);
  return idx < c.k ? raw : (idx < c.n_total ? rc : -1);
}

// Address of the row a code names; a masked code (-1) yields the hot pool
// base, a mapped address, so the load can be issued unconditionally and its
// value cleared when it is written to LDS.
template <int ROW>
__device__ __forceinline__ uintptr_t code_addr(const RowCtx& c, int code) {
  constexpr size_t RB = size_t(ROW) * 2;
  const int cc = code < 0 ? 0 : code;
  const int tier = loc_tier(cc);
  const size_t ix = size_t(loc_index(cc));
  // pool offsets from the hot pool base, selected arithmetically (a select
  // chain would become an indexed table in scratch memory)
  const uintptr_t off = (tier == kTierStaged ? c.d_staging : uintptr_t(0)) +
                        (tier == kTierResident ? c.d_resident : uintptr_t(0)) +
                        (tier == kTierRing ? c.d_ring : uintptr_t(0));
  return c.hot + off + ix * RB;
}

__device__ __forceinline__ uint32_t lo16(uint32_t w) { return w & 0xffffu; }
__device__ __forceinline__ uint32_t hi16(uint32_t w) { return w >> 16; }
__device__ __forceinline__ uint32_t elem(const uint4& v, int e) {
  const uint32_t w = e < 2 ? v.x : (e < 4 ? v.y : (e < 6 ? v.z : v.w));
  return (e & 1) ? hi16(w) : lo16(w);
}

template <class C>
struct Prefetch {
  uint4 t1[C::T1PT][4];
  uint4 t2[C::T2PT];
  uint32_t live;     // bit per loaded chunk: the row is not masked
  int flag;
};

template <class C>
struct Codes {
  int t1[C::T1PT][4];
  int t2[C::T2PT];
  int flag;
};

template <class C>
__device__ __forceinline__ void tile_codes(Codes<C>& cd, const RowCtx& ctx, int t0, int tid) {
#pragma unroll
  for (int a = 0; a < C::T1PT; ++a) {
    const int task = min(tid + a * C::NT, C::T1 - 1);
    const int g4 = task % (TILE / 4);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) cd.t1[a][rr] = raw_code(ctx, t0 + g4 * 4 + rr);
  }
#pragma unroll
  for (int b = 0; b < C::T2PT; ++b) {
    const int task = min(tid + b * C::NT, C::T2 - 1);
    cd.t2[b] = raw_code(ctx, t0 + task / C::NKO);
  }
  cd.flag = raw_code(ctx, t0 + (tid % TILE));
}

// Issues the loads of one tile: every load is unconditional and its value is
// not consumed here, so the wave does not wait for it before the next tile's
// store (a conditional or masked load would make the compiler wait at once).
template <class C>
__device__ __forceinline__ void tile_load(Prefetch<C>& pf, const Codes<C>& cd, const RowCtx& ctx, int t0,
                                          int tid) {
  uint32_t live = 0;
#pragma unroll
  for (int a = 0; a < C::T1PT; ++a) {
    const int task = min(tid + a * C::NT, C::T1 - 1);
    const int g4 = task % (TILE / 4), cv = task / (TILE / 4);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int code = final_code(ctx, t0 + g4 * 4 + rr, cd.t1[a][rr]);
      pf.t1[a][rr] = gload16(code_addr<C::ROW>(ctx, code) + size_t(C::V0 + cv) * 16);
      live |= (code >= 0 ? 1u : 0u) << (a * 4 + rr);
    }
  }
#pragma unroll
  for (int b = 0; b < C::T2PT; ++b) {
    const int task = min(tid + b * C::NT, C::T2 - 1);
    const int code = final_code(ctx, t0 + task / C::NKO, cd.t2[b]);
    pf.t2[b] = gload16(code_addr<C::ROW>(ctx, code) + size_t(C::KO0 + task % C::NKO) * 16);
    live |= (code >= 0 ? 1u : 0u) << (C::T1PT * 4 + b);
  }
  pf.live = live;
  pf.flag = final_code(ctx, t0 + (tid % TILE), cd.flag) >= 0;
}

__device__ __forceinline__ uint4 masked(const uint4& v, bool ok) {
  return make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u);
}

template <class C>
__device__ __forceinline__ void tile_store(const Prefetch<C>& pf, uint16_t* Ks, uint16_t* Vt, int* rowflag, int tid) {
#pragma unroll
  for (int a = 0; a < C::T1PT; ++a) {
    const int task = tid + a * C::NT;
    if (C::T1 % C::NT == 0 || task < C::T1) {
      const int g4 = task % (TILE / 4), cv = task / (TILE / 4);
      uint4 v[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) v[rr] = masked(pf.t1[a][rr], (pf.live >> (a * 4 + rr)) & 1u);
      if (C::V_IN_K) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          *reinterpret_cast<uint4*>(Ks + (g4 * 4 + rr) * C::KSTR + (C::V0 + cv) * 8) = v[rr];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint2 pk;
        pk.x = elem(v[0], e) | (elem(v[1], e) << 16);
        pk.y = elem(v[2], e) | (elem(v[3], e) << 16);
        *reinterpret_cast<uint2*>(Vt + (cv * 8 + e) * C::VSTR + g4 * 4) = pk;
      }
    }
  }
#pragma unroll
  for (int b = 0; b < C::T2PT; ++b) {
    const int task = tid + b * C::NT;
    if (C::T2 % C::NT == 0 || task < C::T2) {
      const int rr = task / C::NKO, ck = task % C::NKO;
      *reinterpret_cast<uint4*>(Ks + rr * C::KSTR + (C::KO0 + ck) * 8) =
          masked(pf.t2[b], (pf.live >> (C::T1PT * 4 + b)) & 1u);
    }
  }
  // 32-bit mask of the tile's live rows, from the first wave's flags
  if (tid < 64) {
    const unsigned long long m = __builtin_amdgcn_ballot_w64(tid < TILE && pf.flag);
    if (tid == 0) rowflag[0] = static_cast<int>(static_cast<uint32_t>(m));
  }
}

template <class C>
__global__ __launch_bounds__(C::NT, 1) void attn_kernel(AttnArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  uint16_t* Ks = reinterpret_cast<uint16_t*>(lds);
  uint16_t* Vt = reinterpret_cast<uint16_t*>(lds + C::LDS_K);
  float* Sx = reinterpret_cast<float*>(lds + C::LDS_K + C::LDS_V);
  int* rowflag = reinterpret_cast<int*>(lds + C::LDS_K + C::LDS_V + C::LDS_S);

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
  const size_t blk = (size_t(qi) * a.head_groups + hg) * a.splits + sp;
  const int hi_half = lane >> 5;

  const int p_j = a.causal[qi];
  if (p_j < 0) {  // inactive query: zero output (the combine pass does it when split)
    if (a.splits == 1 && head < a.H) {
      uint16_t* op = a.out + (size_t(qi) * a.H + head) * C::D_V + dq * (C::D_V / C::NDP);
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
  ctx.ring_base = size_t(r) * a.Rd;
  ctx.ring_row0 = r * a.Rd + lo % a.Rd;
  ctx.ring_end = (r + 1) * a.Rd;
  ctx.hot = reinterpret_cast<uintptr_t>(a.hot);
  ctx.d_staging = reinterpret_cast<uintptr_t>(a.staging) - ctx.hot;
  ctx.d_resident = reinterpret_cast<uintptr_t>(a.resident) - ctx.hot;
  ctx.d_ring = reinterpret_cast<uintptr_t>(a.ring) - ctx.hot;

  const int n_tiles = (ctx.n_total + TILE - 1) / TILE;
  const int tb = int((long long)n_tiles * sp / a.splits);
  const int te = int((long long)n_tiles * (sp + 1) / a.splits);

  // Q fragment: B operand of S^T = K Q^T, head = lane%32, 8 dims per k-step
  bf16x8 qreg[C::KS];
  {
    const uint16_t* qp = a.q + (size_t(qi) * a.H + head) * C::D_QK + dq * (C::D_QK / C::NDP) + hi_half * 8;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
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

  Prefetch<C> pf;
  Codes<C> cd;
  tile_codes<C>(cd, ctx, tb * TILE, tid);
  tile_load<C>(pf, cd, ctx, tb * TILE, tid);
  tile_codes<C>(cd, ctx, (tb + 1) * TILE, tid);

  const uint16_t* ks_row = Ks + (lane & 31) * C::KSTR + dq * (C::D_QK / C::NDP) + hi_half * 8;
  // partial scores as float4: [wave][i/4][lane] (consecutive lanes, 16 B each)
  float4* sx_own = reinterpret_cast<float4*>(Sx) + size_t(w) * 4 * 64 + lane;
  const float4* sx_blk = reinterpret_cast<const float4*>(Sx) + size_t(hb * C::NDP) * 4 * 64 + lane;
  const int vdim0 = dq * (C::D_V / C::NDP) + (lane & 31);

  for (int t = tb; t < te; ++t) {
    __syncthreads();
    tile_store<C>(pf, Ks, Vt, rowflag, tid);
    __syncthreads();
    // unconditional (past the range they read masked or unused, always mapped rows):
    // a conditional prefetch would make the compiler wait for it at once
    tile_load<C>(pf, cd, ctx, (t + 1) * TILE, tid);                    // rows of tile t+1
    tile_codes<C>(cd, ctx, (t + 2) * TILE, tid);                       // codes of tile t+2

    // partial scores over this wave's part of the key width
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const bf16x8 kf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(ks_row + ks * 16));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qreg[ks], acc, 0, 0, 0);
    }
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4)
      sx_own[i4 * 64] = make_float4(acc[4 * i4], acc[4 * i4 + 1], acc[4 * i4 + 2], acc[4 * i4 + 3]);
    __syncthreads();
    float s[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
    // the block's partial scores summed in key-part order (identical in its waves)
#pragma unroll
    for (int q = 0; q < C::NDP; ++q) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const float4 v = sx_blk[(q * 4 + i4) * 64];   // own slice too: no divergent select
        if (q == 0) {
          s[4 * i4] = v.x; s[4 * i4 + 1] = v.y; s[4 * i4 + 2] = v.z; s[4 * i4 + 3] = v.w;
        } else {
          s[4 * i4] += v.x; s[4 * i4 + 1] += v.y; s[4 * i4 + 2] += v.z; s[4 * i4 + 3] += v.w;
        }
      }
    }
    const uint32_t live = static_cast<uint32_t>(rowflag[0]);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = (i >> 2) * 8 + hi_half * 4 + (i & 3);
      s[i] = (live >> row) & 1u ? s[i] * sl2 : -INFINITY;
    }
    // online softmax for head lane%32; the other 16 rows sit in lane ^ 32
    float mt = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mt = fmaxf(mt, s[i]);
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const bool grow = mt > m_run + kRescaleLog2;
    if (__builtin_amdgcn_ballot_w64(grow)) {   // wave-uniform: some head's max moved far
      const float m_new = grow ? mt : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
      m_run = m_new;
#pragma unroll
      for (int d = 0; d < C::DVB; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) O[d][i] *= alpha;
    }
    float ps = 0.f;
    bf16x8 pb0, pb1;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = __builtin_amdgcn_exp2f(s[i] - m_run);
      ps += p;
      if (i < 8) pb0[i] = static_cast<__bf16>(p);
      else pb1[i - 8] = static_cast<__bf16>(p);
    }
    l_run += ps;
    // O^T += V^T P^T over the tile's 32 rows (two 16-row k-steps)
#pragma unroll
    for (int d = 0; d < C::DVB; ++d) {
      const uint16_t* vrow = Vt + (vdim0 + d * 32) * C::VSTR + hi_half * 4;
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        const uint2 x0 = *reinterpret_cast<const uint2*>(vrow + ks2 * 16);
        const uint2 x1 = *reinterpret_cast<const uint2*>(vrow + ks2 * 16 + 8);
        const bf16x8 vf = __builtin_bit_cast(bf16x8, make_uint4(x0.x, x0.y, x1.x, x1.y));
        O[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, ks2 == 0 ? pb0 : pb1, O[d], 0, 0, 0);
      }
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (a.splits == 1) {
    if (head < a.H) {
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      uint16_t* op = a.out + (size_t(qi) * a.H + head) * C::D_V + dq * (C::D_V / C::NDP) + hi_half * 4;
#pragma unroll
      for (int d = 0; d < C::DVB; ++d)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          uint16_t h4[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            h4[e] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(O[d][g * 4 + e] * inv));
          uint2 pk;
          pk.x = uint32_t(h4[0]) | (uint32_t(h4[1]) << 16);
          pk.y = uint32_t(h4[2]) | (uint32_t(h4[3]) << 16);
          *reinterpret_cast<uint2*>(op + d * 32 + g * 8) = pk;
        }
    }
  } else {
    float* po = a.part_o + (blk * 32 * C::HB + hl) * C::D_V + dq * (C::D_V / C::NDP) + hi_half * 4;
#pragma unroll
    for (int d = 0; d < C::DVB; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(po + d * 32 + g * 8) =
            make_float4(O[d][g * 4 + 0], O[d][g * 4 + 1], O[d][g * 4 + 2], O[d][g * 4 + 3]);
    if (dq == 0 && hi_half == 0) {
      float* pm = a.part_ml + (blk * 32 * C::HB + hl) * 2;
      pm[0] = m_run;
      pm[1] = l_tot;
    }
  }
}

// Merge of key splits: out = sum_s 2^(m_s-m) O_s / sum_s 2^(m_s-m) l_s.
// One 128-thread block per (query, head); threads run over value dims.
template <int D_V, int HB>
__global__ __launch_bounds__(128) void combine_kernel(AttnArgs a) {
  constexpr int HPW = 32 * HB;
  const int per_q = a.head_groups * HPW;
  const int qi = a.r0 * a.Q + blockIdx.x / per_q;
  const int hx = blockIdx.x % per_q;
  const int hg = hx / HPW, hl = hx % HPW;
  const int head = hg * HPW + hl;
  if (head >= a.H) return;
  uint16_t* op = a.out + (size_t(qi) * a.H + head) * D_V;
  if (a.causal[qi] < 0) {
    for (int d = threadIdx.x; d < D_V; d += blockDim.x) op[d] = 0;
    return;
  }
  const size_t blk0 = (size_t(qi) * a.head_groups + hg) * a.splits;
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
  for (int d = threadIdx.x; d < D_V; d += blockDim.x) {
    float num = 0.f;
    for (int s = 0; s < a.splits; ++s) num += a.part_o[((blk0 + s) * HPW + hl) * D_V + d] * wsum[s];
    op[d] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(num * inv));
  }
}

template <class C>
hipError_t launch_cfg(const AttnArgs& a, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(attn_kernel<C>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(C::LDS));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int nreq = a.r1 - a.r0;
  if (nreq <= 0) return hipSuccess;
  const int per_req = a.Q * a.head_groups * a.splits;
  const long long blocks = (long long)((nreq + 7) / 8) * 8 * per_req;
  hipLaunchKernelGGL(attn_kernel<C>, dim3(unsigned(blocks)), dim3(C::NT), C::LDS, s, a);
  return hipGetLastError();
}

}  // namespace

bool attn_layout_supported(int row_elems, int d_qk, int v_off, int d_v) {
  return (row_elems == 576 && d_qk == 576 && v_off == 0 && d_v == 512) ||
         (row_elems == 256 && d_qk == 128 && v_off == 128 && d_v == 128);
}

int attn_heads_per_wg(int H) { return H <= 32 ? 32 : 64; }

hipError_t launch_attn(const AttnArgs& a, int row_elems, int d_qk, int v_off, int d_v, hipStream_t s) {
  const int hpw = attn_heads_per_wg(a.H);
  if (row_elems == 576 && d_qk == 576 && v_off == 0 && d_v == 512) {
    if (hpw == 32) return launch_cfg<Cfg<576, 0, 512, 576, 1>>(a, s);
    return launch_cfg<Cfg<576, 0, 512, 576, 2>>(a, s);
  }
  if (row_elems == 256 && d_qk == 128 && v_off == 128 && d_v == 128) {
    if (hpw == 32) return launch_cfg<Cfg<128, 128, 128, 256, 1>>(a, s);
    return launch_cfg<Cfg<128, 128, 128, 256, 2>>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attn_combine(const AttnArgs& a, int d_v, hipStream_t s) {
  const int nreq = a.r1 - a.r0;
  if (nreq <= 0 || a.splits <= 1) return hipSuccess;
  const int hpw = attn_heads_per_wg(a.H);
  const dim3 grid(unsigned(nreq * a.Q * a.head_groups * hpw));
  if (d_v == 512) {
    if (hpw == 32) hipLaunchKernelGGL((combine_kernel<512, 1>), grid, dim3(128), 0, s, a);
    else hipLaunchKernelGGL((combine_kernel<512, 2>), grid, dim3(128), 0, s, a);
  } else if (d_v == 128) {
    if (hpw == 32) hipLaunchKernelGGL((combine_kernel<128, 1>), grid, dim3(128), 0, s, a);
    else hipLaunchKernelGGL((combine_kernel<128, 2>), grid, dim3(128), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvh
