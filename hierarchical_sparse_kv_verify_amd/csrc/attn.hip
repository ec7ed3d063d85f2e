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

constexpr int TILE = 32;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;

template <int D_QK_, int V_OFF_, int D_V_, int ROW_, int HB_>
struct Cfg {
  static constexpr int D_QK = D_QK_, V_OFF = V_OFF_, D_V = D_V_, ROW = ROW_, HB = HB_;
  static constexpr int NW = 2 * HB;
  static constexpr int NT = NW * 64;
  static constexpr int KS = D_QK / 2 / 16;   // 16-wide k-steps over half the key width
  static constexpr int DVB = D_V / 2 / 32;   // 32-wide value blocks over half the value width
  static constexpr int KCH = D_QK / 8;       // 16-byte chunks of the key
  static constexpr int V0 = V_OFF / 8, VCH = D_V / 8;
  static constexpr bool V_IN_K = (V_OFF == 0 && D_V <= D_QK);
  static constexpr int KO0 = V_IN_K ? VCH : 0;          // first key-only chunk
  static constexpr int NKO = V_IN_K ? (KCH - VCH) : KCH;
  static constexpr int KSTR = D_QK + 8;      // key tile row stride (elements): 16 B mod 128 B
  static constexpr int VSTR = TILE + 4;      // transposed value stride (elements)
  static constexpr int T1 = (TILE / 4) * VCH;   // (4-row group, value chunk) load tasks
  static constexpr int T2 = TILE * NKO;         // (row, key-only chunk) load tasks
  static constexpr int T1PT = (T1 + NT - 1) / NT;
  static constexpr int T2PT = (T2 + NT - 1) / NT;
  static constexpr size_t LDS_K = size_t(TILE) * KSTR * 2;
  static constexpr size_t LDS_V = size_t(D_V) * VSTR * 2;
  static constexpr size_t LDS_S = size_t(NW) * 16 * 64 * 4;
  static constexpr size_t LDS = LDS_K + LDS_V + LDS_S + TILE * 4;
  static_assert(D_QK % 32 == 0 && D_V % 64 == 0 && ROW % 8 == 0, "shape");
  static_assert(V_IN_K || V_OFF >= D_QK, "value range must lie inside or after the key range");
  static_assert(LDS <= 160 * 1024, "LDS");
};

struct RowCtx {
  const int32_t* loc;
  int k, n_total, lo, Rd, row;
  size_t ring_base;
  const uint16_t *hot, *staging, *resident, *ring;
};

__device__ inline const uint4* row_src(const RowCtx& c, int idx) {
  if (idx < c.k) {
    const int code = c.loc[idx];
    if (code < 0) return nullptr;
    const int tier = loc_tier(code);
    const size_t ix = size_t(loc_index(code));
    const uint16_t* base = tier == kTierHot ? c.hot : (tier == kTierStaged ? c.staging : c.resident);
    return reinterpret_cast<const uint4*>(base + ix * c.row);
  }
  if (idx < c.n_total) {
    const int pos = c.lo + (idx - c.k);
    return reinterpret_cast<const uint4*>(c.ring + (c.ring_base + size_t(pos % c.Rd)) * c.row);
  }
  return nullptr;
}

__device__ inline uint32_t lo16(uint32_t w) { return w & 0xffffu; }
__device__ inline uint32_t hi16(uint32_t w) { return w >> 16; }
__device__ inline uint32_t elem(const uint4& v, int e) {
  const uint32_t w = e < 2 ? v.x : (e < 4 ? v.y : (e < 6 ? v.z : v.w));
  return (e & 1) ? hi16(w) : lo16(w);
}

template <class C>
struct Prefetch {
  uint4 t1[C::T1PT][4];
  uint4 t2[C::T2PT];
  int flag;
};

template <class C>
__device__ inline void tile_load(Prefetch<C>& pf, const RowCtx& ctx, int t0, int tid) {
  const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int a = 0; a < C::T1PT; ++a) {
    const int task = tid + a * C::NT;
    if (task < C::T1) {
      const int g4 = task / C::VCH, cv = task % C::VCH;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const uint4* p = row_src(ctx, t0 + g4 * 4 + rr);
        pf.t1[a][rr] = p ? p[C::V0 + cv] : z;
      }
    }
  }
#pragma unroll
  for (int b = 0; b < C::T2PT; ++b) {
    const int task = tid + b * C::NT;
    if (task < C::T2) {
      const int rr = task / C::NKO, ck = task % C::NKO;
      const uint4* p = row_src(ctx, t0 + rr);
      pf.t2[b] = p ? p[C::KO0 + ck] : z;
    }
  }
  if (tid < TILE) pf.flag = row_src(ctx, t0 + tid) != nullptr;
}

template <class C>
__device__ inline void tile_store(const Prefetch<C>& pf, uint16_t* Ks, uint16_t* Vt, int* rowflag, int tid) {
#pragma unroll
  for (int a = 0; a < C::T1PT; ++a) {
    const int task = tid + a * C::NT;
    if (task < C::T1) {
      const int g4 = task / C::VCH, cv = task % C::VCH;
      if (C::V_IN_K) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          *reinterpret_cast<uint4*>(Ks + (g4 * 4 + rr) * C::KSTR + (C::V0 + cv) * 8) = pf.t1[a][rr];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint2 pk;
        pk.x = elem(pf.t1[a][0], e) | (elem(pf.t1[a][1], e) << 16);
        pk.y = elem(pf.t1[a][2], e) | (elem(pf.t1[a][3], e) << 16);
        *reinterpret_cast<uint2*>(Vt + (cv * 8 + e) * C::VSTR + g4 * 4) = pk;
      }
    }
  }
#pragma unroll
  for (int b = 0; b < C::T2PT; ++b) {
    const int task = tid + b * C::NT;
    if (task < C::T2) {
      const int rr = task / C::NKO, ck = task % C::NKO;
      *reinterpret_cast<uint4*>(Ks + rr * C::KSTR + (C::KO0 + ck) * 8) = pf.t2[b];
    }
  }
  if (tid < TILE) rowflag[tid] = pf.flag;
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

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hb = w >> 1, dh = w & 1;
  const int hl = hb * 32 + (lane & 31);               // head within the workgroup
  const int head = hg * 32 * C::HB + hl;
  const size_t blk = (size_t(qi) * a.head_groups + hg) * a.splits + sp;
  const int hi_half = lane >> 5;

  const int p_j = a.causal[qi];
  if (p_j < 0) {  // inactive query: zero output (the combine pass does it when split)
    if (a.splits == 1 && head < a.H) {
      uint16_t* op = a.out + (size_t(qi) * a.H + head) * C::D_V + dh * (C::D_V / 2);
      for (int d = hi_half; d < C::D_V / 2 / 4; d += 2)
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
  ctx.loc = a.loc + size_t(qi) * a.k;
  ctx.k = a.k;
  ctx.n_total = a.k + n_ring;
  ctx.lo = lo;
  ctx.Rd = a.Rd;
  ctx.row = C::ROW;
  ctx.ring_base = size_t(r) * a.Rd;
  ctx.hot = a.hot;
  ctx.staging = a.staging;
  ctx.resident = a.resident;
  ctx.ring = a.ring;

  const int n_tiles = (ctx.n_total + TILE - 1) / TILE;
  const int tb = int((long long)n_tiles * sp / a.splits);
  const int te = int((long long)n_tiles * (sp + 1) / a.splits);

  // Q fragment: B operand of S^T = K Q^T, head = lane%32, 8 dims per k-step
  bf16x8 qreg[C::KS];
  {
    const uint16_t* qp = a.q + (size_t(qi) * a.H + head) * C::D_QK + dh * (C::D_QK / 2) + hi_half * 8;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (head < a.H) v = *reinterpret_cast<const uint4*>(qp + ks * 16);
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
  if (tb < te) tile_load<C>(pf, ctx, tb * TILE, tid);

  const uint16_t* ks_row = Ks + (lane & 31) * C::KSTR + dh * (C::D_QK / 2) + hi_half * 8;
  float* sx_own = Sx + size_t(w) * 16 * 64 + lane;
  const float* sx_pair = Sx + size_t(w ^ 1) * 16 * 64 + lane;
  const int vdim0 = dh * (C::D_V / 2) + (lane & 31);

  for (int t = tb; t < te; ++t) {
    __syncthreads();
    tile_store<C>(pf, Ks, Vt, rowflag, tid);
    __syncthreads();
    if (t + 1 < te) tile_load<C>(pf, ctx, (t + 1) * TILE, tid);

    // partial scores over this wave's half of the key width
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const bf16x8 kf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(ks_row + ks * 16));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qreg[ks], acc, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sx_own[i * 64] = acc[i];
    __syncthreads();
    float s[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float o = sx_pair[i * 64];
      const float full = dh == 0 ? acc[i] + o : o + acc[i];   // same order in both waves
      const int row = (i >> 2) * 8 + hi_half * 4 + (i & 3);
      s[i] = rowflag[row] ? full * sl2 : -INFINITY;
    }
    // online softmax for head lane%32; the other 16 rows sit in lane ^ 32
    float mt = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mt = fmaxf(mt, s[i]);
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m_run, mt);
    const float alpha = exp2f(m_run - m_new);
    float ps = 0.f;
    bf16x8 pb0, pb1;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = exp2f(s[i] - m_new);
      ps += p;
      if (i < 8) pb0[i] = static_cast<__bf16>(p);
      else pb1[i - 8] = static_cast<__bf16>(p);
    }
    l_run = l_run * alpha + ps;
    m_run = m_new;
#pragma unroll
    for (int d = 0; d < C::DVB; ++d)
#pragma unroll
      for (int i = 0; i < 16; ++i) O[d][i] *= alpha;
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
      uint16_t* op = a.out + (size_t(qi) * a.H + head) * C::D_V + dh * (C::D_V / 2) + hi_half * 4;
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
    float* po = a.part_o + (blk * 32 * C::HB + hl) * C::D_V + dh * (C::D_V / 2) + hi_half * 4;
#pragma unroll
    for (int d = 0; d < C::DVB; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(po + d * 32 + g * 8) =
            make_float4(O[d][g * 4 + 0], O[d][g * 4 + 1], O[d][g * 4 + 2], O[d][g * 4 + 3]);
    if (dh == 0 && hi_half == 0) {
      float* pm = a.part_ml + (blk * 32 * C::HB + hl) * 2;
      pm[0] = m_run;
      pm[1] = l_tot;
    }
  }
}

// Merge of key splits: out = sum_s 2^(m_s-m) O_s / sum_s 2^(m_s-m) l_s.
template <int D_V, int HB>
__global__ __launch_bounds__(256) void combine_kernel(AttnArgs a) {
  const int qi_local = blockIdx.x / a.head_groups;
  const int hg = blockIdx.x % a.head_groups;
  const int qi = a.r0 * a.Q + qi_local;
  const bool active = a.causal[qi] >= 0;
  for (int hl = 0; hl < 32 * HB; ++hl) {
    const int head = hg * 32 * HB + hl;
    if (head >= a.H) break;
    uint16_t* op = a.out + (size_t(qi) * a.H + head) * D_V;
    if (!active) {
      for (int d = threadIdx.x; d < D_V; d += blockDim.x) op[d] = 0;
      continue;
    }
    const size_t blk0 = (size_t(qi) * a.head_groups + hg) * a.splits;
    float m = kNegBig;
    for (int s = 0; s < a.splits; ++s) m = fmaxf(m, a.part_ml[((blk0 + s) * 32 * HB + hl) * 2]);
    float den = 0.f;
    for (int s = 0; s < a.splits; ++s) {
      const float* pm = a.part_ml + ((blk0 + s) * 32 * HB + hl) * 2;
      den += pm[1] * exp2f(pm[0] - m);
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    for (int d = threadIdx.x; d < D_V; d += blockDim.x) {
      float num = 0.f;
      for (int s = 0; s < a.splits; ++s) {
        const float* pm = a.part_ml + ((blk0 + s) * 32 * HB + hl) * 2;
        num += a.part_o[((blk0 + s) * 32 * HB + hl) * D_V + d] * exp2f(pm[0] - m);
      }
      op[d] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(num * inv));
    }
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
  const dim3 grid(unsigned(nreq * a.Q * a.head_groups));
  const int hpw = attn_heads_per_wg(a.H);
  if (d_v == 512) {
    if (hpw == 32) hipLaunchKernelGGL((combine_kernel<512, 1>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((combine_kernel<512, 2>), grid, dim3(256), 0, s, a);
  } else if (d_v == 128) {
    if (hpw == 32) hipLaunchKernelGGL((combine_kernel<128, 1>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((combine_kernel<128, 2>), grid, dim3(256), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvh
