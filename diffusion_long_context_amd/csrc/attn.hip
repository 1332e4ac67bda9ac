// Bidirectional attention of the decode block's queries over a gathered set of KV tokens.
//
// Focus-dLLM (abstract; Elamur "Summary"): the sparse step runs ordinary bidirectional attention for
// the current block's queries over only the selected KV (plus the block itself); shallow layers and
// the vanilla baseline run it over everything.  Prefilling-dLLM (abstract): the same over chunk KV
// that sits non-contiguously in a paged cache.
//
// bf16 path (the hot one): one workgroup of 4 waves per (split, KV head, sequence) handles all G
// q-heads of the KV head over a contiguous share of the gathered 64-token tiles (tile 0 is the
// block's own tokens).  Tiles are read from HBM with coalesced 16-byte loads into registers one
// round ahead, staged in LDS, and consumed by bf16 MFMA (32x32x16, f32 accumulate):
//   S^T = K Q^T   (A = K rows from LDS, B = Q fragments held in registers),
//   O^T = V^T P^T (A = V columns from LDS, B = the probabilities straight from the S^T registers),
// which keeps every softmax statistic in the lane that owns its query, so the online softmax needs
// one cross-lane exchange per tile.  Within a workgroup, waves that share a head merge through LDS;
// across workgroups the partial (max, sum, O) go to scratch and are
// merged by attn_combine_kernel.
//
// float32 path: a plain per-query-row kernel for the small float32 workload.
#include "fdl_device.h"
#include "fdl_internal.h"

namespace fdl {

struct AttnParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* k_dec;
  const uint16_t* v_dec;
  const int32_t* sel_idx;
  const int32_t* n_sel;
  uint16_t* out;
  float* part_o;     // [B][Hq][S][32][D]
  float2* part_ml;   // [B][Hq][S][32]  (max in log2 units, sum)
  uint32_t* tickets;
  uint32_t* status;
  const int32_t* page_table;
  int Hq, Hkv, T, L, max_sel, unit_log2, n_units, n_splits;
  int page_log2, pages_per_seq, n_pages;
  float scale_log2;  // log2(e) / sqrt(D)
};

template <int G>
struct AttnShape {
  static constexpr int TPR = G == 1 ? 4 : (G == 2 ? 2 : 1);   // tiles per round
  static constexpr int NW = G > 4 ? 8 : 4;                      // waves per workgroup
};

// Element offset of row r of tile e (0 = the block's own tokens, relative to k_dec / v_dec; >= 1:
// list tiles, relative to the cache) and whether the row holds a token.  Branch-free, so that the
// caller can issue every load of a round back to back.
template <int D, bool DENSE, bool PAGED>
__device__ __forceinline__ int64_t attn_row_off(const AttnParams& p, const KvRows<PAGED>& rows, int b,
                                                int g, int e, bool tile_live, int r, int n_list,
                                                const int32_t* __restrict__ sel_row, bool& ok,
                                                bool& bad) {
  if (e == 0) {   // uniform
    ok = tile_live && r < p.T;
    return ((int64_t)(b * p.Hkv + g) * p.T + (r < p.T ? r : p.T - 1)) * D;
  }
  if (!tile_live || p.L == 0) {   // uniform; the caller then reads from k_dec / v_dec
    ok = false;
    return 0;
  }
  const int i = (e - 1) * 64 + r;
  ok = i < n_list;
  const int ii = ok ? i : 0;
  int t = ii;
  if constexpr (!DENSE) {
    const int u = sel_row[ii >> p.unit_log2];
    const bool uok = (unsigned)u < (unsigned)p.n_units;
    bad = bad || (ok && !uok);
    ok = ok && uok;
    t = uok ? (u << p.unit_log2) + (ii & ((1 << p.unit_log2) - 1)) : 0;
  }
  ok = ok && t < p.L;
  t = (t < p.L) ? t : 0;
  bool pbad = false;
  const int64_t off = rows.off(b, g, t, pbad);
  bad = bad || (ok && pbad);
  ok = ok && !pbad;
  return off;
}

template <int D, int G, bool DENSE, bool PAGED>
__global__ __launch_bounds__(AttnShape<G>::NW * 64, 1) void attn_mfma_kernel(const AttnParams p) {
  constexpr int TPR = AttnShape<G>::TPR;
  constexpr int NW = AttnShape<G>::NW;
  constexpr int NT = NW * 64;
  constexpr int HPW = 1;                                // heads per wave
  constexpr int RS = D + 8;                             // LDS row stride (elements)
  constexpr int TILE = 64 * RS;
  constexpr int KS = D / 16;
  constexpr int DT = D / 32;
  constexpr int PROW = D / 8;                           // 16-byte pieces per row
  constexpr int RPP = NT / PROW;                        // rows covered by one pass of the block
  constexpr int RPT = 64 / RPP;                         // rows per thread per tile
  static_assert(NT % PROW == 0 && 64 % RPP == 0, "tile rows must split evenly over the block");
  __shared__ __attribute__((aligned(16))) uint16_t lds[TPR * 2 * TILE];
  __shared__ uint8_t s_valid[TPR][64];
  __shared__ float2 s_ml[4][32];

  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ql = lane & 31, hh = lane >> 5;
  const int Hkv = p.Hkv;
  const int64_t seg = (int64_t)b * Hkv + g;
  const int S = p.n_splits;
  KvRows<PAGED> rows;
  rows.Hkv = Hkv;
  rows.L = p.L;
  rows.D = D;
  rows.page_log2 = p.page_log2;
  rows.pages_per_seq = p.pages_per_seq;
  rows.n_pages = p.n_pages;
  rows.page_table = p.page_table;
  bool bad = false;

  int n_list;
  if (DENSE) {
    n_list = p.L;
  } else {
    int ns = p.n_sel[seg];
    ns = ns < 0 ? 0 : (ns > p.max_sel ? p.max_sel : ns);
    n_list = ns << p.unit_log2;
  }
  if (p.L == 0) n_list = 0;
  const int n_tiles = 1 + (n_list + 63) / 64;
  const int e0 = (int)((int64_t)n_tiles * s / S);
  const int e1 = (int)((int64_t)n_tiles * (s + 1) / S);
  const int32_t* sel_row = DENSE ? nullptr : p.sel_idx + seg * p.max_sel;
  const int chunk = tid % PROW;
  const int rbase = tid / PROW;

  const int slot = (TPR > 1) ? wave / G : 0;
  int heads[HPW];
#pragma unroll
  for (int hi = 0; hi < HPW; ++hi) heads[hi] = (TPR > 1) ? wave % G : wave + NW * hi;

  // Q fragments (B operand of S^T = K Q^T): lane (q, hh) holds q[q][hh*D/2 + 8ks .. +8]
  bf16x8 qf[HPW][KS];
#pragma unroll
  for (int hi = 0; hi < HPW; ++hi) {
    const int h = g * G + heads[hi];
    const bool live = heads[hi] < G && ql < p.T;
    const uint16_t* qrow = p.q + (((int64_t)b * p.Hq + h) * p.T + ql) * D + hh * (D / 2);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (live) v = *reinterpret_cast<const uint4*>(qrow + ks * 8);
      qf[hi][ks] = as_bf16x8(v);
    }
  }

  f32x16 oacc[HPW][DT];
  float m_run[HPW], l_run[HPW];
#pragma unroll
  for (int hi = 0; hi < HPW; ++hi) {
    m_run[hi] = -__builtin_inff();
    l_run[hi] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[hi][dt][r] = 0.f;
  }

  const int rounds = (e1 - e0 + TPR - 1) / TPR;
  uint4 stk[TPR][RPT], stv[TPR][RPT];
  uint32_t okbits = 0;   // bit sl*RPT+m: row (sl, m) of the staged round holds a token

  auto load_round = [&](int rnd) {
    int64_t off[TPR][RPT];
    okbits = 0;
#pragma unroll
    for (int sl = 0; sl < TPR; ++sl) {
      const int e = e0 + rnd * TPR + sl;
      const bool live = e < e1;
#pragma unroll
      for (int m = 0; m < RPT; ++m) {
        bool ok;
        off[sl][m] = attn_row_off<D, DENSE, PAGED>(p, rows, b, g, e, live, rbase + RPP * m, n_list,
                                                   sel_row, ok, bad);
        okbits |= (ok ? 1u : 0u) << (sl * RPT + m);
      }
    }
#pragma unroll
    for (int sl = 0; sl < TPR; ++sl) {
      const int e = e0 + rnd * TPR + sl;
      // the own block, dead slots and an empty cache all read from the (always valid) k_dec / v_dec
      const bool use_dec = (e == 0) || (e >= e1) || (p.L == 0);
      const uint16_t* kb = use_dec ? p.k_dec : p.k;
      const uint16_t* vb = use_dec ? p.v_dec : p.v;
#pragma unroll
      for (int m = 0; m < RPT; ++m) {
        stk[sl][m] = *reinterpret_cast<const uint4*>(kb + off[sl][m] + chunk * 8);
        stv[sl][m] = *reinterpret_cast<const uint4*>(vb + off[sl][m] + chunk * 8);
      }
    }
  };
  auto store_round = [&]() {
    const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int sl = 0; sl < TPR; ++sl)
#pragma unroll
      for (int m = 0; m < RPT; ++m) {
        const bool ok = (okbits >> (sl * RPT + m)) & 1u;
        const int row = rbase + RPP * m;
        *reinterpret_cast<uint4*>(lds + (sl * 2) * TILE + row * RS + chunk * 8) = ok ? stk[sl][m] : zero;
        *reinterpret_cast<uint4*>(lds + (sl * 2 + 1) * TILE + row * RS + chunk * 8) = ok ? stv[sl][m] : zero;
        if (chunk == 0) s_valid[sl][row] = ok ? 1 : 0;
      }
  };

  if (rounds > 0) load_round(0);
  for (int rnd = 0; rnd < rounds; ++rnd) {
    store_round();
    __syncthreads();
    if (rnd + 1 < rounds) load_round(rnd + 1);
    const int e = e0 + rnd * TPR + slot;
    if (e < e1) {
      const uint64_t vm = __ballot(s_valid[slot][lane] != 0);
      const uint16_t* Kt = lds + (slot * 2) * TILE;
      const uint16_t* Vt = Kt + TILE;
#pragma unroll
      for (int hi = 0; hi < HPW; ++hi) {
        if (heads[hi] >= G) continue;
        f32x16 sacc[2];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[st][r] = 0.f;
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const uint4 a = *reinterpret_cast<const uint4*>(Kt + (st * 32 + ql) * RS + hh * (D / 2) + ks * 8);
            sacc[st] = mfma32(as_bf16x8(a), qf[hi][ks], sacc[st]);
          }
        }
        // S^T register r of sub-tile st is token st*32 + 8*(r/4) + 4*hh + r%4 for query ql
        float mx = -__builtin_inff();
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = st * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
            float x = sacc[st][r] * p.scale_log2;
            if (!((vm >> row) & 1ull)) x = -__builtin_inff();
            sacc[st][r] = x;
            mx = fmaxf(mx, x);
          }
        mx = fmaxf(mx, wave_shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run[hi], mx);
        if (m_new == -__builtin_inff()) continue;   // nothing valid seen yet
        const float alpha = exp2f(m_run[hi] - m_new);
        float rs = 0.f;
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float pr = exp2f(sacc[st][r] - m_new);
            sacc[st][r] = pr;
            rs += pr;
          }
        rs += wave_shfl_xor(rs, 32);
        l_run[hi] = l_run[hi] * alpha + rs;
        m_run[hi] = m_new;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[hi][dt][r] *= alpha;
        // O^T += V^T P^T over 4 k-steps of 16 tokens
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int kl = 0; kl < 2; ++kl) {
            uint4 pb;
            pb.x = pack_bf16x2(sacc[st][8 * kl + 0], sacc[st][8 * kl + 1]);
            pb.y = pack_bf16x2(sacc[st][8 * kl + 2], sacc[st][8 * kl + 3]);
            pb.z = pack_bf16x2(sacc[st][8 * kl + 4], sacc[st][8 * kl + 5]);
            pb.w = pack_bf16x2(sacc[st][8 * kl + 6], sacc[st][8 * kl + 7]);
            const bf16x8 bfr = as_bf16x8(pb);
            const int r0 = st * 32 + 16 * kl + 4 * hh;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
              const uint16_t* col = Vt + dt * 32 + ql;
              uint4 av;
              av.x = (uint32_t)col[(r0 + 0) * RS] | ((uint32_t)col[(r0 + 1) * RS] << 16);
              av.y = (uint32_t)col[(r0 + 2) * RS] | ((uint32_t)col[(r0 + 3) * RS] << 16);
              av.z = (uint32_t)col[(r0 + 8) * RS] | ((uint32_t)col[(r0 + 9) * RS] << 16);
              av.w = (uint32_t)col[(r0 + 10) * RS] | ((uint32_t)col[(r0 + 11) * RS] << 16);
              oacc[hi][dt] = mfma32(as_bf16x8(av), bfr, oacc[hi][dt]);
            }
          }
      }
    }
    __syncthreads();
  }

  latch_bad(p.status, bad);

  // ---- this workgroup's result per head: (m, l, O) ------------------------------------------
  float* po_base = p.part_o;
  float2* pml_base = p.part_ml;
  if constexpr (TPR == 1) {
    // one wave owns each head: write straight from registers
#pragma unroll
    for (int hi = 0; hi < HPW; ++hi) {
      if (heads[hi] >= G) continue;
      const int h = g * G + heads[hi];
      const int64_t hb = (int64_t)b * p.Hq + h;
      if (S == 1) {
        if (ql < p.T) {
          const float inv = 1.f / l_run[hi];
          uint16_t* orow = p.out + (hb * p.T + ql) * D;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
              const int d0 = dt * 32 + 8 * rg + 4 * hh;
              uint2 w;
              w.x = pack_bf16x2(oacc[hi][dt][4 * rg] * inv, oacc[hi][dt][4 * rg + 1] * inv);
              w.y = pack_bf16x2(oacc[hi][dt][4 * rg + 2] * inv, oacc[hi][dt][4 * rg + 3] * inv);
              *reinterpret_cast<uint2*>(orow + d0) = w;
            }
        }
      } else {
        float* po = po_base + ((hb * S + s) * 32 + ql) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int rg = 0; rg < 4; ++rg) {
            const int d0 = dt * 32 + 8 * rg + 4 * hh;
            *reinterpret_cast<float4*>(po + d0) =
                make_float4(oacc[hi][dt][4 * rg], oacc[hi][dt][4 * rg + 1], oacc[hi][dt][4 * rg + 2],
                            oacc[hi][dt][4 * rg + 3]);
          }
        if (hh == 0) pml_base[(hb * S + s) * 32 + ql] = make_float2(m_run[hi], l_run[hi]);
      }
    }
  } else {
    // waves sharing a head merge through LDS (tiles are no longer needed)
    constexpr int OS = D + 4;
    float* mo = reinterpret_cast<float*>(lds);
    const int id = heads[0] * TPR + slot;   // unique per wave
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int d = dt * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
        mo[(id * 32 + ql) * OS + d] = oacc[0][dt][r];
      }
    if (hh == 0) s_ml[id][ql] = make_float2(m_run[0], l_run[0]);
    __syncthreads();
    // thread -> (head j, query q, 4 dims)
    constexpr int ITEMS = G * 32 * (D / 4);
    for (int it = tid; it < ITEMS; it += NT) {
      const int j = it / (32 * (D / 4));
      const int q = (it / (D / 4)) % 32;
      const int d0 = (it % (D / 4)) * 4;
      float M = -__builtin_inff();
#pragma unroll
      for (int t = 0; t < TPR; ++t) M = fmaxf(M, s_ml[j * TPR + t][q].x);
      float Ls = 0.f;
      float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
      if (M != -__builtin_inff()) {
#pragma unroll
        for (int t = 0; t < TPR; ++t) {
          const float2 ml = s_ml[j * TPR + t][q];
          if (ml.y == 0.f) continue;
          const float w = exp2f(ml.x - M);
          Ls += ml.y * w;
          const float* src = mo + ((j * TPR + t) * 32 + q) * OS + d0;
          O.x += src[0] * w;
          O.y += src[1] * w;
          O.z += src[2] * w;
          O.w += src[3] * w;
        }
      }
      const int h = g * G + j;
      const int64_t hb = (int64_t)b * p.Hq + h;
      if (S == 1) {
        if (q < p.T) {
          const float inv = 1.f / Ls;
          uint2 w;
          w.x = pack_bf16x2(O.x * inv, O.y * inv);
          w.y = pack_bf16x2(O.z * inv, O.w * inv);
          *reinterpret_cast<uint2*>(p.out + (hb * p.T + q) * D + d0) = w;
        }
      } else {
        *reinterpret_cast<float4*>(po_base + ((hb * S + s) * 32 + q) * D + d0) = O;
        if (d0 == 0) pml_base[(hb * S + s) * 32 + q] = make_float2(M, Ls);
      }
    }
  }
}

// ------------------------------------------------------------------------------------------------
// float32 path: one thread per query row, 32-token chunks staged in LDS (small workloads only).
// ------------------------------------------------------------------------------------------------

struct F32Params {
  const float* q;
  const float* k;
  const float* v;
  const float* k_dec;
  const float* v_dec;
  const int32_t* sel_idx;
  const int32_t* n_sel;
  float* out;
  uint32_t* status;
  const int32_t* page_table;
  int Hq, Hkv, G, T, L, max_sel, unit_log2, n_units, dense;
  int page_log2, pages_per_seq, n_pages;
  float scale;
};

// Row i of the extended list (i < T: own block row i; else list position i - T): element offset
// into k_dec / v_dec (own) or the cache, and whether it holds a token.
template <int D, bool PAGED>
__device__ __forceinline__ int64_t f32_row_off(const F32Params& p, const KvRows<PAGED>& rows, int b,
                                               int g, int i, int n_list, const int32_t* sel_row,
                                               bool& own, bool& ok, bool& bad) {
  own = i < p.T;
  if (own) {
    ok = true;
    return ((int64_t)(b * p.Hkv + g) * p.T + i) * D;
  }
  const int li = i - p.T;
  ok = li < n_list;
  const int ii = ok ? li : 0;
  int t = ii;
  if (!p.dense) {
    const int u = sel_row[ii >> p.unit_log2];
    const bool uok = (unsigned)u < (unsigned)p.n_units;
    bad = bad || (ok && !uok);
    ok = ok && uok;
    t = uok ? (u << p.unit_log2) + (ii & ((1 << p.unit_log2) - 1)) : 0;
  }
  ok = ok && t < p.L;
  t = t < p.L ? t : 0;
  bool pbad = false;
  const int64_t off = rows.off(b, g, t, pbad);
  bad = bad || (ok && pbad);
  ok = ok && !pbad;
  return off;
}

template <int D, bool PAGED>
__global__ __launch_bounds__(64) void attn_f32_kernel(const F32Params p) {
  __shared__ float kc[32][D + 1];
  __shared__ float vc[32][D + 1];
  __shared__ int valid[32];
  const int h = blockIdx.x, b = blockIdx.y;
  const int g = h / p.G;
  const int qi = threadIdx.x;
  const int64_t seg = (int64_t)b * p.Hkv + g;
  KvRows<PAGED> rows;
  rows.Hkv = p.Hkv;
  rows.L = p.L;
  rows.D = D;
  rows.page_log2 = p.page_log2;
  rows.pages_per_seq = p.pages_per_seq;
  rows.n_pages = p.n_pages;
  rows.page_table = p.page_table;
  bool bad = false;
  int n_list;
  if (p.dense) {
    n_list = p.L;
  } else {
    int ns = p.n_sel[seg];
    ns = ns < 0 ? 0 : (ns > p.max_sel ? p.max_sel : ns);
    n_list = ns << p.unit_log2;
  }
  if (p.L == 0) n_list = 0;
  const int32_t* sel_row = p.sel_idx + seg * p.max_sel;
  const int total = p.T + n_list;
  float qr[D], o[D];
  const bool live = qi < p.T;
  const float* qrow = p.q + (((int64_t)b * p.Hq + h) * p.T + (live ? qi : 0)) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qr[d] = qrow[d];
    o[d] = 0.f;
  }
  float m = -__builtin_inff(), l = 0.f;
  for (int c0 = 0; c0 < total; c0 += 32) {
    __syncthreads();
    if (threadIdx.x < 32) {
      const int r = threadIdx.x;
      bool own = false, ok = false;
      const int i = c0 + r < total ? c0 + r : total - 1;
      const int64_t off = f32_row_off<D, PAGED>(p, rows, b, g, i, n_list, sel_row, own, ok, bad);
      ok = ok && (c0 + r < total);
      const float* ks = (own ? p.k_dec : p.k) + off;
      const float* vs = (own ? p.v_dec : p.v) + off;
      for (int d = 0; d < D; ++d) {
        const float kv = ks[d], vv = vs[d];
        kc[r][d] = ok ? kv : 0.f;
        vc[r][d] = ok ? vv : 0.f;
      }
      valid[r] = ok;
    }
    __syncthreads();
    float sc[32];
    float mx = -__builtin_inff();
    for (int r = 0; r < 32; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) acc += qr[d] * kc[r][d];
      sc[r] = valid[r] ? acc * p.scale : -__builtin_inff();
      mx = fmaxf(mx, sc[r]);
    }
    const float m_new = fmaxf(m, mx);
    if (m_new == -__builtin_inff()) continue;
    const float alpha = __expf(m - m_new);
    l *= alpha;
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] *= alpha;
    for (int r = 0; r < 32; ++r) {
      const float pr = valid[r] ? __expf(sc[r] - m_new) : 0.f;
      l += pr;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] += pr * vc[r][d];
    }
    m = m_new;
  }
  if (live) {
    float* orow = p.out + (((int64_t)b * p.Hq + h) * p.T + qi) * D;
    const float inv = 1.f / l;
#pragma unroll
    for (int d = 0; d < D; ++d) orow[d] = o[d] * inv;
  }
  latch_bad(p.status, bad);
}

// ------------------------------------------------------------------------------------------------

int attn_choose_splits(const Geom& g, long long max_list_tokens, int num_cus) {
  const long long tiles = 1 + (max_list_tokens + 63) / 64;
  const long long segs = (long long)g.B * g.Hkv;
  long long s = (2LL * num_cus + segs - 1) / segs;   // about two workgroups per CU
  if (s > tiles) s = tiles;
  if (s < 1) s = 1;
  if (segs > kMaxTickets) s = 1;
  return (int)s;
}

size_t attn_scratch_bytes(const Geom& g, int n_splits) {
  if (n_splits <= 1) return 0;
  const size_t per = (size_t)g.B * g.Hq * n_splits * 32;
  return per * g.D * sizeof(float) + per * sizeof(float2) + 256;
}

template <int D, int G>
static hipError_t launch_mfma(hipStream_t s, const AttnParams& p, dim3 grid, bool dense, bool paged) {
  const dim3 block(AttnShape<G>::NW * 64);
  if (dense) {
    if (paged) hipLaunchKernelGGL((attn_mfma_kernel<D, G, true, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((attn_mfma_kernel<D, G, true, false>), grid, block, 0, s, p);
  } else {
    if (paged) hipLaunchKernelGGL((attn_mfma_kernel<D, G, false, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((attn_mfma_kernel<D, G, false, false>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

template <int D>
static hipError_t launch_mfma_g(hipStream_t s, const AttnParams& p, dim3 grid, int G, bool dense,
                                bool paged) {
  switch (G) {
    case 1: return launch_mfma<D, 1>(s, p, grid, dense, paged);
    case 2: return launch_mfma<D, 2>(s, p, grid, dense, paged);
    case 3: return launch_mfma<D, 3>(s, p, grid, dense, paged);
    case 4: return launch_mfma<D, 4>(s, p, grid, dense, paged);
    case 5: return launch_mfma<D, 5>(s, p, grid, dense, paged);
    case 6: return launch_mfma<D, 6>(s, p, grid, dense, paged);
    case 7: return launch_mfma<D, 7>(s, p, grid, dense, paged);
    case 8: return launch_mfma<D, 8>(s, p, grid, dense, paged);
  }
  return hipErrorInvalidValue;
}

// fp32 path and grouped-query bf16 path (the one-query-head bf16 path is attn_mha.hip's).
static hipError_t launch_attn_other(hipStream_t s, const Geom& g, const void* q, const void* k,
                                    const void* v, const void* k_dec, const void* v_dec,
                                    const int32_t* page_table, const int32_t* sel_idx,
                                    const int32_t* n_sel, int max_sel, int unit_log2, int dense, void* out,
                                    char* scratch, int n_splits, uint32_t* tickets, uint32_t* status) {
  const int unit = 1 << unit_log2;
  const int n_units = (g.L + unit - 1) / unit;
  if (g.dtype == FDL_F32) {
    F32Params p;
    p.q = static_cast<const float*>(q);
    p.k = static_cast<const float*>(k);
    p.v = static_cast<const float*>(v);
    p.k_dec = static_cast<const float*>(k_dec);
    p.v_dec = static_cast<const float*>(v_dec);
    p.sel_idx = sel_idx;
    p.n_sel = n_sel;
    p.out = static_cast<float*>(out);
    p.status = status;
    p.page_table = page_table;
    p.Hq = g.Hq;
    p.Hkv = g.Hkv;
    p.G = g.G;
    p.T = g.T;
    p.L = g.L;
    p.max_sel = max_sel;
    p.unit_log2 = unit_log2;
    p.n_units = n_units;
    p.dense = dense;
    p.page_log2 = g.page_log2;
    p.pages_per_seq = g.pps;
    p.n_pages = g.n_pages;
    p.scale = 1.0f / sqrtf((float)g.D);
    dim3 grid(g.Hq, g.B);
    if (g.D == 128) {
      if (g.paged) hipLaunchKernelGGL((attn_f32_kernel<128, true>), grid, dim3(64), 0, s, p);
      else hipLaunchKernelGGL((attn_f32_kernel<128, false>), grid, dim3(64), 0, s, p);
    } else {
      if (g.paged) hipLaunchKernelGGL((attn_f32_kernel<64, true>), grid, dim3(64), 0, s, p);
      else hipLaunchKernelGGL((attn_f32_kernel<64, false>), grid, dim3(64), 0, s, p);
    }
    return hipGetLastError();
  }
  AttnParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.k_dec = static_cast<const uint16_t*>(k_dec);
  p.v_dec = static_cast<const uint16_t*>(v_dec);
  p.sel_idx = sel_idx;
  p.n_sel = n_sel;
  p.out = static_cast<uint16_t*>(out);
  const size_t per = (size_t)g.B * g.Hq * n_splits * 32;
  p.part_o = reinterpret_cast<float*>(scratch);
  p.part_ml = reinterpret_cast<float2*>(scratch + per * g.D * sizeof(float));
  p.tickets = tickets;
  p.status = status;
  p.page_table = page_table;
  p.Hq = g.Hq;
  p.Hkv = g.Hkv;
  p.T = g.T;
  p.L = g.L;
  p.max_sel = max_sel;
  p.unit_log2 = unit_log2;
  p.n_units = n_units;
  p.n_splits = n_splits;
  p.page_log2 = g.page_log2;
  p.pages_per_seq = g.pps;
  p.n_pages = g.n_pages;
  p.scale_log2 = 1.4426950408889634f / sqrtf((float)g.D);
  dim3 grid(n_splits, g.Hkv, g.B);
  hipError_t err = g.D == 128 ? launch_mfma_g<128>(s, p, grid, g.G, dense != 0, g.paged != 0)
                              : launch_mfma_g<64>(s, p, grid, g.G, dense != 0, g.paged != 0);
  if (err != hipSuccess || n_splits == 1) return err;
  return launch_attn_combine(s, p.part_o, p.part_ml, out, g.B * g.Hq, n_splits, g.T, g.D);
}

hipError_t launch_attn(hipStream_t s, const Geom& g, const void* q, const void* k, const void* v,
                       const void* k_dec, const void* v_dec, const int32_t* page_table,
                       const int32_t* sel_idx, const int32_t* n_sel, int max_sel, int unit_log2,
                       int dense, void* out, char* scratch, int n_splits, uint32_t* tickets,
                       uint32_t* status, int n_hint, const KernelTimer* timer) {
  if (g.dtype == FDL_BF16 && g.G == 1)
    return launch_attn_mha(s, g, q, k, v, k_dec, v_dec, page_table, sel_idx, n_sel, max_sel, unit_log2,
                           dense, out, scratch, n_splits, tickets, status, n_hint, timer);
  if (timer) (void)hipEventRecord(timer->a, s);
  const hipError_t err = launch_attn_other(s, g, q, k, v, k_dec, v_dec, page_table, sel_idx, n_sel,
                                           max_sel, unit_log2, dense, out, scratch, n_splits, tickets,
                                           status);
  if (timer) (void)hipEventRecord(timer->b, s);
  return err;
}

}  // namespace fdl
