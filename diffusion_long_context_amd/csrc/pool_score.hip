// Pooled keys and unit / token scoring, in pinned float32.
//
// Focus-dLLM (abstract; Elamur "Summary"): the predicted queries estimate which KV matters, so
// redundant attention can be skipped.  Prefilling-dLLM (abstract): whole prefix chunks are ranked
// first, then tokens inside the chosen chunks.  The pages give no formula; the reading built here:
// a unit is represented by the float32 sum of its keys, the predicted queries of a KV head's group
// are summed, and the score is the dot product of the two sums.  Every sum is the same
// adjacent-pair tree (operands zero-padded to a power of two; level by level, element 2j plus
// element 2j+1), every product is rounded to float32 before it is added, and nothing is fused, so
// the bits of every score are fixed by the inputs alone.  The whole file is compiled with
// floating-point contraction off for that reason.
//
// All three kernels are HBM-bound streaming reads: each lane issues its whole share of loads before
// the first add, rows are read as full 256-byte (bf16) or 512-byte (float32) lines by consecutive
// lanes, and cross-lane tree levels are xor butterflies (which reproduce the adjacent-pair tree
// exactly because float addition is commutative).
#pragma clang fp contract(off)

#include <type_traits>

#include "fdl_device.h"
#include "fdl_internal.h"
#include "fdl_score.h"

namespace fdl {

// ------------------------------------------------------------------------------------------------
// Key pooling: ks[b][g][n][d] = tree over the unit's tokens of k[b][g][t][d]
// ------------------------------------------------------------------------------------------------

template <typename KT>
__device__ __forceinline__ float2 load_pair(const KT* p);

template <>
__device__ __forceinline__ float2 load_pair<uint16_t>(const uint16_t* p) {
  // non-temporal: the cache is streamed once per pooling
  const uint32_t w = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
  return make_float2(bf16_bits_to_f32(w & 0xFFFFu), bf16_bits_to_f32(w >> 16));
}

template <>
__device__ __forceinline__ float2 load_pair<float>(const float* p) {
  return *reinterpret_cast<const float2*>(p);
}

__device__ __forceinline__ float2 add2(float2 a, float2 b) { return make_float2(a.x + b.x, a.y + b.y); }

constexpr int ilog2_const(int x) { return x <= 1 ? 0 : 1 + ilog2_const(x / 2); }

// Adjacent-pair tree over LEAVES consecutive tokens starting at t0 (tokens >= L are +0).  Every
// load is issued before the first add.  A full, aligned run of rows that lies in one page (or in a
// contiguous cache) is addressed from one base with compile-time strides, which keeps the loads'
// address registers few (and the waves per SIMD many).
template <typename KT, int D, int LEAVES, bool PAGED>
__device__ __forceinline__ float2 leaf_tree(const KT* __restrict__ k, const KvRows<PAGED>& rows, int b,
                                            int g, int t0, int pair, bool& bad) {
  // bf16 leaves stay packed (one register per leaf) until the first tree level converts them
  constexpr bool kPacked = std::is_same<KT, uint16_t>::value && LEAVES >= 2;
  using Leaf = typename std::conditional<kPacked, uint32_t, float2>::type;
  auto load_leaf = [&](const KT* p) -> Leaf {
    if constexpr (kPacked) return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
    else return load_pair<KT>(p);
  };
  Leaf a[LEAVES];
  const int Lb = rows.bound(b);   // this sequence's rows (ragged batches); the stride stays rows.L
  const bool run = (t0 & (LEAVES - 1)) == 0 && t0 + LEAVES <= Lb &&
                   (!PAGED || rows.page_log2 >= ilog2_const(LEAVES));
  // a row whose page id is out of range has no key: it reads a valid row (so that the loads stay
  // unconditional), counts +0 and latches `bad`
  uint64_t badm = 0;
  if (run) {   // uniform per team
    bool rb = false;
    const KT* base = k + rows.off(b, g, t0, rb) + 2 * pair;
    badm = rb ? ~0ull : 0ull;
#pragma unroll
    for (int i = 0; i < LEAVES; ++i) a[i] = load_leaf(base + i * D);
  } else {
#pragma unroll
    for (int i = 0; i < LEAVES; ++i) {
      const int t = t0 + i;
      bool rb = false;
      a[i] = load_leaf(k + rows.off(b, g, t < Lb ? t : (Lb > 0 ? Lb - 1 : 0), rb) + 2 * pair);
      badm |= (uint64_t)(rb && t < Lb) << i;
    }
  }
  bad = bad || badm != 0;
  const int live = Lb - t0;   // leaves at or past it are +0
  auto keep = [&](int i) { return i < live && ((badm >> i) & 1ull) == 0; };
  if constexpr (kPacked) {
    float2 s[LEAVES / 2];
#pragma unroll
    for (int i = 0; i < LEAVES / 2; ++i) {
      const uint32_t w0 = a[2 * i], w1 = a[2 * i + 1];
      const float2 x0 = keep(2 * i) ? make_float2(bf16_bits_to_f32(w0 & 0xFFFFu), bf16_bits_to_f32(w0 >> 16))
                                    : make_float2(0.f, 0.f);
      const float2 x1 = keep(2 * i + 1) ? make_float2(bf16_bits_to_f32(w1 & 0xFFFFu), bf16_bits_to_f32(w1 >> 16))
                                        : make_float2(0.f, 0.f);
      s[i] = add2(x0, x1);
    }
#pragma unroll
    for (int w = LEAVES / 4; w >= 1; w /= 2) {
#pragma unroll
      for (int i = 0; i < w; ++i) s[i] = add2(s[2 * i], s[2 * i + 1]);
    }
    return s[0];
  } else {
#pragma unroll
    for (int i = 0; i < LEAVES; ++i)
      if (!keep(i)) a[i] = make_float2(0.f, 0.f);
#pragma unroll
    for (int w = LEAVES / 2; w >= 1; w /= 2) {
#pragma unroll
      for (int i = 0; i < w; ++i) a[i] = add2(a[2 * i], a[2 * i + 1]);
    }
    return a[0];
  }
}

// Second pass of the pooling of units longer than 64 tokens: ks[b][g][n] = adjacent-pair tree over
// the unit's n_sub sub-unit sums sub[b][g][n * n_sub + i] (each the tree over 64 tokens; indices past
// n_sub_all are +0).  The tree over a power-of-two unit is the tree over its aligned 64-token
// sub-trees, so the bits are those of the one-pass tree.  Thread (unit, dimension pair).
// Units [n0, n0 + n_cnt) of the n_units.
// The G query heads' rows of KV head g staged as [8][32][D] bf16 (rows past T repeat row T - 1; heads
// past G are not read): one query head per KV head loads its 32 rows alone.  Every thread calls it;
// the stage is complete after it.
template <int D>
__device__ __forceinline__ void stage_group_queries(const uint16_t* __restrict__ q, int b, int g, int Hq, int G,
                                                    int T, uint16_t* stage) {
  if (G == 1) {   // uniform
    QsumG1<D, 32, 256> qs1;
    qsum_g1_issue<D, 32, 256>(q + ((int64_t)b * Hq + g) * T * D, T, qs1);
#pragma unroll
    for (int k = 0; k < QsumG1<D, 32, 256>::PER; ++k)
      if (k * 256 + (int)threadIdx.x < 32 * (D / 8)) *reinterpret_cast<uint4*>(stage + (k * 256 + threadIdx.x) * 8) = qs1.v[k];
  } else {
    QsumGrouped<D, 32, 256, 8> qst;
    qsum_grouped_issue<D, 32, 256, 8>(q + (int64_t)b * Hq * T * D, g * G, G, T, qst);
#pragma unroll
    for (int k = 0; k < QsumGrouped<D, 32, 256, 8>::PER; ++k)
      *reinterpret_cast<uint4*>(stage + (k * 256 + threadIdx.x) * 8) = qst.v[k];
  }
  block_sync_lds();
}

template <int D>
__global__ __launch_bounds__(256) void pool_merge_kernel(const float* __restrict__ sub, int n_sub, int n_sub_all,
                                                         int n0, int n_cnt, int n_units, int Hkv,
                                                         float* __restrict__ ks) {
  constexpr int kTeam = D / 2;
  constexpr int kTeams = 256 / kTeam;
  const int team = threadIdx.x / kTeam, pair = threadIdx.x % kTeam;
  const int n = n0 + blockIdx.x * kTeams + team;
  const int g = blockIdx.y, b = blockIdx.z;
  if (n >= n0 + n_cnt) return;
  const float* src = sub + ((int64_t)b * Hkv + g) * n_sub_all * D + 2 * pair;
  float2 a[64];
  // every load unconditional (clamped index), masked afterwards: a guarded load would be waited for
  // on its own
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    const int si = n * n_sub + i;
    a[i] = *reinterpret_cast<const float2*>(src + (int64_t)(si < n_sub_all ? si : n_sub_all - 1) * D);
  }
#pragma unroll
  for (int i = 0; i < 64; ++i)
    if (!(i < n_sub && n * n_sub + i < n_sub_all)) a[i] = make_float2(0.f, 0.f);
#pragma unroll
  for (int w = 32; w >= 1; w /= 2) {
    if (w < n_sub) {   // uniform: levels of the n_sub-leaf tree only
#pragma unroll
      for (int i = 0; i < w; ++i) a[i] = add2(a[2 * i], a[2 * i + 1]);
    }
  }
  *reinterpret_cast<float2*>(ks + (((int64_t)b * Hkv + g) * n_units + n) * D + 2 * pair) = a[0];
}

// One "team" of D/2 threads per unit; thread `pair` owns dimensions 2*pair and 2*pair+1.
template <typename KT, int D, int LEAVES, bool PAGED>
__global__ __launch_bounds__(256) void pool_keys_kernel(const KT* __restrict__ k, KvRows<PAGED> rows,
                                                        int unit_log2, int n_units,
                                                        float* __restrict__ ks,
                                                        uint32_t* __restrict__ status) {
  extern __shared__ float2 sub_sums[];  // [teams][n_sub][D/2], only when unit > LEAVES
  constexpr int kTeam = D / 2;
  constexpr int kTeams = 256 / kTeam;
  // a team of 64 threads is one wave: its unit, rows and page entries are then uniform (scalar
  // registers and scalar loads), and the loads' only per-lane address part is the column pair
  const int team = kTeam == 64 ? __builtin_amdgcn_readfirstlane(threadIdx.x / kTeam) : threadIdx.x / kTeam;
  const int pair = threadIdx.x % kTeam;
  const int g = blockIdx.y, b = blockIdx.z;
  const int n_raw = blockIdx.x * kTeams + team;
  const bool live = n_raw < n_units;
  const int n = live ? n_raw : n_units - 1;
  const int unit = 1 << unit_log2;
  const int t_unit = n << unit_log2;
  bool bad = false;
  float2 r;
  if (unit <= LEAVES) {
    r = leaf_tree<KT, D, LEAVES, PAGED>(k, rows, b, g, t_unit, pair, bad);
  } else {
    const int n_sub = unit / LEAVES;
    float2* mine = sub_sums + (size_t)team * n_sub * kTeam;
    for (int sb = 0; sb < n_sub; ++sb)
      mine[sb * kTeam + pair] = leaf_tree<KT, D, LEAVES, PAGED>(k, rows, b, g, t_unit + sb * LEAVES, pair, bad);
    // tree over the sub-unit sums; each thread only touches its own column, so no barrier
    for (int w = n_sub / 2; w >= 1; w /= 2)
      for (int i = 0; i < w; ++i)
        mine[i * kTeam + pair] = add2(mine[(2 * i) * kTeam + pair], mine[(2 * i + 1) * kTeam + pair]);
    r = mine[pair];
  }
  if (live) {
    float* dst = ks + (((int64_t)b * rows.Hkv + g) * n_units + n) * D;
    *reinterpret_cast<float2*>(dst + 2 * pair) = r;
  }
  latch_bad(status, bad);
}

template <bool PAGED>
static KvRows<PAGED> make_rows(const Geom& g, const int32_t* page_table) {
  KvRows<PAGED> r;
  r.Hkv = g.Hkv;
  r.L = g.L;
  r.D = g.D;
  r.page_log2 = g.page_log2;
  r.pages_per_seq = g.pps;
  r.n_pages = g.n_pages;
  r.page_table = page_table;
  r.lens = g.lens;
  return r;
}

template <typename KT, int D, bool PAGED>
static hipError_t pool_dispatch(hipStream_t s, const Geom& g, const KT* k, const int32_t* page_table,
                                int unit_log2, float* ks, uint32_t* status, float* sub, size_t sub_bytes) {
  const int unit = 1 << unit_log2;
  const int n_units = (g.L + unit - 1) / unit;
  if (n_units == 0) return hipSuccess;
  const KvRows<PAGED> rows = make_rows<PAGED>(g, page_table);
  constexpr int kTeams = 256 / (D / 2);
  const int n_sub_all = (g.L + 63) / 64;
  if (unit > 64 && unit / 64 <= 64 && sub != nullptr &&
      (size_t)g.B * g.Hkv * n_sub_all * D * sizeof(float) <= sub_bytes) {
    // two passes: 64-token sub-unit sums over the whole chip, then the tree over each unit's
    // sub-sums (one pass would give each unit's 64-token runs to one team, one after another)
    dim3 g1((n_sub_all + kTeams - 1) / kTeams, g.Hkv, g.B);
    hipLaunchKernelGGL((pool_keys_kernel<KT, D, 64, PAGED>), g1, dim3(256), 0, s, k, rows, 6, n_sub_all, sub,
                       status);
    dim3 g2((n_units + kTeams - 1) / kTeams, g.Hkv, g.B);
    hipLaunchKernelGGL((pool_merge_kernel<D>), g2, dim3(256), 0, s, sub, unit / 64, n_sub_all, 0, n_units, n_units,
                       g.Hkv, ks);
    return hipGetLastError();
  }
  dim3 grid((n_units + kTeams - 1) / kTeams, g.Hkv, g.B);
  size_t lds = 0;
  if (unit > 64) lds = (size_t)kTeams * (unit / 64) * (D / 2) * sizeof(float2);
  switch (unit_log2) {
#define FDL_POOL_CASE(LG)                                                                          \
  case LG:                                                                                         \
    hipLaunchKernelGGL((pool_keys_kernel<KT, D, (1 << LG), PAGED>), grid, dim3(256), lds, s, k,   \
                       rows, unit_log2, n_units, ks, status);                                      \
    break;
    FDL_POOL_CASE(0) FDL_POOL_CASE(1) FDL_POOL_CASE(2) FDL_POOL_CASE(3) FDL_POOL_CASE(4)
    FDL_POOL_CASE(5)
#undef FDL_POOL_CASE
    default: {
      auto kern = pool_keys_kernel<KT, D, 64, PAGED>;
      if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
      }
      hipLaunchKernelGGL(kern, grid, dim3(256), lds, s, k, rows, unit_log2, n_units, ks, status);
    }
  }
  return hipGetLastError();
}

hipError_t launch_pool_keys(hipStream_t s, const Geom& g, const void* k, const int32_t* page_table,
                            int unit_log2, float* ks, uint32_t* status, float* sub, size_t sub_bytes) {
  if (g.dtype == FDL_BF16) {
    const uint16_t* kk = static_cast<const uint16_t*>(k);
    if (g.paged)
      return g.D == 128 ? pool_dispatch<uint16_t, 128, true>(s, g, kk, page_table, unit_log2, ks, status, sub, sub_bytes)
                        : pool_dispatch<uint16_t, 64, true>(s, g, kk, page_table, unit_log2, ks, status, sub, sub_bytes);
    return g.D == 128 ? pool_dispatch<uint16_t, 128, false>(s, g, kk, page_table, unit_log2, ks, status, sub, sub_bytes)
                      : pool_dispatch<uint16_t, 64, false>(s, g, kk, page_table, unit_log2, ks, status, sub, sub_bytes);
  }
  const float* kk = static_cast<const float*>(k);
  if (g.paged)
    return g.D == 128 ? pool_dispatch<float, 128, true>(s, g, kk, page_table, unit_log2, ks, status, sub, sub_bytes)
                      : pool_dispatch<float, 64, true>(s, g, kk, page_table, unit_log2, ks, status, sub, sub_bytes);
  return g.D == 128 ? pool_dispatch<float, 128, false>(s, g, kk, page_table, unit_log2, ks, status, sub, sub_bytes)
                    : pool_dispatch<float, 64, false>(s, g, kk, page_table, unit_log2, ks, status, sub, sub_bytes);
}

// ------------------------------------------------------------------------------------------------
// Cache write with the pooling of the units it touches: the new rows [t0, t0 + n_tok) of every
// (sequence, KV head) go to the cache (contiguous or paged), and each touched unit's keys are pooled
// from the rows it then holds -- the new rows straight from the registers they were loaded into, so
// the written keys are read once instead of written and read back by a separate pooling.
// ------------------------------------------------------------------------------------------------

struct CacheWrite {
  const void* k_new;   // [B][Hkv][n_tok][D]
  const void* v_new;
  void* k;             // cache: [B][Hkv][L][D], or the page pool [n_pages][Hkv][P][D]
  void* v;
  int t0, n_tok;
};

template <typename KT>
struct PairOf {
  using T = float2;
};
template <>
struct PairOf<uint16_t> {
  using T = uint32_t;   // two bf16 kept packed
};

// One team of D/2 threads per run of RUN tokens (RUN = min(unit, 64)) of the touched units; thread
// `pair` owns dimensions 2 pair, 2 pair + 1.  Every row of the run is read from the new rows when it
// is written, else from the cache (rows past L read a valid row and count +0); the written rows of K
// and V are stored to the cache; with pooling, the run's adjacent-pair tree goes to out[b][g][run]
// (the pooled keys when the unit is the run, else the sub-sums of the two-pass pooling).
template <typename KT, int D, int RUN, bool PAGED>
__global__ __launch_bounds__(256) void cache_write_pool_kernel(CacheWrite w, KvRows<PAGED> rows, int run0,
                                                               int n_runs, int out_units, float* __restrict__ out,
                                                               uint32_t* __restrict__ status) {
  using PT = typename PairOf<KT>::T;
  constexpr int kTeam = D / 2;
  constexpr int kTeams = 256 / kTeam;
  const int team = kTeam == 64 ? __builtin_amdgcn_readfirstlane(threadIdx.x / kTeam) : threadIdx.x / kTeam;
  const int pair = threadIdx.x % kTeam;
  const int g = blockIdx.y, b = blockIdx.z;
  const int run = run0 + blockIdx.x * kTeams + team;
  if (run >= run0 + n_runs) return;
  const int t_run = run * RUN;
  const int64_t seg = (int64_t)b * rows.Hkv + g;
  const KT* kn = static_cast<const KT*>(w.k_new) + seg * w.n_tok * D + 2 * pair;
  const KT* vn = static_cast<const KT*>(w.v_new) + seg * w.n_tok * D + 2 * pair;
  KT* kc = static_cast<KT*>(w.k);
  KT* vc = static_cast<KT*>(w.v);
  PT ka[RUN], va[RUN];
  // every load unconditional: the source is chosen by address (a guarded load would be waited for on
  // its own); a row's cache offset is uniform per team and recomputed for the stores rather than kept.
  // A row whose page id is out of range has no place in the cache: it is neither stored nor read
  // (its cache load reads page 0 and is dropped), it counts +0 in the pooled keys, and it latches
  // ST_BAD_INDEX (bit i of badm: row t_run + i).
  uint64_t badm = 0;
#pragma unroll
  for (int i = 0; i < RUN; ++i) {
    const int t = t_run + i;
    const bool in = t >= w.t0 && t < w.t0 + w.n_tok;   // uniform per team
    bool rb = false;
    const int64_t coff = rows.off(b, g, t < rows.L ? t : rows.L - 1, rb);
    badm |= (uint64_t)(rb && t < rows.L) << i;
    const int64_t noff = (int64_t)(in ? t - w.t0 : 0) * D;
    ka[i] = *reinterpret_cast<const PT*>(in ? kn + noff : kc + coff + 2 * pair);
    va[i] = *reinterpret_cast<const PT*>(in ? vn + noff : vc + coff + 2 * pair);
  }
#pragma unroll
  for (int i = 0; i < RUN; ++i) {
    const int t = t_run + i;
    if (t >= w.t0 && t < w.t0 + w.n_tok && ((badm >> i) & 1ull) == 0) {   // uniform per team
      bool unused = false;
      const int64_t coff = rows.off(b, g, t, unused) + 2 * pair;
      *reinterpret_cast<PT*>(kc + coff) = ka[i];
      *reinterpret_cast<PT*>(vc + coff) = va[i];
    }
  }
  latch_bad(status, badm != 0);
  if (out == nullptr) return;
  float2 x[RUN];
#pragma unroll
  for (int i = 0; i < RUN; ++i) {
    if constexpr (std::is_same<KT, uint16_t>::value)
      x[i] = make_float2(bf16_bits_to_f32(ka[i] & 0xFFFFu), bf16_bits_to_f32(ka[i] >> 16));
    else
      x[i] = ka[i];
    if (t_run + i >= rows.L || ((badm >> i) & 1ull) != 0) x[i] = make_float2(0.f, 0.f);
  }
#pragma unroll
  for (int wdt = RUN / 2; wdt >= 1; wdt /= 2) {
#pragma unroll
    for (int i = 0; i < wdt; ++i) x[i] = add2(x[2 * i], x[2 * i + 1]);
  }
  *reinterpret_cast<float2*>(out + (seg * out_units + run) * D + 2 * pair) = x[0];
}

template <typename KT, int D, bool PAGED>
static hipError_t cache_write_dispatch(hipStream_t s, const Geom& g, const CacheWrite& w, const int32_t* page_table,
                                       int unit_log2, float* ks, uint32_t* status, float* sub, size_t sub_bytes) {
  const KvRows<PAGED> rows = make_rows<PAGED>(g, page_table);
  constexpr int kTeams = 256 / (D / 2);
  const int unit = 1 << unit_log2;
  const int run_tok = ks == nullptr ? 64 : (unit < 64 ? unit : 64);
  const int n_runs_all = (g.L + run_tok - 1) / run_tok;
  int r0, r1;   // runs [r0, r1)
  int u0 = 0, u1 = 0;
  if (ks == nullptr) {
    r0 = w.t0 / run_tok;
    r1 = (w.t0 + w.n_tok - 1) / run_tok + 1;
  } else {
    u0 = w.t0 >> unit_log2;
    u1 = ((w.t0 + w.n_tok - 1) >> unit_log2) + 1;
    r0 = (int)(((int64_t)u0 << unit_log2) / run_tok);
    r1 = (int)(((int64_t)u1 << unit_log2) / run_tok);
    if (r1 > n_runs_all) r1 = n_runs_all;
  }
  float* out = ks;
  int out_units = (g.L + unit - 1) / unit;
  if (ks != nullptr && unit > 64) {
    if (unit / 64 > 64 || sub == nullptr || (size_t)g.B * g.Hkv * n_runs_all * D * sizeof(float) > sub_bytes)
      return hipErrorOutOfMemory;
    out = sub;
    out_units = n_runs_all;
  }
  if (run_tok != 16 && run_tok != 32 && run_tok != 64) return hipErrorInvalidValue;
  const dim3 grid((r1 - r0 + kTeams - 1) / kTeams, g.Hkv, g.B);
  switch (run_tok) {
    case 16: hipLaunchKernelGGL((cache_write_pool_kernel<KT, D, 16, PAGED>), grid, dim3(256), 0, s, w, rows, r0, r1 - r0,
                                out_units, out, status); break;
    case 32: hipLaunchKernelGGL((cache_write_pool_kernel<KT, D, 32, PAGED>), grid, dim3(256), 0, s, w, rows, r0, r1 - r0,
                                out_units, out, status); break;
    default: hipLaunchKernelGGL((cache_write_pool_kernel<KT, D, 64, PAGED>), grid, dim3(256), 0, s, w, rows, r0, r1 - r0,
                                out_units, out, status);
  }
  if (ks == nullptr || unit <= 64) return hipGetLastError();
  const dim3 g2((u1 - u0 + kTeams - 1) / kTeams, g.Hkv, g.B);
  hipLaunchKernelGGL((pool_merge_kernel<D>), g2, dim3(256), 0, s, sub, unit / 64, n_runs_all, u0, u1 - u0,
                     (g.L + unit - 1) / unit, g.Hkv, ks);
  return hipGetLastError();
}

hipError_t launch_cache_write(hipStream_t s, const Geom& g, const void* k_new, const void* v_new, int t0, int n_tok,
                              void* k, void* v, const int32_t* page_table, int unit_log2, float* ks, uint32_t* status,
                              float* sub, size_t sub_bytes) {
  const CacheWrite w{k_new, v_new, k, v, t0, n_tok};
  if (g.dtype == FDL_BF16) {
    if (g.paged)
      return g.D == 128 ? cache_write_dispatch<uint16_t, 128, true>(s, g, w, page_table, unit_log2, ks, status, sub, sub_bytes)
                        : cache_write_dispatch<uint16_t, 64, true>(s, g, w, page_table, unit_log2, ks, status, sub, sub_bytes);
    return g.D == 128 ? cache_write_dispatch<uint16_t, 128, false>(s, g, w, page_table, unit_log2, ks, status, sub, sub_bytes)
                      : cache_write_dispatch<uint16_t, 64, false>(s, g, w, page_table, unit_log2, ks, status, sub, sub_bytes);
  }
  if (g.paged)
    return g.D == 128 ? cache_write_dispatch<float, 128, true>(s, g, w, page_table, unit_log2, ks, status, sub, sub_bytes)
                      : cache_write_dispatch<float, 64, true>(s, g, w, page_table, unit_log2, ks, status, sub, sub_bytes);
  return g.D == 128 ? cache_write_dispatch<float, 128, false>(s, g, w, page_table, unit_log2, ks, status, sub, sub_bytes)
                    : cache_write_dispatch<float, 64, false>(s, g, w, page_table, unit_log2, ks, status, sub, sub_bytes);
}

// ------------------------------------------------------------------------------------------------
// Predicted-query sum: qs[d] = tree over the group's heads (padded to 2^m) of the tree over the T
// slots (padded to 2^m; non-predicted slots +0) of q[b][h][p][d].  Computed by threads d < D of the
// block into LDS; every q load is issued before the first add.
// ------------------------------------------------------------------------------------------------

// ------------------------------------------------------------------------------------------------
// Level-1 unit scores from pooled keys: scores[b][g][n] = dot(qs, ks[b][g][n])
// ------------------------------------------------------------------------------------------------

constexpr int kUnitsPerWg = 64;

template <typename QT, int D, int TMAX>
__global__ __launch_bounds__(256) void score_units_kernel(const QT* __restrict__ q,
                                                          const uint64_t* __restrict__ pred_mask,
                                                          const float* __restrict__ ks, int Hq,
                                                          int Hkv, int G, int T, int n_units,
                                                          float* __restrict__ scores, const int32_t* lens,
                                                          int L, int unit_log2) {
  constexpr int LPR = D / 16;            // lanes per row
  constexpr int kRowsPerWave = 64 / LPR;
  constexpr int kRowsPerPass = 4 * kRowsPerWave;
  constexpr int kPasses = kUnitsPerWg / kRowsPerPass;
  __shared__ float qs[D];
  const int g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane % LPR;
  const int n0 = blockIdx.x * kUnitsPerWg;
  const float* ksg = ks + ((int64_t)b * Hkv + g) * n_units * D;

  // this lane's row loads go out before the query sum, so they are in flight meanwhile
  float x[kPasses][16];
#pragma unroll
  for (int ps = 0; ps < kPasses; ++ps) {
    int n = n0 + ps * kRowsPerPass + wave * kRowsPerWave + lane / LPR;
    n = n < n_units ? n : n_units - 1;
    load16<float>(ksg + (int64_t)n * D + 16 * j, x[ps]);
  }
  if constexpr (std::is_same<QT, uint16_t>::value && TMAX == 32) {
    __shared__ __attribute__((aligned(16))) uint16_t stage[8 * 32 * D];
    if (G == 1) {   // uniform: one query head per KV head, its 32 rows alone (the same tree and bits)
      QsumG1<D, 32, 256> qs1;
      qsum_g1_issue<D, 32, 256>(q + ((int64_t)b * Hq + g) * T * D, T, qs1);
      qsum_g1_finish<D, 32, 256>(qs1, pred_mask[b], T, reinterpret_cast<float*>(stage), qs);
    } else {
      QsumGrouped<D, 32, 256, 8> qst;
      qsum_grouped_issue<D, 32, 256, 8>(q + (int64_t)b * Hq * T * D, g * G, G, T, qst);
      qsum_grouped_finish<D, 32, 256, 8>(qst, pred_mask[b], G, T, stage, qs);
    }
  } else {
    query_sum_to_lds<QT, D, TMAX>(q, pred_mask[b], b, g, Hq, G, T, qs);
  }
  __syncthreads();
  float qv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) qv[i] = qs[16 * j + i];
  // a ragged batch's units past the sequence's own score +0
  const int nb = lens == nullptr ? n_units : (seq_len(lens, b, L) + (1 << unit_log2) - 1) >> unit_log2;
#pragma unroll
  for (int ps = 0; ps < kPasses; ++ps) {
    const int n = n0 + ps * kRowsPerPass + wave * kRowsPerWave + lane / LPR;
    const float sc = row_dot<LPR>(x[ps], qv);
    if (n < n_units && j == 0) scores[((int64_t)b * Hkv + g) * n_units + n] = n < nb ? sc : 0.f;
  }
}

template <typename QT, int D>
static void launch_su(hipStream_t s, const Geom& g, const QT* q, const uint64_t* pm, const float* ks,
                      int n_units, int ulog, float* scores) {
  dim3 grid((n_units + kUnitsPerWg - 1) / kUnitsPerWg, g.Hkv, g.B);
  if (g.T <= 32)
    hipLaunchKernelGGL((score_units_kernel<QT, D, 32>), grid, dim3(256), 0, s, q, pm, ks, g.Hq, g.Hkv,
                       g.G, g.T, n_units, scores, g.lens, g.L, ulog);
  else
    hipLaunchKernelGGL((score_units_kernel<QT, D, 64>), grid, dim3(256), 0, s, q, pm, ks, g.Hq, g.Hkv,
                       g.G, g.T, n_units, scores, g.lens, g.L, ulog);
}

hipError_t launch_score_units(hipStream_t s, const Geom& g, const void* q, const uint64_t* pred_mask,
                              const float* ks, int n_units, int unit_log2, float* scores) {
  if (n_units == 0) return hipSuccess;
  if (g.dtype == FDL_BF16) {
    const uint16_t* qq = static_cast<const uint16_t*>(q);
    if (g.D == 128) launch_su<uint16_t, 128>(s, g, qq, pred_mask, ks, n_units, unit_log2, scores);
    else launch_su<uint16_t, 64>(s, g, qq, pred_mask, ks, n_units, unit_log2, scores);
  } else {
    const float* qq = static_cast<const float*>(q);
    if (g.D == 128) launch_su<float, 128>(s, g, qq, pred_mask, ks, n_units, unit_log2, scores);
    else launch_su<float, 64>(s, g, qq, pred_mask, ks, n_units, unit_log2, scores);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------
// Per-query (max) unit scores: scores[b][g][n] = max over the group's predicted queries q of the
// pinned dot(q, ks[b][g][n]) (+0 when nothing is predicted; -0 reads +0).  The group's query rows are
// staged in LDS once (bf16, one round of 16-byte loads); each lane group keeps its unit rows in
// registers and runs the row dot of every predicted query against them.
// ------------------------------------------------------------------------------------------------

template <int D>
__global__ __launch_bounds__(256) void score_units_max_kernel(const uint16_t* __restrict__ q,
                                                              const uint64_t* __restrict__ pred_mask,
                                                              const float* __restrict__ ks, int Hq, int Hkv,
                                                              int G, int T, int n_units, float* __restrict__ scores) {
  constexpr int LPR = D / 16;
  constexpr int kRowsPerWave = 64 / LPR;
  constexpr int kRowsPerPass = 4 * kRowsPerWave;
  constexpr int kPasses = kUnitsPerWg / kRowsPerPass;
  __shared__ __attribute__((aligned(16))) uint16_t stage[8 * 32 * D];
  const int g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane % LPR;
  const int n0 = blockIdx.x * kUnitsPerWg;
  const float* ksg = ks + ((int64_t)b * Hkv + g) * n_units * D;
  float x[kPasses][16];
#pragma unroll
  for (int ps = 0; ps < kPasses; ++ps) {
    int n = n0 + ps * kRowsPerPass + wave * kRowsPerWave + lane / LPR;
    n = n < n_units ? n : n_units - 1;
    load16<float>(ksg + (int64_t)n * D + 16 * j, x[ps]);
  }
  stage_group_queries<D>(q, b, g, Hq, G, T, stage);
  const uint64_t pred = pred_mask[b] & (T >= 64 ? ~0ull : ((1ull << T) - 1ull));
  float best[kPasses];
#pragma unroll
  for (int ps = 0; ps < kPasses; ++ps) best[ps] = -__builtin_inff();
  for (int jh = 0; jh < G; ++jh) {
    for (uint64_t m = pred; m != 0ull; m &= m - 1ull) {   // uniform: the predicted positions
      const int pp = __builtin_ctzll(m);
      const uint4* src = reinterpret_cast<const uint4*>(stage + (jh * 32 + pp) * D + 16 * j);
      const uint4 a = src[0], c = src[1];
      const uint32_t w[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
      float qv[16];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        qv[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
        qv[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
      }
#pragma unroll
      for (int ps = 0; ps < kPasses; ++ps) best[ps] = fmaxf(best[ps], row_dot<LPR>(x[ps], qv));
    }
  }
#pragma unroll
  for (int ps = 0; ps < kPasses; ++ps) {
    const int n = n0 + ps * kRowsPerPass + wave * kRowsPerWave + lane / LPR;
    if (n < n_units && j == 0) scores[((int64_t)b * Hkv + g) * n_units + n] = pred != 0ull ? best[ps] + 0.f : 0.f;
  }
}

hipError_t launch_score_units_max(hipStream_t s, const Geom& g, const void* q, const uint64_t* pred_mask,
                                  const float* ks, int n_units, float* scores) {
  if (n_units == 0) return hipSuccess;
  if (g.dtype != FDL_BF16 || g.T > 32 || g.G > 8) return hipErrorInvalidValue;
  dim3 grid((n_units + kUnitsPerWg - 1) / kUnitsPerWg, g.Hkv, g.B);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  if (g.D == 128)
    hipLaunchKernelGGL((score_units_max_kernel<128>), grid, dim3(256), 0, s, qq, pred_mask, ks, g.Hq, g.Hkv, g.G,
                       g.T, n_units, scores);
  else
    hipLaunchKernelGGL((score_units_max_kernel<64>), grid, dim3(256), 0, s, qq, pred_mask, ks, g.Hq, g.Hkv, g.G,
                       g.T, n_units, scores);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------
// Softmax-mass unit scores: every predicted query q of the group attends to the units' mean keys
// (key sum / valid tokens of the unit) with the scale 1/sqrt(D), softmax over the head's units;
// scores[b][g][n] = sum over those queries of the probability of unit n (zeros when nothing is
// predicted).  Three launches: the scaled logits of every (predicted query, unit) into the scratch
// z[b][g][G * T][n_units] (same row layout and dot product as the max scorer), one wave per
// (query, head) for the query's log-sum-exp statistics, and one workgroup per (unit chunk, head)
// summing the probabilities.
// ------------------------------------------------------------------------------------------------

template <int D>
__global__ __launch_bounds__(256) void mass_logits_kernel(const uint16_t* __restrict__ q,
                                                          const uint64_t* __restrict__ pred_mask,
                                                          const float* __restrict__ ks, int Hq, int Hkv, int G,
                                                          int T, int n_units, int unit_log2, int L,
                                                          float* __restrict__ z) {
  constexpr int LPR = D / 16;
  constexpr int kRowsPerWave = 64 / LPR;
  constexpr int kRowsPerPass = 4 * kRowsPerWave;
  constexpr int kPasses = kUnitsPerWg / kRowsPerPass;
  __shared__ __attribute__((aligned(16))) uint16_t stage[8 * 32 * D];
  const int g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane % LPR;
  const int n0 = blockIdx.x * kUnitsPerWg;
  const float* ksg = ks + ((int64_t)b * Hkv + g) * n_units * D;
  float x[kPasses][16];
  float scale[kPasses];   // 1 / (valid tokens of the unit * sqrt(D))
#pragma unroll
  for (int ps = 0; ps < kPasses; ++ps) {
    int n = n0 + ps * kRowsPerPass + wave * kRowsPerWave + lane / LPR;
    n = n < n_units ? n : n_units - 1;
    load16<float>(ksg + (int64_t)n * D + 16 * j, x[ps]);
    const int first = n << unit_log2;
    const int cnt = (L - first) < (1 << unit_log2) ? (L - first) : (1 << unit_log2);
    scale[ps] = 1.f / ((float)cnt * sqrtf((float)D));
  }
  stage_group_queries<D>(q, b, g, Hq, G, T, stage);
  const uint64_t pred = pred_mask[b] & (T >= 64 ? ~0ull : ((1ull << T) - 1ull));
  float* zg = z + ((int64_t)b * Hkv + g) * (int64_t)G * T * n_units;
  for (int jh = 0; jh < G; ++jh) {
    for (uint64_t m = pred; m != 0ull; m &= m - 1ull) {   // uniform: the predicted positions
      const int pp = __builtin_ctzll(m);
      const uint4* src = reinterpret_cast<const uint4*>(stage + (jh * 32 + pp) * D + 16 * j);
      const uint4 a = src[0], c = src[1];
      const uint32_t w[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
      float qv[16];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        qv[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
        qv[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
      }
      float* zrow = zg + (int64_t)(jh * T + pp) * n_units;
#pragma unroll
      for (int ps = 0; ps < kPasses; ++ps) {
        const float d = row_dot<LPR>(x[ps], qv);
        const int n = n0 + ps * kRowsPerPass + wave * kRowsPerWave + lane / LPR;
        if (n < n_units && j == 0) zrow[n] = d * scale[ps];
      }
    }
  }
}

// One wave per (predicted query slot, head): max and sum of exp over the head's units.
__global__ __launch_bounds__(64) void mass_stats_kernel(const uint64_t* __restrict__ pred_mask, int Hkv, int G,
                                                        int T, int n_units, const float* __restrict__ z,
                                                        float2* __restrict__ stats) {
  const int slot = blockIdx.x, g = blockIdx.y, b = blockIdx.z;   // slot = jh * T + position
  const int lane = threadIdx.x;
  if (!((pred_mask[b] >> (slot % T)) & 1ull)) return;   // uniform
  const int64_t row = ((int64_t)b * Hkv + g) * G * T + slot;
  const float* zr = z + row * n_units;
  float m = -__builtin_inff();
  for (int n = lane; n < n_units; n += 64) m = fmaxf(m, zr[n]);
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  float sum = 0.f;
  for (int n = lane; n < n_units; n += 64) sum += expf(zr[n] - m);
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 64);
  if (lane == 0) stats[row] = make_float2(m, sum);
}

// One workgroup per (chunk of 256 units, head): each thread sums its unit's probabilities over the
// predicted queries.
__global__ __launch_bounds__(256) void mass_sum_kernel(const uint64_t* __restrict__ pred_mask, int Hkv, int G,
                                                       int T, int n_units, const float* __restrict__ z,
                                                       const float2* __restrict__ stats, float* __restrict__ scores) {
  const int g = blockIdx.y, b = blockIdx.z;
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= n_units) return;
  const uint64_t pred = pred_mask[b] & (T >= 64 ? ~0ull : ((1ull << T) - 1ull));
  const int64_t row0 = ((int64_t)b * Hkv + g) * G * T;
  float acc = 0.f;
  for (int jh = 0; jh < G; ++jh) {
    for (uint64_t m = pred; m != 0ull; m &= m - 1ull) {   // uniform
      const int64_t row = row0 + jh * T + __builtin_ctzll(m);
      const float2 st = stats[row];
      acc += expf(z[row * n_units + n] - st.x) / st.y;
    }
  }
  scores[((int64_t)b * Hkv + g) * n_units + n] = acc;
}

size_t mass_scratch_bytes(const Geom& g, int n_units) {
  const size_t rows = (size_t)g.B * g.Hkv * g.G * g.T;
  return ((rows * n_units * sizeof(float) + 255) & ~(size_t)255) + rows * sizeof(float2);
}

hipError_t launch_score_units_mass(hipStream_t s, const Geom& g, const void* q, const uint64_t* pred_mask,
                                   const float* ks, int n_units, int unit_log2, float* scores, char* scratch) {
  if (n_units == 0) return hipSuccess;
  if (g.dtype != FDL_BF16 || g.T > 32 || g.G > 8) return hipErrorInvalidValue;
  const size_t rows = (size_t)g.B * g.Hkv * g.G * g.T;
  float* z = reinterpret_cast<float*>(scratch);
  float2* stats = reinterpret_cast<float2*>(scratch + ((rows * n_units * sizeof(float) + 255) & ~(size_t)255));
  dim3 grid((n_units + kUnitsPerWg - 1) / kUnitsPerWg, g.Hkv, g.B);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  if (g.D == 128)
    hipLaunchKernelGGL((mass_logits_kernel<128>), grid, dim3(256), 0, s, qq, pred_mask, ks, g.Hq, g.Hkv, g.G, g.T,
                       n_units, unit_log2, g.L, z);
  else
    hipLaunchKernelGGL((mass_logits_kernel<64>), grid, dim3(256), 0, s, qq, pred_mask, ks, g.Hq, g.Hkv, g.G, g.T,
                       n_units, unit_log2, g.L, z);
  hipLaunchKernelGGL(mass_stats_kernel, dim3(g.G * g.T, g.Hkv, g.B), dim3(64), 0, s, pred_mask, g.Hkv, g.G, g.T,
                     n_units, z, stats);
  hipLaunchKernelGGL(mass_sum_kernel, dim3((n_units + 255) / 256, g.Hkv, g.B), dim3(256), 0, s, pred_mask, g.Hkv,
                     g.G, g.T, n_units, z, stats, scores);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------
// Level-2 token scores inside candidate units (chunks), keys read through the page table:
// scores[b][g][c][i] = dot(qs, k[token = cand_idx[b][g][c] * unit + i])
// ------------------------------------------------------------------------------------------------

constexpr int kTokensPerWg = 256;

template <typename KT, int D, int TMAX, bool PAGED>
__global__ __launch_bounds__(256) void score_tokens_kernel(
    const KT* __restrict__ q, const uint64_t* __restrict__ pred_mask, const KT* __restrict__ k,
    KvRows<PAGED> rows, int Hq, int G, int T, int unit_log2, const int32_t* __restrict__ cand_idx,
    int n_cand, float* __restrict__ scores, uint32_t* __restrict__ status) {
  constexpr int LPR = D / 16;
  constexpr int kRowsPerWave = 64 / LPR;
  constexpr int kRowsPerPass = 4 * kRowsPerWave;
  constexpr int kPasses = kTokensPerWg / kRowsPerPass;
  __shared__ float qs[D];
  const int g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane % LPR;
  const int64_t total = (int64_t)n_cand << unit_log2;
  const int64_t r0 = (int64_t)blockIdx.x * kTokensPerWg;
  const int n_units = (rows.L + (1 << unit_log2) - 1) >> unit_log2;
  const int32_t* cands = cand_idx + ((int64_t)b * rows.Hkv + g) * n_cand;
  bool bad = false;

  // candidate units -> tokens -> (pages) -> rows, each stage's loads issued together
  int tok[kPasses];
  bool ok[kPasses];
#pragma unroll
  for (int ps = 0; ps < kPasses; ++ps) {
    int64_t r = r0 + ps * kRowsPerPass + wave * kRowsPerWave + lane / LPR;
    ok[ps] = r < total;
    r = ok[ps] ? r : 0;
    const int u = cands[(int)(r >> unit_log2)];
    const bool uok = (unsigned)u < (unsigned)n_units;
    bad = bad || (ok[ps] && !uok);
    int t = uok ? (u << unit_log2) + (int)(r & ((1 << unit_log2) - 1)) : 0;
    ok[ps] = ok[ps] && uok && t < rows.L;
    tok[ps] = t < rows.L ? t : 0;
  }
  int64_t off[kPasses];
#pragma unroll
  for (int ps = 0; ps < kPasses; ++ps) {
    bool pbad = false;
    off[ps] = rows.off(b, g, tok[ps], pbad);
    ok[ps] = ok[ps] && !pbad;
    bad = bad || pbad;
  }
  float x[kPasses][16];
#pragma unroll
  for (int ps = 0; ps < kPasses; ++ps) load16<KT>(k + off[ps] + 16 * j, x[ps]);
  query_sum_to_lds<KT, D, TMAX>(q, pred_mask[b], b, g, Hq, G, T, qs);
  __syncthreads();
  float qv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) qv[i] = qs[16 * j + i];
#pragma unroll
  for (int ps = 0; ps < kPasses; ++ps) {
    const int64_t r = r0 + ps * kRowsPerPass + wave * kRowsPerWave + lane / LPR;
    const float sc = row_dot<LPR>(x[ps], qv);
    if (r < total && j == 0)
      scores[((int64_t)b * rows.Hkv + g) * total + r] = ok[ps] ? sc : -__builtin_inff();
  }
  latch_bad(status, bad);
}

template <typename KT, int D, bool PAGED>
static void launch_st(hipStream_t s, const Geom& g, const KT* q, const uint64_t* pm, const KT* k,
                      const int32_t* page_table, int unit_log2, const int32_t* cand_idx, int n_cand,
                      float* scores, uint32_t* status) {
  const int64_t total = (int64_t)n_cand << unit_log2;
  const KvRows<PAGED> rows = make_rows<PAGED>(g, page_table);
  dim3 grid((unsigned)((total + kTokensPerWg - 1) / kTokensPerWg), g.Hkv, g.B);
  if (g.T <= 32)
    hipLaunchKernelGGL((score_tokens_kernel<KT, D, 32, PAGED>), grid, dim3(256), 0, s, q, pm, k, rows, g.Hq,
                       g.G, g.T, unit_log2, cand_idx, n_cand, scores, status);
  else
    hipLaunchKernelGGL((score_tokens_kernel<KT, D, 64, PAGED>), grid, dim3(256), 0, s, q, pm, k, rows, g.Hq,
                       g.G, g.T, unit_log2, cand_idx, n_cand, scores, status);
}

template <typename KT, int D>
static void launch_st_p(hipStream_t s, const Geom& g, const KT* q, const uint64_t* pm, const KT* k,
                        const int32_t* pt, int unit_log2, const int32_t* cand_idx, int n_cand,
                        float* scores, uint32_t* status) {
  if (g.paged) launch_st<KT, D, true>(s, g, q, pm, k, pt, unit_log2, cand_idx, n_cand, scores, status);
  else launch_st<KT, D, false>(s, g, q, pm, k, pt, unit_log2, cand_idx, n_cand, scores, status);
}

hipError_t launch_score_tokens(hipStream_t s, const Geom& g, const void* q, const uint64_t* pred_mask,
                               const void* k, const int32_t* page_table, int unit_log2,
                               const int32_t* cand_idx, int n_cand, float* scores,
                               uint32_t* status) {
  const int64_t total = (int64_t)n_cand << unit_log2;
  if (total == 0) return hipSuccess;
  if (g.dtype == FDL_BF16) {
    const uint16_t* qq = static_cast<const uint16_t*>(q);
    const uint16_t* kk = static_cast<const uint16_t*>(k);
    if (g.D == 128) launch_st_p<uint16_t, 128>(s, g, qq, pred_mask, kk, page_table, unit_log2, cand_idx, n_cand, scores, status);
    else launch_st_p<uint16_t, 64>(s, g, qq, pred_mask, kk, page_table, unit_log2, cand_idx, n_cand, scores, status);
  } else {
    const float* qq = static_cast<const float*>(q);
    const float* kk = static_cast<const float*>(k);
    if (g.D == 128) launch_st_p<float, 128>(s, g, qq, pred_mask, kk, page_table, unit_log2, cand_idx, n_cand, scores, status);
    else launch_st_p<float, 64>(s, g, qq, pred_mask, kk, page_table, unit_log2, cand_idx, n_cand, scores, status);
  }
  return hipGetLastError();
}

}  // namespace fdl
