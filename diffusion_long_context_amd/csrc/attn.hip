// Bidirectional attention of the decode block's queries over a gathered set of KV tokens: the
// float32 path (small workloads) and the entry that routes bf16 work to the streaming kernel.
//
// Focus-dLLM (abstract; Elamur "Summary"): the sparse step runs ordinary bidirectional attention for
// the current block's queries over only the selected KV (plus the block itself); shallow layers and
// the vanilla baseline run it over everything.  Prefilling-dLLM (abstract): the same over chunk KV
// that sits non-contiguously in a paged cache.
//
// bf16 (every head layout, contiguous or paged): attn_mha.hip.
// float32: a plain per-query-row kernel.
#include "fdl_device.h"
#include "fdl_internal.h"

namespace fdl {

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
  const int32_t* lens;   // per-sequence lengths (ragged batch), or NULL
};

// Row i of the extended list (i < T: own block row i; else list position i - T): element offset
// into k_dec / v_dec (own) or the cache, and whether it holds a token.
template <int D, bool PAGED>
__device__ __forceinline__ int64_t f32_row_off(const F32Params& p, const KvRows<PAGED>& rows, int b,
                                               int g, int i, int n_list, const int32_t* sel_row,
                                               bool& own, bool& ok, bool& bad, int Lb, int nb) {
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
    const bool uok = (unsigned)u < (unsigned)nb;
    bad = bad || (ok && !uok);
    ok = ok && uok;
    t = uok ? (u << p.unit_log2) + (ii & ((1 << p.unit_log2) - 1)) : 0;
  }
  ok = ok && t < Lb;
  t = t < Lb ? t : 0;
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
  const int Lb = seq_len(p.lens, b, p.L);   // this sequence's cached tokens
  const int nb = (Lb + (1 << p.unit_log2) - 1) >> p.unit_log2;
  int n_list;
  if (p.dense) {
    n_list = Lb;
  } else {
    int ns = p.n_sel[seg];
    ns = ns < 0 ? 0 : (ns > p.max_sel ? p.max_sel : ns);
    n_list = ns << p.unit_log2;
  }
  if (Lb == 0) n_list = 0;
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
      const int64_t off = f32_row_off<D, PAGED>(p, rows, b, g, i, n_list, sel_row, own, ok, bad, Lb, nb);
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

size_t attn_scratch_bytes(const Geom& g, int n_splits) {
  if (n_splits <= 1) return 0;
  const size_t per = (size_t)g.B * g.Hq * n_splits * 32;
  return per * g.D * sizeof(float) + per * sizeof(float2) + 256;
}

static hipError_t launch_attn_f32(hipStream_t s, const Geom& g, const void* q, const void* k,
                                  const void* v, const void* k_dec, const void* v_dec,
                                  const int32_t* page_table, const int32_t* sel_idx, const int32_t* n_sel,
                                  int max_sel, int unit_log2, int dense, void* out, uint32_t* status) {
  const int unit = 1 << unit_log2;
  const int n_units = (g.L + unit - 1) / unit;
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
  p.lens = g.lens;
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

hipError_t launch_attn(hipStream_t s, const Geom& g, const void* q, const void* k, const void* v,
                       const void* k_dec, const void* v_dec, const int32_t* page_table,
                       const int32_t* sel_idx, const int32_t* n_sel, int max_sel, int unit_log2,
                       int dense, void* out, char* scratch, int n_splits, uint32_t* tickets,
                       uint32_t* status, int n_hint, const KernelTimer* timer, bool safe) {
  if (g.dtype == FDL_BF16)
    return launch_attn_mha(s, g, q, k, v, k_dec, v_dec, page_table, sel_idx, n_sel, max_sel, unit_log2,
                           dense, out, scratch, n_splits, tickets, status, n_hint, timer, nullptr, safe);
  if (timer) (void)hipEventRecord(timer->a, s);
  const hipError_t err = launch_attn_f32(s, g, q, k, v, k_dec, v_dec, page_table, sel_idx, n_sel,
                                         max_sel, unit_log2, dense, out, status);
  if (timer) (void)hipEventRecord(timer->b, s);
  return err;
}

}  // namespace fdl