// Keep the sinks plus the top-K units (level 1), or a chunk's anchor plus its top-K tokens
// (level 2).
//
// Focus-dLLM (abstract; Elamur "Summary"): attention sinks are always preserved and their locations
// are reused in deeper layers; the predicted queries keep only the most relevant KV.
// Prefilling-dLLM (abstract): top-K chunks, then token-level sparsity inside each chunk, whose
// leading beginning-of-sequence token serves as an anchor.
//
// One 256-thread workgroup per segment; the selection itself is select_top64 (up to 256 units, top-K
// <= 64) or select_core (fdl_select.h).
#include "fdl_device.h"
#include "fdl_internal.h"
#include "fdl_select.h"

namespace fdl {

constexpr int kSelThreads = 256;
constexpr int kMaxSelN = 8192;
constexpr int kSelPerThread = kMaxSelN / kSelThreads;

// Level 1, one selection per sequence: unit i's key is that of its scores summed over the Hkv <= 32
// heads with the adjacent-pair tree (padded with +0 to 32 leaves, which changes no sum but the sign
// of a zero, and the keys take -0 as +0).
__device__ __forceinline__ float heads_tree_sum(const float* __restrict__ s, int H, int stride, int i) {
  float v[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) v[k] = k < H ? s[(int64_t)k * stride + i] : 0.f;
#pragma unroll
  for (int w = 16; w >= 1; w >>= 1)
#pragma unroll
    for (int j = 0; j < w; ++j) v[j] = v[2 * j] + v[2 * j + 1];
  return v[0];
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(
    const float* __restrict__ scores, int n_units, int unit_log2, const int32_t* __restrict__ sink_pos,
    const int32_t* __restrict__ n_sinks, int max_sinks, const int32_t* __restrict__ cand_idx,
    int n_cand, int top_k, int force_first, int max_sel, int Hkv, int32_t* __restrict__ sel_idx,
    int32_t* __restrict__ n_sel, uint32_t* __restrict__ status, int shared, const int32_t* __restrict__ lens,
    int L) {
  __shared__ uint32_t keys[kMaxSelN];
  __shared__ uint32_t forced[kMaxSelN / 32];
  __shared__ int hist[4 * 256];
  __shared__ int tmp[8];

  const int tid = threadIdx.x;
  const int g = blockIdx.y, b = blockIdx.z, c = blockIdx.x;
  const bool level2 = cand_idx != nullptr;
  // level 1 of a ragged batch: the sequence's own units; the scores rows keep n_units entries
  const int n = level2 ? (1 << unit_log2)
                       : (lens == nullptr ? n_units : (seq_len(lens, b, L) + (1 << unit_log2) - 1) >> unit_log2);
  const int64_t seg = (int64_t)b * Hkv + g;
  const float* sc = level2 ? scores + (seg * n_cand + c) * (int64_t)n : scores + seg * n_units;

  if (shared && !level2) {   // uniform; every head's workgroup derives the same keys
    const float* sb = scores + (int64_t)b * Hkv * n;
    for (int i = tid; i < n; i += kSelThreads) keys[i] = order_key(heads_tree_sum(sb, Hkv, n, i));
  } else {
    for (int i = tid; i < n; i += kSelThreads) keys[i] = order_key(sc[i]);
  }
  for (int i = tid; i < (n + 31) / 32; i += kSelThreads) forced[i] = 0u;
  __syncthreads();
  if (level2) {
    if (force_first && tid == 0) forced[0] = 1u;
  } else if (sink_pos != nullptr) {
    int ns = n_sinks[b];
    ns = ns < max_sinks ? ns : max_sinks;
    for (int s = tid; s < ns; s += kSelThreads) {
      const int p = sink_pos[(int64_t)b * max_sinks + s];
      if (p < 0) continue;
      const int u = p >> unit_log2;
      if (u < n) atomicOr(&forced[u >> 5], 1u << (u & 31));
    }
  }
  __syncthreads();

  const SelScratch scr{hist, tmp};
  int32_t* out = sel_idx + seg * (int64_t)max_sel;
  int base = 0;
  if (level2) {
    const int nf = force_first ? 1 : 0;   // the only forced member at level 2
    const int per_seg = nf + (top_k < n - nf ? top_k : n - nf);
    out += (int64_t)c * per_seg;
    const int u = cand_idx[seg * n_cand + c];
    const int n_units_all = n_units;
    if ((unsigned)u >= (unsigned)n_units_all) {
      if (tid == 0) latch(status, ST_BAD_INDEX);
      base = -1;
    } else {
      base = u << unit_log2;
    }
  }
  SelResult r;
  if (!level2 && n <= kSelThreads && top_k <= 64) {   // uniform: the sort-and-threshold form
    // runs live in keys past the n keys it reads; the counts in hist
    r = select_top64<kSelThreads>(keys, forced, n, top_k, keys + kSelThreads, hist,
                                  [&](int gpos, int, int i) {
                                    if (gpos < max_sel) out[gpos] = i;
                                  });
  } else {
    r = select_core<kSelThreads, kSelPerThread>(keys, forced, n, top_k, scr,
                                 [&](int pos, int i) { out[pos] = (base < 0) ? -1 : base + i; });
  }
  if (tid == 0 && c == 0) {
    n_sel[seg] = level2 ? n_cand * ((force_first ? 1 : 0) + r.kk) : r.total;
  }
}

// Token-granular sink retention: the attended token list of a (sequence, KV head) is the tokens
// of its selected units (ascending unit ids, each unit's valid tokens) merged with the sink tokens
// that lie outside those units (each once), ascending.  One workgroup per (b, head).  Positions
// are computed, not appended: a unit token goes to (its rank among the unit tokens) + (extra sinks
// below it), an extra sink to (unit tokens below it) + (its rank among the extra sinks); every
// position stays below units * unit + sinks <= max_tok whatever the lists hold.
constexpr int kExpandMaxSel = 4096;
constexpr int kExpandMaxSinks = 512;

__device__ __forceinline__ int count_below(const int* a, int n, int v) {   // a ascending: #{a[i] < v}
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < v) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(256) void expand_tokens_kernel(
    const int32_t* __restrict__ sel_idx, const int32_t* __restrict__ n_sel, int max_sel, int unit_log2, int L,
    int n_units, const int32_t* __restrict__ sink_pos, const int32_t* __restrict__ n_sinks, int max_sinks, int Hkv,
    int32_t* __restrict__ tok_idx, int32_t* __restrict__ n_tok, int max_tok, uint32_t* __restrict__ status) {
  __shared__ int s_blk[kExpandMaxSel];     // unit ids (invalid ones become empty units)
  __shared__ int s_pre[kExpandMaxSel + 1]; // unit tokens before unit i
  __shared__ int s_ext[kExpandMaxSinks];   // extra sinks, ascending
  __shared__ int s_raw[kExpandMaxSinks];
  __shared__ int s_keep[kExpandMaxSinks];
  __shared__ int s_next;
  const int tid = threadIdx.x, g = blockIdx.x, b = blockIdx.y;
  const int64_t seg = (int64_t)b * Hkv + g;
  const int unit = 1 << unit_log2;
  int ns = n_sel[seg];
  ns = ns < 0 ? 0 : (ns > max_sel ? max_sel : ns);
  bool bad = false;
  for (int i = tid; i < ns; i += 256) {
    const int u = sel_idx[seg * max_sel + i];
    const bool ok = (unsigned)u < (unsigned)n_units;
    bad = bad || !ok;
    s_blk[i] = ok ? u : -1;
  }
  int nk = sink_pos != nullptr ? n_sinks[b] : 0;
  nk = nk < 0 ? 0 : (nk > max_sinks ? max_sinks : nk);
  for (int i = tid; i < nk; i += 256) s_raw[i] = sink_pos[(int64_t)b * max_sinks + i];
  __syncthreads();
  if (tid == 0) {   // exclusive prefix of the unit lengths (at most kExpandMaxSel serial adds)
    int acc = 0;
    for (int i = 0; i < ns; ++i) {
      s_pre[i] = acc;
      const int u = s_blk[i];
      const int len = u < 0 ? 0 : ((L - (u << unit_log2)) < unit ? (L - (u << unit_log2)) : unit);
      acc += len;
    }
    s_pre[ns] = acc;
    s_next = 0;
  }
  __syncthreads();
  // extra sinks: valid, first occurrence, outside every selected unit; then each kept one goes to
  // its rank among the kept ones (their values are distinct)
  for (int i = tid; i < nk; i += 256) {
    const int t = s_raw[i];
    bool keep = t >= 0 && t < L;
    for (int j = 0; keep && j < i; ++j) keep = s_raw[j] != t;
    if (keep) {
      const int u = t >> unit_log2;
      for (int j = 0; keep && j < ns; ++j) keep = s_blk[j] != u;
    }
    s_keep[i] = keep ? 1 : 0;
  }
  __syncthreads();
  for (int i = tid; i < nk; i += 256) {
    if (!s_keep[i]) continue;
    const int t = s_raw[i];
    int rank = 0;
    for (int j = 0; j < nk; ++j) rank += (s_keep[j] && s_raw[j] < t) ? 1 : 0;
    s_ext[rank] = t;
    atomicAdd(&s_next, 1);
  }
  __syncthreads();
  const int n_ext = s_next;
  const int total_units = s_pre[ns];
  int32_t* out = tok_idx + seg * (int64_t)max_tok;
  for (int idx = tid; idx < total_units; idx += 256) {
    int lo = 0, hi = ns - 1;   // the unit holding token idx: the last i with s_pre[i] <= idx
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_pre[mid] <= idx) lo = mid;
      else hi = mid - 1;
    }
    const int t = (s_blk[lo] << unit_log2) + (idx - s_pre[lo]);
    out[idx + count_below(s_ext, n_ext, t)] = t;
  }
  for (int e = tid; e < n_ext; e += 256) {
    const int t = s_ext[e];
    // unit tokens below t: the units (ascending) whose id is below t's unit
    int lo = 0, hi = ns;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (s_blk[mid] < (t >> unit_log2)) lo = mid + 1;
      else hi = mid;
    }
    out[s_pre[lo] + e] = t;
  }
  if (tid == 0) n_tok[seg] = total_units + n_ext;
  latch_bad(status, bad);
}

bool expand_tokens_ok(int max_sel, int max_sinks) {
  return max_sel <= kExpandMaxSel && max_sinks <= kExpandMaxSinks;
}

hipError_t launch_expand_tokens(hipStream_t s, const Geom& g, const int32_t* sel_idx, const int32_t* n_sel,
                                int max_sel, int unit_log2, const int32_t* sink_pos, const int32_t* n_sinks,
                                int max_sinks, int32_t* tok_idx, int32_t* n_tok, int max_tok, uint32_t* status) {
  const int n_units = (g.L + (1 << unit_log2) - 1) >> unit_log2;
  hipLaunchKernelGGL(expand_tokens_kernel, dim3(g.Hkv, g.B), dim3(256), 0, s, sel_idx, n_sel, max_sel, unit_log2,
                     g.L, n_units, sink_pos, n_sinks, max_sinks, g.Hkv, tok_idx, n_tok, max_tok, status);
  return hipGetLastError();
}

hipError_t launch_select(hipStream_t s, const Geom& g, const float* scores, int n_units,
                         int unit_log2, const int32_t* sink_pos, const int32_t* n_sinks,
                         int max_sinks, const int32_t* cand_idx, int n_cand, int top_k,
                         int force_first, int max_sel, int32_t* sel_idx, int32_t* n_sel,
                         uint32_t* status, int shared) {
  dim3 grid(cand_idx ? n_cand : 1, g.Hkv, g.B);
  if (grid.x == 0) return hipSuccess;
  hipLaunchKernelGGL(select_kernel, grid, dim3(kSelThreads), 0, s, scores, n_units, unit_log2,
                     sink_pos, n_sinks, max_sinks, cand_idx, n_cand, top_k, force_first, max_sel,
                     g.Hkv, sel_idx, n_sel, status, shared, cand_idx == nullptr ? g.lens : nullptr, g.L);
  return hipGetLastError();
}

}  // namespace fdl
