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
    int32_t* __restrict__ n_sel, uint32_t* __restrict__ status, int shared) {
  __shared__ uint32_t keys[kMaxSelN];
  __shared__ uint32_t forced[kMaxSelN / 32];
  __shared__ int hist[4 * 256];
  __shared__ int tmp[8];

  const int tid = threadIdx.x;
  const int g = blockIdx.y, b = blockIdx.z, c = blockIdx.x;
  const bool level2 = cand_idx != nullptr;
  const int n = level2 ? (1 << unit_log2) : n_units;
  const int64_t seg = (int64_t)b * Hkv + g;
  const float* sc = level2 ? scores + (seg * n_cand + c) * (int64_t)n : scores + seg * n;

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

hipError_t launch_select(hipStream_t s, const Geom& g, const float* scores, int n_units,
                         int unit_log2, const int32_t* sink_pos, const int32_t* n_sinks,
                         int max_sinks, const int32_t* cand_idx, int n_cand, int top_k,
                         int force_first, int max_sel, int32_t* sel_idx, int32_t* n_sel,
                         uint32_t* status, int shared) {
  dim3 grid(cand_idx ? n_cand : 1, g.Hkv, g.B);
  if (grid.x == 0) return hipSuccess;
  hipLaunchKernelGGL(select_kernel, grid, dim3(kSelThreads), 0, s, scores, n_units, unit_log2,
                     sink_pos, n_sinks, max_sinks, cand_idx, n_cand, top_k, force_first, max_sel,
                     g.Hkv, sel_idx, n_sel, status, shared);
  return hipGetLastError();
}

}  // namespace fdl
