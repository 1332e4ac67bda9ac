// Keep the sinks plus the top-K units (level 1), or a chunk's anchor plus its top-K tokens
// (level 2).
//
// Focus-dLLM (abstract; Elamur "Summary"): attention sinks are always preserved and their locations
// are reused in deeper layers; the predicted queries keep only the most relevant KV.
// Prefilling-dLLM (abstract): top-K chunks, then token-level sparsity inside each chunk, whose
// leading beginning-of-sequence token serves as an anchor.
//
// One 256-thread workgroup per segment.  Scores become order-preserving 32-bit keys (-0 == +0, NaN
// lowest); a 4-pass, 8-bit radix select over the keys finds the K-th best key, and ties at that key
// go to the lower index.  Compaction is an ordered block scan, so the output comes out ascending.
// Everything is integer work on the keys, hence exact and deterministic.
#include "fdl_device.h"
#include "fdl_internal.h"

namespace fdl {

constexpr int kSelThreads = 256;
constexpr int kMaxSelN = 8192;
constexpr int kSelPerThread = kMaxSelN / kSelThreads;

// Exclusive scan of one int per thread over the 256-thread block; also returns the total.
__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  int off = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kSelThreads / 64; ++w) {
    const int t = tmp[w];
    if (w < wave) off += t;
    total += t;
  }
  __syncthreads();
  return off + incl - v;
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(
    const float* __restrict__ scores, int n_units, int unit_log2, const int32_t* __restrict__ sink_pos,
    const int32_t* __restrict__ n_sinks, int max_sinks, const int32_t* __restrict__ cand_idx,
    int n_cand, int top_k, int force_first, int max_sel, int Hkv, int32_t* __restrict__ sel_idx,
    int32_t* __restrict__ n_sel, uint32_t* __restrict__ status) {
  __shared__ uint32_t keys[kMaxSelN];
  __shared__ uint32_t forced[kMaxSelN / 32];
  __shared__ int hist[256];
  __shared__ int tmp[8];
  __shared__ uint32_t s_digit;
  __shared__ int s_above;

  const int tid = threadIdx.x;
  const int g = blockIdx.y, b = blockIdx.z, c = blockIdx.x;
  const bool level2 = cand_idx != nullptr;
  const int n = level2 ? (1 << unit_log2) : n_units;
  const int64_t seg = (int64_t)b * Hkv + g;
  const float* sc = level2 ? scores + (seg * n_cand + c) * (int64_t)n : scores + seg * n;

  for (int i = tid; i < n; i += kSelThreads) keys[i] = order_key(sc[i]);
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

  // ownership for the ordered phases: thread t owns [t*E, (t+1)*E)
  const int E = (n + kSelThreads - 1) / kSelThreads;
  const int i0 = tid * E;
  int nf_local = 0;
  for (int e = 0; e < E; ++e) {
    const int i = i0 + e;
    if (i < n && ((forced[i >> 5] >> (i & 31)) & 1u)) ++nf_local;
  }
  int n_forced;
  (void)block_excl_scan(nf_local, tmp, n_forced);
  const int n_elig = n - n_forced;
  const int kk = top_k < n_elig ? top_k : n_elig;

  // radix select of the kk-th best key among eligible elements
  uint32_t prefix = 0u, pmask = 0u;
  int rem = kk;
  const bool take_all = (kk == n_elig);
  if (kk > 0 && !take_all) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      hist[tid] = 0;
      __syncthreads();
      for (int i = tid; i < n; i += kSelThreads) {
        const uint32_t k = keys[i];
        if (((forced[i >> 5] >> (i & 31)) & 1u) == 0u && (k & pmask) == prefix)
          atomicAdd(&hist[(k >> shift) & 255u], 1);
      }
      __syncthreads();
      if (tid < 64) {
        // lane l sums bins 255-4l .. 252-4l (descending digits)
        int cnt[4], s = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          cnt[e] = hist[255 - 4 * tid - e];
          s += cnt[e];
        }
        int incl = s;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int u = __shfl_up(incl, o, 64);
          if (tid >= o) incl += u;
        }
        const uint64_t hit = __ballot(incl >= rem);
        const int first = __ffsll((unsigned long long)hit) - 1;
        if (tid == first) {
          int above = incl - s;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (above + cnt[e] >= rem) {
              s_digit = (uint32_t)(255 - 4 * tid - e);
              s_above = above;
              break;
            }
            above += cnt[e];
          }
        }
      }
      __syncthreads();
      prefix |= s_digit << shift;
      pmask |= 255u << shift;
      rem -= s_above;
      __syncthreads();
    }
  }
  const uint32_t theta = prefix;

  // ordered compaction: ties at theta go to the lowest indices
  int tie_local = 0;
  for (int e = 0; e < E; ++e) {
    const int i = i0 + e;
    if (i < n && ((forced[i >> 5] >> (i & 31)) & 1u) == 0u && keys[i] == theta) ++tie_local;
  }
  int tie_total;
  int tie_rank = block_excl_scan(tie_local, tmp, tie_total);
  uint32_t selbits = 0u;   // E <= 32
  int sel_local = 0;
  for (int e = 0; e < E; ++e) {
    const int i = i0 + e;
    if (i >= n) break;
    const bool f = ((forced[i >> 5] >> (i & 31)) & 1u) != 0u;
    bool take = f;
    if (!f && kk > 0) {
      const uint32_t k = keys[i];
      if (take_all || k > theta) {
        take = true;
      } else if (k == theta) {
        take = tie_rank < rem;
        ++tie_rank;
      }
    }
    if (take) {
      selbits |= 1u << e;
      ++sel_local;
    }
  }
  int sel_total;
  int pos = block_excl_scan(sel_local, tmp, sel_total);

  int32_t* out = sel_idx + seg * (int64_t)max_sel;
  int base = 0;
  if (level2) {
    const int per_seg = (force_first ? 1 : 0) + kk;
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
  for (int e = 0; e < E; ++e) {
    if ((selbits >> e) & 1u) {
      const int i = i0 + e;
      out[pos++] = (base < 0) ? -1 : base + i;
    }
  }
  if (tid == 0 && c == 0) {
    n_sel[seg] = level2 ? n_cand * ((force_first ? 1 : 0) + kk) : sel_total;
  }
}

hipError_t launch_select(hipStream_t s, const Geom& g, const float* scores, int n_units,
                         int unit_log2, const int32_t* sink_pos, const int32_t* n_sinks,
                         int max_sinks, const int32_t* cand_idx, int n_cand, int top_k,
                         int force_first, int max_sel, int32_t* sel_idx, int32_t* n_sel,
                         uint32_t* status) {
  dim3 grid(cand_idx ? n_cand : 1, g.Hkv, g.B);
  if (grid.x == 0) return hipSuccess;
  hipLaunchKernelGGL(select_kernel, grid, dim3(kSelThreads), 0, s, scores, n_units, unit_log2,
                     sink_pos, n_sinks, max_sinks, cand_idx, n_cand, top_k, force_first, max_sel,
                     g.Hkv, sel_idx, n_sel, status);
  return hipGetLastError();
}

}  // namespace fdl
