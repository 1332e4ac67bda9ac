// Exact top-K selection with forced members, for one workgroup over keys held in LDS; shared by the
// selection kernel and the fused select-and-attend kernel.
//
// Keys are order-preserving 32-bit images of the scores (order_key: -0 == +0, NaN lowest).  The
// forced members (sink blocks, or a chunk's anchor) are always taken; among the others the K best
// keys are taken, ties at the K-th key going to the lower index.  A 4-pass, 8-bit radix select finds
// the K-th key; an ordered block scan then emits the taken indices in ascending order.  All integer
// work, hence exact and deterministic.
#pragma once

#include "fdl_device.h"

namespace fdl {

// LDS scratch of select_core: hist[256], tmp[NT / 64], digit, above.
struct SelScratch {
  int* hist;
  int* tmp;
  uint32_t* digit;
  int* above;
};

// Exclusive scan of one int per thread over an NT-thread block; also returns the total.
template <int NT>
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
  for (int w = 0; w < NT / 64; ++w) {
    const int t = tmp[w];
    if (w < wave) off += t;
    total += t;
  }
  __syncthreads();
  return off + incl - v;
}

struct SelResult {
  int total;   // members emitted (forced + chosen)
  int kk;      // chosen among the non-forced: min(top_k, n - forced)
};

// n <= 32 * NT.  emit(pos, i) is called by the owning thread for every taken index i, with pos its
// rank in ascending order.  Every thread of the block must call this.
template <int NT, typename Emit>
__device__ SelResult select_core(const uint32_t* keys, const uint32_t* forced, int n, int top_k,
                                 const SelScratch& sc, Emit emit) {
  const int tid = threadIdx.x;
  // ownership for the ordered phases: thread t owns [t*E, (t+1)*E)
  const int E = (n + NT - 1) / NT;
  const int i0 = tid * E;
  int nf_local = 0;
  for (int e = 0; e < E; ++e) {
    const int i = i0 + e;
    if (i < n && ((forced[i >> 5] >> (i & 31)) & 1u)) ++nf_local;
  }
  int n_forced;
  (void)block_excl_scan<NT>(nf_local, sc.tmp, n_forced);
  const int n_elig = n - n_forced;
  const int kk = top_k < n_elig ? top_k : n_elig;

  // radix select of the kk-th best key among the eligible elements
  uint32_t prefix = 0u, pmask = 0u;
  int rem = kk;
  const bool take_all = (kk == n_elig);
  if (kk > 0 && !take_all) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += NT) sc.hist[i] = 0;
      __syncthreads();
      for (int i = tid; i < n; i += NT) {
        const uint32_t k = keys[i];
        if (((forced[i >> 5] >> (i & 31)) & 1u) == 0u && (k & pmask) == prefix)
          atomicAdd(&sc.hist[(k >> shift) & 255u], 1);
      }
      __syncthreads();
      if (tid < 64) {
        // lane l sums bins 255-4l .. 252-4l (descending digits)
        int cnt[4], s = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          cnt[e] = sc.hist[255 - 4 * tid - e];
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
              *sc.digit = (uint32_t)(255 - 4 * tid - e);
              *sc.above = above;
              break;
            }
            above += cnt[e];
          }
        }
      }
      __syncthreads();
      prefix |= *sc.digit << shift;
      pmask |= 255u << shift;
      rem -= *sc.above;
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
  int tie_rank = block_excl_scan<NT>(tie_local, sc.tmp, tie_total);
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
  int pos = block_excl_scan<NT>(sel_local, sc.tmp, sel_total);
  for (int e = 0; e < E; ++e)
    if ((selbits >> e) & 1u) emit(pos++, i0 + e);
  return {sel_total, kk};
}

}  // namespace fdl

namespace fdl {

// One compare-exchange step of a descending bitonic sort across the 64 lanes of a wave.
template <int K, int J>
__device__ __forceinline__ void bitonic_step(uint64_t& v, int lane) {
  const uint64_t o = ((uint64_t)lane_xor<J>((uint32_t)(v >> 32)) << 32) | lane_xor<J>((uint32_t)v);
  const bool keep_max = ((lane & J) == 0) != ((lane & K) != 0);
  v = keep_max ? (v > o ? v : o) : (v < o ? v : o);
}
template <int K, int J>
__device__ __forceinline__ void bitonic_merge(uint64_t& v, int lane) {
  bitonic_step<K, J>(v, lane);
  if constexpr (J > 1) bitonic_merge<K, J / 2>(v, lane);
}
// Sorts the wave's 64 values descending: lane l ends with the l-th largest.
template <int K = 64>
__device__ __forceinline__ void wave_sort_desc(uint64_t& v, int lane) {
  if constexpr (K > 2) wave_sort_desc<K / 2>(v, lane);
  bitonic_merge<K, K / 2>(v, lane);
}

// The same selection as select_core for n <= NT, ranked without a histogram.  Each element becomes
// one 64-bit code: (key, or all ones when forced) in the high word, the complemented index in the
// low word, so descending code order is forced first, then key descending, then index ascending --
// exactly the ranking select_core applies.  Each wave sorts its 64 codes (bitonic, in registers),
// the sorted runs meet in LDS, and a code's rank is its place in its own run plus, for every other
// run, a binary search for how many codes there are larger.  Codes ranked below nf + kk are taken;
// the taken indices are emitted in ascending order by an ordered scan.
// runs: LDS [NT] 64-bit; bits: LDS [NT / 32]; nfw: LDS [NT / 64]; tmp: LDS [NT / 64].
template <int NT, typename Emit>
__device__ SelResult select_small(const uint32_t* keys, const uint32_t* forced, int n, int top_k, uint64_t* runs,
                                  uint32_t* bits, int* nfw, int* tmp, Emit emit) {
  constexpr int NW = NT / 64;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  uint64_t v = 0;   // below every valid code
  bool f = false;
  if (t < n) {
    f = (forced[t >> 5] >> (t & 31)) & 1u;
    v = ((uint64_t)(f ? 0xFFFFFFFFu : keys[t]) << 32) | (uint64_t)(~(uint32_t)t);
  }
  const uint64_t fb = __ballot(f);
  if (lane == 0) nfw[wave] = __popcll(fb);
  wave_sort_desc(v, lane);
  runs[t] = v;
  if (t < NT / 32) bits[t] = 0u;
  __syncthreads();
  int n_forced = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) n_forced += nfw[w];
  const int n_elig = n - n_forced;
  const int kk = top_k < n_elig ? top_k : n_elig;
  // count, in every run, the entries larger than v (in its own run that is its lane); the NW binary
  // searches advance together so that their reads are in flight at once
  int lo[NW], hi[NW];
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    lo[w] = 0;
    hi[w] = 64;
  }
#pragma unroll
  for (int it = 0; it < 7; ++it) {
    uint64_t probe[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int mid = (lo[w] + hi[w]) >> 1;
      probe[w] = runs[w * 64 + (mid < 64 ? mid : 63)];
    }
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int mid = (lo[w] + hi[w]) >> 1;
      const bool gt = mid < 64 && probe[w] > v;
      lo[w] = gt ? mid + 1 : lo[w];
      hi[w] = gt ? hi[w] : mid;
    }
  }
  int rank = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) rank += lo[w];
  if (v != 0 && rank < n_forced + kk) {
    const int i = (int)(~(uint32_t)v);
    atomicOr(&bits[i >> 5], 1u << (i & 31));
  }
  __syncthreads();
  // output position of index t = taken indices below t: popcounts of the bit words (no scan)
  int pos = 0, total = 0;
#pragma unroll
  for (int w = 0; w < NT / 32; ++w) {
    const uint32_t word = bits[w];
    const int c = __popc(word);
    total += c;
    pos += (w < (t >> 5)) ? c : (w == (t >> 5) ? __popc(word & ((1u << (t & 31)) - 1u)) : 0);
  }
  const bool mine = t < n && ((bits[t >> 5] >> (t & 31)) & 1u);
  if (mine) emit(pos, t);
  return {total, kk};
}

}  // namespace fdl
