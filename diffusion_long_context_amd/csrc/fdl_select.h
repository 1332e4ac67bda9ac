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

// Inclusive prefix sum along each 16-lane row (DPP row shifts by 1, 2, 4, 8; lanes without a source
// add 0).
__device__ __forceinline__ int row_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);
  return x;
}

// Inclusive prefix sum over the 64 lanes: row scans, then each row adds the totals of the rows
// before it (read from lanes 15, 31, 47).
__device__ __forceinline__ int wave_incl_scan(int x) {
  const int incl = row_incl_scan(x);
  const int r0 = __builtin_amdgcn_readlane(incl, 15), r1 = __builtin_amdgcn_readlane(incl, 31),
            r2 = __builtin_amdgcn_readlane(incl, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return incl + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

// LDS scratch of select_core: hist[4 * 256] (one histogram per radix pass), tmp[NT / 64].
struct SelScratch {
  int* hist;
  int* tmp;
};

// Exclusive scan of one int per thread over an NT-thread block; also returns the total.  One
// barrier; tmp must not be written again before a later barrier.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int& total) {
  constexpr int NW = NT / 64;
  static_assert(NW <= 16, "wave totals in one row of lanes");
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int incl = wave_incl_scan(v);
  if (lane == 63) tmp[wave] = incl;
  block_sync_lds();
  const int wt = row_incl_scan(lane < NW ? tmp[lane] : 0);
  total = __builtin_amdgcn_readlane(wt, NW - 1);
  const int off = wave > 0 ? __builtin_amdgcn_readlane(wt, wave > 0 ? wave - 1 : 0) : 0;
  return off + incl - v;
}

struct SelResult {
  int total;   // members emitted (forced + chosen)
  int kk;      // chosen among the non-forced: min(top_k, n - forced)
};

// n <= EMAX * NT (EMAX a multiple of 4; keys and forced hold at least EMAX * NT elements).
// emit(pos, i) is called by the owning thread for every taken index i, with pos its rank in
// ascending order.  Every thread of the block must call this.
// Thread t owns the E4 consecutive elements from t E4 (E4 = ceil(n / NT) rounded up to 4) and holds
// their keys and forced bits in registers for every phase.  Barriers: one to clear the histograms,
// one per radix pass, one for the ordered scan.  Every wave counts the forced members and finds each
// pass's digit itself (the same integers in every wave), so nothing is broadcast; each pass has a
// histogram of its own, so none is cleared in between.
template <int NT, int EMAX, typename Emit>
__device__ SelResult select_core(const uint32_t* keys, const uint32_t* forced, int n, int top_k,
                                 const SelScratch& sc, Emit emit) {
  static_assert(EMAX % 4 == 0 && EMAX <= 32, "register-held elements");
  const int tid = threadIdx.x, lane = tid & 63;
  if (n <= 0) return {0, 0};   // uniform
  const int E4 = (((n + NT - 1) / NT) + 3) & ~3;
  const int i0 = tid * E4;
  const int n_words = (n + 31) / 32;
  int fl = 0;
  for (int w = lane; w < n_words; w += 64) {
    uint32_t word = forced[w];
    if (w == n_words - 1 && (n & 31) != 0) word &= (1u << (n & 31)) - 1u;
    fl += __popc(word);
  }
  const int n_forced = __builtin_amdgcn_readlane(wave_incl_scan(fl), 63);
  const int n_elig = n - n_forced;
  const int kk = top_k < n_elig ? top_k : n_elig;

  // this thread's keys and forced bits (bit e: element i0 + e); elements past n are not live
  uint32_t kv[EMAX];
#pragma unroll
  for (int c = 0; c < EMAX / 4; ++c) {
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (4 * c < E4) v = *reinterpret_cast<const uint4*>(keys + i0 + 4 * c);   // uniform bound
    kv[4 * c] = v.x;
    kv[4 * c + 1] = v.y;
    kv[4 * c + 2] = v.z;
    kv[4 * c + 3] = v.w;
  }
  const int wi = (i0 >> 5) < n_words - 1 ? (i0 >> 5) : n_words - 1;
  const int wj = wi + 1 < n_words ? wi + 1 : n_words - 1;
  const uint64_t fw = (uint64_t)forced[wi] | ((uint64_t)forced[wj] << 32);
  const int live_n = n - i0 < 0 ? 0 : (n - i0 > E4 ? E4 : n - i0);
  const uint32_t live = live_n >= 32 ? 0xFFFFFFFFu : ((1u << live_n) - 1u);
  const uint32_t fb = (uint32_t)(fw >> (i0 & 31)) & live;
  const uint32_t elig = live & ~fb;

  // radix select of the kk-th best key among the eligible elements
  uint32_t prefix = 0u, pmask = 0u;
  int rem = kk;
  const bool take_all = (kk == n_elig);
  if (kk > 0 && !take_all) {   // uniform
    for (int i = tid; i < 4 * 256; i += NT) sc.hist[i] = 0;
    block_sync_lds();
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      int* h = sc.hist + 256 * pass;
      // in chunks of 4 owned elements, skipping the chunks past E4 (a uniform test)
#pragma unroll
      for (int c = 0; c < EMAX / 4; ++c) {
        if (4 * c >= E4) break;
#pragma unroll
        for (int e = 4 * c; e < 4 * c + 4; ++e)
          if (((elig >> e) & 1u) && (kv[e] & pmask) == prefix) atomicAdd(&h[(kv[e] >> shift) & 255u], 1);
      }
      block_sync_lds();
      // lane l holds bins 255-4l .. 252-4l (descending digits); the first lane whose running count
      // reaches rem holds the digit
      int cnt[4], sl = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        cnt[e] = h[255 - 4 * lane - e];
        sl += cnt[e];
      }
      const int incl = wave_incl_scan(sl);
      const uint64_t hit = __ballot(incl >= rem);
      const int first = __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)hit) - 1);
      // within the lane, the first of its bins (descending) where the count reaches rem, and the
      // members above that bin
      int a = incl - sl, found = -1, above = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (found < 0 && a + cnt[e] >= rem) {
          found = e;
          above = a;
        }
        a += cnt[e];
      }
      const int dig = 255 - 4 * lane - (found < 0 ? 0 : found);
      const uint32_t digit = (uint32_t)__builtin_amdgcn_readlane(dig, first);
      prefix |= digit << shift;
      pmask |= 255u << shift;
      rem -= __builtin_amdgcn_readlane(above, first);
    }
  }
  const uint32_t theta = prefix;

  // ordered emission: per thread, members above theta (and forced ones) and ties at theta, counted
  // together in one scan (16 bits each); ties go to the lowest indices
  uint32_t above_m = fb, tie_m = 0u;
  if (kk > 0) {   // uniform
#pragma unroll
    for (int c = 0; c < EMAX / 4; ++c) {
      if (4 * c >= E4) break;
#pragma unroll
      for (int e = 4 * c; e < 4 * c + 4; ++e) {
        const bool el = (elig >> e) & 1u;
        above_m |= (el && (take_all || kv[e] > theta)) ? 1u << e : 0u;
        tie_m |= (el && !take_all && kv[e] == theta) ? 1u << e : 0u;
      }
    }
  }
  int tot;
  const int ex = block_excl_scan<NT>(__popc(above_m) | (__popc(tie_m) << 16), sc.tmp, tot);
  const int tr = ex >> 16;
  // ties of this thread still taken: the lowest ones, up to rem - tr
  const int my_ties = rem - tr <= 0 ? 0 : rem - tr;
  uint32_t take_m = above_m;
  uint32_t tm = tie_m;
  for (int c = 0; c < my_ties && tm != 0u; ++c) {
    take_m |= tm & (0u - tm);   // lowest remaining tie
    tm &= tm - 1u;
  }
  int pos = (ex & 0xFFFF) + (tr < rem ? tr : rem);
  for (uint32_t m = take_m; m != 0u; m &= m - 1u) emit(pos++, i0 + __builtin_ctz(m));
  const int tot_ties = tot >> 16;
  return {(tot & 0xFFFF) + (tot_ties < rem ? tot_ties : rem), kk};
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
  block_sync_lds();
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
  block_sync_lds();
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

// 32-bit descending bitonic sort across the wave: lane l ends with the l-th largest value.
// Lanes that keep the larger value at step (K, J) of the network, as a 64-bit lane mask.
constexpr uint64_t keep_max_mask(int K, int J) {
  uint64_t m = 0;
  for (int l = 0; l < 64; ++l)
    if (((l & J) == 0) != ((l & K) != 0)) m |= 1ull << l;
  return m;
}

// v = m[lane] ? a : b, with m a wave-uniform lane mask (one VALU select on a scalar pair).
__device__ __forceinline__ uint32_t select_lanes(uint64_t m, uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(b), "v"(a), "s"(m));
  return r;
}

// hi / lo = max / min of v and the value of lane (lane ^ J).  For J = 1, 2, 8 the partner's value is
// read through a DPP operand of the max and the min themselves; J = 4 takes one DPP move first
// (half-row mirror, then the quad reversal in the operand: lane ^ 7 ^ 3); 16 and 32 use the row /
// half swaps.  The leading s_nop covers the wait states a DPP read of a just-written VGPR needs.
template <int J>
__device__ __forceinline__ void xor_minmax(uint32_t v, uint32_t& hi, uint32_t& lo) {
  if constexpr (J == 1) {
    asm("s_nop 1\n\tv_max_u32_dpp %0, %2, %2 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_min_u32_dpp %1, %2, %2 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
        : "=&v"(hi), "=&v"(lo) : "v"(v));
  } else if constexpr (J == 2) {
    asm("s_nop 1\n\tv_max_u32_dpp %0, %2, %2 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_min_u32_dpp %1, %2, %2 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf"
        : "=&v"(hi), "=&v"(lo) : "v"(v));
  } else if constexpr (J == 8) {
    asm("s_nop 1\n\tv_max_u32_dpp %0, %2, %2 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_min_u32_dpp %1, %2, %2 row_ror:8 row_mask:0xf bank_mask:0xf"
        : "=&v"(hi), "=&v"(lo) : "v"(v));
  } else if constexpr (J == 4) {
    uint32_t t;
    asm("s_nop 1\n\tv_mov_b32_dpp %2, %3 row_half_mirror row_mask:0xf bank_mask:0xf\n\ts_nop 1\n\t"
        "v_max_u32_dpp %0, %2, %3 quad_perm:[3,2,1,0] row_mask:0xf bank_mask:0xf\n\t"
        "v_min_u32_dpp %1, %2, %3 quad_perm:[3,2,1,0] row_mask:0xf bank_mask:0xf"
        : "=&v"(hi), "=&v"(lo), "=&v"(t) : "v"(v));
  } else {
    static_assert(J == 16 || J == 32, "lane distance");
    // after a swap of v with itself the lanes with bit J set hold the partner in the first result,
    // the others in the second
    const auto r = J == 16 ? __builtin_amdgcn_permlane16_swap(v, v, false, false)
                           : __builtin_amdgcn_permlane32_swap(v, v, false, false);
    constexpr uint64_t up = J == 16 ? 0xFFFF0000FFFF0000ull : 0xFFFFFFFF00000000ull;
    const uint32_t o = select_lanes(up, r[0], r[1]);
    hi = v > o ? v : o;
    lo = v < o ? v : o;
  }
}

template <int K, int J>
__device__ __forceinline__ void bitonic_step32(uint32_t& v) {
  uint32_t hi, lo;
  xor_minmax<J>(v, hi, lo);
  v = select_lanes(keep_max_mask(K, J), hi, lo);
}
template <int K, int J>
__device__ __forceinline__ void bitonic_merge32(uint32_t& v) {
  bitonic_step32<K, J>(v);
  if constexpr (J > 1) bitonic_merge32<K, J / 2>(v);
}
template <int K = 64>
__device__ __forceinline__ void wave_sort_desc32(uint32_t& v) {
  if constexpr (K > 2) wave_sort_desc32<K / 2>(v);
  bitonic_merge32<K, K / 2>(v);
}


// The same selection as select_core for n <= NT and top_k <= 64, found through a threshold.  The
// eligible keys (forced units and threads past n count as 0, which no eligible key is below) are
// sorted within each wave; a tournament then keeps the 64 largest: two descending runs A and B
// give the 64 largest of their union as the bitonic sequence max(A[l], B[63 - l]), which the last
// six steps of the sort put in order.  The kk-th largest value theta is the threshold: every
// eligible unit with a larger key is taken, and of those equal to theta the lowest-indexed ones, as
// many as are still missing.  Forced units are always taken.  Ballots count all three kinds per
// wave, so the output positions need no further pass: emit(gpos, lpos, i) gets unit i's place in
// the ascending list of every taken unit (gpos) and in the list of the forced units (ascending)
// followed by the chosen ones (ascending) (lpos).
// runs: LDS [NT - 64] words; cnt: LDS [2 * NT / 64 + 1] ints.
template <int NT, typename Emit>
__device__ SelResult select_top64(const uint32_t* keys, const uint32_t* forced, int n, int top_k, uint32_t* runs,
                                  int* cnt, Emit emit) {
  constexpr int NW = NT / 64;
  static_assert(NW >= 1 && (NW & (NW - 1)) == 0 && NW <= 16, "power-of-two wave count, one row of lanes");
  const int t = threadIdx.x, lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
  int* n_f = cnt;               // [NW] forced units per wave
  int* n_gt = cnt + NW;         // [NW] eligible keys above theta | equal to theta << 16
  int* theta_w = cnt + 2 * NW;  // [1]
  const bool valid = t < n;
  const bool f = valid && ((forced[t >> 5] >> (t & 31)) & 1u) != 0u;
  const bool elig = valid && !f;
  const uint32_t key = valid ? keys[t] : 0u;
  uint32_t v = elig ? key : 0u;
  const uint64_t fmask = __ballot(f);
  if (lane == 0) n_f[wave] = __popcll(fmask);
  wave_sort_desc32(v);
  // tournament: at each level waves [half, 2 half) hand their runs to waves [0, half); every level
  // has slots of its own, so a level's writers never meet the previous level's readers
  uint32_t* slots = runs;
#pragma unroll
  for (int half = NW / 2; half >= 1; half >>= 1) {
    if (wave >= half && wave < 2 * half) slots[(wave - half) * 64 + lane] = v;
    block_sync_lds();
    if (wave < half) {
      const uint32_t o = slots[wave * 64 + 63 - lane];
      v = v > o ? v : o;
      bitonic_merge32<64, 32>(v);
    }
    slots += half * 64;
  }
  if constexpr (NW == 1) block_sync_lds();   // n_f
  // Per-wave counts are combined lane-parallel: lane w < NW holds wave w's count and a scan along
  // the 16-lane row gives the prefixes (rather than every wave adding all NW counts in scalar code).
  const int fl = lane < NW ? n_f[lane] : 0;
  const int f_incl = row_incl_scan(fl);
  const int n_forced = __builtin_amdgcn_readlane(f_incl, NW - 1);
  const int n_elig = n - n_forced;
  const int kk = top_k < n_elig ? top_k : n_elig;
  if (wave == 0) {
    // with nothing to take the threshold is all ones, which no key reaches (+inf's key is below)
    const uint32_t th = (uint32_t)__builtin_amdgcn_readlane((int)v, kk > 0 ? kk - 1 : 0);
    if (lane == 0) *theta_w = kk > 0 ? (int)th : -1;
  }
  block_sync_lds();
  const uint32_t theta = (uint32_t)__builtin_amdgcn_readfirstlane(*theta_w);
  const bool gt = elig && key > theta, eq = elig && key == theta;
  const uint64_t gmask = __ballot(gt), emask = __ballot(eq);
  if (lane == 0) n_gt[wave] = __popcll(gmask) | (__popcll(emask) << 16);
  block_sync_lds();
  const int both = lane < NW ? n_gt[lane] : 0;
  const int gtl = both & 0xFFFF, eql = both >> 16;
  const int gt_incl = row_incl_scan(gtl), eq_incl = row_incl_scan(eql);
  const int rem = kk - __builtin_amdgcn_readlane(gt_incl, NW - 1);   // ties still to take, lowest index first
  int tw = rem - (eq_incl - eql);   // wave (lane)'s share of them
  tw = tw < 0 ? 0 : (tw > eql ? eql : tw);
  const int cw = gtl + tw;
  const int c_incl = row_incl_scan(cw);
  const int f_base = __builtin_amdgcn_readlane(f_incl - fl, wave);
  const int c_base = __builtin_amdgcn_readlane(c_incl - cw, wave);
  const int my_ties = __builtin_amdgcn_readlane(tw, wave);
  const uint64_t below = (1ull << lane) - 1ull;
  const bool chosen = gt || (eq && __popcll(emask & below) < my_ties);
  const uint64_t cmask = __ballot(chosen);
  if (f || chosen) {
    const int fr = f_base + __popcll(fmask & below), cr = c_base + __popcll(cmask & below);
    emit(fr + cr, f ? fr : n_forced + cr, t);
  }
  return {n_forced + (kk > 0 ? kk : 0), kk};
}

}  // namespace fdl
