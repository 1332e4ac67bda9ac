// Pinned float32 pieces of the scoring path, shared by the scoring kernels and the fused
// select-and-attend kernel so that both produce the same bits.
//
// Every sum is the adjacent-pair tree (operands zero-padded to a power of two; level by level,
// element 2j plus element 2j+1), every product is rounded to float32 before it is added, and nothing
// is contracted into a fused multiply-add: each function turns contraction off for its own body.
#pragma once

#include "fdl_device.h"

namespace fdl {

template <typename QT>
__device__ __forceinline__ float load_q(const QT* q);
template <>
__device__ __forceinline__ float load_q<uint16_t>(const uint16_t* q) {
  return bf16_bits_to_f32(*q);
}
template <>
__device__ __forceinline__ float load_q<float>(const float* q) {
  return *q;
}

__device__ __forceinline__ int pow2_ceil(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// TMAX: 32 or 64, a compile-time bound on T.
template <typename QT, int D, int TMAX>
__device__ __forceinline__ void query_sum_to_lds(const QT* __restrict__ q, uint64_t pred, int b, int g,
                                                 int Hq, int G, int T, float* qs_lds) {
#pragma clang fp contract(off)
  const int d = threadIdx.x;
  if (d >= D) return;
  const int T2 = pow2_ceil(T);
  const int G2 = pow2_ceil(G);
  float hv[8];
  for (int j = 0; j < 8; ++j) {
    hv[j] = 0.f;
    if (j < G) {   // uniform
      const int h = g * G + j;
      const QT* qh = q + ((int64_t)b * Hq + h) * T * D + d;
      float a[TMAX];
#pragma unroll
      for (int p = 0; p < TMAX; ++p) a[p] = load_q<QT>(qh + (int64_t)(p < T ? p : T - 1) * D);
      // keep the scheduler from interleaving the tree with the loads: all TMAX loads must be in
      // flight together, not issued pairwise behind waits
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int p = 0; p < TMAX; ++p)
        if (!(p < T && ((pred >> p) & 1ull))) a[p] = 0.f;
#pragma unroll
      for (int lvl = 0; lvl < 6; ++lvl) {
        if ((TMAX >> (lvl + 1)) >= 1 && (1 << lvl) < T2) {
#pragma unroll
          for (int i = 0; i < (TMAX >> (lvl + 1)); ++i) a[i] = a[2 * i] + a[2 * i + 1];
        }
      }
      hv[j] = a[0];
    }
  }
#pragma unroll
  for (int lvl = 0; lvl < 3; ++lvl) {
    if ((1 << lvl) < G2) {
#pragma unroll
      for (int i = 0; i < (4 >> lvl); ++i) hv[i] = hv[2 * i] + hv[2 * i + 1];
    }
  }
  qs_lds[d] = hv[0];
}

// query_sum_to_lds for bf16 queries with every thread of an NT-thread block loading: the TMAX rows
// of each of the G (<= GMAX) heads go to stage [GMAX][TMAX][D] (bf16 bits, LDS) as 16-byte chunks in
// one round trip, then the block's threads build the same trees from LDS.  Same bits.  Two halves, so
// that a caller can issue other loads between them: qsum_grouped_issue loads this thread's chunks
// into registers; qsum_grouped_finish (every thread calls it) stages them and sums.
template <int D, int TMAX, int NT, int GMAX>
struct QsumGrouped {
  static constexpr int CPR = D / 8;                  // 16-byte chunks per row
  static constexpr int CH = GMAX * TMAX * CPR;       // chunks of the stage
  static constexpr int PER = CH / NT;
  static_assert(GMAX == 8, "the head tree has three levels");
  static_assert(CH % NT == 0, "every thread moves the same number of chunks");
  uint4 v[PER];
};

// q: the sequence's queries [Hq][T][D]; g0: the group's first query head.
template <int D, int TMAX, int NT, int GMAX>
__device__ __forceinline__ void qsum_grouped_issue(const uint16_t* __restrict__ q, int g0, int G, int T,
                                                   QsumGrouped<D, TMAX, NT, GMAX>& st) {
  using S = QsumGrouped<D, TMAX, NT, GMAX>;
  const int t = threadIdx.x;
#pragma unroll
  for (int k = 0; k < S::PER; ++k) {
    const int c = k * NT + t;
    const int j = c / (TMAX * S::CPR), p = (c / S::CPR) % TMAX, ch = c % S::CPR;
    const int jj = j < G ? j : G - 1;   // heads past G read a valid row and are never used
    st.v[k] = *reinterpret_cast<const uint4*>(q + ((int64_t)(g0 + jj) * T + (p < T ? p : T - 1)) * D + ch * 8);
  }
}

// The trees over a filled stage ([GMAX][TMAX][D] bf16, visible to every thread), by all NT threads:
// thread t takes the dimension pair (2c, 2c + 1), c = t % (D / 2), of heads t / (D / 2), + NT / (D / 2),
// ... (one 32-bit read per slot) and builds each head's adjacent-pair tree over the TMAX slots; once
// every thread's stage reads are done the head sums take the stage's place, and threads d < D build
// the tree over the heads.  The additions and their order per dimension are those of one thread
// running both trees; spreading the heads over the block's threads only shortens the chain of reads.
// Every thread must call it (two barriers); qs_lds is complete after the caller's next barrier.
template <int D, int TMAX, int NT, int GMAX>
__device__ __forceinline__ void qsum_grouped_tree(uint64_t pred, int G, int T, uint16_t* stage, float* qs_lds) {
#pragma clang fp contract(off)
  constexpr int PAIRS = D / 2;
  static_assert(NT % PAIRS == 0 && GMAX == 8, "a whole number of heads per pass; the head tree is over 8");
  constexpr int JSTEP = NT / PAIRS;
  constexpr int JPER = (GMAX + JSTEP - 1) / JSTEP;
  const int t = threadIdx.x;
  const int c = t % PAIRS, j0 = t / PAIRS;
  const int T2 = pow2_ceil(T);
  const int G2 = pow2_ceil(G);
  const uint32_t* st32 = reinterpret_cast<const uint32_t*>(stage);
  float s0[JPER], s1[JPER];
#pragma unroll
  for (int k = 0; k < JPER; ++k) {
    const int j = j0 + k * JSTEP;
    const int jr = j < GMAX ? j : 0;
    // every read is unconditional (a masked read becomes a branch and a wait per element), and the
    // head's reads all go out before its tree starts
    uint32_t raw[TMAX];
#pragma unroll
    for (int p = 0; p < TMAX; ++p) raw[p] = st32[(jr * TMAX + p) * PAIRS + c];
    __builtin_amdgcn_sched_barrier(0);
    float a0[TMAX], a1[TMAX];
#pragma unroll
    for (int p = 0; p < TMAX; ++p) {
      const bool keep = j < G && p < T && ((pred >> p) & 1ull);
      a0[p] = keep ? bf16_bits_to_f32(raw[p] & 0xFFFFu) : 0.f;
      a1[p] = keep ? bf16_bits_to_f32(raw[p] >> 16) : 0.f;
    }
#pragma unroll
    for (int lvl = 0; lvl < 6; ++lvl) {
      if ((TMAX >> (lvl + 1)) >= 1 && (1 << lvl) < T2) {
#pragma unroll
        for (int i = 0; i < (TMAX >> (lvl + 1)); ++i) {
          a0[i] = a0[2 * i] + a0[2 * i + 1];
          a1[i] = a1[2 * i] + a1[2 * i + 1];
        }
      }
    }
    s0[k] = a0[0];
    s1[k] = a1[0];
  }
  block_sync_lds();   // every stage read is done: the head sums take the stage's place
  float* hs = reinterpret_cast<float*>(stage);
#pragma unroll
  for (int k = 0; k < JPER; ++k) {
    const int j = j0 + k * JSTEP;
    if (j < GMAX) *reinterpret_cast<float2*>(hs + j * D + 2 * c) = make_float2(s0[k], s1[k]);
  }
  block_sync_lds();
  if (t < D) {
    float hv[GMAX];
#pragma unroll
    for (int j = 0; j < GMAX; ++j) hv[j] = hs[j * D + t];
#pragma unroll
    for (int lvl = 0; lvl < 3; ++lvl) {
      if ((1 << lvl) < G2) {
#pragma unroll
        for (int i = 0; i < (4 >> lvl); ++i) hv[i] = hv[2 * i] + hv[2 * i + 1];
      }
    }
    qs_lds[t] = hv[0];
  }
}

template <int D, int TMAX, int NT, int GMAX>
__device__ __forceinline__ void qsum_grouped_finish(const QsumGrouped<D, TMAX, NT, GMAX>& st, uint64_t pred, int G,
                                                    int T, uint16_t* stage, float* qs_lds) {
  using S = QsumGrouped<D, TMAX, NT, GMAX>;
  const int t = threadIdx.x;
#pragma unroll
  for (int k = 0; k < S::PER; ++k) *reinterpret_cast<uint4*>(stage + (k * NT + t) * 8) = st.v[k];
  block_sync_lds();
  qsum_grouped_tree<D, TMAX, NT, GMAX>(pred, G, T, stage, qs_lds);
}

// The same stage filled by LDS fetches (no registers held while they fly): chunk c = k NT + t lands
// at stage + 8 c.  The caller must wait for its own fetches (vector-memory count) and then meet the
// other waves at a barrier before qsum_grouped_tree.
template <int D, int TMAX, int NT, int GMAX>
__device__ __forceinline__ void qsum_grouped_fetch(const uint16_t* __restrict__ q, int g0, int G, int T,
                                                   uint16_t* stage) {
  using S = QsumGrouped<D, TMAX, NT, GMAX>;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
#pragma unroll
  for (int k = 0; k < S::PER; ++k) {
    const int c = k * NT + wave * 64 + lane;
    const int j = c / (TMAX * S::CPR), p = (c / S::CPR) % TMAX, ch = c % S::CPR;
    const int jj = j < G ? j : G - 1;
    const void* src = q + ((int64_t)(g0 + jj) * T + (p < T ? p : T - 1)) * D + ch * 8;
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(stage + (k * NT + wave * 64) * 8),
                                     16, 0, 0);
  }
}

// query_sum_to_lds for one query head (G = 1) with every thread of an NT-thread block loading: row
// p of the head's queries is read as D / 8 sixteen-byte chunks, masked (p predicted and p < T) into
// qbuf [TMAX][D] float32 in LDS, and threads d < D then build the same adjacent-pair tree over the
// TMAX rows as query_sum_to_lds.  Same bits; one round trip instead of TMAX narrow loads per thread.
// Two halves, so that a caller can issue other loads between them: qsum_g1_issue loads this thread's
// chunks into registers; qsum_g1_finish (every thread calls it) stages them and sums.
template <int D, int TMAX, int NT>
struct QsumG1 {
  static constexpr int CPR = D / 8;   // 16-byte chunks per row
  static constexpr int PER = (TMAX * CPR + NT - 1) / NT;
  static_assert(TMAX * CPR <= NT || (TMAX * CPR) % NT == 0, "chunking");
  uint4 v[PER];
};

template <int D, int TMAX, int NT>
__device__ __forceinline__ void qsum_g1_issue(const uint16_t* __restrict__ qh, int T, QsumG1<D, TMAX, NT>& st) {
  using S = QsumG1<D, TMAX, NT>;
  const int t = threadIdx.x;
#pragma unroll
  for (int k = 0; k < S::PER; ++k) {
    const int c = k * NT + t;
    const int p = c / S::CPR, ch = c % S::CPR;
    st.v[k] = make_uint4(0u, 0u, 0u, 0u);
    if (c < TMAX * S::CPR) st.v[k] = *reinterpret_cast<const uint4*>(qh + (int64_t)(p < T ? p : T - 1) * D + ch * 8);
  }
}

template <int D, int TMAX, int NT>
__device__ __forceinline__ void qsum_g1_finish(const QsumG1<D, TMAX, NT>& st, uint64_t pred, int T, float* qbuf,
                                               float* qs_lds) {
#pragma clang fp contract(off)
  using S = QsumG1<D, TMAX, NT>;
  const int t = threadIdx.x;
#pragma unroll
  for (int k = 0; k < S::PER; ++k) {
    const int c = k * NT + t;
    if (c < TMAX * S::CPR) {
      const int p = c / S::CPR, ch = c % S::CPR;
      const bool keep = p < T && ((pred >> p) & 1ull);
      const uint32_t w[4] = {st.v[k].x, st.v[k].y, st.v[k].z, st.v[k].w};
      float* dst = qbuf + p * D + ch * 8;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dst[2 * e] = keep ? bf16_bits_to_f32(w[e] & 0xFFFFu) : 0.f;
        dst[2 * e + 1] = keep ? bf16_bits_to_f32(w[e] >> 16) : 0.f;
      }
    }
  }
  block_sync_lds();
  if (t < D) {
    const int T2 = pow2_ceil(T);
    float a[TMAX];
#pragma unroll
    for (int p = 0; p < TMAX; ++p) a[p] = qbuf[p * D + t];
#pragma unroll
    for (int lvl = 0; lvl < 6; ++lvl) {
      if ((TMAX >> (lvl + 1)) >= 1 && (1 << lvl) < T2) {
#pragma unroll
        for (int i = 0; i < (TMAX >> (lvl + 1)); ++i) a[i] = a[2 * i] + a[2 * i + 1];
      }
    }
    qs_lds[t] = a[0];
  }
}

// Pinned dot product of one row: lane j of an LPR-lane team holds dimensions [16j, 16j+16).
// Local tree over its 16 products (levels 0-3), then xor butterflies across the team.
template <int LPR>
__device__ __forceinline__ float row_dot(const float (&x)[16], const float (&qv)[16]) {
#pragma clang fp contract(off)
  float p[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) p[i] = x[i] * qv[i];
#pragma unroll
  for (int w = 8; w >= 1; w /= 2) {
#pragma unroll
    for (int i = 0; i < w; ++i) p[i] = p[2 * i] + p[2 * i + 1];
  }
  float s = p[0];
  // cross-lane tree levels; a + b and b + a round alike, so both lanes of a pair hold the same sum
  if constexpr (LPR > 1) s = s + __uint_as_float(lane_xor<1>(__float_as_uint(s)));
  if constexpr (LPR > 2) s = s + __uint_as_float(lane_xor<2>(__float_as_uint(s)));
  if constexpr (LPR > 4) s = s + __uint_as_float(lane_xor<4>(__float_as_uint(s)));
  if constexpr (LPR > 8) s = s + __uint_as_float(lane_xor<8>(__float_as_uint(s)));
  static_assert(LPR <= 16, "row_dot: at most 16 lanes per row");
  return s;
}

template <typename KT>
__device__ __forceinline__ void load16(const KT* src, float (&x)[16]);

template <>
__device__ __forceinline__ void load16<uint16_t>(const uint16_t* src, float (&x)[16]) {
  const uint4* p = reinterpret_cast<const uint4*>(src);
  const uint4 a = p[0], c = p[1];
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
    x[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
  }
}

template <>
__device__ __forceinline__ void load16<float>(const float* src, float (&x)[16]) {
  const float4* p = reinterpret_cast<const float4*>(src);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const float4 v = p[c];
    x[4 * c] = v.x;
    x[4 * c + 1] = v.y;
    x[4 * c + 2] = v.z;
    x[4 * c + 3] = v.w;
  }
}

}  // namespace fdl
