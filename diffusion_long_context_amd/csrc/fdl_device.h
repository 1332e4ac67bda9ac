// Device-side building blocks shared by the libfdllm kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fdl {

// Device status bits, latched with atomicOr and read by fdl_get_status.
enum : uint32_t {
  ST_SINK_OVERFLOW = 1u << 0,   // more sinks than max_sinks
  ST_CAND_OVERFLOW = 1u << 1,   // more sink candidates than the workspace holds
  ST_BAD_INDEX = 1u << 2,       // unit / page id out of range (row skipped)
  ST_SEL_OVERFLOW = 1u << 3,    // more selected units than max_sel (list truncated)
  ST_SYNC_FALLBACK = 1u << 4,   // a fused split scored every block itself (informational)
  ST_PLACEMENT = 1u << 5,       // a split's sibling ran on another XCD (informational; handled)
  ST_SPLIT_PLACEMENT = 1u << 6, // splits that merge through L2 ran on different XCDs (output invalid)
};

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Two floats -> two bf16 (round to nearest even) in one word, lo in bits 0-15: one
// v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Round-to-nearest-even float -> bf16 bits.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return pack_bf16x2(f, 0.f) & 0xFFFFu;
}

// 2^x with the bare hardware instruction: results below 2^-126 come out as zero, which changes no
// softmax weight the kernels use (they are sums of at least one term equal to 1).
__device__ __forceinline__ float exp2_fast(float x) {
  return __builtin_amdgcn_exp2f(x);
}

// Unsigned key whose order is the numeric order of a float: -0 == +0, NaN lowest (0).
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (f != f) ? 0u : k;
}

// D[32x32] += A[32x16] * B[16x32], bf16 in, f32 accumulate.  Lane l supplies A[l%32][8*(l/32)+e]
// and B[8*(l/32)+e][l%32] for e = 0..7; it receives D[8*(r/4) + 4*(l/32) + r%4][l%32] in
// register r = 0..15.
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) {
  return __builtin_bit_cast(bf16x8, v);
}

template <typename T>
__device__ __forceinline__ T wave_shfl_xor(T v, int mask) {
  return __shfl_xor(v, mask, 64);
}

// Value of lane (lane ^ J) for a compile-time J, without the LDS pipe: DPP quad permutes for 1 and 2;
// for 4 the half-row mirror (lane ^ 7) followed by the quad reversal (lane ^ 3); for 8 a rotation of
// the 16-lane row by 8; for 16 and 32 the row / half swaps.  A swap of a register with itself
// leaves, in every lane, the lane's own value in one result and the partner's in the other (when
// the two are equal either is right).
template <int J>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
  if constexpr (J == 1) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
  else if constexpr (J == 2) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);
  else if constexpr (J == 4) {
    const int m = __builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false);   // row_half_mirror
    return (uint32_t)__builtin_amdgcn_mov_dpp(m, 0x1B, 0xF, 0xF, false);      // quad_perm 3,2,1,0
  } else if constexpr (J == 8) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false);   // row_ror 8
  else if constexpr (J == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (r[0] == v) ? r[1] : r[0];
  } else if constexpr (J == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (r[0] == v) ? r[1] : r[0];
  } else {
    return (uint32_t)__shfl_xor((int)v, J, 64);
  }
}

__device__ __forceinline__ float lane_xor32f(float v) { return __uint_as_float(lane_xor<32>(__float_as_uint(v))); }

// Workgroup barrier for LDS traffic only: this wave's LDS operations are complete, then s_barrier.
// __syncthreads() also waits for every outstanding vector-memory operation (its release fence has to
// cover LDS written by global->LDS fetches still in flight), which would hold the barrier behind
// loads and fetches issued for later use.  The memory clobbers keep the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void block_sync_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The raw HW_REG_XCC_ID register of the calling wave (which XCD, accelerator complex die, it runs on).
__device__ __forceinline__ uint32_t xcc_reg() {
  return __builtin_amdgcn_s_getreg((31 << 11) | (0 << 6) | 20);
}

// Merge ticket of the splits of one head that hand partial results over through their XCD's L2.  A
// 64-bit word (two of the uint32 slots at `word`, 8-byte aligned): the number of takers in bits 0-7
// and, from bit 8, a 6-bit count of takers per XCD.  Returns the caller's place (0-based); for every
// caller, *all_here tells whether all NS takers so far counted, itself included, ran on its XCD --
// for the last taker (place NS - 1) that is every split of the head.  One thread per workgroup.
__device__ __forceinline__ uint32_t take_ticket(uint32_t* word, int NS, bool* all_here) {
  const uint32_t x = xcc_reg() & 7u;
  const uint64_t inc = 1ull + (1ull << (8 + 6 * x));
  const uint64_t old = __hip_atomic_fetch_add(reinterpret_cast<uint64_t*>(word), inc, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t now = old + inc;
  *all_here = ((now >> (8 + 6 * x)) & 63ull) == (now & 0xFFull);
  (void)NS;
  return (uint32_t)(old & 0xFFull);
}

// Leaves a ticket word at zero for the next launch (the last taker, after its merge).
__device__ __forceinline__ void reset_ticket(uint32_t* word) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(word), 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void latch(uint32_t* status, uint32_t bit) {
  atomicOr(status, bit);
}

// Cached tokens of sequence b: lens[b] clamped to [0, L] for a ragged batch, L otherwise.
__device__ __forceinline__ int seq_len(const int32_t* lens, int b, int L) {
  if (lens == nullptr) return L;
  const int v = lens[b];
  return v < 0 ? 0 : (v > L ? L : v);
}

// Element offset of row (b, g, t), 0 <= t < L, of a KV cache: contiguous [B][Hkv][L][D] or paged
// [n_pages][Hkv][page_tokens][D] through page_table [B][pages_per_seq].  Branch-free: a bad page id
// sets `bad` and the row of page 0 is addressed instead, so every returned offset is dereferenceable
// and the caller can issue its loads unconditionally (a load inside a divergent branch whose value
// is used after the branch costs a full memory round trip per load).
template <bool PAGED>
struct KvRows {
  int32_t Hkv, L, D;   // L: the row stride of a sequence (ctx_len)
  int32_t page_log2, pages_per_seq, n_pages;
  const int32_t* page_table;
  const int32_t* lens = nullptr;   // per-sequence lengths of a ragged batch (contiguous caches)

  // valid rows of sequence b
  __device__ __forceinline__ int bound(int b) const { return seq_len(lens, b, L); }

  __device__ __forceinline__ int64_t off(int b, int g, int t, bool& bad) const {
    if constexpr (!PAGED) {
      return ((int64_t)(b * Hkv + g) * L + t) * D;
    } else {
      const int pp = page_table[(int64_t)b * pages_per_seq + (t >> page_log2)];
      const bool good = (unsigned)pp < (unsigned)n_pages;
      bad = bad || !good;
      const int64_t pg = good ? pp : 0;
      return (((pg * Hkv + g) << page_log2) | (int64_t)(t & ((1 << page_log2) - 1))) * (int64_t)D;
    }
  }
};

// Latch ST_BAD_INDEX once per wave if any lane saw a bad index.
__device__ __forceinline__ void latch_bad(uint32_t* status, bool bad) {
  const uint64_t m = __ballot(bad);
  if (m && (threadIdx.x & 63) == (unsigned)(__ffsll((unsigned long long)m) - 1)) latch(status, ST_BAD_INDEX);
}

}  // namespace fdl
