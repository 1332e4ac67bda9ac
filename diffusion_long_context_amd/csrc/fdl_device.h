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
};

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round-to-nearest-even float -> bf16 bits (finite inputs; used for probabilities and outputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
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

// Value of lane (lane ^ J) for a compile-time J: quad permutes for 1 and 2, swizzles (within 32
// lanes) for 4, 8 and 16, the half swap for 32.
template <int J>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
  if constexpr (J == 1) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
  else if constexpr (J == 2) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);
  else if constexpr (J == 4 || J == 8 || J == 16) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, (J << 10) | 0x1F);
  else if constexpr (J == 32) {
    // swap of the two 32-lane halves; in every lane one of the two results is the lane's own value
    // and the other the partner's (when they are equal, either is right)
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (r[0] == v) ? r[1] : r[0];
  } else {
    return (uint32_t)__shfl_xor((int)v, J, 64);
  }
}

__device__ __forceinline__ float lane_xor32f(float v) { return __uint_as_float(lane_xor<32>(__float_as_uint(v))); }

__device__ __forceinline__ void latch(uint32_t* status, uint32_t bit) {
  atomicOr(status, bit);
}

// Element offset of row (b, g, t), 0 <= t < L, of a KV cache: contiguous [B][Hkv][L][D] or paged
// [n_pages][Hkv][page_tokens][D] through page_table [B][pages_per_seq].  Branch-free: a bad page id
// sets `bad` and the row of page 0 is addressed instead, so every returned offset is dereferenceable
// and the caller can issue its loads unconditionally (a load inside a divergent branch whose value
// is used after the branch costs a full memory round trip per load).
template <bool PAGED>
struct KvRows {
  int32_t Hkv, L, D;
  int32_t page_log2, pages_per_seq, n_pages;
  const int32_t* page_table;

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
