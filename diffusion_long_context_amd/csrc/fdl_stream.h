// Streaming rows of a bf16 cache from HBM straight into LDS (gfx950 LDS DMA), shared by the
// attention and sink-detection kernels.
//
// global_load_lds_dwordx4 moves 1 KiB per instruction: 64 lanes x 16 bytes, lane l's bytes landing
// at the destination + 16 l, so the lane -> global chunk map chooses the LDS layout.  Rows are
// stored with their 16-byte chunks XOR-swizzled by the row index so that the MFMA operand reads are
// free of bank conflicts.  A fetch only counts as done in vmcnt, so an LDS read of the destination
// must follow an explicit full vector-memory wait.
#pragma once

#include <hip/hip_runtime.h>

namespace fdl {

typedef __attribute__((address_space(3))) void lds_void_t;

// Cache policy of the streaming fetches: non-temporal (each KV row is read once per launch).
constexpr int kStreamPolicy = 2;

__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Row geometry of a D-wide bf16 row for 1 KiB fetches.
template <int D>
struct RowChunks {
  static constexpr int PROW = D / 8;                 // 16-byte chunks per row
  static constexpr int ROWS_PER_INSTR = 64 / PROW;   // rows one 1 KiB fetch covers
};

// LDS chunk swizzle: chunk c of row r is stored at chunk slot c ^ swz(r).  swz permutes the low 4
// bits of the row (bits 2 and 3 swapped) so that (a) the 16 rows read together by the K-operand
// loads hit 16 different slots and (b) rows r and r + 4, which the two lane halves read together
// for V, fall in different halves of the row's banks.
__device__ __forceinline__ int swz(int r) { return (r & 3) | ((r >> 1) & 4) | ((r << 1) & 8); }

}  // namespace fdl
