// Streaming-bandwidth probe: the rate a plain read (or copy) of one large buffer reaches on this
// chip, measured with the same kind of loads the attention kernels use.  It is the practical
// ceiling the HBM-bound kernels are compared with next to the vendor peak: a kernel can only be
// as fast as the memory system delivers a perfectly coalesced stream.
//
// Read (vector registers): every thread keeps kUnroll 16-byte non-temporal loads in flight and
// folds them into a running xor, which one lane per wave writes out (so the loads cannot be
// dropped).  Read (LDS DMA): the same stream fetched straight into LDS with global_load_lds_dwordx4,
// as the attention kernels fetch their tiles, each wave cycling over its own LDS slots.  Copy: the
// read stream written to a second buffer.  Tiles: the attention kernels' own pattern (per-workgroup
// regions, one 16 KiB K + V tile in flight per wave, through LDS).
#include "fdl_device.h"
#include "fdl_internal.h"
#include "fdl_stream.h"

namespace fdl {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 512;
constexpr int kUnroll = 8;

__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                                   uint32_t* __restrict__ out) {
  const size_t stride = (size_t)gridDim.x * kProbeThreads;
  size_t i = (size_t)blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // one word per wave
  for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) out[(size_t)blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6)] = acc;
}

// Each wave fetches 1 KiB per instruction into one of its kUnroll LDS slots, waits for the batch,
// and reads one word of it back (so that the fetches are consumed).
__global__ __launch_bounds__(kProbeThreads) void probe_read_lds_kernel(const char* __restrict__ src, size_t n1k,
                                                                       uint32_t* __restrict__ out) {
  __shared__ __attribute__((aligned(1024))) uint32_t lds[kProbeThreads / 64][kUnroll][256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const size_t waves = (size_t)gridDim.x * (kProbeThreads / 64);
  size_t i = (size_t)blockIdx.x * (kProbeThreads / 64) + wave;   // 1 KiB chunk index
  uint32_t acc = 0;
  for (; i + (kUnroll - 1) * waves < n1k; i += kUnroll * waves) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      __builtin_amdgcn_global_load_lds(src + (i + u * waves) * 1024 + 16 * lane, (lds_void_t*)&lds[wave][u][0], 16,
                                       0, kStreamPolicy);
    wait_vm0();
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= lds[wave][u][lane];
  }
  for (; i < n1k; i += waves) {
    __builtin_amdgcn_global_load_lds(src + i * 1024 + 16 * lane, (lds_void_t*)&lds[wave][0][0], 16, 0,
                                     kStreamPolicy);
    wait_vm0();
    acc ^= lds[wave][0][lane];
  }
  for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  if (lane == 0) out[(size_t)blockIdx.x * (kProbeThreads / 64) + wave] = acc;
}

__global__ __launch_bounds__(kProbeThreads) void probe_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                                   size_t n16) {
  const size_t stride = (size_t)gridDim.x * kProbeThreads;
  size_t i = (size_t)blockIdx.x * kProbeThreads + threadIdx.x;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) __builtin_nontemporal_store(v[u], dst + i + u * stride);
  }
  for (; i < n16; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// The attention kernels' own pattern: the first half of the buffer stands for K and the second for
// V; workgroup w owns one region of each (`region` bytes, a multiple of 8 KiB) and each of its 8
// waves takes the region's 16 KiB tiles (8 KiB of K and the matching 8 KiB of V) w, w + 8, ... with
// one tile in flight: wait for it, read it back from LDS, request the next into the same slot.
__global__ __launch_bounds__(kProbeThreads, 1) void probe_tiles_kernel(const char* __restrict__ k,
                                                                      const char* __restrict__ v, size_t region,
                                                                      uint32_t* __restrict__ out) {
  constexpr int NW = kProbeThreads / 64;
  __shared__ __attribute__((aligned(1024))) uint32_t slot[NW][4096];   // 16 KiB per wave
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n_tiles = (int)(region / 8192);
  const size_t base = (size_t)blockIdx.x * region;
  auto request = [&](int t) {
    const size_t a = base + (size_t)t * 8192 + 16 * lane;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      __builtin_amdgcn_global_load_lds(k + a + j * 1024, (lds_void_t*)&slot[wave][j * 256], 16, 0, kStreamPolicy);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      __builtin_amdgcn_global_load_lds(v + a + j * 1024, (lds_void_t*)&slot[wave][2048 + j * 256], 16, 0,
                                       kStreamPolicy);
  };
  uint32_t acc = 0;
  if (wave < n_tiles) request(wave);
  for (int t = wave; t < n_tiles; t += NW) {
    wait_vm0();
    uint32_t r[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = slot[wave][j * 512 + lane];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc ^= r[j];
    __builtin_amdgcn_s_waitcnt(0xC07F);   // the reads are done before the slot is refilled
    if (t + NW < n_tiles) request(t + NW);
  }
  for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  if (lane == 0) out[(size_t)blockIdx.x * NW + wave] = acc;
}

size_t probe_out_words(int n_blocks) { return (size_t)n_blocks * (kProbeThreads / 64); }

size_t probe_tile_region(size_t bytes, int n_blocks) { return (bytes / 2 / (size_t)n_blocks) & ~(size_t)8191; }

hipError_t launch_probe(hipStream_t st, int mode, const void* src, size_t bytes, void* dst, int n_blocks) {
  if (mode == 0) {
    hipLaunchKernelGGL(probe_read_kernel, dim3(n_blocks), dim3(kProbeThreads), 0, st,
                       static_cast<const u32x4*>(src), bytes / 16, static_cast<uint32_t*>(dst));
  } else if (mode == 1) {
    hipLaunchKernelGGL(probe_read_lds_kernel, dim3(n_blocks), dim3(kProbeThreads), 0, st,
                       static_cast<const char*>(src), bytes / 1024, static_cast<uint32_t*>(dst));
  } else if (mode == 3) {
    const char* k = static_cast<const char*>(src);
    hipLaunchKernelGGL(probe_tiles_kernel, dim3(n_blocks), dim3(kProbeThreads), 0, st, k, k + bytes / 2,
                       probe_tile_region(bytes, n_blocks), static_cast<uint32_t*>(dst));
  } else {
    hipLaunchKernelGGL(probe_copy_kernel, dim3(n_blocks), dim3(kProbeThreads), 0, st,
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), bytes / 16);
  }
  return hipGetLastError();
}

}  // namespace fdl
