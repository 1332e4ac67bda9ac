// Attention-sink detection at the source layer.
//
// Focus-dLLM (abstract; Elamur "Summary" and "Key points"): highly influential attention sinks must
// survive pruning, and since sink locations agree across layers they are found once and reused
// deeper.  The pages give no detection rule; the reading built here: for every q-head and
// predicted position p, take the softmax row of q_p . k_t / sqrt(D) over all cached tokens and the
// block's own tokens; a cached token whose mean weight over the predicted positions reaches tau for
// some head is a sink; the union over heads is the sequence's sink list (ascending).
//
// One pass over K (the only full-K read of a step): each wave streams 64-token tiles through bf16
// MFMA (S^T = K Q^T) and keeps a running log-sum-exp per query.  Because a running log-sum-exp never
// exceeds the final one, the mass a token gets under the running statistics is an upper bound of
// its true mass, so every token whose bound reaches tau (less a small rounding margin) is recorded
// as a candidate.  After the pass the partial statistics are merged into the exact log-sum-exp, the
// few candidates are re-scored exactly in float32, and survivors are set in a per-sequence bitmap
// that is compacted into the ascending sink list.
#include "fdl_device.h"
#include "fdl_internal.h"

namespace fdl {

__global__ void fill_u32_kernel(uint32_t* __restrict__ p, size_t n, uint32_t v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

hipError_t launch_fill_u32(hipStream_t s, uint32_t* p, size_t n, uint32_t v) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

constexpr float kCandSlack = 0.999f;   // candidates use tau * (1 - 1e-3): absorbs float32 rounding

struct SinkParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* k_dec;
  const uint64_t* pred_mask;
  float2* stats;         // [B][Hq][n_parts][32]  (running max in log2 units, running sum)
  float* lse2;           // [B][Hq][32]
  uint32_t* cand_count;  // [B]
  uint32_t* cand;        // [B][cand_cap]  (h << 24 | t)
  uint32_t* bitmap;      // [B][words]
  uint32_t* status;
  int Hq, Hkv, G, T, L, n_splits, cand_cap, words;
  float scale_log2, tau;
};

template <int D>
__global__ __launch_bounds__(256) void sink_scan_kernel(const SinkParams p) {
  constexpr int KS = D / 16;
  __shared__ float ebuf[4][64][33];
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ql = lane & 31, hh = lane >> 5;
  const int g = h / p.G;
  const uint64_t pred = p.pred_mask[b];
  const int n_pred = __popcll(pred);
  const int n_parts = p.n_splits * 4;
  float2* st_out = p.stats + (((int64_t)b * p.Hq + h) * n_parts + s * 4 + wave) * 32;
  float m_run = -__builtin_inff(), l_run = 0.f;
  if (n_pred > 0) {
    const bool qlive = ql < p.T && ((pred >> ql) & 1ull);
    bf16x8 qf[KS];
    const uint16_t* qrow = p.q + (((int64_t)b * p.Hq + h) * p.T + (ql < p.T ? ql : 0)) * D + hh * (D / 2);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (ql < p.T) v = *reinterpret_cast<const uint4*>(qrow + ks * 8);
      qf[ks] = as_bf16x8(v);
    }
    const float inv_np = 1.f / (float)n_pred;
    const int n_tiles = 1 + (p.L + 63) / 64;
    const int e0 = (int)((int64_t)n_tiles * s / p.n_splits);
    const int e1 = (int)((int64_t)n_tiles * (s + 1) / p.n_splits);
    const uint16_t* kdec = p.k_dec + ((int64_t)b * p.Hkv + g) * p.T * D;
    const uint16_t* kctx = p.k + ((int64_t)b * p.Hkv + g) * (int64_t)p.L * D;
    for (int e = e0 + wave; e < e1; e += 4) {
      // A operand straight from HBM: lane (token, hh) reads 8 dims per k-step
      uint4 ka[2][KS];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int r = st * 32 + ql;
        const uint16_t* row = nullptr;
        if (e == 0) {
          if (r < p.T) row = kdec + (int64_t)r * D;
        } else {
          const int t = (e - 1) * 64 + r;
          if (t < p.L) row = kctx + (int64_t)t * D;
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          ka[st][ks] = row ? *reinterpret_cast<const uint4*>(row + hh * (D / 2) + ks * 8)
                           : make_uint4(0u, 0u, 0u, 0u);
      }
      const int nvalid = (e == 0) ? p.T : min(64, p.L - (e - 1) * 64);
      f32x16 sacc[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[st][r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) sacc[st] = mfma32(as_bf16x8(ka[st][ks]), qf[ks], sacc[st]);
      }
      float mx = -__builtin_inff();
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = st * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
          float x = sacc[st][r] * p.scale_log2;
          if (row >= nvalid) x = -__builtin_inff();
          sacc[st][r] = x;
          mx = fmaxf(mx, x);
        }
      mx = fmaxf(mx, wave_shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = exp2f(m_run - m_new);
      float rs = 0.f;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) rs += exp2f(sacc[st][r] - m_new);
      rs += wave_shfl_xor(rs, 32);
      l_run = l_run * alpha + rs;
      m_run = m_new;
      if (e == 0) continue;   // the block's own tokens are never sinks
      // upper-bound masses under the running statistics, summed over predicted queries
      const float lse = m_run + __log2f(l_run);
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = st * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
          ebuf[wave][row][ql] = qlive ? exp2f(sacc[st][r] - lse) : 0.f;
        }
      wave_lds_sync();
      float u = 0.f;
#pragma unroll
      for (int j = 0; j < 32; ++j) u += ebuf[wave][lane][j];
      u *= inv_np;
      if (lane < nvalid && u >= p.tau * kCandSlack) {
        const int t = (e - 1) * 64 + lane;
        const uint32_t idx = atomicAdd(&p.cand_count[b], 1u);
        if ((int)idx < p.cand_cap)
          p.cand[(int64_t)b * p.cand_cap + idx] = ((uint32_t)h << 24) | (uint32_t)t;
        else
          latch(p.status, ST_CAND_OVERFLOW);
      }
      wave_lds_sync();
    }
  }
  if (hh == 0) st_out[ql] = make_float2(m_run, l_run);
}

__global__ __launch_bounds__(64) void sink_lse_kernel(const SinkParams p) {
  const int h = blockIdx.x, b = blockIdx.y, q = threadIdx.x;
  if (q >= 32) return;
  const int n_parts = p.n_splits * 4;
  const float2* st = p.stats + ((int64_t)b * p.Hq + h) * n_parts * 32 + q;
  float M = -__builtin_inff();
  for (int i = 0; i < n_parts; ++i) M = fmaxf(M, st[i * 32].x);
  float S = 0.f;
  for (int i = 0; i < n_parts; ++i) {
    const float2 v = st[i * 32];
    if (v.y > 0.f) S += v.y * exp2f(v.x - M);
  }
  p.lse2[((int64_t)b * p.Hq + h) * 32 + q] = M + __log2f(S);
}

// One wave per candidate: lane q (a predicted position) re-scores q . k_t in float32.
template <int D>
__global__ __launch_bounds__(256) void sink_final_kernel(const SinkParams p) {
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t pred = p.pred_mask[b];
  const int n_pred = __popcll(pred);
  if (n_pred == 0) return;
  int count = (int)p.cand_count[b];
  count = count < p.cand_cap ? count : p.cand_cap;
  for (int c = blockIdx.x * 4 + wave; c < count; c += gridDim.x * 4) {
    const uint32_t code = p.cand[(int64_t)b * p.cand_cap + c];
    const int h = (int)(code >> 24), t = (int)(code & 0xFFFFFFu);
    const int g = h / p.G;
    float e = 0.f;
    if (lane < p.T && ((pred >> lane) & 1ull)) {
      const uint16_t* qr = p.q + (((int64_t)b * p.Hq + h) * p.T + lane) * D;
      const uint16_t* kr = p.k + (((int64_t)b * p.Hkv + g) * p.L + t) * D;
      float acc = 0.f;
#pragma unroll 8
      for (int d = 0; d < D; d += 8) {
        const uint4 qa = *reinterpret_cast<const uint4*>(qr + d);
        const uint4 ka = *reinterpret_cast<const uint4*>(kr + d);
        const uint32_t qw[4] = {qa.x, qa.y, qa.z, qa.w};
        const uint32_t kw[4] = {ka.x, ka.y, ka.z, ka.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc += bf16_bits_to_f32(qw[i] & 0xFFFFu) * bf16_bits_to_f32(kw[i] & 0xFFFFu);
          acc += bf16_bits_to_f32(qw[i] >> 16) * bf16_bits_to_f32(kw[i] >> 16);
        }
      }
      e = exp2f(acc * p.scale_log2 - p.lse2[((int64_t)b * p.Hq + h) * 32 + lane]);
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) e += wave_shfl_xor(e, o);
    if (lane == 0 && e / (float)n_pred >= p.tau)
      atomicOr(&p.bitmap[(int64_t)b * p.words + (t >> 5)], 1u << (t & 31));
  }
}

// float32 path (small workloads): thread = query row; two passes over the keys.
template <int D>
__global__ __launch_bounds__(64) void sink_f32_kernel(const float* __restrict__ q,
                                                      const float* __restrict__ k,
                                                      const float* __restrict__ k_dec,
                                                      const uint64_t* __restrict__ pred_mask,
                                                      uint32_t* __restrict__ bitmap, int Hq, int Hkv,
                                                      int G, int T, int L, int words, float tau) {
  __shared__ float kc[32][D + 1];
  __shared__ float ev[32][65];
  const int h = blockIdx.x, b = blockIdx.y, qi = threadIdx.x;
  const int g = h / G;
  const uint64_t pred = pred_mask[b];
  const int n_pred = __popcll(pred);
  if (n_pred == 0) return;
  const bool live = qi < T && ((pred >> qi) & 1ull);
  float qr[D];
  const float* qrow = q + (((int64_t)b * Hq + h) * T + (qi < T ? qi : 0)) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) qr[d] = qrow[d];
  const float scale = 1.0f / sqrtf((float)D);
  const float* kd = k_dec + ((int64_t)b * Hkv + g) * T * D;
  const float* kx = k + ((int64_t)b * Hkv + g) * (int64_t)L * D;
  const int total = T + L;
  // pass 1: log-sum-exp over own block + cached tokens
  float m = -__builtin_inff(), l = 0.f;
  for (int c0 = 0; c0 < total; c0 += 32) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < 32 * D; idx += 64) {
      const int r = idx / D, d = idx % D, i = c0 + r;
      kc[r][d] = (i < T) ? kd[(int64_t)i * D + d] : (i < total ? kx[(int64_t)(i - T) * D + d] : 0.f);
    }
    __syncthreads();
    for (int r = 0; r < 32 && c0 + r < total; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) acc += qr[d] * kc[r][d];
      const float x = acc * scale;
      const float mn = fmaxf(m, x);
      l = l * __expf(m - mn) + __expf(x - mn);
      m = mn;
    }
  }
  const float lse = m + __logf(l);
  // pass 2: masses of cached tokens
  for (int c0 = 0; c0 < L; c0 += 32) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < 32 * D; idx += 64) {
      const int r = idx / D, d = idx % D, t = c0 + r;
      kc[r][d] = t < L ? kx[(int64_t)t * D + d] : 0.f;
    }
    __syncthreads();
    for (int r = 0; r < 32; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) acc += qr[d] * kc[r][d];
      ev[r][qi] = live ? __expf(acc * scale - lse) : 0.f;
    }
    __syncthreads();
    if (qi < 32 && c0 + qi < L) {
      float a = 0.f;
      for (int j = 0; j < 64; ++j) a += ev[qi][j];
      if (a / (float)n_pred >= tau) {
        const int t = c0 + qi;
        atomicOr(&bitmap[(int64_t)b * words + (t >> 5)], 1u << (t & 31));
      }
    }
  }
}

// Bitmap -> ascending sink positions; one workgroup per sequence.
__global__ __launch_bounds__(256) void sink_compact_kernel(const uint32_t* __restrict__ bitmap,
                                                           int words, int max_sinks,
                                                           int32_t* __restrict__ sink_pos,
                                                           int32_t* __restrict__ n_sinks,
                                                           uint32_t* __restrict__ status) {
  __shared__ int tmp[4];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int per = (words + 255) / 256;
  const int w0 = tid * per;
  int cnt = 0;
  for (int i = 0; i < per; ++i)
    if (w0 + i < words) cnt += __popc(bitmap[(int64_t)b * words + w0 + i]);
  int incl = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  int off = 0, total = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    if (w < wave) off += tmp[w];
    total += tmp[w];
  }
  int pos = off + incl - cnt;
  for (int i = 0; i < per; ++i) {
    const int wi = w0 + i;
    if (wi >= words) break;
    uint32_t bits = bitmap[(int64_t)b * words + wi];
    while (bits) {
      const int bit = __ffs(bits) - 1;
      bits &= bits - 1;
      if (pos < max_sinks) sink_pos[(int64_t)b * max_sinks + pos] = wi * 32 + bit;
      ++pos;
    }
  }
  // pad the rest of the list with -1 so stale entries never look like sinks
  for (int i = total + tid; i < max_sinks; i += 256) sink_pos[(int64_t)b * max_sinks + i] = -1;
  if (tid == 0) {
    n_sinks[b] = total < max_sinks ? total : max_sinks;
    if (total > max_sinks) latch(status, ST_SINK_OVERFLOW);
  }
}

size_t sink_scratch_bytes(const Geom& g, int* n_splits, int* cand_cap) {
  const int n_tiles = 1 + (g.L + 63) / 64;
  // about two workgroups (8 waves) per CU over all (head, sequence) pairs
  int s = (int)((2LL * 256 + (long long)g.B * g.Hq - 1) / ((long long)g.B * g.Hq));
  if (s > (n_tiles + 3) / 4) s = (n_tiles + 3) / 4;
  if (s < 1) s = 1;
  *n_splits = s;
  *cand_cap = 16384;
  const int words = (g.L + 31) / 32;
  size_t bytes = 0;
  bytes += (size_t)g.B * g.Hq * s * 4 * 32 * sizeof(float2);   // stats
  bytes += (size_t)g.B * g.Hq * 32 * sizeof(float);            // lse2
  bytes += 256 + (size_t)g.B * sizeof(uint32_t);               // cand_count (+align)
  bytes += (size_t)g.B * words * sizeof(uint32_t);             // bitmap
  bytes += (size_t)g.B * (*cand_cap) * sizeof(uint32_t);       // candidates
  return bytes + 1024;
}

hipError_t launch_sinks(hipStream_t st, const Geom& g, const void* q, const uint64_t* pred_mask,
                        const void* k, const void* k_dec, float tau, int max_sinks,
                        int32_t* sink_pos, int32_t* n_sinks, char* scratch, int n_splits,
                        int cand_cap, uint32_t* status, int num_cus) {
  (void)num_cus;
  const int words = (g.L + 31) / 32;
  char* cur = scratch;
  auto take = [&](size_t bytes) {
    char* r = cur;
    cur += (bytes + 255) & ~(size_t)255;
    return r;
  };
  SinkParams p;
  p.stats = reinterpret_cast<float2*>(take((size_t)g.B * g.Hq * n_splits * 4 * 32 * sizeof(float2)));
  p.lse2 = reinterpret_cast<float*>(take((size_t)g.B * g.Hq * 32 * sizeof(float)));
  // cand_count and bitmap are contiguous so one fill clears both
  p.cand_count = reinterpret_cast<uint32_t*>(cur);
  p.bitmap = p.cand_count + g.B;
  take(((size_t)g.B + (size_t)g.B * words) * sizeof(uint32_t));
  p.cand = reinterpret_cast<uint32_t*>(take((size_t)g.B * cand_cap * sizeof(uint32_t)));
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.k_dec = static_cast<const uint16_t*>(k_dec);
  p.pred_mask = pred_mask;
  p.status = status;
  p.Hq = g.Hq;
  p.Hkv = g.Hkv;
  p.G = g.G;
  p.T = g.T;
  p.L = g.L;
  p.n_splits = n_splits;
  p.cand_cap = cand_cap;
  p.words = words;
  p.scale_log2 = 1.4426950408889634f / sqrtf((float)g.D);
  p.tau = tau;
  hipError_t err = launch_fill_u32(st, p.cand_count, (size_t)g.B + (size_t)g.B * words, 0u);
  if (err != hipSuccess) return err;
  if (g.dtype == FDL_F32) {
    dim3 grid(g.Hq, g.B);
    const float* qq = static_cast<const float*>(q);
    const float* kk = static_cast<const float*>(k);
    const float* kd = static_cast<const float*>(k_dec);
    if (g.D == 128)
      hipLaunchKernelGGL((sink_f32_kernel<128>), grid, dim3(64), 0, st, qq, kk, kd, pred_mask,
                         p.bitmap, g.Hq, g.Hkv, g.G, g.T, g.L, words, tau);
    else
      hipLaunchKernelGGL((sink_f32_kernel<64>), grid, dim3(64), 0, st, qq, kk, kd, pred_mask,
                         p.bitmap, g.Hq, g.Hkv, g.G, g.T, g.L, words, tau);
  } else {
    dim3 grid(n_splits, g.Hq, g.B);
    if (g.D == 128)
      hipLaunchKernelGGL((sink_scan_kernel<128>), grid, dim3(256), 0, st, p);
    else
      hipLaunchKernelGGL((sink_scan_kernel<64>), grid, dim3(256), 0, st, p);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(sink_lse_kernel, dim3(g.Hq, g.B), dim3(64), 0, st, p);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    dim3 fgrid(64, g.B);
    if (g.D == 128)
      hipLaunchKernelGGL((sink_final_kernel<128>), fgrid, dim3(256), 0, st, p);
    else
      hipLaunchKernelGGL((sink_final_kernel<64>), fgrid, dim3(256), 0, st, p);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(sink_compact_kernel, dim3(g.B), dim3(256), 0, st, p.bitmap, words, max_sinks,
                     sink_pos, n_sinks, status);
  return hipGetLastError();
}

}  // namespace fdl
