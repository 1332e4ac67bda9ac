// Past-confidence-guided query prediction, and the unmask update that closes a denoising step: one
// wave per sequence, one lane per position of the decode block.
//
// Focus-dLLM (abstract; Elamur "Summary" and "Key points"): the previous step's confidence picks the
// still-masked positions most likely to be decoded next (the top k), and each is widened into a
// local window; the union is the predicted query set.  Ties go to the lower position and NaN ranks
// lowest; no previous confidence predicts the whole block.  After a step, the masked positions of
// highest confidence (the same ranking) are the ones it decodes.
#include "fdl_device.h"
#include "fdl_internal.h"

namespace fdl {

// Rank of this lane's position among the masked positions of one sequence: how many masked
// positions rank strictly above it (higher confidence, or equal and lower position).  *is_masked
// gets the lane's flag; lanes at or past T are unmasked.  Reads only, each lane its own position.
// The flag and the confidence are read together (one round trip, not two), and each masked
// position's key reaches every lane through a scalar register, the masked set being one ballot.
__device__ __forceinline__ int masked_rank(int T, const float* __restrict__ conf, const uint8_t* masked,
                                           int lane, int* is_masked) {
  const bool in = lane < T;
  const uint8_t mf = in ? masked[lane] : (uint8_t)0;
  const float c = in ? conf[lane] : 0.f;
  const int m = mf != 0 ? 1 : 0;
  const uint32_t key = order_key(c);
  uint64_t left = __ballot(m);   // wave-uniform
  int rank = 0;
  while (left != 0ull) {
    const int j = __builtin_ctzll(left);
    left &= left - 1ull;
    const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane((int)key, j);
    rank += (kj > key || (kj == key && j < lane)) ? 1 : 0;
  }
  *is_masked = m;
  return rank;
}

__global__ __launch_bounds__(64) void predict_kernel(int T, const float* __restrict__ prev_conf,
                                                     const uint8_t* __restrict__ masked, int top_k,
                                                     int window, uint64_t* __restrict__ pred_mask,
                                                     int32_t* __restrict__ n_pred) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const uint64_t all = (T == 64) ? ~0ull : ((1ull << T) - 1ull);
  uint64_t pred;
  if (prev_conf == nullptr) {
    pred = all;
  } else {
    int m;
    const int rank = masked_rank(T, prev_conf + (int64_t)b * T, masked + (int64_t)b * T, lane, &m);
    const uint64_t chosen = __ballot(m && rank < top_k);
    const int w = window < 64 ? window : 64;
    pred = 0;
    for (int s = -w; s <= w; ++s) {
      if (s >= 64 || s <= -64) continue;
      pred |= (s >= 0) ? (chosen << s) : (chosen >> (-s));
    }
    pred &= all;
  }
  if (lane == 0) {
    pred_mask[b] = pred;
    n_pred[b] = __popcll(pred);
  }
}

// Decode the n_unmask best-ranked masked positions of each sequence: masked[b][i] := 0 in place
// (every lane reads its own flag before any lane writes) and, when decoded != NULL, decoded[b][r] =
// the position of rank r for r below the number decoded, -1 beyond.
__global__ __launch_bounds__(64) void unmask_kernel(int T, const float* __restrict__ conf, uint8_t* masked,
                                                    int n_unmask, int32_t* __restrict__ decoded) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  int m;
  const int rank = masked_rank(T, conf + (int64_t)b * T, masked + (int64_t)b * T, lane, &m);
  const bool take = m && rank < n_unmask;
  if (take) masked[(int64_t)b * T + lane] = 0;
  if (decoded != nullptr) {
    int32_t* row = decoded + (int64_t)b * n_unmask;
    if (take) row[rank] = lane;
    const int n_masked = __popcll(__ballot(m));
    for (int r = (n_masked < n_unmask ? n_masked : n_unmask) + lane; r < n_unmask; r += 64) row[r] = -1;
  }
}

hipError_t launch_unmask(hipStream_t s, int batch, int T, const float* conf, uint8_t* masked, int n_unmask,
                         int32_t* decoded) {
  hipLaunchKernelGGL(unmask_kernel, dim3(batch), dim3(64), 0, s, T, conf, masked, n_unmask, decoded);
  return hipGetLastError();
}

hipError_t launch_predict(hipStream_t s, int batch, int T, const float* prev_conf,
                          const uint8_t* masked, int top_k, int window, uint64_t* pred_mask,
                          int32_t* n_pred) {
  hipLaunchKernelGGL(predict_kernel, dim3(batch), dim3(64), 0, s, T, prev_conf, masked, top_k,
                     window, pred_mask, n_pred);
  return hipGetLastError();
}

}  // namespace fdl
