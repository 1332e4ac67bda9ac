// Past-confidence-guided query prediction: one wave per sequence.
//
// Focus-dLLM (abstract; Elamur "Summary" and "Key points"): the previous step's confidence picks the
// still-masked positions most likely to be decoded next (the top k), and each is widened into a
// local window; the union is the predicted query set.  Ties go to the lower position and NaN ranks
// lowest; no previous confidence predicts the whole block.
#include "fdl_device.h"
#include "fdl_internal.h"

namespace fdl {

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
    const int m = (lane < T && masked[(int64_t)b * T + lane] != 0) ? 1 : 0;
    const uint32_t key = m ? order_key(prev_conf[(int64_t)b * T + lane]) : 0u;
    // rank among masked slots: how many masked slots rank strictly above this one
    int rank = 0;
    for (int j = 0; j < T; ++j) {
      const uint32_t kj = __shfl(key, j, 64);
      const int mj = __shfl(m, j, 64);
      rank += (mj && (kj > key || (kj == key && j < lane))) ? 1 : 0;
    }
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

hipError_t launch_predict(hipStream_t s, int batch, int T, const float* prev_conf,
                          const uint8_t* masked, int top_k, int window, uint64_t* pred_mask,
                          int32_t* n_pred) {
  hipLaunchKernelGGL(predict_kernel, dim3(batch), dim3(64), 0, s, T, prev_conf, masked, top_k,
                     window, pred_mask, n_pred);
  return hipGetLastError();
}

}  // namespace fdl
