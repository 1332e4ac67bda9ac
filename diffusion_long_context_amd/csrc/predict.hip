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
#include "fdl_predict.h"

namespace fdl {

__global__ __launch_bounds__(64) void predict_kernel(int T, const float* __restrict__ prev_conf,
                                                     const uint8_t* __restrict__ masked, int top_k,
                                                     int window, uint64_t* __restrict__ pred_mask,
                                                     int32_t* __restrict__ n_pred) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const uint64_t pred = predict_mask(T, prev_conf ? prev_conf + (int64_t)b * T : nullptr, masked + (int64_t)b * T,
                                     top_k, window, lane);
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
