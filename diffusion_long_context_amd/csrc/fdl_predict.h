// Past-confidence-guided query prediction for one sequence, computed by one full wave (one lane per
// position of the decode block, T <= 64).  Used by the prediction and unmask kernels and by the sink
// scan, which computes the prediction itself when it is the step's first reader of it.
//
// Focus-dLLM (abstract; Elamur "Summary" and "Key points"): the previous step's confidence picks the
// still-masked positions most likely to be decoded next (the top k), and each is widened into a
// local window; the union is the predicted query set.  Ties go to the lower position and NaN ranks
// lowest; no previous confidence predicts the whole block.
#pragma once

#include "fdl_device.h"

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

// The predicted query set of one sequence as a T-bit mask (the same in every lane); all 64 lanes
// of the wave must call.  conf == NULL: the whole block.
__device__ __forceinline__ uint64_t predict_mask(int T, const float* __restrict__ conf, const uint8_t* masked,
                                                 int top_k, int window, int lane) {
  const uint64_t all = (T == 64) ? ~0ull : ((1ull << T) - 1ull);
  if (conf == nullptr) return all;
  int m;
  const int rank = masked_rank(T, conf, masked, lane, &m);
  const uint64_t chosen = __ballot(m && rank < top_k);
  const int w = window < 64 ? window : 64;
  uint64_t pred = 0;
  for (int s = -w; s <= w; ++s) {
    if (s >= 64 || s <= -64) continue;
    pred |= (s >= 0) ? (chosen << s) : (chosen >> (-s));
  }
  return pred & all;
}

}  // namespace fdl
