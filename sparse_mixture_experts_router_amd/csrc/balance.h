// Balance statistics of "Keeping the experts busy" (balance-loss equation)
// and of the routing-collapse passage of "Mixture of Experts and Guided
// Decoding" (auxiliary-loss equation):
//   f_e = counts_e / (T k), P_e = prob_sum_e / T, raw = N sum_e f_e P_e,
//   aux = [raw, alpha raw]
// computed by the first 256 threads of a workgroup in a fixed order (thread
// i adds experts i, i + 256, ... with fused multiply-adds, then a tree over
// the 256 partial sums), so every caller gets bitwise the same values.  All
// threads of the workgroup must call it (it holds barriers); any output may
// be null.
#pragma once

#include "moe_internal.h"

namespace moe {

__device__ inline void balance_block(int n_tok, int N, int k, const int32_t* counts,
                                     const float* prob_sum, float alpha, float* f_out,
                                     float* P_out, float* aux_out, float* s_part /* [256] */) {
  const int t = threadIdx.x;
  if (t < 256) {
    float part = 0.f;
    for (int e = t; e < N; e += 256) {
      float f = 0.f, p = 0.f;
      if (n_tok > 0) {
        f = static_cast<float>(counts[e]) / (static_cast<float>(n_tok) * static_cast<float>(k));
        p = prob_sum[e] / static_cast<float>(n_tok);
      }
      if (f_out != nullptr) f_out[e] = f;
      if (P_out != nullptr) P_out[e] = p;
      part = fmaf(f, p, part);
    }
    s_part[t] = part;
  }
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (t < w) s_part[t] += s_part[t + w];
    __syncthreads();
  }
  if (t == 0 && aux_out != nullptr) {
    const float raw = static_cast<float>(N) * s_part[0];
    aux_out[0] = raw;
    aux_out[1] = alpha * raw;
  }
}

}  // namespace moe
