// Gate-weighted combine and the balance statistics.
//
// Combine ("Mixture of experts and speculative decoding", "Opening the hood:
// the MoE layer precisely", equation for y; "MoE inference: the call centre
// with 256 specialists ...", "The bare mechanism", weighted combination and
// shared experts):
//   y[t] = sum_{slot < k} g[t, slot] * Y[inv_row[t, slot]]  +  sum_s Yshared_s[t]
// accumulated in fp32 in slot order, then rounded once to the output type.
//
// Balance statistics ("Keeping the experts busy", balance-loss equation;
// "Mixture of Experts and Guided Decoding", auxiliary-loss equation):
//   f_e = counts_e / (T k), P_e = prob_sum_e / T, loss = alpha N sum_e f_e P_e.
#include "mfma.h"
#include "vec.h"
#include "balance.h"

namespace moe {
namespace {

// Rows at or past plan[kPlanRowSplit] arrive as plan[kPlanParts] fp32 partial
// sums (a down pass split over its reduction); they are added in part order
// before the gate multiply.
template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ yperm,
                                                      const float* __restrict__ ypart,
                                                      const int32_t* __restrict__ plan,
                                                      const int32_t* __restrict__ inv_row,
                                                      const float* __restrict__ gate,
                                                      const int32_t* __restrict__ offsets, int N,
                                                      int n_tok, int d, int k, int S,
                                                      T* __restrict__ y) {
  constexpr int V = Vec<T>::kN;
  const int t = blockIdx.x;
  __shared__ int s_row[kMaxTopK + kMaxShared];
  __shared__ float s_g[kMaxTopK];
  if (threadIdx.x < k) {
    s_row[threadIdx.x] = inv_row[static_cast<size_t>(t) * k + threadIdx.x];
    s_g[threadIdx.x] = gate[static_cast<size_t>(t) * k + threadIdx.x];
  } else if (threadIdx.x < k + S) {
    const int s = threadIdx.x - k;
    s_row[threadIdx.x] = offsets[N + s] + t;
  }
  __syncthreads();
  const int parts = plan[kPlanParts], row_split = plan[kPlanRowSplit];
  const size_t pstride = static_cast<size_t>(plan[kPlanStride]) * d;
  for (int c = threadIdx.x * V; c < d; c += 256 * V) {
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;
    for (int s = 0; s < k + S; ++s) {
      const int row = s_row[s];
      if (row < 0) continue;  // dropped by the capacity
      float v[V];
      if (parts > 0 && row >= row_split) {
        const float* src = ypart + static_cast<size_t>(row - row_split) * d + c;
#pragma unroll
        for (int i = 0; i < V; i += 4) Vec<float>::load(src + i, v + i);
        for (int q = 1; q < parts; ++q) {
          float u[V];
#pragma unroll
          for (int i = 0; i < V; i += 4) Vec<float>::load(src + q * pstride + i, u + i);
#pragma unroll
          for (int i = 0; i < V; ++i) v[i] += u[i];
        }
      } else {
        Vec<T>::load(yperm + static_cast<size_t>(row) * d + c, v);
      }
      const float gs = s < k ? s_g[s] : 1.0f;
#pragma unroll
      for (int i = 0; i < V; ++i) acc[i] = fmaf(gs, v[i], acc[i]);
    }
    Vec<T>::store(y + static_cast<size_t>(t) * d + c, acc);
  }
}

__global__ __launch_bounds__(256) void balance_kernel(int n_tok, int N, int k,
                                                      const int32_t* __restrict__ counts,
                                                      const float* __restrict__ prob_sum,
                                                      float alpha, float* __restrict__ f_out,
                                                      float* __restrict__ P_out,
                                                      float* __restrict__ aux_out) {
  __shared__ float s_part[256];
  balance_block(n_tok, N, k, counts, prob_sum, alpha, f_out, P_out, aux_out, s_part);
}

}  // namespace

hipError_t launch_combine(int dtype, const void* yperm, const float* ypart,
                          const int32_t* plan, const int32_t* inv_row, const float* topk_gate,
                          const int32_t* offsets, int N, int T_, int d, int k, int S, void* y,
                          hipStream_t s) {
  if (dtype == 1)
    hipLaunchKernelGGL(combine_kernel<bf16_t>, dim3(T_), dim3(256), 0, s,
                       static_cast<const bf16_t*>(yperm), ypart, plan, inv_row, topk_gate,
                       offsets, N, T_, d, k, S, static_cast<bf16_t*>(y));
  else
    hipLaunchKernelGGL(combine_kernel<float>, dim3(T_), dim3(256), 0, s,
                       static_cast<const float*>(yperm), ypart, plan, inv_row, topk_gate,
                       offsets, N, T_, d, k, S, static_cast<float*>(y));
  return hipGetLastError();
}

hipError_t launch_balance(int T_, int N, int k, const int32_t* counts, const float* prob_sum,
                          float alpha, float* f_out, float* P_out, float* aux_out,
                          hipStream_t s) {
  hipLaunchKernelGGL(balance_kernel, dim3(1), dim3(256), 0, s, T_, N, k, counts, prob_sum, alpha,
                     f_out, P_out, aux_out);
  return hipGetLastError();
}

}  // namespace moe
