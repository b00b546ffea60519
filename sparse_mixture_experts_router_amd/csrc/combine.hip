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

// 16 bytes of a row as fp32 values: 8 bf16 or 4 fp32.
template <typename T> __device__ __forceinline__ void widen16(u32x4 r, float* v);
template <> __device__ __forceinline__ void widen16<bf16_t>(u32x4 r, float* v) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(r[i] << 16);
    v[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
  }
}
template <> __device__ __forceinline__ void widen16<float>(u32x4 r, float* v) {
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(r[i]);
}

// The expert outputs are read exactly once, so their loads are nontemporal
// (no L2 or Infinity Cache allocation): the DeepSeek-V3-shaped combine
// 235 -> 208 us, the Qwen3-shaped one 249 -> 211 us.
__device__ __forceinline__ u32x4 load_once(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
template <typename T> __device__ __forceinline__ void load_once(const T* p, float* v) {
  widen16<T>(load_once(static_cast<const void*>(p)), v);
}

// Rows at or past plan[kPlanRowSplit] arrive as plan[kPlanParts] fp32 partial
// sums (a down pass split over its reduction); they are added in part order
// before the gate multiply.
// y[t] for one token (one workgroup), any row layout: rows at or past
// plan[kPlanRowSplit] are the sum of plan[kPlanParts] fp32 parts.
template <typename T>
__device__ __forceinline__ void combine_token(const T* __restrict__ yperm,
                                              const float* __restrict__ ypart, int parts,
                                              int row_split, size_t pstride, const int* s_row,
                                              const float* s_g, int t, int d, int k, int S,
                                              T* __restrict__ y) {
  constexpr int V = Vec<T>::kN;
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
        for (int i = 0; i < V; i += 4) load_once<float>(src + i, v + i);
        for (int q = 1; q < parts; ++q) {
          float u[V];
#pragma unroll
          for (int i = 0; i < V; i += 4) load_once<float>(src + q * pstride + i, u + i);
#pragma unroll
          for (int i = 0; i < V; ++i) v[i] += u[i];
        }
      } else {
        load_once<T>(yperm + static_cast<size_t>(row) * d + c, v);
      }
      const float gs = s < k ? s_g[s] : 1.0f;
#pragma unroll
      for (int i = 0; i < V; ++i) acc[i] = fmaf(gs, v[i], acc[i]);
    }
    Vec<T>::store(y + static_cast<size_t>(t) * d + c, acc);
  }
}

// KS = 0: any slot count, one slot at a time.  KS = k + S > 0: a token whose
// rows are all whole rows of yperm (no split parts) requests all KS row
// loads of a 16-byte column chunk before the first is added (in slot order),
// so they overlap instead of queueing; other tokens take the general loop.
template <typename T, int KS>
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
  if constexpr (KS > 0) {
    int row[KS];
    float gs[KS];
    bool whole = true;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      row[s] = s_row[s];
      gs[s] = s < k ? s_g[s] : 1.0f;
      whole = whole && (parts == 0 || row[s] < row_split);
    }
    if (whole) {
      for (int c = threadIdx.x * V; c < d; c += 256 * V) {
        u32x4 raw[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s)
          raw[s] = row[s] >= 0 ? load_once(yperm + static_cast<size_t>(row[s]) * d + c)
                               : u32x4{0u, 0u, 0u, 0u};
        float acc[V];
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] = 0.f;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          if (row[s] < 0) continue;  // dropped by the capacity
          float v[V];
          widen16<T>(raw[s], v);
#pragma unroll
          for (int i = 0; i < V; ++i) acc[i] = fmaf(gs[s], v[i], acc[i]);
        }
        Vec<T>::store(y + static_cast<size_t>(t) * d + c, acc);
      }
      return;
    }
  }
  combine_token<T>(yperm, ypart, parts, row_split, pstride, s_row, s_g, t, d, k, S, y);
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

template <typename T>
void launch_combine_t(const T* yperm, const float* ypart, const int32_t* plan,
                      const int32_t* inv_row, const float* gate, const int32_t* offsets, int N,
                      int T_, int d, int k, int S, T* y, hipStream_t s) {
#define MOE_COMBINE(KS)                                                                   \
  hipLaunchKernelGGL((combine_kernel<T, KS>), dim3(T_), dim3(256), 0, s, yperm, ypart, plan, \
                     inv_row, gate, offsets, N, T_, d, k, S, y)
  switch (k + S) {  // the slot counts of the usual layers get the overlapped loads
    case 1: MOE_COMBINE(1); break;
    case 2: MOE_COMBINE(2); break;
    case 3: MOE_COMBINE(3); break;
    case 4: MOE_COMBINE(4); break;
    case 8: MOE_COMBINE(8); break;
    case 9: MOE_COMBINE(9); break;
    default: MOE_COMBINE(0); break;
  }
#undef MOE_COMBINE
}

}  // namespace

hipError_t launch_combine(int dtype, const void* yperm, const float* ypart,
                          const int32_t* plan, const int32_t* inv_row, const float* topk_gate,
                          const int32_t* offsets, int N, int T_, int d, int k, int S, void* y,
                          hipStream_t s) {
  if (dtype == 1)
    launch_combine_t(static_cast<const bf16_t*>(yperm), ypart, plan, inv_row, topk_gate, offsets,
                     N, T_, d, k, S, static_cast<bf16_t*>(y), s);
  else
    launch_combine_t(static_cast<const float*>(yperm), ypart, plan, inv_row, topk_gate, offsets,
                     N, T_, d, k, S, static_cast<float*>(y), s);
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
