// Routing kernel: router GEMM, top-k selection, gates and per-block statistics
// in one launch.
//
// Steps (pages: "Mixture of experts and speculative decoding", "Following one
// token through an MoE layer" steps 1-3 and "Opening the hood: the MoE layer
// precisely"; "MoE inference: the call centre with 256 specialists ...", "The
// bare mechanism"):
//   r[t, e]  = sum_j x[t, j] W_r[e, j] (+ logit_bias[e])     fp32 accumulate
//   key      = r + select_bias[e]                           one fp32 RN add
//   TopK     = k largest keys, equal keys -> lower e, slot 0 = largest
//   g        = softmax of the kept r                         fp32, sums to 1
// and, for the balance statistics of "Keeping the experts busy", per block of
// 64 tokens: the number of assignments to each expert and the sum over tokens
// of the full softmax of r.  Each assignment also gets its rank among the
// block's assignments to the same expert (ordered by token), which the
// grouping step turns into a row index.
//
// Layout: one workgroup of 4 wavefronts per 64 tokens.  Wave w computes the
// 16 x N_pad logits of tokens 16w .. 16w+15 with 16x16 MFMA blocks; the router
// weight slice (N_pad rows x 128 bytes) is staged once per K step in LDS and
// shared by the 4 waves.  The logits then go through LDS so that each token's
// N scores sit in one group of G = min(64, N_pad) lanes, where top-k runs as k
// rounds of a butterfly arg-max over shuffles.
#include "mfma.h"

#include <math.h>

namespace moe {
namespace {

// a before b in the selection order: higher key, equal keys -> lower index.
__device__ __forceinline__ bool before(float ka, int ea, float kb, int eb) {
  return ka > kb || (ka == kb && ea < eb);
}

template <int G>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int off = G / 2; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int off = G / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

template <typename T, int NB>
__global__ __launch_bounds__(256) void route_kernel(
    const T* __restrict__ x, const T* __restrict__ wr, const float* __restrict__ logit_bias,
    const float* __restrict__ select_bias, int n_tok, int d, int N, int k,
    float* __restrict__ logits_out, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_gate, int32_t* __restrict__ lrank,
    int32_t* __restrict__ blk_counts, float* __restrict__ blk_psum) {
  constexpr int NP = NB * 16;          // experts padded to the MFMA block
  constexpr int ROWB = 128;            // bytes of a row slice per K step
  constexpr int G = NP < 64 ? NP : 64; // lanes per token in the selection
  constexpr int EPL = NP / G;          // experts per lane
  constexpr int TPW = 64 / G;          // tokens a wave selects at once
  constexpr int LD = NP + 1;           // fp32 logits row stride in LDS
  constexpr int TILE_BYTES = NP * ROWB;
  constexpr int LOGIT_BYTES = kRouteTokens * LD * 4;
  constexpr int UNION_BYTES = TILE_BYTES > LOGIT_BYTES ? TILE_BYTES : LOGIT_BYTES;

  __shared__ __attribute__((aligned(16))) char s_union[UNION_BYTES];
  __shared__ uint32_t s_mask[NP][2];             // tokens of the block that chose e
  __shared__ float s_psum[4 * TPW * NP];         // per (wave, group) probability sums
  __shared__ int32_t s_sel[kRouteTokens * kMaxTopK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int t0 = blockIdx.x * kRouteTokens;

  for (int i = tid; i < NP * 2; i += 256) (&s_mask[0][0])[i] = 0u;

  // ------------------------------------------------------------ router GEMM
  const size_t row_bytes = static_cast<size_t>(d) * sizeof(T);
  const int nsteps = static_cast<int>(row_bytes / ROWB);
  const int ta = t0 + wave * 16 + (lane & 15);
  const bool a_ok = ta < n_tok;
  const char* a_row = reinterpret_cast<const char*>(x) +
                      static_cast<size_t>(a_ok ? ta : 0) * row_bytes + 16 * (lane >> 4);
  const char* w_bytes = reinterpret_cast<const char*>(wr);

  f32x4 acc[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int s = 0; s < nsteps; ++s) {
    for (int c = tid; c < NP * 8; c += 256) {
      const int row = c >> 3, ch = c & 7;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (row < N)
        v = *reinterpret_cast<const u32x4*>(w_bytes + static_cast<size_t>(row) * row_bytes +
                                            static_cast<size_t>(s) * ROWB + ch * 16);
      *reinterpret_cast<u32x4*>(s_union + lds_swz(row, ch)) = v;
    }
    u32x4 a0 = u32x4{0u, 0u, 0u, 0u}, a1 = a0;
    if (a_ok) {
      a0 = *reinterpret_cast<const u32x4*>(a_row + static_cast<size_t>(s) * ROWB);
      a1 = *reinterpret_cast<const u32x4*>(a_row + static_cast<size_t>(s) * ROWB + 64);
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int row = j * 16 + (lane & 15);
      const u32x4 b0 = *reinterpret_cast<const u32x4*>(s_union + lds_swz(row, lane >> 4));
      const u32x4 b1 = *reinterpret_cast<const u32x4*>(s_union + lds_swz(row, 4 + (lane >> 4)));
      acc[j] = Mfma<T>::step(a0, b0, acc[j]);
      acc[j] = Mfma<T>::step(a1, b1, acc[j]);
    }
    __syncthreads();
  }

  // ------------------------------------------------------- logits to LDS
  float* s_logit = reinterpret_cast<float*>(s_union);
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int e = j * 16 + (lane & 15);
    const float lb = (logit_bias != nullptr && e < N) ? logit_bias[e] : 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tt = wave * 16 + 4 * (lane >> 4) + r;
      const float v = acc[j][r] + lb;
      s_logit[tt * LD + e] = v;
      if (logits_out != nullptr && e < N && t0 + tt < n_tok)
        logits_out[static_cast<size_t>(t0 + tt) * N + e] = v;
    }
  }
  __syncthreads();

  // ------------------------------------------------------------- selection
  const int grp = lane / G;
  const int gl = lane % G;
  float psum[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) psum[i] = 0.f;

  for (int base = 0; base < 16; base += TPW) {
    const int tt = wave * 16 + base + grp;  // token inside the block
    const int t = t0 + tt;
    const bool tok_ok = t < n_tok;          // uniform inside a lane group

    float r[EPL], key[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = gl + G * i;
      if (e < N) {
        r[i] = s_logit[tt * LD + e];
        key[i] = select_bias != nullptr ? __fadd_rn(r[i], select_bias[e]) : r[i];
      } else {
        r[i] = -INFINITY;
        key[i] = -INFINITY;
      }
    }

    // router probabilities over all N experts (balance statistic P)
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < EPL; ++i) m = fmaxf(m, r[i]);
    m = group_max<G>(m);
    float ex[EPL], se = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      ex[i] = (gl + G * i < N) ? expf(r[i] - m) : 0.f;
      se += ex[i];
    }
    se = group_sum<G>(se);
    if (tok_ok) {
#pragma unroll
      for (int i = 0; i < EPL; ++i) psum[i] += ex[i] / se;
    }

    // k rounds of arg-max over the group
    uint32_t taken = 0u;
    int slot_e = 0;
    float slot_r = -INFINITY;
    for (int s = 0; s < k; ++s) {
      float bk = -INFINITY;
      int be = 0x7fffffff;
      float br = 0.f;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int e = gl + G * i;
        if (e < N && !((taken >> i) & 1u) && before(key[i], e, bk, be)) {
          bk = key[i];
          be = e;
          br = r[i];
        }
      }
#pragma unroll
      for (int off = G / 2; off >= 1; off >>= 1) {
        const float ok = __shfl_xor(bk, off, 64);
        const int oe = __shfl_xor(be, off, 64);
        const float orr = __shfl_xor(br, off, 64);
        if (before(ok, oe, bk, be)) {
          bk = ok;
          be = oe;
          br = orr;
        }
      }
      if (be % G == gl) taken |= 1u << (be / G);
      if (gl == s) {
        slot_e = be;
        slot_r = br;
      }
    }

    // gates: softmax over the kept (unbiased) logits, slot s held by lane s
    const bool holds = gl < k;
    const float gm = group_max<G>(holds ? slot_r : -INFINITY);
    const float ge = holds ? expf(slot_r - gm) : 0.f;
    const float gs = group_sum<G>(ge);
    if (tok_ok && holds) {
      const size_t o = static_cast<size_t>(t) * k + gl;
      topk_idx[o] = slot_e;
      topk_gate[o] = ge / gs;
      s_sel[tt * kMaxTopK + gl] = slot_e;
      atomicOr(&s_mask[slot_e][tt >> 5], 1u << (tt & 31));
    }
  }

#pragma unroll
  for (int i = 0; i < EPL; ++i) s_psum[(wave * TPW + grp) * NP + gl + G * i] = psum[i];
  __syncthreads();

  // ---------------------------------------------- block statistics and ranks
  const int n_here = min(kRouteTokens, n_tok - t0);
  for (int i = tid; i < n_here * k; i += 256) {
    const int tt = i / k, s = i - tt * k;
    const int e = s_sel[tt * kMaxTopK + s];
    const uint64_t mk = static_cast<uint64_t>(s_mask[e][0]) |
                        (static_cast<uint64_t>(s_mask[e][1]) << 32);
    const uint64_t below = tt == 0 ? 0ull : (mk & ((1ull << tt) - 1ull));
    lrank[static_cast<size_t>(t0 + tt) * k + s] = __popcll(below);
  }
  for (int e = tid; e < N; e += 256) {
    blk_counts[static_cast<size_t>(blockIdx.x) * N + e] =
        __popc(s_mask[e][0]) + __popc(s_mask[e][1]);
    float acc_p = 0.f;
    for (int w = 0; w < 4 * TPW; ++w) acc_p += s_psum[w * NP + e];
    blk_psum[static_cast<size_t>(blockIdx.x) * N + e] = acc_p;
  }
}

template <typename T, int NB>
hipError_t launch_route_t(const void* x, const void* w_router, const float* logit_bias,
                          const float* select_bias, int T_, int d, int N, int k,
                          float* logits_out, int32_t* topk_idx, float* topk_gate,
                          int32_t* lrank, int32_t* blk_counts, float* blk_psum,
                          hipStream_t s) {
  const int blocks = (T_ + kRouteTokens - 1) / kRouteTokens;
  hipLaunchKernelGGL((route_kernel<T, NB>), dim3(blocks), dim3(256), 0, s,
                     static_cast<const T*>(x), static_cast<const T*>(w_router), logit_bias,
                     select_bias, T_, d, N, k, logits_out, topk_idx, topk_gate, lrank,
                     blk_counts, blk_psum);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_route_d(int N, const void* x, const void* w_router, const float* lb,
                          const float* sb, int T_, int d, int k, float* lo, int32_t* idx,
                          float* gate, int32_t* lrank, int32_t* bc, float* bp,
                          hipStream_t s) {
  if (N <= 16) return launch_route_t<T, 1>(x, w_router, lb, sb, T_, d, N, k, lo, idx, gate, lrank, bc, bp, s);
  if (N <= 32) return launch_route_t<T, 2>(x, w_router, lb, sb, T_, d, N, k, lo, idx, gate, lrank, bc, bp, s);
  if (N <= 64) return launch_route_t<T, 4>(x, w_router, lb, sb, T_, d, N, k, lo, idx, gate, lrank, bc, bp, s);
  if (N <= 128) return launch_route_t<T, 8>(x, w_router, lb, sb, T_, d, N, k, lo, idx, gate, lrank, bc, bp, s);
  if (N <= 256) return launch_route_t<T, 16>(x, w_router, lb, sb, T_, d, N, k, lo, idx, gate, lrank, bc, bp, s);
  return launch_route_t<T, 32>(x, w_router, lb, sb, T_, d, N, k, lo, idx, gate, lrank, bc, bp, s);
}

}  // namespace

hipError_t launch_route(int dtype, const void* x, const void* w_router,
                        const float* logit_bias, const float* select_bias, int T_, int d,
                        int N, int k, float* logits_out, int32_t* topk_idx,
                        float* topk_gate, int32_t* lrank, int32_t* blk_counts,
                        float* blk_psum, hipStream_t s) {
  if (dtype == 1)
    return launch_route_d<bf16_t>(N, x, w_router, logit_bias, select_bias, T_, d, k, logits_out,
                                  topk_idx, topk_gate, lrank, blk_counts, blk_psum, s);
  return launch_route_d<float>(N, x, w_router, logit_bias, select_bias, T_, d, k, logits_out,
                               topk_idx, topk_gate, lrank, blk_counts, blk_psum, s);
}

}  // namespace moe
