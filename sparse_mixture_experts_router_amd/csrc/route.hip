// Routing: router GEMM, top-k selection, gates and per-block statistics.
//
// What one routing block computes, and the pages that define it, is stated
// in route_tile.h, which holds that block for these kernels and for the
// all-token expert pass.
//
// One workgroup (4 wavefronts) owns 64 tokens x N_pad experts.  The 64 x-rows
// and the N_pad router rows stream through a global -> LDS ring (32 K-elements
// per stage, direct 16-byte loads) into 16x16 MFMA blocks; for N_pad >= 64 the
// wavefronts split the experts, otherwise the tokens.  With few tokens the
// reduction dimension is split over workgroups as well (split-K): each writes
// fp32 partial logits and a second kernel adds them in a fixed order, so the
// logits (and hence the routing) stay deterministic.  The selection then runs
// on the logits tile in LDS: each token's N scores sit in one group of 16
// lanes (4 tokens per wavefront at a time), and top-k is k rounds of a
// butterfly arg-max over __shfl_xor on a packed 64-bit (key, index) order.
#include "route_tile.h"

namespace moe {
namespace {

// Router GEMM on a global -> LDS ring; FUSED: followed by the selection.
template <typename T, int NB, bool FUSED>
__global__ __launch_bounds__(256) void route_gemm_kernel(RouteArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds[RouteShape<NB>::LDS_BYTES];
  route_gemm_block<T, NB, FUSED>(a, blockIdx.x, blockIdx.y, lds);
}

// Sum of the split-K partial logits (fixed order) + logit_bias, then the
// selection, with 16 wavefronts (8 for more than 256 experts, whose logits
// tile and per-lane keys need the LDS and registers): each runs the
// selection of 4 tokens at once (a 4-wavefront workgroup looped over 16
// tokens per wavefront, and with one workgroup per 64-token block most CUs
// idled).
constexpr int select_threads(int nb) { return nb >= 32 ? 512 : 1024; }
template <int NB>
__global__ __launch_bounds__(select_threads(NB)) void route_select_kernel(RouteArgs a) {
  using S = RouteShape<NB>;
  constexpr int NP = S::NP, LD = S::LD, NT = select_threads(NB);
  __shared__ float s_logit[kRouteTokens * LD];
  __shared__ uint32_t s_mask[NP][2];
  __shared__ float s_psum[(NT / 64) * NP];
  __shared__ int32_t s_sel[kRouteTokens * kMaxTopK];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kRouteTokens;
  for (int i = tid; i < NP * 2; i += NT) (&s_mask[0][0])[i] = 0u;
  const int n_here = min(kRouteTokens, a.n_tok - t0);
  if (a.N % 4 == 0 && a.ksplit <= 8) {
    // (many tokens, few splits) 16-byte loads of 4 experts; every (token, 4 experts) quad of the tile
    // is a lane's, and its ksplit partials are all requested before the sum
    // (added in split order), so the loads overlap instead of queueing
    const int nq = a.N / 4;
    constexpr int U = 1;  // quads per thread and pass (the 1024 threads cover a tile in 4 passes)
    for (int q0 = tid; q0 < kRouteTokens * nq; q0 += NT * U) {
      f32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int k0 = 0; k0 < a.ksplit; k0 += 8) {  // 8 splits x U quads in flight
        f32x4 pv[8][U];
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int q = q0 + u * NT, tt = q / nq;
            pv[kk][u] = (k0 + kk < a.ksplit && q < kRouteTokens * nq && tt < n_here)
                            ? *reinterpret_cast<const f32x4*>(
                                  a.partial +
                                  (static_cast<size_t>(k0 + kk) * a.n_tok + t0 + tt) * a.N +
                                  (q - tt * nq) * 4)
                            : f32x4{0.f, 0.f, 0.f, 0.f};
          }
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
#pragma unroll
          for (int u = 0; u < U; ++u)
            if (k0 + kk < a.ksplit) v[u] += pv[kk][u];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int q = q0 + u * NT;
        if (q >= kRouteTokens * nq) continue;
        const int tt = q / nq, e0 = (q - tt * nq) * 4;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          float x = v[u][c];
          if (tt < n_here) {
            if (a.logit_bias != nullptr) x += a.logit_bias[e0 + c];
            if (a.logits_out != nullptr) a.logits_out[static_cast<size_t>(t0 + tt) * a.N + e0 + c] = x;
          }
          s_logit[tt * LD + e0 + c] = tt < n_here ? x : 0.f;
        }
      }
    }
    for (int i = tid; i < kRouteTokens * (NP - a.N); i += NT) {  // padding experts
      const int tt = i / (NP - a.N);
      s_logit[tt * LD + a.N + (i - tt * (NP - a.N))] = 0.f;
    }
  } else {  // (few tokens, many splits) one (token, expert) pair per lane
    for (int i = tid; i < kRouteTokens * NP; i += NT) {  // padding tokens and experts
      const int tt = i / NP, e = i - tt * NP;
      if (tt >= n_here || e >= a.N) s_logit[tt * LD + e] = 0.f;
    }
    for (int i = tid; i < n_here * a.N; i += NT) {
      const int tt = i / a.N, e = i - tt * a.N;
      const int t = t0 + tt;
      // up to 32 partials requested before the first is added (in split order)
      float v = 0.f;
      for (int k0 = 0; k0 < a.ksplit; k0 += 32) {
        float pv[32];
#pragma unroll
        for (int q = 0; q < 32; ++q)
          pv[q] = k0 + q < a.ksplit
                      ? a.partial[(static_cast<size_t>(k0 + q) * a.n_tok + t) * a.N + e]
                      : 0.f;
#pragma unroll
        for (int q = 0; q < 32; ++q)
          if (k0 + q < a.ksplit) v += pv[q];
      }
      if (a.logit_bias != nullptr) v += a.logit_bias[e];
      if (a.logits_out != nullptr) a.logits_out[static_cast<size_t>(t) * a.N + e] = v;
      s_logit[tt * LD + e] = v;
    }
  }
  __syncthreads();
  select_tile<NB, NT / 64>(s_logit, blockIdx.x, t0, a.n_tok, a.N, a.k, a.select_bias, a.topk_idx,
                           a.topk_gate, a.lrank, a.blk_counts, a.blk_psum, s_mask, s_psum, s_sel);
}

template <typename T, int NB>
hipError_t launch_nb(const RouteArgs& a, hipStream_t s) {
  const int blocks = (a.n_tok + kRouteTokens - 1) / kRouteTokens;
  if (a.ksplit == 1) {
    hipLaunchKernelGGL((route_gemm_kernel<T, NB, true>), dim3(blocks, 1), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((route_gemm_kernel<T, NB, false>), dim3(blocks, a.ksplit), dim3(256), 0, s,
                     a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((route_select_kernel<NB>), dim3(blocks), dim3(select_threads(NB)), 0, s, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const RouteArgs& a, hipStream_t s) {
  if (a.N <= 16) return launch_nb<T, 1>(a, s);
  if (a.N <= 32) return launch_nb<T, 2>(a, s);
  if (a.N <= 64) return launch_nb<T, 4>(a, s);
  if (a.N <= 128) return launch_nb<T, 8>(a, s);
  if (a.N <= 256) return launch_nb<T, 16>(a, s);
  return launch_nb<T, 32>(a, s);
}

}  // namespace

int route_split(int T_, int d, int dtype) {
  const int nsteps = d * (dtype == 1 ? 2 : 4) / kRowBytes;
  const int blocks = (T_ + kRouteTokens - 1) / kRouteTokens;
  if (blocks <= 0) return 1;  // no tokens: nothing to split
  // about two workgroups per CU (a router workgroup's short reduction is
  // latency-bound, so a second one per CU hides the first's waits), at
  // least 4 K steps each
  int ks = (512 + blocks - 1) / blocks;
  const int max_ks = nsteps / 4 > 0 ? nsteps / 4 : 1;
  ks = ks < 1 ? 1 : (ks > max_ks ? max_ks : ks);
  const int per = (nsteps + ks - 1) / ks;
  return (nsteps + per - 1) / per;  // no empty split
}

int route_dense_parts(int T_, int d, int N, int dtype, int cus) {
  // The router kernel streams all N router rows through LDS for every 64
  // tokens, as 64-byte row pieces; with N > 128 that is most of its traffic
  // (DeepSeek-V3 shape: 128 token blocks x 3.7 MB of router rows against
  // 117 MB of x).  The large-tile kernel's 256-token tiles of whole 128-byte
  // lines move a quarter of those router bytes.  At 128 experts its 256
  // columns are half idle and it still wins (Qwen3 shape: router GEMM and
  // selection 73.6 -> 64.9 us).  Parts: enough to put about one workgroup on
  // every compute unit, at most 8 (the selection kernel's fast path sums up
  // to 8 partials per load round).
  if (dtype != 1 || N < 128 || N > 256 || T_ < 2048) return 0;
  const int tiles = (T_ + 255) / 256;
  int parts = (cus + tiles - 1) / tiles;
  parts = parts < 1 ? 1 : (parts > 8 ? 8 : parts);
  while (parts > 1 && (parts - 1) * split_share(d / 64, parts) >= d / 64) --parts;
  return dense_gemm_fits(T_, d, N, parts) ? parts : 0;
}

hipError_t launch_route(int dtype, const void* x, const void* w_router, const float* logit_bias,
                        const float* select_bias, int T_, int d, int N, int k, int ksplit,
                        bool dense, float* partial, float* logits_out, int32_t* topk_idx,
                        float* topk_gate, int32_t* lrank, int32_t* blk_counts, float* blk_psum,
                        hipStream_t s) {
  RouteArgs a{};
  a.x = x;
  a.wr = w_router;
  a.logit_bias = logit_bias;
  a.select_bias = select_bias;
  a.n_tok = T_;
  a.d = d;
  a.N = N;
  a.k = k;
  const int nsteps = d * (dtype == 1 ? 2 : 4) / kRowBytes;
  a.ksplit = ksplit < 1 ? 1 : ksplit;
  a.steps_per_split = (nsteps + a.ksplit - 1) / a.ksplit;
  a.partial = partial;
  a.logits_out = logits_out;
  a.topk_idx = topk_idx;
  a.topk_gate = topk_gate;
  a.lrank = lrank;
  a.blk_counts = blk_counts;
  a.blk_psum = blk_psum;
  if (a.ksplit > 1 && partial == nullptr) return hipErrorInvalidValue;
  if (dense) {
    // the router GEMM on the large-tile kernel: fp32 partial logits
    // [ksplit, T, N], then the selection kernel adds them in part order
    if (dtype != 1 || N < 128 || N > 256 || partial == nullptr) return hipErrorInvalidValue;
    GemmArgs g{};
    g.a = x;
    g.w0 = w_router;
    g.a_rows = T_;
    g.n_experts = 1;
    g.k_dim = d;
    g.n_dim = N;
    g.out_part = partial;
    g.dense_parts = a.ksplit;
    hipError_t e = launch_dense_gemm(g, s);
    if (e != hipSuccess) return e;
    const int blocks = (T_ + kRouteTokens - 1) / kRouteTokens;
    if (N > 128)
      hipLaunchKernelGGL((route_select_kernel<16>), dim3(blocks), dim3(select_threads(16)), 0, s, a);
    else
      hipLaunchKernelGGL((route_select_kernel<8>), dim3(blocks), dim3(select_threads(8)), 0, s, a);
    return hipGetLastError();
  }
  if (dtype == 1) return launch_t<bf16_t>(a, s);
  return launch_t<float>(a, s);
}

}  // namespace moe
