// Routing: router GEMM, top-k selection, gates and per-block statistics.
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
#include "lds_ring.h"
#include "mfma.h"

#include <math.h>

namespace moe {
namespace {

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

// Compile-time layout of one routing workgroup for NB 16-expert blocks.
template <int NB>
struct RouteShape {
  static constexpr int NP = NB * 16;                    // experts padded to 16
  static constexpr int G = 16;                          // lanes per token in the selection
  static constexpr int EPL = NP / G;                    // experts per lane (= NB)
  static constexpr int TPW = 64 / G;                    // tokens a wave selects at once
  static constexpr int LD = NP + 1;                     // fp32 logits row stride in LDS
  static constexpr int WE = NB < 4 ? NB : 4;            // wavefronts across experts
  static constexpr int WT = 4 / WE;                     // wavefronts across tokens
  static constexpr int TB = 4 / WT;                     // 16-token blocks per wavefront
  static constexpr int EB = NB / WE;                    // 16-expert blocks per wavefront
  static constexpr int BLOCKS = (4 + NB + 3) / 4 * 4;   // 1 KB ring blocks per stage
  static constexpr int LPW = BLOCKS / 4;                // loads per lane per K step
  static constexpr int STAGES = NB >= 32 ? 3 : 4;
  static constexpr int STAGE = BLOCKS * 1024;
  static constexpr int RING = STAGES * STAGE;
  static constexpr int LOGITS = kRouteTokens * LD * 4;
  static constexpr int UNION = RING > LOGITS ? RING : LOGITS;
  static_assert(NB == 1 || NB == 2 || NB == 4 || NB == 8 || NB == 16 || NB == 32, "NB");
};

// Selection order as one integer: higher key first, equal keys (IEEE, so the
// key is normalised from -0 to +0) -> lower expert index first.  The fp32 key
// is mapped to an order-preserving uint32 in the high half; the low half is
// the complement of the index.  0 sorts below every real expert.
__device__ __forceinline__ uint64_t order_key(float key, int e) {
  uint32_t u = __float_as_uint(key + 0.0f);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<uint64_t>(u) << 32) | (0xffffffffu - static_cast<uint32_t>(e));
}

__device__ __forceinline__ uint64_t group16_max(uint64_t v) {
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) {
    const uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), off, 64);
    const uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), off, 64);
    const uint64_t o = (static_cast<uint64_t>(hi) << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

// ---------------------------------------------------------------- selection
// Top-k, gates, block statistics and ranks for the 64-token tile whose fp32
// logits (logit_bias included) are in s_logit[tt * LD + e], with NW
// wavefronts (64 NW threads).  A group of 16 lanes handles one token (4
// tokens per wavefront at a time, 64 / NW tokens per wavefront in all); lane
// gl holds experts gl, gl + 16, ...
template <int NB, int NW>
__device__ __forceinline__ void select_tile(const float* s_logit, int t0, int n_tok, int N, int k,
                            const float* __restrict__ select_bias, int32_t* __restrict__ topk_idx,
                            float* __restrict__ topk_gate, int32_t* __restrict__ lrank,
                            int32_t* __restrict__ blk_counts, float* __restrict__ blk_psum,
                            uint32_t (*s_mask)[2], float* s_psum, int32_t* s_sel) {
  using S = RouteShape<NB>;
  constexpr int G = S::G, EPL = S::EPL, TPW = S::TPW, LD = S::LD, NP = S::NP;
  constexpr int TOKW = kRouteTokens / NW;  // tokens per wavefront
  static_assert(TOKW % TPW == 0, "whole lane groups");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = lane / G;
  const int gl = lane % G;
  float psum[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) psum[i] = 0.f;
  // this lane's experts' selection biases, the same for every token
  float sbias[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = gl + G * i;
    sbias[i] = (e < N && select_bias != nullptr) ? select_bias[e] : 0.f;
  }

#pragma unroll 1
  for (int base = 0; base < TOKW; base += TPW) {
    const int tt = wave * TOKW + base + grp;  // token inside the block
    const int t = t0 + tt;
    const bool tok_ok = t < n_tok;          // uniform inside a lane group

    float r[EPL];
    uint64_t okey[EPL];  // selection order of each of this lane's experts
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = gl + G * i;
      r[i] = e < N ? s_logit[tt * LD + e] : -INFINITY;
      const float key = (e < N && select_bias != nullptr) ? __fadd_rn(r[i], sbias[i]) : r[i];
      okey[i] = e < N ? order_key(key, e) : 0ull;
    }

    // router probabilities over all N experts (balance statistic P)
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < EPL; ++i) m = fmaxf(m, r[i]);
    m = group_max<G>(m);
    float se = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      // exp2-based exponential: the statistic P tolerates its ~1e-7 relative error
      r[i] = (gl + G * i < N) ? __expf(r[i] - m) : 0.f;  // r now holds exp(r - m)
      se += r[i];
    }
    se = group_sum<G>(se);
    if (tok_ok) {
#pragma unroll
      for (int i = 0; i < EPL; ++i) psum[i] += r[i] / se;
    }

    // k rounds of arg-max over the group; the owner lane marks the winner
    // taken; lane s keeps the winner of round s
    uint32_t taken = 0u;
    int slot_e = 0;
#pragma unroll 1
    for (int s = 0; s < k; ++s) {
      uint64_t best = 0ull;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const uint64_t o = ((taken >> i) & 1u) ? 0ull : okey[i];
        best = o > best ? o : best;
      }
      best = group16_max(best);
      const int be = static_cast<int>(0xffffffffu - static_cast<uint32_t>(best));
      if (be % G == gl) taken |= 1u << (be / G);
      if (gl == s) slot_e = be;
    }

    // gates: softmax over the kept (unbiased) logits, slot s held by lane s
    const bool holds = gl < k;
    const float slot_r = holds ? s_logit[tt * LD + slot_e] : -INFINITY;
    const float gm = group_max<G>(slot_r);
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

  // add the 4 lane groups of the wavefront (fixed order), then one row per wave
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    psum[i] += __shfl_xor(psum[i], 16, 64);
    psum[i] += __shfl_xor(psum[i], 32, 64);
  }
  if (grp == 0) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) s_psum[wave * NP + gl + G * i] = psum[i];
  }
  __syncthreads();

  // ---------------------------------------------- block statistics and ranks
  const int n_here = min(kRouteTokens, n_tok - t0);
  for (int i = tid; i < n_here * k; i += 64 * NW) {
    const int tt = i / k, s = i - tt * k;
    const int e = s_sel[tt * kMaxTopK + s];
    const uint64_t mk = static_cast<uint64_t>(s_mask[e][0]) |
                        (static_cast<uint64_t>(s_mask[e][1]) << 32);
    const uint64_t below = tt == 0 ? 0ull : (mk & ((1ull << tt) - 1ull));
    lrank[static_cast<size_t>(t0 + tt) * k + s] = __popcll(below);
  }
  for (int e = tid; e < N; e += 64 * NW) {
    blk_counts[static_cast<size_t>(blockIdx.x) * N + e] =
        __popc(s_mask[e][0]) + __popc(s_mask[e][1]);
    float acc_p = 0.f;
    for (int w = 0; w < NW; ++w) acc_p += s_psum[w * NP + e];
    blk_psum[static_cast<size_t>(blockIdx.x) * N + e] = acc_p;
  }
}

struct RouteArgs {
  const void* x;
  const void* wr;
  const float* logit_bias;
  const float* select_bias;
  int n_tok, d, N, k;
  int ksplit;             // workgroups along the reduction dimension
  int steps_per_split;    // K steps (64-byte row slices) per split
  float* partial;         // [ksplit, T, N] when ksplit > 1
  float* logits_out;      // [T, N] or NULL
  int32_t* topk_idx;
  float* topk_gate;
  int32_t* lrank;
  int32_t* blk_counts;
  float* blk_psum;
};

// Router GEMM on a global -> LDS ring; FUSED: followed by the selection.
template <typename T, int NB, bool FUSED>
__global__ __launch_bounds__(256) void route_gemm_kernel(RouteArgs a) {
  using S = RouteShape<NB>;
  constexpr int NP = S::NP, LD = S::LD, STAGES = S::STAGES, STAGE = S::STAGE, LPW = S::LPW;
  constexpr int TB = S::TB, EB = S::EB;

  __shared__ __attribute__((aligned(1024))) char s_union[S::UNION];
  __shared__ uint32_t s_mask[NP][2];             // tokens of the block that chose e
  __shared__ float s_psum[4 * NP];               // per-wavefront probability sums
  __shared__ int32_t s_sel[kRouteTokens * kMaxTopK];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t0 = blockIdx.x * kRouteTokens;
  const int ks = blockIdx.y;
  if (FUSED)
    for (int i = tid; i < NP * 2; i += 256) (&s_mask[0][0])[i] = 0u;

  // ------------------------------------------------------------ router GEMM
  const size_t row_bytes = static_cast<size_t>(a.d) * sizeof(T);
  const int nsteps = static_cast<int>(row_bytes / kRowBytes);
  const int k0 = ks * a.steps_per_split;
  const int nloc = min(a.steps_per_split, nsteps - k0);

  // ring block b: rows 16b .. 16b+15 of the stage; blocks 0-3 hold the 64
  // token rows, blocks 4 .. 4+NB-1 the router rows, the rest repeat block 0
  const int lchunk = ring_lane_chunk(lane);
  const char* src[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int b = wave * LPW + j;
    const int row = (b < 4 + NB ? b : 0) * 16 + (lane >> 2);
    const char* p;
    if (row < 64) {
      const int t = min(t0 + row, a.n_tok - 1);
      p = reinterpret_cast<const char*>(a.x) + static_cast<size_t>(t) * row_bytes;
    } else {
      const int e = min(row - 64, a.N - 1);
      p = reinterpret_cast<const char*>(a.wr) + static_cast<size_t>(e) * row_bytes;
    }
    src[j] = p + static_cast<size_t>(k0) * kRowBytes + lchunk * 16;
  }
  auto issue = [&](int step) {
    const size_t koff = static_cast<size_t>(min(step, nloc - 1)) * kRowBytes;
    char* st = s_union + (step % STAGES) * STAGE + wave * LPW * 1024;
#pragma unroll
    for (int j = 0; j < LPW; ++j) load_lds16(src[j] + koff, st + j * 1024);
  };

  const int wt = wave / S::WE, we = wave % S::WE;
  f32x4 acc[TB][EB];
#pragma unroll
  for (int i = 0; i < TB; ++i)
#pragma unroll
    for (int j = 0; j < EB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int p = 0; p < STAGES - 1; ++p) issue(p);
  const int frow = lane & 15, fchunk = lane >> 4;
  for (int s = 0; s < nloc; ++s) {
    // step s has landed once only the STAGES - 2 younger steps are pending
    wait_vmem<(STAGES - 2) * LPW>();
    stage_barrier();
    issue(s + STAGES - 1);  // into the buffer read in step s - 1
    const char* st = s_union + (s % STAGES) * STAGE;
    u32x4 af[TB], bf[EB];
#pragma unroll
    for (int i = 0; i < TB; ++i)
      af[i] = *reinterpret_cast<const u32x4*>(st + swz64((wt * TB + i) * 16 + frow, fchunk));
#pragma unroll
    for (int j = 0; j < EB; ++j)
      bf[j] = *reinterpret_cast<const u32x4*>(st + swz64(64 + (we * EB + j) * 16 + frow, fchunk));
#pragma unroll
    for (int i = 0; i < TB; ++i)
#pragma unroll
      for (int j = 0; j < EB; ++j) acc[i][j] = Mfma<T>::step(af[i], bf[j], acc[i][j]);
  }
  __syncthreads();  // drains the ring (tail re-reads included) before LDS reuse

  // ----------------------------------------------- partial logits: out, done
  if (!FUSED) {
    float* part = a.partial + static_cast<size_t>(ks) * a.n_tok * a.N;
#pragma unroll
    for (int i = 0; i < TB; ++i)
#pragma unroll
      for (int j = 0; j < EB; ++j) {
        const int e = (we * EB + j) * 16 + frow;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = t0 + (wt * TB + i) * 16 + 4 * fchunk + r;
          if (e < a.N && t < a.n_tok) part[static_cast<size_t>(t) * a.N + e] = acc[i][j][r];
        }
      }
    return;
  }

  // ------------------------------------------------------- logits to LDS
  float* s_logit = reinterpret_cast<float*>(s_union);
#pragma unroll
  for (int i = 0; i < TB; ++i)
#pragma unroll
    for (int j = 0; j < EB; ++j) {
      const int e = (we * EB + j) * 16 + frow;
      const float lb = (a.logit_bias != nullptr && e < a.N) ? a.logit_bias[e] : 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tt = (wt * TB + i) * 16 + 4 * fchunk + r;
        const float v = acc[i][j][r] + lb;
        s_logit[tt * LD + e] = v;
        if (a.logits_out != nullptr && e < a.N && t0 + tt < a.n_tok)
          a.logits_out[static_cast<size_t>(t0 + tt) * a.N + e] = v;
      }
    }
  __syncthreads();
  select_tile<NB, 4>(s_logit, t0, a.n_tok, a.N, a.k, a.select_bias, a.topk_idx, a.topk_gate,
                     a.lrank, a.blk_counts, a.blk_psum, s_mask, s_psum, s_sel);
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
  select_tile<NB, NT / 64>(s_logit, t0, a.n_tok, a.N, a.k, a.select_bias, a.topk_idx,
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
