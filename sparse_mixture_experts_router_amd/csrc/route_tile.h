// One routing block (router GEMM, top-k selection, gates, block statistics),
// shared by the routing kernels (route.hip) and the all-token expert pass,
// whose gate/up launch runs the routing of its batch in one extra workgroup
// (grouped_gemm.hip).
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
#pragma once

#include "balance.h"
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
  // LDS of one routing block: the ring / logits union, then the per-expert
  // token masks, the per-wavefront probability sums and the selected experts
  static constexpr int OFF_MASK = UNION;
  static constexpr int OFF_PSUM = OFF_MASK + NP * 2 * 4;
  static constexpr int OFF_SEL = OFF_PSUM + 4 * NP * 4;
  static constexpr int LDS_BYTES = OFF_SEL + kRouteTokens * kMaxTopK * 4;
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
__device__ __forceinline__ void select_tile(const float* s_logit, int blk, int t0, int n_tok, int N, int k,
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
    blk_counts[static_cast<size_t>(blk) * N + e] =
        __popc(s_mask[e][0]) + __popc(s_mask[e][1]);
    float acc_p = 0.f;
    for (int w = 0; w < NW; ++w) acc_p += s_psum[w * NP + e];
    blk_psum[static_cast<size_t>(blk) * N + e] = acc_p;
  }
}


// Router GEMM of the 64-token block `bx`, reduction piece `ks`, on a global
// -> LDS ring, by one 256-thread workgroup; FUSED: followed by the
// selection.  `lds` holds RouteShape<NB>::LDS_BYTES, 1024-byte aligned.
template <typename T, int NB, bool FUSED>
__device__ __forceinline__ void route_gemm_block(const RouteArgs& a, int bx, int ks, char* lds) {
  using S = RouteShape<NB>;
  constexpr int NP = S::NP, LD = S::LD, STAGES = S::STAGES, STAGE = S::STAGE, LPW = S::LPW;
  constexpr int TB = S::TB, EB = S::EB;

  char* const s_union = lds;
  auto s_mask = reinterpret_cast<uint32_t(*)[2]>(lds + S::OFF_MASK);  // tokens that chose e
  float* const s_psum = reinterpret_cast<float*>(lds + S::OFF_PSUM);  // per-wavefront sums
  int32_t* const s_sel = reinterpret_cast<int32_t*>(lds + S::OFF_SEL);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t0 = bx * kRouteTokens;
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
  select_tile<NB, 4>(s_logit, bx, t0, a.n_tok, a.N, a.k, a.select_bias, a.topk_idx, a.topk_gate,
                     a.lrank, a.blk_counts, a.blk_psum, s_mask, s_psum, s_sel);
}


// The routing of an all-token expert pass (AllTokenRoute, moe_internal.h),
// by one 256-thread workgroup.

template <typename T, int NB>
__device__ __forceinline__ void all_token_route(const AllTokenRoute& r, char* lds) {
  using S = RouteShape<NB>;
  constexpr int NP = S::NP;
  route_gemm_block<T, NB, true>(r.a, 0, 0, lds);
  // The selection's last phase only reads s_sel, s_mask and s_psum, which
  // are final since its barrier; the logits tile is dead.
  const auto s_mask = reinterpret_cast<const uint32_t(*)[2]>(lds + S::OFF_MASK);
  const float* const s_psum = reinterpret_cast<const float*>(lds + S::OFF_PSUM);
  const int32_t* const s_sel = reinterpret_cast<const int32_t*>(lds + S::OFF_SEL);
  const int tid = threadIdx.x;
  const int T_ = r.a.n_tok, N = r.a.N, k = r.a.k, G = N + r.S;
  for (int i = tid; i < T_ * k; i += 256) {
    const int t = i / k, s = i - t * k;
    const int e = s_sel[t * kMaxTopK + s];
    const uint64_t mk = static_cast<uint64_t>(s_mask[e][0]) |
                        (static_cast<uint64_t>(s_mask[e][1]) << 32);
    const int rank = __popcll(t == 0 ? 0ull : (mk & ((1ull << t) - 1ull)));
    r.inv_row[i] = (r.capacity <= 0 || rank < r.capacity) ? e * T_ + t : -1;
  }
  for (int e = tid; e < G; e += 256) {
    if (e < N) {
      const int c = __popc(s_mask[e][0]) + __popc(s_mask[e][1]);
      float ps = 0.f;  // the block sum, in the order of select_tile's
      for (int w = 0; w < 4; ++w) ps += s_psum[w * NP + e];
      r.counts[e] = c;
      r.prob_sum[e] = ps;
      if (r.user_counts != nullptr) r.user_counts[e] = c;
      if (r.user_prob_sum != nullptr) r.user_prob_sum[e] = ps;
    } else {
      r.counts[e] = T_;
    }
  }
  for (int g = tid; g <= G; g += 256) r.offsets[g] = g * T_;
  if (tid == 0) {
    const bool split = r.down_parts > 1;
    r.plan[kPlanParts] = split ? r.down_parts : 0;
    r.plan[kPlanRowSplit] = split ? 0 : G * T_;
    r.plan[kPlanStride] = split ? G * T_ : 0;
    r.plan[kPlanTailTiles] = 0;
  }
  if (r.f != nullptr || r.P != nullptr || r.aux != nullptr) {
    __syncthreads();  // counts and prob_sum written; the LDS is free
    balance_block(T_, N, k, r.counts, r.prob_sum, r.alpha, r.f, r.P, r.aux,
                  reinterpret_cast<float*>(lds));
  }
}

}  // namespace
}  // namespace moe
