// Grouped expert GEMMs on the matrix cores.
//
// Each expert is a SwiGLU feed-forward network ("MoE inference: the call
// centre with 256 specialists ...", "The bare mechanism": the FFN it replaces
// is down(act(gate(x)) * up(x)) with SiLU as the activation), run only on the
// rows routed to it.  With the rows of every expert laid out contiguously
// (expert-major, see permute.hip):
//
//   up pass    H[row, n] = SiLU(sum_j X[tok(row), j] Wg[e][n, j])
//                          * (sum_j X[tok(row), j] Wu[e][n, j])
//   down pass  Y[row, c] = sum_n H[row, n] Wd[e][c, n]
//
// Both are C = A B^T with the reduction dimension contiguous in A and B (the
// weights' [out, in] layout), so the MFMA fragments are plain 16-byte row
// reads.  A workgroup owns one BM-row tile of one expert (from the device-built
// tile list) and a BN-column slice; shared experts are extra groups whose
// rows are all tokens.  The up pass gathers X rows through sorted_tok instead
// of materialising a permuted copy, keeps gate and up accumulators side by
// side and applies SiLU(gate) * up in the epilogue, so the gate and up
// activations never reach memory.
//
// Pipeline: 4 wavefronts; per K step (128 bytes of every A row) the A and B
// slices of a later step are fetched into registers while the current ones
// are multiplied out of LDS (two LDS stages, one barrier per step that does
// not wait for the loads in flight).
//
// FP8 weights (TW = uint8_t: OCP E4M3 codes, one fp32 scale per output
// channel): a K step then reads 64 bytes of every weight row, and each
// 8-code chunk is widened to 8 bf16 (exactly) between its register and its
// LDS slot, so the LDS layout and the MFMAs are those of bf16 weights.  The
// scale multiplies each output channel's fp32 sum in the epilogue (before
// SiLU in the gated pass): sum_j x_j (q_nj s_n) = s_n sum_j x_j q_nj.
#include <type_traits>

#include "lds_ring.h"
#include "mfma.h"
#include "route_tile.h"

namespace moe {
namespace {


// All-token expert pass (GemmArgs' all_tok = T > 0): workgroup row b < G =
// all_groups is expert b on every token (rows b T .. b T + T - 1; the gated
// pass reads x rows 0 .. T - 1, the plain pass its own group's rows), with
// no tile list.  ROUTE (gated pass): workgroup (G, 0) routes the batch
// meanwhile (all_token_route), in this kernel's LDS.
template <typename T, typename TW, bool GATED, int BM, int BN, int WM, int WN, bool ROUTE = false>
__global__ __launch_bounds__(256) void grouped_gemm_kernel(GemmArgs g, AllTokenRoute route) {
  constexpr bool FP8W = sizeof(TW) == 1;
  constexpr int PD = (GATED || FP8W) ? 2 : 1;  // K steps of loads in flight
  static_assert(!FP8W || sizeof(T) == 2, "FP8 weights with bf16 activations");
  constexpr int ROWB = 128;
  constexpr int WROWB = FP8W ? 64 : ROWB;   // weight bytes of a row per K step
  constexpr int CPL = FP8W ? 2 : 1;         // 16-byte LDS chunks filled per 16-byte load
  constexpr int NMAT = GATED ? 2 : 1;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MB = WTM / 16, NBK = WTN / 16;
  constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB;
  constexpr int STAGE = A_BYTES + NMAT * B_BYTES;
  constexpr int A_LD = BM * 8 / 256;  // 16-byte chunks per thread per K step
  constexpr int B_LD = BN * 8 / 256 / CPL;  // 16-byte weight loads per thread per K step
  static_assert(WM * WN == 4, "4 wavefronts");
  static_assert(A_LD >= 1 && B_LD >= 1, "tile too small for 256 threads");
  static_assert(MB >= 1 && NBK >= 1, "wave tile below one MFMA block");

  static_assert(!ROUTE || (GATED && BM == 32), "routing in the all-token gate/up pass");
  static_assert(!ROUTE || RouteShape<4>::LDS_BYTES <= 2 * STAGE, "routing block LDS");

  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

  int e, m0, seg, mvalid, arow0;
  if (g.all_tok > 0) {
    e = blockIdx.x;
    if (e >= g.all_groups) {
      if constexpr (ROUTE) {
        if (blockIdx.y == 0) {
          if (route.a.N <= 16) all_token_route<T, 1>(route, smem);
          else if (route.a.N <= 32) all_token_route<T, 2>(route, smem);
          else all_token_route<T, 4>(route, smem);
        }
      }
      return;
    }
    m0 = 0;
    seg = e * g.all_tok;
    mvalid = g.all_tok;
    arow0 = GATED ? 0 : seg;  // every expert of the gated pass reads x rows 0 .. T - 1
  } else {
    const int tile = blockIdx.x;
    if (tile >= *g.ntiles) return;
    const int2 te = g.tiles[tile];
    e = te.x;
    m0 = te.y;
    seg = g.offsets[e];
    mvalid = min(BM, g.offsets[e + 1] - seg - m0);
    arow0 = seg;
  }
  const int n0 = blockIdx.y * BN;
  const bool split = !GATED && g.ksplit > 1;   // blockIdx.z: part of the reduction

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  const size_t row_bytes = static_cast<size_t>(g.k_dim) * sizeof(T);
  const size_t wrow_bytes = static_cast<size_t>(g.k_dim) * sizeof(TW);
  const size_t mat_elems = static_cast<size_t>(g.n_dim) * g.k_dim;
  const bool routed = e < g.n_experts;
  const int es = routed ? e : e - g.n_experts;
  const char* w0 = reinterpret_cast<const char*>(routed ? g.w0 : g.ws0) + es * mat_elems * sizeof(TW);
  const char* w1 = GATED ? reinterpret_cast<const char*>(routed ? g.w1 : g.ws1) + es * mat_elems * sizeof(TW)
                         : nullptr;

  // per-thread global sources as byte offsets (rows beyond the tile are
  // clamped to a valid row; their results are discarded in the epilogue)
  const char* a_base = reinterpret_cast<const char*>(g.a);
  size_t a_off[A_LD];
  int a_dst[A_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int c = tid + 256 * i;
    const int r = c >> 3, ch = c & 7;
    const int grow = arow0 + m0 + min(r, mvalid - 1);
    const int src_row = min(max(g.gather != nullptr ? g.gather[grow] : grow, 0), g.a_rows - 1);
    a_off[i] = static_cast<size_t>(src_row) * row_bytes + ch * 16;
    a_dst[i] = lds_swz(r, ch);
  }
  size_t b_off[B_LD];
  int b_dst[B_LD];  // first of the CPL consecutive chunks a load fills
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const int c = tid + 256 * i;
    const int r = c / (8 / CPL), ch = (c % (8 / CPL)) * CPL;
    const int n = min(n0 + r, g.n_dim - 1);
    b_off[i] = static_cast<size_t>(n) * wrow_bytes + (ch / CPL) * 16;
    b_dst[i] = r * 128 + ch;  // row and chunk, swizzled at the store
  }

  f32x4 acc[NMAT][MB][NBK];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NBK; ++j) acc[m][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  int nsteps = static_cast<int>(row_bytes / ROWB);
  if (split) {  // this workgroup's share of the K steps
    const int per = (nsteps + g.ksplit - 1) / g.ksplit;
    const int k0 = min(static_cast<int>(blockIdx.z) * per, nsteps - 1);  // loads stay in the row
    nsteps = max(min(per, nsteps - static_cast<int>(blockIdx.z) * per), 0);
#pragma unroll
    for (int i = 0; i < A_LD; ++i) a_off[i] += static_cast<size_t>(k0) * ROWB;
#pragma unroll
    for (int i = 0; i < B_LD; ++i) b_off[i] += static_cast<size_t>(k0) * WROWB;
  }

  // PD = 2: two register slots of K-step loads; step s + 2 is loaded while
  // step s is multiplied out of LDS and step s + 1 waits in the other slot,
  // so two steps of loads are in flight (the gated pass, which streams two
  // weight matrices, and FP8 weights, half the bytes per step).  PD = 1: one
  // slot, step s + 1 loaded during step s (the bf16 plain pass: with its
  // decode split's short K loops a deeper prologue measured slower).  Steps
  // past the end re-read the last one.
  u32x4 ra[PD][A_LD];
  u32x4 rb0[PD][B_LD], rb1[PD][B_LD];
  auto load_step = [&](int slot, int s) {
    const int sc = min(s, nsteps - 1);
    const size_t koff = static_cast<size_t>(sc) * ROWB;
    const size_t kwoff = static_cast<size_t>(sc) * WROWB;
#pragma unroll
    for (int i = 0; i < A_LD; ++i)
      ra[slot][i] = *reinterpret_cast<const u32x4*>(a_base + a_off[i] + koff);
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      rb0[slot][i] = *reinterpret_cast<const u32x4*>(w0 + b_off[i] + kwoff);
      if (GATED) rb1[slot][i] = *reinterpret_cast<const u32x4*>(w1 + b_off[i] + kwoff);
    }
    // issue them here, ahead of this step's MFMAs
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  auto store_step = [&](int slot, int stage) {
    char* nx = smem + stage * STAGE;
#pragma unroll
    for (int i = 0; i < A_LD; ++i) *reinterpret_cast<u32x4*>(nx + a_dst[i]) = ra[slot][i];
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const int r = b_dst[i] >> 7, ch = b_dst[i] & 127;
#pragma unroll
      for (int h = 0; h < CPL; ++h) {
        const int dst = lds_swz(r, ch + h);
        if (FP8W) {
          *reinterpret_cast<u32x4*>(nx + A_BYTES + dst) =
              e4m3x8_to_bf16(make_uint2(rb0[slot][i][2 * h], rb0[slot][i][2 * h + 1]));
          if (GATED)
            *reinterpret_cast<u32x4*>(nx + A_BYTES + B_BYTES + dst) =
                e4m3x8_to_bf16(make_uint2(rb1[slot][i][2 * h], rb1[slot][i][2 * h + 1]));
        } else {
          *reinterpret_cast<u32x4*>(nx + A_BYTES + dst) = rb0[slot][i];
          if (GATED) *reinterpret_cast<u32x4*>(nx + A_BYTES + B_BYTES + dst) = rb1[slot][i];
        }
      }
    }
  };
  auto compute = [&](int stage) {
    const char* st = smem + stage * STAGE;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const int ch = kc * 4 + (lane >> 4);
      u32x4 af[MB];
#pragma unroll
      for (int i = 0; i < MB; ++i)
        af[i] = *reinterpret_cast<const u32x4*>(st + lds_swz(wm * WTM + i * 16 + (lane & 15), ch));
#pragma unroll
      for (int j = 0; j < NBK; ++j) {
        const int br = wn * WTN + j * 16 + (lane & 15);
        const u32x4 bf0 = *reinterpret_cast<const u32x4*>(st + A_BYTES + lds_swz(br, ch));
#pragma unroll
        for (int i = 0; i < MB; ++i) acc[0][i][j] = Mfma<T>::step(af[i], bf0, acc[0][i][j]);
        if (GATED) {
          const u32x4 bf1 = *reinterpret_cast<const u32x4*>(st + A_BYTES + B_BYTES + lds_swz(br, ch));
#pragma unroll
          for (int i = 0; i < MB; ++i)
            acc[NMAT - 1][i][j] = Mfma<T>::step(af[i], bf1, acc[NMAT - 1][i][j]);
        }
      }
    }
  };

  if (nsteps > 0 && PD == 2) {
    load_step(0, 0);
    load_step(1, 1);
    store_step(0, 0);
    lds_barrier();
    // steps s (stage 0, slot 0) and s + 1 (stage 1, slot 1)
    for (int s = 0; s + 1 < nsteps; s += 2) {
      load_step(0, s + 2);
      compute(0);
      store_step(1, 1);
      lds_barrier();
      load_step(1, s + 3);
      compute(1);
      store_step(0, 0);
      lds_barrier();
    }
    if (nsteps & 1) compute(0);  // the last (even-numbered) step sits in stage 0
  } else if (nsteps > 0) {
    load_step(0, 0);
    store_step(0, 0);
    lds_barrier();
    for (int s = 0; s < nsteps; ++s) {
      const bool more = s + 1 < nsteps;
      if (more) load_step(0, s + 1);
      compute(s & 1);
      if (more) store_step(0, (s + 1) & 1);
      lds_barrier();
    }
  }

  // epilogue
  T* out = static_cast<T*>(g.out);
  const float* scale0 = nullptr;  // FP8 weights: per-output-channel scales of this expert
  const float* scale1 = nullptr;
  if (FP8W) {
    scale0 = (routed ? g.sc0 : g.ssc0) + static_cast<size_t>(es) * g.n_dim;
    if (GATED) scale1 = (routed ? g.sc1 : g.ssc1) + static_cast<size_t>(es) * g.n_dim;
  }
#pragma unroll
  for (int i = 0; i < MB; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = wm * WTM + i * 16 + 4 * (lane >> 4) + r;
      if (row >= mvalid) continue;
      T* orow = out + static_cast<size_t>(seg + m0 + row) * g.n_dim;
#pragma unroll
      for (int j = 0; j < NBK; ++j) {
        const int col = n0 + wn * WTN + j * 16 + (lane & 15);
        if (col >= g.n_dim) continue;
        float v;
        if (GATED) {
          float a = acc[0][i][j][r], b = acc[NMAT - 1][i][j][r];
          if (FP8W) {
            a *= scale0[col];
            b *= scale1[col];
          }
          v = a / (1.0f + __expf(-a)) * b;
        } else {
          v = acc[0][i][j][r];
          if (FP8W) v *= scale0[col];
        }
        if (split)
          g.out_part[(static_cast<size_t>(blockIdx.z) * g.a_rows + seg + m0 + row) * g.n_dim + col] = v;
        else
          orow[col] = from_f32<T>(v);
      }
    }
  }
}

template <typename T, typename TW, bool GATED, int BM, int BN, int WM, int WN>
hipError_t launch_t(const GemmArgs& g, const AllTokenRoute* route, hipStream_t s) {
  const unsigned rows = g.all_tok > 0 ? g.all_groups + (route != nullptr ? 1 : 0) : g.tiles_cap;
  dim3 grid(rows, (g.n_dim + BN - 1) / BN, (!GATED && g.ksplit > 1) ? g.ksplit : 1);
  if constexpr (GATED && BM == 32) {
    if (route != nullptr) {
      hipLaunchKernelGGL((grouped_gemm_kernel<T, TW, GATED, BM, BN, WM, WN, true>), grid, dim3(256),
                         0, s, g, *route);
      return hipGetLastError();
    }
  }
  if (route != nullptr) return hipErrorInvalidValue;
  hipLaunchKernelGGL((grouped_gemm_kernel<T, TW, GATED, BM, BN, WM, WN>), grid, dim3(256), 0, s, g,
                     AllTokenRoute{});
  return hipGetLastError();
}

template <typename T, typename TW, bool GATED>
hipError_t launch_bm(const GemmArgs& g, int bm, const AllTokenRoute* route, hipStream_t s) {
  if (bm == 32) return launch_t<T, TW, GATED, 32, 64, 1, 4>(g, route, s);
  if (g.all_tok > 0) return hipErrorInvalidValue;  // all-token passes: 32-row tiles
  return launch_t<T, TW, GATED, 128, 128, 2, 2>(g, route, s);
}

}  // namespace

hipError_t launch_generic_gemm(int dtype, bool gated, int bm, const GemmArgs& g, hipStream_t s,
                               const AllTokenRoute* route) {
  if (route != nullptr && (!gated || g.all_tok <= 0 || g.all_tok > kRouteTokens ||
                           route->a.N > 64 || route->a.ksplit != 1))
    return hipErrorInvalidValue;
  if (dtype == 1 && g.wfp8)
    return gated ? launch_bm<bf16_t, uint8_t, true>(g, bm, route, s)
                 : launch_bm<bf16_t, uint8_t, false>(g, bm, route, s);
  if (g.wfp8) return hipErrorInvalidValue;
  if (dtype == 1)
    return gated ? launch_bm<bf16_t, bf16_t, true>(g, bm, route, s)
                 : launch_bm<bf16_t, bf16_t, false>(g, bm, route, s);
  return gated ? launch_bm<float, float, true>(g, bm, route, s)
               : launch_bm<float, float, false>(g, bm, route, s);
}

// Split of the down pass over workgroups for few-row (weight-streaming)
// shapes: as many pieces as keep every workgroup of the pass resident at
// once (about 4 of these 24 KB-LDS workgroups per CU), so the pass runs as
// one round with all of its loads in flight, each piece >= 16 K steps.  FP8
// weights stream half the bytes per K step: twice the pieces (measured on
// the Mixtral-shaped decode: down pass 0.118 -> 0.108 ms).
// tiles_est: row tiles the pass will have (at most its tile capacity).
int down_split(int dtype, bool fp8w, const GemmPick& pick, long tiles_est, int n_dim, int k_dim,
               int cus) {
  if (pick.variant != 0 || pick.bm != 32) return 1;
  const long blocks = tiles_est * ((n_dim + 63) / 64);
  const int nsteps = static_cast<int>(static_cast<long>(k_dim) * (dtype == 1 ? 2 : 4) / 128);
  long ks = blocks > 0 ? ((fp8w ? 8L : 4L) * cus) / blocks : 1;
  ks = ks > 8 ? 8 : ks;
  ks = ks > nsteps / 16 ? nsteps / 16 : ks;
  return ks < 2 ? 1 : static_cast<int>(ks);
}

GemmPick pick_gemm(int dtype, bool /*fp8w*/, bool /*gated*/, long rows_per_expert, size_t a_bytes,
                   size_t w_bytes, int k_dim) {
  const bool small_offsets = a_bytes < (size_t{1} << 32) && w_bytes < (size_t{1} << 32);
  // the large-tile kernel streams whole pairs of 128-byte row buffers
  if (dtype != 1 || !small_offsets || k_dim % 128 != 0)
    return GemmPick{0, rows_per_expert <= 48 ? 32 : 128};
  if (rows_per_expert <= 48) return GemmPick{0, 32};
  // 256-row tiles from 192 rows per expert on: a part-filled tile's clamped
  // rows re-read one line, so the fuller tiles' higher FLOPs per staged byte
  // win.  DeepSeek-V3-shaped prefill (256 rows per expert): 8.14 -> 7.83 ms
  // with bf16 weights, 7.99 -> 7.11 ms with FP8 (128-row tiles before).
  if (rows_per_expert >= 192) return GemmPick{1, 256};
  return GemmPick{1, 128};
}

hipError_t launch_gemm(int dtype, bool gated, GemmPick pick, const GemmArgs& g, hipStream_t s,
                       const AllTokenRoute* route) {
  if (g.all_tok > 0 && pick.variant != 0) return hipErrorInvalidValue;
  if (pick.variant == 1 && dtype == 1) return launch_expert_gemm(gated, pick.bm, g, s);
  return launch_generic_gemm(dtype, gated, pick.bm, g, s, route);
}

}  // namespace moe
