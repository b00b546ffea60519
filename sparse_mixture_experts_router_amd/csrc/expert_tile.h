// Pieces of the large-tile expert GEMM kernel (expert_gemm.hip): the work
// decode of a workgroup in each of its modes and the tile epilogue.
#pragma once

#include "moe_internal.h"

namespace moe {

// Calls of one kind spread over `slots` MFMA slots: slots per call (>= 1).
constexpr int slots_per(int slots, int calls) {
  return calls > 0 && slots / calls > 0 ? slots / calls : 1;
}

// Work items: the (row tile, column tile) pairs of the scan's item list, then
// (plain pass only) the pieces (part, tile, column tile) of the last `tail`
// row tiles when the scan split them over their reduction.  Each XCD (blocks
// take XCDs round-robin) gets an equal contiguous share of both lists and
// runs it in order, so the workgroups it runs at once are one block of the
// list: one expert's row tiles next to a band of its weight tiles.  Returns
// false for a block with no work; part = -1 for an unsplit item, else the
// piece's index among `parts`.
__device__ __forceinline__ bool decode_work(const GemmArgs& g, bool gated, int cols, int& tile,
                                            int& nt, int& part, int& parts) {
  const int bid = blockIdx.x, xcd = bid & 7, idx = bid >> 3;
  const int n_nt = (g.n_dim + cols - 1) / cols;
  const int ntl = *g.ntiles;
  int tail = 0;
  parts = 1;
  if (!gated && g.plan != nullptr) {
    tail = g.plan[kPlanTailTiles];
    if (tail > 0) parts = g.plan[kPlanParts];
  }
  const int nrm = ntl - tail;
  const long w_nrm = g.nitems != nullptr ? *g.nitems : static_cast<long>(nrm) * n_nt;
  const long w_spl = static_cast<long>(tail) * n_nt * parts;
  const long n_lo = w_nrm * xcd / 8, n_cnt = w_nrm * (xcd + 1) / 8 - n_lo;
  const long s_lo = w_spl * xcd / 8, s_cnt = w_spl * (xcd + 1) / 8 - s_lo;
  part = -1;
  if (idx < n_cnt) {
    const int v = g.items[n_lo + idx];
    tile = v >> kItemColBits;
    nt = v & ((1 << kItemColBits) - 1);
    return true;
  }
  if (idx - n_cnt < s_cnt) {
    const int lin = static_cast<int>(s_lo + idx - n_cnt);
    part = lin / (tail * n_nt);
    const int rem = lin - part * (tail * n_nt);
    tile = nrm + rem / n_nt;
    nt = rem % n_nt;
    return true;
  }
  return false;
}

// Work of the weight-gradient mode: tile w of groups x row tiles x column
// tiles, group-major.  Inside a group the tiles go in bands of kKBand row
// tiles, column by column inside a band, and the list is cut into chunks of
// kKChunk tiles (4 x 4 blocks) dealt to the 8 XCDs in turn:
//  * a chunk fetches 4 row tiles and 4 column tiles into one L2 for its 16
//    tiles (a line of 16 tiles along the smaller dimension needed 1 + 16 and
//    took 3.06 against 2.91 ms for the Mixtral-shaped weight gradients);
//  * each group's tiles spread over the XCDs, since one group's reduction
//    can be many times another's (under a skewed router a hot expert's tiles
//    in 128-tile chunks sat on one XCD: 8.4 instead of 5.5 ms for the
//    Qwen3-shaped weight gradients).
constexpr int kKBand = 4, kKChunk = 16;
__device__ __forceinline__ bool decode_kwork(const GemmArgs& g, int bm, int cols, int& grp,
                                             int& m0, int& n0) {
  const int mt = (g.a_rows + bm - 1) / bm, nt = (g.n_dim + cols - 1) / cols;
  const int bid = blockIdx.x, xcd = bid & 7, idx = bid >> 3;
  const long per = static_cast<long>(mt) * nt;
  const long w = (static_cast<long>(idx / kKChunk) * 8 + xcd) * kKChunk + idx % kKChunk;
  if (w >= per * g.groups) return false;
  grp = static_cast<int>(w / per);
  const int rem = static_cast<int>(w - grp * per);
  const int band = rem / (kKBand * nt);
  const int hb = min(kKBand, mt - band * kKBand);  // rows of this band
  const int r = rem - band * kKBand * nt;
  m0 = (band * kKBand + r % hb) * bm;
  n0 = (r / hb) * cols;
  return true;
}
inline long kmajor_grid(const GemmArgs& g, int bm, int cols) {
  const long mt = (g.a_rows + bm - 1) / bm, nt = (g.n_dim + cols - 1) / cols;
  const long chunks = (mt * nt * g.groups + kKChunk - 1) / kKChunk;
  return 8L * ((chunks + 7) / 8) * kKChunk;
}

// Grid of the large-tile kernels: every XCD's share of the work items fits in
// blocks / 8 slots (the split pieces number at most one round of g.cus
// workgroups).
inline long expert_grid(const GemmArgs& g, bool gated, int cols) {
  const long n_nt = (g.n_dim + cols - 1) / cols;
  const long per_xcd = (static_cast<long>(g.tiles_cap) * n_nt + 7) / 8 +
                       (gated ? 0 : (g.cus + 7) / 8) + 1;
  return 8 * per_xcd;
}

// 16-byte store with the non-temporal policy.
__device__ __forceinline__ void store16(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// Writes a wavefront's accumulator block (GATED: SiLU(gate) * up first) in
// passes of PCOLS columns per row: each pass is staged row-major in LDS at
// stg (rows padded by 16 bytes, so the four row groups of an MFMA result
// land in distinct banks), then leaves in whole 16-byte row chunks.
//  SBF16 : staged and written as bf16, 64 columns (128 bytes) per pass;
//  else  : staged as fp32, FCOLS columns per pass (32, or 64 where the LDS
//          holds 8 WTM (256 + 16) bytes of staging), written as bf16 (8
//          columns per lane) or, if out_f32, as fp32 (4 columns per lane).
//          The plain pass uses this one path for both of its outputs, so
//          the accumulators have a single consumer.  With 64 columns every
//          bf16 row write is a whole 128-byte line.
// Row i of the block goes to out[(row0 + i) * ld + col0 + ...]; rows >=
// rows_valid and columns >= cols_valid are not written.
// SCALED (FP8 weights): each accumulator is first multiplied by its output
// column's scale, sc0 for the gate (or plain) columns, sc1 for the up
// columns; both indexed by the output column, col0 + ... .
// The global stores carry the non-temporal policy: no later work of the same
// launch reads an output tile, and keeping them out of the caches leaves room
// for the activation rows and weights other tiles still reuse.
template <bool GATED, bool SBF16, int MB, int NB, int WTM, bool SCALED = false, int FCOLS = 32>
__device__ __forceinline__ void store_block(const f32x4 (&acc)[MB][NB], char* stg, int lane,
                                            void* out, bool out_f32, size_t ld, long row0,
                                            int rows_valid, int col0, int cols_valid,
                                            const float* sc0 = nullptr,
                                            const float* sc1 = nullptr) {
  constexpr int NOUT = GATED ? NB / 2 : NB;
  constexpr int ES = SBF16 ? 2 : 4;              // staged element bytes
  constexpr int PCOLS = SBF16 ? 64 : FCOLS;      // columns per pass
  constexpr int PB = PCOLS / 16;                 // 16-column blocks per pass
  constexpr int SROW = PCOLS * ES + 16;
  static_assert(FCOLS == 32 || FCOLS == 64, "fp32 staging width");
  static_assert(NOUT % PB == 0, "whole passes");
#pragma unroll
  for (int pass = 0; pass < NOUT / PB; ++pass) {
    float s0v[PB], s1v[PB];  // this pass's column scales (SCALED)
#pragma unroll
    for (int jj = 0; jj < PB; ++jj) {
      const int sc = min(col0 + (pass * PB + jj) * 16 + (lane & 15), cols_valid - 1);
      s0v[jj] = SCALED ? sc0[sc] : 1.0f;
      s1v[jj] = SCALED && GATED ? sc1[sc] : 1.0f;
    }
#pragma unroll
    for (int i = 0; i < MB; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = i * 16 + 4 * (lane >> 4) + r;
#pragma unroll
        for (int jj = 0; jj < PB; ++jj) {
          const int j = pass * PB + jj;
          float v;
          if (GATED) {
            float a = acc[i][j][r], b = acc[i][j + NOUT][r];
            if (SCALED) {
              a *= s0v[jj];
              b *= s1v[jj];
            }
            v = a * __builtin_amdgcn_rcpf(1.0f + __expf(-a)) * b;
          } else {
            v = acc[i][j][r];
            if (SCALED) v *= s0v[jj];
          }
          if (SBF16)
            *reinterpret_cast<bf16_t*>(stg + row * SROW + (jj * 16 + (lane & 15)) * ES) =
                f32_to_bf16(v);
          else
            *reinterpret_cast<float*>(stg + row * SROW + (jj * 16 + (lane & 15)) * ES) = v;
        }
      }
    }
    if (SBF16) {
      const int col = col0 + pass * 64 + (lane & 7) * 8;
#pragma unroll
      for (int q = 0; q < WTM / 8; ++q) {
        const int row = q * 8 + (lane >> 3);
        const u32x4 v = *reinterpret_cast<const u32x4*>(stg + row * SROW + (lane & 7) * 16);
        if (row < rows_valid && col < cols_valid)
          store16(static_cast<bf16_t*>(out) + static_cast<size_t>(row0 + row) * ld + col, v);
      }
    } else if (out_f32) {
      constexpr int LPR = PCOLS / 4;  // lanes per row, 4 columns each
      const int col = col0 + pass * PCOLS + (lane % LPR) * 4;
#pragma unroll
      for (int q = 0; q < WTM * LPR / 64; ++q) {
        const int row = q * (64 / LPR) + lane / LPR;
        const u32x4 v = *reinterpret_cast<const u32x4*>(stg + row * SROW + (lane % LPR) * 16);
        if (row < rows_valid && col < cols_valid)
          store16(static_cast<float*>(out) + static_cast<size_t>(row0 + row) * ld + col, v);
      }
    } else {
      constexpr int LPR = PCOLS / 8;  // lanes per row, 8 columns each
      const int col = col0 + pass * PCOLS + (lane % LPR) * 8;
#pragma unroll
      for (int q = 0; q < WTM * LPR / 64; ++q) {
        const int row = q * (64 / LPR) + lane / LPR;
        const char* src = stg + row * SROW + (lane % LPR) * 32;
        const f32x4 a = *reinterpret_cast<const f32x4*>(src);
        const f32x4 b = *reinterpret_cast<const f32x4*>(src + 16);
        u32x4 v;
        v[0] = f32_to_bf16(a[0]) | (static_cast<uint32_t>(f32_to_bf16(a[1])) << 16);
        v[1] = f32_to_bf16(a[2]) | (static_cast<uint32_t>(f32_to_bf16(a[3])) << 16);
        v[2] = f32_to_bf16(b[0]) | (static_cast<uint32_t>(f32_to_bf16(b[1])) << 16);
        v[3] = f32_to_bf16(b[2]) | (static_cast<uint32_t>(f32_to_bf16(b[3])) << 16);
        if (row < rows_valid && col < cols_valid)
          store16(static_cast<bf16_t*>(out) + static_cast<size_t>(row0 + row) * ld + col, v);
      }
    }
  }
}

}  // namespace moe
