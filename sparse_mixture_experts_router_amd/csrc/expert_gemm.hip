// Large-tile bf16 grouped expert GEMM for gfx950 (prefill shapes).
//
// Same computation as grouped_gemm.hip (SwiGLU experts of "MoE inference: the
// call centre with 256 specialists ...", "The bare mechanism", each run only on
// its routed rows):
//   gated  : H[row, n] = SiLU(X Wg[e]^T)[row, n] * (X Wu[e]^T)[row, n]
//   plain  : Y[row, c] = (H Wd[e]^T)[row, c]
// organised for the matrix cores and the LDS of a CDNA4 compute unit:
//
//  * one workgroup = 4 wavefronts owns a BM x BNE tile (BNE effective
//    columns: for the gated pass half are gate rows and half are up rows of
//    the same output columns, so SiLU(gate) * up is formed in registers);
//  * operands arrive in LDS through global_load_lds_dwordx4 (16 bytes per
//    lane straight from global memory into LDS, no register staging), two
//    stages, one barrier per K step; each lane fetches the chunk that lands
//    in its slot of an XOR-swizzled 128-byte row so that the ds_read_b128
//    fragment reads of the MFMA loop are spread over all banks;
//  * each wavefront computes a (BM / WM) x (BNE / WN) block with
//    v_mfma_f32_16x16x32_bf16, so every 16-byte fragment read from LDS feeds
//    BNE / WN / 16 (A) or BM / WM / 16 (B) MFMAs;
//  * blocks are renumbered so that each of the 8 XCDs (which take workgroups
//    round-robin) works through a contiguous range of the (row tile, column
//    tile) order, in which consecutive tiles share a weight tile: the row
//    tiles of one expert read the same weights while they are in that XCD's
//    L2.
#include "mfma.h"

namespace moe {
namespace {

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(1))) void* global_void_ptr;

__device__ __forceinline__ void load_lds16(const char* src, char* lds_dst) {
  __builtin_amdgcn_global_load_lds((global_void_ptr)(src), (lds_void_ptr)(lds_dst), 16, 0, 0);
}

// s_waitcnt vmcnt(0) with the other counters left alone (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]).
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <bool GATED, int BM, int BNE, int WM, int WN>
__global__ __launch_bounds__(256, 1) void expert_gemm_kernel(GemmArgs g) {
  constexpr int ROWB = 128;                 // bytes of every row per K step (64 bf16)
  constexpr int ROWS = BM + BNE;            // rows staged per K step
  constexpr int STAGE = ROWS * ROWB;
  constexpr int BLOCKS = ROWS / 8;          // 1 KB LDS blocks per stage
  constexpr int WTM = BM / WM, WTN = BNE / WN;
  constexpr int MB = WTM / 16, NB = WTN / 16;
  constexpr int NOUT = GATED ? NB / 2 : NB; // output column blocks per wave
  constexpr int COLS = GATED ? BNE / 2 : BNE;   // output columns per tile
  static_assert(WM * WN == 4 && BLOCKS % 4 == 0 && BM % 32 == 0 && BNE % 32 == 0,
                "4 wavefronts, whole blocks");
  static_assert(!GATED || (BNE / 2) % (BNE / 32 * 8) == 0, "a wave's B blocks are all gate or all up");
  static_assert(!GATED || NB % 2 == 0, "gated tiles pair gate and up blocks");

  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

  // ------------------------------------------------------- tile of this block
  const int nblk = gridDim.x;
  const int bid = blockIdx.x;
  const int xq = nblk >> 3, xr = nblk & 7, xcd = bid & 7;
  const int lin = xcd * xq + min(xcd, xr) + (bid >> 3);
  const int tile = lin % g.tiles_cap;
  const int nt = lin / g.tiles_cap;
  if (tile >= *g.ntiles) return;
  const int2 te = g.tiles[tile];
  const int e = te.x, m0 = te.y;
  const int seg = g.offsets[e];
  const int mvalid = min(BM, g.offsets[e + 1] - seg - m0);
  const int n0 = nt * COLS;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  const size_t row_bytes = static_cast<size_t>(g.k_dim) * 2;
  const size_t mat_bytes = static_cast<size_t>(g.n_dim) * row_bytes;
  const bool routed = e < g.n_experts;
  const int es = routed ? e : e - g.n_experts;
  const char* w0 = reinterpret_cast<const char*>(routed ? g.w0 : g.ws0) + es * mat_bytes;
  const char* w1 = GATED ? reinterpret_cast<const char*>(routed ? g.w1 : g.ws1) + es * mat_bytes
                         : nullptr;

  // ------------------------------------------ this lane's global sources
  // Staged rows: A rows 0 .. BM-1 (BM/8 blocks of 8 rows), then B rows (for
  // the gated pass: COLS gate rows, then COLS up rows).  Each wavefront loads
  // BM/32 A blocks and BNE/32 B blocks; lane l fills physical chunk l % 8 of
  // row l / 8 of a block, i.e. logical chunk (l % 8) ^ (l / 8) of that row.
  // Sources are a wave-uniform base plus a 32-bit per-lane byte offset (the
  // host keeps every operand below 4 GiB per base).
  constexpr int A_BPW = BM / 32, B_BPW = BNE / 32;
  const int lchunk = (lane & 7) ^ (lane >> 3);
  const char* const a_base = reinterpret_cast<const char*>(g.a);
  uint32_t a_off[A_BPW];
#pragma unroll
  for (int j = 0; j < A_BPW; ++j) {
    const int R = (wave * A_BPW + j) * 8 + (lane >> 3);
    const int grow = seg + m0 + min(R, mvalid - 1);
    const int srow = min(max(g.gather != nullptr ? g.gather[grow] : grow, 0), g.a_rows - 1);
    a_off[j] = static_cast<uint32_t>(srow) * static_cast<uint32_t>(row_bytes) + lchunk * 16;
  }
  // B blocks of this wave: rows jb0 .. jb0 + 8*B_BPW - 1 of the B part; in the
  // gated pass waves 0-1 hold gate rows and waves 2-3 up rows.
  const int jb0 = wave * B_BPW * 8;
  const bool up_rows = GATED && jb0 >= COLS;
  const char* const b_base = (up_rows ? w1 : w0) + static_cast<size_t>(n0) * row_bytes;
  uint32_t b_off[B_BPW];
#pragma unroll
  for (int j = 0; j < B_BPW; ++j) {
    const int jb = jb0 + j * 8 + (lane >> 3) - (up_rows ? COLS : 0);
    const int n = min(n0 + jb, g.n_dim - 1);
    b_off[j] = static_cast<uint32_t>(n - n0) * static_cast<uint32_t>(row_bytes) + lchunk * 16;
  }

  f32x4 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // LDS row of B fragment block j for this wave
  auto b_row = [&](int j) {
    if (GATED) {
      const int half = j < NOUT ? 0 : COLS;
      const int jj = j < NOUT ? j : j - NOUT;
      return BM + half + wn * (WTN / 2) + jj * 16 + (lane & 15);
    }
    return BM + wn * WTN + j * 16 + (lane & 15);
  };

  const int nsteps = static_cast<int>(row_bytes / ROWB);
  char* const a_lds = smem + wave * A_BPW * 1024;
  char* const b_lds = smem + BM * ROWB + wave * B_BPW * 1024;
  auto issue = [&](int step, int buf) {
    const uint32_t koff = static_cast<uint32_t>(step) * ROWB;
#pragma unroll
    for (int j = 0; j < A_BPW; ++j)
      load_lds16(a_base + (a_off[j] + koff), a_lds + buf * STAGE + j * 1024);
#pragma unroll
    for (int j = 0; j < B_BPW; ++j)
      load_lds16(b_base + (b_off[j] + koff), b_lds + buf * STAGE + j * 1024);
  };
  issue(0, 0);

  for (int s = 0; s < nsteps; ++s) {
    wait_vmem_all();
    __syncthreads();
    if (s + 1 < nsteps) issue(s + 1, (s + 1) & 1);
    const char* st = smem + (s & 1) * STAGE;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const int ch = kc * 4 + (lane >> 4);
      u32x4 af[MB];
#pragma unroll
      for (int i = 0; i < MB; ++i)
        af[i] = *reinterpret_cast<const u32x4*>(st + lds_swz(wm * WTM + i * 16 + (lane & 15), ch));
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const u32x4 bf = *reinterpret_cast<const u32x4*>(st + lds_swz(b_row(j), ch));
#pragma unroll
        for (int i = 0; i < MB; ++i) acc[i][j] = Mfma<bf16_t>::step(af[i], bf, acc[i][j]);
      }
    }
  }

  // -------------------------------------------------------------- epilogue
  bf16_t* out = static_cast<bf16_t*>(g.out);
#pragma unroll
  for (int i = 0; i < MB; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = wm * WTM + i * 16 + 4 * (lane >> 4) + r;
      if (row >= mvalid) continue;
      bf16_t* orow = out + static_cast<size_t>(seg + m0 + row) * g.n_dim;
#pragma unroll
      for (int j = 0; j < NOUT; ++j) {
        const int col = n0 + wn * (GATED ? WTN / 2 : WTN) + j * 16 + (lane & 15);
        if (col >= g.n_dim) continue;
        float v;
        if (GATED) {
          const float a = acc[i][j][r];
          v = a / (1.0f + __expf(-a)) * acc[i][j + NOUT][r];
        } else {
          v = acc[i][j][r];
        }
        orow[col] = f32_to_bf16(v);
      }
    }
  }
}

template <bool GATED, int BM, int BNE, int WM, int WN>
hipError_t launch_v(const GemmArgs& g, hipStream_t s) {
  constexpr int COLS = GATED ? BNE / 2 : BNE;
  const long n_nt = (g.n_dim + COLS - 1) / COLS;
  const long blocks = static_cast<long>(g.tiles_cap) * n_nt;
  hipLaunchKernelGGL((expert_gemm_kernel<GATED, BM, BNE, WM, WN>), dim3(static_cast<unsigned>(blocks)),
                     dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_expert_gemm(bool gated, int bm, const GemmArgs& g, hipStream_t s) {
  if (gated) {
    if (bm == 256) return launch_v<true, 256, 256, 2, 2>(g, s);
    return launch_v<true, 128, 256, 2, 2>(g, s);
  }
  if (bm == 256) return launch_v<false, 256, 256, 2, 2>(g, s);
  return launch_v<false, 128, 256, 2, 2>(g, s);
}

}  // namespace moe
