// Large-tile bf16 grouped expert GEMM for gfx950 (prefill shapes).
//
// Same computation as grouped_gemm.hip (SwiGLU experts of "MoE inference: the
// call centre with 256 specialists ...", "The bare mechanism", each run only on
// its routed rows):
//   gated  : H[row, n] = SiLU(X Wg[e]^T)[row, n] * (X Wu[e]^T)[row, n]
//   plain  : Y[row, c] = (H Wd[e]^T)[row, c]
// organised for the matrix cores and the LDS of a CDNA4 compute unit:
//
//  * one workgroup = 4 wavefronts (2 x 2) owns a BM x BNE tile; BNE counts
//    effective columns: for the gated pass half are gate rows and half up rows
//    of the same output columns, so SiLU(gate) * up is formed in registers;
//  * each wavefront accumulates a (BM/2) x (BNE/2) block with
//    v_mfma_f32_16x16x32_bf16 into AGPRs (256 of them for a 256 x 256 tile),
//    so each 16-byte LDS fragment feeds 8 MFMAs;
//  * operands go global -> LDS with global_load_lds_dwordx4 (no register
//    staging) into two buffers of 64 K-elements: 128 bytes, one whole cache
//    line, of every row, so each load instruction asks the L2 for 8 whole
//    lines (the L2 -> CU path serves half-line requests at about half the
//    rate).  The 16-byte chunks of a row are XOR-swizzled by row, so the
//    fragment reads are free of bank conflicts;
//  * a buffer holds two K steps.  In the first a wavefront runs its MFMAs,
//    issuing the second half of the next buffer's loads in the first half
//    of them and reading the second step's fragments in the second half.  In
//    the second step it runs half its MFMAs, waits for the next buffer and
//    meets the other wavefronts at the pair's one barrier, then runs the rest
//    while it reads the next buffer's first fragments and starts refilling
//    the buffer it has just finished with the K steps two buffers ahead.
//    Loads are spread over the MFMAs because a wavefront issues in order: a
//    load stalled on a full memory queue holds back the MFMAs behind it;
//  * blocks are renumbered so that each of the 8 XCDs (which take workgroups
//    round-robin) works through a contiguous range of (row tile, column tile)
//    pairs ordered by bands of column tiles: the workgroups one XCD runs at a
//    time share their A rows and weight rows in its L2.
#include "expert_tile.h"
#include "lds_ring.h"
#include "mfma.h"

namespace moe {
namespace {

template <int N> struct CInt { static constexpr int value = N; };

typedef __attribute__((ext_vector_type(4))) short s16x4;

// BT: physical 16-byte chunk of logical chunk c in K-row kk of the staged B
// tile is c ^ bt_key(kk).  A transpose read of one wavefront touches the 16
// rows 8 g + 4 h + r (g, r < 4) of a K step; the key gives them 16 distinct
// chunk offsets, spreading the reads over the LDS banks.
__device__ __forceinline__ int bt_key(int kk) { return 2 * ((kk & 3) + 4 * ((kk >> 3) & 3)); }

// A K-row weight fragment (two ds_read_b64_tr_b16: K-rows k0 .. k0 + 3 into
// the low half, k0 + 4 .. k0 + 7 into the high half) from LDS byte address
// `addr` + OFF.  Inline asm rather than the builtin: the compiler makes a
// read through the builtin wait for every global->LDS load in flight
// (vmcnt(0)), which would drain the next buffers' loads each phase.  The
// compiler does not track these reads, so the caller waits for them
// (s_waitcnt lgkmcnt(0)) before anything reads `v`; the outputs are
// early-clobber so that no returning data overwrites the address register.
template <int OFF>
__device__ __forceinline__ void ds_read_tr_frag(u32x4& v, uint32_t addr) {
  typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
  u32x2 lo, hi;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %2 offset:%3\n\t"
      "ds_read_b64_tr_b16 %1, %2 offset:%4"
      : "=&v"(lo), "=&v"(hi)
      : "v"(addr), "i"(OFF), "i"(OFF + 2048));
  v = u32x4{lo[0], lo[1], hi[0], hi[1]};
}

template <bool GATED, int BM, int BNE, int NBUF, bool FP8W, bool BT = false, bool TRIPB = false>
__global__ __launch_bounds__(256, 1) void expert_gemm_kernel(GemmArgs g) {
  // BT: weights as K-rows ([k_dim, n_dim] per expert, rows split between w0
  // and w1 at bt_rows0).  A buffer stages 64 K-rows x 256 columns (512
  // contiguous bytes of each row, whole cache lines), and a B fragment is
  // two ds_read_b64_tr_b16: in a group of 16 lanes, lane j points at 4
  // columns (4 (j % 4) ..) of K-row k0 + j / 4 and lane i receives column i
  // of rows k0 .. k0 + 3, i.e. 4 consecutive K values of one column.
  static_assert(!BT || (!GATED && !FP8W && BNE == 256), "B-row mode: plain bf16, 256 columns");
  // FP8W: weights are E4M3 codes; a buffer holds 64 bytes of each weight row
  // (the same 64 K elements), read as 8-byte fragments and widened to bf16
  // right before their MFMAs; per-column scales are applied in the epilogue.
  constexpr int BROW = FP8W ? 64 : kLineBytes;  // staged bytes of a weight row per buffer
  constexpr int BRPB = 1024 / BROW;             // weight rows per 1 KB load block
  constexpr int ABUF = BM * kLineBytes;           // bytes of the A rows of a buffer
  constexpr int BBUF = BNE * BROW;                // bytes of the weight rows of a buffer
  constexpr int BUF = ABUF + BBUF;                // bytes per buffer
  // TRIPB: the A rows keep NBUF = 2 buffers and the weight rows get a third,
  // so each pair's weight loads are issued a whole pair earlier than its A
  // loads (weights come from HBM, the gathered A rows mostly from L2, which
  // a tile's column tiles share).  2 x 32 KB + 3 x 32 KB = the whole 160 KB.
  static_assert(!TRIPB || (NBUF == 2 && !FP8W && !BT), "TRIPB: bf16 forward, 2 A buffers");
  constexpr int NBB = TRIPB ? 3 : NBUF;           // weight-row buffers
  constexpr int SMEM = TRIPB ? NBUF * ABUF + NBB * BBUF : NBUF * BUF;
  constexpr int WTM = BM / 2, WTN = BNE / 2;   // wavefront block
  constexpr int MB = WTM / 16, NB = WTN / 16;  // 16 x 16 MFMA blocks
  constexpr int NOUT = GATED ? NB / 2 : NB;    // output column blocks per wavefront
  constexpr int COLS = GATED ? BNE / 2 : BNE;  // output columns per tile
  constexpr int A_BPW = BM / 32;               // 1 KB A load blocks (8 rows) per wavefront
  constexpr int B_BPW = BNE / 4 / BRPB;        // 1 KB weight load blocks per wavefront
  constexpr int LPB = A_BPW + B_BPW;           // loads per lane per buffer
  constexpr int LH1 = LPB / 2, LH2 = LPB - LH1;  // issued after the barrier / in the next step
  constexpr int NF = MB + NB;                  // fragments per K step
  static_assert(BM % 64 == 0 && BNE % 64 == 0, "tile shape");
  static_assert(A_BPW % 2 == 0 && (FP8W || B_BPW % 2 == 0),
                "a load's block parity is its index parity");
  static_assert(!GATED || (COLS % (B_BPW * BRPB) == 0 && NB % 2 == 0),
                "a wavefront's B blocks are all gate or all up rows");
  static_assert(NBUF >= 2 && (NBUF - 1) * LPB + LH1 < 64, "vmcnt range");

  __shared__ __attribute__((aligned(1024))) char smem[SMEM];
  // base of the A rows / weight rows of buffer q (TRIPB: separate rings)
  auto abuf = [&](int q) -> char* { return TRIPB ? smem + q * ABUF : smem + q * BUF; };
  auto bbuf = [&](int q) -> char* {
    return TRIPB ? smem + NBUF * ABUF + q * BBUF : smem + q * BUF + ABUF;
  };

  // ------------------------------------------------------- work of this block
  int part = -1, parts = 1, tile, nt;
  if (!decode_work(g, GATED, COLS, tile, nt, part, parts)) return;
  const int2 te = g.tiles[tile];
  const int e = te.x, m0 = te.y;
  const int seg = g.offsets[e];
  const int mvalid = min(BM, g.offsets[e + 1] - seg - m0);
  const int n0 = nt * COLS;

  const int tid = threadIdx.x, lane = tid & 63;
  // wave-uniform, so LDS destinations (M0) and bases live in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  // 16-row blocks of this wavefront's rows that hold tile rows
  const int mlive =
      __builtin_amdgcn_readfirstlane(min(max((mvalid - wm * WTM + 15) / 16, 0), MB));

  const size_t row_bytes = static_cast<size_t>(g.k_dim) * 2;
  const size_t wrow_bytes = static_cast<size_t>(g.k_dim) * (FP8W ? 1 : 2);
  const size_t mat_bytes = static_cast<size_t>(g.n_dim) * wrow_bytes;
  const bool routed = e < g.n_experts;
  const int es = routed ? e : e - g.n_experts;
  const char* w0 = reinterpret_cast<const char*>(routed ? g.w0 : g.ws0) + es * mat_bytes;
  const char* w1 = GATED ? reinterpret_cast<const char*>(routed ? g.w1 : g.ws1) + es * mat_bytes
                         : nullptr;

  // ------------------------------------------ this lane's global sources
  // Staged rows: A rows 0 .. BM-1, then B rows (gated: COLS gate rows, then
  // COLS up rows).  Wavefront w loads A blocks w*A_BPW .. and B blocks
  // w*B_BPW ..; lane l of a block fetches row l / 8 of it, the chunk that
  // line_lane_chunk assigns (FP8 weights: row l / 4 of a 16-row block, 16-byte
  // chunk (l % 4) ^ (l / 16), matching the fragment reads below).  Sources are a wave-uniform base plus a 32-bit
  // per-lane byte offset (the host keeps every operand below 4 GiB per base);
  // rows beyond the tile are clamped to a valid row and discarded at the end.
  const char* const a_base = reinterpret_cast<const char*>(g.a);
  uint32_t a_off[A_BPW];
#pragma unroll
  for (int j = 0; j < A_BPW; ++j) {
    const int R = (wave * A_BPW + j) * 8 + (lane >> 3);
    const int grow = seg + m0 + min(R, mvalid - 1);
    const int srow = min(max(g.gather != nullptr ? g.gather[grow] : grow, 0), g.a_rows - 1);
    a_off[j] = static_cast<uint32_t>(srow) * static_cast<uint32_t>(row_bytes) +
               line_lane_chunk(lane, j) * 16;
  }
  const int jb0 = wave * B_BPW * BRPB;
  const bool up_rows = GATED && jb0 >= COLS;
  const char* b_base = (up_rows ? w1 : w0) + static_cast<size_t>(n0) * wrow_bytes;
  const char* b_base1 = nullptr;  // BT: the weights of K-rows bt_rows0 ..
  const uint32_t ldb = static_cast<uint32_t>(g.n_dim) * 2;  // BT: bytes per K-row
  const int bt_pairs0 = BT ? g.bt_rows0 / 64 : 0;          // BT: buffers taken from w0
  uint32_t b_off[B_BPW];
  if constexpr (BT) {
    const char* const w0r = reinterpret_cast<const char*>(routed ? g.w0 : g.ws0) +
                            static_cast<size_t>(es) * g.bt_rows0 * ldb;
    const char* const w1r = reinterpret_cast<const char*>(routed ? g.w1 : g.ws1);
    b_base = w0r + static_cast<size_t>(n0) * 2;
    b_base1 = w1r == nullptr ? b_base
                             : w1r + static_cast<size_t>(es) * (g.k_dim - g.bt_rows0) * ldb +
                                   static_cast<size_t>(n0) * 2;
    // block j of wavefront w: K-rows 2 (w B_BPW + j) and + 1, 32 lanes each;
    // lane l writes physical chunk l % 32 of its row and fetches the logical
    // chunk the key maps there (columns past n_dim are clamped to a valid
    // chunk; their results are discarded)
#pragma unroll
    for (int j = 0; j < B_BPW; ++j) {
      const int kk = 2 * (wave * B_BPW + j) + (lane >> 5);
      const int col = min(n0 + 8 * ((lane & 31) ^ bt_key(kk)), g.n_dim - 8);
      b_off[j] = static_cast<uint32_t>(kk) * ldb + static_cast<uint32_t>(col - n0) * 2;
    }
  } else {
#pragma unroll
    for (int j = 0; j < B_BPW; ++j) {
      const int jb = jb0 + j * BRPB + lane / (64 / BRPB) - (up_rows ? COLS : 0);
      const int n = min(n0 + jb, g.n_dim - 1);
      const int chunk = FP8W ? ((lane & 3) ^ (lane >> 4)) : line_lane_chunk(lane, j);
      b_off[j] = static_cast<uint32_t>(n - n0) * static_cast<uint32_t>(wrow_bytes) + chunk * 16;
    }
  }
  const int a_dst = wave * A_BPW * 1024;  // inside the A rows of a buffer
  const int b_dst = wave * B_BPW * 1024;  // inside its weight rows

  // buffer loads ("pairs" of K steps) of this item: all, or its part's share
  // even: K is a multiple of 128
  int npairs = static_cast<int>(row_bytes / kLineBytes);
  if (part >= 0) {
    const int per = split_share(npairs, parts);
    const int p0 = part * per;
    npairs = min(per, npairs - p0);
#pragma unroll
    for (int j = 0; j < A_BPW; ++j) a_off[j] += static_cast<uint32_t>(p0) * kLineBytes;
#pragma unroll
    for (int j = 0; j < B_BPW; ++j) b_off[j] += static_cast<uint32_t>(p0) * BROW;
  }
  // Load l (A blocks first, then B blocks) of pair `pair` into A buffer `ab`
  // or weight buffer `bb`.  Pairs past the end re-read the last one (valid
  // addresses) into a buffer nobody reads again, so the loop needs no
  // branches.
  auto issue_one = [&](int pair, int l, int ab, int bb) {
    const uint32_t pc = static_cast<uint32_t>(min(pair, npairs - 1));
    if (l < A_BPW) {
      load_lds16(a_base + (a_off[l] + pc * kLineBytes), abuf(ab) + a_dst + l * 1024);
    } else if constexpr (BT) {
      const bool second = static_cast<int>(pc) >= bt_pairs0;
      const uint32_t prow = (second ? pc - bt_pairs0 : pc) * 64u * ldb;
      load_lds16((second ? b_base1 : b_base) + (b_off[l - A_BPW] + prow),
                 bbuf(bb) + b_dst + (l - A_BPW) * 1024);
    } else {
      load_lds16(b_base + (b_off[l - A_BPW] + pc * BROW), bbuf(bb) + b_dst + (l - A_BPW) * 1024);
    }
  };

  // LDS byte offset (inside a buffer) of fragment f for K step t (0, 1) of
  // the buffer: A blocks 0..MB-1, then B blocks (gated: NOUT gate blocks, then
  // NOUT up blocks of the same columns).  Fragment rows start at multiples of
  // 16, so the swizzle key is the lane's own.
  const int frow = lane & 15;
  const int fkey = swz128_key(frow);
  // K step t reads 16-byte chunk 4t + lane / 16 of each 128-byte A row; with
  // FP8 weights chunk 2 (lane / 16) + t instead (the same elements of A and
  // B always meet in one MFMA, in any fixed order), so that one 16-byte read
  // of a 64-byte weight row gives a lane its codes for both steps.
  const int ca0 = FP8W ? 2 * (lane >> 4) : (lane >> 4);
  const int ca1 = FP8W ? 2 * (lane >> 4) + 1 : 4 + (lane >> 4);
  const int flane0 = frow * kLineBytes + ((ca0 ^ fkey) << 4);
  const int flane1 = frow * kLineBytes + ((ca1 ^ fkey) << 4);
  // (A fragments: inside the A rows; weight fragments: inside the weight rows)
  auto frag_off = [&](int f, int t) {
    int r;
    if (f < MB) {
      r = wm * WTM + f * 16;
    } else {
      const int j = f - MB;
      if (GATED) r = (j < NOUT ? 0 : COLS) + wn * (WTN / 2) + (j % NOUT) * 16;
      else r = wn * WTN + j * 16;
    }
    return r * kLineBytes + (t ? flane1 : flane0);
  };
  // FP8 weights: weight fragment j, 16 bytes of a 64-byte row (codes of K
  // chunks 2 (lane / 16) and 2 (lane / 16) + 1: steps 0 and 1 of the buffer);
  // the 16-byte chunks of a row are XOR-swizzled by (row mod 16) / 4, so the
  // 16 lanes of a fragment group hit 16 distinct bank groups.
  const int f8lane = frow * 64 + 16 * ((lane >> 4) ^ (frow >> 2));
  auto frag8_off = [&](int j) {
    const int rb = GATED ? (j < NOUT ? 0 : COLS) + wn * (WTN / 2) + (j % NOUT) * 16
                         : wn * WTN + j * 16;
    return rb * 64 + f8lane;
  };

  f32x4 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 fr[2][NF];  // fragments of the two K steps of a buffer
  u32x4 fb[2][NB];  // FP8 weights: their raw weight fragments (both steps' codes)
  // fragment f of K step t from buffer q (A rows at abuf(q), weight rows at
  // bbuf(qb)) into fragment set SET
  // BT: lane constants of the transpose reads (row 8 (lane / 16) + (lane %
  // 16) / 4 of a K step, columns 4 (lane % 4) .. of the fragment's 16)
  const int bt_lane = (8 * (lane >> 4) + ((lane & 15) >> 2)) * 512 + ((lane & 3) >> 1) * 16 +
                      (lane & 1) * 8;
  const int bt_s = bt_key(8 * (lane >> 4) + ((lane & 15) >> 2));
  auto read_frag = [&](auto set_, int f, const char* a, const char* b, int t) {
    constexpr int SET = decltype(set_)::value;
    if (FP8W && f >= MB) {
      fb[SET][f - MB] = *reinterpret_cast<const u32x4*>(b + frag8_off(f - MB));
    } else if (BT && f >= MB) {
      const int nl = wn * WTN + (f - MB) * 16;  // first local column of the fragment
      const char* p = b + t * 32 * 512 + bt_lane + (((nl >> 3) ^ bt_s) << 4);
      typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * 512));
      u32x4 v;
      v[0] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 0, 1));
      v[1] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 2, 3));
      v[2] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 0, 1));
      v[3] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 2, 3));
      fr[SET][f] = v;
    } else {
      fr[SET][f] = *reinterpret_cast<const u32x4*>((f < MB ? a : b) + frag_off(f, t));
    }
  };

  // prologue: pairs 0 .. NBUF-2 and the first half of pair NBUF-1 in
  // flight; pair 0 landed; the first step's fragments in fr[0].  (A split
  // piece with nothing to reduce skips to the epilogue.)
  // TRIPB: pair 0, then the weight rows of pair 1, then its A rows, in
  // flight; pair 0 landed.
  if (npairs > 0) {
  if constexpr (TRIPB) {
#pragma unroll
    for (int l = 0; l < LPB; ++l) issue_one(0, l, 0, 0);
#pragma unroll
    for (int l = A_BPW; l < LPB; ++l) issue_one(1, l, 1, 1);
#pragma unroll
    for (int l = 0; l < A_BPW; ++l) issue_one(1, l, 1, 1);
    wait_vmem<LPB>();
  } else {
#pragma unroll
    for (int q = 0; q < NBUF - 1; ++q)
#pragma unroll
      for (int l = 0; l < LPB; ++l) issue_one(q, l, q, q);
#pragma unroll
    for (int l = 0; l < LH1; ++l) issue_one(NBUF - 1, l, NBUF - 1, NBUF - 1);
    wait_vmem<(NBUF - 2) * LPB + LH1>();
  }
  stage_barrier();
#pragma unroll
  for (int f = 0; f < NF; ++f) read_frag(CInt<0>{}, f, abuf(0), bbuf(0), 0);

  // Pair p (buffer cur = p mod NBUF) = K steps 2p (fragments in fr[0]) and
  // 2p + 1.
  //  step 2p    : MFMAs; first half: the last LH2 loads of pair p + NBUF - 1
  //               into buffer cur - 1 (free since the previous barrier);
  //               second half: step 2p + 1's fragments into fr[1].
  //  step 2p + 1: half the MFMAs; wait for pair p + 1 (pairs p + 2 ..
  //               p + NBUF - 1 may still be in flight) and meet at the
  //               barrier, after which nobody reads buffer cur again; the
  //               rest of the MFMAs while reading step 2p + 2's fragments
  //               from buffer cur + 1 into fr[0] and issuing the first LH1
  //               loads of pair p + NBUF into buffer cur.
  // TRIPB (A ring of 2, weight ring of 3): the same steps, but the loads in
  // step 2p are the weight rows of pair p + 2 (into weight buffer (p + 2)
  // mod 3, free since the previous barrier) and those after the barrier the
  // A rows of pair p + 2 (into A buffer p mod 2); the wait before the barrier
  // leaves only pair p + 2's weight rows in flight.  A pair's weight rows are
  // thus issued two barriers before they are read, its A rows one.
  // The last row tile of a group is usually part empty: a wavefront runs the
  // MFMAs (and reads the A fragments) of its first LIVE 16-row blocks only,
  // LIVE the smallest of MB, MB/2, MB/4, 0 that covers its rows.  Loads and
  // barriers are the same for every LIVE.
  constexpr int HALF = NB / 2;
  // One half K step: MFMAs of column blocks J0 .. J0 + HALF - 1 on fr[S],
  // with NL calls load(l) and NR calls read(r) spread evenly among them.
  auto half_step = [&](auto s_, auto j0_, auto live_, auto nl_, auto nr_, auto&& load,
                       auto&& read) {
    constexpr int S = decltype(s_)::value, J0 = decltype(j0_)::value;
    constexpr int LIVE = decltype(live_)::value;
    constexpr int NL = decltype(nl_)::value, NR = decltype(nr_)::value;
    constexpr int QH = LIVE * HALF;
    constexpr int QS = QH > 0 ? QH : 1;
    constexpr int LPQ = slots_per(QS, NL);  // slots per load
    constexpr int RPQ = slots_per(QS, NR);  // slots per read
    u32x4 bw = {0u, 0u, 0u, 0u};  // FP8 weights: fragment j widened to bf16
#pragma unroll
    for (int q = 0; q < QS; ++q) {
      if (q < QH) {
        const int i = q % (LIVE > 0 ? LIVE : 1), j = J0 + q / (LIVE > 0 ? LIVE : 1);
        if (FP8W) {
          if (i == 0) {
            // this step's 8 codes: bytes 0-7 (step 0) or 8-15 (step 1); the
            // first MFMA reading them waits out the VALU write
            bw = e4m3x8_to_bf16(make_uint2(fb[S][j][2 * S], fb[S][j][2 * S + 1]));
            mfma_bf16_agpr_after_valu(acc[i][j], fr[S][i], bw);
          } else {
            mfma_bf16_agpr(acc[i][j], fr[S][i], bw);
          }
        } else {
          mfma_bf16_agpr(acc[i][j], fr[S][i], fr[S][MB + j]);
        }
      }
      if (q % RPQ == RPQ - 1 && q / RPQ < NR) read(q / RPQ);
      if (q % LPQ == 0 && q / LPQ < NL) load(q / LPQ);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int r = QS / RPQ; r < NR; ++r) read(r);
#pragma unroll
    for (int l = QS / LPQ; l < NL; ++l) load(l);
  };
  auto k_loop = [&](auto live_) {
    constexpr int LIVE = decltype(live_)::value;
    constexpr int NR = LIVE > 0 ? LIVE + NB : 0;  // fragments a K step reads
    auto none = [](int) {};
    if constexpr (TRIPB) {
      int ca = 0, cb = 0;  // A and weight buffers of pair p (wave-uniform)
      for (int p = 0; p < npairs; ++p) {
        const int na = ca ^ 1;
        const int nb = cb == 2 ? 0 : cb + 1;  // weight buffer of pair p + 1
        const int fb_ = cb == 0 ? 2 : cb - 1;  // of pair p + 2
        const char* const acur = abuf(ca);
        const char* const bcur = bbuf(cb);
        const char* const anxt = abuf(na);
        const char* const bnxt = bbuf(nb);
        auto read1 = [&](int r) {
          read_frag(CInt<1>{}, r < LIVE ? r : MB + r - LIVE, acur, bcur, 1);
        };
        auto read0 = [&](int r) {
          read_frag(CInt<0>{}, r < LIVE ? r : MB + r - LIVE, anxt, bnxt, 0);
        };
        auto load_b = [&](int l) { issue_one(p + 2, A_BPW + l, ca, fb_); };
        auto load_a = [&](int l) { issue_one(p + 2, l, ca, fb_); };
        half_step(CInt<0>{}, CInt<0>{}, live_, CInt<B_BPW>{}, CInt<0>{}, load_b, none);
        half_step(CInt<0>{}, CInt<HALF>{}, live_, CInt<0>{}, CInt<NR>{}, none, read1);
        half_step(CInt<1>{}, CInt<0>{}, live_, CInt<0>{}, CInt<0>{}, none, none);
        wait_vmem<B_BPW>();
        stage_barrier();
        half_step(CInt<1>{}, CInt<HALF>{}, live_, CInt<A_BPW>{}, CInt<NR>{}, load_a, read0);
        ca = na;
        cb = nb;
      }
    } else {
      int cur = 0;  // wave-uniform
      for (int p = 0; p < npairs; ++p) {
        const int prv = cur == 0 ? NBUF - 1 : cur - 1;
        const int nxt = cur == NBUF - 1 ? 0 : cur + 1;
        auto read1 = [&](int r) {
          read_frag(CInt<1>{}, r < LIVE ? r : MB + r - LIVE, abuf(cur), bbuf(cur), 1);
        };
        auto read0 = [&](int r) {
          read_frag(CInt<0>{}, r < LIVE ? r : MB + r - LIVE, abuf(nxt), bbuf(nxt), 0);
        };
        auto load2 = [&](int l) { issue_one(p + NBUF - 1, LH1 + l, prv, prv); };
        auto load1 = [&](int l) { issue_one(p + NBUF, l, cur, cur); };
        half_step(CInt<0>{}, CInt<0>{}, live_, CInt<LH2>{}, CInt<0>{}, load2, none);
        half_step(CInt<0>{}, CInt<HALF>{}, live_, CInt<0>{}, CInt<NR>{}, none, read1);
        half_step(CInt<1>{}, CInt<0>{}, live_, CInt<0>{}, CInt<0>{}, none, none);
        wait_vmem<(NBUF - 2) * LPB>();
        stage_barrier();
        half_step(CInt<1>{}, CInt<HALF>{}, live_, CInt<LH1>{}, CInt<NR>{}, load1, read0);
        cur = nxt;
      }
    }
  };
  if (mlive > MB / 2) k_loop(CInt<MB>{});
  else if (mlive > MB / 4) k_loop(CInt<MB / 2>{});
  else if (mlive > 0) k_loop(CInt<MB / 4>{});
  else k_loop(CInt<0>{});
  }  // npairs > 0

  // -------------------------------------------------------------- epilogue
  wait_vmem<0>();   // this wavefront's last ring loads have landed
  stage_barrier();  // and every wavefront is done with the ring
  mfma_drain();
  constexpr int OC = GATED ? WTN / 2 : WTN;  // output columns per wavefront
  static_assert(4 * WTM * (128 + 16) <= SMEM, "staging space");
  char* const stg = smem + wave * WTM * (128 + 16);
  const int col0 = n0 + wn * OC;
  const float* sc0 = nullptr;  // FP8 weights: this expert's output-channel scales
  const float* sc1 = nullptr;
  if (FP8W) {
    sc0 = (routed ? g.sc0 : g.ssc0) + static_cast<size_t>(es) * g.n_dim;
    if (GATED) sc1 = (routed ? g.sc1 : g.ssc1) + static_cast<size_t>(es) * g.n_dim;
  }
  if (part < 0) {
    store_block<GATED, GATED, MB, NB, WTM, FP8W>(acc, stg, lane, g.out, false, g.n_dim,
                                                 seg + m0 + wm * WTM, mvalid - wm * WTM, col0,
                                                 g.n_dim, sc0, sc1);
  } else if (!GATED) {  // fp32 partial rows of a split tail tile
    const long prow = static_cast<long>(part) * g.plan[kPlanStride] + seg + m0 -
                      g.plan[kPlanRowSplit] + wm * WTM;
    store_block<GATED, false, MB, NB, WTM, FP8W>(acc, stg, lane, g.out_part, true, g.n_dim, prow,
                                                 mvalid - wm * WTM, col0, g.n_dim, sc0, sc1);
  }
}

template <bool GATED, int BM, int BNE, int NBUF, bool FP8W = false, bool BT = false,
          bool TRIPB = false>
hipError_t launch_v(const GemmArgs& g, hipStream_t s) {
  constexpr int COLS = GATED ? BNE / 2 : BNE;
  const long blocks = expert_grid(g, GATED, COLS);
  hipLaunchKernelGGL((expert_gemm_kernel<GATED, BM, BNE, NBUF, FP8W, BT, TRIPB>),
                     dim3(static_cast<unsigned>(blocks)),
                     dim3(256), 0, s, g);
  return hipGetLastError();
}

// ------------------------------------------------------------------------
// Narrow tail tile of the ping-pong kernel: an expert's last row tile when it
// holds at most 64 rows, over two column tiles at once (512 effective
// columns; gated: 256 gate rows then 256 up rows of the weights).
//
// An expert's 256-row tiles and its short last tile read the same weight
// rows.  As a tile of its own the short one ran ahead of its partner (it has
// almost no MFMA work), so the partner fetched the weights from HBM again,
// and it still cost most of a full tile.  Over two column tiles it moves
// about as many bytes per K step as a full tile (64 KB of weights and 8 KB of
// A rows against 32 + 32 KB), so it keeps pace with the two full tiles it is
// listed next to and finds their weight rows in L2, and there are half as
// many of them.  LDS: 2 buffers of 8 KB (A) and 2 of 64 KB (weights).
// Wavefront w owns rows 32 (w / 4) .. + 32 and effective columns 128 (w % 4)
// .. + 128 (gated: 64 gate and 64 up columns of the same 64 outputs); one
// barrier per pair of K steps, the next pair's loads in flight meanwhile.
// FP8W: a weight buffer holds the 128 codes of two pairs per row (whole
// lines, as in the full tiles), loaded every second pair; the fragments and
// their widening are those of the full tiles.
template <bool GATED, bool FP8W>
__device__ __forceinline__ void narrow_tile(const GemmArgs& g, char* smem, int e, int seg, int m0,
                                            int mvalid, int nt) {
  constexpr int ABUF = 64 * kLineBytes, BBUF = 512 * kLineBytes;
  constexpr int COLS = GATED ? 128 : 256;      // output columns of one column tile
  constexpr int HALF = 2 * COLS;               // gated: staged gate rows before the up rows
  constexpr int WTM = 32, MB = 2, NB = 8;      // wavefront block: 32 x 128 effective
  constexpr int NOUT = GATED ? NB / 2 : NB;
  constexpr int OC = GATED ? 64 : 128;         // output columns per wavefront
  static_assert(2 * ABUF + 2 * BBUF <= 160 * 1024, "LDS");
  static_assert(8 * WTM * (256 + 16) <= 2 * ABUF + 2 * BBUF, "staging space");
  auto abuf = [&](int q) -> char* { return smem + q * ABUF; };
  auto bbuf = [&](int q) -> char* { return smem + 2 * ABUF + q * BBUF; };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rh = wave >> 2, cw = wave & 3;
  const int mlive =
      __builtin_amdgcn_readfirstlane(min(max((mvalid - rh * WTM + 15) / 16, 0), MB));
  const size_t row_bytes = static_cast<size_t>(g.k_dim) * 2;
  const size_t wrow_bytes = static_cast<size_t>(g.k_dim) * (FP8W ? 1 : 2);
  const size_t mat_bytes = static_cast<size_t>(g.n_dim) * wrow_bytes;
  const bool routed = e < g.n_experts;
  const int es = routed ? e : e - g.n_experts;
  const char* const w0 = reinterpret_cast<const char*>(routed ? g.w0 : g.ws0) + es * mat_bytes;
  const char* const w1 =
      GATED ? reinterpret_cast<const char*>(routed ? g.w1 : g.ws1) + es * mat_bytes : nullptr;
  const int n0 = nt * COLS;  // first output column; the tile covers 2 COLS of them

  // loads of a pair: the A rows 8 w .. 8 w + 7 (one 1 KB block per
  // wavefront) and the staged weight rows 64 w .. 64 w + 63 (eight blocks);
  // lane l of a block fetches row l / 8, chunk line_lane_chunk; rows past
  // the tile or the matrix are clamped to a valid row
  const char* const a_base = reinterpret_cast<const char*>(g.a);
  uint32_t a_off;
  {
    const int R = wave * 8 + (lane >> 3);
    const int grow = seg + m0 + min(R, mvalid - 1);
    const int srow = min(max(g.gather != nullptr ? g.gather[grow] : grow, 0), g.a_rows - 1);
    a_off = static_cast<uint32_t>(srow) * static_cast<uint32_t>(row_bytes) +
            line_lane_chunk(lane, 0) * 16;
  }
  const int jb0 = wave * 64;
  const bool up_rows = GATED && jb0 >= HALF;
  const char* const b_base = (up_rows ? w1 : w0) + static_cast<size_t>(n0) * wrow_bytes;
  uint32_t b_off[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int jb = jb0 + j * 8 + (lane >> 3) - (up_rows ? HALF : 0);
    const int n = min(n0 + jb, g.n_dim - 1);
    b_off[j] = static_cast<uint32_t>(n - n0) * static_cast<uint32_t>(wrow_bytes) +
               line_lane_chunk(lane, j) * 16;
  }
  const int npairs = static_cast<int>(row_bytes / kLineBytes);  // even
  // the loads of pair `pair`: its A rows, and its weight buffer's rows (FP8:
  // only for even pairs, the buffer of this pair and the next); past the end
  // the last one again, never read
  auto issue = [&](int pair, int q) {
    const uint32_t pc = static_cast<uint32_t>(min(pair, npairs - 1)) * kLineBytes;
    load_lds16(a_base + (a_off + pc), abuf(q) + wave * 1024);
    if (FP8W && (pair & 1)) return;
    const int bq = FP8W ? (pair >> 1) & 1 : q;
    const uint32_t bc = FP8W ? static_cast<uint32_t>(min(pair >> 1, npairs / 2 - 1)) * kLineBytes : pc;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      load_lds16(b_base + (b_off[j] + bc), bbuf(bq) + wave * 8192 + j * 1024);
  };

  const int frow = lane & 15, fkey = frow & 7;
  const int ca0 = FP8W ? 2 * (lane >> 4) : (lane >> 4);
  const int ca1 = FP8W ? 2 * (lane >> 4) + 1 : 4 + (lane >> 4);
  const int fl0 = frow * kLineBytes + ((ca0 ^ fkey) << 4);
  const int fl1 = frow * kLineBytes + ((ca1 ^ fkey) << 4);
  // FP8 weight fragment of the first / second pair of a buffer
  const int f8l0 = frow * kLineBytes + (((lane >> 4) ^ fkey) << 4);
  const int f8l1 = frow * kLineBytes + (((4 + (lane >> 4)) ^ fkey) << 4);
  // BT: lane constants of the transpose reads (K-row 8 (lane / 16) + (lane
  // mod 16) / 4 of a step, columns 4 (lane mod 4) .. of the fragment's 16)
  const int bt_lane = (8 * (lane >> 4) + ((lane & 15) >> 2)) * 512 + ((lane & 3) >> 1) * 16 +
                      (lane & 1) * 8;
  const int bt_s = bt_key(8 * (lane >> 4) + ((lane & 15) >> 2));
  auto b_row = [&](int j) {  // first staged weight row of block j
    if (GATED) return (j < NOUT ? 0 : HALF) + cw * (OC) + (j % NOUT) * 16;
    return cw * 128 + j * 16;
  };

  f32x4 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  issue(0, 0);
  wait_vmem<0>();
  stage_barrier();
  auto run = [&](auto live_) {
    constexpr int LIVE = decltype(live_)::value;
    u32x4 fa[2][MB], fb[2][NB];
    for (int p = 0; p < npairs; ++p) {
      // into the buffers read in pairs p - 1 (A) and p - 2, p - 1 (FP8 weights)
      issue(p + 1, (p + 1) & 1);
      const char* const a = abuf(p & 1);
      const char* const b = bbuf(FP8W ? (p >> 1) & 1 : p & 1);
      if (LIVE > 0) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int fl = t ? fl1 : fl0;
#pragma unroll
          for (int i = 0; i < LIVE; ++i)
            fa[t][i] = *reinterpret_cast<const u32x4*>(a + (rh * WTM + i * 16) * kLineBytes + fl);
          if (!FP8W || t == 0) {
#pragma unroll
            for (int j = 0; j < NB; ++j)
              fb[t][j] = *reinterpret_cast<const u32x4*>(
                  b + b_row(j) * kLineBytes + (FP8W ? ((p & 1) ? f8l1 : f8l0) : fl));
          }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if constexpr (FP8W) {
          // as in the full tiles: widen, then the MFMAs, the first with the
          // VALU -> MFMA wait states; the previous widened fragment stays
          // allocated until the next one's MFMAs are issued
          u32x4 wprev = {0u, 0u, 0u, 0u};
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int j = 0; j < NB; ++j) {
              const u32x4 c = fb[0][j];
              const u32x4 w = e4m3x8_to_bf16(t ? make_uint2(c[2], c[3]) : make_uint2(c[0], c[1]));
              mfma_bf16_agpr_after_valu(acc[0][j], fa[t][0], w);
#pragma unroll
              for (int i = 1; i < LIVE; ++i) mfma_bf16_agpr(acc[i][j], fa[t][i], w);
              asm volatile("" ::"v"(wprev));
              wprev = w;
            }
        } else {
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
              for (int i = 0; i < LIVE; ++i) mfma_bf16_agpr(acc[i][j], fa[t][i], fb[t][j]);
        }
      }
      wait_vmem<0>();  // pair p + 1 landed before anyone reads it
      stage_barrier();
    }
  };
  if (mlive == MB) run(CInt<MB>{});
  else if (mlive > 0) run(CInt<MB / 2>{});
  else run(CInt<0>{});

  // epilogue: every ring read is done (the last barrier), every load landed
  mfma_drain();
  char* const stg = smem + wave * WTM * (256 + 16);
  const float* sc0 = nullptr;  // FP8 weights: this expert's output-channel scales
  const float* sc1 = nullptr;
  if (FP8W) {
    sc0 = (routed ? g.sc0 : g.ssc0) + static_cast<size_t>(es) * g.n_dim;
    if (GATED) sc1 = (routed ? g.sc1 : g.ssc1) + static_cast<size_t>(es) * g.n_dim;
  }
  store_block<GATED, GATED, MB, NB, WTM, FP8W, 64>(acc, stg, lane, g.out, false, g.n_dim,
                                                   seg + m0 + rh * WTM, mvalid - rh * WTM,
                                                   n0 + cw * OC, g.n_dim, sc0, sc1);
}

// ------------------------------------------------------------------------
// Ping-pong variant of the 256 x 256 bf16 tile: 8 wavefronts, two per SIMD.
//
// The tile, its work items, its LDS layout (A rows in 2 buffers, weight rows
// in 3, 128 bytes of every row per buffer) and its epilogue are those of
// expert_gemm_kernel; what differs is who does what when.  Wavefronts 0-3
// (group 0) and 4-7 (group 1) sit one per SIMD each, and each owns a 64 x 128
// block (rows 64 q .., columns 128 g .. of the effective tile, q = wave mod 4,
// g = group).  Every wavefront alternates two phases per pair of K steps:
//   memory : issue its share of later pairs' loads, read all its fragments of
//            this pair from LDS (24 ds_read_b128), wait for them;
//   compute: its 64 MFMAs (two K steps x 4 x 8 blocks), registers only.
// Group 1 runs one phase behind group 0, so in every phase one wavefront of
// each SIMD issues MFMAs while the other does its memory work; a workgroup
// barrier ends every phase.  Group 0 loads the A rows (pair p + 1 during its
// memory phase of pair p), group 1 the weight rows (pair p + 2 during its
// memory phase of pair p), so each buffer is refilled only after both groups
// have read it, and each group waits for its own loads at the end of the
// phase before they are needed.  Phases (h = 0 .. 2n for n pairs):
//   group 0: h = 2p memory(p), h = 2p + 1 compute(p), h = 2n idle;
//   group 1: h = 0 idle, h = 2p + 1 memory(p), h = 2p + 2 compute(p).
// With one wavefront per SIMD (expert_gemm_kernel) the matrix core idles
// whenever that wavefront waits for LDS data, for its loads or at the
// barrier; here the other wavefront of the SIMD covers those waits.
// DENSE (plain pass only): GemmArgs' dense mode, a separate instance so that
// the grouped launches carry no trace of it.  NARROW: the instance that also
// runs narrow tail items (g.narrow); launches without them take the other.
// FP8W: E4M3 weights.  A weight buffer holds 128 codes of each weight row,
// the K elements of two pairs, in the layout and with the loads of a bf16
// buffer (whole 128-byte lines; 64-byte half rows per pair made as many L2
// requests per pair as bf16 weights and gained nothing).  Group 1 loads a
// buffer every second pair, two buffers ahead.  One 16-byte read (chunk
// lane / 16 of the pair's half row) gives a lane the codes of its fragment
// for both K steps of the pair (bytes 0-7 and 8-15), and the A chunks are
// read in the matching order (chunk 2 (lane / 16) + t in step t).  The
// compute phase widens each weight fragment to bf16 right before its MFMAs;
// the epilogue applies the per-output-channel scales.
// BT: weights as K-rows, staged and read as in expert_gemm_kernel's BT mode
// (a weight buffer: 64 K-rows x 512 contiguous bytes, chunks swizzled by
// bt_key; a weight fragment: two ds_read_b64_tr_b16); plain bf16 grouped
// launches without a split reduction.
// KMAJ: the weight-gradient products C_g = A_g B_g^T (GemmArgs' kbase
// fields): A rows are rows of a, B rows rows of w0, both starting at column
// kbase[g], and the reduction runs over that group's columns only; tiles
// from decode_kwork; C_g is written to out or out_alt, staged as bf16; a
// group with nothing to reduce writes zeros.  Against the 4-wavefront
// kernel's mode for these products, same box: 10-11 % faster (DeepSeek-V3-
// shaped weight gradients 12.76 -> 11.35 ms, Mixtral-shaped 2.96 -> 2.66).
template <bool GATED, bool DENSE = false, bool NARROW = false, bool FP8W = false, bool BT = false,
          bool KMAJ = false>
__global__ __launch_bounds__(512, 1) void expert_gemm_pp_kernel(GemmArgs g) {
  static_assert(!(GATED && DENSE), "dense mode: plain pass");
  static_assert(!(DENSE && NARROW), "dense mode: no tail items");
  static_assert(!(FP8W && DENSE), "FP8 weights: grouped launches");
  static_assert(!BT || (!GATED && !DENSE && !NARROW && !FP8W), "K-row mode: plain bf16 pass");
  static_assert(!KMAJ || (!GATED && !DENSE && !NARROW && !FP8W && !BT),
                "weight-gradient mode: plain bf16 pass");
  constexpr int BM = 256, BNE = 256;
  constexpr int ABUF = BM * kLineBytes, BBUF = BNE * kLineBytes;
  constexpr int NA = 2, NBB = 3;               // A and weight ring buffers
  constexpr int SMEM = NA * ABUF + NBB * BBUF;  // 160 KB
  constexpr int WTM = 64, WTN = 128;           // wavefront block
  constexpr int MB = WTM / 16, NB = WTN / 16;  // 4 x 8 MFMA blocks
  constexpr int NOUT = GATED ? NB / 2 : NB;
  constexpr int COLS = GATED ? BNE / 2 : BNE;  // output columns per tile
  constexpr int LPW = 8;                       // group 0: 1 KB A loads per wavefront per pair
  constexpr int LPWB = BBUF / 4 / 1024;        // group 1: 1 KB weight loads per buffer
  constexpr int NF = MB + NB;                  // fragments per K step
  static_assert(4 * LPW * 1024 == ABUF && 4 * LPWB * 1024 == BBUF, "one group fills a ring");
  static_assert(8 * WTM * (256 + 16) <= SMEM, "staging space");

  __shared__ __attribute__((aligned(1024))) char smem[SMEM];
  auto abuf = [&](int q) -> char* { return smem + q * ABUF; };
  auto bbuf = [&](int q) -> char* { return smem + NA * ABUF + q * BBUF; };

  int part = -1, parts = 1, tile = 0, nt = 0, e = 0, m0 = 0, seg = 0, mvalid = 0, n0 = 0;
  long kb = 0;  // KMAJ: first reduction column of the group
  constexpr bool dense = DENSE;
  if constexpr (KMAJ) {
    if (!decode_kwork(g, BM, COLS, e, m0, n0)) return;
    mvalid = min(BM, g.a_rows - m0);
    kb = g.kbase[e];
  } else if (dense) {
    // block b: part b mod parts (with 8 parts every XCD holds one part, so
    // the tiles it runs at once share that part's weight columns in its
    // L2), then column tile and row tile
    const int bid = blockIdx.x;
    parts = g.dense_parts;
    part = bid % parts;
    const int n_nt = (g.n_dim + COLS - 1) / COLS, w = bid / parts;
    tile = w / n_nt;
    nt = w - tile * n_nt;
    m0 = tile * BM;
    if (m0 >= g.a_rows) return;
    mvalid = min(BM, g.a_rows - m0);
  } else {
    if (!decode_work(g, GATED, COLS, tile, nt, part, parts)) return;
    const int2 te = g.tiles[tile];
    e = te.x;
    m0 = te.y;
    seg = g.offsets[e];
    mvalid = min(BM, g.offsets[e + 1] - seg - m0);
    if (NARROW && part < 0 && mvalid <= kNarrowRows) {
      narrow_tile<GATED, FP8W>(g, smem, e, seg, m0, mvalid, nt);
      return;
    }
  }
  if constexpr (!KMAJ) n0 = nt * COLS;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, q = wave & 3;
  const int wm = q, wn = grp;  // rows 64 q .., effective columns 128 g ..
  const int mlive = __builtin_amdgcn_readfirstlane(min(max((mvalid - wm * WTM + 15) / 16, 0), MB));

  const size_t row_bytes = static_cast<size_t>(g.k_dim) * 2;
  const size_t wrow_bytes = static_cast<size_t>(g.k_dim) * (FP8W ? 1 : 2);
  const size_t mat_bytes = static_cast<size_t>(g.n_dim) * wrow_bytes;
  const bool routed = e < g.n_experts;
  const int es = routed ? e : e - g.n_experts;
  // KMAJ: A and B rows both start at the group's first reduction column
  const char* const w0 = KMAJ ? reinterpret_cast<const char*>(g.w0) + kb * 2
                              : reinterpret_cast<const char*>(routed ? g.w0 : g.ws0) + es * mat_bytes;
  const char* const w1 =
      GATED ? reinterpret_cast<const char*>(routed ? g.w1 : g.ws1) + es * mat_bytes : nullptr;

  // This wavefront's loads: group 0 the 8 A blocks of rows 64 q .. 64 q + 63,
  // group 1 the 8 weight blocks of staged weight rows 64 q .. (gated: rows
  // below COLS are gate rows, the rest up rows of the same columns).  Lane l
  // of a block fetches row l / 8 of it, the chunk line_lane_chunk assigns;
  // rows past the tile or the matrix are clamped to a valid row.
  const char* src_base;
  const char* src_base1 = nullptr;  // BT: the weights of K-rows bt_rows0 ..
  const uint32_t ldb = static_cast<uint32_t>(g.n_dim) * 2;  // BT: bytes per K-row
  uint32_t off[LPW] = {};
  if (grp == 0) {
    src_base = reinterpret_cast<const char*>(g.a) + kb * 2;
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int R = q * 64 + j * 8 + (lane >> 3);
      const int grow = seg + m0 + min(R, mvalid - 1);
      const int srow = min(max(g.gather != nullptr ? g.gather[grow] : grow, 0), g.a_rows - 1);
      off[j] = static_cast<uint32_t>(srow) * static_cast<uint32_t>(row_bytes) +
               line_lane_chunk(lane, j) * 16;
    }
  } else if (BT) {
    // block j of wavefront q: K-rows 2 (8 q + j) and + 1 of the buffer, 32
    // lanes each; lane l writes physical chunk l mod 32 of its row and
    // fetches the logical chunk the key maps there (columns past n_dim are
    // clamped to a valid chunk; their results are discarded)
    const char* const w0r = reinterpret_cast<const char*>(routed ? g.w0 : g.ws0) +
                            static_cast<size_t>(es) * g.bt_rows0 * ldb;
    const char* const w1r = reinterpret_cast<const char*>(routed ? g.w1 : g.ws1);
    src_base = w0r + static_cast<size_t>(n0) * 2;
    src_base1 = w1r == nullptr ? src_base
                               : w1r + static_cast<size_t>(es) * (g.k_dim - g.bt_rows0) * ldb +
                                     static_cast<size_t>(n0) * 2;
#pragma unroll
    for (int j = 0; j < LPWB; ++j) {
      const int kk = 2 * (q * LPWB + j) + (lane >> 5);
      const int col = min(n0 + 8 * ((lane & 31) ^ bt_key(kk)), g.n_dim - 8);
      off[j] = static_cast<uint32_t>(kk) * ldb + static_cast<uint32_t>(col - n0) * 2;
    }
  } else {
    const int jb0 = q * 64;
    const bool up_rows = GATED && jb0 >= COLS;
    src_base = (up_rows ? w1 : w0) + static_cast<size_t>(n0) * wrow_bytes;
#pragma unroll
    for (int j = 0; j < LPWB; ++j) {
      const int jb = jb0 + j * 8 + (lane >> 3) - (up_rows ? COLS : 0);
      const int n = min(n0 + jb, g.n_dim - 1);
      off[j] = static_cast<uint32_t>(n - n0) * static_cast<uint32_t>(wrow_bytes) +
               line_lane_chunk(lane, j) * 16;
    }
  }
  int npairs = KMAJ ? static_cast<int>((g.kbase[e + 1] - kb) * 2 / kLineBytes)
                    : static_cast<int>(row_bytes / kLineBytes);
  // the weight rows of a routed expert whose rows fit one tile are read by
  // this tile alone: streamed (non-temporal) past L2, where the gathered A
  // rows that the tile's column neighbours share stay longer
  const bool w_once = !KMAJ && !DENSE && !BT && routed && g.offsets[e + 1] - seg <= BM;
  // source bytes of a row per buffer: A 128 (a pair), weights 128 (a pair;
  // FP8 two pairs, so a pair is 64)
  const int pstep = grp == 0 || !FP8W ? kLineBytes : kLineBytes / 2;
  if (part >= 0) {
    const int per = split_share(npairs, parts);  // even: FP8 buffers stay whole
    const int p0 = part * per;
    npairs = min(per, npairs - p0);
#pragma unroll
    for (int j = 0; j < LPW; ++j) off[j] += static_cast<uint32_t>(p0 * pstep);
  }
  // this wavefront's 8 loads of buffer `buf` (a pair; FP8 weights: the pair
  // pair 2 buf and 2 buf + 1); past the end the last one again, into a buffer
  // nobody reads again
  const int nbufs = grp == 0 || !FP8W ? npairs : npairs / 2;
  const int bt_pairs0 = BT ? g.bt_rows0 / 64 : 0;  // BT: buffers taken from w0
  auto issue = [&](auto grp_, int buf, char* ring, auto nt_) {
    const int bc = min(buf, nbufs - 1);
    const int dst = q * LPW * 1024;
    if (BT && decltype(grp_)::value == 1) {
      const bool second = bc >= bt_pairs0;
      const uint32_t prow = static_cast<uint32_t>(second ? bc - bt_pairs0 : bc) * 64u * ldb;
      const char* const base = second ? src_base1 : src_base;
#pragma unroll
      for (int j = 0; j < LPW; ++j) load_lds16(base + (off[j] + prow), ring + dst + j * 1024);
      return;
    }
    const uint32_t pc = static_cast<uint32_t>(bc * kLineBytes);
    if constexpr (decltype(grp_)::value == 1 && decltype(nt_)::value) {
#pragma unroll
      for (int j = 0; j < LPW; ++j) load_lds16_nt(src_base + (off[j] + pc), ring + dst + j * 1024);
    } else {
#pragma unroll
      for (int j = 0; j < LPW; ++j) load_lds16(src_base + (off[j] + pc), ring + dst + j * 1024);
    }
  };

  // Fragment reads: lane l takes row l mod 16 of a 16-row block, chunk
  // l / 16 (+ 4 for the second K step; FP8 weights: chunk 2 (l / 16) + t)
  // under the row-mod-8 swizzle; an FP8 weight fragment is 16 bytes of a
  // 64-byte staged row.
  const int frow = lane & 15;
  const int fkey = frow & 7;
  const int ca0 = FP8W ? 2 * (lane >> 4) : (lane >> 4);
  const int ca1 = FP8W ? 2 * (lane >> 4) + 1 : 4 + (lane >> 4);
  const int fl0 = frow * kLineBytes + ((ca0 ^ fkey) << 4);
  const int fl1 = frow * kLineBytes + ((ca1 ^ fkey) << 4);
  // FP8 weight fragment of the first / second pair of a buffer
  const int f8l0 = frow * kLineBytes + (((lane >> 4) ^ fkey) << 4);
  const int f8l1 = frow * kLineBytes + (((4 + (lane >> 4)) ^ fkey) << 4);
  // BT: lane constants of the transpose reads (K-row 8 (lane / 16) + (lane
  // mod 16) / 4 of a step, columns 4 (lane mod 4) .. of the fragment's 16)
  const int bt_lane = (8 * (lane >> 4) + ((lane & 15) >> 2)) * 512 + ((lane & 3) >> 1) * 16 +
                      (lane & 1) * 8;
  const int bt_s = bt_key(8 * (lane >> 4) + ((lane & 15) >> 2));
  auto b_row = [&](int j) {  // first staged weight row of block j
    if (GATED) return (j < NOUT ? 0 : COLS) + wn * (WTN / 2) + (j % NOUT) * 16;
    return wn * WTN + j * 16;
  };

  f32x4 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 fr[2][NF];

  // (KMAJ: a group with nothing to reduce loads nothing and writes zeros;
  // npairs is the same for the whole workgroup)
  if (!KMAJ || npairs > 0) {
  // prologue: group 0 A(0); group 1 B(0) then B(1); A(0) and B(0) landed
  // (FP8: weight buffers 0 and 1, pairs 0 .. 3)
  if (grp == 0) {
    issue(CInt<0>{}, 0, abuf(0), CInt<0>{});
    wait_vmem<0>();
  } else if (w_once) {
    issue(CInt<1>{}, 0, bbuf(0), CInt<1>{});
    issue(CInt<1>{}, 1, bbuf(1), CInt<1>{});
    wait_vmem<LPWB>();
  } else {
    issue(CInt<1>{}, 0, bbuf(0), CInt<0>{});
    issue(CInt<1>{}, 1, bbuf(1), CInt<0>{});
    wait_vmem<LPWB>();
  }
  stage_barrier();

  // Each group runs its own straight loop (a shared loop that branches on the
  // group every phase made the compiler move the accumulators out of the
  // AGPRs); both execute 2 n + 3 barriers in all, prologue included.
  auto run = [&](auto live_, auto grp_, auto nt_) {
    constexpr int LIVE = decltype(live_)::value;
    constexpr int G = decltype(grp_)::value;
    auto memory = [&](int p) {
      const char* const a = abuf(p & 1);
      const int qb = FP8W ? (p >> 1) % 3 : p % 3;  // weight buffer of pair p
      const char* const b = bbuf(qb);
      if (G == 0) issue(grp_, p + 1, abuf((p + 1) & 1), nt_);
      else if (!FP8W) issue(grp_, p + 2, bbuf((p + 2) % 3), nt_);
      else if ((p & 1) == 0) issue(grp_, (p >> 1) + 2, bbuf(((p >> 1) + 2) % 3), nt_);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int fl = t ? fl1 : fl0;
#pragma unroll
        for (int i = 0; i < LIVE; ++i)
          fr[t][i] = *reinterpret_cast<const u32x4*>(a + (wm * WTM + i * 16) * kLineBytes + fl);
        if (LIVE > 0 && (!FP8W || t == 0) && !BT) {
#pragma unroll
          for (int j = 0; j < NB; ++j)
            fr[t][MB + j] = *reinterpret_cast<const u32x4*>(
                b + b_row(j) * kLineBytes + (FP8W ? ((p & 1) ? f8l1 : f8l0) : fl));
        }
      }
      if (LIVE > 0 && BT) {
        // weight fragment j: columns wn WTN + 16 j .. of K-rows 32 t + 8
        // (lane / 16) ..; its lane address is recomputed here from the
        // opaque key, so that one address is live at a time instead of a
        // loop-invariant register per fragment
        uint32_t kx = static_cast<uint32_t>(bt_s) << 4;
        uint32_t la = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
                          (const __attribute__((address_space(3))) char*)(b))) +
                      bt_lane;
        asm volatile("" : "+v"(kx), "+v"(la));
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const uint32_t pr = la + ((static_cast<uint32_t>((wn * WTN + j * 16) >> 3) << 4) ^ kx);
          ds_read_tr_frag<0>(fr[0][MB + j], pr);
          ds_read_tr_frag<16384>(fr[1][MB + j], pr);
        }
      }
      // fragments in registers; group 0 leaves A(p + 1) in flight (waited
      // for after its compute phase), group 1 waits for B(p + 1) and leaves
      // B(p + 2) in flight (FP8: after an odd pair, waits for the buffer of
      // the next two pairs and leaves the one after in flight; after an even
      // pair the next pair's buffer is the current one, and only its
      // fragment reads are waited for: group 0 refills A(p)'s buffer right
      // after the barrier)
      if (G == 0) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      else if (!FP8W || (p & 1)) wait_vmem<LPWB>();
      else asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    };
    auto compute = [&]() {
      // the wavefront issuing MFMAs goes first when both wavefronts of its
      // SIMD want an issue slot (the other one's address arithmetic also
      // takes the vector ALU); same box, 3 x 30 steps: Mixtral-shaped
      // prefill 2.284 -> 2.261 ms, DeepSeek-V3 6.761 -> 6.729 ms (the memory
      // phase first instead measured the same as this)
      __builtin_amdgcn_s_setprio(2);
      if constexpr (FP8W) {
        // weight fragment j of step t widened from its 8 codes; the first
        // MFMA reading it carries the VALU -> MFMA wait states.  The previous
        // widened fragment stays allocated until the next one's MFMAs are
        // issued, so a widening never writes registers an MFMA just issued
        // still reads.
        u32x4 wprev = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            if (LIVE == 0) continue;
            const u32x4 c = fr[0][MB + j];
            const u32x4 w = e4m3x8_to_bf16(t ? make_uint2(c[2], c[3]) : make_uint2(c[0], c[1]));
            mfma_bf16_agpr_after_valu(acc[0][j], fr[t][0], w);
#pragma unroll
            for (int i = 1; i < LIVE; ++i) mfma_bf16_agpr(acc[i][j], fr[t][i], w);
            asm volatile("" ::"v"(wprev));
            wprev = w;
          }
      } else {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int i = 0; i < LIVE; ++i) mfma_bf16_agpr(acc[i][j], fr[t][i], fr[t][MB + j]);
      }
      __builtin_amdgcn_s_setprio(0);
    };
    if (G == 0) {
      for (int p = 0; p < npairs; ++p) {
        memory(p);  // phase 2p
        stage_barrier();
        compute();  // phase 2p + 1
        wait_vmem<0>();  // A(p + 1) landed before anyone reads pair p + 1
        stage_barrier();
      }
      stage_barrier();  // phase 2n: idle
    } else {
      stage_barrier();  // phase 0: idle
      for (int p = 0; p < npairs; ++p) {
        memory(p);  // phase 2p + 1
        stage_barrier();
        compute();  // phase 2p + 2
        stage_barrier();
      }
      wait_vmem<0>();  // the loads past the last pair (re-reads nobody uses)
    }
    // one more barrier for both groups, after which nothing is in flight.
    // (A wait for those loads inside the loop, in its last iteration, made
    // the compiler peel that iteration and spill fragment registers there;
    // with BT, right after their transpose reads, which it does not know
    // are still in flight.)
    stage_barrier();
  };
  auto run_g = [&](auto grp_, auto nt_) {
    if (mlive > MB / 2) run(CInt<MB>{}, grp_, nt_);
    else if (mlive > MB / 4) run(CInt<MB / 2>{}, grp_, nt_);
    else if (mlive > 0) run(CInt<MB / 4>{}, grp_, nt_);
    else run(CInt<0>{}, grp_, nt_);
  };
  if (grp == 0) run_g(CInt<0>{}, CInt<0>{});
  else if (w_once) run_g(CInt<1>{}, CInt<1>{});
  else run_g(CInt<1>{}, CInt<0>{});
  }  // !KMAJ || npairs > 0

  // epilogue: every ring read is done (the last barrier), every load landed
  mfma_drain();
  constexpr int OC = GATED ? WTN / 2 : WTN;  // output columns per wavefront
  char* const stg = smem + wave * WTM * (256 + 16);
  const int col0 = n0 + wn * OC;
  const float* sc0 = nullptr;  // FP8 weights: this expert's output-channel scales
  const float* sc1 = nullptr;
  if (FP8W) {
    sc0 = (routed ? g.sc0 : g.ssc0) + static_cast<size_t>(es) * g.n_dim;
    if (GATED) sc1 = (routed ? g.sc1 : g.ssc1) + static_cast<size_t>(es) * g.n_dim;
  }
  if constexpr (KMAJ) {
    const size_t cmat = static_cast<size_t>(g.a_rows) * g.n_dim;
    bf16_t* const c = e < g.alt_from
                          ? static_cast<bf16_t*>(g.out) + static_cast<size_t>(e) * cmat
                          : static_cast<bf16_t*>(g.out_alt) + static_cast<size_t>(e - g.alt_from) * cmat;
    // staged as bf16: 64 columns, whole 128-byte lines of a row, per pass
    // (32 fp32 columns per pass left half lines, and the weight gradients
    // wrote 1.37 GB for 0.94 GB)
    store_block<false, true, MB, NB, WTM>(acc, stg, lane, c, false, g.n_dim, m0 + wm * WTM,
                                          mvalid - wm * WTM, col0, g.n_dim);
  } else if (part < 0) {
    // (the plain pass: fp32 staging, 64 columns per pass, so every row write
    // is a whole 128-byte line)
    store_block<GATED, GATED, MB, NB, WTM, FP8W, 64>(acc, stg, lane, g.out, false, g.n_dim,
                                                     seg + m0 + wm * WTM, mvalid - wm * WTM,
                                                     col0, g.n_dim, sc0, sc1);
  } else if (!GATED) {  // fp32 partial rows of a split tail tile or of a dense part
    const long stride = dense ? g.a_rows : g.plan[kPlanStride];
    const long first = dense ? 0 : g.plan[kPlanRowSplit];
    const long prow = static_cast<long>(part) * stride + seg + m0 - first + wm * WTM;
    store_block<GATED, false, MB, NB, WTM, FP8W, 64>(acc, stg, lane, g.out_part, true, g.n_dim,
                                                     prow, mvalid - wm * WTM, col0, g.n_dim, sc0,
                                                     sc1);
  }
}

template <bool GATED>
hipError_t launch_pp(const GemmArgs& g, hipStream_t s) {
  if (g.dense_parts > 0) return hipErrorInvalidValue;  // launch_dense_gemm
  constexpr int COLS = GATED ? 128 : 256;
  const long blocks = expert_grid(g, GATED, COLS);
  if (g.wfp8 && g.narrow)
    hipLaunchKernelGGL((expert_gemm_pp_kernel<GATED, false, true, true>),
                       dim3(static_cast<unsigned>(blocks)), dim3(512), 0, s, g);
  else if (g.wfp8)
    hipLaunchKernelGGL((expert_gemm_pp_kernel<GATED, false, false, true>),
                       dim3(static_cast<unsigned>(blocks)), dim3(512), 0, s, g);
  else if (g.narrow)
    hipLaunchKernelGGL((expert_gemm_pp_kernel<GATED, false, true>),
                       dim3(static_cast<unsigned>(blocks)), dim3(512), 0, s, g);
  else
    hipLaunchKernelGGL((expert_gemm_pp_kernel<GATED>), dim3(static_cast<unsigned>(blocks)),
                       dim3(512), 0, s, g);
  return hipGetLastError();
}

}  // namespace

bool kmajor_gemm_fits(long a_rows, long n_dim, long k_dim) {
  // whole 128-byte buffers from 16-byte aligned rows, 32-bit lane offsets
  return a_rows > 0 && n_dim > 0 && k_dim % 64 == 0 && n_dim % 8 == 0 &&
         static_cast<size_t>(a_rows) * k_dim * 2 < (size_t{1} << 32) &&
         static_cast<size_t>(n_dim) * k_dim * 2 < (size_t{1} << 32);
}

hipError_t launch_kmajor_gemm(const GemmArgs& g, hipStream_t s) {
  if (!kmajor_gemm_fits(g.a_rows, g.n_dim, g.k_dim)) return hipErrorInvalidValue;
  const long blocks = kmajor_grid(g, 256, 256);
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((expert_gemm_pp_kernel<false, false, false, false, false, true>),
                     dim3(static_cast<unsigned>(blocks)), dim3(512), 0, s, g);
  return hipGetLastError();
}

bool expert_gemm_bt_fits(int bm, int k_dim, int n_dim, int rows0, long a_rows) {
  // whole pairs of 64-row buffers, each from one weight matrix; 16-byte
  // aligned K-rows; 32-bit offsets inside one expert's matrices and into A
  return (bm == 128 || bm == 256) && k_dim % 128 == 0 && rows0 > 0 && rows0 % 64 == 0 &&
         rows0 <= k_dim && n_dim % 8 == 0 && n_dim >= 8 &&
         static_cast<size_t>(k_dim) * n_dim * 2 < (size_t{1} << 32) &&
         static_cast<size_t>(a_rows) * k_dim * 2 < (size_t{1} << 32);
}

hipError_t launch_expert_gemm_bt(int bm, const GemmArgs& g, hipStream_t s) {
  // no split plan: the pieces of a split reduction shift their B offsets
  // along [n_dim, k_dim] rows, which this mode's K-row staging does not do
  if (!expert_gemm_bt_fits(bm, g.k_dim, g.n_dim, g.bt_rows0, g.a_rows) ||
      (g.bt_rows0 < g.k_dim && g.w1 == nullptr) || g.plan != nullptr)
    return hipErrorInvalidValue;
  if (bm == 256) {  // 8-wavefront ping-pong tiles
    hipLaunchKernelGGL((expert_gemm_pp_kernel<false, false, false, false, true>),
                       dim3(static_cast<unsigned>(expert_grid(g, false, 256))), dim3(512), 0, s, g);
    return hipGetLastError();
  }
  if (bm == 128) return launch_v<false, 128, 256, 3, false, true>(g, s);
  return hipErrorInvalidValue;
}

bool dense_gemm_fits(long a_rows, int k_dim, int n_dim, int parts) {
  // whole pairs of 128-byte buffers, each part at least one; 32-bit lane
  // offsets into a and into the weights
  return a_rows > 0 && k_dim % 64 == 0 && n_dim > 0 && n_dim % 8 == 0 && parts >= 1 &&
         parts <= k_dim / 64 && static_cast<size_t>(a_rows) * k_dim * 2 < (size_t{1} << 32) &&
         static_cast<size_t>(n_dim) * k_dim * 2 < (size_t{1} << 32);
}

hipError_t launch_dense_gemm(const GemmArgs& g, hipStream_t s) {
  if (g.dense_parts <= 0 || g.out_part == nullptr || g.w0 == nullptr || g.gather != nullptr ||
      !dense_gemm_fits(g.a_rows, g.k_dim, g.n_dim, g.dense_parts))
    return hipErrorInvalidValue;
  // every part must hold at least one pair of K steps
  const int npairs = g.k_dim * 2 / kLineBytes;
  if ((g.dense_parts - 1) * split_share(npairs, g.dense_parts) >= npairs) return hipErrorInvalidValue;
  const long tiles = (g.a_rows + 255) / 256, n_nt = (g.n_dim + 255) / 256;
  const long blocks = tiles * n_nt * g.dense_parts;
  hipLaunchKernelGGL((expert_gemm_pp_kernel<false, true>), dim3(static_cast<unsigned>(blocks)),
                     dim3(512), 0, s, g);
  return hipGetLastError();
}

int expert_gemm_cols(bool gated, int bm) {
  (void)bm;
  return gated ? 128 : 256;
}

hipError_t launch_expert_gemm(bool gated, int bm, const GemmArgs& g, hipStream_t s) {
  if (g.k_dim % 128 != 0) return hipErrorInvalidValue;  // whole pairs of 128-byte buffers
  // buffers of 64 KB (256-row tiles: 2 fit in the LDS) or 48 KB (128-row
  // tiles: 3 fit, keeping two pairs of K steps in flight)
  if (g.wfp8) {
    // FP8 weights: 48 KB (256-row tiles) or 32 KB (128-row tiles) per buffer,
    // so one more buffer of loads fits in flight than with bf16 weights
    if (bm == 256) {  // 8-wavefront ping-pong tiles
      if (gated) return launch_pp<true>(g, s);
      return launch_pp<false>(g, s);
    }
    if (bm != 128) return hipErrorInvalidValue;
    if (gated) return launch_v<true, 128, 256, 4, true>(g, s);
    return launch_v<false, 128, 256, 4, true>(g, s);
  }
  if (bm == 256) {  // 8-wavefront ping-pong tiles
    if (gated) return launch_pp<true>(g, s);
    return launch_pp<false>(g, s);
  }
  if (bm != 128) return hipErrorInvalidValue;
  if (gated) return launch_v<true, 128, 256, 3>(g, s);
  return launch_v<false, 128, 256, 3>(g, s);
}

}  // namespace moe
