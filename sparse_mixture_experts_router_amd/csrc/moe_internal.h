// Internal declarations shared by the HIP translation units of libmoe.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// ---------------------------------------------------------------- constants
constexpr int kRouteTokens = 64;      // tokens per routing workgroup
constexpr int kMaxExperts = 512;
constexpr int kMaxTopK = 16;
constexpr int kMaxShared = 4;

// ---------------------------------------------------------------- vector types
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;  // one 16-byte fragment
typedef uint16_t bf16_t;  // storage type of a bf16 element

// Workspace carve-out of one forward call (every pointer is device memory).
struct Workspace {
  int32_t* topk_idx;   // [T, k]
  float* topk_gate;    // [T, k]
  int32_t* lrank;      // [T, k]     rank of the assignment inside its block
  float* route_partial;// [ksplit, T, N] split-K partial logits
  int32_t* blk_counts; // [B, N]
  float* blk_psum;     // [B, N]
  int32_t* blk_base;   // [B, N]
  int32_t* counts;     // [N + S]
  float* prob_sum;     // [N]
  int32_t* offsets;    // [N + S + 1]
  int32_t* sorted_tok; // [T k + S T]
  int32_t* inv_row;    // [T, k]
  int2* tiles_up;      // tile list of the gate/up GEMM
  int2* tiles_down;    // tile list of the down GEMM
  int32_t* items_up;   // work items of the large-tile gate/up GEMM (when used)
  int32_t* items_down; // and of the large-tile down GEMM
  int32_t* tbases;     // group tile bases for the items kernel (see ItemSpec)
  int32_t* ntiles;     // [kPlanInts]: entries in tiles_up, tiles_down, then the down-pass
                       // split plan (see kPlan*)
  void* hidden;        // [T k + S T, F]  dtype
  void* yperm;         // [T k + S T, d]  dtype
  float* ypart;        // fp32 partial rows of a down pass split over its reduction
};

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error.
// Router GEMM + selection.  ksplit > 1 splits the reduction over workgroups
// (few tokens): fp32 partial logits [ksplit, T, N] go to `partial` and a
// second kernel sums them in a fixed order before the selection.
// route_dense_parts > 0: the router GEMM runs on the ping-pong expert GEMM
// kernel in its dense mode (256-token tiles, the reduction split into that
// many parts) and ksplit must equal it; 0: the router kernel, ksplit from
// route_split.
int route_split(int T, int d, int dtype);
int route_dense_parts(int T, int d, int N, int dtype, int cus);
hipError_t launch_route(int dtype, const void* x, const void* w_router,
                        const float* logit_bias, const float* select_bias,
                        int T, int d, int N, int k, int ksplit, bool dense, float* partial,
                        float* logits_out, int32_t* topk_idx, float* topk_gate,
                        int32_t* lrank, int32_t* blk_counts, float* blk_psum,
                        hipStream_t s);

// Split of the down pass recorded in the plan: parts > 1 splits every row
// (decode); otherwise tail_nnt > 0 lets the scan split the last row tiles of
// a tail_nnt-column-tile grid that would leave cus compute units mostly idle.
// Work-item lists of the large-tile GEMMs (items kernel, after the scan):
// for every row group (expert) its row tiles x column tiles, in blocks of up
// to 8 row tiles x (window / row tiles) column tiles, so the `window`
// workgroups an XCD runs at once cover one expert's rows next to a band of
// its weight tiles.  nnt = 0: no list for that pass.  The scan writes the
// groups' first tiles to tbases: [0, G] gate/up (G = N + S groups, [G] =
// their total), [G + 1, 2G + 1] down, then the tiles each list covers
// (gate/up, down without the split tail).
struct ItemSpec {
  int nnt_up, nnt_down;  // column tiles of the gate/up and down passes
  int window;            // workgroups one XCD runs at once
  int32_t* items_up;
  int32_t* items_down;
  int32_t* tbases;       // [kTbInts(G)], or null: the scan writes nothing
  // Narrow tail tiles (ping-pong kernel only, an even number of column
  // tiles): a group's last row tile with at most kNarrowRows rows becomes
  // items of two column tiles each, listed next to the items of its full
  // row tiles on the same columns, so that they stream the same weight rows
  // at about the same time.
  int narrow_up, narrow_down;
};
constexpr int kNarrowRows = 64;
// Layout of tbases for G = N + S groups: tile bases of the gate/up list
// [0, G], of the down list [G + 1, 2G + 1], the tiles each list covers
// (2G + 2, 2G + 3), then item bases of the gate/up list [2G + 4, 3G + 4]
// and of the down list [3G + 5, 4G + 5] (the last entry of each: its total).
inline int kTbInts(int G) { return 4 * G + 6; }
__host__ __device__ inline int tb_items_up(int G) { return 2 * G + 4; }
__host__ __device__ inline int tb_items_down(int G) { return 3 * G + 5; }
hipError_t launch_items(const ItemSpec& is, int groups, long max_items, hipStream_t s);
constexpr int kItemColBits = 12;  // column tile in the low bits of an item
constexpr int kItemMaxTiles = 1 << 19;

// Permutation written by the scan kernel itself (sorted_tok != nullptr, for
// small batches) instead of a separate scatter launch.
struct ScatterSpec {
  const int32_t* topk_idx;
  const int32_t* lrank;
  int32_t* sorted_tok;
  int32_t* inv_row;
};
constexpr long kScanScatterMaxRows = 2048;  // two rows per scan thread

// Balance statistics the scan kernel writes as well (each pointer may be
// null): f [N], P [N], aux [2] = [N sum f P, alpha N sum f P].
struct BalanceSpec {
  float* f;
  float* P;
  float* aux;
  float alpha;
};

struct SplitSpec {
  int parts;      // host split of every row (grouped_gemm.hip), or <= 1
  int tail_nnt;   // column tiles of the down pass (0: no tail split)
  int tail_cus;   // compute units one round of workgroups fills
  long tail_cap_rows;  // partial rows the workspace holds over all parts
  int tail_max_parts;  // most parts one tile may be split into
};
hipError_t launch_scan(const int32_t* blk_counts, const float* blk_psum, int T,
                       int N, int k, int S, int capacity, int bm_up, int cap_up, int bm_down,
                       int cap_down, const SplitSpec& split, const ItemSpec& items,
                       const ScatterSpec& sc, const BalanceSpec& bal, int32_t* blk_base,
                       int32_t* counts, float* prob_sum, int32_t* user_counts,
                       float* user_prob_sum, int32_t* offsets, int2* tiles_up,
                       int2* tiles_down, int32_t* ntiles, hipStream_t s);

hipError_t launch_scatter(const int32_t* topk_idx, const int32_t* lrank,
                          const int32_t* blk_base, const int32_t* offsets,
                          int T, int N, int k, int S, int capacity,
                          int32_t* sorted_tok, int32_t* inv_row, hipStream_t s);

// Arguments of the routing kernels (route.hip, route_tile.h).
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

// The routing of an all-token expert pass: every expert's GEMMs run on all T
// (<= 64) tokens of the batch, expert-major (expert g's rows are g T .. g T +
// T - 1, shared experts after the routed ones), so only the combine needs the
// routing.  One workgroup routes the batch (one block, no split of the
// reduction) and writes, besides the indices, gates and logits:
//   inv_row[t, s] = e T + t for slot s's expert e, or -1 when the capacity
//                   drops it (the expert keeps its first `capacity` tokens in
//                   token order; the rank is the block rank the selection
//                   computes);
//   counts[e], prob_sum[e] (and the caller's copies): the router's choice
//                   before any drop, counts[N + s] = T;
//   offsets[g] = g T for g <= N + S (the combine finds shared rows there);
//   plan: the down pass's split over its reduction (parts, first split row
//         0, part stride (N + S) T), or no split;
//   f, P and the loss (balance_block), when asked for.
struct AllTokenRoute {
  RouteArgs a;  // ksplit 1, steps_per_split = every K step
  int S, capacity;
  int down_parts;  // > 1: the down pass writes that many fp32 partial rows
  int32_t* inv_row;
  int32_t* counts;
  float* prob_sum;
  int32_t* user_counts;
  float* user_prob_sum;
  int32_t* offsets;
  int32_t* plan;
  float* f;
  float* P;
  float* aux;
  float alpha;
};

struct GemmArgs {
  const void* a;             // x [T, d] (gather) or hidden [rows, F] (direct)
  const int32_t* gather;     // sorted_tok, or NULL for direct rows
  const void* w0;            // routed weights for expert 0 (gate or down)
  const void* w1;            // routed up weights, gated GEMM only
  const void* ws0;           // shared-expert weights (gate or down)
  const void* ws1;           // shared up weights, gated GEMM only
  const int32_t* offsets;    // [N + S + 1]
  const int2* tiles;         // tile list
  const int32_t* ntiles;     // device count of tiles
  void* out;                 // [rows, n_dim]
  int a_rows;                // rows of a (gathered indices are clamped to it)
  int n_experts;             // routed experts N (e >= N is shared e - N)
  int k_dim;                 // reduction length (d or F)
  int n_dim;                 // output columns (F or d)
  int tiles_cap;             // grid rows
  int ksplit;                // > 1: reduction split over workgroups (plain pass only)
  float* out_part;           // fp32 partial outputs [ksplit, a_rows, n_dim] when ksplit > 1
  const int32_t* plan;       // device split plan of the down pass (kPlan* entries), or null
  const int32_t* items;      // large-tile kernel: work items, (tile << 12) | column tile
  const int32_t* nitems;     // device count of those items (null: tiles x column tiles)
  int narrow;                // ping-pong kernel: the list holds narrow tail items
  // Dense mode of the ping-pong kernel (launch_dense_gemm): > 0 = the rows
  // are all a_rows rows of a, in one group whose weights are w0, with no
  // tile or item list; the reduction is split into this many parts, each
  // writing fp32 partial outputs [parts, a_rows, n_dim] to out_part.
  int dense_parts;
  int cus;                   // compute units of the device (grid sizing)
  bool wfp8;                 // weights are FP8 E4M3 codes with per-output-channel scales
  const float* sc0;          // routed scales [N, n_dim] (gate or down), FP8 weights only
  const float* sc1;          // routed up scales, gated GEMM only
  const float* ssc0;         // shared-expert scales [S, n_dim]
  const float* ssc1;
  // Weight-gradient mode of the large-tile kernel (launch_kmajor_gemm):
  // C_g = A_g B_g^T for groups g, A [a_rows, ...] and B [n_dim, ...] both
  // with row stride k_dim elements, group g reducing over columns
  // kbase[g] .. kbase[g + 1]; C_g is [a_rows, n_dim], written to out (g <
  // alt_from) or out_alt (g >= alt_from).
  const int32_t* kbase;
  void* out_alt;
  int groups;
  int alt_from;
  // B-row mode of the large-tile kernel (launch_expert_gemm_bt): the plain
  // pass with weights given as [k_dim, n_dim] per expert (K-rows, n_dim
  // contiguous) instead of [n_dim, k_dim].  Rows 0 .. bt_rows0 - 1 of the
  // reduction come from w0 / ws0 (expert stride bt_rows0 x n_dim), the rest
  // from w1 / ws1 (stride (k_dim - bt_rows0) x n_dim).
  int bt_rows0;
  // All-token expert pass of the register-staged kernel (grouped_gemm.hip):
  // all_tok = T > 0 makes workgroup row g < all_groups = N + S expert g on
  // every token, rows g T .. g T + T - 1, with no tile list.
  int all_tok;
  int all_groups;
};

// Pairs of K steps (128-byte row buffers) that each of `parts` pieces of an
// n-pair reduction takes in the large-tile GEMM: an even count (its loop
// runs two buffers per iteration), the last piece taking what is left.
__host__ __device__ inline int split_share(int n, int parts) {
  const int per = (n + parts - 1) / parts;
  return (per + 1) & ~1;
}
// The most pieces (<= cap, each >= 8 pairs and none empty) an n-pair
// reduction splits into.
inline int max_split_parts(int n, int cap) {
  int best = 1;
  for (int p = 2; p <= cap; ++p)
    if (n / p >= 8 && (p - 1) * split_share(n, p) < n) best = p;
  return best;
}

// Device-side plan of a down pass whose reduction is split over workgroups,
// written by the scan kernel after ntiles[0..1]: the combine kernel adds the
// fp32 parts of every row at or past kPlanRowSplit.
//   decode : all rows, kPlanParts = the host's split (grouped_gemm.hip);
//   prefill: the last kPlanTailTiles row tiles of the large-tile down GEMM,
//            whose workgroups would otherwise run as a thin last round.
enum { kPlanParts = 0, kPlanRowSplit = 1, kPlanStride = 2, kPlanTailTiles = 3, kPlanInts = 6 };

// Kernel choice for one grouped GEMM: variant 0 = register-staged tiles
// (grouped_gemm.hip, fp32 and few-row shapes), 1 = large direct-to-LDS bf16
// tiles (expert_gemm.hip), which run from the scan's work-item lists; bm =
// rows per tile (the tile list's granularity).
struct GemmPick {
  int variant;
  int bm;
};
// a_bytes / w_bytes: bytes of the A operand (all its rows) and of one expert's
// weight matrix; the direct-to-LDS kernel addresses both with 32-bit offsets.
// fp8w: FP8 expert weights (both kernels take them: the register-staged one
// widens them on their way into LDS, the large-tile one after its LDS reads).
GemmPick pick_gemm(int dtype, bool fp8w, bool gated, long rows_per_expert, size_t a_bytes,
                   size_t w_bytes, int k_dim);
// route: the all-token gate/up pass's routing workgroup, or null.
hipError_t launch_gemm(int dtype, bool gated, GemmPick pick, const GemmArgs& g, hipStream_t s,
                       const AllTokenRoute* route = nullptr);
// bf16 weight-gradient products on the large-tile kernel (GemmArgs' kbase
// fields, segments a multiple of 64); hipErrorInvalidValue when the operands
// do not fit it, as kmajor_gemm_fits tells beforehand.
hipError_t launch_kmajor_gemm(const GemmArgs& g, hipStream_t s);
bool kmajor_gemm_fits(long a_rows, long n_dim, long k_dim);
// The plain grouped GEMM on the large-tile kernel with B given as K-rows
// (GemmArgs' bt_rows0); hipErrorInvalidValue when the shape does not fit it.
hipError_t launch_expert_gemm_bt(int bm, const GemmArgs& g, hipStream_t s);
bool expert_gemm_bt_fits(int bm, int k_dim, int n_dim, int rows0, long a_rows);
hipError_t launch_generic_gemm(int dtype, bool gated, int bm, const GemmArgs& g, hipStream_t s,
                               const AllTokenRoute* route = nullptr);
hipError_t launch_expert_gemm(bool gated, int bm, const GemmArgs& g, hipStream_t s);
// The plain (non-gated) bf16 ping-pong kernel in dense mode (GemmArgs'
// dense_parts): hipErrorInvalidValue when the operands do not fit it.
bool dense_gemm_fits(long a_rows, int k_dim, int n_dim, int parts);
hipError_t launch_dense_gemm(const GemmArgs& g, hipStream_t s);
// Output columns per tile of the large-tile kernel launch_expert_gemm picks.
int expert_gemm_cols(bool gated, int bm);

// y from the per-expert rows: yperm (layer dtype), except rows at or past
// plan[kPlanRowSplit], which are the sum of plan[kPlanParts] fp32 partial
// row sets ypart[part][row - row_split] (part stride plan[kPlanStride] rows).
// Slots with inv_row < 0 (dropped by a capacity) add nothing; shared expert
// s's row for token t is offsets[N + s] + t.
hipError_t launch_combine(int dtype, const void* yperm, const float* ypart,
                          const int32_t* plan, const int32_t* inv_row, const float* topk_gate,
                          const int32_t* offsets, int N, int T, int d, int k, int S, void* y,
                          hipStream_t s);
int down_split(int dtype, bool fp8w, const GemmPick& pick, long tiles_est, int n_dim, int k_dim,
               int cus);

hipError_t launch_balance(int T, int N, int k, const int32_t* counts,
                          const float* prob_sum, float alpha, float* f_out,
                          float* P_out, float* aux_out, hipStream_t s);

// ---------------------------------------------------------------- backward (backward.hip)
// dtype: 1 = bf16, 0 = fp32 (the layer type of every operand but the fp32
// ones named).
// dst[b][c][col0 + r] = src[b][r][c] (r < R), 0 for R <= r < rpad.
hipError_t launch_transpose(int dtype, const void* src, int R, int C, long src_batch, void* dst,
                            long ldd, int col0, int rpad, long dst_batch, int batch,
                            hipStream_t s);
// kbase[g + 1] = kbase[g] + (offsets[g + 1] - offsets[g] rounded up to
// align: 64 or 128).
hipError_t launch_kbase(const int32_t* offsets, int G, int align, int32_t* kbase, hipStream_t s);
// Group g's rows (source row gather[r] or r, times rscale[r] when given) into
// columns kbase[g] .. of dst [C, ldd]; padding columns 0.  kmax: a multiple
// of 64 at least kbase[G].
hipError_t launch_segment_transpose(int dtype, const void* src, int C, int src_rows,
                                    const int32_t* gather, const float* rscale,
                                    const int32_t* offsets, const int32_t* kbase, int G,
                                    long kmax, void* dst, long ldd, hipStream_t s);
hipError_t launch_row_gate(const int32_t* inv_row, const float* gate, const int32_t* offsets,
                           int T, int k, int N, int S, float* rgate, hipStream_t s);
hipError_t launch_swiglu_bwd(int dtype, const void* G_, const void* U, const void* D,
                             const float* rgate, const int32_t* offsets, int G, int F,
                             long rows_max, void* H, void* dAB, float* dg_row, hipStream_t s);
hipError_t launch_router_bwd(int dtype, const float* logits, const int32_t* idx,
                             const float* gate, const int32_t* inv_row, const float* dg_row,
                             const int32_t* counts, int T, int N, int k, float alpha,
                             float aux_grad, int Kr, void* dr_pad, float* dr32, hipStream_t s);
hipError_t launch_colsum(const float* dr32, int T, int N, float* out, hipStream_t s);
hipError_t launch_dx_combine(int dtype, const void* dXp, const float* dxr, const int32_t* inv_row,
                             const int32_t* offsets, int T, int N, int k, int S, int d, void* dx,
                             hipStream_t s);
hipError_t launch_bias_update(const int32_t* counts, int N, float rate, float* bias,
                              hipStream_t s);
// C_g[m][n] = sum over kbase[g] <= j < kbase[g + 1] (or 0 <= j < k_all when
// kbase is null) of a[m][j] b[n][j]; groups >= alt_from write to c_alt.
// Every segment (and k_all) a multiple of 128 elements, or of 64 where the
// bf16 large-tile kernel takes the product (kmajor_gemm_fits); N a multiple
// of 64.
hipError_t launch_kgemm(int dtype, bool out_f32, const void* a, long lda, const void* b, long ldb,
                        int M, int N, int groups, const int32_t* kbase, int k_all, void* c,
                        void* c_alt, int alt_from, hipStream_t s);

// ---------------------------------------------------------------- device helpers
__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  __bf16 b = static_cast<__bf16>(f);  // round to nearest even (v_cvt_pk_bf16_f32)
  return __builtin_bit_cast(bf16_t, b);
}

}  // namespace moe
