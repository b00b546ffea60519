// Host side of libmoe.so: argument validation, workspace carve-out and the
// launch sequence of the layer forward.  Every launch goes on the caller's
// stream; nothing here allocates, frees or waits on the device.
#include "moe.h"
#include "moe_internal.h"
#include "lds_ring.h"  // kRowBytes: the routing block's K step

#include <algorithm>
#include <atomic>
#include <cmath>
#include <stdio.h>
#include <string.h>

namespace moe {
namespace {

thread_local char g_last_error[256] = "";

moe_status fail(moe_status st, const char* what) {
  snprintf(g_last_error, sizeof(g_last_error), "%s", what);
  return st;
}

moe_status hip_fail(hipError_t err, const char* where) {
  snprintf(g_last_error, sizeof(g_last_error), "%s: %s", where, hipGetErrorString(err));
  return MOE_ERR_HIP;
}

constexpr size_t kAlign = 256;
constexpr int R_COUNT_MAX = 32;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Compute units of the current device, asked of the runtime once per device:
// the attribute query costs a host round trip that every decode step would
// otherwise pay.  Devices past the table are asked on every call.
constexpr int kCuCacheDevices = 64;
std::atomic<int> g_cus[kCuCacheDevices];  // 0: not asked yet

int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < kCuCacheDevices) {
    const int v = g_cus[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  if (dev < kCuCacheDevices) g_cus[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Row tiles that a grouped GEMM with `bm`-row tiles can need in the worst
// case: each routed expert with c_e > 0 rows needs ceil(c_e / bm) tiles, and
// sum_e ceil(c_e / bm) <= (T k + N (bm - 1)) / bm; each shared expert needs
// ceil(T / bm).
long tile_capacity(const moe_config& c, int bm) {
  const long tk = static_cast<long>(c.T) * c.top_k;
  const long routed = (tk + static_cast<long>(c.n_experts) * (bm - 1)) / bm;
  const long routed_cap = routed < tk ? routed : tk;
  return routed_cap + static_cast<long>(c.n_shared) * ((c.T + bm - 1) / bm);
}

struct Plan {
  GemmPick up, down;
  int ksplit;  // router reduction split
  int rdense;  // > 0: the router GEMM on the large-tile kernel, ksplit = rdense parts
  int dsplit;  // down-pass reduction split
  SplitSpec split;  // what the scan may record in the down pass's split plan
  int nnt_up, nnt_down;  // column tiles of the large-tile GEMMs (0: generic kernel)
  int narrow_up, narrow_down;  // their lists hold narrow tail items (ping-pong kernel)
  int cus;          // compute units of the current device
  int bm_up, bm_down;
  int cap_up, cap_down;
  bool all_tok;     // all-token expert pass (AllTokenRoute): decode batches
  size_t rows_g;    // rows of the expert passes: T (k + S), or (N + S) T all-token
  size_t total;
  size_t off[R_COUNT_MAX];
};

enum {
  R_IDX, R_GATE, R_LRANK, R_PART, R_BCNT, R_BPS, R_BBASE, R_CNT, R_PS, R_OFF, R_SORT, R_INV,
  R_TUP, R_TDN, R_IUP, R_IDN, R_TB, R_NT, R_HID, R_YP, R_YPART, R_COUNT
};

// Workspace of moe_layer_forward_noalloc: a file-scope device array, one copy
// per GPU (the runtime allocates it when it loads this library's code object
// on that GPU and keeps it until the process ends).  In host code `scratch`
// names a host-side stand-in, not device memory: its device address is asked
// of the runtime once per device, with that device current, and only that
// address is ever handed to kernels.
__device__ __align__(256) char scratch[MOE_NOALLOC_SCRATCH_BYTES];
std::atomic<void*> g_scratch[kCuCacheDevices];  // device address per device, or null

moe_status scratch_address(void** ptr) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return hip_fail(err, "hipGetDevice");
  if (dev < 0 || dev >= kCuCacheDevices)
    return fail(MOE_ERR_UNSUPPORTED, "device index past the scratch address table");
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return hip_fail(err, "hipGetSymbolAddress(scratch)");
    if (p == nullptr) return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) gave NULL");
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return MOE_OK;
}

// bwd: the plan of the backward's routing and plain GEMMs instead: the "up"
// tile list serves the passes with F output columns and K = d (G, U, D), the
// "down" list the pass with d output columns and K = 2F (dXp); no split of
// any reduction, and no forward activations.
Plan make_plan(const moe_config& c, bool bwd = false) {
  Plan p{};
  p.cus = device_cus();
  const long rows_per_expert = static_cast<long>(c.T) * c.top_k / c.n_experts;
  const size_t eb_ = c.dtype == MOE_BF16 ? 2 : 4;
  const bool fp8w = c.weight_format == MOE_WEIGHTS_FP8_E4M3;
  const size_t rows_all = static_cast<size_t>(c.T) * (c.top_k + c.n_shared);
  const size_t w_mat = static_cast<size_t>(c.d_model) * c.d_ff * (fp8w ? 1 : eb_);
  if (bwd) {
    p.up = pick_gemm(c.dtype, false, false, rows_per_expert,
                     static_cast<size_t>(c.T) * c.d_model * eb_, w_mat, c.d_model);
    p.down = pick_gemm(c.dtype, false, false, rows_per_expert, rows_all * 2 * c.d_ff * eb_,
                       2 * w_mat, 2 * c.d_ff);
    // Few rows per expert (decode-sized batches): the backward's plain passes
    // take 256-row large tiles too (the ping-pong kernel).  Each expert's
    // weights still stream once (one row tile per expert), and D and dXp
    // read them as K-rows instead of from transposed copies of every expert
    // weight.  Mixtral-shaped decode backward, same box: 3.34 ms with the
    // transposes, 2.48 with 128-row tiles, 2.07 with 256-row tiles.
    const bool small_off = static_cast<size_t>(c.T) * c.d_model * eb_ < (size_t{1} << 32) &&
                           rows_all * 2 * c.d_ff * eb_ < (size_t{1} << 32) &&
                           2 * w_mat < (size_t{1} << 32);
    if (c.dtype == MOE_BF16 && small_off && c.d_model % 128 == 0 && p.up.variant == 0 &&
        p.down.variant == 0) {
      p.up = GemmPick{1, 256};
      p.down = GemmPick{1, 256};
    }
  } else {
    p.up = pick_gemm(c.dtype, fp8w, true, rows_per_expert,
                     static_cast<size_t>(c.T) * c.d_model * eb_, w_mat, c.d_model);
    p.down = pick_gemm(c.dtype, fp8w, false, rows_per_expert, rows_all * c.d_ff * eb_, w_mat,
                       c.d_ff);
  }
  // the large-tile kernel's work items hold tile indices below kItemMaxTiles
  if (p.up.variant == 1 && tile_capacity(c, p.up.bm) >= kItemMaxTiles) p.up = GemmPick{0, 128};
  if (p.down.variant == 1 && tile_capacity(c, p.down.bm) >= kItemMaxTiles)
    p.down = GemmPick{0, 128};
  p.bm_up = p.up.bm;
  p.bm_down = p.down.bm;
  // All-token expert pass: with at most 32 tokens one 32-row tile per expert
  // holds the whole batch, so running every expert on every token costs the
  // decode GEMMs no more matrix work and no more weight bytes, as long as
  // (nearly) every expert would be active anyway: then only the combine
  // needs the routing, which one workgroup of the gate/up launch computes
  // meanwhile instead of the route, select and scan launches before it.
  // Expected idle experts under uniform routing: N (1 - k/N)^T; the pass is
  // taken when that is below one half (the Mixtral-shaped decode: 8e-4).
  // Each tile then loads all 32 activation rows per K step instead of the
  // few routed ones; with FP8 weights (half the weight bytes per step) that
  // cost more than the routing launches it saves (Mixtral-shaped decode,
  // same box: 0.320 -> 0.334 ms; bf16 weights 0.526 -> 0.512 ms).
  if (!bwd && !fp8w && c.T >= 1 && c.T <= 32 && c.n_experts <= 64 && p.up.variant == 0 &&
      p.up.bm == 32 && p.down.variant == 0 && p.down.bm == 32) {
    const double idle =
        c.n_experts * std::pow(1.0 - static_cast<double>(c.top_k) / c.n_experts, c.T);
    p.all_tok = idle <= 0.5;
  }
  p.cap_up = static_cast<int>(tile_capacity(c, p.bm_up));
  p.cap_down = static_cast<int>(tile_capacity(c, p.bm_down));
  const size_t T = c.T, N = c.n_experts, k = c.top_k, S = c.n_shared;
  const size_t B = (T + kRouteTokens - 1) / kRouteTokens;
  const size_t rows = T * k + S * T;
  p.rows_g = p.all_tok ? (N + S) * T : rows;
  const size_t eb = c.dtype == MOE_BF16 ? 2 : 4;
  size_t sz[R_COUNT];
  sz[R_IDX] = T * k * 4;
  sz[R_GATE] = T * k * 4;
  sz[R_LRANK] = T * k * 4;
  p.rdense = route_dense_parts(c.T, c.d_model, c.n_experts, c.dtype, p.cus);
  p.ksplit = p.rdense > 0 ? p.rdense : route_split(c.T, c.d_model, c.dtype);
  // moe_route routes an all-token batch as its forward does: one workgroup,
  // no split of the reduction, so both give bitwise the same logits,
  // selection and statistics
  if (p.all_tok) {
    p.rdense = 0;
    p.ksplit = 1;
  }
  sz[R_PART] = p.ksplit > 1 ? static_cast<size_t>(p.ksplit) * T * N * 4 : 0;
  sz[R_BCNT] = B * N * 4;
  sz[R_BPS] = B * N * 4;
  sz[R_BBASE] = B * N * 4;
  sz[R_CNT] = (N + S) * 4;
  sz[R_PS] = N * 4;
  sz[R_OFF] = (N + S + 1) * 4;
  sz[R_SORT] = rows * 4;
  sz[R_INV] = T * k * 4;
  sz[R_TUP] = static_cast<size_t>(p.cap_up) * 8;
  sz[R_TDN] = static_cast<size_t>(p.cap_down) * 8;
  // work-item lists of the large-tile kernel (column tiles of the width its
  // chosen instance computes)
  if (p.up.variant == 1) {
    const int cols = expert_gemm_cols(!bwd, p.up.bm);
    p.nnt_up = (c.d_ff + cols - 1) / cols;
  }
  if (p.down.variant == 1) {
    const int cols = expert_gemm_cols(false, p.down.bm);
    p.nnt_down = (c.d_model + cols - 1) / cols;
  }
  // narrow tail items: forward passes on the ping-pong kernel (bf16 or FP8
  // weights, 256-row tiles), with an even number of column tiles
  p.narrow_up = !bwd && c.dtype == MOE_BF16 && p.up.variant == 1 && p.up.bm == 256 &&
                p.nnt_up >= 2 && p.nnt_up % 2 == 0;
  // (down pass: only with few rows per expert.  Measured, same box: the
  // DeepSeek-V3 shape's down launch 2.39 -> 2.24 ms with them, but the
  // Mixtral- and Qwen3-shaped ones, ~1024 rows per expert, 0.717 -> 0.754
  // and 1.674 -> 1.730 ms)
  p.narrow_down = !bwd && c.dtype == MOE_BF16 && p.down.variant == 1 &&
                  p.down.bm == 256 && p.nnt_down >= 2 && p.nnt_down % 2 == 0 &&
                  rows_per_expert <= 384;
  sz[R_IUP] = static_cast<size_t>(p.cap_up) * p.nnt_up * 4;
  sz[R_IDN] = static_cast<size_t>(p.cap_down) * p.nnt_down * 4;
  sz[R_TB] = static_cast<size_t>(kTbInts(static_cast<int>(N + S))) * 4;
  sz[R_NT] = kPlanInts * 4;
  sz[R_HID] = bwd ? 0 : p.rows_g * static_cast<size_t>(c.d_ff) * eb;

  {
    // row tiles the down pass will have: about one per expert that gets
    // rows (at most min(N, T k) of them) or T k / bm, whichever is more,
    // plus the shared experts' tiles, at most the capacity
    const long tk = static_cast<long>(T * k), bm = p.bm_down;
    const long used = static_cast<long>(N) < tk ? static_cast<long>(N) : tk;
    const long routed = (tk + bm - 1) / bm > used ? (tk + bm - 1) / bm : used;
    long est = routed + static_cast<long>(S) * ((static_cast<long>(T) + bm - 1) / bm);
    if (est > p.cap_down) est = p.cap_down;
    if (p.all_tok) est = static_cast<long>(N + S);
    p.dsplit = bwd ? 1 : down_split(c.dtype, fp8w, p.down, est, c.d_model, c.d_ff, p.cus);
  }
  sz[R_YP] = (p.dsplit > 1 || bwd) ? 0 : p.rows_g * static_cast<size_t>(c.d_model) * eb;
  p.split = SplitSpec{p.dsplit, 0, p.cus, 0, 1};
  if (p.dsplit <= 1 && p.down.variant == 1 && !bwd) {
    // tail split of the large-tile down GEMM
    const int nnt = p.nnt_down;
    p.split.tail_nnt = nnt;
    p.split.tail_cap_rows = static_cast<long>(p.cus / nnt) * p.bm_down;
    p.split.tail_max_parts = max_split_parts(c.d_ff * 2 / 128, 8);
    if (p.split.tail_cap_rows < 2L * p.bm_down || p.split.tail_max_parts < 2) {
      p.split.tail_nnt = 0;
      p.split.tail_cap_rows = 0;
    }
  }
  sz[R_YPART] = p.dsplit > 1 ? static_cast<size_t>(p.dsplit) * p.rows_g * c.d_model * 4
                             : static_cast<size_t>(p.split.tail_cap_rows) * c.d_model * 4;
  size_t o = 0;
  for (int i = 0; i < R_COUNT; ++i) {
    p.off[i] = o;
    o += align_up(sz[i] ? sz[i] : 1);
  }
  p.total = o;
  return p;
}

Workspace carve(const Plan& p, void* base) {
  char* b = static_cast<char*>(base);
  Workspace w{};
  w.topk_idx = reinterpret_cast<int32_t*>(b + p.off[R_IDX]);
  w.topk_gate = reinterpret_cast<float*>(b + p.off[R_GATE]);
  w.lrank = reinterpret_cast<int32_t*>(b + p.off[R_LRANK]);
  w.route_partial = reinterpret_cast<float*>(b + p.off[R_PART]);
  w.blk_counts = reinterpret_cast<int32_t*>(b + p.off[R_BCNT]);
  w.blk_psum = reinterpret_cast<float*>(b + p.off[R_BPS]);
  w.blk_base = reinterpret_cast<int32_t*>(b + p.off[R_BBASE]);
  w.counts = reinterpret_cast<int32_t*>(b + p.off[R_CNT]);
  w.prob_sum = reinterpret_cast<float*>(b + p.off[R_PS]);
  w.offsets = reinterpret_cast<int32_t*>(b + p.off[R_OFF]);
  w.sorted_tok = reinterpret_cast<int32_t*>(b + p.off[R_SORT]);
  w.inv_row = reinterpret_cast<int32_t*>(b + p.off[R_INV]);
  w.tiles_up = reinterpret_cast<int2*>(b + p.off[R_TUP]);
  w.tiles_down = reinterpret_cast<int2*>(b + p.off[R_TDN]);
  w.items_up = reinterpret_cast<int32_t*>(b + p.off[R_IUP]);
  w.items_down = reinterpret_cast<int32_t*>(b + p.off[R_IDN]);
  w.tbases = reinterpret_cast<int32_t*>(b + p.off[R_TB]);
  w.ntiles = reinterpret_cast<int32_t*>(b + p.off[R_NT]);
  w.hidden = b + p.off[R_HID];
  w.yperm = b + p.off[R_YP];
  w.ypart = reinterpret_cast<float*>(b + p.off[R_YPART]);
  return w;
}

moe_status check_config(const moe_config* c) {
  if (c == nullptr) return fail(MOE_ERR_INVALID_ARG, "cfg is NULL");
  if (c->T < 0 || c->d_model <= 0 || c->n_experts <= 0 || c->top_k <= 0 || c->d_ff <= 0 ||
      c->n_shared < 0 || c->capacity < 0)
    return fail(MOE_ERR_INVALID_ARG, "sizes must be positive (T, S, capacity >= 0)");
  if (c->top_k > c->n_experts) return fail(MOE_ERR_INVALID_ARG, "top_k > n_experts");
  if (c->dtype != MOE_F32 && c->dtype != MOE_BF16) return fail(MOE_ERR_INVALID_ARG, "bad dtype");
  if (c->weight_format != MOE_WEIGHTS_DTYPE && c->weight_format != MOE_WEIGHTS_FP8_E4M3)
    return fail(MOE_ERR_INVALID_ARG, "bad weight_format");
  if (c->weight_format == MOE_WEIGHTS_FP8_E4M3 && c->dtype != MOE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "FP8 expert weights need dtype MOE_BF16");
  if (c->n_experts > kMaxExperts) return fail(MOE_ERR_UNSUPPORTED, "n_experts > 512");
  if (c->top_k > kMaxTopK) return fail(MOE_ERR_UNSUPPORTED, "top_k > 16");
  if (c->n_shared > kMaxShared) return fail(MOE_ERR_UNSUPPORTED, "n_shared > 4");
  if (c->d_model % 64 != 0 || c->d_ff % 64 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "d_model and d_ff must be multiples of 64");
  const long rows = static_cast<long>(c->T) * (c->top_k + c->n_shared);
  if (rows >= (1L << 30)) return fail(MOE_ERR_UNSUPPORTED, "T * (k + S) too large");
  return MOE_OK;
}

moe_status check_weights(const moe_config& c, const moe_weights* w, bool experts) {
  if (w == nullptr) return fail(MOE_ERR_INVALID_ARG, "weights is NULL");
  if (w->w_router == nullptr) return fail(MOE_ERR_INVALID_ARG, "w_router is NULL");
  if (!aligned16(w->w_router)) return fail(MOE_ERR_INVALID_ARG, "w_router not 16-byte aligned");
  if (!experts) return MOE_OK;
  const void* req[3] = {w->w_gate, w->w_up, w->w_down};
  for (const void* p : req) {
    if (p == nullptr) return fail(MOE_ERR_INVALID_ARG, "expert weight is NULL");
    if (!aligned16(p)) return fail(MOE_ERR_INVALID_ARG, "expert weight not 16-byte aligned");
  }
  if (c.n_shared > 0) {
    const void* sh[3] = {w->ws_gate, w->ws_up, w->ws_down};
    for (const void* p : sh) {
      if (p == nullptr) return fail(MOE_ERR_INVALID_ARG, "shared expert weight is NULL");
      if (!aligned16(p)) return fail(MOE_ERR_INVALID_ARG, "shared weight not 16-byte aligned");
    }
  }
  if (c.weight_format == MOE_WEIGHTS_FP8_E4M3) {
    if (w->w_gate_scale == nullptr || w->w_up_scale == nullptr || w->w_down_scale == nullptr)
      return fail(MOE_ERR_INVALID_ARG, "FP8 expert weight scale is NULL");
    if (c.n_shared > 0 &&
        (w->ws_gate_scale == nullptr || w->ws_up_scale == nullptr || w->ws_down_scale == nullptr))
      return fail(MOE_ERR_INVALID_ARG, "FP8 shared expert weight scale is NULL");
  }
  return MOE_OK;
}

moe_status check_workspace(const Plan& p, const void* ws, size_t ws_bytes) {
  if (ws == nullptr) return fail(MOE_ERR_WORKSPACE, "workspace is NULL");
  if ((reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0)
    return fail(MOE_ERR_WORKSPACE, "workspace not 256-byte aligned");
  if (ws_bytes < p.total) return fail(MOE_ERR_WORKSPACE, "workspace smaller than moe_workspace_size");
  return MOE_OK;
}

void mark(void* const* ev, int i, hipStream_t s) {
  if (ev != nullptr && ev[i] != nullptr) (void)hipEventRecord(static_cast<hipEvent_t>(ev[i]), s);
}

// Shared by moe_route and moe_layer_forward: route + block statistics + scan.
moe_status run_route(const moe_config& c, const Plan& p, const Workspace& ws, const void* x,
                     const moe_weights& w, moe_routing* out, int32_t* idx, float* gate,
                     hipStream_t s) {
  hipError_t err = launch_route(c.dtype, x, w.w_router, w.logit_bias, w.select_bias, c.T,
                                c.d_model, c.n_experts, c.top_k, p.ksplit, p.rdense > 0,
                                ws.route_partial,
                                out ? out->logits : nullptr, idx, gate, ws.lrank, ws.blk_counts,
                                ws.blk_psum, s);
  if (err != hipSuccess) return hip_fail(err, "route kernel");
  return MOE_OK;
}

ItemSpec item_spec(const Plan& p, const Workspace& ws) {
  return ItemSpec{p.nnt_up, p.nnt_down, p.cus / 8 > 0 ? p.cus / 8 : 1,
                  p.nnt_up ? ws.items_up : nullptr, p.nnt_down ? ws.items_down : nullptr,
                  (p.nnt_up || p.nnt_down) ? ws.tbases : nullptr, p.narrow_up, p.narrow_down};
}

// sc.sorted_tok != nullptr: the scan kernel also writes the permutation.
moe_status run_scan(const moe_config& c, const Plan& p, const Workspace& ws, moe_routing* out,
                    const ScatterSpec& sc, hipStream_t s) {
  hipError_t err = launch_scan(ws.blk_counts, ws.blk_psum, c.T, c.n_experts, c.top_k, c.n_shared,
                               c.capacity, p.bm_up, p.cap_up, p.bm_down, p.cap_down, p.split,
                               item_spec(p, ws), sc,
                               out ? BalanceSpec{out->f, out->P, out->aux, out->balance_alpha}
                                   : BalanceSpec{nullptr, nullptr, nullptr, 0.f},
                               ws.blk_base,
                               ws.counts,
                               ws.prob_sum, out ? out->counts : nullptr,
                               out ? out->prob_sum : nullptr, ws.offsets, ws.tiles_up,
                               ws.tiles_down, ws.ntiles, s);
  if (err != hipSuccess) return hip_fail(err, "scan kernel");
  return MOE_OK;
}

// Offsets, tile lists, the permutation (sorted_tok, inv_row) and the
// large-tile GEMMs' work items, from the routing in idx and the block sums.
moe_status run_permute(const moe_config& c, const Plan& p, const Workspace& ws, moe_routing* out,
                       const int32_t* idx, hipStream_t s) {
  moe_status st;
  const long n_rows = static_cast<long>(c.T) * (c.top_k + c.n_shared);
  hipError_t err = hipSuccess;
  if (n_rows <= kScanScatterMaxRows) {  // one launch for scan and permutation
    if ((st = run_scan(c, p, ws, out, ScatterSpec{idx, ws.lrank, ws.sorted_tok, ws.inv_row}, s)) !=
        MOE_OK)
      return st;
  } else {
    if ((st = run_scan(c, p, ws, out, ScatterSpec{}, s)) != MOE_OK) return st;
    err = launch_scatter(idx, ws.lrank, ws.blk_base, ws.offsets, c.T, c.n_experts, c.top_k,
                         c.n_shared, c.capacity, ws.sorted_tok, ws.inv_row, s);
    if (err != hipSuccess) return hip_fail(err, "scatter kernel");
  }
  const long max_items = std::max(static_cast<long>(p.cap_up) * p.nnt_up,
                                  static_cast<long>(p.cap_down) * p.nnt_down);
  if ((err = launch_items(item_spec(p, ws), c.n_experts + c.n_shared, max_items, s)) != hipSuccess)
    return hip_fail(err, "items kernel");
  return MOE_OK;
}

// ---------------------------------------------------------------- backward
// Workspace of moe_layer_backward: the regions of make_plan(c, true) (routing,
// scan, tile lists), then the backward's own.
enum {
  B_LOGITS, B_G, B_U, B_D, B_H, B_DAB, B_DXP, B_RGATE, B_DG, B_DR, B_DR32, B_DXR, B_WDT,
  B_WDT_S, B_WCAT, B_WCAT_S, B_WRT, B_KBASE, B_DOT, B_HT, B_DABT, B_XT, B_XTF, B_DRT, B_COUNT
};

struct BwdPlan {
  Plan p;
  size_t off[B_COUNT];
  size_t total;
  long rows;  // T (k + S): every permuted row the forward may have
  long kseg;  // columns of the transposed segments: their rows rounded up to kalign, summed over groups, in a multiple of 128
  int kalign;  // 64 when the large-tile kernel takes the three segment products (bf16), else 128
  int Kr;     // N rounded up to 128
  int Tp;     // T rounded up to 128
  // D = dy W_down and dXp = [dA dB] [W_gate; W_up] read the weights as
  // K-rows on the large-tile kernels (bf16), else run on transposed copies
  // (W_down -> [N, F, d], [W_gate | W_up] -> [N, d, 2F]) that the workspace
  // then holds.  On 256-row tiles the K-row reads run as fast as the
  // transposed operands (Mixtral-shaped backward: grad_h 1.03, grad_x 1.92
  // ms either way), so the transposes' 1.2 ms go (step 9.0 -> 7.9 ms;
  // Qwen3-shaped 17.3 -> 15.3 ms); 128-row tiles only arise with few rows
  // per expert, where the transposes cost more than the slower K-row reads.
  bool bt_h, bt_x;
};

BwdPlan make_bwd_plan(const moe_config& c) {
  BwdPlan b{};
  b.p = make_plan(c, true);
  const size_t T = c.T, d = c.d_model, F = c.d_ff, N = c.n_experts, S = c.n_shared;
  const size_t G = N + S;
  const size_t eb = c.dtype == MOE_BF16 ? 2 : 4;
  b.rows = static_cast<long>(T) * (c.top_k + c.n_shared);
  // the weight-gradient GEMMs reduce over segments of a multiple of kalign
  // elements (launch_kbase) and over Kr and Tp, multiples of 128; rows of
  // the segment buffers are a multiple of 128 elements long.  64 only where
  // all three segment products run on the large-tile kernel's K-major mode:
  // kgemm_kernel takes its K steps in pairs of 128 bytes
  const long ks128 = (b.rows + 127 * static_cast<long>(G) + 127) / 128 * 128;
  const long dl = static_cast<long>(d), Fl = static_cast<long>(F);
  b.kalign = c.dtype == MOE_BF16 && kmajor_gemm_fits(dl, Fl, ks128) &&
                     kmajor_gemm_fits(Fl, dl, ks128)
                 ? 64
                 : 128;
  b.kseg = b.kalign == 64 ? (b.rows + 63 * static_cast<long>(G) + 127) / 128 * 128 : ks128;
  b.Kr = static_cast<int>((N + 127) / 128 * 128);
  b.Tp = static_cast<int>((T + 127) / 128 * 128);
  const size_t rows = b.rows, ks = b.kseg, Kr = b.Kr, Tp = b.Tp;
  const bool bf = c.dtype == MOE_BF16;
  b.bt_h = bf && b.p.up.variant == 1 &&
           expert_gemm_bt_fits(b.p.up.bm, c.d_model, c.d_ff, c.d_model, c.T);
  b.bt_x = bf && b.p.down.variant == 1 &&
           expert_gemm_bt_fits(b.p.down.bm, 2 * c.d_ff, c.d_model, c.d_ff, b.rows);
  size_t sz[B_COUNT];
  sz[B_LOGITS] = T * N * 4;
  sz[B_G] = sz[B_U] = sz[B_D] = sz[B_H] = rows * F * eb;
  sz[B_DAB] = rows * 2 * F * eb;
  sz[B_DXP] = rows * d * eb;
  sz[B_RGATE] = sz[B_DG] = rows * 4;
  sz[B_DR] = T * Kr * eb;
  sz[B_DR32] = T * N * 4;
  sz[B_DXR] = T * d * 4;
  sz[B_WDT] = b.bt_h ? 0 : N * F * d * eb;
  sz[B_WDT_S] = b.bt_h ? 0 : S * F * d * eb;
  sz[B_WCAT] = b.bt_x ? 0 : N * d * 2 * F * eb;
  sz[B_WCAT_S] = b.bt_x ? 0 : S * d * 2 * F * eb;
  sz[B_WRT] = d * Kr * eb;
  sz[B_KBASE] = (G + 1) * 4;
  sz[B_DOT] = d * ks * eb;
  sz[B_HT] = F * ks * eb;
  sz[B_DABT] = 2 * F * ks * eb;
  sz[B_XT] = d * ks * eb;
  sz[B_XTF] = d * Tp * eb;
  sz[B_DRT] = Kr * Tp * eb;
  size_t o = b.p.total;
  for (int i = 0; i < B_COUNT; ++i) {
    b.off[i] = o;
    o += align_up(sz[i] ? sz[i] : 1);
  }
  b.total = o;
  return b;
}

// One plain (no SiLU) grouped pass of the forward's GEMMs over the permuted
// rows: out[row] = A[row or gather[row]] W_e^T with W_e [n_dim, k_dim].
GemmArgs plain_pass(const moe_config& c, const Plan& p, const Workspace& ws, bool up_list,
                    const void* a, const int32_t* gather, int a_rows, const void* w0,
                    const void* ws0, int k_dim, int n_dim, void* out) {
  GemmArgs g{};
  g.a = a;
  g.gather = gather;
  g.w0 = w0;
  g.ws0 = ws0;
  g.offsets = ws.offsets;
  g.tiles = up_list ? ws.tiles_up : ws.tiles_down;
  g.ntiles = up_list ? ws.ntiles : ws.ntiles + 1;
  g.out = out;
  g.a_rows = a_rows;
  g.n_experts = c.n_experts;
  g.k_dim = k_dim;
  g.n_dim = n_dim;
  g.tiles_cap = up_list ? p.cap_up : p.cap_down;
  g.ksplit = 1;
  g.out_part = nullptr;
  g.plan = nullptr;
  g.items = up_list ? ws.items_up : ws.items_down;
  g.cus = p.cus;
  return g;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

size_t moe_workspace_size(const moe_config* cfg) {
  if (check_config(cfg) != MOE_OK) return 0;
  return make_plan(*cfg).total;
}

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: invalid argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: size outside the supported range";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: HIP runtime or launch failure";
    default: return "unknown moe_status";
  }
}

const char* moe_last_error(void) { return g_last_error; }

moe_status moe_forward_plan(const moe_config* cfg, moe_plan_info* out) {
  g_last_error[0] = '\0';
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (out == nullptr) return fail(MOE_ERR_INVALID_ARG, "out is NULL");
  const Plan p = make_plan(*cfg);
  out->up_kernel = p.up.variant;
  out->up_tile_rows = p.up.bm;
  out->down_kernel = p.down.variant;
  out->down_tile_rows = p.down.bm;
  out->route_split = p.ksplit;
  out->route_kernel = p.rdense > 0 ? 1 : 0;
  out->down_split = p.dsplit;
  out->tail_split_cols = p.split.tail_nnt;
  out->up_narrow_tails = p.narrow_up;
  out->down_narrow_tails = p.narrow_down;
  out->compute_units = p.cus;
  out->all_token_pass = p.all_tok ? 1 : 0;
  out->split_plan_offset = p.off[R_NT] + 2 * sizeof(int32_t);
  out->workspace_bytes = p.total;
  return MOE_OK;
}

moe_status moe_route(const moe_config* cfg, const void* x, const moe_weights* w,
                     moe_routing* out, void* workspace, size_t ws_bytes, void* stream) {
  g_last_error[0] = '\0';
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  const moe_config& c = *cfg;
  if ((st = check_weights(c, w, false)) != MOE_OK) return st;
  if (out == nullptr || out->topk_idx == nullptr || out->topk_gate == nullptr)
    return fail(MOE_ERR_INVALID_ARG, "moe_route needs out->topk_idx and out->topk_gate");
  if (c.T == 0) return MOE_OK;
  if (x == nullptr) return fail(MOE_ERR_INVALID_ARG, "x is NULL");
  if (!aligned16(x)) return fail(MOE_ERR_INVALID_ARG, "x not 16-byte aligned");
  const Plan p = make_plan(c);
  if ((st = check_workspace(p, workspace, ws_bytes)) != MOE_OK) return st;
  const Workspace ws = carve(p, workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = run_route(c, p, ws, x, *w, out, out->topk_idx, out->topk_gate, s)) != MOE_OK) return st;
  if (out->counts != nullptr || out->prob_sum != nullptr || out->f != nullptr ||
      out->P != nullptr || out->aux != nullptr) {
    if ((st = run_scan(c, p, ws, out, ScatterSpec{}, s)) != MOE_OK) return st;
  }
  return MOE_OK;
}

moe_status moe_layer_forward_timed(const moe_config* cfg, const void* x, const moe_weights* w,
                                   void* y, moe_routing* out, void* workspace, size_t ws_bytes,
                                   void* stream, void* const* ev) {
  g_last_error[0] = '\0';
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  const moe_config& c = *cfg;
  if ((st = check_weights(c, w, true)) != MOE_OK) return st;
  if (c.T == 0) return MOE_OK;
  if (x == nullptr || y == nullptr) return fail(MOE_ERR_INVALID_ARG, "x or y is NULL");
  if (!aligned16(x) || !aligned16(y)) return fail(MOE_ERR_INVALID_ARG, "x or y not 16-byte aligned");
  const Plan p = make_plan(c);
  if ((st = check_workspace(p, workspace, ws_bytes)) != MOE_OK) return st;
  const Workspace ws = carve(p, workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);

  int32_t* idx = (out && out->topk_idx) ? out->topk_idx : ws.topk_idx;
  float* gate = (out && out->topk_gate) ? out->topk_gate : ws.topk_gate;

  // all-token pass: the routing runs in the gate/up launch (its two stages
  // are empty here)
  AllTokenRoute rt{};
  mark(ev, MOE_STAGE_ROUTE, s);
  if (!p.all_tok && (st = run_route(c, p, ws, x, *w, out, idx, gate, s)) != MOE_OK) return st;

  mark(ev, MOE_STAGE_PERMUTE, s);
  if (!p.all_tok && (st = run_permute(c, p, ws, out, idx, s)) != MOE_OK) return st;
  hipError_t err = hipSuccess;
  if (p.all_tok) {
    const int eb = c.dtype == MOE_BF16 ? 2 : 4;
    rt.a = RouteArgs{x, w->w_router, w->logit_bias, w->select_bias, c.T, c.d_model,
                     c.n_experts, c.top_k, 1, c.d_model * eb / kRowBytes, nullptr,
                     out ? out->logits : nullptr, idx, gate, ws.lrank, ws.blk_counts,
                     ws.blk_psum};
    rt.S = c.n_shared;
    rt.capacity = c.capacity;
    rt.down_parts = p.dsplit;
    rt.inv_row = ws.inv_row;
    rt.counts = ws.counts;
    rt.prob_sum = ws.prob_sum;
    rt.user_counts = out ? out->counts : nullptr;
    rt.user_prob_sum = out ? out->prob_sum : nullptr;
    rt.offsets = ws.offsets;
    rt.plan = ws.ntiles + 2;
    rt.f = out ? out->f : nullptr;
    rt.P = out ? out->P : nullptr;
    rt.aux = out ? out->aux : nullptr;
    rt.alpha = out ? out->balance_alpha : 0.f;
  }

  mark(ev, MOE_STAGE_EXPERT_UP, s);
  GemmArgs up{};
  up.a = x;
  up.gather = ws.sorted_tok;
  up.w0 = w->w_gate;
  up.w1 = w->w_up;
  up.ws0 = w->ws_gate;
  up.ws1 = w->ws_up;
  up.offsets = ws.offsets;
  up.tiles = ws.tiles_up;
  up.ntiles = ws.ntiles;
  up.out = ws.hidden;
  up.a_rows = c.T;
  up.n_experts = c.n_experts;
  up.k_dim = c.d_model;
  up.n_dim = c.d_ff;
  up.tiles_cap = p.cap_up;
  up.cus = p.cus;
  up.wfp8 = c.weight_format == MOE_WEIGHTS_FP8_E4M3;
  up.sc0 = w->w_gate_scale;
  up.sc1 = w->w_up_scale;
  up.ssc0 = w->ws_gate_scale;
  up.ssc1 = w->ws_up_scale;
  up.items = ws.items_up;
  if (p.nnt_up) {
    up.nitems = ws.tbases + tb_items_up(c.n_experts + c.n_shared) + c.n_experts + c.n_shared;
    up.narrow = p.narrow_up;
  }
  if (p.all_tok) {
    up.gather = nullptr;
    up.all_tok = c.T;
    up.all_groups = c.n_experts + c.n_shared;
  }
  if ((err = launch_gemm(c.dtype, true, p.up, up, s, p.all_tok ? &rt : nullptr)) != hipSuccess)
    return hip_fail(err, "gate/up GEMM");

  mark(ev, MOE_STAGE_EXPERT_DOWN, s);
  GemmArgs dn{};
  dn.a = ws.hidden;
  dn.gather = nullptr;
  dn.w0 = w->w_down;
  dn.ws0 = w->ws_down;
  dn.offsets = ws.offsets;
  dn.tiles = ws.tiles_down;
  dn.ntiles = ws.ntiles + 1;
  dn.out = ws.yperm;
  dn.a_rows = static_cast<int>(p.rows_g);
  dn.n_experts = c.n_experts;
  dn.k_dim = c.d_ff;
  dn.n_dim = c.d_model;
  dn.tiles_cap = p.cap_down;
  dn.ksplit = p.dsplit;
  dn.out_part = ws.ypart;
  dn.plan = ws.ntiles + 2;
  dn.cus = p.cus;
  dn.wfp8 = up.wfp8;
  dn.sc0 = w->w_down_scale;
  dn.ssc0 = w->ws_down_scale;
  dn.items = ws.items_down;
  if (p.nnt_down) {
    dn.nitems = ws.tbases + tb_items_down(c.n_experts + c.n_shared) + c.n_experts + c.n_shared;
    dn.narrow = p.narrow_down;
  }
  if (p.all_tok) {
    dn.all_tok = c.T;
    dn.all_groups = c.n_experts + c.n_shared;
  }
  if ((err = launch_gemm(c.dtype, false, p.down, dn, s)) != hipSuccess)
    return hip_fail(err, "down GEMM");

  mark(ev, MOE_STAGE_COMBINE, s);
  if ((err = launch_combine(c.dtype, ws.yperm, ws.ypart, ws.ntiles + 2, ws.inv_row, gate,
                            ws.offsets, c.n_experts, c.T, c.d_model, c.top_k, c.n_shared, y, s)) !=
      hipSuccess)
    return hip_fail(err, "combine kernel");
  mark(ev, MOE_STAGE_COUNT, s);
  return MOE_OK;
}

moe_status moe_layer_forward(const moe_config* cfg, const void* x, const moe_weights* w, void* y,
                             moe_routing* out, void* workspace, size_t ws_bytes, void* stream) {
  return moe_layer_forward_timed(cfg, x, w, y, out, workspace, ws_bytes, stream, nullptr);
}

moe_status moe_layer_forward_noalloc(const moe_config* cfg, const void* x, const moe_weights* w,
                                     void* y, moe_routing* out, void* stream) {
  g_last_error[0] = '\0';
  const moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  const size_t need = make_plan(*cfg).total;
  if (need > MOE_NOALLOC_SCRATCH_BYTES) {
    snprintf(g_last_error, sizeof(g_last_error),
             "the configuration needs %zu bytes of workspace; moe_layer_forward_noalloc holds "
             "%zu (MOE_NOALLOC_SCRATCH_BYTES)",
             need, static_cast<size_t>(MOE_NOALLOC_SCRATCH_BYTES));
    return MOE_ERR_WORKSPACE;
  }
  void* ws = nullptr;
  const moe_status sa = scratch_address(&ws);
  if (sa != MOE_OK) return sa;
  return moe_layer_forward_timed(cfg, x, w, y, out, ws, MOE_NOALLOC_SCRATCH_BYTES, stream,
                                 nullptr);
}

moe_status moe_balance_stats(int32_t T, int32_t N, int32_t k, const int32_t* counts,
                             const float* prob_sum, float alpha, float* f_out, float* P_out,
                             float* aux_out, void* stream) {
  g_last_error[0] = '\0';
  if (T < 0 || N <= 0 || k <= 0 || k > N) return fail(MOE_ERR_INVALID_ARG, "bad T, N or k");
  if (N > kMaxExperts) return fail(MOE_ERR_UNSUPPORTED, "n_experts > 512");
  if (counts == nullptr || prob_sum == nullptr || f_out == nullptr || P_out == nullptr ||
      aux_out == nullptr)
    return fail(MOE_ERR_INVALID_ARG, "NULL pointer");
  hipError_t err = launch_balance(T, N, k, counts, prob_sum, alpha, f_out, P_out, aux_out,
                                  static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return hip_fail(err, "balance kernel");
  return MOE_OK;
}

size_t moe_backward_workspace_size(const moe_config* cfg) {
  if (check_config(cfg) != MOE_OK) return 0;
  return make_bwd_plan(*cfg).total;
}

moe_status moe_layer_backward_timed(const moe_config* cfg, const void* x, const moe_weights* w,
                                    const void* dy, float alpha, float aux_grad, moe_grads* gr,
                                    void* workspace, size_t ws_bytes, void* stream,
                                    void* const* ev) {
  g_last_error[0] = '\0';
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  const moe_config& c = *cfg;
  if (c.weight_format != MOE_WEIGHTS_DTYPE)
    return fail(MOE_ERR_UNSUPPORTED, "the backward needs expert weights in dtype");
  if ((st = check_weights(c, w, true)) != MOE_OK) return st;
  if (gr == nullptr) return fail(MOE_ERR_INVALID_ARG, "grads is NULL");
  {
    const void* req[5] = {c.T > 0 ? gr->dx : gr->dw_router, gr->dw_router, gr->dw_gate,
                          gr->dw_up, gr->dw_down};
    for (const void* q : req) {
      if (q == nullptr) return fail(MOE_ERR_INVALID_ARG, "required gradient is NULL");
      if (!aligned16(q)) return fail(MOE_ERR_INVALID_ARG, "gradient not 16-byte aligned");
    }
    if (c.n_shared > 0) {
      const void* sh[3] = {gr->dws_gate, gr->dws_up, gr->dws_down};
      for (const void* q : sh) {
        if (q == nullptr) return fail(MOE_ERR_INVALID_ARG, "shared expert gradient is NULL");
        if (!aligned16(q)) return fail(MOE_ERR_INVALID_ARG, "gradient not 16-byte aligned");
      }
    }
  }
  if (c.T > 0) {
    if (x == nullptr || dy == nullptr) return fail(MOE_ERR_INVALID_ARG, "x or dy is NULL");
    if (!aligned16(x) || !aligned16(dy))
      return fail(MOE_ERR_INVALID_ARG, "x or dy not 16-byte aligned");
  }
  const BwdPlan b = make_bwd_plan(c);
  const Plan& p = b.p;
  if ((st = check_workspace(p, workspace, ws_bytes)) != MOE_OK) return st;
  if (ws_bytes < b.total)
    return fail(MOE_ERR_WORKSPACE, "workspace smaller than moe_backward_workspace_size");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int dt = c.dtype, T = c.T, d = c.d_model, F = c.d_ff, N = c.n_experts, k = c.top_k,
            S = c.n_shared, G = N + S;
  const size_t eb = dt == MOE_BF16 ? 2 : 4;
  hipError_t err = hipSuccess;
  if (T == 0) {  // no rows: every weight gradient is zero
    if ((err = launch_kgemm(dt, false, nullptr, 0, nullptr, 0, d, F, G, nullptr, 0, gr->dw_down,
                            gr->dws_down, N, s)) != hipSuccess ||
        (err = launch_kgemm(dt, false, nullptr, 0, nullptr, 0, F, d, G, nullptr, 0, gr->dw_gate,
                            gr->dws_gate, N, s)) != hipSuccess ||
        (err = launch_kgemm(dt, false, nullptr, 0, nullptr, 0, F, d, G, nullptr, 0, gr->dw_up,
                            gr->dws_up, N, s)) != hipSuccess ||
        (err = launch_kgemm(dt, false, nullptr, 0, nullptr, 0, N, d, 1, nullptr, 0,
                            gr->dw_router, nullptr, 1, s)) != hipSuccess)
      return hip_fail(err, "zero gradients");
    if (gr->dlogit_bias != nullptr &&
        (err = launch_colsum(nullptr, 0, N, gr->dlogit_bias, s)) != hipSuccess)
      return hip_fail(err, "zero gradients");
    return MOE_OK;
  }
  const Workspace ws = carve(p, workspace);
  char* base = static_cast<char*>(workspace);
  auto at = [&](int r) { return static_cast<void*>(base + b.off[r]); };
  float* logits = static_cast<float*>(at(B_LOGITS));
  float* rgate = static_cast<float*>(at(B_RGATE));
  float* dg_row = static_cast<float*>(at(B_DG));
  float* dr32 = static_cast<float*>(at(B_DR32));
  float* dxr = static_cast<float*>(at(B_DXR));
  int32_t* kbase = static_cast<int32_t*>(at(B_KBASE));
  const int rows = static_cast<int>(b.rows);

  // routing and grouping, as in the forward
  mark(ev, MOE_BSTAGE_ROUTE, s);
  err = launch_route(dt, x, w->w_router, w->logit_bias, w->select_bias, T, d, N, k, p.ksplit,
                     p.rdense > 0, ws.route_partial, logits, ws.topk_idx, ws.topk_gate, ws.lrank, ws.blk_counts,
                     ws.blk_psum, s);
  if (err != hipSuccess) return hip_fail(err, "route kernel");
  if ((st = run_permute(c, p, ws, nullptr, ws.topk_idx, s)) != MOE_OK) return st;

  // expert weights as K-rows or transposed (BwdPlan); W_r -> [d, Kr] always
  const bool bt_h = b.bt_h, bt_x = b.bt_x;
  mark(ev, MOE_BSTAGE_TRANSPOSE_W, s);
  const long fd = static_cast<long>(F) * d;
  if ((!bt_h &&
       (err = launch_transpose(dt, w->w_down, d, F, fd, at(B_WDT), d, 0, d, fd, N, s)) !=
           hipSuccess) ||
      (!bt_x &&
       ((err = launch_transpose(dt, w->w_gate, F, d, fd, at(B_WCAT), 2 * F, 0, F, 2 * fd, N, s)) !=
            hipSuccess ||
        (err = launch_transpose(dt, w->w_up, F, d, fd, at(B_WCAT), 2 * F, F, F, 2 * fd, N, s)) !=
            hipSuccess)) ||
      (err = launch_transpose(dt, w->w_router, N, d, 0, at(B_WRT), b.Kr, 0, b.Kr, 0, 1, s)) !=
          hipSuccess)
    return hip_fail(err, "weight transpose");
  if (S > 0 &&
      ((!bt_h &&
        (err = launch_transpose(dt, w->ws_down, d, F, fd, at(B_WDT_S), d, 0, d, fd, S, s)) !=
            hipSuccess) ||
       (!bt_x &&
        ((err = launch_transpose(dt, w->ws_gate, F, d, fd, at(B_WCAT_S), 2 * F, 0, F, 2 * fd, S,
                                 s)) != hipSuccess ||
         (err = launch_transpose(dt, w->ws_up, F, d, fd, at(B_WCAT_S), 2 * F, F, F, 2 * fd, S,
                                 s)) != hipSuccess))))
    return hip_fail(err, "weight transpose");

  // G, U (recomputed) and D = dy W_down, all [rows, F]
  mark(ev, MOE_BSTAGE_RECOMPUTE, s);
  GemmArgs ga = plain_pass(c, p, ws, true, x, ws.sorted_tok, T, w->w_gate, w->ws_gate, d, F, at(B_G));
  if ((err = launch_gemm(dt, false, p.up, ga, s)) != hipSuccess) return hip_fail(err, "G GEMM");
  ga = plain_pass(c, p, ws, true, x, ws.sorted_tok, T, w->w_up, w->ws_up, d, F, at(B_U));
  if ((err = launch_gemm(dt, false, p.up, ga, s)) != hipSuccess) return hip_fail(err, "U GEMM");
  mark(ev, MOE_BSTAGE_GRAD_H, s);
  if (bt_h) {
    ga = plain_pass(c, p, ws, true, dy, ws.sorted_tok, T, w->w_down, w->ws_down, d, F, at(B_D));
    ga.bt_rows0 = d;
    err = launch_expert_gemm_bt(p.up.bm, ga, s);
  } else {
    ga = plain_pass(c, p, ws, true, dy, ws.sorted_tok, T, at(B_WDT),
                    S > 0 ? at(B_WDT_S) : nullptr, d, F, at(B_D));
    err = launch_gemm(dt, false, p.up, ga, s);
  }
  if (err != hipSuccess) return hip_fail(err, "D GEMM");

  // gates per row, SwiGLU backward, then dXp = [dA dB] [W_gate; W_up]
  if ((err = launch_row_gate(ws.inv_row, ws.topk_gate, ws.offsets, T, k, N, S, rgate, s)) !=
          hipSuccess ||
      (err = launch_swiglu_bwd(dt, at(B_G), at(B_U), at(B_D), rgate, ws.offsets, G, F, rows,
                               at(B_H), at(B_DAB), dg_row, s)) != hipSuccess)
    return hip_fail(err, "SwiGLU backward");
  mark(ev, MOE_BSTAGE_GRAD_X, s);
  if (bt_x) {
    ga = plain_pass(c, p, ws, false, at(B_DAB), nullptr, rows, w->w_gate, w->ws_gate, 2 * F, d,
                    at(B_DXP));
    ga.w1 = w->w_up;
    ga.ws1 = w->ws_up;
    ga.bt_rows0 = F;
    err = launch_expert_gemm_bt(p.down.bm, ga, s);
  } else {
    ga = plain_pass(c, p, ws, false, at(B_DAB), nullptr, rows, at(B_WCAT),
                    S > 0 ? at(B_WCAT_S) : nullptr, 2 * F, d, at(B_DXP));
    err = launch_gemm(dt, false, p.down, ga, s);
  }
  if (err != hipSuccess) return hip_fail(err, "dX GEMM");

  // router: dr, d logit_bias, dx = dr W_r + the rows' dXp
  if ((err = launch_router_bwd(dt, logits, ws.topk_idx, ws.topk_gate, ws.inv_row, dg_row,
                               ws.counts, T, N, k, alpha, aux_grad, b.Kr, at(B_DR), dr32, s)) !=
      hipSuccess)
    return hip_fail(err, "router backward");
  if (gr->dlogit_bias != nullptr &&
      (err = launch_colsum(dr32, T, N, gr->dlogit_bias, s)) != hipSuccess)
    return hip_fail(err, "logit-bias gradient");
  if ((err = launch_kgemm(dt, true, at(B_DR), b.Kr, at(B_WRT), b.Kr, T, d, 1, nullptr, b.Kr, dxr,
                          nullptr, 1, s)) != hipSuccess ||
      (err = launch_dx_combine(dt, at(B_DXP), dxr, ws.inv_row, ws.offsets, T, N, k, S, d, gr->dx,
                               s)) != hipSuccess)
    return hip_fail(err, "dx");

  // weight gradients over each group's rows
  mark(ev, MOE_BSTAGE_SEGMENTS, s);
  const long ks = b.kseg;
  if ((err = launch_kbase(ws.offsets, G, b.kalign, kbase, s)) != hipSuccess ||
      (err = launch_segment_transpose(dt, dy, d, T, ws.sorted_tok, rgate, ws.offsets, kbase, G, ks,
                                      at(B_DOT), ks, s)) != hipSuccess ||
      (err = launch_segment_transpose(dt, at(B_H), F, rows, nullptr, nullptr, ws.offsets, kbase, G,
                                      ks, at(B_HT), ks, s)) != hipSuccess ||
      (err = launch_segment_transpose(dt, at(B_DAB), 2 * F, rows, nullptr, nullptr, ws.offsets,
                                      kbase, G, ks, at(B_DABT), ks, s)) != hipSuccess ||
      (err = launch_segment_transpose(dt, x, d, T, ws.sorted_tok, nullptr, ws.offsets, kbase, G, ks,
                                      at(B_XT), ks, s)) != hipSuccess)
    return hip_fail(err, "segment transpose");
  const char* dabt = static_cast<const char*>(at(B_DABT));
  mark(ev, MOE_BSTAGE_GRAD_W, s);
  if ((err = launch_kgemm(dt, false, at(B_DOT), ks, at(B_HT), ks, d, F, G, kbase, 0, gr->dw_down,
                          gr->dws_down, N, s)) != hipSuccess ||
      (err = launch_kgemm(dt, false, dabt, ks, at(B_XT), ks, F, d, G, kbase, 0, gr->dw_gate,
                          gr->dws_gate, N, s)) != hipSuccess ||
      (err = launch_kgemm(dt, false, dabt + static_cast<size_t>(F) * ks * eb, ks, at(B_XT), ks, F,
                          d, G, kbase, 0, gr->dw_up, gr->dws_up, N, s)) != hipSuccess)
    return hip_fail(err, "expert weight gradients");
  mark(ev, MOE_BSTAGE_GRAD_WR, s);
  if ((err = launch_transpose(dt, x, T, d, 0, at(B_XTF), b.Tp, 0, b.Tp, 0, 1, s)) != hipSuccess ||
      (err = launch_transpose(dt, at(B_DR), T, b.Kr, 0, at(B_DRT), b.Tp, 0, b.Tp, 0, 1, s)) !=
          hipSuccess ||
      (err = launch_kgemm(dt, false, at(B_DRT), b.Tp, at(B_XTF), b.Tp, N, d, 1, nullptr, b.Tp,
                          gr->dw_router, nullptr, 1, s)) != hipSuccess)
    return hip_fail(err, "router weight gradient");
  mark(ev, MOE_BSTAGE_COUNT, s);
  return MOE_OK;
}

moe_status moe_layer_backward(const moe_config* cfg, const void* x, const moe_weights* w,
                              const void* dy, float alpha, float aux_grad, moe_grads* gr,
                              void* workspace, size_t ws_bytes, void* stream) {
  return moe_layer_backward_timed(cfg, x, w, dy, alpha, aux_grad, gr, workspace, ws_bytes, stream,
                                  nullptr);
}

moe_status moe_update_select_bias(int32_t N, const int32_t* counts, float rate,
                                  float* select_bias, void* stream) {
  g_last_error[0] = '\0';
  if (N <= 0) return fail(MOE_ERR_INVALID_ARG, "N must be positive");
  if (N > kMaxExperts) return fail(MOE_ERR_UNSUPPORTED, "n_experts > 512");
  if (counts == nullptr || select_bias == nullptr) return fail(MOE_ERR_INVALID_ARG, "NULL pointer");
  hipError_t err = launch_bias_update(counts, N, rate, select_bias, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return hip_fail(err, "bias update kernel");
  return MOE_OK;
}

}  // extern "C"
