// Grouping of the routed tokens by expert.
//
// The pages' layer runs each expert only on the tokens that chose it
// ("Mixture of experts and speculative decoding", "A toy MoE layer in
// PyTorch": an expert that no token picked does no work; "Mixture of Experts
// and Guided Decoding", sparse-MoE passage: each expert sees the tokens whose
// top-k contains it).  Instead of one masked pass per expert, the
// assignments are laid out once in expert-major order:
//
//   counts[e]            = total assignments to e (sum of the block counts)
//   offsets[e]           = exclusive prefix sum of counts (shared expert s
//                          follows the routed ones with T rows)
//   row(t, slot)         = offsets[e] + (assignments to e in earlier blocks)
//                          + (rank of t among the block's tokens that chose e)
//   sorted_tok[row]      = t,  inv_row[t, slot] = row
//
// so each expert's rows are contiguous and ordered by token.  The scan kernel
// also writes the tile lists of the two grouped GEMMs (one entry per BM-row
// tile of each non-empty expert), so tile scheduling needs no host round trip.
#include "balance.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kScanThreads = 1024;

// Exclusive prefix sum over v (one value per thread of a 1024-thread block);
// returns the exclusive sum for this thread and the block total in *total.
__device__ int block_exclusive_scan(int v, int* s_tmp, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) s_tmp[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    int w = lane < (kScanThreads / 64) ? s_tmp[lane] : 0;
    int wi = w;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int o = __shfl_up(wi, off, 64);
      if (lane >= off) wi += o;
    }
    if (lane < kScanThreads / 64) s_tmp[16 + lane] = wi - w;  // exclusive per wave
    if (lane == kScanThreads / 64 - 1) s_tmp[32] = wi;
  }
  __syncthreads();
  const int res = s_tmp[16 + wave] + incl - v;
  *total = s_tmp[32];
  __syncthreads();
  return res;
}

// Row i of the permutation: (token, slot) pairs first, then the shared
// experts' rows.
// An assignment whose rank (in token order) within its expert is capacity or
// more (capacity > 0) is dropped: inv_row = -1 and no row.  Shared expert s
// owns rows offsets[N + s] + t.
__device__ __forceinline__ void scatter_row(long i, const int32_t* __restrict__ topk_idx,
                                            const int32_t* __restrict__ lrank,
                                            const int32_t* __restrict__ blk_base,
                                            const int32_t* __restrict__ offsets, int n_tok, int N,
                                            int k, int S, int capacity,
                                            int32_t* __restrict__ sorted_tok,
                                            int32_t* __restrict__ inv_row) {
  const long tk = static_cast<long>(n_tok) * k;
  if (i < tk) {
    const int t = static_cast<int>(i / k);
    const int e = topk_idx[i];
    const int b = t / kRouteTokens;
    const int rank = blk_base[static_cast<size_t>(b) * N + e] + lrank[i];
    if (capacity > 0 && rank >= capacity) {
      inv_row[i] = -1;
      return;
    }
    const int row = offsets[e] + rank;
    // a row outside the expert's segment would mean inconsistent routing
    // outputs; keep every write in bounds regardless
    const bool ok = row >= offsets[e] && row < offsets[e + 1];
    if (ok) sorted_tok[row] = t;
    inv_row[i] = ok ? row : offsets[e];
  } else if (i < tk + static_cast<long>(S) * n_tok) {
    const long j = i - tk;
    const int s = static_cast<int>(j / n_tok), t = static_cast<int>(j - static_cast<long>(s) * n_tok);
    sorted_tok[offsets[N + s] + t] = t;
  }
}

// Items of one row group: its row tiles below tlimit x nnt column tiles, but
// a narrow last tile (ItemSpec) counts nnt / 2 items of two columns each.
__device__ __forceinline__ int group_items(int tbase, int tiles, int tlimit, int rows, int bm,
                                           int nnt, int narrow) {
  const int T = min(tbase + tiles, tlimit) - tbase;
  if (T <= 0) return 0;
  const bool nb = narrow && nnt >= 2 && nnt % 2 == 0 && tbase + tiles <= tlimit &&
                  rows - (tiles - 1) * bm <= kNarrowRows;
  return T * nnt - (nb ? nnt / 2 : 0);
}

// Item i of a large-tile GEMM's list (nnt column tiles, row tiles [0,
// tlimit)): per row group (tile range [tb[g], tb[g + 1]), items from ib[g])
// blocks of up to 8 row tiles x (window / row tiles) column tiles, column by
// column.  A group whose item count is short of tiles x nnt ends with a
// narrow tile: its last block then goes by pairs of columns, the block's
// full tiles on the first column, on the second, then the narrow item of
// both.  The group of item i is found by binary search over ib (ng + 1
// entries, non-decreasing).
__device__ void write_item(int32_t* __restrict__ items, int nnt, const int* tb, const int* ib,
                           int ng, int tlimit, int window, int i) {
  int lo = 0, hi = ng;  // largest g with ib[g] <= i
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (ib[mid] <= i) lo = mid;
    else hi = mid;
  }
  const int base = tb[lo];
  const int T = min(tb[lo + 1], tlimit) - base;
  const bool nb = ib[lo + 1] - ib[lo] != T * nnt;
  const int TW = min(T, 8), CW = max(1, window / TW);
  const int q = i - ib[lo];
  const int nblk = (T + TW - 1) / TW;
  const int b = min(q / (TW * nnt), nblk - 1);
  const int r = q - b * TW * nnt;
  const int tw = min(TW, T - b * TW);
  int t, c;
  if (nb && b == nblk - 1) {
    const int P = 2 * (tw - 1) + 1;  // items per pair of columns
    const int cp = r / P, s = r - cp * P;
    if (s < tw - 1) {
      t = s;
      c = 2 * cp;
    } else if (s < 2 * (tw - 1)) {
      t = s - (tw - 1);
      c = 2 * cp + 1;
    } else {
      t = tw - 1;
      c = 2 * cp;
    }
  } else {
    const int cbi = r / (tw * CW);
    const int r2 = r - cbi * tw * CW;
    c = cbi * CW + r2 / tw;
    t = r2 % tw;
  }
  items[i] = ((base + b * TW + t) << kItemColBits) | c;
}

// One thread per item; blockIdx.y: 0 = gate/up list, 1 = down list.
__global__ __launch_bounds__(256) void items_kernel(ItemSpec is, int ng) {
  __shared__ int s_tb[kMaxExperts + kMaxShared + 1];
  __shared__ int s_ib[kMaxExperts + kMaxShared + 1];
  const int pass = blockIdx.y;
  const int nnt = pass == 0 ? is.nnt_up : is.nnt_down;
  int32_t* items = pass == 0 ? is.items_up : is.items_down;
  if (nnt <= 0 || items == nullptr) return;
  const int32_t* tb = is.tbases + pass * (ng + 1);
  const int32_t* ib = is.tbases + (pass == 0 ? tb_items_up(ng) : tb_items_down(ng));
  for (int g = threadIdx.x; g <= ng; g += 256) {
    s_tb[g] = tb[g];
    s_ib[g] = ib[g];
  }
  const int tlimit = is.tbases[2 * (ng + 1) + pass];
  __syncthreads();
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < s_ib[ng]) write_item(items, nnt, s_tb, s_ib, ng, tlimit, is.window, i);
}

__global__ __launch_bounds__(kScanThreads) void scan_kernel(
    const int32_t* __restrict__ blk_counts, const float* __restrict__ blk_psum, int n_tok, int N,
    int k, int S, int capacity, int bm_up, int cap_up, int bm_down, int cap_down, SplitSpec split,
    ItemSpec ispec, ScatterSpec sc, BalanceSpec bal,
    int32_t* __restrict__ blk_base, int32_t* __restrict__ counts, float* __restrict__ prob_sum,
    int32_t* __restrict__ user_counts, float* __restrict__ user_prob_sum,
    int32_t* __restrict__ offsets, int2* __restrict__ tiles_up, int2* __restrict__ tiles_down,
    int32_t* __restrict__ ntiles) {
  __shared__ int s_cnt[kScanThreads];
  __shared__ float s_ps[kScanThreads];
  __shared__ int s_tmp[64];
  __shared__ int s_tot[kMaxExperts];
  __shared__ int s_nrm_down;  // down-pass tiles not split over the reduction
  __shared__ int s_tbu[kMaxExperts + kMaxShared + 1];  // first tile of each group
  __shared__ int s_tbd[kMaxExperts + kMaxShared + 1];

  const int tid = threadIdx.x;
  const int B = (n_tok + kRouteTokens - 1) / kRouteTokens;
  // threads per expert (N <= 512 -> up to 2 or more), no more than there are
  // blocks: their partial sums are added one after another below.  Lane l
  // of a wavefront takes expert (wave * 64 + l) mod N, so each load of a block
  // row is one contiguous read of consecutive experts.
  const int P = min(kScanThreads / N, B > 0 ? B : 1);
  const int e = tid % N, part = tid / N;
  const bool mine = part < P;
  const int slot = e * P + part;  // this thread's partial in s_cnt / s_ps
  const int b_lo = mine ? static_cast<int>((static_cast<long>(B) * part) / P) : 0;
  const int b_hi = mine ? static_cast<int>((static_cast<long>(B) * (part + 1)) / P) : 0;

  // partial column sums over this thread's range of blocks, 8 blocks' loads
  // requested before they are added (in block order), so a long range costs
  // a few round trips to L2 instead of one per block
  int c = 0;
  float ps = 0.f;
  for (int b0 = b_lo; b0 < b_hi; b0 += 8) {
    int cv[8];
    float pv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool in = b0 + u < b_hi;
      const size_t o = static_cast<size_t>(in ? b0 + u : b_lo) * N + e;
      cv[u] = in ? blk_counts[o] : 0;
      pv[u] = in ? blk_psum[o] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      c += cv[u];
      if (b0 + u < b_hi) ps += pv[u];
    }
  }
  if (mine) {
    s_cnt[slot] = c;
    s_ps[slot] = ps;
  }
  __syncthreads();
  if (mine && part == 0) {
    int run = 0;
    float pr = 0.f;
    for (int p = 0; p < P; ++p) {
      const int v = s_cnt[e * P + p];
      s_cnt[e * P + p] = run;
      run += v;
      pr += s_ps[e * P + p];
    }
    s_tot[e] = run;
    counts[e] = run;
    prob_sum[e] = pr;
    if (user_counts != nullptr) user_counts[e] = run;
    if (user_prob_sum != nullptr) user_prob_sum[e] = pr;
  }
  __syncthreads();
  if (mine) {
    int run = s_cnt[slot];
    for (int b0 = b_lo; b0 < b_hi; b0 += 8) {
      int cv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        cv[u] = b0 + u < b_hi ? blk_counts[static_cast<size_t>(b0 + u) * N + e] : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (b0 + u < b_hi) blk_base[static_cast<size_t>(b0 + u) * N + e] = run;
        run += cv[u];
      }
    }
  }
  __syncthreads();

  // offsets and tile lists over the N + S row groups
  const int NG = N + S;
  // rows per group: an expert's kept assignments, every token for a shared one
  int cg = 0;
  if (tid < N) cg = capacity > 0 ? min(s_tot[tid], capacity) : s_tot[tid];
  else if (tid < NG) cg = n_tok;
  if (tid < NG && tid >= N) counts[tid] = n_tok;
  int total_rows;
  const int off = block_exclusive_scan(cg, s_tmp, &total_rows);
  if (tid < NG) offsets[tid] = off;
  if (tid == 0) offsets[NG] = total_rows;

  const int tu = tid < NG ? (cg + bm_up - 1) / bm_up : 0;
  const int td = tid < NG ? (cg + bm_down - 1) / bm_down : 0;
  int total_up, total_down;
  const int base_up = block_exclusive_scan(tu, s_tmp, &total_up);
  const int base_down = block_exclusive_scan(td, s_tmp, &total_down);
  for (int i = 0; i < tu; ++i)
    if (base_up + i < cap_up) tiles_up[base_up + i] = make_int2(tid, i * bm_up);
  for (int i = 0; i < td; ++i)
    if (base_down + i < cap_down) tiles_down[base_down + i] = make_int2(tid, i * bm_down);
  if (tid == 0) {
    ntiles[0] = min(total_up, cap_up);
    ntiles[1] = min(total_down, cap_down);
  }
  __syncthreads();  // tiles_down and offsets are complete

  // Split plan of the down pass.  Tail split: with W = tiles x column tiles
  // workgroups on `cus` compute units, the last round holds r = W mod cus
  // of them.  When r is small, the last ceil(r / nnt) row tiles are instead
  // split over their reduction into `parts` pieces, so that round runs
  // parts times shorter.
  if (tid == 0) {
    int32_t* plan = ntiles + 2;
    const int ntd = min(total_down, cap_down);
    int parts = 0, row_split = total_rows, stride = 0, tail = 0;
    if (split.parts > 1) {
      parts = split.parts;
      row_split = 0;
      stride = n_tok * (k + S);  // the split GEMM's partial layout: every possible row
    } else if (split.tail_nnt > 0 && ntd > 0) {
      const long W = static_cast<long>(ntd) * split.tail_nnt;
      const long r = W % split.tail_cus;
      if (r > 0) {
        const int t = static_cast<int>((r + split.tail_nnt - 1) / split.tail_nnt);
        int sp = split.tail_cus / (t * split.tail_nnt);
        sp = min(sp, split.tail_max_parts);
        if (sp >= 2 && t < ntd && static_cast<long>(t) * bm_down * sp <= split.tail_cap_rows) {
          const int2 first = tiles_down[ntd - t];
          parts = sp;
          tail = t;
          row_split = offsets[first.x] + first.y;
          stride = t * bm_down;
        }
      }
    }
    plan[kPlanParts] = parts;
    plan[kPlanRowSplit] = row_split;
    plan[kPlanStride] = stride;
    plan[kPlanTailTiles] = tail;
    s_nrm_down = ntd - tail;
    s_tbu[NG] = total_up;
    s_tbd[NG] = total_down;
  }
  if (tid < NG) {
    s_tbu[tid] = base_up;
    s_tbd[tid] = base_down;
  }
  __syncthreads();
  // group tile bases and list lengths for the items kernel
  if (ispec.tbases != nullptr) {
    for (int g = tid; g <= NG; g += kScanThreads) {
      ispec.tbases[g] = s_tbu[g];
      ispec.tbases[NG + 1 + g] = s_tbd[g];
    }
    if (tid == 0) {
      ispec.tbases[2 * (NG + 1)] = min(total_up, cap_up);
      ispec.tbases[2 * (NG + 1) + 1] = s_nrm_down;
    }
    // item bases of both lists (a narrow last tile counts half its columns)
    int iu = 0, idn = 0;
    if (tid < NG) {
      iu = group_items(base_up, tu, min(total_up, cap_up), cg, bm_up, ispec.nnt_up,
                       ispec.narrow_up);
      idn = group_items(base_down, td, s_nrm_down, cg, bm_down, ispec.nnt_down,
                        ispec.narrow_down);
    }
    int tot_u, tot_d;
    const int ibu = block_exclusive_scan(iu, s_tmp, &tot_u);
    const int ibd = block_exclusive_scan(idn, s_tmp, &tot_d);
    if (tid < NG) {
      ispec.tbases[tb_items_up(NG) + tid] = ibu;
      ispec.tbases[tb_items_down(NG) + tid] = ibd;
    }
    if (tid == 0) {
      ispec.tbases[tb_items_up(NG) + NG] = tot_u;
      ispec.tbases[tb_items_down(NG) + NG] = tot_d;
    }
  }
  // small batches: the permutation too (offsets and block bases are complete
  // and visible to the workgroup since the barriers above)
  if (sc.sorted_tok != nullptr) {
    const long n = static_cast<long>(n_tok) * k + static_cast<long>(S) * n_tok;
    for (long i = tid; i < n; i += kScanThreads)
      scatter_row(i, sc.topk_idx, sc.lrank, blk_base, offsets, n_tok, N, k, S, capacity,
                  sc.sorted_tok, sc.inv_row);
  }
  // balance statistics from the totals above (counts and prob_sum are
  // complete and visible to the workgroup since the barriers above)
  if (bal.f != nullptr || bal.P != nullptr || bal.aux != nullptr) {
    __shared__ float s_bal[256];
    balance_block(n_tok, N, k, counts, prob_sum, bal.alpha, bal.f, bal.P, bal.aux, s_bal);
  }
}

__global__ __launch_bounds__(256) void scatter_kernel(
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ lrank,
    const int32_t* __restrict__ blk_base, const int32_t* __restrict__ offsets, int n_tok, int N,
    int k, int S, int capacity, int32_t* __restrict__ sorted_tok, int32_t* __restrict__ inv_row) {
  scatter_row(static_cast<long>(blockIdx.x) * 256 + threadIdx.x, topk_idx, lrank, blk_base,
              offsets, n_tok, N, k, S, capacity, sorted_tok, inv_row);
}

}  // namespace

hipError_t launch_scan(const int32_t* blk_counts, const float* blk_psum, int T_, int N, int k,
                       int S, int capacity, int bm_up, int cap_up, int bm_down, int cap_down,
                       const SplitSpec& split, const ItemSpec& items, const ScatterSpec& sc,
                       const BalanceSpec& bal, int32_t* blk_base, int32_t* counts, float* prob_sum,
                       int32_t* user_counts, float* user_prob_sum, int32_t* offsets,
                       int2* tiles_up, int2* tiles_down, int32_t* ntiles, hipStream_t s) {
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, s, blk_counts, blk_psum, T_, N,
                     k, S, capacity, bm_up, cap_up, bm_down, cap_down, split, items, sc, bal,
                     blk_base,
                     counts, prob_sum,
                     user_counts, user_prob_sum, offsets, tiles_up, tiles_down, ntiles);
  return hipGetLastError();
}

hipError_t launch_items(const ItemSpec& is, int groups, long max_items, hipStream_t s) {
  if ((is.nnt_up <= 0 && is.nnt_down <= 0) || max_items <= 0) return hipSuccess;
  const unsigned bx = static_cast<unsigned>((max_items + 255) / 256);
  hipLaunchKernelGGL(items_kernel, dim3(bx, 2), dim3(256), 0, s, is, groups);
  return hipGetLastError();
}

hipError_t launch_scatter(const int32_t* topk_idx, const int32_t* lrank, const int32_t* blk_base,
                          const int32_t* offsets, int T_, int N, int k, int S, int capacity,
                          int32_t* sorted_tok, int32_t* inv_row, hipStream_t s) {
  const long n = static_cast<long>(T_) * k + static_cast<long>(S) * T_;
  const int blocks = static_cast<int>((n + 255) / 256);
  hipLaunchKernelGGL(scatter_kernel, dim3(blocks), dim3(256), 0, s, topk_idx, lrank, blk_base,
                     offsets, T_, N, k, S, capacity, sorted_tok, inv_row);
  return hipGetLastError();
}

}  // namespace moe
