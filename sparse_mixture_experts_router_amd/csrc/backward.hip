// Layer backward: the kernels of the training pass that the forward's own
// kernels do not cover.
//
// The gradients are those of L = sum(y * dy) + c * aux through the forward
// ("Mixture of experts and speculative decoding", "Opening the hood: the MoE
// layer precisely"; "MoE inference: the call centre with 256 specialists
// ...", "The bare mechanism"), with the balance loss reaching the router
// through P only, f coming from a hard choice ("Mixture of Experts and Guided
// Decoding", the routing-collapse passage after the auxiliary-loss equation).
// A row is one kept (token, slot) assignment or one shared-expert row, in the
// forward's expert-major order; G, U are the recomputed gate/up projections
// and D[row] = dy[token] W_down[e] (all three from the forward's plain grouped
// GEMM, W_down transposed first):
//
//   h        = SiLU(G) U
//   dg[row]  = <D, h>                                  the gate's gradient
//   dA, dB   = (g D) U SiLU'(G), (g D) SiLU(G)         g = the row's gate (1 shared)
//   dXp      = [dA dB] [W_gate; W_up]                  plain GEMM, weights transposed
//   dr[t]    = softmax backward of the kept gates  +  p_t (c - <c, p_t>)
//              with c_e = c N f_e / T (balance loss)   router_bwd_kernel
//   dx[t]    = dr[t] W_r + sum of the token's dXp rows
//   dW_down[e] = sum_rows (g dy)^T h,  dW_gate[e] = dA^T x,  dW_up[e] = dB^T x,
//   dW_r = dr^T x
//
// The weight gradients reduce over rows.  Their operands are first transposed
// into K-major segments, one per expert, each padded with zero columns, so
// that one grouped GEMM with a reduction length per group computes every
// expert's gradient: to a multiple of 64 when the large-tile kernel's
// K-major mode takes the products (bf16), else to a multiple of 128 for
// kgemm_kernel, which takes its K steps in pairs.  (Padding to 128 made the
// DeepSeek-V3-shaped experts, 190-324 rows each, reduce over 321 columns on
// average instead of 292.)
#include "lds_ring.h"
#include "vec.h"

#include <math.h>
#include <type_traits>

namespace moe {
namespace {

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v); }
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }

// ------------------------------------------------------------- transposes
// 64 x 64 tiles through LDS with 16-byte global accesses on both sides: a
// thread moves V = 16 / sizeof(T) consecutive elements of a source row in,
// and V consecutive elements of a destination row out.  Callers keep C,
// col0 and ldd multiples of 64 (every row length here is), so no 16-byte
// access straddles the end of a row.
template <typename T> struct alignas(16) Chunk {
  static constexpr int V = 16 / static_cast<int>(sizeof(T));
  T v[V];
};

// dst[b][c][col0 + r] = src[b][r][c] for r < R, 0 for R <= r < rpad.
// Grid (ceil(rpad / 64), C / 64, batch).
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ src, int R, int C,
                                                        long src_batch, T* __restrict__ dst,
                                                        long ldd, int col0, int rpad,
                                                        long dst_batch) {
  constexpr int V = Chunk<T>::V, CPR = 64 / V, RPP = 256 / CPR;
  __shared__ __attribute__((aligned(16))) T tile[64][64 + V];
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const T* s = src + blockIdx.z * src_batch;
  T* d = dst + blockIdx.z * dst_batch;
  const int t = threadIdx.x, ch = (t % CPR) * V;
  for (int i = t / CPR; i < 64; i += RPP) {
    const int r = r0 + i, c = c0 + ch;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < R && c < C) v = *reinterpret_cast<const u32x4*>(s + static_cast<long>(r) * C + c);
    *reinterpret_cast<u32x4*>(&tile[i][ch]) = v;
  }
  __syncthreads();
  for (int j = t / CPR; j < 64; j += RPP) {
    const int c = c0 + j, r = r0 + ch;
    if (c >= C || r >= rpad) continue;
    Chunk<T> out;
#pragma unroll
    for (int q = 0; q < V; ++q) out.v[q] = tile[ch + q][j];
    T* o = d + static_cast<long>(c) * ldd + col0 + r;
    if (r + V <= rpad) {
      *reinterpret_cast<Chunk<T>*>(o) = out;
    } else {
      for (int q = 0; q < V && r + q < rpad; ++q) o[q] = out.v[q];
    }
  }
}

// Segment starts: kbase[0] = 0, kbase[g + 1] = kbase[g] + (rows of group g
// rounded up to `align`, a power of two).  One workgroup; groups <= 1024.
__global__ __launch_bounds__(1024) void kbase_kernel(const int32_t* __restrict__ offsets, int G,
                                                     int align, int32_t* __restrict__ kbase) {
  __shared__ int s[1024];
  const int t = threadIdx.x;
  s[t] = t < G ? ((offsets[t + 1] - offsets[t] + align - 1) & ~(align - 1)) : 0;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int add = t >= off ? s[t - off] : 0;
    __syncthreads();
    s[t] += add;
    __syncthreads();
  }
  if (t < G) kbase[t + 1] = s[t];
  if (t == 0) kbase[0] = 0;
}

// Rows of every group, transposed into its segment: for group g's j-th row
// (permuted row offsets[g] + j; source row gather[that] or that row itself),
// dst[c][kbase[g] + j] = scale * src[source row][c], with scale = rscale[row]
// (or 1); columns of the padding are 0.  Grid (kmax / 64, C / 64); a
// 64-column block lies inside one segment, so it finds its group by binary
// search over kbase.  16-byte accesses as in transpose_kernel.
template <typename T>
__global__ __launch_bounds__(256) void segment_transpose_kernel(
    const T* __restrict__ src, int C, int src_rows, const int32_t* __restrict__ gather,
    const float* __restrict__ rscale, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ kbase, int G, T* __restrict__ dst, long ldd) {
  constexpr int V = Chunk<T>::V, CPR = 64 / V, RPP = 256 / CPR;
  __shared__ __attribute__((aligned(16))) T tile[64][64 + V];
  __shared__ int s_row[64];
  __shared__ float s_sc[64];
  const int k0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  if (k0 >= kbase[G]) return;  // uniform over the workgroup
  int lo = 0, hi = G;          // kbase[lo] <= k0 < kbase[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (kbase[mid] <= k0) lo = mid;
    else hi = mid;
  }
  const int j0 = k0 - kbase[lo];
  const int off = offsets[lo], cnt = offsets[lo + 1] - off;
  const int t = threadIdx.x;
  if (t < 64) {
    const int j = j0 + t;
    int row = -1;
    float sc = 0.f;
    if (j < cnt) {
      row = gather != nullptr ? gather[off + j] : off + j;
      row = min(max(row, 0), src_rows - 1);
      sc = rscale != nullptr ? rscale[off + j] : 1.f;
    }
    s_row[t] = row;
    s_sc[t] = sc;
  }
  __syncthreads();
  const int ch = (t % CPR) * V;
  for (int i = t / CPR; i < 64; i += RPP) {
    const int row = s_row[i], c = c0 + ch;
    Chunk<T> v;
    if (row >= 0 && c < C) {
      v = *reinterpret_cast<const Chunk<T>*>(src + static_cast<long>(row) * C + c);
      if (rscale != nullptr) {
        const float sc = s_sc[i];
#pragma unroll
        for (int q = 0; q < V; ++q) v.v[q] = from_f32<T>(sc * to_f32<T>(v.v[q]));
      }
    } else {
#pragma unroll
      for (int q = 0; q < V; ++q) v.v[q] = T(0);
    }
    *reinterpret_cast<Chunk<T>*>(&tile[i][ch]) = v;
  }
  __syncthreads();
  for (int j = t / CPR; j < 64; j += RPP) {
    const int c = c0 + j;
    if (c >= C) continue;
    Chunk<T> out;
#pragma unroll
    for (int q = 0; q < V; ++q) out.v[q] = tile[ch + q][j];
    *reinterpret_cast<Chunk<T>*>(dst + static_cast<long>(c) * ldd + k0 + ch) = out;
  }
}

// ------------------------------------------------------------- row kernels
// Gate of every permuted row: the (token, slot) gate for a kept routed row,
// 1 for a shared-expert row.
__global__ __launch_bounds__(256) void row_gate_kernel(const int32_t* __restrict__ inv_row,
                                                       const float* __restrict__ gate,
                                                       const int32_t* __restrict__ offsets,
                                                       int n_tok, int k, int N, int S,
                                                       float* __restrict__ rgate) {
  const long i = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
  const long tk = static_cast<long>(n_tok) * k;
  if (i < tk) {
    const int r = inv_row[i];
    if (r >= 0) rgate[r] = gate[i];
  } else if (i < tk + static_cast<long>(S) * n_tok) {
    const long j = i - tk;
    const int s = static_cast<int>(j / n_tok), t = static_cast<int>(j - static_cast<long>(s) * n_tok);
    rgate[offsets[N + s] + t] = 1.f;
  }
}

// Sum over a workgroup of 256 in a fixed order (lanes by butterfly, then the
// four wavefronts in order); every thread gets the total.
__device__ __forceinline__ float block_sum256(float v, float* s_red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) s_red[wave] = v;
  __syncthreads();
  const float t = ((s_red[0] + s_red[1]) + s_red[2]) + s_red[3];
  __syncthreads();
  return t;
}

// One workgroup per permuted row r < offsets[G]: h = SiLU(G) U (written to
// H), dg_row[r] = <D, h>, and [dA | dB] with the row's gate applied to D.
template <typename T>
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(
    const T* __restrict__ Gm, const T* __restrict__ Um, const T* __restrict__ Dm,
    const float* __restrict__ rgate, const int32_t* __restrict__ offsets, int G, int F,
    T* __restrict__ H, T* __restrict__ dAB, float* __restrict__ dg_row) {
  __shared__ float s_red[4];
  const int r = blockIdx.x;
  if (r >= offsets[G]) return;  // uniform over the workgroup
  constexpr int V = Vec<T>::kN;
  const float gt = rgate[r];
  const long ro = static_cast<long>(r) * F;
  float part = 0.f;
  for (int c = threadIdx.x * V; c < F; c += 256 * V) {
    float a[V], b[V], dd[V], h[V], da[V], db[V];
    Vec<T>::load(Gm + ro + c, a);
    Vec<T>::load(Um + ro + c, b);
    Vec<T>::load(Dm + ro + c, dd);
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const float s = 1.f / (1.f + expf(-a[v]));
      h[v] = a[v] * s * b[v];
      part += dd[v] * h[v];
      const float dh = gt * dd[v];
      da[v] = dh * b[v] * (s + a[v] * s * (1.f - s));
      db[v] = dh * a[v] * s;
    }
    Vec<T>::store(H + ro + c, h);
    Vec<T>::store(dAB + 2 * ro + c, da);
    Vec<T>::store(dAB + 2 * ro + F + c, db);
  }
  const float tot = block_sum256(part, s_red);
  if (threadIdx.x == 0) dg_row[r] = tot;
}

// Router gradient, one wavefront per token (4 per workgroup):
//   p = softmax(r_t) over all N, c_e = aux_grad alpha N (count_e / (T k)) / T,
//   dr[e] = p_e (c_e - sum_j c_j p_j)                        balance loss via P
//   dr[idx_s] += g_s (dg_s - sum_l g_l dg_l)                 kept-gate softmax
// (dg_s = dg_row of the slot's row, 0 for a dropped slot).  Writes dr in the
// layer type padded with zeros to Kr columns (the GEMM operand) and as fp32.
template <typename T>
__global__ __launch_bounds__(256) void router_bwd_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ idx,
    const float* __restrict__ gate, const int32_t* __restrict__ inv_row,
    const float* __restrict__ dg_row, const int32_t* __restrict__ counts, int n_tok, int N, int k,
    float alpha, float aux_grad, int Kr, T* __restrict__ dr_pad, float* __restrict__ dr32) {
  __shared__ float s_dr[4][kMaxExperts];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  const bool ok = t < n_tok;
  constexpr int EPL = kMaxExperts / 64;
  const float* rt = logits + static_cast<long>(ok ? t : 0) * N;
  float p[EPL], c[EPL];
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + 64 * j;
    p[j] = (ok && e < N) ? rt[e] : -INFINITY;
    m = fmaxf(m, p[j]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  float se = 0.f;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + 64 * j;
    p[j] = (ok && e < N) ? expf(p[j] - m) : 0.f;
    se += p[j];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) se += __shfl_xor(se, off, 64);
  const float tk = static_cast<float>(n_tok) * static_cast<float>(k);
  float cp = 0.f;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + 64 * j;
    p[j] = ok ? p[j] / se : 0.f;
    c[j] = e < N ? aux_grad * alpha * static_cast<float>(N) *
                       (static_cast<float>(counts[e]) / tk) / static_cast<float>(n_tok)
                 : 0.f;
    cp += c[j] * p[j];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) cp += __shfl_xor(cp, off, 64);
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + 64 * j;
    if (e < N) s_dr[wave][e] = p[j] * (c[j] - cp);
  }
  __syncthreads();
  // kept-gate softmax: lane s < k holds slot s
  float gs = 0.f, dg = 0.f;
  int es = 0;
  if (ok && lane < k) {
    const long o = static_cast<long>(t) * k + lane;
    es = idx[o];
    gs = gate[o];
    const int row = inv_row[o];
    dg = row >= 0 ? dg_row[row] : 0.f;
  }
  float gd = gs * dg;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) gd += __shfl_xor(gd, off, 64);
  if (ok && lane < k) s_dr[wave][es] += gs * (dg - gd);  // distinct experts per token
  __syncthreads();
  if (!ok) return;
  for (int e = lane; e < Kr; e += 64) {
    const float v = e < N ? s_dr[wave][e] : 0.f;
    dr_pad[static_cast<long>(t) * Kr + e] = from_f32<T>(v);
    if (e < N) dr32[static_cast<long>(t) * N + e] = v;
  }
}

// d logit_bias[e] = sum_t dr32[t, e]: one workgroup per expert; thread i
// adds tokens i, i + 256, ... (eight loads in flight), then the fixed-order
// workgroup sum.
__global__ __launch_bounds__(256) void colsum_kernel(const float* __restrict__ dr32, int n_tok,
                                                     int N, float* __restrict__ out) {
  __shared__ float s_red[4];
  const int e = blockIdx.x;
  float acc = 0.f;
  for (int t0 = threadIdx.x; t0 < n_tok; t0 += 256 * 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int t = t0 + 256 * u;
      v[u] = t < n_tok ? dr32[static_cast<long>(t) * N + e] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += v[u];
  }
  const float tot = block_sum256(acc, s_red);
  if (threadIdx.x == 0) out[e] = tot;
}

// dx[t] = dxr[t] + the token's kept routed rows of dXp (slot order) + its
// shared rows, accumulated in fp32, rounded once.  One workgroup per token.
template <typename T>
__global__ __launch_bounds__(256) void dx_combine_kernel(
    const T* __restrict__ dXp, const float* __restrict__ dxr, const int32_t* __restrict__ inv_row,
    const int32_t* __restrict__ offsets, int N, int k, int S, int d, T* __restrict__ dx) {
  constexpr int V = Vec<T>::kN;
  const int t = blockIdx.x;
  for (int c = threadIdx.x * V; c < d; c += 256 * V) {
    float acc[V], v[V];
    Vec<float>::load(dxr + static_cast<long>(t) * d + c, acc);
    if constexpr (V == 8) Vec<float>::load(dxr + static_cast<long>(t) * d + c + 4, acc + 4);
    for (int s = 0; s < k; ++s) {
      const int r = inv_row[static_cast<long>(t) * k + s];
      if (r < 0) continue;
      Vec<T>::load(dXp + static_cast<long>(r) * d + c, v);
#pragma unroll
      for (int i = 0; i < V; ++i) acc[i] += v[i];
    }
    for (int s = 0; s < S; ++s) {
      Vec<T>::load(dXp + static_cast<long>(offsets[N + s] + t) * d + c, v);
#pragma unroll
      for (int i = 0; i < V; ++i) acc[i] += v[i];
    }
    Vec<T>::store(dx + static_cast<long>(t) * d + c, acc);
  }
}

// Selection-bias step of auxiliary-loss-free routing ("The bare mechanism",
// auxiliary-loss-free variant; the rule is this library's reading):
// bias[e] += rate * sign(mean load - count[e]), the sign taken exactly as
// sign(sum_j count[j] - N count[e]).  One workgroup.
__global__ __launch_bounds__(512) void bias_update_kernel(const int32_t* __restrict__ counts,
                                                          int N, float rate,
                                                          float* __restrict__ bias) {
  __shared__ long long s[512];
  const int t = threadIdx.x;
  const long long c = t < N ? counts[t] : 0;
  s[t] = c;
  __syncthreads();
  for (int off = 256; off >= 1; off >>= 1) {
    if (t < off) s[t] += s[t + off];
    __syncthreads();
  }
  if (t < N) {
    const long long diff = s[0] - static_cast<long long>(N) * c;
    const float step = diff > 0 ? rate : (diff < 0 ? -rate : 0.f);
    bias[t] = bias[t] + step;
  }
}

// ------------------------------------------------------------- kgemm
// Grouped GEMM with a reduction length per group (the weight gradients):
//   C_g[m][n] = sum_{kk in [kbase[g], kbase[g+1])} A[m][kk] B[n][kk]
// for m < M, n < N; A, B row-major with pitches lda, ldb (elements), every
// segment a multiple of 128 elements (zero padded), so the K steps of 128
// bytes per row come in pairs.  N is a multiple of 64.  Groups >= alt_from
// write to c_alt instead (shared experts).  128 x 128 tiles, 4 wavefronts of
// 64 x 64.  Rows of 128 bytes in LDS, their 16-byte chunks XOR-swizzled by
// row mod 8 (swz128), so each 16-lane phase of a fragment read lands in 16
// different bank groups.  Each thread stages its 16-byte slices of a K step
// in registers:
// the loads of step s + 2 are issued while step s is multiplied out of one
// LDS buffer and step s + 1 is stored into the other, and the barrier that
// ends a step waits only for LDS traffic.  The epilogue stages each
// wavefront's block through LDS and writes whole 16-byte row chunks.
struct KgArgs {
  const void* a;
  const void* b;
  long lda, ldb;
  int M, N;
  const int32_t* kbase;  // [groups + 1], or null: one group over [0, k_all)
  int k_all;
  void* c;
  void* c_alt;
  int alt_from;
};

template <typename TO>
constexpr int kgemm_lds_bytes() {
  // two buffers of A and B tiles (128 rows x 128 bytes), or the epilogue's
  // four staged 64 x 64 blocks, whichever is larger
  return 4 * 128 * 128 > 4 * 64 * (64 * static_cast<int>(sizeof(TO)) + 16)
             ? 4 * 128 * 128
             : 4 * 64 * (64 * static_cast<int>(sizeof(TO)) + 16);
}

template <typename T, typename TO>
__global__ __launch_bounds__(256) void kgemm_kernel(KgArgs g) {
  __shared__ __attribute__((aligned(16))) char lds_raw[kgemm_lds_bytes<TO>()];
  // buffer P, operand X (0 = A, 1 = B)
  auto buf = [&](int P, int X) { return lds_raw + (P * 2 + X) * 128 * 128; };
  const int grp = blockIdx.y;
  const int ntn = (g.N + 127) / 128;
  const int m0 = (blockIdx.x / ntn) * 128, n0 = (blockIdx.x % ntn) * 128;
  const long kb = g.kbase != nullptr ? g.kbase[grp] : 0;
  const long ke = g.kbase != nullptr ? g.kbase[grp + 1] : g.k_all;
  const int nsteps = static_cast<int>((ke - kb) * static_cast<long>(sizeof(T)) / 128);  // even
  const char* A = static_cast<const char*>(g.a) + kb * static_cast<long>(sizeof(T));
  const char* B = static_cast<const char*>(g.b) + kb * static_cast<long>(sizeof(T));
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const char* pa[4];
  const char* pb[4];
  int lo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = tid + 256 * i, row = q >> 3, ch = q & 7;
    const long ar = min(m0 + row, g.M - 1), br = min(n0 + row, g.N - 1);
    pa[i] = A + ar * g.lda * static_cast<long>(sizeof(T)) + ch * 16;
    pb[i] = B + br * g.ldb * static_cast<long>(sizeof(T)) + ch * 16;
    lo[i] = swz128(row, ch);
  }
  u32x4 ra[2][4], rb[2][4];
  // loads of step s (clamped into the segment) into register slot P
  auto gload = [&](auto slot, int s) {
    constexpr int P = decltype(slot)::value;
    const long off = static_cast<long>(min(s, nsteps - 1)) * 128;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[P][i] = *reinterpret_cast<const u32x4*>(pa[i] + off);
      rb[P][i] = *reinterpret_cast<const u32x4*>(pb[i] + off);
    }
  };
  auto sstore = [&](auto slot) {
    constexpr int P = decltype(slot)::value;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<u32x4*>(buf(P, 0) + lo[i]) = ra[P][i];
      *reinterpret_cast<u32x4*>(buf(P, 1) + lo[i]) = rb[P][i];
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](auto stage) {
    constexpr int P = decltype(stage)::value;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x4 af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        af[i] = *reinterpret_cast<const u32x4*>(
            buf(P, 0) + swz128(wm * 64 + i * 16 + (lane & 15), kk * 4 + (lane >> 4)));
        bf[i] = *reinterpret_cast<const u32x4*>(
            buf(P, 1) + swz128(wn * 64 + i * 16 + (lane & 15), kk * 4 + (lane >> 4)));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = Mfma<T>::step(af[i], bf[j], acc[i][j]);
    }
  };

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  if (nsteps > 0) {
    gload(S0{}, 0);
    gload(S1{}, 1);
    sstore(S0{});
    lds_barrier();
    // (the scheduling barriers keep each step's loads ahead of its MFMAs:
    // issued late, they would leave one step of latency hiding instead of two)
    for (int s = 0; s < nsteps; s += 2) {
      // step s from LDS buffer 0; step s + 1 waits in register slot 1
      gload(S0{}, s + 2);
      __builtin_amdgcn_sched_barrier(0);
      compute(S0{});
      sstore(S1{});
      lds_barrier();
      // step s + 1 from buffer 1; step s + 2 waits in slot 0
      gload(S1{}, s + 3);
      __builtin_amdgcn_sched_barrier(0);
      compute(S1{});
      sstore(S0{});
      lds_barrier();
    }
  }

  // epilogue: the wavefront's 64 x 64 block through LDS (rows of 64 outputs
  // padded by 16 bytes), then 16-byte row chunks
  constexpr int V = 16 / static_cast<int>(sizeof(TO));
  constexpr int RB = 64 * static_cast<int>(sizeof(TO)) + 16;  // staged row bytes
  char* stg = lds_raw + wave * 64 * RB;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = i * 16 + 4 * (lane >> 4) + r, col = j * 16 + (lane & 15);
        *reinterpret_cast<TO*>(stg + row * RB + col * static_cast<int>(sizeof(TO))) =
            from_f32<TO>(acc[i][j][r]);
      }
  lds_barrier();
  const bool alt = grp >= g.alt_from;
  TO* C = static_cast<TO*>(alt ? g.c_alt : g.c) +
          static_cast<long>(alt ? grp - g.alt_from : grp) * g.M * g.N;
  constexpr int CPR = 64 / V;  // 16-byte chunks per staged row
#pragma unroll
  for (int it = 0; it < 64 * CPR / 64; ++it) {
    const int q = lane + 64 * it, row = q / CPR, c = (q % CPR) * V;
    const int grow = m0 + wm * 64 + row, gcol = n0 + wn * 64 + c;
    if (grow < g.M && gcol < g.N)
      *reinterpret_cast<u32x4*>(C + static_cast<long>(grow) * g.N + gcol) =
          *reinterpret_cast<const u32x4*>(stg + row * RB + c * static_cast<int>(sizeof(TO)));
  }
}

}  // namespace

// ------------------------------------------------------------- launchers
template <typename T>
static hipError_t transpose_t(const void* src, int R, int C, long src_batch, void* dst, long ldd,
                              int col0, int rpad, long dst_batch, int batch, hipStream_t s) {
  if (rpad <= 0 || C <= 0 || batch <= 0) return hipSuccess;
  const dim3 grid((rpad + 63) / 64, (C + 63) / 64, batch);
  hipLaunchKernelGGL(transpose_kernel<T>, grid, dim3(256), 0, s, static_cast<const T*>(src), R, C,
                     src_batch, static_cast<T*>(dst), ldd, col0, rpad, dst_batch);
  return hipGetLastError();
}

hipError_t launch_transpose(int dtype, const void* src, int R, int C, long src_batch, void* dst,
                            long ldd, int col0, int rpad, long dst_batch, int batch,
                            hipStream_t s) {
  if (dtype == 1)
    return transpose_t<bf16_t>(src, R, C, src_batch, dst, ldd, col0, rpad, dst_batch, batch, s);
  return transpose_t<float>(src, R, C, src_batch, dst, ldd, col0, rpad, dst_batch, batch, s);
}

hipError_t launch_kbase(const int32_t* offsets, int G, int align, int32_t* kbase, hipStream_t s) {
  hipLaunchKernelGGL(kbase_kernel, dim3(1), dim3(1024), 0, s, offsets, G, align, kbase);
  return hipGetLastError();
}

hipError_t launch_segment_transpose(int dtype, const void* src, int C, int src_rows,
                                    const int32_t* gather, const float* rscale,
                                    const int32_t* offsets, const int32_t* kbase, int G,
                                    long kmax, void* dst, long ldd, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(kmax / 64), (C + 63) / 64);
  if (dtype == 1)
    hipLaunchKernelGGL(segment_transpose_kernel<bf16_t>, grid, dim3(256), 0, s,
                       static_cast<const bf16_t*>(src), C, src_rows, gather, rscale, offsets,
                       kbase, G, static_cast<bf16_t*>(dst), ldd);
  else
    hipLaunchKernelGGL(segment_transpose_kernel<float>, grid, dim3(256), 0, s,
                       static_cast<const float*>(src), C, src_rows, gather, rscale, offsets,
                       kbase, G, static_cast<float*>(dst), ldd);
  return hipGetLastError();
}

hipError_t launch_row_gate(const int32_t* inv_row, const float* gate, const int32_t* offsets,
                           int T_, int k, int N, int S, float* rgate, hipStream_t s) {
  const long n = static_cast<long>(T_) * (k + S);
  hipLaunchKernelGGL(row_gate_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                     s, inv_row, gate, offsets, T_, k, N, S, rgate);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(int dtype, const void* G_, const void* U, const void* D,
                             const float* rgate, const int32_t* offsets, int G, int F,
                             long rows_max, void* H, void* dAB, float* dg_row, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(rows_max));
  if (dtype == 1)
    hipLaunchKernelGGL(swiglu_bwd_kernel<bf16_t>, grid, dim3(256), 0, s,
                       static_cast<const bf16_t*>(G_), static_cast<const bf16_t*>(U),
                       static_cast<const bf16_t*>(D), rgate, offsets, G, F,
                       static_cast<bf16_t*>(H), static_cast<bf16_t*>(dAB), dg_row);
  else
    hipLaunchKernelGGL(swiglu_bwd_kernel<float>, grid, dim3(256), 0, s,
                       static_cast<const float*>(G_), static_cast<const float*>(U),
                       static_cast<const float*>(D), rgate, offsets, G, F,
                       static_cast<float*>(H), static_cast<float*>(dAB), dg_row);
  return hipGetLastError();
}

hipError_t launch_router_bwd(int dtype, const float* logits, const int32_t* idx,
                             const float* gate, const int32_t* inv_row, const float* dg_row,
                             const int32_t* counts, int T_, int N, int k, float alpha,
                             float aux_grad, int Kr, void* dr_pad, float* dr32, hipStream_t s) {
  const dim3 grid((T_ + 3) / 4);
  if (dtype == 1)
    hipLaunchKernelGGL(router_bwd_kernel<bf16_t>, grid, dim3(256), 0, s, logits, idx, gate,
                       inv_row, dg_row, counts, T_, N, k, alpha, aux_grad, Kr,
                       static_cast<bf16_t*>(dr_pad), dr32);
  else
    hipLaunchKernelGGL(router_bwd_kernel<float>, grid, dim3(256), 0, s, logits, idx, gate,
                       inv_row, dg_row, counts, T_, N, k, alpha, aux_grad, Kr,
                       static_cast<float*>(dr_pad), dr32);
  return hipGetLastError();
}

hipError_t launch_colsum(const float* dr32, int T_, int N, float* out, hipStream_t s) {
  hipLaunchKernelGGL(colsum_kernel, dim3(N), dim3(256), 0, s, dr32, T_, N, out);
  return hipGetLastError();
}

hipError_t launch_dx_combine(int dtype, const void* dXp, const float* dxr, const int32_t* inv_row,
                             const int32_t* offsets, int T_, int N, int k, int S, int d, void* dx,
                             hipStream_t s) {
  if (dtype == 1)
    hipLaunchKernelGGL(dx_combine_kernel<bf16_t>, dim3(T_), dim3(256), 0, s,
                       static_cast<const bf16_t*>(dXp), dxr, inv_row, offsets, N, k, S, d,
                       static_cast<bf16_t*>(dx));
  else
    hipLaunchKernelGGL(dx_combine_kernel<float>, dim3(T_), dim3(256), 0, s,
                       static_cast<const float*>(dXp), dxr, inv_row, offsets, N, k, S, d,
                       static_cast<float*>(dx));
  return hipGetLastError();
}

hipError_t launch_bias_update(const int32_t* counts, int N, float rate, float* bias,
                              hipStream_t s) {
  hipLaunchKernelGGL(bias_update_kernel, dim3(1), dim3(512), 0, s, counts, N, rate, bias);
  return hipGetLastError();
}

// out_f32: C is fp32 (else the layer type).  groups <= 65535.
hipError_t launch_kgemm(int dtype, bool out_f32, const void* a, long lda, const void* b, long ldb,
                        int M, int N, int groups, const int32_t* kbase, int k_all, void* c,
                        void* c_alt, int alt_from, hipStream_t s) {
  if (M <= 0 || N <= 0 || groups <= 0) return hipSuccess;
  if (dtype == 1 && !out_f32 && kbase != nullptr && lda == ldb) {
    // grouped bf16 products on the forward's 256 x 256 LDS-DMA kernel
    GemmArgs ga{};
    ga.a = a;
    ga.w0 = b;
    ga.a_rows = M;
    ga.n_dim = N;
    ga.k_dim = static_cast<int>(lda);
    ga.kbase = kbase;
    ga.groups = groups;
    ga.out = c;
    ga.out_alt = c_alt;
    ga.alt_from = alt_from;
    const hipError_t e = launch_kmajor_gemm(ga, s);
    if (e != hipErrorInvalidValue) return e;  // else: operands it does not take
  }
  KgArgs g{a, b, lda, ldb, M, N, kbase, k_all, c, c_alt, alt_from};
  const dim3 grid(static_cast<unsigned>(((M + 127) / 128) * ((N + 127) / 128)), groups);
  if (dtype == 1) {
    if (out_f32)
      hipLaunchKernelGGL((kgemm_kernel<bf16_t, float>), grid, dim3(256), 0, s, g);
    else
      hipLaunchKernelGGL((kgemm_kernel<bf16_t, bf16_t>), grid, dim3(256), 0, s, g);
  } else {
    hipLaunchKernelGGL((kgemm_kernel<float, float>), grid, dim3(256), 0, s, g);
  }
  return hipGetLastError();
}

}  // namespace moe
