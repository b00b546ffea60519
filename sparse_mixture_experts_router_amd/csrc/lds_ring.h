// Helpers for the global -> LDS ring buffers of the route and GEMM kernels.
#pragma once

#include "moe_internal.h"

namespace moe {

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(1))) void* global_void_ptr;

__device__ __forceinline__ void load_lds16(const char* src, char* lds_dst) {
  __builtin_amdgcn_global_load_lds((global_void_ptr)(src), (lds_void_ptr)(lds_dst), 16, 0, 0);
}
// The same load with the non-temporal cache policy (nt): for lines read
// once, so that they give way first in L2 to lines other workgroups reuse.
__device__ __forceinline__ void load_lds16_nt(const char* src, char* lds_dst) {
  __builtin_amdgcn_global_load_lds((global_void_ptr)(src), (lds_void_ptr)(lds_dst), 16, 0, 2);
}

// s_waitcnt vmcnt(N) lgkmcnt(0), expcnt untouched (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]).
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier that does not drain outstanding global->LDS loads
// (__syncthreads() would wait for all of them and serialise the ring).
// Callers first wait for exactly the loads they need with wait_vmem<N>().
// The empty asm statements keep the compiler from moving memory accesses
// across it.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Workgroup barrier once this wavefront's LDS accesses have completed; its
// global loads into registers keep flying (__syncthreads() would wait for
// them too).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

constexpr int kRowBytes = 64;  // bytes of every staged row per K step (32 bf16)

// Byte offset of 16-byte chunk c (0..3) of staged row r: 64-byte rows, chunk
// index XOR-ed with bits 1-2 of the row, so the 8 lanes of a ds_read_b128
// group (8 consecutive rows, same logical chunk) hit 8 distinct bank groups.
__device__ __forceinline__ int swz64(int r, int c) { return r * kRowBytes + ((c ^ ((r >> 1) & 3)) << 4); }

// For a 1 KB ring block (16 rows of 64 bytes) written by one
// global_load_lds_dwordx4, lane l lands in physical chunk l % 4 of row l / 4;
// the logical chunk it must fetch so that the block matches swz64:
__device__ __forceinline__ int ring_lane_chunk(int lane) { return (lane & 3) ^ ((lane >> 3) & 3); }

// 128-byte rows: one whole cache line per row and buffer (two K steps of 32
// bf16).  Chunk c (0..7) of row r is stored at chunk c ^ (r mod 8).
//
// Why that key: gfx950 serves a ds_read_b128 in four phases of 16 lanes, and
// a phase is not 16 consecutive lanes.  Lanes 0-7 share a phase with lanes
// 24-31, and lanes 8-15 with 16-23 (likewise in the upper half), which an
// in-bounds probe of the LDS bank-conflict counter showed: lanes l and l + 8
// (l < 8) never conflict, while l and l + 24 do.  An MFMA fragment read
// (lane l: row l mod 16, chunk l / 16 + 4 t) therefore pairs rows 0-7 of
// chunk 2q with rows 8-15 of chunk 2q + 1, and the reverse.  A row is half of
// the 64 banks' 256 bytes, so its bank group is 8 (r mod 2) + physical chunk,
// and with key r mod 8 each phase's 16 lanes land on 16 distinct groups.  The
// key (r mod 8) ^ (bit 3 of r), right for phases of consecutive lanes, made
// every fragment read a 2-way conflict (LDS bank-conflict cycles were half of
// the LDS active cycles in the expert GEMMs).  Writes of whole rows (8 lanes
// per row, as the global -> LDS loads and the register-staged stores issue
// them) are conflict-free under either key.
constexpr int kLineBytes = 128;
__device__ __forceinline__ int swz128_key(int r) { return r & 7; }
__device__ __forceinline__ int swz128(int r, int c) { return r * kLineBytes + ((c ^ swz128_key(r)) << 4); }

// For a 1 KB block (8 rows of 128 bytes) written by one
// global_load_lds_dwordx4, lane l lands in physical chunk l % 8 of row
// 8 blk + l / 8 (whose key is l / 8); the logical chunk it must fetch so that
// the block matches swz128:
__device__ __forceinline__ int line_lane_chunk(int lane, int /*blk*/) { return (lane & 7) ^ (lane >> 3); }

}  // namespace moe
