// Helpers for the global -> LDS ring buffers of the route and GEMM kernels.
#pragma once

#include "moe_internal.h"

namespace moe {

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(1))) void* global_void_ptr;

__device__ __forceinline__ void load_lds16(const char* src, char* lds_dst) {
  __builtin_amdgcn_global_load_lds((global_void_ptr)(src), (lds_void_ptr)(lds_dst), 16, 0, 0);
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
// bf16).  Chunk c (0..7) of row r is stored at chunk c ^ key(r), with
// key(r) = (r mod 8) ^ (bit 3 of r): the 16 lanes of a ds_read_b128 fragment
// group (16 consecutive rows, one logical chunk) then hit 16 distinct 16-byte
// bank groups of a 256-byte bank row, and any 8 consecutive ones 8 distinct
// groups of a 128-byte one.
constexpr int kLineBytes = 128;
__device__ __forceinline__ int swz128_key(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int swz128(int r, int c) { return r * kLineBytes + ((c ^ swz128_key(r)) << 4); }

// For a 1 KB block (8 rows of 128 bytes, block index blk within the buffer)
// written by one global_load_lds_dwordx4, lane l lands in physical chunk
// l % 8 of row 8 blk + l / 8; the logical chunk it must fetch so that the
// block matches swz128:
__device__ __forceinline__ int line_lane_chunk(int lane, int blk) {
  return (lane & 7) ^ (lane >> 3) ^ (blk & 1);
}

}  // namespace moe
