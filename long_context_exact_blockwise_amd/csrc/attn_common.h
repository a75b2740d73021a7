// Device helpers shared by the bf16 attention kernels (forward and backward),
// gfx950.  Included by the kernel translation units only.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime.h>

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Row-major placement of 16-byte chunk c of key row `key` in a tile.  K rows
// are read 16 bytes per lane, 16 rows at a time at one chunk column: XOR the
// column with the row so those 16 reads hit 16 different 16-byte bank groups.
// V rows are read by the transpose loads 8 rows x 4 chunks at a time: XOR the
// 4-chunk group with the row so the 8 rows spread over the banks.
template <int D>
__device__ __forceinline__ int k_off(int key, int c) {
  const int cs = (D == 128) ? (c ^ (key & 15)) : (c ^ ((key >> 1) & 7));
  return key * (D * 2) + cs * 16;
}
template <int D>
__device__ __forceinline__ int v_off(int key, int c) {
  const int cs = (D == 128) ? (c ^ ((key & 3) << 2)) : (c ^ (((key >> 1) & 1) << 2));
  return key * (D * 2) + cs * 16;
}

// One placement for both read kinds: chunk c of row r goes to chunk
// c ^ u(r), u a bit permutation of the row's low bits (D = 128: u = 4 (r & 3)
// + ((r >> 2) & 3); D = 64: u = 4 ((r >> 1) & 1) + ((r >> 2) & 3)).  Sixteen
// consecutive rows read at one chunk column (16-byte row reads) and the 4
// rows x 4 chunks a transpose read takes per half-wave both land on distinct
// banks of the 64.  u depends on r mod 16 only, so row offsets that are
// multiples of 16 are instruction immediates.
template <int D>
__device__ __forceinline__ int u_swz(int r) {
  return D == 128 ? (4 * (r & 3) + ((r >> 2) & 3)) : (4 * ((r >> 1) & 1) + ((r >> 2) & 3));
}
template <int D>
__device__ __forceinline__ int u_off(int row, int c) {
  return row * (D * 2) + (c ^ u_swz<D>(row)) * 16;
}

__device__ __forceinline__ float pair_max(float x) {
  // max(x[lane], x[lane ^ 32]) on every lane
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Direct global->LDS copies (global_load_lds_dword / _dwordx4).  Base
// pointers and LDS addresses are wave-uniform.  The copies are issued from
// inline assembly so that the compiler does not track them: its own tracking
// would wait for every copy in flight before the next LDS read of any buffer,
// which serialises the prefetch with the compute.  The kernel waits for its
// copies itself (s_waitcnt vmcnt) before the barrier that publishes a buffer.
//
// Every block rewrites its base SGPRs with a scalar self-copy (s_mov_b64 s,
// s) before the loads: a VMEM instruction may read an SGPR only five wait
// states after a VALU instruction wrote it (the base comes from
// v_readfirstlane, and a spilled SGPR is restored by v_readlane), the
// compiler inserts no wait states for instructions inside inline assembly,
// and an SGPR last written by a scalar instruction needs none.  Without it
// the load can take a stale base address.  The copy also gives the one wait
// state a load needs after M0 is written.

// A wave-uniform pointer as a 64-bit scalar value (readfirstlane returns
// int: widen through uint32_t, never by sign extension).
__device__ __forceinline__ uint64_t sbase(const char* p) {
  const uint64_t bv = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)bv);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(bv >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// 16 bytes per lane (global_load_lds_dwordx4): lane i's bytes, from base +
// voff, land at LDS byte lds_addr + 16 i.
__device__ __forceinline__ void lds_dma16(const char* base, uint32_t voff, uint32_t lds_addr) {
  uint64_t bs = sbase(base);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %[sv], m0\n\t"
      "s_mov_b32 m0, %[m0]\n\t"
      "s_mov_b64 %[bs], %[bs]\n\t"
      "global_load_lds_dwordx4 %[o0], %[bs]\n\t"
      "s_mov_b32 m0, %[sv]"
      : [sv] "=&s"(saved), [bs] "+s"(bs)
      : [o0] "v"(voff), [m0] "s"(__builtin_amdgcn_readfirstlane(lds_addr))
      : "memory");
}

// The same for 4 bytes per lane (global_load_lds_dword): lane i's dword lands
// at LDS byte lds_addr + 4 i.
__device__ __forceinline__ void lds_dma4(const char* base, uint32_t voff, uint32_t lds_addr) {
  uint64_t bs = sbase(base);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %[sv], m0\n\t"
      "s_mov_b32 m0, %[m0]\n\t"
      "s_mov_b64 %[bs], %[bs]\n\t"
      "global_load_lds_dword %[o0], %[bs]\n\t"
      "s_mov_b32 m0, %[sv]"
      : [sv] "=&s"(saved), [bs] "+s"(bs)
      : [o0] "v"(voff), [m0] "s"(__builtin_amdgcn_readfirstlane(lds_addr))
      : "memory");
}

// Four direct global->LDS copies of 16 bytes per lane under one M0: copy j
// lands lane i's bytes at LDS byte lds_addr + 1 KiB j + 16 i from global
// base + off[j] + 1 KiB j (the instruction offset moves both addresses, so
// off[j] is the lane's global offset with 1 KiB j taken out).  base and
// lds_addr are wave-uniform.
__device__ __forceinline__ void lds_dma_x4(const char* base, const uint32_t (&off)[4], uint32_t lds_addr) {
  uint64_t bs = sbase(base);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %[sv], m0\n\t"
      "s_mov_b32 m0, %[m0]\n\t"
      "s_mov_b64 %[bs], %[bs]\n\t"
      "global_load_lds_dwordx4 %[o0], %[bs]\n\t"
      "global_load_lds_dwordx4 %[o1], %[bs] offset:1024\n\t"
      "global_load_lds_dwordx4 %[o2], %[bs] offset:2048\n\t"
      "global_load_lds_dwordx4 %[o3], %[bs] offset:3072\n\t"
      "s_mov_b32 m0, %[sv]"
      : [sv] "=&s"(saved), [bs] "+s"(bs)
      : [o0] "v"(off[0]), [o1] "v"(off[1]), [o2] "v"(off[2]), [o3] "v"(off[3]),
        [m0] "s"(__builtin_amdgcn_readfirstlane(lds_addr))
      : "memory");
}

// The same with one 4-byte copy first: lane i's dword lands at lds_addr + 4 i
// from global dbase + doff (256 bytes for the wave), then copy j lands at
// lds_addr + 256 + 1 KiB j from base + off[j] + 256 + 1 KiB j.
__device__ __forceinline__ void lds_dma_1x4(const char* dbase, uint32_t doff, const char* base, const uint32_t (&off)[4],
                                            uint32_t lds_addr) {
  uint64_t ds = sbase(dbase), bs = sbase(base);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %[sv], m0\n\t"
      "s_mov_b32 m0, %[m0]\n\t"
      "s_mov_b64 %[ds], %[ds]\n\t"
      "s_mov_b64 %[bs], %[bs]\n\t"
      "global_load_lds_dword %[od], %[ds]\n\t"
      "global_load_lds_dwordx4 %[o0], %[bs] offset:256\n\t"
      "global_load_lds_dwordx4 %[o1], %[bs] offset:1280\n\t"
      "global_load_lds_dwordx4 %[o2], %[bs] offset:2304\n\t"
      "global_load_lds_dwordx4 %[o3], %[bs] offset:3328\n\t"
      "s_mov_b32 m0, %[sv]"
      : [sv] "=&s"(saved), [ds] "+s"(ds), [bs] "+s"(bs)
      : [o0] "v"(off[0]), [o1] "v"(off[1]), [o2] "v"(off[2]), [o3] "v"(off[3]), [od] "v"(doff),
        [m0] "s"(__builtin_amdgcn_readfirstlane(lds_addr))
      : "memory");
}
// Two-copy forms (D = 64: two 1 KiB chunks per wave).
__device__ __forceinline__ void lds_dma_x2(const char* base, const uint32_t (&off)[4], uint32_t lds_addr) {
  uint64_t bs = sbase(base);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %[sv], m0\n\t"
      "s_mov_b32 m0, %[m0]\n\t"
      "s_mov_b64 %[bs], %[bs]\n\t"
      "global_load_lds_dwordx4 %[o0], %[bs]\n\t"
      "global_load_lds_dwordx4 %[o1], %[bs] offset:1024\n\t"
      "s_mov_b32 m0, %[sv]"
      : [sv] "=&s"(saved), [bs] "+s"(bs)
      : [o0] "v"(off[0]), [o1] "v"(off[1]), [m0] "s"(__builtin_amdgcn_readfirstlane(lds_addr))
      : "memory");
}
__device__ __forceinline__ void lds_dma_1x2(const char* dbase, uint32_t doff, const char* base, const uint32_t (&off)[4],
                                            uint32_t lds_addr) {
  uint64_t ds = sbase(dbase), bs = sbase(base);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %[sv], m0\n\t"
      "s_mov_b32 m0, %[m0]\n\t"
      "s_mov_b64 %[ds], %[ds]\n\t"
      "s_mov_b64 %[bs], %[bs]\n\t"
      "global_load_lds_dword %[od], %[ds]\n\t"
      "global_load_lds_dwordx4 %[o0], %[bs] offset:256\n\t"
      "global_load_lds_dwordx4 %[o1], %[bs] offset:1280\n\t"
      "s_mov_b32 m0, %[sv]"
      : [sv] "=&s"(saved), [ds] "+s"(ds), [bs] "+s"(bs)
      : [o0] "v"(off[0]), [o1] "v"(off[1]), [od] "v"(doff), [m0] "s"(__builtin_amdgcn_readfirstlane(lds_addr))
      : "memory");
}

// LDS byte address of a generic pointer into the dynamic LDS array.
__device__ __forceinline__ uint32_t lds_addr_of(const char* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// s_waitcnt lgkmcnt(0) with the other counters left alone: this wave's LDS
// writes have landed (before a barrier that hands them to other waves).
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier without a memory fence: every wait a barrier needs here
// is explicit (the copies' vmcnt; LDS reads are consumed before the barrier).
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace
}  // namespace ra
