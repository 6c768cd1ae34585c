// Shared device helpers for the gfx950 attention kernels: vector types, bf16
// packing, wave64 lane exchanges through DPP, and the launch-side status codes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.hpp"

namespace pkva {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

// Non-temporal store for results that a later kernel reads: the line streams
// to memory now instead of staying dirty in the caches, where the next kernel,
// often a bandwidth-bound decode, would pay for its write-back.
template <typename V>
__device__ __forceinline__ void store_nt(V* p, V v) {
  __builtin_nontemporal_store(v, p);
}

// Non-temporal 16-byte load for data read exactly once (streamed K/V rows).
__device__ __forceinline__ uint4 load_nt16(const void* p) {
  const u32x4_t w = __builtin_nontemporal_load((const u32x4_t*)p);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// ------------------------------------------------ global -> LDS copies
// s_waitcnt vmcnt(N) alone (gfx9 encoding: vmcnt[3:0], expcnt[6:4],
// lgkmcnt[11:8], vmcnt[5:4] in [15:14]; the others at their maximum).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// One 16-byte-per-lane DMA copy global -> LDS from a uniform base plus a
// per-lane 32-bit offset: lane i's 16 bytes land at LDS byte lds + 16 * i.
// Issued as inline assembly so the compiler does not track it: it would
// otherwise wait for every copy in flight before each LDS read it cannot
// prove disjoint. Completion is awaited with counted vmcnt waits.
// The instruction takes the wave's LDS base in M0, a register the compiler
// reserves: the statement saves M0 in a scratch SGPR, sets it (one wait
// state before the copy reads it), and puts the saved value back (one wait
// state before anything after the statement may read it), so the compiler's
// own view of M0 stays true.
// The base and the LDS address are uniform by construction; passing them
// through readfirstlane lets the compiler prove it, so they always get the
// scalar registers the instruction needs.
__device__ __forceinline__ void dma16(const void* base, uint32_t off, uint32_t lds) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const uint64_t sb = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t sl = __builtin_amdgcn_readfirstlane(lds);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0"
      : "=&s"(saved)
      : "v"(off), "s"((const void*)(uintptr_t)sb), "s"(sl)
      : "memory");
}

// The same copy from a per-lane 64-bit address (rows gathered from anywhere
// in a pool that may exceed 4 GiB).
__device__ __forceinline__ void dma16_addr(const void* addr, uint32_t lds) {
  const uint32_t sl = __builtin_amdgcn_readfirstlane(lds);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0"
      : "=&s"(saved)
      : "v"(addr), "s"(sl)
      : "memory");
}

// ---------------------------------------------------------------- bf16 bits
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> two bf16 (round to nearest even) packed low|high.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

// Dot product of two packed bf16 pairs, accumulated into c in fp32.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// ------------------------------------------------------- lane exchanges
// Value of the partner lane whose index differs from ours in bit BIT (and
// possibly in lower bits). BIT 0..3 stay inside a 16-lane DPP row:
//   bit 0: quad_perm [1,0,3,2]   (lane ^ 1)
//   bit 1: quad_perm [2,3,0,1]   (lane ^ 2)
//   bit 2: row_half_mirror       (lane ^ 7 inside each 8-lane half row)
//   bit 3: row_mirror            (lane ^ 15 inside each 16-lane row)
// The masks {1, 2, 7, 15} are linearly independent over GF(2), so a
// butterfly over them covers every lane of a 16-lane group exactly once.
// Bits 4 and 5 use a cross-row permute (lane ^ 16, lane ^ 32).
template <int BIT>
__device__ __forceinline__ float xchg(float x) {
  static_assert(BIT >= 0 && BIT <= 5, "lane bit out of range");
  const int xi = __float_as_int(x);
  if constexpr (BIT == 0) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, xi, 0xB1, 0xF, 0xF, false));
  } else if constexpr (BIT == 1) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, xi, 0x4E, 0xF, 0xF, false));
  } else if constexpr (BIT == 2) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, xi, 0x141, 0xF, 0xF, false));
  } else if constexpr (BIT == 3) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, xi, 0x140, 0xF, 0xF, false));
  } else if constexpr (BIT == 4) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute((int)((threadIdx.x ^ 16u) << 2), xi));
  } else {
    return __int_as_float(__builtin_amdgcn_ds_bpermute((int)((threadIdx.x ^ 32u) << 2), xi));
  }
}

template <int N>
struct Log2 { static constexpr int value = 1 + Log2<N / 2>::value; };
template <>
struct Log2<1> { static constexpr int value = 0; };

// Reduce-scatter of N partial sums across an aligned group of LG lanes.
// On return lane `li` (index inside the group) holds in v[0..NV) the full
// group sums of heads  (li / max(1, LG/N)) * NV + i,  NV = max(1, N/LG).
template <int N, int BIT, int n>
__device__ __forceinline__ void reduce_scatter_step(float (&v)[N], int li) {
  if constexpr (BIT >= 0) {
    if constexpr (n > 1) {
      constexpr int half = n / 2;
      const bool up = (li >> BIT) & 1;
#pragma unroll
      for (int i = 0; i < half; ++i) {
        const float send = up ? v[i] : v[i + half];
        const float keep = up ? v[i + half] : v[i];
        v[i] = keep + xchg<BIT>(send);
      }
      reduce_scatter_step<N, BIT - 1, half>(v, li);
    } else {
      v[0] += xchg<BIT>(v[0]);
      reduce_scatter_step<N, BIT - 1, 1>(v, li);
    }
  }
}

template <int LG, int N>
__device__ __forceinline__ void reduce_scatter(float (&v)[N], int li) {
  reduce_scatter_step<N, Log2<LG>::value - 1, N>(v, li);
}

// Sum over an aligned group of LG lanes (LG <= 16); every lane gets the same sum.
template <int LG>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (LG >= 16) x += xchg<3>(x);
  if constexpr (LG >= 8) x += xchg<2>(x);
  if constexpr (LG >= 4) x += xchg<1>(x);
  if constexpr (LG >= 2) x += xchg<0>(x);
  return x;
}

// Wave64-wide max and sum (every lane gets the result).
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, xchg<0>(x));
  x = fmaxf(x, xchg<1>(x));
  x = fmaxf(x, xchg<2>(x));
  x = fmaxf(x, xchg<3>(x));
  x = fmaxf(x, xchg<4>(x));
  x = fmaxf(x, xchg<5>(x));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
  x += xchg<0>(x);
  x += xchg<1>(x);
  x += xchg<2>(x);
  x += xchg<3>(x);
  x += xchg<4>(x);
  x += xchg<5>(x);
  return x;
}

}  // namespace pkva
