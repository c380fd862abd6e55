// Device helpers shared by the NSA kernels (gfx950 / CDNA4, wave64).
//
// MFMA tile conventions used throughout (v_mfma_f32_16x16x32_bf16):
//   lane l, lg = l / 16 (k-slot group), lr = l % 16
//   A operand (16 x 32): row lr, eight k-slots of group lg
//   B operand (32 x 16): column lr, the same eight k-slots of group lg
//   D (16 x 16 fp32):    element i (0..3) is row 4*lg + i, column lr
// Only the pairing of A and B k-slots matters for the product, so the kernels
// choose whichever key/channel order makes the global loads contiguous.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nsa_internal.hpp"

namespace nsa {

// Profiling hook: thread 0 records the constant 100 MHz clock at point `slot`
// of this workgroup (clk is null unless the caller asked for a phase clock).
__device__ __forceinline__ void clk_stamp(uint64_t* clk, int slot) {
  if (clk != nullptr && threadIdx.x == 0) clk[(size_t)blockIdx.x * kClkSlots + slot] = __builtin_amdgcn_s_memrealtime();
}

typedef short bf16x8_t __attribute__((__vector_size__(8 * sizeof(short))));
typedef float f32x4_t __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t u32x4_t __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef uint32_t u32x2_t __attribute__((__vector_size__(2 * sizeof(uint32_t))));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWave = 64;

__device__ __forceinline__ f32x4_t mfma_bf16(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

typedef short bf16x4_t __attribute__((__vector_size__(4 * sizeof(short))));

// v_mfma_f32_16x16x16_bf16: A row lr / B column lr hold k-slots 4*lg .. 4*lg+3
// (two packed dwords); D as above.  Its B layout is the D layout of the 16x16x32
// product, so a logit tile feeds it directly.
__device__ __forceinline__ f32x4_t mfma16_bf16(const u32x2_t& a, const u32x2_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4_t, a),
                                                   __builtin_bit_cast(bf16x4_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 pair (lo in bits 0..15), round to nearest even: one
// v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}
// fp32 -> bf16 bits, round to nearest even.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return pack_bf16x2(f, 0.f) & 0xFFFFu; }

// Global loads of 16 / 8 bytes.  Every caller proves the address in bounds
// before calling; out-of-range rows are replaced by zeros at the call site.
__device__ __forceinline__ u32x4_t ld16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}
__device__ __forceinline__ u32x2_t ld8(const uint16_t* p) {
  return *reinterpret_cast<const u32x2_t*>(p);
}

// Gate network (a sigmoid of one linear layer of a query head): the part of the
// dot product of the bf16 query row q and weight row w (both DK long) that lane
// part `part` of four covers, elements [part*DK/4, (part+1)*DK/4).  The caller
// adds the four parts in a fixed order.
template <int DK>
__device__ __forceinline__ float gate_dot_quarter(const uint16_t* q, const uint16_t* w, int part) {
  constexpr int E = DK / 4;
  static_assert(E % 8 == 0, "a quarter of the row must be whole 16-byte loads");
  u32x4_t a[E / 8], c[E / 8];
#pragma unroll
  for (int i = 0; i < E / 8; ++i) {
    a[i] = *reinterpret_cast<const u32x4_t*>(q + part * E + 8 * i);
    c[i] = *reinterpret_cast<const u32x4_t*>(w + part * E + 8 * i);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < E / 8; ++i)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      s = fmaf(__uint_as_float(a[i][u] << 16), __uint_as_float(c[i][u] << 16), s);
      s = fmaf(__uint_as_float(a[i][u] & 0xFFFF0000u), __uint_as_float(c[i][u] & 0xFFFF0000u), s);
    }
  return s;
}
// Logistic sigmoid 1 / (1 + e^-z) with the hardware base-2 exponential.
__device__ __forceinline__ float gate_sigmoid(float z) {
  return 1.0f / (1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * z));
}

// Cross-lane reductions over the four lane groups (lanes lr, lr+16, lr+32, lr+48).
__device__ __forceinline__ float max_over_groups(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}
__device__ __forceinline__ float sum_over_groups(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// The same reductions with the gfx950 lane-swap instructions (no LDS round trip):
// permlane16_swap exchanges lane groups 0<->1 and 2<->3, permlane32_swap the two
// wave halves; the element-wise combination of the two results is the reduction.
__device__ __forceinline__ float max_over_groups_swap(float v) {
  const uint32_t x = __float_as_uint(v);
  auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t y = __float_as_uint(v);
  auto b = __builtin_amdgcn_permlane32_swap(y, y, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_over_groups_swap(float v) {
  const uint32_t x = __float_as_uint(v);
  auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t y = __float_as_uint(v);
  auto b = __builtin_amdgcn_permlane32_swap(y, y, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Sum over the 16 lanes of each lane group (a DPP row); the total lands in the
// group's last lane (lanes 15, 31, 47, 63).  Lanes whose DPP source lies outside
// the row read 0.
__device__ __forceinline__ float row_sum_to_last(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xF, 0xF, false));  // row_shr:1
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xF, 0xF, false));  // row_shr:2
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xF, 0xF, false));  // row_shr:4
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xF, 0xF, false));  // row_shr:8
  return v;
}

// Wave-wide direct global -> LDS copy of 64 x 16 bytes: lane l reads 16 bytes at
// `src` (its own address) and LDS receives them at lds_base + 16 * l.  lds_base
// must be the same for every lane.  Completion is tracked by vmcnt only.
//
// Written as inline asm on purpose: the compiler then does not see an LDS store
// here, so it does not drain every outstanding copy (vmcnt(0)) before each later
// LDS read or barrier -- which would serialise the copy of the next tiles with
// the compute on the current one.  The kernels order the copies themselves:
// wait_vmem_le<N>() for their own copies, then lds_barrier() for everyone's.
// The instruction has no register results; m0 (the LDS base) needs one wait
// state after it is written.
__device__ __forceinline__ void copy16_to_lds(const void* src, void* lds_base) {
  const uint32_t lds = (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)(uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds_base);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds)
               : "memory", "m0");
}
// The same copy with a wave-uniform base address and this lane's 32-bit byte
// offset (the scalar-base form of the instruction: no per-lane 64-bit address
// arithmetic).
__device__ __forceinline__ void copy16_to_lds_sb(const void* base, uint32_t voff, void* lds_base) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const uint64_t sb = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32)) << 32) |
                      (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint32_t lds = (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)(uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds_base);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sb), "s"(lds)
               : "memory", "m0");
}
// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr_of(const void* shared_ptr) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)shared_ptr;
}
// The two copies above with the LDS destination given as a wave-uniform LDS byte
// address (lane l's 16 bytes land at lds_addr + 16 * l): no generic-to-LDS
// pointer conversion per copy.
__device__ __forceinline__ void copy16_to_lds_at(const void* src, uint32_t lds_addr) {
  const uint32_t lds = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void copy16_sb_at(const void* base, uint32_t voff, uint32_t lds_addr) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const uint64_t sb = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32)) << 32) |
                      (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint32_t lds = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sb), "s"(lds)
               : "memory", "m0");
}
// Workgroup barrier that is also a compiler memory barrier, without the implied
// wait for outstanding vector-memory operations of __syncthreads().  LDS
// operations issued before it by the compiler are complete once their results
// were consumed; callers wait for their own LDS copies first.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// Wait until at most N of this wave's vector-memory operations are outstanding
// (they complete in issue order), leaving the export and LDS counters alone.
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | 0x0070 | 0x0F00 | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_vmem() { wait_vmem_le<0>(); }

// Select 16-bit half `h` (0 low, 1 high) of a and b and pack as (a_h | b_h << 16):
// one v_perm_b32 (byte selectors 0-3 pick from the second operand, 4-7 from the first).
__device__ __forceinline__ uint32_t pack_halves(uint32_t a, uint32_t b, int h) {
  return __builtin_amdgcn_perm(b, a, h ? 0x07060302u : 0x05040100u);
}

// Exclusive prefix sum over the NT threads of a block (NT/64 waves).  `scratch`
// holds at least NT/64 ints in LDS.  Returns the exclusive prefix; *total gets the sum.
template <int NT>
__device__ __forceinline__ int block_scan(int v, int* scratch, int* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) scratch[wave] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    int s = scratch[w];
    if (w < wave) base += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

}  // namespace nsa
