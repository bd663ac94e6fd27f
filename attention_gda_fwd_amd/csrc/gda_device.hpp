// gda_device.hpp - gfx950 device helpers shared by the libgda kernels.
//
// Lane layouts below were checked on gfx950 hardware:
//  * v_mfma_f32_16x16x32_bf16 (D[16x16] += A[16x32] B[32x16]): lane l holds
//    A[l%16][8*(l/16) .. +8], B[8*(l/16) .. +8][l%16], D[4*(l/16) .. +4][l%16].
//  * ds_read_b64_tr_b16: inside each group of 16 lanes, lane i receives element
//    i%4 of the 4-element row addressed by lane 4*j + i/4, for j = 0..3. So if
//    lanes 4j..4j+3 address the 16 consecutive columns c0..c0+15 of row r_j (4
//    columns each), lane i receives column c0+i of rows r_0..r_3: a transposed
//    read of a row-major tile.
//  * v_permlane16_swap / v_permlane32_swap called with the same register twice
//    return, in their two results, the values of lanes l and l^16 (l^32).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gda {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short shortx4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ floatx4 mfma_16x16x32(const bf16x8& a, const bf16x8& b,
                                                  const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// max / sum of a value over lanes l, l^16, l^32, l^48 (the four lane groups that
// hold one column of a 16x16 MFMA tile).
__device__ __forceinline__ float col_max4(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float col_sum4(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// fp32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Flags of the call options (the values of GDA_LAMBDA_LOGITS / GDA_GATE_LOGITS).
constexpr int kLambdaLogits = 1, kGateLogits = 2;

// 1 / (1 + e^-x) in fp32, for lambda and gate given as logits (a few ulp; 0 and 1
// at the extremes, never NaN for finite x).
__device__ __forceinline__ float sigmoid_f32(float x) { return 1.f / (1.f + __expf(-x)); }

// Read-only 16-byte global load.
__device__ __forceinline__ u32x4 ldg16(const void* p) { return *(const u32x4*)p; }

typedef __attribute__((address_space(3))) void lds_void;

// Direct global -> LDS copy of 16 bytes per lane from sbase + voff (sbase
// wave-uniform, voff a per-lane 32-bit byte offset): lane i's bytes land at
// lds_base + 16*i (lds_base wave-uniform). Written as inline asm so that the
// compiler does not track it as an LDS write: its conservative waits would
// otherwise hold every later transposed LDS read (which carries no alias
// information) until this copy completes. The instruction has no VGPR result;
// callers wait for it explicitly (s_waitcnt vmcnt(0) + barrier) before reading
// the destination, and any vmcnt wait the compiler emits for its own loads stays
// conservative because vector-memory loads complete in order.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, lds_void* lds_base) {
  const uint64_t a = (uint64_t)(uintptr_t)sbase;
  // readfirstlane returns a signed int: go through uint32_t so that the low
  // half is zero-extended, never sign-extended into the high half.
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint64_t base = ((uint64_t)hi << 32) | (uint64_t)lo;
  const uint32_t m0v = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(base), "s"(m0v)
               : "memory", "m0");
}

// The same copy with the LDS destination given as a wave-uniform LDS byte address.
__device__ __forceinline__ void dma16_lds(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  const uint64_t a = (uint64_t)(uintptr_t)sbase;
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint64_t base = ((uint64_t)hi << 32) | (uint64_t)lo;
  const uint32_t m0v = (uint32_t)__builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(base), "s"(m0v)
               : "memory", "m0");
}

// The same copy with the nontemporal hint: for data read once (a KV cache
// stream). Each instruction should cover whole 128-byte lines; a line read in
// two halves by two nontemporal instructions can be fetched twice.
__device__ __forceinline__ void dma16_lds_nt(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  const uint64_t a = (uint64_t)(uintptr_t)sbase;
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint64_t base = ((uint64_t)hi << 32) | (uint64_t)lo;
  const uint32_t m0v = (uint32_t)__builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               :
               : "v"(voff), "s"(base), "s"(m0v)
               : "memory", "m0");
}

// Completes the loads that wrote v here. The compiler waits for a load just
// before the first instruction that reads its result; when that first read sits
// inside a loop, the wait (a vmcnt count that ignores the direct-to-LDS copies it
// cannot see, and loads complete in order) runs every iteration and drains every
// copy in flight. An empty asm that reads v moves the wait here, once.
__device__ __forceinline__ void settle(const bf16x8& v) { asm volatile("" : : "v"(v)); }

// Wait until at most N of this wave's vector-memory operations are outstanding
// (they complete in order, so the oldest ones have landed). Also a compiler
// memory barrier: no LDS read of the landed data is moved above it.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

__device__ __forceinline__ u32x2 ldg8(const void* p) { return *(const u32x2*)p; }

}  // namespace gda
