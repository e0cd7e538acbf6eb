// common.hpp — device-side building blocks for the gfx950 attention kernels.
//
// Lane layouts used here were measured on MI355X (gfx950) with an in-bounds probe of the
// compiler builtins, and are restated where used:
//
//  v_mfma_f32_32x32x16_bf16  A[32x16], B[16x32], D[32x32]
//    A: lane l holds row m = l%32, k = 8*(l/32) + i (i = 0..7)
//    B: lane l holds col n = l%32, k = 8*(l/32) + i
//    D: lane l holds col n = l%32, rows m = 8*(j/4) + 4*(l/32) + j%4 (j = 0..15)
//  v_mfma_f32_16x16x32_bf16  A[16x32], B[32x16], D[16x16]
//    A: lane l holds row m = l%16, k = 8*(l/16) + i
//    B: lane l holds col n = l%16, k = 8*(l/16) + i
//    D: lane l holds col n = l%16, rows m = 4*(l/16) + j (j = 0..3)
//  ds_read_b64_tr_b16: inside each group of 16 lanes, lane i receives in slot j the element
//    (i % 4) of the 8-byte row addressed by lane 4*j + i/4 of the same group.
//  global_load_lds_dwordx4: lane l's 16 bytes land at LDS (M0 base) + 16*l.
//
// Because a contraction is a sum over k, any permutation of the k index is allowed as long
// as both operands use the same one; the kernels exploit that to feed the score accumulator
// registers straight back into the P·V product without a trip through LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint16_t bf16_t;  // storage type of bf16 in memory

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;
typedef __attribute__((address_space(1))) void gbl_void_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16-byte global load reinterpreted as 8 bf16.
__device__ __forceinline__ bf16x8 load_bf16x8(const bf16_t* p) {
  uint4 u = *reinterpret_cast<const uint4*>(p);
  return __builtin_bit_cast(bf16x8, u);
}
// Query operand load with a sign mask XORed into every bf16 (0x80008000 negates the eight
// values, 0 leaves them).
__device__ __forceinline__ bf16x8 load_q_bf16x8(const bf16_t* p, uint32_t sign) {
  uint4 u = *reinterpret_cast<const uint4*>(p);
  u.x ^= sign;
  u.y ^= sign;
  u.z ^= sign;
  u.w ^= sign;
  return __builtin_bit_cast(bf16x8, u);
}
__device__ __forceinline__ bf16x8 zero_bf16x8() {
  return __builtin_bit_cast(bf16x8, make_uint4(0u, 0u, 0u, 0u));
}
// 16-byte LDS read (ds_read_b128).
__device__ __forceinline__ bf16x8 lds_read_bf16x8(const char* lds_base, uint32_t byte_off) {
  uint4 u = *reinterpret_cast<const uint4*>(lds_base + byte_off);
  return __builtin_bit_cast(bf16x8, u);
}
// Two transposed 8-byte LDS reads -> one 8-element MFMA operand.
__device__ __forceinline__ bf16x8 lds_read_tr_pair(const char* lds_base, uint32_t off_lo,
                                                   uint32_t off_hi) {
  i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(lds_base + off_lo));
  i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(lds_base + off_hi));
  uint2 ulo = __builtin_bit_cast(uint2, lo);
  uint2 uhi = __builtin_bit_cast(uint2, hi);
  return __builtin_bit_cast(bf16x8, make_uint4(ulo.x, ulo.y, uhi.x, uhi.y));
}

// ------------------------------------------------------------------------------------------
// LDS addressed by 32-bit byte addresses. The compiler folds a compile-time offset of up to
// 64 KiB into the instruction's offset field, so reads at (base register + constant) need no
// address arithmetic even when the LDS footprint exceeds 64 KiB.
// ------------------------------------------------------------------------------------------
typedef __attribute__((address_space(3))) uint4 lds_uint4_t;

__device__ __forceinline__ uint32_t lds_addr(const void* shared_ptr) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)shared_ptr;
}
__device__ __forceinline__ bf16x8 lds_read_b128_at(uint32_t addr) {
  return __builtin_bit_cast(bf16x8, *(const lds_uint4_t*)(uintptr_t)addr);
}
__device__ __forceinline__ bf16x8 lds_read_tr_pair_at(uint32_t lo, uint32_t hi) {
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(uintptr_t)lo);
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(uintptr_t)hi);
  const uint2 ua = __builtin_bit_cast(uint2, a);
  const uint2 ub = __builtin_bit_cast(uint2, b);
  return __builtin_bit_cast(bf16x8, make_uint4(ua.x, ua.y, ub.x, ub.y));
}

// Asynchronous 16-byte-per-lane global -> LDS copy written as one instruction with a scalar
// base: lane l reads sbase + voff (bytes) and its 16 bytes land at LDS address lds + 16*l
// (`lds` is wave-uniform and goes through M0). The compiler does not see this LDS write, so it
// adds no waits of its own before later LDS reads: the caller orders them with an explicit
// vmcnt wait and a workgroup barrier.
__device__ __forceinline__ void dma16_sbase(const void* sbase, uint32_t voff, uint32_t lds) {
  // The base and the LDS address are wave-uniform: pin them to scalar registers. readfirstlane
  // returns a signed int, so each half is zero-extended explicitly.
  const uint64_t p = (uint64_t)(uintptr_t)sbase;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  const uint64_t ps = ((uint64_t)hi << 32) | (uint64_t)lo;
  // The compiler's hazard checks do not look inside inline assembly. s_nop 4 provides the wait
  // states this load needs after the instructions that produce its operands: 5 after a VALU
  // write of an SGPR it reads, 1 after an SALU write of M0.
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(ps),
               "{m0}"((uint32_t)__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

// The same copy from a per-lane 64-bit source address (rows gathered from anywhere).
__device__ __forceinline__ void dma16_vaddr(const void* gsrc, uint32_t lds) {
  // s_nop 4: the wait states after the SALU write of M0 (see dma16_sbase).
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gsrc),
               "{m0}"((uint32_t)__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

// 4-byte-per-lane variant: lane l's word lands at LDS address lds + 4*l.
__device__ __forceinline__ void dma4_vaddr(const void* gsrc, uint32_t lds) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dword %0, off" ::"v"(gsrc),
               "{m0}"((uint32_t)__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

// Waits until every vector memory instruction of this wave (copies included) has completed.
__device__ __forceinline__ void wait_dma_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 pair, round-to-nearest-even (one gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float xor_shuffle(float v, int mask) { return __shfl_xor(v, mask, 64); }

template <int N>
using icn = std::integral_constant<int, N>;

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(icn<I>{});
    static_for<I + 1, N>(f);
  }
}

__device__ __forceinline__ float max3f(float a, float b, float c) {
  return fmaxf(fmaxf(a, b), c);
}

// Value of v held by lane l^32 (one v_permlane32_swap).
__device__ __forceinline__ float other_half(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const uint32_t lo = r[0], hi = r[1];
  // lanes 0..31: r[1] holds lane l+32's value; lanes 32..63: r[0] holds lane l-32's value
  return __builtin_bit_cast(float, ((threadIdx.x & 63) < 32) ? hi : lo);
}
__device__ __forceinline__ float max_halves(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const uint32_t lo = r[0], hi = r[1];
  return fmaxf(__builtin_bit_cast(float, lo), __builtin_bit_cast(float, hi));
}

// Maximum-free softmax check. A unit's weights are computed as exp2(x - mu) against a row's
// reference mu, with no maximum taken; the unit is accepted when the row's running fp32 weight
// sum afterwards lies in (0, 2^64]: positive (the row has a reference) and small enough that no
// weight, nor |O| <= (weight sum) * max|V| for any V below 2^60, comes near fp32 overflow. The
// compare is on the bits, so 0, inf and NaN all fail.
constexpr uint32_t kSumLimitBits = 0x5f800000u;  // 2^64
__device__ __forceinline__ bool sum_ok(float s) {
  return __builtin_bit_cast(uint32_t, s) - 1u < kSumLimitBits;
}

// Sum of the two bf16 values of a packed pair, added to c (one v_dot2c_f32_bf16).
__device__ __forceinline__ float add_bf16_pair(uint32_t pair, float c) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t p = __builtin_bit_cast(bf16x2_t, pair);
  const bf16x2_t one = __builtin_bit_cast(bf16x2_t, 0x3f803f80u);
  return __builtin_amdgcn_fdot2_f32_bf16(p, one, c, false);
}

// ------------------------------------------------------------------------------------------
// Swizzled LDS tile layout. A tile holds ROWS rows of D bf16 (CPR = D/8 chunks of 16 bytes
// per row). Row r's chunk c is stored in 16-byte slot r*CPR + (c ^ swz(r)); the XOR only
// touches the low bits of c, so it stays inside the row. The swizzle makes both readers
// conflict-free on the 64 x 4-byte LDS banks: the MFMA K-operand read (16 consecutive rows,
// one chunk each) and the transposed V read (4..16 rows x 2..4 chunks per instruction).
// ------------------------------------------------------------------------------------------
template <int D>
struct Swz;
template <>
struct Swz<64> {  // 8 chunks per row
  static __device__ __forceinline__ uint32_t f(uint32_t r) {
    return (((r >> 1) & 1u) << 2) | ((r >> 2) & 3u);
  }
};
template <>
struct Swz<128> {  // 16 chunks per row
  static __device__ __forceinline__ uint32_t f(uint32_t r) { return ((r & 3u) << 2) | ((r >> 2) & 3u); }
};
template <>
struct Swz<576> {  // 72 chunks per row: XOR inside aligned groups of 8 chunks
  static __device__ __forceinline__ uint32_t f(uint32_t r) { return (r >> 1) & 7u; }
};

template <int D>
__device__ __forceinline__ uint32_t slot_of(uint32_t r, uint32_t c) {
  return r * (D / 8) + (c ^ Swz<D>::f(r));
}
// byte offset of element (r, e) of a D-wide tile (e must stay inside one 16-byte chunk group)
template <int D>
__device__ __forceinline__ uint32_t elem_off(uint32_t r, uint32_t e) {
  return slot_of<D>(r, e >> 3) * 16u + (e & 7u) * 2u;
}

}  // namespace attn
