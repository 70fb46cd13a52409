// Device helpers shared by the gfx950 kernels: vector types, MFMA wrappers,
// bf16 rounding and wave-level reductions.  Wavefronts are 64 lanes wide.
#pragma once
#include <type_traits>

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fdl {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// D(16x16) += A(16x32) * B(32x16), bf16 inputs, fp32 accumulate.
// Lane l supplies A row (l % 16) and B column (l % 16), each with the 8
// reduction elements of slot group (l / 16).  The result lane l holds is
// C[4 * (l / 16) + e][l % 16] in element e (e = 0..3).
__device__ __forceinline__ f32x4 mfma16(const u32x4 &a, const u32x4 &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// D(32x32) += A(32x16) * B(16x32).  Lane l supplies A row (l % 32) and B column
// (l % 32) with slot group (l / 32).  Element e of lane l holds
// C[8 * (e / 4) + 4 * (l / 32) + (e % 4)][l % 32].
__device__ __forceinline__ f32x16 mfma32(const u32x4 &a, const u32x4 &b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// fp32 -> bf16 bits, round to nearest even; NaN -> quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16_rne(lo) | ((uint32_t)f32_to_bf16_rne(hi) << 16);
}

// Two fp32 -> packed bf16 with the conversion instruction (v_cvt_pk_bf16_f32,
// round to nearest even); lo in the low half.
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

// Lane exchanges on the ALU instead of the LDS crossbar (`ds_bpermute`):
// DPP moves for partners inside a row of 16 lanes and the gfx950 permlane
// swaps across rows.  The whole wave must be active.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
// The value held by lane ^ 1, ^ 2, ^ 4, ^ 8.
__device__ __forceinline__ float lane_xor1(float v) { return dpp_mov<0xB1>(v); }  // quad_perm 1032
__device__ __forceinline__ float lane_xor2(float v) { return dpp_mov<0x4E>(v); }  // quad_perm 2301
__device__ __forceinline__ float lane_xor8(float v) { return dpp_mov<0x128>(v); }  // row_ror:8
__device__ __forceinline__ float lane_xor4(float v) {
  const float down = dpp_mov<0x124>(v), up = dpp_mov<0x12C>(v);  // row_ror:4 (lane - 4), :12 (+ 4)
  return (threadIdx.x & 4) ? down : up;
}
// Sum and maximum over lanes l, l ^ 16, l ^ 32, l ^ 48, the same in every one
// of them.  The sum adds (row 0 + row 1) + (row 2 + row 3) for every lane, as
// two xor-16 and xor-32 shuffle-and-add steps do (addition is commutative).
__device__ __forceinline__ float rows4_sum(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float s = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}
__device__ __forceinline__ float rows4_max(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float s = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS traffic,
// not for its outstanding global loads (which stay in flight across it).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// 2^x with the hardware approximation (v_exp_f32, about 1 ulp; denormal
// results flush to zero).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ u32x4 ld16(const void *p) {
  return *reinterpret_cast<const u32x4 *>(p);
}

// Raw buffer view of [base, base + bytes) (base and bytes wave-uniform): a
// 16-byte load at a byte offset at or past `bytes` returns zeros and touches
// no memory (the buffer range check); bytes = 0 makes every load such a load.
// Descriptor word 3 selects 32-bit raw elements (the gfx9-family layout).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_view(const void *base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 buffer_ld16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// Rings of LDS buffers filled by buffer loads that write LDS directly
// (buffer_load ... lds: lane l of a 16-byte load fills 16 bytes at the
// wave-uniform LDS address + 16 l).  Each buffer is its own __shared__ object
// and the rings are unrolled over compile-time buffer indices, so the
// compiler knows which buffer an LDS read touches and waits only for loads
// into that one.

// f(integral_constant<int, I>) for I = B .. E-1 (compile-time ring indices).
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// An index the optimiser cannot split, so that an LDS read's address stays
// one step off its buffer (the alias information the waits rely on).
__device__ __forceinline__ int opaque_index(int x) {
  asm("v_mov_b32 %0, %1" : "=v"(x) : "v"(x));
  return x;
}

// Workgroup barrier once this wave's ring loads up to the awaited buffer are
// done and its LDS accesses have completed (s_waitcnt encoding W): every
// wave's loads of that buffer are then in LDS, every wave has finished with
// the buffer the next loads refill, and LDS written before the barrier is
// visible after it.  The barrier instruction alone orders none of this; the
// compiler-only fences keep LDS accesses on their side of it.
template <int W>
__device__ __forceinline__ void ring_barrier() {
  __builtin_amdgcn_s_waitcnt(W);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// s_waitcnt operand: vector memory count <= n, LDS count 0, export count free.
constexpr int vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0070; }

__device__ __forceinline__ void st16(void *p, const u32x4 &v) {
  *reinterpret_cast<u32x4 *>(p) = v;
}

}  // namespace fdl
