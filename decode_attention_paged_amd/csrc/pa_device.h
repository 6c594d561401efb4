// Device helpers shared by the paged decode-attention kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// ---------------------------------------------------------------- loads
// 128-bit global load; the pointer must be 16-byte aligned.
// 16 KiB of zeros in global memory: the source of the loads a kernel issues
// for a tile past the end of its split, so that every loop iteration issues
// the same loads (the compiler's wait counts then stay exact); they hit L2.
static __device__ __attribute__((aligned(16))) uint32_t g_zero_tile[4096] = {};

__device__ __forceinline__ u32x4 ld128(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// 128-bit streaming load for data read exactly once (KV tiles): the
// non-temporal policy keeps it from displacing reusable lines and measured
// ~13% more read bandwidth from HBM on MI355X than the default policy.
__device__ __forceinline__ u32x4 ld128_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
// 64-bit streaming load (8-byte aligned pointer), same policy.
__device__ __forceinline__ u32x2 ld64_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
}

// Two FP8 E4M3 codes (bytes 0-1 of w, or 2-3 with HI) as a bfloat16 pair:
// exact, every E4M3 value is a bfloat16 value.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
// Eight FP8 codes (two words) as eight bfloat16 values, in order.
__device__ __forceinline__ u32x4 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  return u32x4{fp8x2_to_bf16x2<false>(w0), fp8x2_to_bf16x2<true>(w0), fp8x2_to_bf16x2<false>(w1),
               fp8x2_to_bf16x2<true>(w1)};
}

// Reinterpret a 32-bit lane value as float.  Takes the value (not a vector
// element lvalue): bit-casting an ext_vector element directly reads element 0.
__device__ __forceinline__ float as_f32(uint32_t u) { return __builtin_bit_cast(float, u); }

// Wait until every vector-memory access this thread issued has completed
// (s_waitcnt vmcnt(0); gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8]
// | vmcnt_hi[15:14], the other counters left at their maxima).  The signal
// fences keep the compiler from moving memory accesses across the wait.
__device__ __forceinline__ void wait_stores_done() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16lo(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float bf16hi(uint32_t u) { return __builtin_bit_cast(float, u & 0xffff0000u); }

// Two floats -> packed bf16 pair (round to nearest even, v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2 r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint16_t to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// bf16x2 . bf16x2 + acc in float (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                        __builtin_bit_cast(bf16x2, b), acc, false);
}

// ---------------------------------------------------------------- math
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// ---------------------------------------------------------------- cross-lane
// DPP move within rows of 16 lanes; bound_ctrl keeps every lane written.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                                0xf, 0xf, true));
}
constexpr int kDppQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;
constexpr int kDppRowHalfMirror = 0x141;

// Sum over each aligned group of N lanes (N = 8, 16); every lane gets the sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 8 || N == 16, "group size");
  if constexpr (N == 16) {
    x += dpp<kDppRowRor8>(x);
    x += dpp<kDppRowRor4>(x);
  } else {
    x += dpp<kDppRowHalfMirror>(x);
  }
  x += dpp<kDppQuadXor2>(x);
  x += dpp<kDppQuadXor1>(x);
  return x;
}

__device__ __forceinline__ float shfl_xor(float x, int m) { return __shfl_xor(x, m, 64); }

// permlane16_swap(x, x) hands every lane both x[l & ~16] and x[l | 16];
// permlane32_swap(x, x) both x[l & ~32] and x[l | 32] (v_permlane*_swap_b32,
// gfx950).  Combining the pair gives an all-reduce over lanes l, l^16 (l^32)
// without going through LDS.
__device__ __forceinline__ float max_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x),
                                            false, false);
  return fmaxf(__builtin_bit_cast(float, (int)r[0]), __builtin_bit_cast(float, (int)r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x),
                                            false, false);
  return fmaxf(__builtin_bit_cast(float, (int)r[0]), __builtin_bit_cast(float, (int)r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x),
                                            false, false);
  return __builtin_bit_cast(float, (int)r[0]) + __builtin_bit_cast(float, (int)r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x),
                                            false, false);
  return __builtin_bit_cast(float, (int)r[0]) + __builtin_bit_cast(float, (int)r[1]);
}

__device__ __forceinline__ float readlane(float x, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Workgroups are dispatched round-robin over the 8 XCDs by linear id, head
// index fastest.  The split index is rotated by the sequence index so that
// the always-active low splits of short sequences do not pile onto the same
// XCDs when a sequence has few workgroups per split.
__device__ __forceinline__ int split_of_block(int by, int b, int S) { return (by + b) % S; }

// Splits: sequence with `pages` pages uses ceil(pages / c) splits of c pages.
__device__ __forceinline__ int splits_of(int pages, int c) { return (pages + c - 1) / c; }

}  // namespace pa
