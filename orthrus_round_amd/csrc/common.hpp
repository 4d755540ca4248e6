// Shared device helpers for the Orthrus gfx950 kernels: element types, MFMA fragments,
// wavefront reductions, Philox4x64-10 and host-side validation/error plumbing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>
#include <cstdio>
#include <string>

#include "../../include/orthrus.h"

namespace orthrus {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// ---------------------------------------------------------------------------------------
// MFMA 32x32 fragments.  For an A operand [32 x KSTEP] (rows x k) lane l holds row l%32 and
// KW consecutive k values starting at KW*(l/32); the B operand is the same with columns.
// The 16 accumulator values of lane l belong to column l%32 and rows
// (i/4)*8 + (l/32)*4 + i%4, i = 0..15.
// ---------------------------------------------------------------------------------------
// Compile-time loop: f(Int<0>{}), ..., f(Int<N-1>{}), so that indices stay constants.
template <int I> struct Int { static constexpr int value = I; };
template <int N, int I = 0, typename F> __device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(Int<I>{});
    static_for<N, I + 1>(f);
  }
}

template <typename T> struct Mfma;

template <> struct Mfma<bf16> {
  static constexpr int KSTEP = 16;  // k per instruction
  static constexpr int KW = 8;      // k values per lane
  typedef bf16x8 frag;
  __device__ __forceinline__ static f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mfma<float> {
  static constexpr int KSTEP = 2;
  static constexpr int KW = 1;
  typedef float frag;
  __device__ __forceinline__ static f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// Row of accumulator value i for lane-half h.
__device__ __forceinline__ int acc_row(int i, int h) { return (i >> 2) * 8 + h * 4 + (i & 3); }

// ---------------------------------------------------------------------------------------
// Wavefront helpers
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, kWave); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, shfl_xor_f(v, m));
  return v;
}
// RMSNorm workgroups (standalone and fused into the residual GEMM's reduce) have one thread per
// 16-byte chunk of the row, rounded up to whole waves, at most kNormMaxChunks; longer rows use
// kNormMaxChunks threads and a strided loop.
constexpr int kNormMaxChunks = 1024;
inline int norm_threads(int n, int elem_bytes) {
  const int chunks = (int)(((int64_t)n * elem_bytes + 15) / 16);
  const int t = ((chunks + 63) / 64) * 64;
  return t < 64 ? 64 : (t > kNormMaxChunks ? kNormMaxChunks : t);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor_f(v, m);
  return v;
}

// Order-preserving map of a float to uint32 (larger float -> larger key; NaN treated large).
__device__ __forceinline__ uint32_t ordered_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float ordered_key_inv(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}
// (value, index) packed so that a larger packed value = larger value, then SMALLER index.
__device__ __forceinline__ uint64_t pack_argmax(float v, int32_t idx) {
  return ((uint64_t)ordered_key(v) << 32) | (uint32_t)(0x7fffffff - idx);
}
__device__ __forceinline__ int32_t unpack_idx(uint64_t p) { return 0x7fffffff - (int32_t)(uint32_t)(p & 0xffffffffu); }
__device__ __forceinline__ float unpack_val(uint64_t p) { return ordered_key_inv((uint32_t)(p >> 32)); }

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = __shfl_xor((uint32_t)v, m, kWave);
  uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, kWave);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// ---------------------------------------------------------------------------------------
// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11).  Two 64x64->128 multiplies per round by
// fixed odd constants; the high halves are XORed with the other words and the round key; the
// key is bumped by two Weyl constants between rounds.
// ---------------------------------------------------------------------------------------
struct u64x4 { uint64_t x[4]; };

__device__ __forceinline__ u64x4 philox4x64_10(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3,
                                               uint64_t k0, uint64_t k1) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) { k0 += W0; k1 += W1; }
    uint64_t hi0 = __umul64hi(M0, c0), lo0 = M0 * c0;
    uint64_t hi1 = __umul64hi(M1, c2), lo1 = M1 * c2;
    uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
  }
  u64x4 o; o.x[0] = c0; o.x[1] = c1; o.x[2] = c2; o.x[3] = c3;
  return o;
}

// u = ((w >> 41) + 0.5) * 2^-23, exact in fp32, in (0, 1).
__device__ __forceinline__ float word_to_uniform(uint64_t w) {
  return ((float)(uint32_t)(w >> 41) + 0.5f) * 1.1920928955078125e-07f;
}

// Uniform of item `index` of a draw with counter (index/4, c1, c2, c3), word index%4.
__device__ __forceinline__ float philox_uniform(uint64_t seed, uint64_t stream, int64_t index, int64_t c1,
                                                int64_t c2, int64_t c3) {
  u64x4 w = philox4x64_10((uint64_t)(index >> 2), (uint64_t)c1, (uint64_t)c2, (uint64_t)c3, seed, stream);
  const int k = (int)(index & 3);  // selects, not a runtime array index (which would go to scratch)
  return word_to_uniform(k == 0 ? w.x[0] : k == 1 ? w.x[1] : k == 2 ? w.x[2] : w.x[3]);
}

// ---------------------------------------------------------------------------------------
// Host-side plumbing
// ---------------------------------------------------------------------------------------
void set_error(const std::string& msg);
int32_t fail(int32_t status, const char* fmt, ...);
int32_t check_launch(const char* what);
inline size_t dtype_size(int32_t dt) { return dt == ORTHRUS_BF16 ? 2 : 4; }
inline bool valid_dtype(int32_t dt) { return dt == ORTHRUS_BF16 || dt == ORTHRUS_F32; }

#define ORTHRUS_REQUIRE(cond, status, ...) \
  do { if (!(cond)) return ::orthrus::fail((status), __VA_ARGS__); } while (0)

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Kernels that take more than 64 KiB of dynamic LDS opt in, once per kernel.  Kernels of one
// signature share a pointer type, so the kernels already done are kept by address.
void allow_lds_once(const void* kernel, size_t bytes);
template <typename K>
inline void allow_lds(K kernel, size_t bytes) {
  if (bytes > 65536) allow_lds_once(reinterpret_cast<const void*>(kernel), bytes);
}

}  // namespace orthrus
