// Device helpers shared by the LeapQuant kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace lq {

__device__ __forceinline__ float as_f(uint32_t x) { return __uint_as_float(x); }
__device__ __forceinline__ uint32_t as_u(float x) { return __float_as_uint(x); }

typedef int v4i __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// Raw buffer resource over [base, base + bytes): a load at or past `bytes`
// returns zeros and moves no data (gfx9 descriptor word 3: 32-bit data format).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), 0x00020000);
}

// DPP lane permutations inside a 16-lane row (gfx9 encodings).
enum : int {
  DPP_QUAD_XOR1 = 0xB1,    // quad_perm [1,0,3,2]
  DPP_QUAD_XOR2 = 0x4E,    // quad_perm [2,3,0,1]
  DPP_HALF_MIRROR = 0x141, // lane l <- lane 7-l inside each half row
  DPP_MIRROR = 0x140,      // lane l <- lane 15-l inside the row
};

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                               0xF, 0xF, false));
}

// Sum over aligned groups of N lanes (N in 1,2,4,8,16) inside a 16-lane row.
// Every lane of a group ends with the bit-identical sum (each step adds a
// lane's value to its partner's, and x + y == y + x exactly). All lanes of the
// wave must be active.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp<DPP_QUAD_XOR1>(x);
  if constexpr (N >= 4) x += dpp<DPP_QUAD_XOR2>(x);
  if constexpr (N >= 8) x += dpp<DPP_HALF_MIRROR>(x);
  if constexpr (N >= 16) x += dpp<DPP_MIRROR>(x);
  return x;
}

template <int N>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (N >= 2) x = fmaxf(x, dpp<DPP_QUAD_XOR1>(x));
  if constexpr (N >= 4) x = fmaxf(x, dpp<DPP_QUAD_XOR2>(x));
  if constexpr (N >= 8) x = fmaxf(x, dpp<DPP_HALF_MIRROR>(x));
  if constexpr (N >= 16) x = fmaxf(x, dpp<DPP_MIRROR>(x));
  return x;
}

// Max over aligned groups of N lanes of a non-negative float's bit pattern
// (for x >= 0 the fp32 order is the unsigned order of the bits).
template <int N>
__device__ __forceinline__ uint32_t group_umax(uint32_t x) {
  auto d = [](uint32_t v, auto ctrl) {
    return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), decltype(ctrl)::value, 0xF, 0xF, false));
  };
  if constexpr (N >= 2) x = max(x, d(x, std::integral_constant<int, DPP_QUAD_XOR1>{}));
  if constexpr (N >= 4) x = max(x, d(x, std::integral_constant<int, DPP_QUAD_XOR2>{}));
  if constexpr (N >= 8) x = max(x, d(x, std::integral_constant<int, DPP_HALF_MIRROR>{}));
  if constexpr (N >= 16) x = max(x, d(x, std::integral_constant<int, DPP_MIRROR>{}));
  return x;
}

__device__ __forceinline__ uint32_t rows_umax(uint32_t x) {
  auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = max(uint32_t(p[0]), uint32_t(p[1]));
  auto q = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return max(uint32_t(q[0]), uint32_t(q[1]));
}

constexpr float kLog2e = 1.4426950408889634f;  // log2(e)

// exp(x) as 2^(x log2 e) on the transcendental unit (about 1 ulp of exp2,
// plus the rounding of the product: relative error ~ |x| 2^-24).
__device__ __forceinline__ float exp_fast(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

// Sum / max over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48)
// with the gfx950 row-swap instructions. Every lane ends with the same value.
__device__ __forceinline__ float rows_sum(float x) {
  auto p = __builtin_amdgcn_permlane16_swap(as_u(x), as_u(x), false, false);
  x = as_f(p[0]) + as_f(p[1]);
  auto q = __builtin_amdgcn_permlane32_swap(as_u(x), as_u(x), false, false);
  return as_f(q[0]) + as_f(q[1]);
}

__device__ __forceinline__ float rows_max(float x) {
  auto p = __builtin_amdgcn_permlane16_swap(as_u(x), as_u(x), false, false);
  x = fmaxf(as_f(p[0]), as_f(p[1]));
  auto q = __builtin_amdgcn_permlane32_swap(as_u(x), as_u(x), false, false);
  return fmaxf(as_f(q[0]), as_f(q[1]));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return as_f(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return as_f(w & 0xFFFF0000u); }

// One activation value (fp32 or bf16) at element index idx.
template <bool BF16>
__device__ __forceinline__ float load_act(const void* p, size_t idx) {
  if constexpr (BF16) {
    return as_f(uint32_t(reinterpret_cast<const uint16_t*>(p)[idx]) << 16);
  } else {
    return reinterpret_cast<const float*>(p)[idx];
  }
}

// 16 consecutive fp32 values from a 16-byte aligned address.
__device__ __forceinline__ void load16(const float* p, float (&x)[16]) {
  const float4* p4 = reinterpret_cast<const float4*>(p);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    float4 t = p4[w];
    x[4 * w + 0] = t.x;
    x[4 * w + 1] = t.y;
    x[4 * w + 2] = t.z;
    x[4 * w + 3] = t.w;
  }
}

__device__ __forceinline__ void store16(float* p, const float (&x)[16]) {
  float4* p4 = reinterpret_cast<float4*>(p);
#pragma unroll
  for (int w = 0; w < 4; ++w) p4[w] = make_float4(x[4 * w], x[4 * w + 1], x[4 * w + 2], x[4 * w + 3]);
}

// SplitMix64 (Steele, Lea & Flood, OOPSLA 2014): output number n (1-based)
// of the generator started from state 0.
__host__ __device__ constexpr uint64_t splitmix64(uint64_t n) {
  uint64_t z = n * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Power-method start vector entry v0[l][j]: the top 23 bits m of output
// l*d_v + j + 1 give (2m + 1 - 2^23) / 2^23, exact in fp32.
__host__ __device__ constexpr float start_vec(int l, int j, int d_v) {
  const uint64_t m = splitmix64(uint64_t(l) * uint64_t(d_v) + uint64_t(j) + 1ull) >> 41;
  return float(int32_t(2 * m + 1) - (1 << 23)) * 0x1p-23f;
}

// The start vectors of up to R compensators at head dimension D, evaluated at
// compile time: the same for every head and every window.
template <int R, int D>
struct StartVectors {
  float v[R][D];
  constexpr StartVectors() : v{} {
    for (int l = 0; l < R; ++l)
      for (int j = 0; j < D; ++j) v[l][j] = start_vec(l, j, D);
  }
};

}  // namespace lq
