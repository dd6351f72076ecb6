// Cross-lane reductions with the work split across lanes (gfx950, wave64):
// the sum or maximum of several values over a group of lanes, arranged so
// that each lane ends with the totals of some of the values instead of all of
// them. A row swap or DPP step then combines two values per instruction
// pair, where a full reduction of each value would spend one per value.
#pragma once

#include "lq_common.h"

namespace lq {

// Column sums over the four 16-lane rows of a wave, the work split across the
// rows: each row-swap step pairs two columns, one kept by each half of the
// lanes. For CB >= 4, lane row g ends with the totals of columns
// g * CB / 4 + m (m < CB / 4); for CB = 2, with column g / 2's total.
template <int CB>
__device__ __forceinline__ void rows_sum_split(float (&p)[CB], float (&out)[CB >= 4 ? CB / 4 : 1]) {
  constexpr int H = CB / 2;
  float q[H];
#pragma unroll
  for (int m = 0; m < H; ++m) {
    auto s = __builtin_amdgcn_permlane32_swap(as_u(p[m]), as_u(p[m + H]), false, false);
    q[m] = as_f(s[0]) + as_f(s[1]);  // lanes 0-31: column m; lanes 32-63: column m + H
  }
  if constexpr (CB >= 4) {
    constexpr int Q = CB / 4;
#pragma unroll
    for (int m = 0; m < Q; ++m) {
      auto s = __builtin_amdgcn_permlane16_swap(as_u(q[m]), as_u(q[m + Q]), false, false);
      out[m] = as_f(s[0]) + as_f(s[1]);  // even rows: q[m]; odd rows: q[m + Q]
    }
  } else {
    auto s = __builtin_amdgcn_permlane16_swap(as_u(q[0]), as_u(q[0]), false, false);
    out[0] = as_f(s[0]) + as_f(s[1]);
  }
}

// The same split for maxima, and its inverse: NV values per lane row (row g
// holding columns g * NV + m) gathered so that every lane holds all 4 NV in
// column order.
template <int CB>
__device__ __forceinline__ void rows_max_split(float (&p)[CB], float (&out)[CB / 4]) {
  static_assert(CB >= 4, "columns per thread");
  constexpr int H = CB / 2, Q = CB / 4;
  float q[H];
#pragma unroll
  for (int m = 0; m < H; ++m) {
    auto s = __builtin_amdgcn_permlane32_swap(as_u(p[m]), as_u(p[m + H]), false, false);
    q[m] = fmaxf(as_f(s[0]), as_f(s[1]));
  }
#pragma unroll
  for (int m = 0; m < Q; ++m) {
    auto s = __builtin_amdgcn_permlane16_swap(as_u(q[m]), as_u(q[m + Q]), false, false);
    out[m] = fmaxf(as_f(s[0]), as_f(s[1]));
  }
}

template <int NV>
__device__ __forceinline__ void rows_gather(const float (&x)[NV], float (&out)[4 * NV]) {
  float y[2 * NV];
#pragma unroll
  for (int m = 0; m < NV; ++m) {  // rows (0, 1) and (2, 3): the even row's values first
    auto s = __builtin_amdgcn_permlane16_swap(as_u(x[m]), as_u(x[m]), false, false);
    y[m] = as_f(s[0]), y[NV + m] = as_f(s[1]);
  }
#pragma unroll
  for (int k = 0; k < 2 * NV; ++k) {  // lanes 0-31 and 32-63: the lower half's values first
    auto s = __builtin_amdgcn_permlane32_swap(as_u(y[k]), as_u(y[k]), false, false);
    out[k] = as_f(s[0]), out[2 * NV + k] = as_f(s[1]);
  }
}

// Maxima of 16 per-row values over the 16 lanes of a DPP row, the work split
// so that lane c ends with value c's maximum: each step pairs lane c with
// c ^ 15, c ^ 7, c ^ 2, c ^ 1 and keeps the half of the values whose index
// bit matches c's (bit 3, 2, 1, 0), the partner sending the other half.
__device__ __forceinline__ float row_max_split16(const float (&x)[16], int c) {
  float a8[8], a4[4], a2[2];
  const bool b3 = c & 8, b2 = c & 4, b1 = c & 2, b0 = c & 1;
#pragma unroll
  for (int k = 0; k < 8; ++k)
    a8[k] = fmaxf(b3 ? x[k + 8] : x[k], dpp<DPP_MIRROR>(b3 ? x[k] : x[k + 8]));
#pragma unroll
  for (int k = 0; k < 4; ++k)
    a4[k] = fmaxf(b2 ? a8[k + 4] : a8[k], dpp<DPP_HALF_MIRROR>(b2 ? a8[k] : a8[k + 4]));
#pragma unroll
  for (int k = 0; k < 2; ++k)
    a2[k] = fmaxf(b1 ? a4[k + 2] : a4[k], dpp<DPP_QUAD_XOR2>(b1 ? a4[k] : a4[k + 2]));
  return fmaxf(b0 ? a2[1] : a2[0], dpp<DPP_QUAD_XOR1>(b0 ? a2[0] : a2[1]));
}

// M[x][..] *= (value of lane x of this thread's DPP row) for x = X..15.
template <int X, int CB, typename T>
__device__ __forceinline__ void scale_rows_bcast(T (&M)[4][CB], float r) {
  if constexpr (X < 16) {
    const float f = __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, r), 0x150 + X, 0xF, 0xF, false));
#pragma unroll
    for (int bb = 0; bb < CB; ++bb) M[X >> 2][bb][X & 3] *= f;
    scale_rows_bcast<X + 1, CB>(M, r);
  }
}

}  // namespace lq
