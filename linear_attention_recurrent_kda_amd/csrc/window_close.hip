// LeapQuant window close and initial encode on gfx950.
//
// At a window boundary (LeapQuant abstract: quantize once at the window end)
// the buffered token updates are folded into the dense state, the largest
// outliers are re-extracted as r rank-one compensator tokens (abstract and
// wink.run article, compensator tokens; here a T-step power method with
// deflation from fixed SplitMix64 start vectors), the remaining residual is
// balanced per key row (article, residual smoothing) and requantised to
// symmetric int8/int4 with per-value-column scales.
//
// One workgroup of 256 threads per head. The d_k x d_v fp32 state lives in
// registers: the 16 x 16 thread grid gives thread (ti, tj) the block of key
// rows [ti*B, ti*B+B) and value columns [tj*B, tj*B+B), B = D/16. A 16-lane
// DPP row holds one block row (all tj), so sums over value columns are DPP
// reductions; sums over key rows combine the four rows of a wave with the
// gfx950 row-swap instructions and the four waves through LDS. Reductions
// run in a fixed order, so the result is deterministic.
#include "lq_common.h"
#include "lq_launch.h"

namespace lq {

namespace {

template <int B>
__device__ __forceinline__ void loadB(const float* p, float (&x)[B]) {
  if constexpr (B % 4 == 0) {
#pragma unroll
    for (int w = 0; w < B / 4; ++w) {
      const float4 t = reinterpret_cast<const float4*>(p)[w];
      x[4 * w] = t.x;
      x[4 * w + 1] = t.y;
      x[4 * w + 2] = t.z;
      x[4 * w + 3] = t.w;
    }
  } else {
    const float2 t = *reinterpret_cast<const float2*>(p);
    x[0] = t.x;
    x[1] = t.y;
  }
}

template <int B>
__device__ __forceinline__ void storeB(float* p, const float (&x)[B]) {
  if constexpr (B % 4 == 0) {
#pragma unroll
    for (int w = 0; w < B / 4; ++w)
      reinterpret_cast<float4*>(p)[w] = make_float4(x[4 * w], x[4 * w + 1], x[4 * w + 2], x[4 * w + 3]);
  } else {
    *reinterpret_cast<float2*>(p) = make_float2(x[0], x[1]);
  }
}

// B codes of one value column (key channels i0..i0+B-1) -> signed ints
template <int B, int BITS>
__device__ __forceinline__ void load_codes(const uint8_t* p, int (&c)[B]) {
  if constexpr (BITS == 8) {
    uint64_t w = 0;
    if constexpr (B == 8) w = *reinterpret_cast<const uint64_t*>(p);
    else if constexpr (B == 4) w = *reinterpret_cast<const uint32_t*>(p);
    else w = *reinterpret_cast<const uint16_t*>(p);
#pragma unroll
    for (int a = 0; a < B; ++a) c[a] = int(int8_t(uint8_t(w >> (8 * a))));
  } else {
    uint32_t w = 0;
    if constexpr (B == 8) w = *reinterpret_cast<const uint32_t*>(p);
    else if constexpr (B == 4) w = *reinterpret_cast<const uint16_t*>(p);
    else w = *p;
#pragma unroll
    for (int a = 0; a < B; ++a) c[a] = int(((w >> (4 * a)) & 0xFu) ^ 0x8u) - 8;
  }
}

template <int B, int BITS>
__device__ __forceinline__ void store_codes(uint8_t* p, const int (&c)[B]) {
  if constexpr (BITS == 8) {
    uint64_t w = 0;
#pragma unroll
    for (int a = 0; a < B; ++a) w |= uint64_t(uint8_t(c[a])) << (8 * a);
    if constexpr (B == 8) *reinterpret_cast<uint64_t*>(p) = w;
    else if constexpr (B == 4) *reinterpret_cast<uint32_t*>(p) = uint32_t(w);
    else *reinterpret_cast<uint16_t*>(p) = uint16_t(w);
  } else {
    uint32_t w = 0;
#pragma unroll
    for (int a = 0; a < B; ++a) w |= (uint32_t(c[a]) & 0xFu) << (4 * a);
    if constexpr (B == 8) *reinterpret_cast<uint32_t*>(p) = w;
    else if constexpr (B == 4) *reinterpret_cast<uint16_t*>(p) = uint16_t(w);
    else *p = uint8_t(w);
  }
}

// 6-bit codes (code = 4 hi + lo), two planes per head: hi in [-8, 7] as
// 4-bit nibbles, [d_v][d_k/2] like 4-bit codes; then lo = code & 3 as 2-bit
// fields in 32-bit words W[j % 16][i / 16][j / 16] (value column j, key
// channel i). Channel c of a 16-channel group sits at bit
// 8 (p % 4) + 2 (p / 4), p = c/2 for even c and 8 + c/2 for odd c.
__device__ __forceinline__ int lo_bit(int c) {
  const int p = (c & 1) ? 8 + (c >> 1) : (c >> 1);
  return 8 * (p & 3) + 2 * (p >> 2);
}

template <int D>
__device__ __forceinline__ size_t lo_word(int j, int g) {
  constexpr int NJ = D / 16;
  return size_t(D * D / 2) + 4 * size_t(((j & 15) * NJ + g) * NJ + (j >> 4));
}

// B codes of value column j, key channels i0..i0+B-1 (i0 % B == 0, B <= 16).
template <int B, int D>
__device__ __forceinline__ void load_codes6(const uint8_t* head, int j, int i0, int (&c)[B]) {
  int hi[B];
  load_codes<B, 4>(head + size_t(j) * (D / 2) + i0 / 2, hi);
  const uint32_t w = *reinterpret_cast<const uint32_t*>(head + lo_word<D>(j, i0 / 16));
#pragma unroll
  for (int a = 0; a < B; ++a) c[a] = 4 * hi[a] + int((w >> lo_bit((i0 + a) & 15)) & 3u);
}

template <int D, int BITS, bool KDA, bool DENSE>
__global__ void __launch_bounds__(256) close_kernel(CloseArgs a) {
  constexpr int B = D / 16;
  constexpr int Q = (1 << (BITS - 1)) - 1;  // 127, 31 or 7
  constexpr int CB = D * BITS / 8;  // code bytes per value column (8 and 4 bits)
  constexpr int HB = D * D * BITS / 8;  // code bytes per head
  constexpr int CH = 16;            // entries staged in LDS per fold pass
  constexpr int GL = KDA ? D : 1;   // G values per entry
  __shared__ float sh_n[2][16];     // partial squared norms (double-buffered)
  __shared__ float sh_c[2][4][D];   // per-wave column partials (double-buffered)
  __shared__ __align__(16) float sh_k[DENSE ? 1 : CH][D];
  __shared__ __align__(16) float sh_u[DENSE ? 1 : CH][D];
  __shared__ __align__(16) float sh_g[DENSE ? 1 : CH][GL];
  __shared__ uint32_t sh_lo[BITS == 6 ? D : 1][BITS == 6 ? D / 16 : 1];  // 6-bit: lo words per column

  const int t = threadIdx.x, tj = t & 15, ti = t >> 4, lane = t & 63, wave = t >> 6;
  const int H = a.heads;
  int b = blockIdx.x / H;
  const int h = blockIdx.x % H;
  if (a.seq_ids) {
    b = a.seq_ids[b];
    if (b < 0 || b >= a.batch) {
      if (t == 0 && a.err) atomicOr(a.err, LQ_DEVERR_BAD_SEQ);
      return;
    }
  }
  const int bh = b * H + h;
  const size_t hD = size_t(bh) * D;
  const int i0 = ti * B, j0 = tj * B;
  const int r = a.r;
  const size_t erow = size_t(bh) * (r + a.w_max);  // first entry row of this head

  // ---- the dense state block M[x][bb] = S[i0 + x][j0 + bb]
  float M[B][B];
  if constexpr (DENSE) {
#pragma unroll
    for (int bb = 0; bb < B; ++bb) {
      float col[B];
      loadB<B>(a.S + (hD + j0 + bb) * D + i0, col);
#pragma unroll
      for (int x = 0; x < B; ++x) M[x][bb] = col[x];
    }
  } else {
    // fold: S = exp(G_n) (.) diag(s) C diag(c) + sum_e exp(G_n - G_e) (.) k_e u_e^T
    // over the entries e < r + n (compensators carry G_e = 0); G_n is the G of
    // the last entry (0 when there is none)
    const int n = __builtin_amdgcn_readfirstlane(a.blen[bh]);
    if (n < 0 || n > a.w_max) {  // corrupted buffer length: leave the head untouched
      if (t == 0 && a.err) atomicOr(a.err, LQ_DEVERR_BAD_LEN);
      return;
    }
    const int E = r + n;
    float si[B], cj[B], Gn[KDA ? B : 1];
    loadB<B>(a.s + hD + i0, si);
    loadB<B>(a.c + hD + j0, cj);
    if constexpr (KDA) {
      if (E > 0) loadB<B>(a.eg + (erow + E - 1) * D + i0, Gn);
      else
#pragma unroll
        for (int x = 0; x < B; ++x) Gn[x] = 0.f;
    } else {
      Gn[0] = E > 0 ? a.eg[erow + E - 1] : 0.f;
    }
    const uint8_t* cb = static_cast<const uint8_t*>(a.codes) + size_t(bh) * HB;
#pragma unroll
    for (int bb = 0; bb < B; ++bb) {
      int code[B];
      if constexpr (BITS == 6) load_codes6<B, D>(cb, j0 + bb, i0, code);
      else load_codes<B, BITS>(cb + size_t(j0 + bb) * CB + i0 * BITS / 8, code);
#pragma unroll
      for (int x = 0; x < B; ++x) M[x][bb] = (si[x] * float(code[x])) * cj[bb];
    }
#pragma unroll
    for (int x = 0; x < B; ++x) {
      const float e = expf(KDA ? Gn[x] : Gn[0]);
#pragma unroll
      for (int bb = 0; bb < B; ++bb) M[x][bb] *= e;
    }
    // entries, CH at a time: the workgroup stages the rows in LDS with one
    // round of loads, then every thread applies them to its block
    constexpr int V4 = D / 4;                       // float4 per row
    constexpr int PER = (CH * V4 + 255) / 256;      // float4 per thread per array
    for (int m0 = 0; m0 < E; m0 += CH) {
      const int cnt = min(CH, E - m0);
      __syncthreads();  // the previous pass has consumed the staged rows
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        const int idx = t + 256 * p;
        if (idx < cnt * V4) {
          const int row = idx / V4, c4 = idx % V4;
          const size_t g = (erow + m0 + row) * D + 4 * c4;
          reinterpret_cast<float4*>(&sh_k[row][0])[c4] = *reinterpret_cast<const float4*>(a.ek + g);
          reinterpret_cast<float4*>(&sh_u[row][0])[c4] = *reinterpret_cast<const float4*>(a.eu + g);
          if constexpr (KDA) reinterpret_cast<float4*>(&sh_g[row][0])[c4] = *reinterpret_cast<const float4*>(a.eg + g);
        }
      }
      if constexpr (!KDA) {
        if (t < cnt) sh_g[t][0] = a.eg[erow + m0 + t];
      }
      __syncthreads();
      for (int m = 0; m < cnt; ++m) {
        float km[B], um[B];
        loadB<B>(&sh_k[m][i0], km);
        loadB<B>(&sh_u[m][j0], um);
        if constexpr (KDA) {
          float gm[B];
          loadB<B>(&sh_g[m][i0], gm);
#pragma unroll
          for (int x = 0; x < B; ++x) km[x] *= expf(Gn[x] - gm[x]);
        } else {
          const float f = expf(Gn[0] - sh_g[m][0]);
#pragma unroll
          for (int x = 0; x < B; ++x) km[x] *= f;
        }
#pragma unroll
        for (int x = 0; x < B; ++x)
#pragma unroll
          for (int bb = 0; bb < B; ++bb) M[x][bb] = fmaf(km[x], um[bb], M[x][bb]);
      }
    }
  }

  // ---- compensators: power method with deflation. One barrier per
  // iteration: kappa = M v is complete inside each 16-lane row; the column
  // partials of M^T kappa and the squared norm of kappa go to LDS together
  // (double-buffered, so the next iteration may write while this one is read)
  bool live = true;
  int par = 0;
  for (int l = 0; l < r; ++l) {
    float kk[B], w[B], v[B];
#pragma unroll
    for (int x = 0; x < B; ++x) kk[x] = w[x] = 0.f;
    if (live) {
      float p = 0.f;
      if (!DENSE && a.warm) {
        // warm start: the value of compensator l of the window being closed
        // (entry l is rewritten only after this compensator is extracted)
        loadB<B>(a.eu + (erow + l) * D + j0, v);
#pragma unroll
        for (int bb = 0; bb < B; ++bb) p = fmaf(v[bb], v[bb], p);
        p = group_sum<16>(p);  // the same total in every row
      }
      if (!(p > 0.f) || !isfinite(p)) {  // cold start, or no usable warm vector
        p = 0.f;
#pragma unroll
        for (int bb = 0; bb < B; ++bb) {
          v[bb] = start_vec(l, j0 + bb, D);
          p = fmaf(v[bb], v[bb], p);
        }
        p = group_sum<16>(p);
      }
      const float inv_nv = __builtin_amdgcn_rsqf(p);
#pragma unroll
      for (int bb = 0; bb < B; ++bb) v[bb] *= inv_nv;
      for (int it = 0; it < a.T; ++it) {
        // kappa = M v  (sum over value columns: DPP across the 16 tj lanes)
        float kap[B];
        float pk = 0.f;
#pragma unroll
        for (int x = 0; x < B; ++x) {
          float s = 0.f;
#pragma unroll
          for (int bb = 0; bb < B; ++bb) s = fmaf(M[x][bb], v[bb], s);
          kap[x] = group_sum<16>(s);
          pk = fmaf(kap[x], kap[x], pk);
        }
        // M^T kappa (sum over key rows: the wave's four rows, then the waves)
#pragma unroll
        for (int bb = 0; bb < B; ++bb) {
          float s = 0.f;
#pragma unroll
          for (int x = 0; x < B; ++x) s = fmaf(M[x][bb], kap[x], s);
          s = rows_sum(s);
          if (lane < 16) sh_c[par][wave][j0 + bb] = s;
        }
        if (tj == 0) sh_n[par][ti] = pk;
        __syncthreads();
        float nk2 = 0.f;
#pragma unroll
        for (int q = 0; q < 16; ++q) nk2 += sh_n[par][q];
        if (!(nk2 > 0.f) || !isfinite(nk2)) {  // uniform: every thread read the same sums
          live = false;
          break;
        }
        const float inv_rk = __builtin_amdgcn_rsqf(nk2);
#pragma unroll
        for (int x = 0; x < B; ++x) kk[x] = kap[x] * inv_rk;
        // w = M^T k = (M^T kappa) / |kappa|
        float pw = 0.f;
#pragma unroll
        for (int bb = 0; bb < B; ++bb) {
          const int j = j0 + bb;
          w[bb] = ((sh_c[par][0][j] + sh_c[par][1][j]) + (sh_c[par][2][j] + sh_c[par][3][j])) * inv_rk;
          pw = fmaf(w[bb], w[bb], pw);
        }
        par ^= 1;
        pw = group_sum<16>(pw);  // the same total in every row
        if (!(pw > 0.f) || !isfinite(pw)) {
          live = false;
          break;
        }
        const float inv_rw = __builtin_amdgcn_rsqf(pw);
#pragma unroll
        for (int bb = 0; bb < B; ++bb) v[bb] = w[bb] * inv_rw;
      }
    }
    if (!live) {
#pragma unroll
      for (int x = 0; x < B; ++x) kk[x] = w[x] = 0.f;
    }
    // compensator l is entry l: a unit key, its value, and G = 0 (window position 0)
    if (tj == 0) storeB<B>(a.ek + (erow + l) * D + i0, kk);
    if (ti == 0) storeB<B>(a.eu + (erow + l) * D + j0, w);
    if constexpr (KDA) {
      if (tj == 0) {
        float z[B];
#pragma unroll
        for (int x = 0; x < B; ++x) z[x] = 0.f;
        storeB<B>(a.eg + (erow + l) * D + i0, z);
      }
    } else if (t == 0) {
      a.eg[erow + l] = 0.f;
    }
#pragma unroll
    for (int x = 0; x < B; ++x)
#pragma unroll
      for (int bb = 0; bb < B; ++bb) M[x][bb] = fmaf(-kk[x], w[bb], M[x][bb]);
  }

  if (a.dbg) {
#pragma unroll
    for (int bb = 0; bb < B; ++bb) {
      float col[B];
#pragma unroll
      for (int x = 0; x < B; ++x) col[x] = M[x][bb];
      storeB<B>(a.dbg + (hD + j0 + bb) * D + i0, col);
    }
  }

  // ---- key-row smoothing scales
  float sa[B];
#pragma unroll
  for (int x = 0; x < B; ++x) {
    float m = 0.f;
#pragma unroll
    for (int bb = 0; bb < B; ++bb) m = fmaxf(m, fabsf(M[x][bb]));
    m = group_max<16>(m);
    sa[x] = (a.smoothing && m > 0.f) ? m : 1.f;
    const float rs = 1.f / sa[x];
#pragma unroll
    for (int bb = 0; bb < B; ++bb) M[x][bb] *= rs;
  }

  // ---- value-column scales and codes
  __syncthreads();  // the power method's last reads of sh_c are done
#pragma unroll
  for (int bb = 0; bb < B; ++bb) {
    float m = 0.f;
#pragma unroll
    for (int x = 0; x < B; ++x) m = fmaxf(m, fabsf(M[x][bb]));
    m = rows_max(m);
    if (lane < 16) sh_c[0][wave][j0 + bb] = m;
  }
  if constexpr (BITS == 6) {
    for (int idx = t; idx < D * (D / 16); idx += 256) sh_lo[idx / (D / 16)][idx % (D / 16)] = 0u;
  }
  __syncthreads();
  float cs[B], inv[B];
#pragma unroll
  for (int bb = 0; bb < B; ++bb) {
    const int j = j0 + bb;
    const float m = fmaxf(fmaxf(sh_c[0][0][j], sh_c[0][1][j]), fmaxf(sh_c[0][2][j], sh_c[0][3][j]));
    cs[bb] = m / float(Q);
    inv[bb] = m > 0.f ? float(Q) / m : 0.f;
  }
  uint8_t* cb = static_cast<uint8_t*>(a.codes) + size_t(bh) * HB;
#pragma unroll
  for (int bb = 0; bb < B; ++bb) {
    int code[B];
#pragma unroll
    for (int x = 0; x < B; ++x) {
      const float qv = fminf(fmaxf(rintf(M[x][bb] * inv[bb]), -float(Q)), float(Q));
      code[x] = int(qv);
    }
    if constexpr (BITS == 6) {
      int hi[B];
      uint32_t lo = 0;
#pragma unroll
      for (int x = 0; x < B; ++x) {
        hi[x] = code[x] >> 2;  // arithmetic: floor(code / 4)
        lo |= uint32_t(code[x] & 3) << lo_bit((i0 + x) & 15);
      }
      store_codes<B, 4>(cb + size_t(j0 + bb) * (D / 2) + i0 / 2, hi);
      atomicOr(&sh_lo[j0 + bb][i0 / 16], lo);  // the threads of a 16-channel group meet in LDS
    } else {
      store_codes<B, BITS>(cb + size_t(j0 + bb) * CB + i0 * BITS / 8, code);
    }
  }
  if constexpr (BITS == 6) {
    __syncthreads();
    for (int idx = t; idx < D * (D / 16); idx += 256) {
      const int j = idx / (D / 16), g = idx % (D / 16);
      *reinterpret_cast<uint32_t*>(cb + lo_word<D>(j, g)) = sh_lo[j][g];
    }
  }
  if (tj == 0) storeB<B>(a.s + hD + i0, sa);
  if (ti == 0) storeB<B>(a.c + hD + j0, cs);
  if (t == 0) a.blen[bh] = 0;
}

template <int D, int BITS, bool KDA, bool DENSE>
hipError_t launch(const CloseArgs& a, int n_blocks, hipStream_t stream) {
  hipLaunchKernelGGL((close_kernel<D, BITS, KDA, DENSE>), dim3(n_blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int D, int BITS>
hipError_t launch_b(const lq_dims& d, const CloseArgs& a, int nb, hipStream_t s) {
  if (a.S)
    return d.decay_per_channel ? launch<D, BITS, true, true>(a, nb, s) : launch<D, BITS, false, true>(a, nb, s);
  return d.decay_per_channel ? launch<D, BITS, true, false>(a, nb, s) : launch<D, BITS, false, false>(a, nb, s);
}

template <int D>
hipError_t launch_d(const lq_dims& d, const CloseArgs& a, int nb, hipStream_t s) {
  switch (d.bits) {
    case 8: return launch_b<D, 8>(d, a, nb, s);
    case 6: return launch_b<D, 6>(d, a, nb, s);
    default: return launch_b<D, 4>(d, a, nb, s);
  }
}

}  // namespace

hipError_t launch_close(const lq_dims& d, const CloseArgs& a, int n_blocks, hipStream_t stream) {
  switch (d.d_k) {
    case 32: return launch_d<32>(d, a, n_blocks, stream);
    case 64: return launch_d<64>(d, a, n_blocks, stream);
    default: return launch_d<128>(d, a, n_blocks, stream);
  }
}

}  // namespace lq
