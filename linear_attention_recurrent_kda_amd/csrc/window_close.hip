// LeapQuant window close and initial encode on gfx950.
//
// At a window boundary (LeapQuant abstract: a single requantization per window)
// the buffered token updates are folded into the dense state, the largest
// outliers are re-extracted as r rank-one compensator tokens (abstract and
// wink.run article, compensator tokens; here a T-step power method with
// deflation from fixed SplitMix64 start vectors), the remaining residual is
// balanced per key row (article, residual smoothing) and requantised to
// symmetric int8/6-bit/int4 codes with per-value-column scales.
//
// One workgroup of 128 threads (two waves) per head. The d_k x d_v fp32 state
// lives in registers: the 8 x 16 thread grid gives thread (ti, tj) the block
// of key rows [ti*RB, ti*RB+RB) and value columns [tj*CB, tj*CB+CB), with
// RB = D/8 and CB = D/16 (16 x 8 at D = 128). A 16-lane DPP row holds one
// block row (all tj), so sums over value columns are DPP reductions; sums over
// key rows combine the four rows of a wave with the gfx950 row-swap
// instructions, the work split so that each row keeps a quarter of the
// columns, and the two waves through LDS. Tall blocks keep the reduction work
// per power iteration low (16 DPP sums and 6 row swaps per 256 FMA), and at
// D = 128 a thread owns whole 16-channel code groups. The fold of the buffered
// entries is an fp32 matrix-core update whose output tiles land on these same
// register blocks. Reductions run in a fixed order, so the result is
// deterministic.
#include "lq_common.h"
#include "lq_launch.h"
#include "lq_rows.h"

namespace lq {

namespace {

constexpr int NT = 128;  // threads per head

typedef float v4f __attribute__((ext_vector_type(4)));

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

// NB bytes (2, 4, 8 or 16, naturally aligned) as little-endian 32-bit words.
template <int NB>
__device__ __forceinline__ void load_bytes(const uint8_t* p, uint32_t (&w)[(NB + 3) / 4]) {
  if constexpr (NB == 16) {
    const uint4 t = *reinterpret_cast<const uint4*>(p);
    w[0] = t.x, w[1] = t.y, w[2] = t.z, w[3] = t.w;
  } else if constexpr (NB == 8) {
    const uint2 t = *reinterpret_cast<const uint2*>(p);
    w[0] = t.x, w[1] = t.y;
  } else if constexpr (NB == 4) {
    w[0] = *reinterpret_cast<const uint32_t*>(p);
  } else {
    static_assert(NB == 2, "code bytes per block column");
    w[0] = *reinterpret_cast<const uint16_t*>(p);
  }
}

template <int NB>
__device__ __forceinline__ void store_bytes(uint8_t* p, const uint32_t (&w)[(NB + 3) / 4]) {
  if constexpr (NB == 16) *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  else if constexpr (NB == 8) *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
  else if constexpr (NB == 4) *reinterpret_cast<uint32_t*>(p) = w[0];
  else *reinterpret_cast<uint16_t*>(p) = uint16_t(w[0]);
}

// N codes of one value column (consecutive key channels) at p -> signed ints.
// 8 bits: one byte each; 4 bits: two's-complement nibbles, even channel low.
template <int N, int BITS>
__device__ __forceinline__ void load_codes(const uint8_t* p, int (&c)[N]) {
  constexpr int NB = N * BITS / 8;
  uint32_t w[(NB + 3) / 4];
  load_bytes<NB>(p, w);
#pragma unroll
  for (int a = 0; a < N; ++a) {
    if constexpr (BITS == 8) c[a] = int(int8_t(uint8_t(w[a / 4] >> (8 * (a % 4)))));
    else c[a] = int(((w[a / 8] >> (4 * (a % 8))) & 0xFu) ^ 0x8u) - 8;
  }
}

template <int N, int BITS>
__device__ __forceinline__ void store_codes(uint8_t* p, const int (&c)[N]) {
  constexpr int NB = N * BITS / 8;
  uint32_t w[(NB + 3) / 4];
#pragma unroll
  for (int q = 0; q < (NB + 3) / 4; ++q) w[q] = 0u;
#pragma unroll
  for (int a = 0; a < N; ++a) {
    if constexpr (BITS == 8) w[a / 4] |= uint32_t(uint8_t(c[a])) << (8 * (a % 4));
    else w[a / 8] |= (uint32_t(c[a]) & 0xFu) << (4 * (a % 8));
  }
  store_bytes<NB>(p, w);
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

// N codes of value column j, key channels i0..i0+N-1 (i0 % N == 0, N <= 16).
template <int N, int D>
__device__ __forceinline__ void load_codes6(const uint8_t* head, int j, int i0, int (&c)[N]) {
  int hi[N];
  load_codes<N, 4>(head + size_t(j) * (D / 2) + i0 / 2, hi);
  const uint32_t w = *reinterpret_cast<const uint32_t*>(head + lo_word<D>(j, i0 / 16));
#pragma unroll
  for (int a = 0; a < N; ++a) c[a] = 4 * hi[a] + int((w >> lo_bit((i0 + a) & 15)) & 3u);
}

__device__ __forceinline__ uint32_t or_swap16(uint32_t x) {  // x | x of lane ^ 16
  auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return uint32_t(p[0]) | uint32_t(p[1]);
}

__device__ __forceinline__ uint32_t or_swap32(uint32_t x) {  // x | x of lane ^ 32
  auto p = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return uint32_t(p[0]) | uint32_t(p[1]);
}

// Power-method start vectors for up to 8 compensators (the ABI's limit).
template <int D>
__constant__ constexpr StartVectors<8, D> kStart{};

template <int D, int BITS, bool KDA, bool DENSE>
__global__ void __launch_bounds__(NT) close_kernel(CloseArgs a) {
  constexpr int RB = D / 8;   // key rows per thread
  constexpr int CB = D / 16;  // value columns per thread
  constexpr int Q = (1 << (BITS - 1)) - 1;  // 127, 31 or 7
  constexpr int HB = D * D * BITS / 8;      // code bytes per head
  constexpr int CH = 16;                    // entries staged in LDS per fold pass
  constexpr int V4 = D / 4;                 // float4 per entry row
  constexpr int PER = CH * V4 / NT;         // float4 per thread per staged array
  static_assert(NT % V4 == 0 && PER >= 1 && PER * NT == CH * V4, "staging shape");
  __shared__ float sh_n[2][2];                // per-wave squared norms (double-buffered)
  __shared__ __align__(16) float sh_c[2][2][D];  // per-wave column partials (double-buffered)
  __shared__ __align__(16) float sh_k[DENSE ? 1 : CH][D];  // keys scaled by their decay to the window end
  __shared__ __align__(16) float sh_u[DENSE ? 1 : CH][D];

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
  const int i0 = ti * RB, j0 = tj * CB;
  const int r = a.r;
  const size_t erow = size_t(bh) * (r + a.w_max);  // first entry row of this head

  // ---- the dense state block M[x][bb] = S[i0 + x][j0 + bb]
  // (four consecutive key rows of one value column form one MFMA accumulator)
  v4f M[RB / 4][CB];
  if constexpr (DENSE) {
#pragma unroll
    for (int bb = 0; bb < CB; ++bb) {
      float col[RB];
      loadB<RB>(a.S + (hD + j0 + bb) * D + i0, col);
#pragma unroll
      for (int x = 0; x < RB; ++x) M[x >> 2][bb][x & 3] = col[x];
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
    float si[RB], cj[CB], Gn[KDA ? RB : 1];
    loadB<RB>(a.s + hD + i0, si);
    loadB<CB>(a.c + hD + j0, cj);
    if constexpr (KDA) {
      if (E > 0) loadB<RB>(a.eg + (erow + E - 1) * D + i0, Gn);
      else
#pragma unroll
        for (int x = 0; x < RB; ++x) Gn[x] = 0.f;
    } else {
      Gn[0] = E > 0 ? a.eg[erow + E - 1] : 0.f;
    }
    const uint8_t* cb = static_cast<const uint8_t*>(a.codes) + size_t(bh) * HB;
#pragma unroll
    for (int x = 0; x < RB; ++x) si[x] *= expf(KDA ? Gn[x] : Gn[0]);  // the residual's decay to the window end
#pragma unroll
    for (int bb = 0; bb < CB; ++bb) {
      int code[RB];
      if constexpr (BITS == 6) load_codes6<RB, D>(cb, j0 + bb, i0, code);
      else load_codes<RB, BITS>(cb + size_t(j0 + bb) * (D * BITS / 8) + i0 * BITS / 8, code);
#pragma unroll
      for (int x = 0; x < RB; ++x) M[x >> 2][bb][x & 3] = (si[x] * float(code[x])) * cj[bb];
    }
    // entries, CH at a time: the workgroup stages the rows in LDS with one
    // round of loads, each key already multiplied by its decay to the window
    // end; then every thread applies them to its block. A thread stages the
    // same four key channels of every row it loads (NT is a multiple of V4).
    const int c4 = t % V4;
    float4 gq = make_float4(0.f, 0.f, 0.f, 0.f);  // KDA: G_n of the staged channels
    if constexpr (KDA) {
      if (E > 0) gq = *reinterpret_cast<const float4*>(a.eg + (erow + E - 1) * D + 4 * c4);
    }
    // The rank-CH update M += K^T U of a pass runs on the matrix cores
    // (v_mfma_f32_16x16x4f32, four entries per instruction). Its 16 x 16
    // output tile puts rows 4 (lane / 16) + q of column lane % 16 in lane
    // 'lane', register q; the operands' rows and columns are chosen so that
    // these are exactly this thread's key rows i0 + 4 a + q and value column
    // j0 + bb, for tile (a, bb).
    const int e_of_lane = lane >> 4;  // the operands' entry within a block of four
    const int a_row = wave * 4 * RB + RB * ((lane & 15) >> 2) + (lane & 3);  // + 4 a
    const int b_col = CB * (lane & 15);                                      // + bb
    for (int m0 = 0; m0 < E; m0 += CH) {
      const int cnt = min(CH, E - m0);
      __syncthreads();  // the previous pass has consumed the staged rows
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        const int row = (t + NT * p) / V4;  // covers all CH rows; rows past cnt are zeros
        float4 kq = make_float4(0.f, 0.f, 0.f, 0.f), uq = kq;
        if (row < cnt) {
          const size_t g = (erow + m0 + row) * D + 4 * c4;
          kq = *reinterpret_cast<const float4*>(a.ek + g);
          uq = *reinterpret_cast<const float4*>(a.eu + g);
          if constexpr (KDA) {
            const float4 ge = *reinterpret_cast<const float4*>(a.eg + g);
            kq.x *= expf(gq.x - ge.x);
            kq.y *= expf(gq.y - ge.y);
            kq.z *= expf(gq.z - ge.z);
            kq.w *= expf(gq.w - ge.w);
          } else {
            const float f = expf(Gn[0] - a.eg[erow + m0 + row]);
            kq.x *= f, kq.y *= f, kq.z *= f, kq.w *= f;
          }
        }
        reinterpret_cast<float4*>(&sh_k[row][0])[c4] = kq;
        reinterpret_cast<float4*>(&sh_u[row][0])[c4] = uq;
      }
      __syncthreads();
      const int nkb = (cnt + 3) >> 2;
      for (int kb = 0; kb < nkb; ++kb) {
        const int e = 4 * kb + e_of_lane;
        float ka[RB / 4], ub[CB];
#pragma unroll
        for (int q = 0; q < RB / 4; ++q) ka[q] = sh_k[e][a_row + 4 * q];
        loadB<CB>(&sh_u[e][b_col], ub);
#pragma unroll
        for (int q = 0; q < RB / 4; ++q)
#pragma unroll
          for (int bb = 0; bb < CB; ++bb) M[q][bb] = __builtin_amdgcn_mfma_f32_16x16x4f32(ka[q], ub[bb], M[q][bb], 0, 0, 0);
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
    float kk[RB], w[CB], v[CB];
#pragma unroll
    for (int x = 0; x < RB; ++x) kk[x] = 0.f;
#pragma unroll
    for (int bb = 0; bb < CB; ++bb) w[bb] = 0.f;
    if (live) {
      float p = 0.f;
      if (!DENSE && a.warm) {
        // warm start: the value of compensator l of the window being closed
        // (entry l is rewritten only after this compensator is extracted)
        loadB<CB>(a.eu + (erow + l) * D + j0, v);
#pragma unroll
        for (int bb = 0; bb < CB; ++bb) p = fmaf(v[bb], v[bb], p);
        p = group_sum<16>(p);  // the same total in every row
      }
      if (!(p > 0.f) || !isfinite(p)) {  // cold start, or no usable warm vector
        p = 0.f;
#pragma unroll
        for (int bb = 0; bb < CB; ++bb) {
          v[bb] = kStart<D>.v[l][j0 + bb];
          p = fmaf(v[bb], v[bb], p);
        }
        p = group_sum<16>(p);
      }
      const float inv_nv = __builtin_amdgcn_rsqf(p);
#pragma unroll
      for (int bb = 0; bb < CB; ++bb) v[bb] *= inv_nv;
      float inv_rk = 0.f;
      for (int it = 0; it < a.T; ++it) {
        // kappa = M v (sum over value columns: DPP across the 16 tj lanes),
        // kept in kk; only the last iteration's is scaled to the unit key
        float pk = 0.f;
#pragma unroll
        for (int x = 0; x < RB; ++x) {
          float s = 0.f;
#pragma unroll
          for (int bb = 0; bb < CB; ++bb) s = fmaf(M[x >> 2][bb][x & 3], v[bb], s);
          kk[x] = group_sum<16>(s);
          pk = fmaf(kk[x], kk[x], pk);
        }
        // M^T kappa (sum over key rows: the wave's four rows, then the two waves)
        {
          float cs[CB], tot[CB >= 4 ? CB / 4 : 1];
#pragma unroll
          for (int bb = 0; bb < CB; ++bb) {
            float s = 0.f;
#pragma unroll
            for (int x = 0; x < RB; ++x) s = fmaf(M[x >> 2][bb][x & 3], kk[x], s);
            cs[bb] = s;
          }
          rows_sum_split<CB>(cs, tot);
          const int g = lane >> 4;
          static_assert(CB == 8 || CB == 4 || CB == 2, "columns per thread");
          if constexpr (CB == 8) {
            *reinterpret_cast<float2*>(&sh_c[par][wave][j0 + 2 * g]) = make_float2(tot[0], tot[1]);
          } else if constexpr (CB == 4) {
            sh_c[par][wave][j0 + g] = tot[0];
          } else {
            sh_c[par][wave][j0 + (g >> 1)] = tot[0];  // rows 2m and 2m+1 hold the same total
          }
        }
        pk = rows_sum(pk);  // the wave's rows; pk was already equal across the 16 tj lanes
        if (lane == 0) sh_n[par][wave] = pk;
        __syncthreads();
        const float nk2 = sh_n[par][0] + sh_n[par][1];
        if (!(nk2 > 0.f) || !isfinite(nk2)) {  // uniform: every thread read the same sums
          live = false;
          break;
        }
        inv_rk = __builtin_amdgcn_rsqf(nk2);
        // w = M^T k = (M^T kappa) / |kappa|
        float pw = 0.f;
#pragma unroll
        for (int bb = 0; bb < CB; ++bb) {
          const int j = j0 + bb;
          w[bb] = (sh_c[par][0][j] + sh_c[par][1][j]) * inv_rk;
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
        for (int bb = 0; bb < CB; ++bb) v[bb] = w[bb] * inv_rw;
      }
#pragma unroll
      for (int x = 0; x < RB; ++x) kk[x] *= inv_rk;
    }
    if (!live) {
#pragma unroll
      for (int x = 0; x < RB; ++x) kk[x] = 0.f;
#pragma unroll
      for (int bb = 0; bb < CB; ++bb) w[bb] = 0.f;
    }
    // compensator l is entry l: a unit key, its value, and G = 0 (window position 0)
    if (tj == 0) storeB<RB>(a.ek + (erow + l) * D + i0, kk);
    if (ti == 0) storeB<CB>(a.eu + (erow + l) * D + j0, w);
    if constexpr (KDA) {
      if (tj == 0) {
        float z[RB];
#pragma unroll
        for (int x = 0; x < RB; ++x) z[x] = 0.f;
        storeB<RB>(a.eg + (erow + l) * D + i0, z);
      }
    } else if (t == 0) {
      a.eg[erow + l] = 0.f;
    }
#pragma unroll
    for (int x = 0; x < RB; ++x)
#pragma unroll
      for (int bb = 0; bb < CB; ++bb) M[x >> 2][bb][x & 3] = fmaf(-kk[x], w[bb], M[x >> 2][bb][x & 3]);
  }

  if (a.dbg) {
#pragma unroll
    for (int bb = 0; bb < CB; ++bb) {
      float col[RB];
#pragma unroll
      for (int x = 0; x < RB; ++x) col[x] = M[x >> 2][bb][x & 3];
      storeB<RB>(a.dbg + (hD + j0 + bb) * D + i0, col);
    }
  }

  // ---- key-row smoothing scales. At D = 128 a thread's 16 rows are the 16
  // lanes of its DPP row: lane tj takes row i0 + tj's maximum and reciprocal,
  // and the reciprocals are broadcast back.
  float sa[RB];
  if constexpr (RB == 16) {
    float rx[RB];
#pragma unroll
    for (int x = 0; x < RB; ++x) {
      float m = 0.f;
#pragma unroll
      for (int bb = 0; bb < CB; ++bb) m = fmaxf(m, fabsf(M[x >> 2][bb][x & 3]));
      rx[x] = m;
    }
    const float m = row_max_split16(rx, tj);
    sa[0] = (a.smoothing && m > 0.f) ? m : 1.f;
    scale_rows_bcast<0, CB>(M, 1.f / sa[0]);
  } else {
#pragma unroll
    for (int x = 0; x < RB; ++x) {
      float m = 0.f;
#pragma unroll
      for (int bb = 0; bb < CB; ++bb) m = fmaxf(m, fabsf(M[x >> 2][bb][x & 3]));
      m = group_max<16>(m);
      sa[x] = (a.smoothing && m > 0.f) ? m : 1.f;
      const float rs = 1.f / sa[x];
#pragma unroll
      for (int bb = 0; bb < CB; ++bb) M[x >> 2][bb][x & 3] *= rs;
    }
  }

  // ---- value-column scales and codes. For CB >= 4 the column maxima are
  // split across the wave's rows (row g: columns j0 + g CB/4 + m), each row
  // divides for its own columns, and the reciprocals are gathered back.
  __syncthreads();  // the power method's last reads of sh_c are done
  constexpr int NV = CB >= 4 ? CB / 4 : 1;
  float cs[CB], inv[CB];
  if constexpr (CB >= 4) {
    float cm[CB], tot[NV];
#pragma unroll
    for (int bb = 0; bb < CB; ++bb) {
      float m = 0.f;
#pragma unroll
      for (int x = 0; x < RB; ++x) m = fmaxf(m, fabsf(M[x >> 2][bb][x & 3]));
      cm[bb] = m;
    }
    rows_max_split<CB>(cm, tot);
    const int jg = j0 + (lane >> 4) * NV;
#pragma unroll
    for (int m = 0; m < NV; ++m) sh_c[0][wave][jg + m] = tot[m];
    __syncthreads();
    float iv[NV];
#pragma unroll
    for (int m = 0; m < NV; ++m) {
      const float mx = fmaxf(sh_c[0][0][jg + m], sh_c[0][1][jg + m]);
      cs[m] = mx / float(Q);
      iv[m] = mx > 0.f ? float(Q) / mx : 0.f;
    }
    rows_gather<NV>(iv, inv);
  } else {
#pragma unroll
    for (int bb = 0; bb < CB; ++bb) {
      float m = 0.f;
#pragma unroll
      for (int x = 0; x < RB; ++x) m = fmaxf(m, fabsf(M[x >> 2][bb][x & 3]));
      m = rows_max(m);
      if (lane < 16) sh_c[0][wave][j0 + bb] = m;
    }
    __syncthreads();
#pragma unroll
    for (int bb = 0; bb < CB; ++bb) {
      const float m = fmaxf(sh_c[0][0][j0 + bb], sh_c[0][1][j0 + bb]);
      cs[bb] = m / float(Q);
      inv[bb] = m > 0.f ? float(Q) / m : 0.f;
    }
  }
  uint8_t* cb = static_cast<uint8_t*>(a.codes) + size_t(bh) * HB;
#pragma unroll
  for (int bb = 0; bb < CB; ++bb) {
    const int j = j0 + bb;
    int code[RB];
#pragma unroll
    for (int x = 0; x < RB; ++x) {
      // M inv + 1.5 2^23 rounds once to the nearest integer, ties to even,
      // and the low bits of the sum's pattern are that integer in two's
      // complement. No clamp: |M| is at most its column's maximum, so
      // |M inv| <= Q (1 + 2^-24) < Q + 1/2.
      code[x] = int(__float_as_uint(fmaf(M[x >> 2][bb][x & 3], inv[bb], 12582912.f)) - 0x4B400000u);
    }
    if constexpr (BITS == 6) {
      int hi[RB];
      uint32_t lo = 0;
#pragma unroll
      for (int x = 0; x < RB; ++x) {
        hi[x] = code[x] >> 2;  // arithmetic: floor(code / 4)
        lo |= uint32_t(code[x] & 3) << lo_bit((i0 + x) & 15);
      }
      store_codes<RB, 4>(cb + size_t(j) * (D / 2) + i0 / 2, hi);
      // a 16-channel group's low bits are one word; below D = 128 the threads
      // of a group (ti, ti ^ 1 [, ti ^ 2]) sit at lanes l ^ 16 (and l ^ 32)
      if constexpr (RB <= 8) lo = or_swap16(lo);
      if constexpr (RB <= 4) lo = or_swap32(lo);
      if (ti % (16 / RB) == 0) *reinterpret_cast<uint32_t*>(cb + lo_word<D>(j, i0 / 16)) = lo;
    } else {
      store_codes<RB, BITS>(cb + size_t(j) * (D * BITS / 8) + i0 * BITS / 8, code);
    }
  }
  if constexpr (RB == 16) {
    a.s[hD + i0 + tj] = sa[0];
  } else {
    if (tj == 0) storeB<RB>(a.s + hD + i0, sa);
  }
  if constexpr (CB >= 4) {
    if (wave == 0) {
#pragma unroll
      for (int m = 0; m < NV; ++m) a.c[hD + j0 + (lane >> 4) * NV + m] = cs[m];
    }
  } else {
    if (ti == 0) storeB<CB>(a.c + hD + j0, cs);
  }
  if (t == 0) a.blen[bh] = 0;
}

template <int D, int BITS, bool KDA, bool DENSE>
hipError_t launch(const CloseArgs& a, int n_blocks, hipStream_t stream) {
  hipLaunchKernelGGL((close_kernel<D, BITS, KDA, DENSE>), dim3(n_blocks), dim3(NT), 0, stream, a);
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
