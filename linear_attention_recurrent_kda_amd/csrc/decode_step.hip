// LeapQuant decode step for GDN / KDA recurrent states on gfx950.
//
// Per-window quantization (LeapQuant abstract; wink.run article, first
// technique): inside a window the low-bit state is fixed and each token's
// update is buffered in fp32; the token's output is read from the fixed state
// plus the buffered updates. Compensators are rank-one terms of the same form
// as token updates sitting at window position 0 (abstract; article, second
// technique). The gated delta rule itself follows Gated DeltaNet (Yang et al.)
// and Kimi Delta Attention (Kimi Linear report).
//
// One workgroup of 2*D threads per head. For D = 128 the code matrix is
// [d_v][d_k] int8 = 128 columns of 128 bytes: eight lanes read one column with
// 16-byte loads (64 lanes cover eight consecutive columns = 1 KiB), each lane
// owns key channels [16*li, 16*li+16). Every code feeds two FMAs, one for the
// key readout and one for the query readout, so the whole residual is read from
// HBM once per token. Partial dots are reduced over the eight lanes with DPP.
#include "lq_common.h"
#include "lq_launch.h"

namespace lq {

namespace {

constexpr int MAX_COMP = 8;
constexpr int MAX_WMAX = 64;
constexpr int MAX_ROWS = MAX_COMP + MAX_WMAX + 1;  // compensators, buffer entries, the k.q row
constexpr int PF = 10;                             // value rows prefetched per thread

template <int BITS>
struct CodeChunk;  // the codes of 16 consecutive key channels
template <>
struct CodeChunk<8> {
  using T = uint4;
};
template <>
struct CodeChunk<4> {
  using T = uint2;
};

// Codes are stored two's complement; xor with the sign bit turns them into
// unsigned code + 128 (int8) or code + 8 (int4) so one ubyte convert decodes a
// value. The offset times sum(z) is removed afterwards.
__device__ __forceinline__ void acc_u8x4(uint32_t w, const float* zk, const float* zq, float& ak,
                                         float& aq) {
  const uint32_t u = w ^ 0x80808080u;
  const float c0 = float(u & 0xFFu), c1 = float((u >> 8) & 0xFFu);
  const float c2 = float((u >> 16) & 0xFFu), c3 = float(u >> 24);
  ak = fmaf(c0, zk[0], ak);
  aq = fmaf(c0, zq[0], aq);
  ak = fmaf(c1, zk[1], ak);
  aq = fmaf(c1, zq[1], aq);
  ak = fmaf(c2, zk[2], ak);
  aq = fmaf(c2, zq[2], aq);
  ak = fmaf(c3, zk[3], ak);
  aq = fmaf(c3, zq[3], aq);
}

// Eight int4 codes: byte m holds key channel 2m (low nibble) and 2m+1 (high).
__device__ __forceinline__ void acc_u4x8(uint32_t w, const float* zk, const float* zq, float& ak,
                                         float& aq) {
  const uint32_t u = w ^ 0x88888888u;
  const uint32_t lo = u & 0x0F0F0F0Fu, hi = (u >> 4) & 0x0F0F0F0Fu;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const float e = float((lo >> (8 * m)) & 0xFFu), o = float((hi >> (8 * m)) & 0xFFu);
    ak = fmaf(e, zk[2 * m], ak);
    aq = fmaf(e, zq[2 * m], aq);
    ak = fmaf(o, zk[2 * m + 1], ak);
    aq = fmaf(o, zq[2 * m + 1], aq);
  }
}

__device__ __forceinline__ void lds16(const float* p, float (&x)[16]) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float4 t = reinterpret_cast<const float4*>(p)[w];
    x[4 * w] = t.x;
    x[4 * w + 1] = t.y;
    x[4 * w + 2] = t.z;
    x[4 * w + 3] = t.w;
  }
}

template <int D, int BITS, bool KDA, bool BF16>
__global__ void __launch_bounds__(2 * D) decode_step_kernel(StepArgs a) {
  constexpr int NT = 2 * D;
  constexpr int LPC = D / 16;     // lanes per value column
  constexpr int NG = NT / LPC;    // column groups per workgroup (32)
  constexpr int CPT = D / NG;     // value columns per thread
  constexpr int CB = D * BITS / 8;  // code bytes per value column
  constexpr float OFF = BITS == 8 ? 128.f : 8.f;
  using CT = typename CodeChunk<BITS>::T;

  __shared__ __align__(16) float s_z[2][D];   // s (.) exp(G_t) (.) x   for x = k, q
  __shared__ __align__(16) float s_xb[2][D];  // exp(G_t) (.) x
  __shared__ __align__(16) float s_x[2][D];   // x
  __shared__ __align__(16) float s_G[KDA ? D : 4];
  __shared__ float s_y[2][D];                 // code readout c_j * sum_i C_ij z_i
  __shared__ float s_p[2][D];                 // value-side partial sums of the upper half
  __shared__ float s_kap[2][MAX_ROWS];
  __shared__ float s_kq;

  const int bh = blockIdx.x;
  const int t = threadIdx.x;
  const int grp = t / LPC, li = t % LPC, i0 = li * 16;
  const int r = a.r, w_max = a.w_max;
  const size_t hD = size_t(bh) * D;
  const size_t brow = size_t(bh) * w_max;  // first buffer row of this head

  // (1) issue the residual loads first: CPT columns x 16 key channels
  const uint8_t* cbase = static_cast<const uint8_t*>(a.codes) + hD * CB + i0 * BITS / 8;
  CT cw[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) cw[c] = *reinterpret_cast<const CT*>(cbase + size_t(grp + NG * c) * CB);
  float cj[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) cj[c] = a.c[hD + grp + NG * c];

  const int n = a.blen[bh];
  if (n >= w_max || n < 0) {  // precondition violated: leave the head untouched
    if (t == 0 && a.err) atomicOr(a.err, n < 0 ? LQ_DEVERR_BAD_LEN : LQ_DEVERR_BUFFER_FULL);
    return;
  }
  const int E = r + n;  // key rows: r compensators then n buffered tokens

  float G = 0.f;  // GDN: cumulative log-decay of this token since the window start
  if constexpr (!KDA) G = (n > 0 ? a.bg[brow + n - 1] : 0.f) + a.g[bh];

  // (2) per key channel: x, exp(G_t) (.) x, s (.) exp(G_t) (.) x
  float vj = 0.f, beta = 0.f;
  if (t < D) {
    const int i = t;
    const float kx = load_act<BF16>(a.k, hD + i);
    const float qx = load_act<BF16>(a.q, hD + i);
    const float si = a.s[hD + i];
    float e;
    if constexpr (KDA) {
      const float Gi = (n > 0 ? a.bg[(brow + n - 1) * D + i] : 0.f) + a.g[hD + i];
      s_G[i] = Gi;
      e = expf(Gi);
    } else {
      e = expf(G);
    }
    const float kb = e * kx, qb = e * qx;
    s_x[0][i] = kx;
    s_x[1][i] = qx;
    s_xb[0][i] = kb;
    s_xb[1][i] = qb;
    s_z[0][i] = si * kb;
    s_z[1][i] = si * qb;
    vj = load_act<BF16>(a.v, hD + i);
    beta = a.beta[bh];
  }

  // (3) prefetch the first chunk of key rows and this thread's value rows
  auto key_row = [&](int e) -> const float* {
    return e < r ? a.ck + (size_t(bh) * r + e) * D : a.bk + (brow + (e - r)) * D;
  };
  float kr[16], gr[16];
  float Gm = 0.f;
#pragma unroll
  for (int x = 0; x < 16; ++x) kr[x] = gr[x] = 0.f;
  if (grp < E) {
    load16(key_row(grp) + i0, kr);
    if (grp >= r) {
      if constexpr (KDA) load16(a.bg + (brow + (grp - r)) * D + i0, gr);
      else Gm = a.bg[brow + (grp - r)];
    }
  }
  const int j = t % D, half = t / D;
  auto val_row = [&](int e) -> float {
    return e < r ? a.cu[(size_t(bh) * r + e) * D + j] : a.bu[(brow + (e - r)) * D + j];
  };
  float uv[PF];
#pragma unroll
  for (int p = 0; p < PF; ++p) {
    const int e = half + 2 * p;
    uv[p] = e < E ? val_row(e) : 0.f;
  }

  __syncthreads();

  // (4) residual readout: y^x_j = c_j * sum_i C_ij z^x_i for both x in one pass
  {
    float zk[16], zq[16];
    lds16(&s_z[0][i0], zk);
    lds16(&s_z[1][i0], zq);
    float Zk = 0.f, Zq = 0.f;
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      Zk += zk[x];
      Zq += zq[x];
    }
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      float ak = 0.f, aq = 0.f;
      if constexpr (BITS == 8) {
        acc_u8x4(cw[c].x, zk + 0, zq + 0, ak, aq);
        acc_u8x4(cw[c].y, zk + 4, zq + 4, ak, aq);
        acc_u8x4(cw[c].z, zk + 8, zq + 8, ak, aq);
        acc_u8x4(cw[c].w, zk + 12, zq + 12, ak, aq);
      } else {
        acc_u4x8(cw[c].x, zk + 0, zq + 0, ak, aq);
        acc_u4x8(cw[c].y, zk + 8, zq + 8, ak, aq);
      }
      ak = fmaf(-OFF, Zk, ak);
      aq = fmaf(-OFF, Zq, aq);
      ak = group_sum<LPC>(ak);
      aq = group_sum<LPC>(aq);
      if (li == 0) {
        s_y[0][grp + NG * c] = cj[c] * ak;
        s_y[1][grp + NG * c] = cj[c] * aq;
      }
    }
  }

  // (5) key-side dots. Row e < r: compensator key . (exp(G_t) (.) x);
  // r <= e < E: buffered key . (exp(G_t - G_m) (.) x); e == E: k_t . q_t.
  for (int e0 = 0; e0 <= E; e0 += NG) {
    const int e = e0 + grp;
    if (e0 > 0) {
#pragma unroll
      for (int x = 0; x < 16; ++x) kr[x] = 0.f;
      if (e < E) {
        load16(key_row(e) + i0, kr);
        if (e >= r) {
          if constexpr (KDA) load16(a.bg + (brow + (e - r)) * D + i0, gr);
          else Gm = a.bg[brow + (e - r)];
        }
      }
    }
    float dk = 0.f, dq = 0.f;
    if (e < r) {
      float xk[16], xq[16];
      lds16(&s_xb[0][i0], xk);
      lds16(&s_xb[1][i0], xq);
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        dk = fmaf(kr[x], xk[x], dk);
        dq = fmaf(kr[x], xq[x], dq);
      }
    } else if (e < E) {
      float xk[16], xq[16];
      lds16(&s_x[0][i0], xk);
      lds16(&s_x[1][i0], xq);
      if constexpr (KDA) {
        float Gt[16];
        lds16(&s_G[i0], Gt);
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          const float f = expf(Gt[x] - gr[x]) * kr[x];
          dk = fmaf(f, xk[x], dk);
          dq = fmaf(f, xq[x], dq);
        }
      } else {
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          dk = fmaf(kr[x], xk[x], dk);
          dq = fmaf(kr[x], xq[x], dq);
        }
      }
    } else if (e == E) {
      float xk[16], xq[16];
      lds16(&s_x[0][i0], xk);
      lds16(&s_x[1][i0], xq);
#pragma unroll
      for (int x = 0; x < 16; ++x) dk = fmaf(xk[x], xq[x], dk);
    }
    dk = group_sum<LPC>(dk);
    dq = group_sum<LPC>(dq);
    if (li == 0) {
      if (e < E) {
        if constexpr (!KDA) {
          if (e >= r) {
            const float f = expf(G - Gm);
            dk *= f;
            dq *= f;
          }
        }
        s_kap[0][e] = dk;
        s_kap[1][e] = dq;
      } else if (e == E) {
        s_kq = dk;
      }
    }
  }
  __syncthreads();

  // (6) value-side sums: y^x_j += sum_e U_e[j] kappa^x_e, entries split between
  // the two halves of the workgroup (half h takes e = h, h+2, ...)
  float pk = 0.f, pq = 0.f;
#pragma unroll
  for (int p = 0; p < PF; ++p) {
    const int e = half + 2 * p;
    if (e < E) {
      pk = fmaf(uv[p], s_kap[0][e], pk);
      pq = fmaf(uv[p], s_kap[1][e], pq);
    }
  }
  for (int e = half + 2 * PF; e < E; e += 2) {
    const float u = val_row(e);
    pk = fmaf(u, s_kap[0][e], pk);
    pq = fmaf(u, s_kap[1][e], pq);
  }
  if (half == 1) {
    s_p[0][j] = pk;
    s_p[1][j] = pq;
  }
  __syncthreads();

  // (7) delta, output, append (k_t, u_t, G_t) to the window buffer
  const size_t slot = brow + n;
  if (half == 0) {
    const float yk = s_y[0][j] + (pk + s_p[0][j]);
    const float yq = s_y[1][j] + (pq + s_p[1][j]);
    const float u = beta * (vj - yk);
    a.o[hD + j] = yq + s_kq * u;
    a.bu[slot * D + j] = u;
  } else {
    a.bk[slot * D + j] = s_x[0][j];
    if constexpr (KDA) a.bg[slot * D + j] = s_G[j];
  }
  if (t == 0) {
    if constexpr (!KDA) a.bg[slot] = G;
    a.blen[bh] = n + 1;
  }
}

template <int D, int BITS, bool KDA, bool BF16>
hipError_t launch(const lq_dims& d, const StepArgs& a, hipStream_t stream) {
  const int blocks = d.batch * d.heads;
  hipLaunchKernelGGL((decode_step_kernel<D, BITS, KDA, BF16>), dim3(blocks), dim3(2 * D), 0, stream, a);
  return hipGetLastError();
}

template <int D, int BITS>
hipError_t launch_db(const lq_dims& d, const StepArgs& a, hipStream_t s) {
  const bool kda = d.decay_per_channel != 0, bf16 = d.act_dtype == LQ_ACT_BF16;
  if (kda) return bf16 ? launch<D, BITS, true, true>(d, a, s) : launch<D, BITS, true, false>(d, a, s);
  return bf16 ? launch<D, BITS, false, true>(d, a, s) : launch<D, BITS, false, false>(d, a, s);
}

template <int D>
hipError_t launch_d(const lq_dims& d, const StepArgs& a, hipStream_t s) {
  return d.bits == 8 ? launch_db<D, 8>(d, a, s) : launch_db<D, 4>(d, a, s);
}

}  // namespace

hipError_t launch_decode_step(const lq_dims& d, const StepArgs& a, hipStream_t stream) {
  switch (d.d_k) {
    case 32: return launch_d<32>(d, a, stream);
    case 64: return launch_d<64>(d, a, stream);
    default: return launch_d<128>(d, a, stream);
  }
}

}  // namespace lq
