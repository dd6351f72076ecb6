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
// One workgroup of D threads (two waves for D = 128) per head, small enough
// that every head of a 2048-head batch is resident at once. The residual
// readout y^x = C^T z^x for x in {k, q} is a dense int8 contraction and runs on
// the matrix cores: the codes, loaded straight from HBM in the MFMA operand
// layout (16 bytes per lane: 16 key channels of one value column), are the A
// operand of v_mfma_i32_16x16x64_i8; z^x is a 30-bit fixed-point vector with a
// power-of-two block scale, split into four signed 8-bit limbs that form the
// B operand's columns. The int32 accumulation is exact, so the only rounding
// is the fixed-point conversion of z (below fp32 accumulation error) and the
// final fp32 combination. int4 codes need no decode: a nibble masked into a
// byte's high half is the int8 16*code. Loads are issued in the order they are
// consumed (each lane group's key rows straight into registers, per-channel
// inputs, codes); the key-side dots run while the codes arrive.
#include "lq_common.h"
#include "lq_launch.h"

namespace lq {

namespace {

constexpr int MAX_COMP = 8;
constexpr int MAX_WMAX = 64;
constexpr int MAX_ROWS = MAX_COMP + MAX_WMAX + 1;  // compensators, buffer entries, the k.q row

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

typedef int v4i __attribute__((ext_vector_type(4)));

template <int D, bool KDA>
struct StepShape {
  static constexpr int NT = D >= 128 ? 128 : 64;  // threads per head
  static constexpr int NW = NT / 64;              // waves
  static constexpr int RB = D / 16;               // 16-column MFMA row blocks of the code matrix
  static constexpr int RBW = RB / NW;             // row blocks per wave
  static constexpr int KB = (D + 63) / 64;        // 64-channel MFMA k blocks
  static constexpr int LPC = D / 16;              // lanes per key row in the key-side dots
  static constexpr int NG = NT / LPC;             // key-row lane groups
  static constexpr int NH = NT / D;               // threads sharing one value column's sums
  static constexpr int KPF = KDA ? 1 : 2;         // key rows per group prefetched into registers
  static constexpr int PF = 24 / NH;              // value-row entries loaded per thread
};

// Code bytes one lane feeds to one MFMA: 16 key channels of one value column.
template <int BITS>
struct CodeLoad;
template <>
struct CodeLoad<8> {
  using T = uint4;
  __device__ static v4i operand(const T& w) { return v4i{int(w.x), int(w.y), int(w.z), int(w.w)}; }
};
template <>
struct CodeLoad<4> {
  using T = uint2;
  // Nibble n (two's complement) masked into a byte's high half is the int8
  // 16*n, exactly. Even channels (low nibbles) go first, then odd ones; the
  // MFMA's B operand is written in the same channel order.
  __device__ static v4i operand(const T& w) {
    return v4i{int((w.x << 4) & 0xF0F0F0F0u), int((w.y << 4) & 0xF0F0F0F0u), int(w.x & 0xF0F0F0F0u),
               int(w.y & 0xF0F0F0F0u)};
  }
};

// Byte position, inside a lane's 16-channel group, of channel c of that group.
template <int BITS>
__device__ __forceinline__ int chan_pos(int c) {
  if constexpr (BITS == 8) return c;
  else return (c & 1) ? 8 + (c >> 1) : (c >> 1);
}

template <int D, int BITS, bool KDA, bool BF16>
__global__ void __launch_bounds__((StepShape<D, KDA>::NT)) decode_step_kernel(StepArgs a) {
  using SS = StepShape<D, KDA>;
  constexpr int NT = SS::NT, NW = SS::NW, RBW = SS::RBW, KB = SS::KB, LPC = SS::LPC, NG = SS::NG;
  constexpr int NH = SS::NH, KPF = SS::KPF, PF = SS::PF;
  constexpr int CB = D * BITS / 8;  // code bytes per value column
  using CL = CodeLoad<BITS>;
  using CT = typename CL::T;

  __shared__ __align__(16) float s_x[2][D];                // x for x = k, q
  __shared__ __align__(16) float s_G[KDA ? D : 4];         // KDA: G_t per key channel
  __shared__ __align__(16) int8_t s_B[KB][16][64];         // MFMA B operand: z limbs
  __shared__ float s_c[D];                                 // value-column scales
  __shared__ float s_y[2][D];                              // code readout
  __shared__ float s_p[NH > 1 ? 2 : 1][D];                 // value-side partials of the other part
  __shared__ float s_kap[2][MAX_ROWS];                     // kappa^k, kappa^q per entry
  __shared__ float s_red[3][NW];                           // per-wave k.q and max |z^x|

  const int bh = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int grp = t / LPC, li = t % LPC, i0 = li * 16;
  const int r = a.r, w_max = a.w_max;
  const size_t hD = size_t(bh) * D;
  const size_t brow = size_t(bh) * w_max;  // first buffer row of this head

  const int n = a.blen[bh];
  if (n >= w_max || n < 0) {  // precondition violated: leave the head untouched
    if (t == 0 && a.err) atomicOr(a.err, n < 0 ? LQ_DEVERR_BAD_LEN : LQ_DEVERR_BUFFER_FULL);
    return;
  }
  // entries e = 0..E-1: r compensators (window position 0, G = 0), then the
  // n buffered tokens (G = G_m)
  const int E = r + n;
  auto key_row = [&](int e) -> const float* {
    return e < r ? a.ck + (size_t(bh) * r + e) * D : a.bk + (brow + (e - r)) * D;
  };

  // (1) issue the head's loads in the order they are consumed: this group's
  // key rows, per-channel inputs, residual codes. Loads return in order, so the
  // key-side dots do not wait for the codes.
  float kr[KPF][16], gr[KPF][16];
#pragma unroll
  for (int q = 0; q < KPF; ++q) {
    const int e = grp + NG * q;
#pragma unroll
    for (int x = 0; x < 16; ++x) kr[q][x] = gr[q][x] = 0.f;
    if (e < E) {
      load16(key_row(e) + i0, kr[q]);
      if constexpr (KDA)
        if (e >= r) load16(a.bg + (brow + (e - r)) * D + i0, gr[q]);
    }
  }
  float Gm[KPF];
#pragma unroll
  for (int q = 0; q < KPF; ++q) {
    const int e = grp + NG * q;
    Gm[q] = (!KDA && e >= r && e < E) ? a.bg[brow + (e - r)] : 0.f;
  }
  float kx = 0.f, qx = 0.f, si = 0.f, vj = 0.f, gi = 0.f, Gp = 0.f, cc = 0.f;
  if (t < D) {
    kx = load_act<BF16>(a.k, hD + t);
    qx = load_act<BF16>(a.q, hD + t);
    si = a.s[hD + t];
    vj = load_act<BF16>(a.v, hD + t);
    cc = a.c[hD + t];
    if constexpr (KDA) {
      gi = a.g[hD + t];
      Gp = n > 0 ? a.bg[(brow + n - 1) * D + t] : 0.f;
    }
  }
  float G = 0.f;  // GDN: cumulative log-decay of this token since the window start
  if constexpr (!KDA) G = (n > 0 ? a.bg[brow + n - 1] : 0.f) + a.g[bh];
  const float beta = a.beta[bh];
  // residual codes in MFMA A-operand order: lane -> value column 16*rb + lane%16,
  // key channels 64*kb + 16*(lane/16) .. +16
  CT cw[RBW][KB];
  {
    const int jl = lane & 15, il = 16 * (lane >> 4);
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int j = 16 * (wave * RBW + rb) + jl, i = 64 * kb + il;
        if (i < D) cw[rb][kb] = *reinterpret_cast<const CT*>(static_cast<const uint8_t*>(a.codes) + hD * CB +
                                                           size_t(j) * CB + i * BITS / 8);
        else cw[rb][kb] = CT{};
      }
  }

  // (2) per key channel: z^x = s (.) exp(G_t) (.) x, the block max |z^x|, k_t . q_t
  float zk = 0.f, zq = 0.f, Gi = 0.f;
  if (t < D) {
    Gi = KDA ? Gp + gi : G;
    const float e = expf(Gi);
    zk = si * (e * kx);
    zq = si * (e * qx);
    s_x[0][t] = kx;
    s_x[1][t] = qx;
    if constexpr (KDA) s_G[t] = Gi;
    s_c[t] = cc;
  }
  {
    const float kq = rows_sum(group_sum<16>(kx * qx));
    const float mk = rows_max(group_max<16>(fabsf(zk)));
    const float mq = rows_max(group_max<16>(fabsf(zq)));
    if (lane == 0) {
      s_red[0][wave] = kq;
      s_red[1][wave] = mk;
      s_red[2][wave] = mq;
    }
  }
  __syncthreads();

  // (3) z^x as a 30-bit fixed-point integer with a power-of-two block scale,
  // split into four signed 8-bit limbs: the MFMA B operand (columns 4x+l)
  float zscale[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    float m = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) m = fmaxf(m, s_red[1 + x][w]);
    int ex = 0;
    frexpf(m, &ex);                 // m < 2^ex
    zscale[x] = ldexpf(1.f, ex - 30);  // z = Z * zscale, |Z| < 2^30
    if (t < D) {
      const int Z = int(rintf(ldexpf(x == 0 ? zk : zq, 30 - ex)));
      const int l0 = int(int8_t(Z & 0xFF));
      const int z1 = (Z - l0) >> 8;
      const int l1 = int(int8_t(z1 & 0xFF));
      const int z2 = (z1 - l1) >> 8;
      const int l2 = int(int8_t(z2 & 0xFF));
      const int l3 = (z2 - l2) >> 8;
      const int kb = t >> 6, pos = (t & 48) | chan_pos<BITS>(t & 15);
      s_B[kb][4 * x + 0][pos] = int8_t(l0);
      s_B[kb][4 * x + 1][pos] = int8_t(l1);
      s_B[kb][4 * x + 2][pos] = int8_t(l2);
      s_B[kb][4 * x + 3][pos] = int8_t(l3);
    }
  }
  if constexpr (D < 64) {  // the upper half of the single k block is padding
    for (int idx = t; idx < 16 * 64; idx += NT)
      if ((idx & 63) >= D) s_B[0][idx >> 6][idx & 63] = 0;
  }

  // (4) key-side dots while the codes are still arriving:
  //   kappa^x_e = sum_i k_e,i exp(G_t,i - G_e,i) x_i
  // (GDN: the decay ratio is one scalar exp(G_t - G_e) applied after the sum)
  {
    float xk[16], xq[16], Gt[16];
    lds16(&s_x[0][i0], xk);
    lds16(&s_x[1][i0], xq);
    if constexpr (KDA) lds16(&s_G[i0], Gt);
    for (int e0 = 0; e0 < E; e0 += NG * KPF) {
#pragma unroll
      for (int q = 0; q < KPF; ++q) {
        const int e = e0 + grp + NG * q;
        float row[16], gm[16];
        if (e0 == 0) {
#pragma unroll
          for (int x = 0; x < 16; ++x) row[x] = kr[q][x], gm[x] = gr[q][x];
        } else {
#pragma unroll
          for (int x = 0; x < 16; ++x) row[x] = gm[x] = 0.f;
          if (e < E) {
            load16(key_row(e) + i0, row);
            if constexpr (KDA)
              if (e >= r) load16(a.bg + (brow + (e - r)) * D + i0, gm);
          }
        }
        float dk = 0.f, dq = 0.f;
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          float f = row[x];
          if constexpr (KDA) f *= expf(Gt[x] - gm[x]);
          dk = fmaf(f, xk[x], dk);
          dq = fmaf(f, xq[x], dq);
        }
        dk = group_sum<LPC>(dk);
        dq = group_sum<LPC>(dq);
        if (li == 0 && e < E) {
          if constexpr (!KDA) {
            const float gme = e0 == 0 ? Gm[q] : (e >= r ? a.bg[brow + (e - r)] : 0.f);
            const float f = expf(G - gme);
            dk *= f;
            dq *= f;
          }
          s_kap[0][e] = dk;
          s_kap[1][e] = dq;
        }
      }
    }
  }

  // value rows for the sums after the readout (clamped, so every load is valid)
  const int j = t % D, part = t / D;
  auto val_row = [&](int e) -> float {  // entry e in 0..E-1
    return e < r ? a.cu[(size_t(bh) * r + e) * D + j] : a.bu[(brow + (e - r)) * D + j];
  };
  float uv[PF];
  {
    const int elast = E > 0 ? E - 1 : 0;
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int e = part + NH * p;
      uv[p] = E > 0 ? val_row(e < elast ? e : elast) : 0.f;
    }
  }
  __syncthreads();

  // (5) residual readout on the matrix cores: for every value column j and
  // x in {k, q}, sum_i C_ij Z^x_i exactly in int32, limb by limb; then
  // y^x_j = c_j * zscale_x * sum_l 256^l D[j][4x+l]
  {
    v4i bop[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      bop[kb] = *reinterpret_cast<const v4i*>(&s_B[kb][lane & 15][16 * (lane >> 4)]);
    const int col = lane & 15, limb = lane & 3, xs = col >> 2;
    const float lw = float(1 << (8 * limb)) * (BITS == 4 ? 0.0625f : 1.f) * (xs == 0 ? zscale[0] : zscale[1]);
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
      v4i acc = {0, 0, 0, 0};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(CL::operand(cw[rb][kb]), bop[kb], acc, 0, 0, 0);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float f = float(acc[v]) * lw;
        f += dpp<DPP_QUAD_XOR1>(f);
        f += dpp<DPP_QUAD_XOR2>(f);
        const int jj = 16 * (wave * RBW + rb) + 4 * (lane >> 4) + v;
        if (limb == 0 && col < 8) s_y[xs][jj] = s_c[jj] * f;
      }
    }
  }
  __syncthreads();

  // (6) value-side sums: y^x_j += sum_e U_e[j] kappa^x_e (entries split over
  // the NH threads of a column)
  float pk = 0.f, pq = 0.f;
#pragma unroll
  for (int p = 0; p < PF; ++p) {
    const int e = part + NH * p;
    if (e < E) {
      pk = fmaf(uv[p], s_kap[0][e], pk);
      pq = fmaf(uv[p], s_kap[1][e], pq);
    }
  }
  for (int e = part + NH * PF; e < E; e += NH) {
    const float u = val_row(e);
    pk = fmaf(u, s_kap[0][e], pk);
    pq = fmaf(u, s_kap[1][e], pq);
  }
  if constexpr (NH > 1) {
    if (part == 1) {
      s_p[0][j] = pk;
      s_p[1][j] = pq;
    }
    __syncthreads();
    if (part == 0) {
      pk += s_p[0][j];
      pq += s_p[1][j];
    }
  }

  // (7) delta, output, append (k_t, u_t, G_t) to the window buffer
  if (part == 0) {
    float kqs = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) kqs += s_red[0][w];
    const float yk = s_y[0][j] + pk;
    const float yq = s_y[1][j] + pq;
    const float u = beta * (vj - yk);
    const size_t slot = brow + n;
    a.o[hD + j] = yq + kqs * u;
    a.bu[slot * D + j] = u;
    a.bk[slot * D + j] = s_x[0][j];
    if constexpr (KDA) a.bg[slot * D + j] = s_G[j];
    if (t == 0) {
      if constexpr (!KDA) a.bg[slot] = G;
      a.blen[bh] = n + 1;
    }
  }
}

template <int D, int BITS, bool KDA, bool BF16>
hipError_t launch(const lq_dims& d, const StepArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((decode_step_kernel<D, BITS, KDA, BF16>), dim3(d.batch * d.heads),
                     dim3((StepShape<D, KDA>::NT)), 0, stream, a);
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
