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

// N consecutive fp32 values (N in 2, 4, 8) from a 4N-byte aligned address
// (global or LDS).
template <int N>
__device__ __forceinline__ void loadN(const float* p, float (&x)[N]) {
  if constexpr (N == 2) {
    const float2 t = *reinterpret_cast<const float2*>(p);
    x[0] = t.x, x[1] = t.y;
  } else {
#pragma unroll
    for (int w = 0; w < N / 4; ++w) {
      const float4 t = reinterpret_cast<const float4*>(p)[w];
      x[4 * w] = t.x, x[4 * w + 1] = t.y, x[4 * w + 2] = t.z, x[4 * w + 3] = t.w;
    }
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
  static constexpr int CPL = D / 16;              // key channels per lane in the key-side dots
  static constexpr int NG = NT / 16;              // key-row lane groups (16 lanes per row)
  static constexpr int NQ = D / 4;                // value-column quads (value sums, outputs)
  static constexpr int EP = NT / NQ;              // entry phases sharing one quad
  static constexpr int PRE = 24;                  // entries whose rows are prefetched into registers
  static constexpr int KPF = PRE / NG;            // key rows per lane group prefetched
  static constexpr int PFE = PRE / EP;            // value rows per thread prefetched
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

template <bool BF16>
__device__ __forceinline__ float4 load_act4(const void* p, size_t idx) {  // idx multiple of 4
  if constexpr (BF16) {
    const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + idx);
    return make_float4(bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y));
  } else {
    return *reinterpret_cast<const float4*>(static_cast<const float*>(p) + idx);
  }
}

template <int D, int BITS, bool KDA, bool BF16>
__global__ void __launch_bounds__((StepShape<D, KDA>::NT)) decode_step_kernel(StepArgs a) {
  using SS = StepShape<D, KDA>;
  constexpr int NT = SS::NT, NW = SS::NW, RBW = SS::RBW, KB = SS::KB, CPL = SS::CPL, NG = SS::NG;
  constexpr int KPF = SS::KPF, NQ = SS::NQ, EP = SS::EP, PFE = SS::PFE;
  constexpr int CB = D * BITS / 8;  // code bytes per value column
  constexpr float L2E = 1.4426950408889634f;
  using CL = CodeLoad<BITS>;
  using CT = typename CL::T;

  __shared__ __align__(16) float s_x[2][D];         // x for x = k, q
  __shared__ __align__(16) float s_G[KDA ? D : 4];  // KDA: G_t per key channel
  __shared__ __align__(16) int8_t s_B[KB][16][64];  // MFMA B operand: z limbs
  __shared__ __align__(16) float s_c[D];            // value-column scales
  __shared__ __align__(16) float s_y[2][D];         // code readout
  __shared__ __align__(16) float s_vs[EP][2][D];    // value-side partial sums per entry phase
  __shared__ float s_kap[2][MAX_ROWS];              // kappa^k, kappa^q per entry
  __shared__ float s_red[3][NW];                    // per-wave k.q and max |z^x| (bits)

  const int bh = blockIdx.x;
  const int n = a.blen[bh];  // first: every entry address depends on it
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int grp = t / 16, li = t % 16, i0 = li * CPL;
  const int q4 = t % NQ, ph = t / NQ;  // value-column quad and entry phase
  const bool chan = NT == D || t < D;  // thread owns key channel t
  const int tc = chan ? t : 0;
  const int r = a.r, NE = r + a.w_max;
  const size_t hD = size_t(bh) * D;
  // this head's entry rows (per-lane offsets below stay 32-bit)
  float* const ekh = a.ek + size_t(bh) * NE * D;
  float* const euh = a.eu + size_t(bh) * NE * D;
  float* const egh = a.eg + size_t(bh) * NE * (KDA ? D : 1);

  // (1) loads that do not depend on the buffer length: residual codes in MFMA
  // A-operand order (lane -> value column 16*rb + lane%16, key channels
  // 64*kb + 16*(lane/16) .. +16), per-channel inputs, this thread's v quad
  CT cw[RBW][KB];
  {
    const int jl = lane & 15, il = 16 * (lane >> 4);
    const uint8_t* base = static_cast<const uint8_t*>(a.codes) + hD * CB;
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int j = 16 * (wave * RBW + rb) + jl, i = 64 * kb + il;
        if (i < D) cw[rb][kb] = *reinterpret_cast<const CT*>(base + j * CB + i * BITS / 8);
        else cw[rb][kb] = CT{};
      }
  }
  float kx = load_act<BF16>(a.k, hD + tc), qx = load_act<BF16>(a.q, hD + tc);
  const float si = a.s[hD + tc], cc = a.c[hD + tc];
  float gi = 0.f;
  if constexpr (KDA) gi = a.g[hD + tc];
  if (!chan) kx = qx = 0.f;
  const float4 v4 = load_act4<BF16>(a.v, hD + 4 * q4);
  const float beta = a.beta[bh];

  if (n >= a.w_max || n < 0) {  // precondition violated: leave the head untouched
    if (t == 0 && a.err) atomicOr(a.err, n < 0 ? LQ_DEVERR_BAD_LEN : LQ_DEVERR_BUFFER_FULL);
    return;
  }
  // entries e = 0..E-1: r compensators (window position 0, G = 0), then the n
  // buffered tokens; loads of entries past E are clamped to entry E-1 (or 0)
  const int E = r + n, elast = E > 0 ? E - 1 : 0;

  // (2) entry loads: this group's key rows (and their G), this thread's value rows
  float kr[KPF][CPL], gr[KDA ? KPF : 1][CPL], Gm[KPF];
#pragma unroll
  for (int k = 0; k < KPF; ++k) {
    const int e = grp + NG * k, ec = e < elast ? e : elast;
    loadN(ekh + ec * D + i0, kr[k]);
    if constexpr (KDA) loadN(egh + ec * D + i0, gr[k]);  // zero rows for compensators
    else Gm[k] = egh[ec];
  }
  float4 uv[PFE];
#pragma unroll
  for (int k = 0; k < PFE; ++k) {
    const int e = ph + EP * k, ec = e < elast ? e : elast;
    uv[k] = *reinterpret_cast<const float4*>(euh + ec * D + 4 * q4);
  }
  // G_{t-1}: G of the last entry (compensators carry 0), 0 with no entries
  float Gp = 0.f;
  if constexpr (KDA) Gp = E > 0 ? egh[(E - 1) * D + tc] : 0.f;
  else Gp = E > 0 ? egh[E - 1] : 0.f;
  const float G = KDA ? 0.f : Gp + a.g[bh];  // GDN: G_t

  // (3) per key channel: z^x = s (.) exp(G_t) (.) x, block max |z^x|, k_t . q_t
  const float Gi = KDA ? Gp + gi : G;
  const float eG = exp_fast(Gi);
  const float zk = si * (eG * kx), zq = si * (eG * qx);
  if (chan) {
    s_x[0][t] = kx;
    s_x[1][t] = qx;
    if constexpr (KDA) s_G[t] = Gi;
    s_c[t] = cc;
  }
  {
    const float kq = rows_sum(group_sum<16>(kx * qx));
    const uint32_t mk = rows_umax(group_umax<16>(as_u(fabsf(zk))));
    const uint32_t mq = rows_umax(group_umax<16>(as_u(fabsf(zq))));
    if (lane == 0) {
      s_red[0][wave] = kq;
      s_red[1][wave] = as_f(mk);
      s_red[2][wave] = as_f(mq);
    }
  }
  __syncthreads();

  // (4) z^x as a 30-bit fixed-point integer with a power-of-two block scale,
  // split into four signed 8-bit limbs: the MFMA B operand (columns 4x+l)
  float zscale[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    uint32_t mb = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) mb = max(mb, as_u(s_red[1 + x][w]));
    int ex = 0;
    frexpf(as_f(mb), &ex);             // max |z| < 2^ex
    zscale[x] = ldexpf(1.f, ex - 30);  // z = Z * zscale, |Z| < 2^30
    if (chan) {
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
  // (D = 32: the A operand is zero past channel D, so the B operand's unwritten
  // padding bytes never contribute)

  // (5) key-side dots: kappa^x_e = sum_i k_e,i exp(G_t,i - G_e,i) x_i
  // (GDN: the decay ratio is one scalar exp(G_t - G_e) applied after the sum)
  {
    float xk[CPL], xq[CPL], Gt[CPL];
    loadN(&s_x[0][i0], xk);
    loadN(&s_x[1][i0], xq);
    if constexpr (KDA) {
      loadN(&s_G[i0], Gt);
#pragma unroll
      for (int x = 0; x < CPL; ++x) Gt[x] *= L2E;
    }
    for (int e0 = 0; e0 < E; e0 += NG * KPF) {
#pragma unroll
      for (int k = 0; k < KPF; ++k) {
        const int e = e0 + grp + NG * k;
        float row[CPL], gm[CPL], gsc = Gm[k];
        if (e0 == 0) {
#pragma unroll
          for (int x = 0; x < CPL; ++x) {
            row[x] = kr[k][x];
            if constexpr (KDA) gm[x] = gr[k][x];
          }
        } else {  // entries beyond the prefetched ones (long windows)
          const int ec = e < elast ? e : elast;
          loadN(ekh + ec * D + i0, row);
          if constexpr (KDA) loadN(egh + ec * D + i0, gm);
          else gsc = egh[ec];
        }
        float dk = 0.f, dq = 0.f;
#pragma unroll
        for (int x = 0; x < CPL; ++x) {
          float f = row[x];
          if constexpr (KDA) f *= __builtin_amdgcn_exp2f(fmaf(gm[x], -L2E, Gt[x]));
          dk = fmaf(f, xk[x], dk);
          dq = fmaf(f, xq[x], dq);
        }
        dk = group_sum<16>(dk);
        dq = group_sum<16>(dq);
        if constexpr (!KDA) {
          const float f = exp_fast(G - gsc);
          dk *= f;
          dq *= f;
        }
        if (li == 0 && e < E) {
          s_kap[0][e] = dk;
          s_kap[1][e] = dq;
        }
      }
    }
  }
  __syncthreads();

  // (6) residual readout on the matrix cores: for every value column j and
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

  // (7) value-side sums: sum_e u_e[j] kappa^x_e for this thread's four value
  // columns over the entries of its phase (e = ph, ph + EP, ...)
  {
    float4 pk = make_float4(0.f, 0.f, 0.f, 0.f), pq = pk;
#pragma unroll
    for (int k = 0; k < PFE; ++k) {
      const int e = ph + EP * k;
      if (e < E) {
        const float ak = s_kap[0][e], aq = s_kap[1][e];
        pk.x = fmaf(uv[k].x, ak, pk.x), pk.y = fmaf(uv[k].y, ak, pk.y);
        pk.z = fmaf(uv[k].z, ak, pk.z), pk.w = fmaf(uv[k].w, ak, pk.w);
        pq.x = fmaf(uv[k].x, aq, pq.x), pq.y = fmaf(uv[k].y, aq, pq.y);
        pq.z = fmaf(uv[k].z, aq, pq.z), pq.w = fmaf(uv[k].w, aq, pq.w);
      }
    }
    for (int e = ph + EP * PFE; e < E; e += EP) {
      const float4 u = *reinterpret_cast<const float4*>(euh + e * D + 4 * q4);
      const float ak = s_kap[0][e], aq = s_kap[1][e];
      pk.x = fmaf(u.x, ak, pk.x), pk.y = fmaf(u.y, ak, pk.y), pk.z = fmaf(u.z, ak, pk.z), pk.w = fmaf(u.w, ak, pk.w);
      pq.x = fmaf(u.x, aq, pq.x), pq.y = fmaf(u.y, aq, pq.y), pq.z = fmaf(u.z, aq, pq.z), pq.w = fmaf(u.w, aq, pq.w);
    }
    *reinterpret_cast<float4*>(&s_vs[ph][0][4 * q4]) = pk;
    *reinterpret_cast<float4*>(&s_vs[ph][1][4 * q4]) = pq;
  }
  __syncthreads();

  // (8) delta, output, append (k_t, u_t, G_t) as entry E: one thread per
  // value-column quad
  if (t < NQ) {
    float kqs = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) kqs += s_red[0][w];
    float4 yk = *reinterpret_cast<const float4*>(&s_y[0][4 * q4]);
    float4 yq = *reinterpret_cast<const float4*>(&s_y[1][4 * q4]);
#pragma unroll
    for (int p = 0; p < EP; ++p) {
      const float4 a4 = *reinterpret_cast<const float4*>(&s_vs[p][0][4 * q4]);
      const float4 b4 = *reinterpret_cast<const float4*>(&s_vs[p][1][4 * q4]);
      yk.x += a4.x, yk.y += a4.y, yk.z += a4.z, yk.w += a4.w;
      yq.x += b4.x, yq.y += b4.y, yq.z += b4.z, yq.w += b4.w;
    }
    float4 u, o;
    u.x = beta * (v4.x - yk.x), u.y = beta * (v4.y - yk.y), u.z = beta * (v4.z - yk.z), u.w = beta * (v4.w - yk.w);
    o.x = fmaf(kqs, u.x, yq.x), o.y = fmaf(kqs, u.y, yq.y), o.z = fmaf(kqs, u.z, yq.z), o.w = fmaf(kqs, u.w, yq.w);
    *reinterpret_cast<float4*>(a.o + hD + 4 * q4) = o;
    *reinterpret_cast<float4*>(euh + E * D + 4 * q4) = u;
    *reinterpret_cast<float4*>(ekh + E * D + 4 * q4) = *reinterpret_cast<const float4*>(&s_x[0][4 * q4]);
    if constexpr (KDA)
      *reinterpret_cast<float4*>(egh + E * D + 4 * q4) = *reinterpret_cast<const float4*>(&s_G[4 * q4]);
    if (t == 0) {
      if constexpr (!KDA) egh[E] = G;
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
