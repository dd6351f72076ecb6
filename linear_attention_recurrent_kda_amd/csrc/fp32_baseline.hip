// FP32-state decode baseline and the dense dequantiser (gfx950).
//
// The baseline is one exact token of the gated delta rule (Gated DeltaNet,
// Yang et al.; per-channel decay as in Kimi Delta Attention) with the state
// kept in fp32, the format the LeapQuant pages compare against: per head it
// reads and writes the whole d_k x d_v state once.
//
// Layout [d_v][d_k] (the state transposed): value column j is d_k contiguous
// floats, so each column's update is independent:
//   u_j = beta (v_j - sum_i alpha_i S_ij k_i),
//   S_ij <- alpha_i S_ij + k_i u_j,   o_j = sum_i S_ij q_i.
// One workgroup of 2*D threads per head; D/16 lanes share a column and each
// lane owns 16 key channels as four 16-byte pieces. Piece w of lane li is
// float4 number (D/16) w + li of the column, so one load or store instruction
// of a column's lanes covers D contiguous bytes (whole cache lines); lanes
// holding interleaved channels only changes which partial sums meet in the
// cross-lane reduction. The state is streamed once per token, so its loads
// and stores carry the non-temporal hint.
#include "lq_common.h"
#include "lq_launch.h"

namespace lq {

namespace {

template <int D, bool KDA, bool BF16>
__global__ void __launch_bounds__(2 * D) baseline_kernel(BaselineArgs a) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  constexpr int NT = 2 * D;
  constexpr int LPC = D / 16;
  constexpr int NG = NT / LPC;
  constexpr int CPT = D / NG;
  __shared__ __align__(16) float s_k[D];
  __shared__ __align__(16) float s_q[D];
  __shared__ __align__(16) float s_al[KDA ? D : 4];

  const int bh = blockIdx.x, t = threadIdx.x;
  const int grp = t / LPC, li = t % LPC;
  const size_t hD = size_t(bh) * D;
  f4* const Sh = reinterpret_cast<f4*>(a.S + hD * D);
  // float4 index of piece w of this lane in column j
  auto at = [&](int j, int w) { return size_t(j) * (D / 4) + LPC * w + li; };

  f4 S[CPT][4];
#pragma unroll
  for (int c = 0; c < CPT; ++c)
#pragma unroll
    for (int w = 0; w < 4; ++w) S[c][w] = __builtin_nontemporal_load(Sh + at(grp + NG * c, w));
  float vj[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) vj[c] = load_act<BF16>(a.v, hD + grp + NG * c);
  const float beta = a.beta[bh];
  float alpha = 1.f;
  if constexpr (!KDA) alpha = expf(a.g[bh]);
  if (t < D) {
    s_k[t] = load_act<BF16>(a.k, hD + t);
    s_q[t] = load_act<BF16>(a.q, hD + t);
    if constexpr (KDA) s_al[t] = expf(a.g[hD + t]);
  }
  __syncthreads();

  // the same channels of k, q and the decay as the lane's pieces of S
  f4 kk[4], qq[4], al[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    kk[w] = reinterpret_cast<const f4*>(s_k)[LPC * w + li];
    qq[w] = reinterpret_cast<const f4*>(s_q)[LPC * w + li];
    if constexpr (KDA) al[w] = reinterpret_cast<const f4*>(s_al)[LPC * w + li];
    else al[w] = f4{alpha, alpha, alpha, alpha};
  }

#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    float dk = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        S[c][w][e] *= al[w][e];
        dk = fmaf(S[c][w][e], kk[w][e], dk);
      }
    dk = group_sum<LPC>(dk);
    const float u = beta * (vj[c] - dk);
    float dq = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        S[c][w][e] = fmaf(kk[w][e], u, S[c][w][e]);
        dq = fmaf(S[c][w][e], qq[w][e], dq);
      }
    dq = group_sum<LPC>(dq);
#pragma unroll
    for (int w = 0; w < 4; ++w) __builtin_nontemporal_store(S[c][w], Sh + at(grp + NG * c, w));
    if (li == 0) a.o[hD + grp + NG * c] = dq;
  }
}

// Shat_0 = sum_{l<r} k_l u_l^T + diag(s) C diag(c) (compensator entries plus
// residual), written [d_v][d_k].
template <int D, int BITS>
__global__ void __launch_bounds__(256) dequant_kernel(lq_state st, int r, int n_ent, float* out) {
  const int bh = blockIdx.x;
  const size_t hD = size_t(bh) * D, erow = size_t(bh) * n_ent;
  for (int idx = threadIdx.x; idx < D * D; idx += 256) {
    const int j = idx / D, i = idx % D;
    const uint8_t* head = static_cast<const uint8_t*>(st.codes) + size_t(bh) * (D * D * BITS / 8);
    int code;
    if constexpr (BITS == 8) {
      code = int(int8_t(head[j * D + i]));
    } else {
      const uint8_t byte = head[j * (D / 2) + i / 2];
      const uint32_t nib = (i & 1) ? (byte >> 4) : (byte & 0xFu);
      code = int(nib ^ 0x8u) - 8;
      if constexpr (BITS == 6) {  // nibble = hi; lo = 2-bit field of the second plane
        constexpr int NJ = D / 16;
        const int c = i & 15, p = (c & 1) ? 8 + (c >> 1) : (c >> 1);
        const uint32_t w = *reinterpret_cast<const uint32_t*>(
            head + D * D / 2 + 4 * (((j & 15) * NJ + (i >> 4)) * NJ + (j >> 4)));
        code = 4 * code + int((w >> (8 * (p & 3) + 2 * (p >> 2))) & 3u);
      }
    }
    float val = (st.row_scale[hD + i] * float(code)) * st.col_scale[hD + j];
    for (int l = 0; l < r; ++l) val = fmaf(st.ent_k[(erow + l) * D + i], st.ent_u[(erow + l) * D + j], val);
    out[(hD + j) * D + i] = val;
  }
}

template <int D, bool KDA, bool BF16>
hipError_t launch(const lq_dims& d, const BaselineArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((baseline_kernel<D, KDA, BF16>), dim3(d.batch * d.heads), dim3(2 * D), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const lq_dims& d, const BaselineArgs& a, hipStream_t s) {
  const bool kda = d.decay_per_channel != 0, bf16 = d.act_dtype == LQ_ACT_BF16;
  if (kda) return bf16 ? launch<D, true, true>(d, a, s) : launch<D, true, false>(d, a, s);
  return bf16 ? launch<D, false, true>(d, a, s) : launch<D, false, false>(d, a, s);
}

template <int D, int BITS>
hipError_t launch_dq(const lq_dims& d, const lq_state& st, float* out, hipStream_t stream) {
  hipLaunchKernelGGL((dequant_kernel<D, BITS>), dim3(d.batch * d.heads), dim3(256), 0, stream, st,
                     d.n_comp, d.n_comp + d.w_max, out);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dq_d(const lq_dims& d, const lq_state& st, float* out, hipStream_t s) {
  switch (d.bits) {
    case 8: return launch_dq<D, 8>(d, st, out, s);
    case 6: return launch_dq<D, 6>(d, st, out, s);
    default: return launch_dq<D, 4>(d, st, out, s);
  }
}

}  // namespace

hipError_t launch_baseline(const lq_dims& d, const BaselineArgs& a, hipStream_t stream) {
  switch (d.d_k) {
    case 32: return launch_d<32>(d, a, stream);
    case 64: return launch_d<64>(d, a, stream);
    default: return launch_d<128>(d, a, stream);
  }
}

hipError_t launch_dequantize(const lq_dims& d, const lq_state& st, float* out, hipStream_t stream) {
  switch (d.d_k) {
    case 32: return launch_dq_d<32>(d, st, out, stream);
    case 64: return launch_dq_d<64>(d, st, out, stream);
    default: return launch_dq_d<128>(d, st, out, stream);
  }
}

}  // namespace lq
