// Prefill for the LeapQuant handoff (gfx950): the exact gated delta rule over
// a prompt chunk with the state kept in fp32, so that decoding starts from a
// real prompt. The per-window quantization of the LeapQuant pages (wink.run
// article, per-window quantization; LeapQuant abstract) applies to the
// decoded tokens; the prompt runs at full precision and its final state is
// encoded once at the handoff (the encode entry point, launched after this
// kernel by the C ABI).
//
// One workgroup of 256 threads per head keeps the d_k x d_v state in
// registers for the whole chunk (16 x 16 thread grid, thread (ti, tj) holds
// key rows [ti*B, ti*B+B) and value columns [tj*B, tj*B+B), B = D/16), so the
// state is read and written once per chunk, not once per token. Per token,
// decay first (Gated DeltaNet scalar gate; Kimi Delta Attention per-channel
// gate):
//   S' = alpha (.)_rows S,  u = beta (v - S'^T k),  o = S'^T q + (k . q) u,
//   S = S' + k u^T
// (o = S^T q with S = S' + k u^T). The two column sums S'^T k and S'^T q and
// the partial k . q travel through LDS together: one barrier per token,
// double-buffered. The next token's inputs are loaded while the current one
// is computed.
#include "lq_common.h"
#include "lq_launch.h"

namespace lq {

namespace {

template <int N>
__device__ __forceinline__ void ld(const float* p, float (&x)[N]) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int w = 0; w < N / 4; ++w) {
      const float4 t = reinterpret_cast<const float4*>(p)[w];
      x[4 * w] = t.x, x[4 * w + 1] = t.y, x[4 * w + 2] = t.z, x[4 * w + 3] = t.w;
    }
  } else {
    const float2 t = *reinterpret_cast<const float2*>(p);
    x[0] = t.x, x[1] = t.y;
  }
}

template <int N>
__device__ __forceinline__ void st(float* p, const float (&x)[N]) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int w = 0; w < N / 4; ++w)
      reinterpret_cast<float4*>(p)[w] = make_float4(x[4 * w], x[4 * w + 1], x[4 * w + 2], x[4 * w + 3]);
  } else {
    *reinterpret_cast<float2*>(p) = make_float2(x[0], x[1]);
  }
}

// N consecutive activations (fp32 or bf16) starting at element idx.
template <int N, bool BF16>
__device__ __forceinline__ void ld_act(const void* p, size_t idx, float (&x)[N]) {
  if constexpr (BF16) {
    const uint16_t* b = static_cast<const uint16_t*>(p) + idx;
#pragma unroll
    for (int a = 0; a < N; ++a) x[a] = as_f(uint32_t(b[a]) << 16);
  } else {
    ld<N>(static_cast<const float*>(p) + idx, x);
  }
}

// One token's inputs as one thread needs them.
template <int B, bool KDA>
struct Tok {
  float k[B], q[B], v[B], g[KDA ? B : 1], beta;
};

template <int D, bool KDA, bool BF16>
__device__ __forceinline__ void load_tok(const PrefillArgs& a, int t, int bh, int i0, int j0,
                                         Tok<D / 16, KDA>& x) {
  constexpr int B = D / 16;
  const size_t row = (size_t(t) * a.n_heads + bh) * D;  // [token][head][channel]
  ld_act<B, BF16>(a.k, row + i0, x.k);
  ld_act<B, BF16>(a.q, row + i0, x.q);
  ld_act<B, BF16>(a.v, row + j0, x.v);
  if constexpr (KDA) ld<B>(a.g + row + i0, x.g);
  else x.g[0] = a.g[size_t(t) * a.n_heads + bh];
  x.beta = a.beta[size_t(t) * a.n_heads + bh];
}

template <int D, bool KDA, bool BF16>
__global__ void __launch_bounds__(256) prefill_kernel(PrefillArgs a) {
  constexpr int B = D / 16;
  __shared__ float sh_kq[2][4];       // per-wave partial k . q
  __shared__ float sh_p[2][4][2][D];  // per-wave column partials of S'^T k and S'^T q

  const int t = threadIdx.x, tj = t & 15, ti = t >> 4, lane = t & 63, wave = t >> 6;
  const int bh = blockIdx.x;
  const size_t hD = size_t(bh) * D;
  const int i0 = ti * B, j0 = tj * B;

  float M[B][B];  // M[x][c] = S[i0 + x][j0 + c]
#pragma unroll
  for (int c = 0; c < B; ++c) {
    float col[B];
    ld<B>(a.S + (hD + j0 + c) * D + i0, col);
#pragma unroll
    for (int x = 0; x < B; ++x) M[x][c] = col[x];
  }

  Tok<B, KDA> cur, nxt;
  if (a.n_tokens > 0) load_tok<D, KDA, BF16>(a, 0, bh, i0, j0, cur);
  int par = 0;
  for (int tt = 0; tt < a.n_tokens; ++tt) {
    if (tt + 1 < a.n_tokens) load_tok<D, KDA, BF16>(a, tt + 1, bh, i0, j0, nxt);
    // decay, then the column partials of S'^T k and S'^T q over this thread's rows
    float al[B];
#pragma unroll
    for (int x = 0; x < B; ++x) al[x] = exp_fast(KDA ? cur.g[x] : cur.g[0]);
    float pk[B], pq[B], kq = 0.f;
#pragma unroll
    for (int x = 0; x < B; ++x) kq = fmaf(cur.k[x], cur.q[x], kq);
#pragma unroll
    for (int c = 0; c < B; ++c) {
      float sk = 0.f, sq = 0.f;
#pragma unroll
      for (int x = 0; x < B; ++x) {
        M[x][c] *= al[x];
        sk = fmaf(M[x][c], cur.k[x], sk);
        sq = fmaf(M[x][c], cur.q[x], sq);
      }
      pk[c] = rows_sum(sk);
      pq[c] = rows_sum(sq);
    }
    kq = rows_sum(kq);  // the wave's four key-row groups
    if (lane < 16) {
      st<B>(&sh_p[par][wave][0][j0], pk);
      st<B>(&sh_p[par][wave][1][j0], pq);
      if (lane == 0) sh_kq[par][wave] = kq;
    }
    __syncthreads();
    const float kqs = (sh_kq[par][0] + sh_kq[par][1]) + (sh_kq[par][2] + sh_kq[par][3]);
    float u[B], o[B];
#pragma unroll
    for (int c = 0; c < B; ++c) {
      const int j = j0 + c;
      const float yk = (sh_p[par][0][0][j] + sh_p[par][1][0][j]) + (sh_p[par][2][0][j] + sh_p[par][3][0][j]);
      const float yq = (sh_p[par][0][1][j] + sh_p[par][1][1][j]) + (sh_p[par][2][1][j] + sh_p[par][3][1][j]);
      u[c] = cur.beta * (cur.v[c] - yk);
      o[c] = fmaf(kqs, u[c], yq);
    }
#pragma unroll
    for (int x = 0; x < B; ++x)
#pragma unroll
      for (int c = 0; c < B; ++c) M[x][c] = fmaf(cur.k[x], u[c], M[x][c]);
    if (ti == 0) st<B>(a.o + (size_t(tt) * a.n_heads + bh) * D + j0, o);
    par ^= 1;
    cur = nxt;
  }

#pragma unroll
  for (int c = 0; c < B; ++c) {
    float col[B];
#pragma unroll
    for (int x = 0; x < B; ++x) col[x] = M[x][c];
    st<B>(a.S + (hD + j0 + c) * D + i0, col);
  }
}

template <int D, bool KDA, bool BF16>
hipError_t launch(const lq_dims& d, const PrefillArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((prefill_kernel<D, KDA, BF16>), dim3(d.batch * d.heads), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const lq_dims& d, const PrefillArgs& a, hipStream_t s) {
  const bool kda = d.decay_per_channel != 0, bf16 = d.act_dtype == LQ_ACT_BF16;
  if (kda) return bf16 ? launch<D, true, true>(d, a, s) : launch<D, true, false>(d, a, s);
  return bf16 ? launch<D, false, true>(d, a, s) : launch<D, false, false>(d, a, s);
}

}  // namespace

hipError_t launch_prefill(const lq_dims& d, const PrefillArgs& a, hipStream_t stream) {
  switch (d.d_k) {
    case 32: return launch_d<32>(d, a, stream);
    case 64: return launch_d<64>(d, a, stream);
    default: return launch_d<128>(d, a, stream);
  }
}

}  // namespace lq
