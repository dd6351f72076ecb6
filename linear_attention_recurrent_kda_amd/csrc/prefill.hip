// Prefill for the LeapQuant handoff (gfx950): the exact gated delta rule over
// a prompt chunk with the state kept in fp32, so that decoding starts from a
// real prompt. The per-window quantization of the LeapQuant pages (wink.run
// article, per-window quantization; LeapQuant abstract) applies to the
// decoded tokens; the prompt runs at full precision and its final state is
// encoded once at the handoff (the encode entry point, launched after this
// kernel by the C ABI).
//
// Per token, decay first (Gated DeltaNet scalar gate; Kimi Delta Attention
// per-channel gate):
//   S' = alpha (.)_rows S,  u = beta (v - S'^T k),  S = S' + k u^T,  o = S^T q
// (o = S'^T q + (k . q) u). Two kernels, both keeping the state in registers
// for the whole chunk (read and written once):
//
// - prefill_blocks_kernel (GDN at either activation type, and KDA with bf16
//   activations): 128 threads per head on an 8 x 16 grid, each with a block
//   of D/8 key rows by D/16 value columns; the column partials of S'^T k and
//   S'^T q and the partial k . q are summed over the wave's rows with the
//   row-swap instructions (the work split across the rows) and over the two
//   waves through LDS, one barrier per token, double-buffered; the next
//   token's inputs load (as raw bf16 pairs or fp32 words) while the current
//   one computes. GDN keeps the scalar decay as one scale per head.
// - prefill_columns_kernel (KDA with fp32 activations): every value column j
//   evolves on its own (u_j needs column j of S' and k; o_j column j of S and
//   q), so one thread owns one column, all d_k key rows, and a token costs it
//   two passes over its column with no exchange between threads. k, q and
//   beta are the same for every thread of a head and arrive through scalar
//   loads as instruction operands; the per-channel gates are exponentiated
//   two channels per lane and broadcast with readlane. One wave covers 64
//   columns of a head. (The blocks kernel spills at this instantiation.)
#include "lq_common.h"
#include "lq_launch.h"
#include "lq_rows.h"

namespace lq {

namespace {

// ---- bf16 activations: 128 threads per head, 16 x 8 register blocks

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

// N consecutive activations (N even) at element idx (even), kept as they are
// loaded: bf16 pairs in N/2 words, or N fp32 words.
template <int N, bool BF16>
struct Raw {
  uint32_t w[BF16 ? N / 2 : N];
};

// fp32 rows move in 16-byte pieces; bf16 rows in 8-byte pieces, the alignment
// the C ABI requires of bf16 activations.
template <int N, bool BF16>
__device__ __forceinline__ void ld_raw(const void* p, size_t idx, Raw<N, BF16>& r) {
  constexpr int NW = BF16 ? N / 2 : N;
  const uint32_t* b = static_cast<const uint32_t*>(p) + (BF16 ? idx / 2 : idx);
  if constexpr (BF16 && NW % 2 == 0) {
#pragma unroll
    for (int w = 0; w < NW / 2; ++w) {
      const uint2 t = reinterpret_cast<const uint2*>(b)[w];
      r.w[2 * w] = t.x, r.w[2 * w + 1] = t.y;
    }
  } else if constexpr (NW % 4 == 0) {
#pragma unroll
    for (int w = 0; w < NW / 4; ++w) {
      const uint4 t = reinterpret_cast<const uint4*>(b)[w];
      r.w[4 * w] = t.x, r.w[4 * w + 1] = t.y, r.w[4 * w + 2] = t.z, r.w[4 * w + 3] = t.w;
    }
  } else if constexpr (NW == 2) {
    const uint2 t = *reinterpret_cast<const uint2*>(b);
    r.w[0] = t.x, r.w[1] = t.y;
  } else {
    r.w[0] = b[0];
  }
}

template <int N, bool BF16>
__device__ __forceinline__ float raw_at(const Raw<N, BF16>& r, int a) {
  if constexpr (BF16) return (a & 1) ? bf16_hi(r.w[a / 2]) : bf16_lo(r.w[a / 2]);
  else return as_f(r.w[a]);
}

// One token's inputs as one thread needs them, as loaded.
template <int RB, int CB, bool KDA, bool BF16>
struct Tok {
  Raw<RB, BF16> k, q;
  Raw<CB, BF16> v;
  float g[KDA ? RB : 1], beta;
};

template <int D, bool KDA, bool BF16>
__device__ __forceinline__ void load_tok(const PrefillArgs& a, int t, int bh, int i0, int j0,
                                         Tok<D / 8, D / 16, KDA, BF16>& x) {
  constexpr int RB = D / 8, CB = D / 16;
  const size_t row = (size_t(t) * a.n_heads + bh) * D;  // [token][head][channel]
  ld_raw<RB, BF16>(a.k, row + i0, x.k);
  ld_raw<RB, BF16>(a.q, row + i0, x.q);
  ld_raw<CB, BF16>(a.v, row + j0, x.v);
  if constexpr (KDA) ld<RB>(a.g + row + i0, x.g);
  else x.g[0] = a.g[size_t(t) * a.n_heads + bh];
  x.beta = a.beta[size_t(t) * a.n_heads + bh];
}

template <int D, bool KDA, bool BF16>
__global__ void __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2))) prefill_blocks_kernel(PrefillArgs a) {
  constexpr int RB = D / 8, CB = D / 16;  // key rows and value columns per thread
  __shared__ float sh_kq[2][2];           // per-wave partial k . q (double-buffered)
  __shared__ __align__(16) float sh_p[2][2][2][D];  // per-wave column partials of S'^T k and S'^T q

  const int t = threadIdx.x, tj = t & 15, ti = t >> 4, lane = t & 63, wave = t >> 6;
  const int bh = blockIdx.x;
  const size_t hD = size_t(bh) * D;
  const int i0 = ti * RB, j0 = tj * CB;

  float M[RB][CB];  // M[x][c] = S[i0 + x][j0 + c]
#pragma unroll
  for (int c = 0; c < CB; ++c) {
    float col[RB];
    ld<RB>(a.S + (hD + j0 + c) * D + i0, col);
#pragma unroll
    for (int x = 0; x < RB; ++x) M[x][c] = col[x];
  }

  Tok<RB, CB, KDA, BF16> cur, nxt;
  if (a.n_tokens > 0) load_tok<D, KDA, BF16>(a, 0, bh, i0, j0, cur);
  int par = 0;
  // GDN: the state is S = gam * M, one scale per head, so a token's decay is
  // one multiply of gam instead of one per element; M is rescaled to S only
  // when gam falls below 2^-32 (and at the end)
  float gam = 1.f;
  for (int tt = 0; tt < a.n_tokens; ++tt) {
    if (tt + 1 < a.n_tokens) load_tok<D, KDA, BF16>(a, tt + 1, bh, i0, j0, nxt);
    float kx[RB], qx[RB];
#pragma unroll
    for (int x = 0; x < RB; ++x) kx[x] = raw_at(cur.k, x), qx[x] = raw_at(cur.q, x);
    // decay, then the column partials of S'^T k (pkq[c]) and S'^T q
    // (pkq[CB + c]) over this thread's rows
    float pkq[2 * CB], kq = 0.f;
#pragma unroll
    for (int x = 0; x < RB; ++x) kq = fmaf(kx[x], qx[x], kq);
#pragma unroll
    for (int c = 0; c < 2 * CB; ++c) pkq[c] = 0.f;
    if constexpr (!KDA) {
      gam *= exp_fast(cur.g[0]);
      if (!(gam >= 0x1p-32f)) {  // the same for every thread of the head
#pragma unroll
        for (int x = 0; x < RB; ++x)
#pragma unroll
          for (int c = 0; c < CB; ++c) M[x][c] *= gam;
        gam = 1.f;
      }
    }
#pragma unroll
    for (int x = 0; x < RB; ++x) {
      if constexpr (KDA) {
        const float al = exp_fast(cur.g[x]);
#pragma unroll
        for (int c = 0; c < CB; ++c) M[x][c] *= al;
      }
#pragma unroll
      for (int c = 0; c < CB; ++c) {
        pkq[c] = fmaf(M[x][c], kx[x], pkq[c]);
        pkq[CB + c] = fmaf(M[x][c], qx[x], pkq[CB + c]);
      }
    }
    // sums over key rows: the wave's four row groups with the work split
    // (lane row g ends with 2CB/4 consecutive sums: of S'^T k for g < 2, of
    // S'^T q for g >= 2), then the two waves through LDS
    {
      constexpr int NV = 2 * CB / 4;
      float tot[NV];
      rows_sum_split<2 * CB>(pkq, tot);
      const int g = lane >> 4;
      float* dst = &sh_p[par][wave][g >> 1][j0 + (g & 1) * NV];
      if constexpr (NV == 4) *reinterpret_cast<float4*>(dst) = make_float4(tot[0], tot[1], tot[2], tot[3]);
      else if constexpr (NV == 2) *reinterpret_cast<float2*>(dst) = make_float2(tot[0], tot[1]);
      else *dst = tot[0];
    }
    kq = rows_sum(kq);
    if (lane == 0) sh_kq[par][wave] = kq;
    __syncthreads();
    const float kqs = sh_kq[par][0] + sh_kq[par][1];
    float u[CB], o[CB];
#pragma unroll
    for (int c = 0; c < CB; ++c) {
      const int j = j0 + c;
      const float yk = gam * (sh_p[par][0][0][j] + sh_p[par][1][0][j]);
      const float yq = gam * (sh_p[par][0][1][j] + sh_p[par][1][1][j]);
      u[c] = cur.beta * (raw_at(cur.v, c) - yk);
      o[c] = fmaf(kqs, u[c], yq);
    }
    // S += k u^T, i.e. M += k (u / gam)^T
    float um[CB];
    const float ig = KDA ? 1.f : __builtin_amdgcn_rcpf(gam);
#pragma unroll
    for (int c = 0; c < CB; ++c) um[c] = KDA ? u[c] : u[c] * ig;
#pragma unroll
    for (int x = 0; x < RB; ++x)
#pragma unroll
      for (int c = 0; c < CB; ++c) M[x][c] = fmaf(kx[x], um[c], M[x][c]);
    if (ti == 0) st<CB>(a.o + (size_t(tt) * a.n_heads + bh) * D + j0, o);
    par ^= 1;
    cur = nxt;
  }

#pragma unroll
  for (int c = 0; c < CB; ++c) {
    float col[RB];
#pragma unroll
    for (int x = 0; x < RB; ++x) col[x] = KDA ? M[x][c] : M[x][c] * gam;
    st<RB>(a.S + (hD + j0 + c) * D + i0, col);
  }
}

// ---- fp32 activations: one thread per value column

// Read-only inputs seen through the constant address space: a load at a
// uniform address then goes through the scalar unit into SGPRs, where every
// lane reads it as an instruction operand.
template <typename T>
using cptr = const __attribute__((address_space(4))) T*;

template <typename T>
__device__ __forceinline__ cptr<T> as_const(const void* p) {
  return (cptr<T>)(p);
}

// Uniform activation value (fp32 or bf16) at element row + i, row even. The
// scalar unit loads whole dwords: a bf16 pair is read as one word and split.
template <bool BF16>
__device__ __forceinline__ float act_at(const void* p, size_t row, int i) {
  if constexpr (BF16) {
    const uint32_t w = as_const<uint32_t>(p)[(row + i) / 2];
    return (i & 1) ? bf16_hi(w) : bf16_lo(w);
  } else {
    return as_const<float>(p)[row + i];
  }
}

// Per-lane activation value (fp32 or bf16) at element idx.
template <bool BF16>
__device__ __forceinline__ float act_lane(const void* p, size_t idx) {
  if constexpr (BF16) return as_f(uint32_t(static_cast<const uint16_t*>(p)[idx]) << 16);
  else return static_cast<const float*>(p)[idx];
}

template <int D, bool KDA, bool BF16>
__global__ void __launch_bounds__(64) prefill_columns_kernel(PrefillArgs a) {
  static_assert(KDA, "per-channel decay only: GDN runs the blocks kernel");
  constexpr int WPH = D > 64 ? D / 64 : 1;  // waves per head
  const int lane = threadIdx.x;
  const int bh = blockIdx.x / WPH;
  const int j = (blockIdx.x % WPH) * 64 + lane;  // this thread's value column
  const bool col = D >= 64 || j < D;            // D = 32: the upper half-wave idles
  const size_t hD = size_t(bh) * D;

  float M[D];  // M[i] = S[i][j]
  if (col) {
#pragma unroll
    for (int w = 0; w < D / 4; ++w) {
      const float4 t = reinterpret_cast<const float4*>(a.S + (hD + j) * D)[w];
      M[4 * w] = t.x, M[4 * w + 1] = t.y, M[4 * w + 2] = t.z, M[4 * w + 3] = t.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < D; ++i) M[i] = 0.f;
  }

  // Inputs of token tt + 1 are loaded while token tt computes: the per-lane v
  // and gate values into registers, the uniform beta into a scalar register,
  // and one touch per line of its k and q rows, which warms the cache for that
  // token's scalar loads.
  const int n_tok = a.n_tokens;
  auto th_of = [&](int tt) { return size_t(tt) * a.n_heads + bh; };  // [token][head]
  const int pfi = min(2 * lane, D - 2);  // element of a k / q row this lane touches
  const int jc = min(j, D - 1);          // in-bounds column for the idle lanes' loads
  const int gc = min(lane, D - 1);       // this lane's first gate channel
  // loads without branches (clamped indices), so that no join forces an early wait
  auto load_tok = [&](int tt, float& beta, float& vj, float& e0, float& e1) {
    const size_t th = th_of(tt), row = th * D;
    beta = as_const<float>(a.beta)[th];
    vj = act_lane<BF16>(a.v, row + jc);
    e0 = a.g[row + gc];
    e1 = D > 64 ? a.g[row + 64 + lane] : 0.f;
  };
  float beta_c = 0.f, vj_c = 0.f, e0_c = 0.f, e1_c = 0.f;
  if (n_tok > 0) load_tok(0, beta_c, vj_c, e0_c, e1_c);
  for (int tt = 0; tt < n_tok; ++tt) {
    const size_t th = th_of(tt);
    const size_t row = th * D;
    const int tn = min(tt + 1, n_tok - 1);  // the last token reloads itself
    float beta_n = 0.f, vj_n = 0.f, e0_n = 0.f, e1_n = 0.f;
    load_tok(tn, beta_n, vj_n, e0_n, e1_n);
    const size_t rown = th_of(tn) * D;
    const float touch = act_lane<BF16>(a.k, rown + pfi) + act_lane<BF16>(a.q, rown + pfi);
    __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the token's arithmetic
    // pass 1: decay, and u_j = beta (v_j - sum_i S'[i][j] k_i); alpha_i =
    // exp(g_i), lane l holding channels l and l + 64
    float s[4] = {0.f, 0.f, 0.f, 0.f};
    const float a0 = expf(e0_c), a1 = expf(e1_c);
#pragma unroll
    for (int i = 0; i < D; ++i) {
      const float al = as_f(__builtin_amdgcn_readlane(as_u(i < 64 ? a0 : a1), i & 63));
      M[i] *= al;
      s[i & 3] = fmaf(M[i], act_at<BF16>(a.k, row, i), s[i & 3]);
    }
    const float u = col ? beta_c * (vj_c - ((s[0] + s[1]) + (s[2] + s[3]))) : 0.f;
    // pass 2: S = S' + k u^T, and o_j = sum_i S[i][j] q_i
    float p[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < D; ++i) {
      M[i] = fmaf(act_at<BF16>(a.k, row, i), u, M[i]);
      p[i & 3] = fmaf(M[i], act_at<BF16>(a.q, row, i), p[i & 3]);
    }
    // the next token's loads are complete here, before the output store: a
    // wait at the loop's end then never covers the store
    asm volatile("" ::"v"(touch), "v"(vj_n), "v"(e0_n), "v"(e1_n));
    if (col) a.o[row + j] = (p[0] + p[1]) + (p[2] + p[3]);
    beta_c = beta_n, vj_c = vj_n, e0_c = e0_n, e1_c = e1_n;
  }

  if (col) {
#pragma unroll
    for (int w = 0; w < D / 4; ++w)
      reinterpret_cast<float4*>(a.S + (hD + j) * D)[w] = make_float4(M[4 * w], M[4 * w + 1], M[4 * w + 2], M[4 * w + 3]);
  }
}

template <int D, bool KDA, bool BF16>
hipError_t launch(const lq_dims& d, const PrefillArgs& a, hipStream_t stream) {
  if constexpr (BF16 || !KDA) {
    hipLaunchKernelGGL((prefill_blocks_kernel<D, KDA, BF16>), dim3(d.batch * d.heads), dim3(128), 0, stream, a);
  } else {
    constexpr int WPH = D > 64 ? D / 64 : 1;
    hipLaunchKernelGGL((prefill_columns_kernel<D, KDA, BF16>), dim3(d.batch * d.heads * WPH), dim3(64), 0,
                       stream, a);
  }
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
