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
// (o = S'^T q + (k . q) u). Three kernels, all keeping the state on chip for
// the whole prompt (read and written once):
//
// - prefill_chunk_kernel (d = 128, GDN and KDA): chunks of 16 tokens, whose
//   products and state update run on the matrix cores (described at the
//   kernel).
// - prefill_blocks_kernel (d < 128: GDN, and KDA with bf16 activations): 128
//   threads per head on an 8 x 16 grid, each with a block of D/8 key rows by
//   D/16 value columns; the column partials of S'^T k and S'^T q and the
//   partial k . q are summed over the wave's rows with the row-swap
//   instructions (the work split across the rows) and over the two waves
//   through LDS, one barrier per token, double-buffered; the next token's
//   inputs load while the current one computes. GDN keeps the scalar decay as
//   one scale per head.
// - prefill_columns_kernel (d < 128, KDA with fp32 activations): every value
//   column j evolves on its own (u_j needs column j of S' and k; o_j column j
//   of S and q), so one thread owns one column, all d_k key rows, and a token
//   costs it two passes over its column with no exchange between threads. k,
//   q and beta are the same for every thread of a head and arrive through
//   scalar loads as instruction operands; the per-channel gates are
//   exponentiated two channels per lane and broadcast with readlane.
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

// ---- GDN at d = 128: chunks of 16 tokens on the matrix cores
//
// Within a chunk of C tokens with start state S0 and cumulative log-decay
// G_t (through token t, inclusive), the recurrence unrolls to
//   (alpha_t S_{t-1})^T k_t = e^{G_t} S0^T k_t + sum_{s<t} e^{G_t-G_s} (k_s.k_t) u_s
//   o_t = e^{G_t} S0^T q_t + sum_{s<=t} e^{G_t-G_s} (k_s.q_t) u_s
//   S_C = e^{G_C} S0 + sum_s e^{G_C-G_s} k_s u_s^T
// so the u_t solve a unit lower-triangular C x C system per value column,
//   u_t + beta_t sum_{s<t} A_ts u_s = beta_t (v_t - e^{G_t} S0^T k_t),
// A_ts = e^{G_t-G_s} k_t.k_s. The products K S0, Q S0, K K^T, Q K^T and the
// rank-C state update are fp32 MFMA contractions (v_mfma_f32_16x16x4f32); the
// triangular solves and the outputs run on the vector ALU, one thread per
// value column. It is the same recurrence, reassociated: results agree with
// the token-by-token form to fp32 rounding.
//
// 128 threads, two waves; wave w holds value columns [64w, 64w + 64) of all
// 128 key rows, in the MFMA accumulator layout: lane (g = lane / 16,
// c = lane % 16) holds S[16 TR + 4 g + r][64 w + 16 TC + c] in M[TR][TC][r].
// As the B operand of K S0 those registers need no movement: MFMA (TR, r)
// contracts over key rows 16 TR + 4 g + r (g = the lane group), and its A
// operand reads K at the same rows.

// x of the lane N below inside the 16-lane row, 0 for the row's first N lanes
template <int N>
__device__ __forceinline__ float dpp_shr(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x110 + N, 0xF, 0xF, true));
}

template <bool BF16, bool KDA>
__global__ void __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2))) prefill_chunk_kernel(PrefillArgs a) {
  constexpr int D = 128, C = 16, KS = D + 4;  // KS: padded LDS row (bank spread)
  typedef float v4f __attribute__((ext_vector_type(4)));
  __shared__ __align__(16) float sh_k[C][KS];
  __shared__ __align__(16) float sh_qu[C][KS];  // q of the chunk, then its u
  __shared__ __align__(16) float sh_r[2][C][64];  // per wave: v, then beta (v - e^G S0^T k), token-major
  __shared__ float sh_a[C][C];                   // beta_t A_ts, s < t
  __shared__ float sh_b[C][C];                   // e^{G_t-G_s} k_s.q_t, s <= t
  __shared__ float sh_G[C], sh_beta[C];          // GDN: G_t; beta_t
  __shared__ int sh_fast[2];                     // KDA: per-wave vote on the chunk's decay range
  // KDA: g, then G_t per key channel in base-2 units (G_t log2 e), so that
  // every decay factor e^{G_t - G_s} is a single exp2 of a difference
  __shared__ __align__(16) float sh_g[KDA ? C : 1][KS];
  __shared__ __align__(16) float sh_eC[KDA ? D : 1];  // KDA: e^{G_C} per key channel
  __shared__ __align__(16) float sh_GC[KDA ? D : 1];  // KDA: G_C per key channel
  // per wave: e^G S0^T q. KDA keeps it over sh_g, whose last use is the K S0
  // pass (that keeps the workgroup's LDS within four workgroups per CU)
  __shared__ __align__(16) float sh_pg[KDA ? 1 : 2 * C * 64];
  float(*sh_p)[C][64] = reinterpret_cast<float(*)[C][64]>(KDA ? &sh_g[0][0] : sh_pg);
  static_assert(!KDA || C * KS >= 2 * C * 64, "e^G S0^T q fits over sh_g");

  // Lane-derived indices are re-derived in every phase from an opaque copy of
  // the thread index, so that the compiler forms each phase's addresses there
  // instead of keeping dozens of them live across the chunk loop.
  const int w = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
  auto lane_id = [] {
    int x = int(threadIdx.x) & 63;
    asm volatile("" : "+v"(x));
    return x;
  };
  int lane = lane_id(), g = lane >> 4, c = lane & 15;
  const int bh = blockIdx.x;
  const size_t hD = size_t(bh) * D;
  const int NH = a.n_heads, n_tok = a.n_tokens;

  v4f M[8][4];
#pragma unroll
  for (int TC = 0; TC < 4; ++TC) {
    const float* col = a.S + (hD + 64 * w + 16 * TC + c) * D + 4 * g;  // + 16 TR: immediate offsets
#pragma unroll
    for (int TR = 0; TR < 8; ++TR) {
      const float4 x = *reinterpret_cast<const float4*>(col + 16 * TR);
      M[TR][TC] = v4f{x.x, x.y, x.z, x.w};
    }
  }

  // A chunk's inputs as loaded (thread t: token row t / 8 of the chunk, 16
  // channels from (t % 8) * 16, of k, q and v; wave 0 lane l < 16: token l's
  // g and beta). The next chunk's loads are issued once the current one is
  // staged, so they are in flight during its arithmetic.
  constexpr int NWD = BF16 ? 8 : 16;  // 32-bit words per 16 values
  struct Raw {
    uint32_t k[NWD], q[NWD], v[NWD];
    float g, beta;
    float gv[KDA ? 16 : 1];  // KDA: the gates of the same 16 channels
  };
  auto fetch = [&](int cc, Raw& x) {
    const int l = lane_id(), tt = 64 * w + l;
    const int tok = min(cc + (tt >> 3), n_tok - 1);  // clamped: rows past the prompt are zeroed when staged
    const size_t off = ((size_t(tok) * NH + bh) * D + (tt & 7) * 16) * (BF16 ? 2 : 4);
    if constexpr (BF16) {  // 8-byte pieces: the alignment the C ABI requires of bf16 activations
#pragma unroll
      for (int h = 0; h < NWD / 2; ++h) {
        const uint2 xk = *reinterpret_cast<const uint2*>(static_cast<const char*>(a.k) + off + 8 * h);
        const uint2 xq = *reinterpret_cast<const uint2*>(static_cast<const char*>(a.q) + off + 8 * h);
        const uint2 xv = *reinterpret_cast<const uint2*>(static_cast<const char*>(a.v) + off + 8 * h);
        x.k[2 * h] = xk.x, x.k[2 * h + 1] = xk.y;
        x.q[2 * h] = xq.x, x.q[2 * h + 1] = xq.y;
        x.v[2 * h] = xv.x, x.v[2 * h + 1] = xv.y;
      }
    } else {
#pragma unroll
      for (int h = 0; h < NWD / 4; ++h) {
        const uint4 xk = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.k) + off + 16 * h);
        const uint4 xq = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.q) + off + 16 * h);
        const uint4 xv = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.v) + off + 16 * h);
        x.k[4 * h] = xk.x, x.k[4 * h + 1] = xk.y, x.k[4 * h + 2] = xk.z, x.k[4 * h + 3] = xk.w;
        x.q[4 * h] = xq.x, x.q[4 * h + 1] = xq.y, x.q[4 * h + 2] = xq.z, x.q[4 * h + 3] = xq.w;
        x.v[4 * h] = xv.x, x.v[4 * h + 1] = xv.y, x.v[4 * h + 2] = xv.z, x.v[4 * h + 3] = xv.w;
      }
    }
    if constexpr (KDA) {
      const float4* pg = reinterpret_cast<const float4*>(a.g + (size_t(tok) * NH + bh) * D + (tt & 7) * 16);
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const float4 xg = pg[h];
        x.gv[4 * h] = xg.x, x.gv[4 * h + 1] = xg.y, x.gv[4 * h + 2] = xg.z, x.gv[4 * h + 3] = xg.w;
      }
    }
    if (w == 0) {
      const size_t th = size_t(min(cc + (l & 15), n_tok - 1)) * NH + bh;
      if constexpr (!KDA) x.g = a.g[th];
      x.beta = a.beta[th];
    }
  };
  auto val = [](const uint32_t(&wd)[NWD], int i) {  // element i of 16
    if constexpr (BF16) return (i & 1) ? bf16_hi(wd[i >> 1]) : bf16_lo(wd[i >> 1]);
    else return as_f(wd[i]);
  };
  Raw cur;
  if (n_tok > 0) fetch(0, cur);

  for (int c0 = 0; c0 < n_tok; c0 += C) {
    const int nc = min(C, n_tok - c0);
    __syncthreads();  // the previous chunk's reads of sh_k, sh_qu and sh_r are done
    // ---- stage k, q and v (fp32; rows past the prompt zero), G and beta
    {
      lane = lane_id();
      const int tt = 64 * w + lane, tr = tt >> 3, ch = (tt & 7) * 16;
      const bool in = tr < nc;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        float4 xk = make_float4(0.f, 0.f, 0.f, 0.f), xq = xk, xv = xk;
        if (in) {
          xk = make_float4(val(cur.k, 4 * h), val(cur.k, 4 * h + 1), val(cur.k, 4 * h + 2), val(cur.k, 4 * h + 3));
          xq = make_float4(val(cur.q, 4 * h), val(cur.q, 4 * h + 1), val(cur.q, 4 * h + 2), val(cur.q, 4 * h + 3));
          xv = make_float4(val(cur.v, 4 * h), val(cur.v, 4 * h + 1), val(cur.v, 4 * h + 2), val(cur.v, 4 * h + 3));
        }
        *reinterpret_cast<float4*>(&sh_k[tr][ch + 4 * h]) = xk;
        *reinterpret_cast<float4*>(&sh_qu[tr][ch + 4 * h]) = xq;
        // v goes where the right-hand side will be built: sh_r[wave of the column]
        *reinterpret_cast<float4*>(&sh_r[ch >> 6][tr][(ch & 63) + 4 * h]) = xv;
        if constexpr (KDA)
          *reinterpret_cast<float4*>(&sh_g[tr][ch + 4 * h]) =
              in ? make_float4(cur.gv[4 * h], cur.gv[4 * h + 1], cur.gv[4 * h + 2], cur.gv[4 * h + 3])
                 : make_float4(0.f, 0.f, 0.f, 0.f);
      }
      if (w == 0) {  // G_t = sum of g_s over s <= t: an inclusive scan over lanes 0-15
        const bool tin = lane < nc;  // (nc <= 16)
        float G = (tin && !KDA) ? cur.g : 0.f;
        const float bt = tin ? cur.beta : 0.f;
        G += dpp_shr<1>(G);
        G += dpp_shr<2>(G);
        G += dpp_shr<4>(G);
        G += dpp_shr<8>(G);
        if (lane < C) sh_G[lane] = G, sh_beta[lane] = bt;
      }
    }
    if (c0 + C < n_tok) fetch(c0 + C, cur);
    __syncthreads();
    // KDA: whether every channel's decay over the chunk stays within 2^-64,
    // so that e^{G_t} and e^{-G_s} are both safe in fp32 (uniform per chunk)
    bool fast = false;
    if constexpr (KDA) {  // G_t per key channel: thread i sums its channel over the chunk in place
      const int i = 64 * w + lane_id();
      float G = 0.f;
#pragma unroll
      for (int tk = 0; tk < C; ++tk) {
        G = fmaf(sh_g[tk][i], kLog2e, G);
        sh_g[tk][i] = G;
      }
      sh_GC[i] = G;
      const int all_ok = __all(G >= -64.f);  // G is G_C here (false for NaN)
      if (lane_id() == 0) sh_fast[w] = all_ok;
      __syncthreads();
      fast = sh_fast[0] != 0 && sh_fast[1] != 0;
      // ---- KDA with a wider decay range: for the 120 pairs s < t,
      // beta_t sum_i k_t,i k_s,i e^{G_t,i - G_s,i} and
      // sum_i q_t,i k_s,i e^{G_t,i - G_s,i} (one decay factor serves both),
      // each summed over the channels by one thread with every factor a
      // single exp2 of a difference (at most 1); then the 16 pairs s = t,
      // q_t . k_t, by all threads: eight lanes per token, 16 channels each
      if (!fast) {
        const int t0 = 64 * w + lane_id();
        if (t0 < 120) {
          int tk = 1, base = 0;  // t0 = t (t - 1) / 2 + s
          for (int t2 = 2; t2 < C; ++t2)
            if (t2 * (t2 - 1) / 2 <= t0) tk = t2, base = t2 * (t2 - 1) / 2;
          const int s2 = t0 - base;
          float ak = 0.f, aq = 0.f;
#pragma unroll 4
          for (int i = 0; i < D; i += 4) {
            const float4 k4 = *reinterpret_cast<const float4*>(&sh_k[tk][i]);
            const float4 q4 = *reinterpret_cast<const float4*>(&sh_qu[tk][i]);
            const float4 ks = *reinterpret_cast<const float4*>(&sh_k[s2][i]);
            const float4 gt = *reinterpret_cast<const float4*>(&sh_g[tk][i]);
            const float4 gs = *reinterpret_cast<const float4*>(&sh_g[s2][i]);
            const float e0 = ks.x * __builtin_amdgcn_exp2f(gt.x - gs.x), e1 = ks.y * __builtin_amdgcn_exp2f(gt.y - gs.y);
            const float e2 = ks.z * __builtin_amdgcn_exp2f(gt.z - gs.z), e3 = ks.w * __builtin_amdgcn_exp2f(gt.w - gs.w);
            ak = fmaf(k4.x, e0, ak), aq = fmaf(q4.x, e0, aq);
            ak = fmaf(k4.y, e1, ak), aq = fmaf(q4.y, e1, aq);
            ak = fmaf(k4.z, e2, ak), aq = fmaf(q4.z, e2, aq);
            ak = fmaf(k4.w, e3, ak), aq = fmaf(q4.w, e3, aq);
            asm volatile("" ::: "memory");  // one step's LDS reads at a time (register pressure)
          }
          sh_a[tk][s2] = sh_beta[tk] * ak;
          sh_b[tk][s2] = aq;
        }
        {
          const int tk = t0 >> 3, i0 = 16 * (t0 & 7);  // lanes 8m..8m+7 of a wave share a token
          float aq = 0.f;
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            const float4 k4 = *reinterpret_cast<const float4*>(&sh_k[tk][i0 + 4 * h]);
            const float4 q4 = *reinterpret_cast<const float4*>(&sh_qu[tk][i0 + 4 * h]);
            aq = fmaf(q4.x, k4.x, aq), aq = fmaf(q4.y, k4.y, aq);
            aq = fmaf(q4.z, k4.z, aq), aq = fmaf(q4.w, k4.w, aq);
          }
          aq = group_sum<8>(aq);
          if ((t0 & 7) == 0) sh_b[tk][tk] = aq;
        }
      }
      if (!fast) __syncthreads();  // the pair sums' reads of k, q and G are done
      // Each thread turns 16 channels of one token into the operands the
      // matrix-core phases use, in place: k_t e^{G_t} (for K S0) over G,
      // q_t e^{G_t} (Q S0) over q, and over k either k_t e^{-G_t} (fast: the
      // pair products' right operand, turned into the state update's by the
      // solve phase) or k_t e^{G_C - G_t} (the state update's); the threads
      // of token 0 put e^{G_C} in sh_eC. Each factor is computed once per
      // element instead of once per operand slot of every wave.
      {
        lane = lane_id();
        const int tt = 64 * w + lane, tr = tt >> 3, ch = (tt & 7) * 16;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const int c4 = ch + 4 * h;
          const float4 G4 = *reinterpret_cast<const float4*>(&sh_g[tr][c4]);
          const float4 C4 = *reinterpret_cast<const float4*>(&sh_GC[c4]);
          const float4 k4 = *reinterpret_cast<const float4*>(&sh_k[tr][c4]);
          const float4 q4 = *reinterpret_cast<const float4*>(&sh_qu[tr][c4]);
          const float4 e = make_float4(__builtin_amdgcn_exp2f(G4.x), __builtin_amdgcn_exp2f(G4.y),
                                       __builtin_amdgcn_exp2f(G4.z), __builtin_amdgcn_exp2f(G4.w));
          const float4 f = make_float4(__builtin_amdgcn_exp2f(fast ? -G4.x : C4.x - G4.x),
                                       __builtin_amdgcn_exp2f(fast ? -G4.y : C4.y - G4.y),
                                       __builtin_amdgcn_exp2f(fast ? -G4.z : C4.z - G4.z),
                                       __builtin_amdgcn_exp2f(fast ? -G4.w : C4.w - G4.w));
          *reinterpret_cast<float4*>(&sh_g[tr][c4]) = make_float4(k4.x * e.x, k4.y * e.y, k4.z * e.z, k4.w * e.w);
          *reinterpret_cast<float4*>(&sh_qu[tr][c4]) = make_float4(q4.x * e.x, q4.y * e.y, q4.z * e.z, q4.w * e.w);
          *reinterpret_cast<float4*>(&sh_k[tr][c4]) = make_float4(k4.x * f.x, k4.y * f.y, k4.z * f.z, k4.w * f.w);
          if (tr == 0)
            *reinterpret_cast<float4*>(&sh_eC[c4]) = make_float4(__builtin_amdgcn_exp2f(C4.x), __builtin_amdgcn_exp2f(C4.y),
                                                                 __builtin_amdgcn_exp2f(C4.z), __builtin_amdgcn_exp2f(C4.w));
        }
      }
      __syncthreads();
    }

    // ---- pair coefficients on the matrix cores: K K^T (wave 0) or Q K^T
    // (wave 1), entry (t = 4g + r, s = c). GDN: the plain rows, then the
    // scalar decay e^{G_t - G_s}. KDA in the fast case: x_t e^{G_t} against
    // k_s e^{-G_s}, so the per-channel decay is inside the contraction.
    if (!KDA || fast) {
      lane = lane_id(), g = lane >> 4, c = lane & 15;
      float(*ra)[KS] = w == 0 ? (KDA ? sh_g : sh_k) : sh_qu;
      v4f X = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
      for (int kb = 0; kb < D / 4; ++kb) {
        const float b = sh_k[c][4 * kb + g];
        const float av = ra[c][4 * kb + g];
        X = __builtin_amdgcn_mfma_f32_16x16x4f32(av, b, X, 0, 0, 0);
      }
      const float Gs = KDA ? 0.f : sh_G[c];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tk = 4 * g + r;
        const float f = KDA ? 1.f : exp_fast(sh_G[tk] - Gs);
        if (w == 0) sh_a[tk][c] = c < tk ? sh_beta[tk] * f * X[r] : 0.f;
        else sh_b[tk][c] = c <= tk ? f * X[r] : 0.f;
      }
    }

    // ---- K S0, then Q S0, for this wave's columns (token 4g + r, column
    // 64w + 16TC + c), each turned into its LDS form before the next
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      if (KDA && pass == 1) __syncthreads();  // K S0's reads of sh_g are done before sh_p overwrites it
      lane = lane_id(), g = lane >> 4, c = lane & 15;
      float(*src)[KS] = pass == 0 ? (KDA ? sh_g : sh_k) : sh_qu;  // (KDA: decayed operands)
      v4f P[4];
#pragma unroll
      for (int TC = 0; TC < 4; ++TC) P[TC] = v4f{0.f, 0.f, 0.f, 0.f};
      // operands one row block ahead of the products that use them (a fence
      // per block keeps the loads from piling up further ahead)
      // (KDA: the operand row is x_t (.) e^{G_t}, the decay through token t)
      auto opnd = [&](int row) { return src[c][row]; };
      float ak[4], an[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ak[r] = opnd(4 * g + r);
#pragma unroll
      for (int TR = 0; TR < 8; ++TR) {
        if (TR < 7) {
#pragma unroll
          for (int r = 0; r < 4; ++r) an[r] = opnd(16 * (TR + 1) + 4 * g + r);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int TC = 0; TC < 4; ++TC) P[TC] = __builtin_amdgcn_mfma_f32_16x16x4f32(ak[r], M[TR][TC][r], P[TC], 0, 0, 0);
        asm volatile("" ::: "memory");
#pragma unroll
        for (int r = 0; r < 4; ++r) ak[r] = an[r];
      }
      // right-hand sides beta (v - e^G S0^T k), or the e^G S0^T q terms
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tk = 4 * g + r;
        const float eG = KDA ? 1.f : exp_fast(sh_G[tk]), bt = sh_beta[tk];
#pragma unroll
        for (int TC = 0; TC < 4; ++TC) {
          if (pass == 0) sh_r[w][tk][16 * TC + c] = bt * (sh_r[w][tk][16 * TC + c] - eG * P[TC][r]);
          else sh_p[w][tk][16 * TC + c] = eG * P[TC][r];
        }
      }
    }
    __syncthreads();

    // ---- per value column (lane): forward substitution for u, then o
    {
      lane = lane_id();
      const int J = 64 * w + lane;
      float u[C];
      // token by token: u_t from the earlier u, then o_t (a fence per token
      // keeps the uniform coefficient loads from all being hoisted ahead)
#pragma unroll
      for (int tk = 0; tk < C; ++tk) {
        float x = sh_r[w][tk][lane];
#pragma unroll
        for (int s2 = 0; s2 < tk; ++s2) x = fmaf(-sh_a[tk][s2], u[s2], x);
        u[tk] = x;
        float o = sh_p[w][tk][lane];
#pragma unroll
        for (int s2 = 0; s2 <= tk; ++s2) o = fmaf(sh_b[tk][s2], u[s2], o);
        if (tk < nc) a.o[(size_t(c0 + tk) * NH + bh) * D + J] = o;
        asm volatile("" ::: "memory");
      }
      // (q in sh_qu was last read before the previous barrier)
#pragma unroll
      for (int tk = 0; tk < C; ++tk) sh_qu[tk][J] = u[tk];
      if (KDA && fast) {  // key channel J: k_t e^{-G_t} (the pair products' operand) to k_t e^{G_C - G_t}
        const float e = sh_eC[J];
#pragma unroll
        for (int tk = 0; tk < C; ++tk) sh_k[tk][J] *= e;
      }
    }
    __syncthreads();

    // ---- S = e^{G_C} S0 + sum_s e^{G_C - G_s} k_s u_s^T
    {
      lane = lane_id(), g = lane >> 4, c = lane & 15;
      const float GC = sh_G[C - 1], eC = exp_fast(GC);
#pragma unroll
      for (int TR = 0; TR < 8; ++TR) {
        if constexpr (KDA) {  // row 16 TR + 4 g + r decays by e^{G_C} of its key channel
          const float4 e4 = *reinterpret_cast<const float4*>(&sh_eC[16 * TR + 4 * g]);
          const v4f e = v4f{e4.x, e4.y, e4.z, e4.w};
#pragma unroll
          for (int TC = 0; TC < 4; ++TC) M[TR][TC] *= e;
        } else {
#pragma unroll
          for (int TC = 0; TC < 4; ++TC) M[TR][TC] *= eC;
        }
      }
#pragma unroll
      for (int kb = 0; kb < C / 4; ++kb) {
        const int s2 = 4 * kb + g;
        const float f = KDA ? 1.f : exp_fast(GC - sh_G[s2]);
        float ub[4];
#pragma unroll
        for (int TC = 0; TC < 4; ++TC) ub[TC] = sh_qu[s2][64 * w + 16 * TC + c];
#pragma unroll
        for (int TR = 0; TR < 8; ++TR) {
          // (KDA: k_s e^{G_C - G_s}, precomputed)
          const float ak = KDA ? sh_k[s2][16 * TR + c] : f * sh_k[s2][16 * TR + c];
#pragma unroll
          for (int TC = 0; TC < 4; ++TC) M[TR][TC] = __builtin_amdgcn_mfma_f32_16x16x4f32(ak, ub[TC], M[TR][TC], 0, 0, 0);
        }
      }
    }
  }

  const int lane_o = lane_id();
#pragma unroll
  for (int TC = 0; TC < 4; ++TC) {
    float* col = a.S + (hD + 64 * w + 16 * TC + (lane_o & 15)) * D + 4 * (lane_o >> 4);
#pragma unroll
    for (int TR = 0; TR < 8; ++TR)
      *reinterpret_cast<float4*>(col + 16 * TR) = make_float4(M[TR][TC][0], M[TR][TC][1], M[TR][TC][2], M[TR][TC][3]);
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
  if constexpr (D == 128) {
    hipLaunchKernelGGL((prefill_chunk_kernel<BF16, KDA>), dim3(d.batch * d.heads), dim3(128), 0, stream, a);
  } else if constexpr (BF16 || !KDA) {
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
