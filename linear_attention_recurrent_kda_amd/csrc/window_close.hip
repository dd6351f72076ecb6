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
// block row (all tj), so sums over value columns stay inside the row: DPP
// reductions, or at D = 128 a transpose through the wave's own LDS (each lane
// adds up one key row). Sums over key rows combine the four rows of a wave
// with the gfx950 row-swap instructions, the work split so that each row
// keeps a quarter of the columns, and the two waves through LDS. Tall blocks
// keep the reduction work per power iteration low, and at D = 128 a thread
// owns whole 16-channel code groups. The fold of the buffered
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

// The close's writes (codes, scales, compensator rows) use streaming stores:
// the kernel is bound by its arithmetic, and the next decode step then reads
// the new state without first evicting it from the caches (write-back stores
// measured 0.4-0.5 us slower on that first step, the close itself unchanged).
// The price is write requests: a code row is written half by each wave, and
// streamed halves often leave the L2 as separate requests (at 4 bits, 29%
// more bytes written than with write-back stores, within the close's time).
template <int B>
__device__ __forceinline__ void storeB(float* p, const float (&x)[B]) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  typedef float f2 __attribute__((ext_vector_type(2)));
  if constexpr (B % 4 == 0) {
#pragma unroll
    for (int w = 0; w < B / 4; ++w)
      __builtin_nontemporal_store(f4{x[4 * w], x[4 * w + 1], x[4 * w + 2], x[4 * w + 3]}, reinterpret_cast<f4*>(p) + w);
  } else {
    __builtin_nontemporal_store(f2{x[0], x[1]}, reinterpret_cast<f2*>(p));
  }
}

// x[B] held alike by the lanes of a group: lane q of the group (q < B / 4)
// stores float4 q of it, so one instruction writes the group's whole B-float
// segment and the wave's adjacent segments form whole lines. B = 2: lane 0
// stores both floats. The caller selects the lanes (q below the count).
// The elements pass through an empty asm before the lane's choice among them:
// a choice between elements still in memory would otherwise be folded into a
// load from a lane-dependent address, which keeps x in scratch memory.
template <int B>
__device__ __forceinline__ void storeSplit(float* p, const float (&x)[B], int q) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  if constexpr (B % 4 == 0) {
    float y[B];
#pragma unroll
    for (int e = 0; e < B; ++e) {
      y[e] = x[e];
      asm("" : "+v"(y[e]));
    }
    f4 v = f4{y[0], y[1], y[2], y[3]};
#pragma unroll
    for (int m = 1; m < B / 4; ++m) {
      const bool take = q == m;
      v.x = take ? y[4 * m] : v.x;
      v.y = take ? y[4 * m + 1] : v.y;
      v.z = take ? y[4 * m + 2] : v.z;
      v.w = take ? y[4 * m + 3] : v.w;
    }
    __builtin_nontemporal_store(v, reinterpret_cast<f4*>(p) + q);
  } else {
    storeB<B>(p, x);
  }
}
template <int B>
constexpr int split_lanes = B % 4 == 0 ? B / 4 : 1;

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
  if constexpr (NB == 16) __builtin_nontemporal_store(v4u{w[0], w[1], w[2], w[3]}, reinterpret_cast<v4u*>(p));
  else if constexpr (NB == 8) __builtin_nontemporal_store(v2u{w[0], w[1]}, reinterpret_cast<v2u*>(p));
  else if constexpr (NB == 4) __builtin_nontemporal_store(w[0], reinterpret_cast<uint32_t*>(p));
  else __builtin_nontemporal_store(uint16_t(w[0]), reinterpret_cast<uint16_t*>(p));
}

// N codes packed little-endian (4 bits: even channel in the low nibble). Only
// the low BITS bits of each c[a] are read, so bit patterns whose low bits are
// the two's-complement codes pack as they are: bytes (or nibble pairs) are
// gathered four at a time with byte permutes.
template <int N, int BITS>
__device__ __forceinline__ void store_codes(uint8_t* p, const uint32_t (&c)[N]) {
  static_assert(BITS == 8 || BITS == 4, "code width");
  constexpr int NB = N * BITS / 8;
  uint32_t b[NB];  // byte m of the packed codes in the low 8 bits (higher bits ignored)
#pragma unroll
  for (int m = 0; m < NB; ++m) b[m] = BITS == 8 ? c[m] : (c[2 * m] & 0xFu) | (c[2 * m + 1] << 4);
  uint32_t w[(NB + 3) / 4];
  if constexpr (NB >= 4) {
#pragma unroll
    for (int q = 0; q < NB / 4; ++q) {
      const uint32_t lo = __builtin_amdgcn_perm(b[4 * q + 1], b[4 * q], 0x0c0c0400u);  // bytes 0, 1
      const uint32_t hi = __builtin_amdgcn_perm(b[4 * q + 3], b[4 * q + 2], 0x0c0c0400u);
      w[q] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
    }
  } else {
    static_assert(NB == 2, "code bytes per block column");
    w[0] = __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u);
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

// The codes of N consecutive key channels i0.. of value column j (i0 % N == 0,
// N <= 16) as loaded words, unpacked to signed ints later: 8 bits one byte
// each; 4 bits two's-complement nibbles, even channel low; 6 bits the hi
// nibbles plus the 16-channel group's low-bit word.
template <int N, int BITS, int D>
struct CodeWords {
  static constexpr int NB = N * (BITS == 6 ? 4 : BITS) / 8;  // bytes of the (hi) plane
  uint32_t w[(NB + 3) / 4];
  uint32_t lo;

  __device__ __forceinline__ void load(const uint8_t* head, int j, int i0) {
    if constexpr (BITS == 6) {
      load_bytes<NB>(head + size_t(j) * (D / 2) + i0 / 2, w);
      lo = *reinterpret_cast<const uint32_t*>(head + lo_word<D>(j, i0 / 16));
    } else {
      load_bytes<NB>(head + size_t(j) * (D * BITS / 8) + i0 * BITS / 8, w);
      lo = 0u;
    }
  }

  __device__ __forceinline__ void unpack(int i0, int (&c)[N]) const {
#pragma unroll
    for (int a = 0; a < N; ++a) {
      if constexpr (BITS == 8) {
        c[a] = int(int8_t(uint8_t(w[a / 4] >> (8 * (a % 4)))));
      } else {
        const int hi = int(((w[a / 8] >> (4 * (a % 8))) & 0xFu) ^ 0x8u) - 8;
        if constexpr (BITS == 6) c[a] = 4 * hi + int((lo >> lo_bit((i0 + a) & 15)) & 3u);
        else c[a] = hi;
      }
    }
  }
};

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

// ACT: 0 for a plain close (or the dense encode); 1 or 2 when the close
// first takes one decode token on every head (fp32 or bf16 activations): the
// window's last token, folded in registers instead of appended.
template <bool BF16>
__device__ __forceinline__ uint32_t act_bits(const void* p, size_t i) {  // converted by act_f
  if constexpr (BF16) return static_cast<const uint16_t*>(p)[i];
  else return static_cast<const uint32_t*>(p)[i];
}
template <bool BF16>
__device__ __forceinline__ float act_f(uint32_t b) {
  return __uint_as_float(BF16 ? b << 16 : b);
}

template <int D, int BITS, bool KDA, bool DENSE, int ACT, bool KB>
__global__ void __launch_bounds__(NT) close_kernel(CloseArgs a) {
  static_assert(!(DENSE && ACT), "the dense encode takes no token");
  // KB: the buffered tokens' key rows hold bf16 keys (bf16 activations: a
  // token's key row is its bf16 input in the row's first half; compensator
  // rows stay fp32); a token of the same width as the buffer
  static_assert(!(KB && DENSE) && (ACT == 0 || KB == (ACT == 2)), "key row width");
  constexpr int RB = D / 8;   // key rows per thread
  constexpr int CB = D / 16;  // value columns per thread
  constexpr int Q = (1 << (BITS - 1)) - 1;  // 127, 31 or 7
  constexpr int HB = D * D * BITS / 8;      // code bytes per head
  constexpr int CH0 = D == 128 ? 20 : 32;   // entries staged in LDS by the first fold pass
  constexpr int CH1 = 16;                   // ... by each later pass (windows past CH0 entries)
  constexpr int V4 = D / 4;                 // float4 per entry row
  constexpr int PER0 = CH0 * V4 / NT;       // float4 per thread per staged array, first pass
  constexpr int PER1 = CH1 * V4 / NT;       // ... later passes
  static_assert(NT % V4 == 0 && PER1 >= 1 && PER1 * NT == CH1 * V4 && PER0 * NT == CH0 * V4, "staging shape");
  __shared__ float sh_n[2];                   // per-wave squared norms of the final kappa
  __shared__ __align__(16) float sh_c[2][2][D];  // per-wave column partials (double-buffered)
  __shared__ __align__(16) float sh_k[DENSE ? 1 : CH0][D];  // keys scaled by their decay to the window end
  __shared__ __align__(16) float sh_u[DENSE ? 1 : CH0][D];
  // D = 128: the row partials of kappa = M v, per 16-lane row [tj][x] (rows
  // of 20 floats, 16-byte aligned; 336 floats per lane row, so the four lane
  // rows of a wave start 16 banks apart), and the row totals [ti][x]
  constexpr int PX = 20, PR = 16 * PX + 16;
  __shared__ __align__(16) float sh_p[RB == 16 ? 8 * PR : 1];
  __shared__ __align__(16) float sh_t[RB == 16 ? 8 : 1][16];
  __shared__ __align__(16) float sh_tok[ACT ? 3 : 1][D];  // the token's k, q and v

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
  int n_stored = 0;  // the head's stored buffer length (close only)
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
    // The buffer length is read first; the code words and scales, which do
    // not depend on it, go out while it is in flight. Every load of the fold
    // is issued before the first of them is used, so that a head waits for
    // memory once: this thread's code words, its scales, G_n, and the first
    // CH0 entry rows (all of them when r + n <= CH0).
    n_stored = __builtin_amdgcn_readfirstlane(a.blen[bh]);
    const uint8_t* cb = static_cast<const uint8_t*>(a.codes) + size_t(bh) * HB;
    CodeWords<RB, BITS, D> cw[CB];
#pragma unroll
    for (int bb = 0; bb < CB; ++bb) cw[bb].load(cb, j0 + bb, i0);
    __builtin_amdgcn_sched_barrier(0);  // (keeps the length's first use after these loads)
    // The loads use the stored length clamped to [0, w_max] (with a token,
    // the caller's position); the stored length itself is checked after the
    // fold, before anything is written, and a corrupted one (or, with a
    // token, one that is not the caller's position) leaves the head
    // untouched. No branch stands between these loads and their use.
    const int n = ACT != 0 ? a.n_at : min(max(n_stored, 0), a.w_max);
    const int E = r + n;
    // the token's k, q and v at channel t: loaded now, put in LDS once the
    // first staged rows are (so that no wait for them holds back the fold's
    // loads), read after the fold, whose barriers order them
    // (as loaded bits, the index clamped rather than branched on, so that
    // nothing waits for them before the stores)
    uint32_t tkk = 0u, tkq = 0u, tkv = 0u;
    if constexpr (ACT != 0) {
      const size_t it = hD + (t < D ? t : 0);
      tkk = act_bits<ACT == 2>(a.k, it);
      tkq = act_bits<ACT == 2>(a.q, it);
      tkv = act_bits<ACT == 2>(a.v, it);
    }
    float si[RB], cj[CB], Gn[KDA ? RB : 1];
    loadB<RB>(a.s + hD + i0, si);
    loadB<CB>(a.c + hD + j0, cj);
    if constexpr (KDA) {  // (compensator G rows are 0 by definition and not read)
      if (n > 0) loadB<RB>(a.eg + (erow + E - 1) * D + i0, Gn);
      else
#pragma unroll
        for (int x = 0; x < RB; ++x) Gn[x] = 0.f;
    } else {
      Gn[0] = E > 0 ? a.eg[erow + E - 1] : 0.f;
    }
    // with a token, the window ends at its G_t = G_n + g_t: everything is
    // decayed to it (the decay the step applies before the delta)
    if constexpr (ACT != 0) {
      if constexpr (KDA) {
        float gt[RB];
        loadB<RB>(a.g + hD + i0, gt);
#pragma unroll
        for (int x = 0; x < RB; ++x) Gn[x] += gt[x];
      } else {
        Gn[0] += a.g[bh];
      }
    }
    // Entry rows go through LDS, each key multiplied by its decay to the
    // window end; every thread then applies them to its block. A thread
    // stages the same four key channels of every row it loads (NT is a
    // multiple of V4). The loads are range-checked buffer loads over this
    // head's E rows: rows at or past E read as zeros, and (KDA) a
    // compensator's G row is addressed past the end of the G range, which
    // starts at entry r.
    const int c4 = t % V4;
    float4 gq = make_float4(0.f, 0.f, 0.f, 0.f);  // KDA: G_n (or G_t) of the staged channels
    if constexpr (KDA) {
      if (n > 0) gq = *reinterpret_cast<const float4*>(a.eg + (erow + E - 1) * D + 4 * c4);
      if constexpr (ACT != 0) {
        const float4 g4 = *reinterpret_cast<const float4*>(a.g + hD + 4 * c4);
        gq.x += g4.x, gq.y += g4.y, gq.z += g4.z, gq.w += g4.w;
      }
    }
    const auto rk = buf_rsrc(a.ek + erow * D, uint32_t(E) * D * 4);
    const auto ru = buf_rsrc(a.eu + erow * D, uint32_t(E) * D * 4);
    const auto rg = KDA ? buf_rsrc(a.eg + (erow + r) * D, uint32_t(n) * D * 4) : buf_rsrc(a.eg + erow, uint32_t(E) * 4);
    auto ld4 = [](__amdgpu_buffer_rsrc_t rs, uint32_t off) {
      const v4u q = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
      return make_float4(as_f(q[0]), as_f(q[1]), as_f(q[2]), as_f(q[3]));
    };
    // rows m0 .. m0 + NP * NT / V4 - 1: loads, then (decay, LDS) once they are in
    float4 kq[PER0], uq[PER0], ge[KDA ? PER0 : 1];
    float gs[PER0];
    auto stage_load = [&](auto np, int m0) {
      constexpr int NP = decltype(np)::value;
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int e = m0 + (t + NT * p) / V4;
        const uint32_t off = uint32_t(e * D + 4 * c4) * 4;
        if (KB && e >= r) {  // a token's bf16 key: four channels in 8 bytes
          const v2u q2 = __builtin_amdgcn_raw_buffer_load_b64(rk, uint32_t(e * D * 4 + 8 * c4), 0, 0);
          kq[p] = make_float4(as_f(q2[0]), as_f(q2[1]), 0.f, 0.f);
        } else {
          kq[p] = ld4(rk, off);
        }
        uq[p] = ld4(ru, off);
        if constexpr (KDA) ge[p] = ld4(rg, e >= r ? uint32_t((e - r) * D + 4 * c4) * 4 : 0x80000000u);
        else gs[p] = as_f(__builtin_amdgcn_raw_buffer_load_b32(rg, uint32_t(e) * 4, 0, 0));
      }
    };
    auto stage_store = [&](auto np, int m0) {
      constexpr int NP = decltype(np)::value;
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int row = (t + NT * p) / V4;
        const bool in = m0 + row < E;  // rows past E: zeros (no decay factor, which could overflow)
        float4 k4 = kq[p];
        if (KB && m0 + row >= r) {
          const uint32_t lo = __float_as_uint(k4.x), hi = __float_as_uint(k4.y);
          k4 = make_float4(as_f(lo << 16), as_f(lo & 0xFFFF0000u), as_f(hi << 16), as_f(hi & 0xFFFF0000u));
        }
        if constexpr (KDA) {
          k4.x *= in ? expf(gq.x - ge[p].x) : 0.f;
          k4.y *= in ? expf(gq.y - ge[p].y) : 0.f;
          k4.z *= in ? expf(gq.z - ge[p].z) : 0.f;
          k4.w *= in ? expf(gq.w - ge[p].w) : 0.f;
        } else {
          const float f = in ? expf(Gn[0] - gs[p]) : 0.f;
          k4.x *= f, k4.y *= f, k4.z *= f, k4.w *= f;
        }
        reinterpret_cast<float4*>(&sh_k[row][0])[c4] = k4;
        reinterpret_cast<float4*>(&sh_u[row][0])[c4] = uq[p];
      }
    };
    stage_load(std::integral_constant<int, PER0>{}, 0);
    // the first pass's rows go to LDS before the residual is built, which
    // frees their registers for it
    stage_store(std::integral_constant<int, PER0>{}, 0);
    if constexpr (ACT != 0) {
      if (t < D) sh_tok[0][t] = act_f<ACT == 2>(tkk), sh_tok[1][t] = act_f<ACT == 2>(tkq), sh_tok[2][t] = act_f<ACT == 2>(tkv);
    }
    // the residual M = diag(s exp(G_n)) C diag(c), decayed to the window end
#pragma unroll
    for (int x = 0; x < RB; ++x) si[x] *= expf(KDA ? Gn[x] : Gn[0]);
#pragma unroll
    for (int bb = 0; bb < CB; ++bb) {
      int code[RB];
      cw[bb].unpack(i0, code);
#pragma unroll
      for (int x = 0; x < RB; ++x) M[x >> 2][bb][x & 3] = (si[x] * float(code[x])) * cj[bb];
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
    int m0 = 0;
    while (true) {
      const int cnt = min(m0 == 0 ? CH0 : CH1, E - m0);
      __syncthreads();  // the staged rows are in LDS
      const int nkb = (cnt + 3) >> 2;  // rows from cnt up to 4 nkb are zeros
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
      m0 += m0 == 0 ? CH0 : CH1;
      if (m0 >= E) break;
      __syncthreads();  // the pass has consumed the staged rows
      stage_load(std::integral_constant<int, PER1>{}, m0);
      stage_store(std::integral_constant<int, PER1>{}, m0);
    }
    // (uniform: every thread read the same word)
    if (ACT != 0 ? n_stored != a.n_at : (n_stored < 0 || n_stored > a.w_max)) {
      if (t == 0 && a.err) atomicOr(a.err, LQ_DEVERR_BAD_LEN);
      return;
    }
  }

  int par = 0;
  // w = M^T kap for this thread's value columns: the sum over key rows, first
  // the wave's four rows with the work split (each row swap pairs two
  // columns, one kept by each half of the lanes), then the two waves through
  // LDS, double-buffered so that consecutive sums need one barrier each
  auto colsum = [&](const float(&kap)[RB], float(&w)[CB]) {
    float cs[CB], tot[CB >= 4 ? CB / 4 : 1];
#pragma unroll
    for (int bb = 0; bb < CB; ++bb) {
      float s = 0.f;
#pragma unroll
      for (int x = 0; x < RB; ++x) s = fmaf(M[x >> 2][bb][x & 3], kap[x], s);
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
    __syncthreads();
#pragma unroll
    for (int bb = 0; bb < CB; ++bb) w[bb] = sh_c[par][0][j0 + bb] + sh_c[par][1][j0 + bb];
    par ^= 1;
  };

  // ---- the window's last token (a decode step on the folded state, the
  // gated delta rule): M is now the state decayed to the token, so
  // u = beta (v - M^T k), M += k u^T, o = M^T q. The token is not appended:
  // the close empties the buffer.
  if constexpr (ACT != 0) {
    float kr[RB], qr[RB], vv[CB], y[CB], u[CB];
    loadB<RB>(&sh_tok[0][i0], kr);
    loadB<RB>(&sh_tok[1][i0], qr);
    loadB<CB>(&sh_tok[2][j0], vv);
    const float beta = a.beta[bh];
    colsum(kr, y);
#pragma unroll
    for (int bb = 0; bb < CB; ++bb) u[bb] = beta * (vv[bb] - y[bb]);
#pragma unroll
    for (int x = 0; x < RB; ++x)
#pragma unroll
      for (int bb = 0; bb < CB; ++bb) M[x >> 2][bb][x & 3] = fmaf(kr[x], u[bb], M[x >> 2][bb][x & 3]);
    colsum(qr, y);
    if (ti < split_lanes<CB>) storeSplit<CB>(a.o + hD + j0, y, ti);
  }

  // ---- compensators: power method with deflation. One barrier per
  // iteration: kappa = M v is complete inside each 16-lane row, and the
  // column partials of M^T kappa go to LDS (double-buffered, so the next
  // iteration may write while this one is read). The iteration keeps kappa
  // and c = M^T kappa unnormalised: the next v is c, of unit direction
  // c / |c| = w / |w| with w = M^T (kappa / |kappa|), and |kappa| is only
  // needed once, after the last iteration, for the unit key k and its value
  // w = c / |kappa|. kappa = 0 exactly when c = 0 (|kappa|^2 = v . c), so
  // |c|^2 zero or not finite flags a degenerate head.
  bool live = true;
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
      // v stays unnormalised: the unit vector is v sv, and sv multiplies the
      // row totals of M v instead of every element of v
      float sv = __builtin_amdgcn_rsqf(p);
      for (int it = 0; it < a.T; ++it) {
        // kappa = (M v) sv: the sum over value columns runs across the 16 tj lanes
        if constexpr (RB == 16) {
          // one row per lane: every lane writes its 16 row partials, lane tj
          // adds up the 16 partials of row i0 + tj, and every lane reads the
          // 16 totals back. Only this wave's lanes take part, so the wave's
          // in-order LDS accesses order them (no workgroup barrier).
          float sx[RB];
#pragma unroll
          for (int x = 0; x < RB; ++x) {
            float s = 0.f;
#pragma unroll
            for (int bb = 0; bb < CB; ++bb) s = fmaf(M[x >> 2][bb][x & 3], v[bb], s);
            sx[x] = s;
          }
          float* P = &sh_p[ti * PR];
#pragma unroll
          for (int k = 0; k < 4; ++k)
            *reinterpret_cast<float4*>(&P[tj * PX + 4 * k]) = make_float4(sx[4 * k], sx[4 * k + 1], sx[4 * k + 2], sx[4 * k + 3]);
          __builtin_amdgcn_wave_barrier();
          float tot = 0.f;
#pragma unroll
          for (int q = 0; q < 16; ++q) tot += P[q * PX + tj];
          sh_t[ti][tj] = tot * sv;
          __builtin_amdgcn_wave_barrier();
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float4 t4 = *reinterpret_cast<const float4*>(&sh_t[ti][4 * k]);
            kk[4 * k] = t4.x, kk[4 * k + 1] = t4.y, kk[4 * k + 2] = t4.z, kk[4 * k + 3] = t4.w;
          }
          __builtin_amdgcn_wave_barrier();  // these reads precede the next iteration's writes
        } else {
#pragma unroll
          for (int x = 0; x < RB; ++x) {
            float s = 0.f;
#pragma unroll
            for (int bb = 0; bb < CB; ++bb) s = fmaf(M[x >> 2][bb][x & 3], v[bb], s);
            kk[x] = group_sum<16>(s) * sv;
          }
        }
        // c = M^T kappa, kept for the value
        colsum(kk, w);
        float pc = 0.f;
#pragma unroll
        for (int bb = 0; bb < CB; ++bb) pc = fmaf(w[bb], w[bb], pc);
        pc = group_sum<16>(pc);  // the same total in every row
        if (!(pc > 0.f) || !isfinite(pc)) {  // uniform: every thread read the same sums
          live = false;
          break;
        }
        sv = __builtin_amdgcn_rsqf(pc);
#pragma unroll
        for (int bb = 0; bb < CB; ++bb) v[bb] = w[bb];
      }
      if (live) {
        // |kappa|^2 of the last iteration: the thread's rows (equal across
        // the 16 tj lanes), the wave's four rows, then the two waves
        float pk = 0.f;
#pragma unroll
        for (int x = 0; x < RB; ++x) pk = fmaf(kk[x], kk[x], pk);
        pk = rows_sum(pk);
        if (lane == 0) sh_n[wave] = pk;
        __syncthreads();
        // (the next write of sh_n comes after at least one more iteration
        // barrier, which both waves reach only after this read)
        const float nk2 = sh_n[0] + sh_n[1];
        if (!(nk2 > 0.f) || !isfinite(nk2)) {
          live = false;
        } else {
          const float inv_rk = __builtin_amdgcn_rsqf(nk2);
#pragma unroll
          for (int x = 0; x < RB; ++x) kk[x] *= inv_rk;
#pragma unroll
          for (int bb = 0; bb < CB; ++bb) w[bb] *= inv_rk;
        }
      }
    }
    if (!live) {
#pragma unroll
      for (int x = 0; x < RB; ++x) kk[x] = 0.f;
#pragma unroll
      for (int bb = 0; bb < CB; ++bb) w[bb] = 0.f;
    }
    // compensator l is entry l: a unit key, its value, and G = 0 (window position 0)
    // (kk is alike across a row's 16 tj lanes, w across the 8 ti rows)
    if (tj < split_lanes<RB>) storeSplit<RB>(a.ek + (erow + l) * D + i0, kk, tj);
    if (ti < split_lanes<CB>) storeSplit<CB>(a.eu + (erow + l) * D + j0, w, ti);
    if constexpr (KDA) {
      typedef float f4 __attribute__((ext_vector_type(4)));
      static_assert(RB % 4 == 0, "key rows per thread");
      if (tj < RB / 4) __builtin_nontemporal_store(f4{0.f, 0.f, 0.f, 0.f}, reinterpret_cast<f4*>(a.eg + (erow + l) * D + i0) + tj);
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
    uint32_t pat[RB];
#pragma unroll
    for (int x = 0; x < RB; ++x) {
      // M inv + 1.5 2^23 rounds once to the nearest integer, ties to even,
      // and the low 22 bits of the sum's pattern are that integer in two's
      // complement (the pattern minus that of 1.5 2^23, whose low 22 bits are
      // zero). No clamp: |M| is at most its column's maximum, so
      // |M inv| <= Q (1 + 2^-24) < Q + 1/2.
      pat[x] = __float_as_uint(fmaf(M[x >> 2][bb][x & 3], inv[bb], 12582912.f));
    }
    if constexpr (BITS == 6) {
      uint32_t hi[RB];
      uint32_t lo = 0;
#pragma unroll
      for (int x = 0; x < RB; ++x) {
        hi[x] = pat[x] >> 2;  // bits 2-5 of the code: floor(code / 4) as a nibble
        lo |= (pat[x] & 3u) << lo_bit((i0 + x) & 15);
      }
      store_codes<RB, 4>(cb + size_t(j) * (D / 2) + i0 / 2, hi);
      // a 16-channel group's low bits are one word; below D = 128 the threads
      // of a group (ti, ti ^ 1 [, ti ^ 2]) sit at lanes l ^ 16 (and l ^ 32)
      if constexpr (RB <= 8) lo = or_swap16(lo);
      if constexpr (RB <= 4) lo = or_swap32(lo);
      if (ti % (16 / RB) == 0) __builtin_nontemporal_store(lo, reinterpret_cast<uint32_t*>(cb + lo_word<D>(j, i0 / 16)));
    } else {
      store_codes<RB, BITS>(cb + size_t(j) * (D * BITS / 8) + i0 * BITS / 8, pat);
    }
  }
  if constexpr (RB == 16) {
    a.s[hD + i0 + tj] = sa[0];
  } else {
    if (tj < split_lanes<RB>) storeSplit<RB>(a.s + hD + i0, sa, tj);
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

template <int D, int BITS, bool KDA, bool DENSE, int ACT, bool KB>
hipError_t launch(const CloseArgs& a, int n_blocks, hipStream_t stream) {
  hipLaunchKernelGGL((close_kernel<D, BITS, KDA, DENSE, ACT, KB>), dim3(n_blocks), dim3(NT), 0, stream, a);
  return hipGetLastError();
}

template <int D, int BITS, bool KDA>
hipError_t launch_k(const lq_dims& d, const CloseArgs& a, int nb, hipStream_t s) {
  if (a.S) return launch<D, BITS, KDA, true, 0, false>(a, nb, s);
  const bool kb = d.act_dtype == LQ_ACT_BF16;  // buffered keys (and the token) in bf16
  if (!a.q) return kb ? launch<D, BITS, KDA, false, 0, true>(a, nb, s) : launch<D, BITS, KDA, false, 0, false>(a, nb, s);
  return kb ? launch<D, BITS, KDA, false, 2, true>(a, nb, s) : launch<D, BITS, KDA, false, 1, false>(a, nb, s);
}

template <int D, int BITS>
hipError_t launch_b(const lq_dims& d, const CloseArgs& a, int nb, hipStream_t s) {
  return d.decay_per_channel ? launch_k<D, BITS, true>(d, a, nb, s) : launch_k<D, BITS, false>(d, a, nb, s);
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
