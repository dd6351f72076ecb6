// LeapQuant decode step for GDN / KDA recurrent states on gfx950.
//
// Per-window quantization (LeapQuant abstract; wink.run article, first
// technique): the quantized state stays frozen for a window, each token's
// update joins an fp32 buffer, and a token's output combines the frozen state
// with that buffer. Compensators are rank-one terms shaped like token updates,
// parked at window position 0 (abstract; article, second technique). The gated delta rule itself follows Gated DeltaNet (Yang et al.)
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
// byte's high half is the int8 16*code. When the caller gives the window
// position, loads are issued in the order they are consumed (per-channel
// inputs, each lane group's entry rows straight into registers, then the
// codes); otherwise every entry address waits for the head's buffer length,
// and half of the codes are issued while it is in flight. Either way the
// key-side dots run while the last codes arrive. The output and the appended
// entry are written with streaming stores.
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

// Cache policies of the state loads: the codes (the bulk of the state, read
// once per step) stream with the non-temporal hint; the entry rows keep the
// default policy (the non-temporal hint measured slower for them).
constexpr int CODES_POLICY = 2;
constexpr int ENTRY_POLICY = 0;

// N consecutive fp32 values (N in 2, 4, 8) at byte offset off of a buffer.
template <int N>
__device__ __forceinline__ void buf_loadN(__amdgpu_buffer_rsrc_t r, uint32_t off, float (&x)[N]) {
  if constexpr (N == 2) {
    const v2u t = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, ENTRY_POLICY);
    x[0] = __uint_as_float(t[0]), x[1] = __uint_as_float(t[1]);
  } else {
#pragma unroll
    for (int w = 0; w < N / 4; ++w) {
      const v4u t = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16 * w, 0, ENTRY_POLICY);
#pragma unroll
      for (int c = 0; c < 4; ++c) x[4 * w + c] = __uint_as_float(t[c]);
    }
  }
}

__device__ __forceinline__ float4 buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const v4u t = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, ENTRY_POLICY);
  return make_float4(__uint_as_float(t[0]), __uint_as_float(t[1]), __uint_as_float(t[2]), __uint_as_float(t[3]));
}

// Key rows. A compensator's key (entry e < r) is fp32; with bf16 activations
// a buffered token's key is its bf16 input, held as d_k bf16 values in the
// first half of its row (exact, and half the bytes). key_load fetches N
// channels at channel i0 of row e as loaded words (a bf16 row fills the first
// N/2); key_widen turns them into fp32 where they are used.
template <bool BF16, int D, int N>
__device__ __forceinline__ void key_load(__amdgpu_buffer_rsrc_t rk, int e, int r, int i0, float (&x)[N]) {
  if (BF16 && e >= r) {
    const uint32_t off = uint32_t(e * D * 4 + i0 * 2);
    if constexpr (N == 8) {
      const v4u t = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, ENTRY_POLICY);
#pragma unroll
      for (int c = 0; c < 4; ++c) x[c] = __uint_as_float(t[c]);
    } else if constexpr (N == 4) {
      const v2u t = __builtin_amdgcn_raw_buffer_load_b64(rk, off, 0, ENTRY_POLICY);
      x[0] = __uint_as_float(t[0]), x[1] = __uint_as_float(t[1]);
    } else {
      static_assert(N == 2, "key channels per lane");
      x[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rk, off, 0, ENTRY_POLICY));
    }
#pragma unroll
    for (int c = N / 2; c < N; ++c) x[c] = 0.f;
  } else {
    buf_loadN(rk, uint32_t(e * D + i0) * 4, x);
  }
}
template <bool BF16, int N>
__device__ __forceinline__ void key_widen(int e, int r, const float (&w)[N], float (&x)[N]) {
  if (BF16 && e >= r) {
#pragma unroll
    for (int c = 0; c < N; ++c) {
      const uint32_t b = __float_as_uint(w[c / 2]);
      x[c] = __uint_as_float((c & 1) ? (b & 0xFFFF0000u) : (b << 16));
    }
  } else {
#pragma unroll
    for (int c = 0; c < N; ++c) x[c] = w[c];
  }
}

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

// Code bytes one lane feeds to the matrix cores: 16 key channels of one
// value column. load() fetches them from the column's bytes at key channel
// i; mfma() accumulates sum_i code_i * z_i * SCALE^-1 for the 16 channels
// against the z-limb operand, whose channel order matches chan_pos<BITS>.
template <int BITS>
struct CodeLoad;
template <>
struct CodeLoad<8> {
  using T = uint4;
  static constexpr float INV_SCALE = 1.f;
  __device__ static T load(__amdgpu_buffer_rsrc_t r, uint32_t col, int i, int) {
    const v4u w = __builtin_amdgcn_raw_buffer_load_b128(r, col + i, 0, CODES_POLICY);
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
  __device__ static v4i mfma(v4i z, const T& w, v4i acc) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(z, v4i{int(w.x), int(w.y), int(w.z), int(w.w)}, acc, 0, 0, 0);
  }
};
// Nibble n (two's complement) masked into a byte's high half is the int8
// 16*n, exactly. Even channels (low nibbles) go first, then odd ones.
__device__ __forceinline__ v4i nibbles_x16(uint2 w) {
  return v4i{int((w.x << 4) & 0xF0F0F0F0u), int((w.y << 4) & 0xF0F0F0F0u), int(w.x & 0xF0F0F0F0u),
             int(w.y & 0xF0F0F0F0u)};
}
template <>
struct CodeLoad<4> {
  using T = uint2;
  static constexpr float INV_SCALE = 0.0625f;  // bytes hold 16 * code
  __device__ static T load(__amdgpu_buffer_rsrc_t r, uint32_t col, int i, int) {
    const v2u w = __builtin_amdgcn_raw_buffer_load_b64(r, col + i / 2, 0, CODES_POLICY);
    return make_uint2(w[0], w[1]);
  }
  __device__ static v4i mfma(v4i z, const T& w, v4i acc) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(z, nibbles_x16(w), acc, 0, 0, 0);
  }
};
// 6-bit codes (code = 4 hi + lo): hi in the head's first plane as 4-bit
// nibbles, laid out and loaded like 4-bit codes; lo as 2-bit fields in the
// second plane (loaded separately, see HeadStep::load_lo), placed so that
// field m of byte k (bits 8k + 2m) is operand position 4m + k. The byte 16*hi
// (high nibble) and 4*lo (bits 2-3) do not overlap, so their bitwise or is
// the int8 4*code: one product per block.
template <>
struct CodeLoad<6> {
  using T = uint2;
  static constexpr float INV_SCALE = 0.25f;  // bytes hold 4 * code
  __device__ static T load(__amdgpu_buffer_rsrc_t r, uint32_t col, int i, int d) {
    return CodeLoad<4>::load(r, col, i, d);
  }
  __device__ static v4i mfma(v4i z, const T& w, uint32_t l, v4i acc) {
    const v4i lo4 = v4i{int((l << 2) & 0x0C0C0C0Cu), int(l & 0x0C0C0C0Cu), int((l >> 2) & 0x0C0C0C0Cu),
                        int((l >> 4) & 0x0C0C0C0Cu)};
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(z, nibbles_x16(w) | lo4, acc, 0, 0, 0);
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

// One head's decode step, split into the loads (all issued first, into
// registers) and the arithmetic that consumes them.
template <int D, int BITS, bool KDA, bool BF16>
struct HeadStep {
  using SS = StepShape<D, KDA>;
  static constexpr int NT = SS::NT, NW = SS::NW, RBW = SS::RBW, KB = SS::KB, CPL = SS::CPL, NG = SS::NG;
  static constexpr int KPF = SS::KPF, NQ = SS::NQ, EP = SS::EP, PFE = SS::PFE;
  static constexpr int CB = D * (BITS == 6 ? 4 : BITS) / 8;  // bytes per value column (6 bits: hi plane)
  static constexpr int HEAD_CODE_BYTES = D * D * BITS / 8;
  static constexpr float L2E = 1.4426950408889634f;
  using CL = CodeLoad<BITS>;
  using CT = typename CL::T;

  struct Smem {
    __align__(16) float x[2][D];         // x for x = k, q
    __align__(16) float G[KDA ? D : 4];  // KDA: G_t per key channel
    __align__(16) int8_t B[KB][16][64];  // z limbs (MFMA A operand)
    __align__(16) float c[D];            // value-column scales
    __align__(16) float y[2][D];         // code readout
    __align__(16) float vs[EP][2][D];    // value-side partial sums per entry phase
    float kap[2][MAX_ROWS];              // kappa^k, kappa^q per entry
    float red[3][NW];                    // per-wave k.q and max |z^x| (bits)
  };

  // Inputs of one head in registers.
  struct In {
    CT cw[RBW][KB];  // residual codes, MFMA operand order
    uint32_t lo6[BITS == 6 ? KB : 1][BITS == 6 ? RBW : 1];  // 6 bits: lo fields of the same blocks
    uint32_t kx_raw, qx_raw;  // q_t, k_t as loaded (bf16 or fp32 bits); converted when used
    uint32_t vj_raw;          // v_t of this thread's value column as loaded (bf16 or fp32 bits)
    float si, cc, gi, beta, gs, Gp;
    float kr[KPF][CPL], gr[KDA ? KPF : 1][CPL], Gm[KPF];  // kr: key rows as loaded (key_load)
    float4 uv[PFE];
  };

  struct Ptr {  // this head's rows (per-lane offsets stay 32-bit)
    size_t hD;
    float *ek, *eu, *eg;
  };

  // KDA: the G rows are read only for the n buffered entries. Compensators sit
  // at window position 0 (G_e = 0), so the G buffer starts at entry r and a
  // compensator row's offset lies past its end: it reads as zeros and moves
  // no data.
  __device__ static __forceinline__ __amdgpu_buffer_rsrc_t g_rsrc(const StepArgs& a, const Ptr& P, int n) {
    if constexpr (KDA) return buf_rsrc(P.eg + a.r * D, uint32_t(n) * D * 4);
    else return buf_rsrc(P.eg, uint32_t(a.r + n) * 4);
  }
  __device__ static __forceinline__ uint32_t g_off(const StepArgs& a, int e, int i0) {
    if constexpr (KDA) return e >= a.r ? uint32_t((e - a.r) * D + i0) * 4 : 0x80000000u;
    else return uint32_t(e) * 4;
  }

  __device__ static __forceinline__ Ptr ptr(const StepArgs& a, int bh) {
    const int NE = a.r + a.w_max;
    return Ptr{size_t(bh) * D, a.ek + size_t(bh) * NE * D, a.eu + size_t(bh) * NE * D,
               a.eg + size_t(bh) * NE * (KDA ? D : 1)};
  }

  // Loads that do not depend on the buffer length, issued while it is in
  // flight: the first half of the codes, then the per-channel inputs.
  __device__ static __forceinline__ void load_early(const StepArgs& a, int bh, In& h) {
    const Ptr P = ptr(a, bh);
    load_codes(a, P, h, 0, RBW / 2);
    if constexpr (BITS == 6) load_lo(a, P, h);
    __builtin_amdgcn_sched_barrier(0);  // keep these codes first in the issue order
    load_inputs(a, bh, h);
  }

  // The per-channel inputs: activations, scales, decay, beta.
  __device__ static __forceinline__ void load_inputs(const StepArgs& a, int bh, In& h) {
    const int t = threadIdx.x;
    const bool chan = NT == D || t < D;
    const int tc = chan ? t : 0;
    const Ptr P = ptr(a, bh);
    if constexpr (BF16) {
      h.kx_raw = static_cast<const uint16_t*>(a.k)[P.hD + tc];
      h.qx_raw = static_cast<const uint16_t*>(a.q)[P.hD + tc];
      h.vj_raw = static_cast<const uint16_t*>(a.v)[P.hD + tc];
    } else {
      h.kx_raw = static_cast<const uint32_t*>(a.k)[P.hD + tc];
      h.qx_raw = static_cast<const uint32_t*>(a.q)[P.hD + tc];
      h.vj_raw = static_cast<const uint32_t*>(a.v)[P.hD + tc];
    }
    h.si = a.s[P.hD + tc];
    h.cc = a.c[P.hD + tc];
    h.gi = KDA ? a.g[P.hD + tc] : 0.f;
    h.gs = KDA ? 0.f : a.g[bh];
    h.beta = a.beta[bh];
    // the buffer length is checked after these loads are issued
    __builtin_amdgcn_sched_barrier(0);
  }

  // The loads that need the buffer length n (0 <= n < w_max): the entries,
  // then the second half of the codes.
  __device__ static __forceinline__ void load(const StepArgs& a, int bh, int n, In& h) {
    load_entries(a, bh, n, h);
    // The second half of the codes is issued last: loads complete in issue
    // order, so the entry arithmetic can start while those codes stream in.
    load_codes(a, ptr(a, bh), h, RBW / 2, RBW);
  }

  // Every load of a head whose buffer length n is known at launch, in the
  // order the arithmetic uses them: the per-channel inputs, the entry rows,
  // then all the codes.
  __device__ static __forceinline__ void load_known(const StepArgs& a, int bh, int n, In& h) {
    load_inputs(a, bh, h);
    load_entries(a, bh, n, h);
    __builtin_amdgcn_sched_barrier(0);
    const Ptr P = ptr(a, bh);
    load_codes(a, P, h, 0, RBW);
    if constexpr (BITS == 6) load_lo(a, P, h);
  }

  // The entry rows (prefetched part) and G of the last entry.
  __device__ static __forceinline__ void load_entries(const StepArgs& a, int bh, int n, In& h) {
    const int t = threadIdx.x;
    const int grp = t / 16, li = t % 16, i0 = li * CPL;
    const int q4 = t % NQ, ph = t / NQ;
    const bool chan = NT == D || t < D;
    const int tc = chan ? t : 0;
    const Ptr P = ptr(a, bh);
    // entries e = 0..E-1: r compensators (window position 0, G = 0), then the
    // n buffered tokens. The entry buffers end at entry E, so rows past the
    // last entry read as zeros and cost no memory traffic.
    const int E = a.r + n;
    const auto rk = buf_rsrc(P.ek, uint32_t(E) * D * 4), ru = buf_rsrc(P.eu, uint32_t(E) * D * 4);
    const auto rg = g_rsrc(a, P, n);
#pragma unroll
    for (int k = 0; k < KPF; ++k) {
      const int e = grp + NG * k;
      key_load<BF16, D>(rk, e, a.r, i0, h.kr[k]);
      if constexpr (KDA) buf_loadN(rg, g_off(a, e, i0), h.gr[k]);  // zero rows for compensators
      else h.Gm[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rg, g_off(a, e, 0), 0, ENTRY_POLICY));
    }
#pragma unroll
    for (int k = 0; k < PFE; ++k) h.uv[k] = buf_load4(ru, uint32_t((ph + EP * k) * D + 4 * q4) * 4);
    // G_{t-1}: G of the last entry; 0 with no buffered token (compensators carry 0)
    if constexpr (KDA) h.Gp = n > 0 ? P.eg[(E - 1) * D + tc] : 0.f;
    else h.Gp = E > 0 ? P.eg[E - 1] : 0.f;
  }

  // Codes of row blocks [lo, hi) in MFMA operand order: lane -> value column
  // 16*rb + lane%16, key channels 64*kb + 16*(lane/16) .. +16.
  __device__ static __forceinline__ void load_codes(const StepArgs& a, const Ptr& P, In& h, int lo, int hi) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int jl = lane & 15, il = 16 * (lane >> 4);
    const auto rc = buf_rsrc(static_cast<const uint8_t*>(a.codes) + size_t(HEAD_CODE_BYTES) * (P.hD / D),
                             HEAD_CODE_BYTES);
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
      if (rb < lo || rb >= hi) continue;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int j = 16 * (wave * RBW + rb) + jl, i = 64 * kb + il;
        if (D >= 64 || i < D) h.cw[rb][kb] = CL::load(rc, uint32_t(j * CB), i, D);
        else h.cw[rb][kb] = CT{};
      }
    }
  }

  // 6 bits: the lo fields of every block of this lane. The second plane holds
  // 32-bit words W[j % 16][i / 16][j / 16] (j value column, i key channel),
  // so a lane's words for its row blocks (consecutive j / 16) are adjacent.
  __device__ static __forceinline__ void load_lo(const StepArgs& a, const Ptr& P, In& h) {
    if constexpr (BITS == 6) {
      const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
      const auto rc = buf_rsrc(static_cast<const uint8_t*>(a.codes) + size_t(HEAD_CODE_BYTES) * (P.hD / D),
                               HEAD_CODE_BYTES);
      constexpr int NJ = D / 16;  // column groups j / 16, and channel groups i / 16
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int g = 4 * kb + (lane >> 4);
        const uint32_t off = uint32_t(D * D / 2) + 4u * uint32_t(((lane & 15) * NJ + g) * NJ + wave * RBW);
        if (D >= 64 || 16 * g < D) {
          if constexpr (RBW == 4) {
            const v4u w = __builtin_amdgcn_raw_buffer_load_b128(rc, off, 0, CODES_POLICY);
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) h.lo6[kb][rb] = w[rb];
          } else {
            static_assert(RBW == 2, "row blocks per wave");
            const v2u w = __builtin_amdgcn_raw_buffer_load_b64(rc, off, 0, CODES_POLICY);
            h.lo6[kb][0] = w[0], h.lo6[kb][1] = w[1];
          }
        } else {
#pragma unroll
          for (int rb = 0; rb < RBW; ++rb) h.lo6[kb][rb] = 0u;
        }
      }
    }
  }

  // The step of head bh from its loaded inputs; writes o, appends entry E.
  __device__ static __forceinline__ void compute(const StepArgs& a, int bh, int n, const In& h, Smem& sm) {
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int grp = t / 16, li = t % 16, i0 = li * CPL;
    const int q4 = t % NQ, ph = t / NQ;
    const bool chan = NT == D || t < D;
    const Ptr P = ptr(a, bh);
    const int E = a.r + n;
    const float G = KDA ? 0.f : h.Gp + h.gs;  // GDN: G_t
    const float kx = !chan ? 0.f : BF16 ? as_f(h.kx_raw << 16) : as_f(h.kx_raw);
    const float qx = !chan ? 0.f : BF16 ? as_f(h.qx_raw << 16) : as_f(h.qx_raw);

    // (1) per key channel: z^x = s (.) exp(G_t) (.) x, block max |z^x|, k_t . q_t
    const float Gi = KDA ? h.Gp + h.gi : G;
    const float eG = exp_fast(Gi);
    const float zk = h.si * (eG * kx), zq = h.si * (eG * qx);
    if (chan) {
      sm.x[0][t] = kx;
      sm.x[1][t] = qx;
      if constexpr (KDA) sm.G[t] = Gi;
      sm.c[t] = h.cc;
    }
    {
      const float kq = rows_sum(group_sum<16>(kx * qx));
      const uint32_t mk = rows_umax(group_umax<16>(as_u(fabsf(zk))));
      const uint32_t mq = rows_umax(group_umax<16>(as_u(fabsf(zq))));
      if (lane == 0) {
        sm.red[0][wave] = kq;
        sm.red[1][wave] = as_f(mk);
        sm.red[2][wave] = as_f(mq);
      }
    }
    __syncthreads();

    // (2) z^x as a 30-bit fixed-point integer with a power-of-two block scale,
    // split into four signed 8-bit limbs (rows 4x+l of the MFMA A operand)
    float zscale[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      uint32_t mb = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) mb = max(mb, as_u(sm.red[1 + x][w]));
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
        sm.B[kb][4 * x + 0][pos] = int8_t(l0);
        sm.B[kb][4 * x + 1][pos] = int8_t(l1);
        sm.B[kb][4 * x + 2][pos] = int8_t(l2);
        sm.B[kb][4 * x + 3][pos] = int8_t(l3);
      }
    }
    // (D = 32: the code operand is zero past channel D, so the limb operand's
    // unwritten padding bytes never contribute)

    // (3) key-side dots: kappa^x_e = sum_i k_e,i exp(G_t,i - G_e,i) x_i
    // (GDN: the decay ratio is one scalar exp(G_t - G_e) applied after the sum)
    {
      float xk[CPL], xq[CPL], Gt[CPL];
      loadN(&sm.x[0][i0], xk);
      loadN(&sm.x[1][i0], xq);
      if constexpr (KDA) {
        loadN(&sm.G[i0], Gt);
#pragma unroll
        for (int x = 0; x < CPL; ++x) Gt[x] *= L2E;
      }
      const auto rk = buf_rsrc(P.ek, uint32_t(E) * D * 4);
      const auto rg = g_rsrc(a, P, n);
      int e0 = 0;
      do {  // at least one pass, so that kappa of the prefetched rows is always written
#pragma unroll
        for (int k = 0; k < KPF; ++k) {
          const int e = e0 + grp + NG * k;
          // a 16-lane row group shares e: skipped groups leave whole rows idle
          if (e >= E && e0 + NG * k > 0) {
            if (li == 0) sm.kap[0][e] = sm.kap[1][e] = 0.f;
            continue;
          }
          float row[CPL], gm[CPL], gsc = h.Gm[k];
          if (e0 == 0) {
            key_widen<BF16>(e, a.r, h.kr[k], row);
            if constexpr (KDA) {
#pragma unroll
              for (int x = 0; x < CPL; ++x) gm[x] = h.gr[k][x];
            }
          } else {  // entries beyond the prefetched ones (long windows)
            float w[CPL];
            key_load<BF16, D>(rk, e, a.r, i0, w);
            key_widen<BF16>(e, a.r, w, row);
            if constexpr (KDA) buf_loadN(rg, g_off(a, e, i0), gm);
            else gsc = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rg, g_off(a, e, 0), 0, ENTRY_POLICY));
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
          // rows past the last entry read as zeros: kappa = 0 there
          if (li == 0) {
            sm.kap[0][e] = dk;
            sm.kap[1][e] = dq;
          }
        }
        e0 += NG * KPF;
      } while (e0 < E);
    }
    __syncthreads();

    // (5a) the first half of the residual readout (see (5)): its codes were
    // loaded first, so the matrix cores take it while (4) runs on the VALU
    v4i aop[KB], acc[RBW];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      aop[kb] = *reinterpret_cast<const v4i*>(&sm.B[kb][lane & 15][16 * (lane >> 4)]);
#pragma unroll
    for (int rb = 0; rb < RBW / 2; ++rb) {
      acc[rb] = v4i{0, 0, 0, 0};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        if constexpr (BITS == 6) acc[rb] = CL::mfma(aop[kb], h.cw[rb][kb], h.lo6[kb][rb], acc[rb]);
        else acc[rb] = CL::mfma(aop[kb], h.cw[rb][kb], acc[rb]);
    }

    // (4) value-side sums: sum_e u_e[j] kappa^x_e for this thread's four value
    // columns over the entries of its phase (e = ph, ph + EP, ...)
    {
      float4 pk = make_float4(0.f, 0.f, 0.f, 0.f), pq = pk;
#pragma unroll
      for (int k = 0; k < PFE; ++k) {
        const int e = ph + EP * k;
        if (e >= E && k > 0) continue;  // (past the last entry u = 0 and kappa = 0)
        const float ak = sm.kap[0][e], aq = sm.kap[1][e];
        pk.x = fmaf(h.uv[k].x, ak, pk.x), pk.y = fmaf(h.uv[k].y, ak, pk.y);
        pk.z = fmaf(h.uv[k].z, ak, pk.z), pk.w = fmaf(h.uv[k].w, ak, pk.w);
        pq.x = fmaf(h.uv[k].x, aq, pq.x), pq.y = fmaf(h.uv[k].y, aq, pq.y);
        pq.z = fmaf(h.uv[k].z, aq, pq.z), pq.w = fmaf(h.uv[k].w, aq, pq.w);
      }
      const auto ru = buf_rsrc(P.eu, uint32_t(E) * D * 4);
      for (int e = ph + EP * PFE; e < E; e += EP) {
        const float4 u = buf_load4(ru, uint32_t(e * D + 4 * q4) * 4);
        const float ak = sm.kap[0][e], aq = sm.kap[1][e];
        pk.x = fmaf(u.x, ak, pk.x), pk.y = fmaf(u.y, ak, pk.y), pk.z = fmaf(u.z, ak, pk.z), pk.w = fmaf(u.w, ak, pk.w);
        pq.x = fmaf(u.x, aq, pq.x), pq.y = fmaf(u.y, aq, pq.y), pq.z = fmaf(u.z, aq, pq.z), pq.w = fmaf(u.w, aq, pq.w);
      }
      *reinterpret_cast<float4*>(&sm.vs[ph][0][4 * q4]) = pk;
      *reinterpret_cast<float4*>(&sm.vs[ph][1][4 * q4]) = pq;
    }
    // (5) residual readout on the matrix cores: for every value column j and
    // x in {k, q}, sum_i Z^x_i C_ij exactly in int32, limb by limb (A = limbs,
    // rows 4x+l; B = codes, columns j). Lane l of row block rb then holds the
    // four limb sums of x = l/16 for column j = 16 rb + l%16 and combines them:
    // y^x_j / c_j = zscale_x * sum_l 256^l D[4x+l][j].
    {
#pragma unroll
      for (int rb = RBW / 2; rb < RBW; ++rb) {
        acc[rb] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          if constexpr (BITS == 6) acc[rb] = CL::mfma(aop[kb], h.cw[rb][kb], h.lo6[kb][rb], acc[rb]);
          else acc[rb] = CL::mfma(aop[kb], h.cw[rb][kb], acc[rb]);
      }
      const int xs = lane >> 4;
      const float zs = (xs == 0 ? zscale[0] : zscale[1]) * CL::INV_SCALE;
      if (xs < 2) {
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) {
          float f = fmaf(float(acc[rb][3]), 16777216.f, float(acc[rb][2]) * 65536.f);
          f = fmaf(float(acc[rb][1]), 256.f, f) + float(acc[rb][0]);
          sm.y[xs][16 * (wave * RBW + rb) + (lane & 15)] = f * zs;
        }
      }
    }

    __syncthreads();

    // (6) delta, output, append (k_t, u_t, G_t) as entry E: one thread per
    // value column (a short chain per thread: this is the step's tail)
    if (chan) {
      const int j = t;
      float kqs = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) kqs += sm.red[0][w];
      const float cj = sm.c[j];
      float yk = sm.y[0][j] * cj, yq = sm.y[1][j] * cj;
#pragma unroll
      for (int p = 0; p < EP; ++p) yk += sm.vs[p][0][j], yq += sm.vs[p][1][j];
      const float vj = BF16 ? as_f(h.vj_raw << 16) : as_f(h.vj_raw);
      const float u = h.beta * (vj - yk);
      // The output and the appended entry go out with the streaming (nt)
      // policy: the entry is read again one step later, after the rest of the
      // step's state has streamed through, and o by the next consumer (the
      // policy measured faster than write-back stores for both).
      constexpr int STORE_POLICY = 2;
      __builtin_amdgcn_raw_buffer_store_b32(as_u(fmaf(kqs, u, yq)), buf_rsrc(a.o + P.hD, D * 4), j * 4, 0,
                                            STORE_POLICY);
      __builtin_amdgcn_raw_buffer_store_b32(as_u(u), buf_rsrc(P.eu + E * D, D * 4), j * 4, 0, STORE_POLICY);
      if constexpr (BF16)  // a token's key row holds its bf16 input (key_load)
        __builtin_amdgcn_raw_buffer_store_b16(uint16_t(h.kx_raw), buf_rsrc(P.ek + E * D, D * 2), j * 2, 0, STORE_POLICY);
      else
        __builtin_amdgcn_raw_buffer_store_b32(as_u(kx), buf_rsrc(P.ek + E * D, D * 4), j * 4, 0, STORE_POLICY);
      if constexpr (KDA)
        __builtin_amdgcn_raw_buffer_store_b32(as_u(Gi), buf_rsrc(P.eg + E * D, D * 4), j * 4, 0, STORE_POLICY);
      if (t == 0) {
        if constexpr (!KDA) P.eg[E] = G;
        a.blen[bh] = n + 1;
      }
    }
  }
};

// One workgroup per head: a batch of a few thousand heads is resident on the
// chip at once, every head's loads are in flight from the start, and no
// workgroup waits for another. (Several heads per workgroup with the next
// head's loads overlapping the current head's arithmetic measured slower.)
template <int D, int BITS, bool KDA, bool BF16, bool AT>
__global__ void __launch_bounds__((StepShape<D, KDA>::NT)) __attribute__((amdgpu_waves_per_eu(KDA ? 3 : 4)))
decode_step_kernel(StepArgs a) {
  using HS = HeadStep<D, BITS, KDA, BF16>;
  __shared__ typename HS::Smem sm;
  const int bh = blockIdx.x;
  if constexpr (AT) {
    // Every head's buffer holds a.n_at tokens (the caller's schedule says so):
    // no load waits for the length, so the loads go out in the order the
    // arithmetic uses them. The stored length is loaded first and must agree,
    // before anything is written.
    const uint32_t n_raw = __builtin_amdgcn_raw_buffer_load_b32(buf_rsrc(a.blen + bh, 4), 0, 0, 0);
    const int n = a.n_at;
    typename HS::In in;
    HS::load_known(a, bh, n, in);
    if (int(__builtin_amdgcn_readfirstlane(int(n_raw))) != n) {
      if (threadIdx.x == 0 && a.err) atomicOr(a.err, LQ_DEVERR_BAD_LEN);
      return;
    }
    HS::compute(a, bh, n, in, sm);
    return;
  }
  // The buffer length comes first (every entry address depends on it) and
  // through the vector memory path, whose loads complete in issue order: the
  // wait for it then lets the loads issued after it stay in flight.
  const uint32_t n_raw = __builtin_amdgcn_raw_buffer_load_b32(buf_rsrc(a.blen + bh, 4), 0, 0, 0);
  __builtin_amdgcn_sched_barrier(0);
  typename HS::In in;
  HS::load_early(a, bh, in);
  const int n = __builtin_amdgcn_readfirstlane(int(n_raw));
  if (n < 0 || n >= a.w_max) {  // precondition violated: the head is left untouched
    if (threadIdx.x == 0 && a.err) atomicOr(a.err, n < 0 ? LQ_DEVERR_BAD_LEN : LQ_DEVERR_BUFFER_FULL);
    return;
  }
  HS::load(a, bh, n, in);
  HS::compute(a, bh, n, in, sm);
}

template <int D, int BITS, bool KDA, bool BF16>
hipError_t launch(const lq_dims& d, const StepArgs& a, hipStream_t stream) {
  if (a.n_at >= 0)
    hipLaunchKernelGGL((decode_step_kernel<D, BITS, KDA, BF16, true>), dim3(d.batch * d.heads),
                       dim3((StepShape<D, KDA>::NT)), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_step_kernel<D, BITS, KDA, BF16, false>), dim3(d.batch * d.heads),
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
  switch (d.bits) {
    case 8: return launch_db<D, 8>(d, a, s);
    case 6: return launch_db<D, 6>(d, a, s);
    default: return launch_db<D, 4>(d, a, s);
  }
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
