// Host model of the device addressing of the decode step, the window close
// (csrc/decode_step.hip, csrc/window_close.hip, with or without the window's
// last token taken inside the close) and the FP32-state baseline
// (csrc/fp32_baseline.hip): every global load and store,
// buffer-descriptor range and LDS index those kernels form, written out again
// on the host and checked, for every thread of the workgroup, against the
// sizes the C ABI documents (lq_state_sizes) and the kernels' LDS arrays.
//
// Checked for d in {32, 64, 128}, 8-, 6- and 4-bit codes, scalar and
// per-channel decay, fp32 and bf16 activations, r = 0..8 compensators, buffer
// capacities w_max from 1 to 64 and every buffer length a launch accepts:
//  - a buffer descriptor's range lies inside its allocation (the hardware
//    returns zeros past the descriptor, never past the allocation);
//  - every access that must return data lies inside its descriptor (reads
//    past a descriptor are allowed only where the kernel relies on the zeros);
//  - every plain pointer access and every LDS index lies inside its array.
// Exit status 0 and one summary line when every check holds; the first
// violation is printed with its configuration and exits with status 1.
#include <cstdint>
#include <cstdio>
#include <cstdlib>

// Planted-mistake switches for the model's own test (defaults are the real
// sizes): the kappa rows of the decode step's LDS, slack taken off the entry
// rows a state holds per head, and a shift of the FP32 baseline's pieces.
#ifndef MODEL_KAPPA_ROWS
#define MODEL_KAPPA_ROWS (8 + 64 + 1)
#endif
#ifndef MODEL_G_COMP_OFF  // the decode step's offset for a compensator's G row
#define MODEL_G_COMP_OFF 0x80000000LL
#endif
#ifndef MODEL_ENTRY_SLACK
#define MODEL_ENTRY_SLACK 0
#endif
#ifndef MODEL_BL_PIECE_OFF  // shift of the FP32 baseline's float4 pieces
#define MODEL_BL_PIECE_OFF 0
#endif

namespace {

long long checks = 0;

struct Cfg {
  int D, BITS, KDA, BF16, r, w_max, n, bh, BH;
};

void fail(const Cfg& c, const char* what, long long off, long long lo, long long hi, int t) {
  std::printf("VIOLATION %s: offset %lld not in [%lld, %lld) -- d=%d bits=%d kda=%d bf16=%d r=%d w_max=%d n=%d bh=%d/%d thread=%d\n",
              what, off, lo, hi, c.D, c.BITS, c.KDA, c.BF16, c.r, c.w_max, c.n, c.bh, c.BH, t);
  std::exit(1);
}

// [off, off + size) must lie inside [lo, hi)
void in(const Cfg& c, const char* what, long long off, long long size, long long lo, long long hi, int t) {
  ++checks;
  if (off < lo || off + size > hi) fail(c, what, off, lo, hi, t);
}

// A B-float segment at byte offset seg held alike by a lane group: lane q
// (q < B/4) stores float4 q; B = 2: lane 0 stores both floats.
void split_store(const Cfg& c, const char* what, long long seg, int B, int q, long long lo, long long hi, int t) {
  if (B % 4 == 0) {
    if (q < B / 4) in(c, what, seg + 16LL * q, 16, lo, hi, t);
  } else if (q == 0) {
    in(c, what, seg, 4LL * B, lo, hi, t);
  }
}

// ---- sizes, as lq_state_sizes (bytes)
struct Sizes {
  long long codes, s, c, ek, eu, eg, blen, act_qk, act_v, g, beta, o, head_codes;
  int NE;
};

Sizes sizes(const Cfg& c) {
  Sizes z{};
  const long long BH = c.BH, D = c.D;
  z.NE = c.r + c.w_max - MODEL_ENTRY_SLACK;
  z.head_codes = D * D * c.BITS / 8;
  z.codes = BH * z.head_codes;
  z.s = z.c = BH * D * 4;
  z.ek = z.eu = BH * z.NE * D * 4;
  z.eg = BH * z.NE * (c.KDA ? D : 1) * 4;
  z.blen = BH * 4;
  z.act_qk = z.act_v = BH * D * (c.BF16 ? 2 : 4);
  z.g = BH * (c.KDA ? D : 1) * 4;
  z.beta = BH * 4;
  z.o = BH * D * 4;
  return z;
}

// A range-checked buffer load of `size` bytes at byte offset off of a
// descriptor over `range` bytes: either wholly inside (it reads memory) or
// wholly at or past the end (it returns zeros and moves no data), and below
// 2^32 with the load's size.
void buffer_load(const Cfg& c, const char* what, long long off, long long size, long long range, int t) {
  ++checks;
  if (off + size > (1LL << 32)) fail(c, what, off, 0, 1LL << 32, t);
  if (off < range && off + size > range) fail(c, what, off, 0, range, t);
}

// A key-row load of entry e < E at channel i0, n channels: fp32 (compensators,
// or every row with fp32 activations) or, with bf16 activations, a buffered
// token's bf16 key in the first half of its row; inside the row and the
// key descriptor either way.
void key_row(const Cfg& c, const char* what, int e, int i0, int n, long long rk_size, int t) {
  const int D = c.D;
  const bool b16 = c.BF16 && e >= c.r;
  const long long off = b16 ? (long long)e * D * 4 + i0 * 2 : (long long)(e * D + i0) * 4;
  const long long size = b16 ? n * 2 : n * 4;
  const long long row_end = (long long)e * D * 4 + (b16 ? D * 2 : D * 4);
  in(c, what, off, size, (long long)e * D * 4, row_end, t);
  in(c, what, off, size, 0, rk_size, t);
}

// ---------------------------------------------------------------- decode step
// A G load of entry e < E (the decode step's g_off): GDN one float at 4e;
// KDA the channels i0.. of row e - r, or, for a compensator row (e < r), an
// offset past the descriptor's end that stays below 2^32 with the load's
// 16-byte steps, so the load returns zeros and moves no data.
void g_row(const Cfg& c, const char* what, int e, int i0, int cpl, long long rg_size, int t) {
  if (!c.KDA) {
    in(c, what, (long long)e * 4, 4, 0, rg_size, t);
    return;
  }
  if (e >= c.r) {
    in(c, what, (long long)((e - c.r) * c.D + i0) * 4, cpl * 4, 0, rg_size, t);
    return;
  }
  const long long off = MODEL_G_COMP_OFF;
  ++checks;
  if (off < rg_size || off + cpl * 4 > (1LL << 32)) fail(c, "compensator G offset", off, rg_size, 1LL << 32, t);
}

// (leapquant_decode_step_at takes n from its caller, 0 <= n < w_max checked on
// the host, and addresses every buffer exactly as below for that n.)
void decode_step(const Cfg& c) {
  const Sizes z = sizes(c);
  const int D = c.D, BITS = c.BITS, KDA = c.KDA;
  // StepShape
  const int NT = D >= 128 ? 128 : 64, NW = NT / 64, RB = D / 16, RBW = RB / NW, KB = (D + 63) / 64;
  const int CPL = D / 16, NG = NT / 16, NQ = D / 4, EP = NT / NQ, PRE = 24, KPF = PRE / NG, PFE = PRE / EP;
  const int CB = D * (BITS == 6 ? 4 : BITS) / 8;
  const int MAX_ROWS = MODEL_KAPPA_ROWS;
  const long long act = c.BF16 ? 2 : 4;
  const long long bh = c.bh, hD = bh * D;
  const int NE = c.r + c.w_max, E = c.r + c.n;  // the kernel's own row count
  // descriptors: base offset inside the allocation and size
  const long long ek0 = bh * NE * D * 4, eu0 = ek0, eg0 = bh * NE * (KDA ? D : 1) * 4;
  const long long rk_size = (long long)E * D * 4;
  // the G descriptor: KDA starts at entry r and covers the n buffered rows
  // (compensator rows are addressed past its end and read as zeros)
  const long long rg0 = KDA ? eg0 + (long long)c.r * D * 4 : eg0;
  const long long rg_size = KDA ? (long long)c.n * D * 4 : (long long)E * 4;
  const long long rc0 = bh * z.head_codes, rc_size = z.head_codes;
  in(c, "codes descriptor", rc0, rc_size, 0, z.codes, -1);
  in(c, "entry-key descriptor", ek0, rk_size, 0, z.ek, -1);
  in(c, "entry-value descriptor", eu0, rk_size, 0, z.eu, -1);
  in(c, "entry-G descriptor", rg0, rg_size, eg0, eg0 + (long long)NE * (KDA ? D : 1) * 4, -1);
  in(c, "length load", bh * 4, 4, 0, z.blen, -1);
  for (int t = 0; t < NT; ++t) {
    const int lane = t & 63, wave = t >> 6;
    const bool chan = NT == D || t < D;
    const int tc = chan ? t : 0;
    // load_early / load: codes in MFMA operand order
    for (int rb = 0; rb < RBW; ++rb)
      for (int kb = 0; kb < KB; ++kb) {
        const int jl = lane & 15, il = 16 * (lane >> 4);
        const int j = 16 * (wave * RBW + rb) + jl, i = 64 * kb + il;
        if (D >= 64 || i < D) {
          const long long off = (long long)j * CB + (BITS == 8 ? i : i / 2);
          const long long bytes = BITS == 8 ? 16 : 8;
          // every code load returns data: inside the head's (hi-plane) bytes
          in(c, "code load", off, bytes, 0, BITS == 6 ? (long long)D * D / 2 : rc_size, t);
        }
      }
    if (BITS == 6) {
      const int NJ = D / 16;
      for (int kb = 0; kb < KB; ++kb) {
        const int g = 4 * kb + (lane >> 4);
        if (D >= 64 || 16 * g < D) {
          const long long off = (long long)D * D / 2 + 4LL * (((lane & 15) * NJ + g) * NJ + wave * RBW);
          in(c, "6-bit low plane load", off, RBW == 4 ? 16 : 8, (long long)D * D / 2, rc_size, t);
        }
      }
    }
    in(c, "k/q load", (hD + tc) * act, act, 0, z.act_qk, t);
    in(c, "v load", (hD + tc) * act, act, 0, z.act_v, t);
    in(c, "s load", (hD + tc) * 4, 4, 0, z.s, t);
    in(c, "c load", (hD + tc) * 4, 4, 0, z.c, t);
    in(c, "g load", KDA ? (hD + tc) * 4 : bh * 4, 4, 0, z.g, t);
    in(c, "beta load", bh * 4, 4, 0, z.beta, t);
    // entries: rows e < E hold data and must be inside the descriptor
    const int grp = t / 16, li = t % 16, i0 = li * CPL, q4 = t % NQ, ph = t / NQ;
    for (int k = 0; k < KPF; ++k) {
      const int e = grp + NG * k;
      if (e < E) {
        key_row(c, "entry key row", e, i0, CPL, rk_size, t);
        g_row(c, "entry G row", e, i0, CPL, rg_size, t);
      }
    }
    for (int k = 0; k < PFE; ++k) {
      const int e = ph + EP * k;
      if (e < E) in(c, "entry value row", (long long)(e * D + 4 * q4) * 4, 16, 0, rk_size, t);
    }
    // G of the last entry, plain pointer into the head's entry block (KDA:
    // only with a buffered token, compensators carry G = 0)
    if (KDA && c.n > 0) in(c, "last G", eg0 + (long long)((E - 1) * D + tc) * 4, 4, eg0, eg0 + (long long)NE * D * 4, t);
    if (!KDA && E > 0) in(c, "last G", eg0 + (long long)(E - 1) * 4, 4, eg0, eg0 + (long long)NE * 4, t);
    // compute: LDS indices
    if (chan) {
      in(c, "lds x", t, 1, 0, D, t);
      const int kbl = t >> 6, pos = (t & 48) | (BITS == 8 ? (t & 15) : ((t & 1) ? 8 + ((t & 15) >> 1) : ((t & 15) >> 1)));
      in(c, "lds limb block", kbl, 1, 0, KB, t);
      in(c, "lds limb position", pos, 1, 0, 64, t);
    }
    // key-side dots: every pass of the row groups
    int e0 = 0;
    do {
      for (int k = 0; k < KPF; ++k) {
        const int e = e0 + grp + NG * k;
        if (e >= E && e0 + NG * k > 0) {
          in(c, "lds kappa (zero row)", e, 1, 0, MAX_ROWS, t);
          continue;
        }
        in(c, "lds kappa", e, 1, 0, MAX_ROWS, t);
        if (e0 > 0) {  // rows past the prefetch, loaded in the pass
          key_row(c, "entry key row (pass)", e, i0, CPL, rk_size, t);
          g_row(c, "entry G row (pass)", e, i0, CPL, rg_size, t);
        }
      }
      e0 += NG * KPF;
    } while (e0 < E);
    for (int k = 0; k < PFE; ++k) {
      const int e = ph + EP * k;
      if (e >= E && k > 0) continue;
      in(c, "lds kappa read", e, 1, 0, MAX_ROWS, t);
    }
    for (int e = ph + EP * PFE; e < E; e += EP) {
      in(c, "entry value row (loop)", (long long)(e * D + 4 * q4) * 4, 16, 0, rk_size, t);
      in(c, "lds kappa read (loop)", e, 1, 0, MAX_ROWS, t);
    }
    in(c, "lds value partials", (long long)ph * 2 * D + 4 * q4, 4, 0, (long long)EP * 2 * D, t);
    in(c, "lds limb operand row", lane & 15, 1, 0, 16, t);
    for (int rb = 0; rb < RBW; ++rb) {
      if ((lane >> 4) < 2) in(c, "lds readout", 16 * (wave * RBW + rb) + (lane & 15), 1, 0, D, t);
    }
    // stores
    if (chan) {
      in(c, "o store", (hD + t) * 4, 4, 0, z.o, t);
      in(c, "appended value", eu0 + (long long)(E * D + t) * 4, 4, eu0, eu0 + (long long)NE * D * 4, t);
      if (c.BF16) {  // a token's bf16 key in the first half of its row (a D * 2-byte descriptor)
        in(c, "appended key (bf16)", (long long)t * 2, 2, 0, (long long)D * 2, t);
        in(c, "appended key row", ek0 + (long long)E * D * 4, (long long)D * 2, ek0, ek0 + (long long)NE * D * 4, t);
      } else {
        in(c, "appended key", ek0 + (long long)(E * D + t) * 4, 4, ek0, ek0 + (long long)NE * D * 4, t);
      }
      if (KDA) in(c, "appended G", eg0 + (long long)(E * D + t) * 4, 4, eg0, eg0 + (long long)NE * D * 4, t);
      if (t == 0) {
        if (!KDA) in(c, "appended G", eg0 + (long long)E * 4, 4, eg0, eg0 + (long long)NE * 4, t);
        in(c, "length store", bh * 4, 4, 0, z.blen, t);
      }
    }
  }
}

// ---------------------------------------------------------------- window close / encode
void close_kernel(const Cfg& c, bool dense, bool warm, bool step = false) {
  const Sizes z = sizes(c);
  const int D = c.D, BITS = c.BITS, KDA = c.KDA, NT = 128;
  const int RB = D / 8, CB = D / 16, CH0 = D == 128 ? 20 : 32, CH1 = 16, V4 = D / 4;
  const int PER0 = CH0 * V4 / NT, PER1 = CH1 * V4 / NT, PX = 20, PR = 16 * PX + 16;
  if (PER0 * NT != CH0 * V4 || PER1 * NT != CH1 * V4) fail(c, "staging shape", PER0, 0, 0, -1);
  const long long bh = c.bh, hD = bh * D, erow = bh * (long long)(c.r + c.w_max);
  const int n = c.n, E = c.r + n, r = c.r;
  const long long HB = (long long)D * D * BITS / 8;
  for (int t = 0; t < NT; ++t) {
    const int tj = t & 15, ti = t >> 4, lane = t & 63, wave = t >> 6;
    const int i0 = ti * RB, j0 = tj * CB;
    if (dense) {
      for (int bb = 0; bb < CB; ++bb) in(c, "dense state load", ((hD + j0 + bb) * D + i0) * 4, RB * 4, 0, (long long)c.BH * D * D * 4, t);
    } else {
      if (step) {  // the token: k, q, v into LDS rows; its decay; beta
        const int ab = c.BF16 ? 2 : 4;
        if (t < D) {
          in(c, "token k/q load", (hD + t) * ab, ab, 0, z.act_qk, t);
          in(c, "token v load", (hD + t) * ab, ab, 0, z.act_v, t);
          in(c, "lds token rows", t, 1, 0, D, t);
        }
        if (KDA) {
          in(c, "token decay rows", (hD + i0) * 4, RB * 4, 0, z.g, t);
          in(c, "token decay quad", (hD + 4 * (t % V4)) * 4, 16, 0, z.g, t);
        } else {
          in(c, "token decay", bh * 4, 4, 0, z.g, t);
        }
        in(c, "token beta", bh * 4, 4, 0, z.beta, t);
      }
      in(c, "s load", (hD + i0) * 4, RB * 4, 0, z.s, t);
      in(c, "c load", (hD + j0) * 4, CB * 4, 0, z.c, t);
      if (KDA && n > 0) in(c, "last G row", ((erow + E - 1) * D + i0) * 4, RB * 4, 0, z.eg, t);
      if (!KDA && E > 0) in(c, "last G", (erow + E - 1) * 4, 4, 0, z.eg, t);
      for (int bb = 0; bb < CB; ++bb) {
        const long long head = bh * HB;
        if (BITS == 6) {
          in(c, "6-bit hi codes", head + (long long)(j0 + bb) * (D / 2) + i0 / 2, RB / 2, head, head + (long long)D * D / 2, t);
          const int NJ = D / 16, j = j0 + bb, g = i0 / 16;
          const long long w = (long long)D * D / 2 + 4LL * (((j & 15) * NJ + g) * NJ + (j >> 4));
          in(c, "6-bit lo word", head + w, 4, head + (long long)D * D / 2, head + HB, t);
        } else {
          in(c, "codes", head + (long long)(j0 + bb) * (D * BITS / 8) + i0 * BITS / 8, RB * BITS / 8, head, head + HB, t);
        }
      }
      const int c4 = t % V4;
      if (KDA && n > 0) in(c, "last G quad", ((erow + E - 1) * D + 4 * c4) * 4, 16, 0, z.eg, t);
      // range-checked row descriptors: keys and values over this head's E
      // rows; G (KDA) over its n buffered rows from entry r, (GDN) E floats
      const long long rk0 = erow * D * 4, rk_size = (long long)E * D * 4;
      const long long rg0 = KDA ? (erow + r) * D * 4 : erow * 4;
      const long long rg_size = KDA ? (long long)n * D * 4 : (long long)E * 4;
      in(c, "close key/value descriptor", rk0, rk_size, 0, z.ek, -1);
      in(c, "close G descriptor", rg0, rg_size, 0, z.eg, -1);
      // passes: the first stages CH0 rows, each later one CH1
      for (int m0 = 0; m0 < E || m0 == 0; m0 += m0 == 0 ? CH0 : CH1) {
        const int ch = m0 == 0 ? CH0 : CH1, np = m0 == 0 ? PER0 : PER1;
        const int cnt = E - m0 < ch ? E - m0 : ch;
        for (int p = 0; p < np; ++p) {
          const int row = (t + NT * p) / V4, e = m0 + row;
          in(c, "lds staged row", row, 1, 0, ch, t);
          if (c.BF16 && !dense && e >= r) {  // a token's bf16 key: four channels in 8 bytes of the row's first half
            const long long off = (long long)e * D * 4 + 8 * c4;
            if (off + 8 > (long long)e * D * 4 + D * 2) fail(c, "staged bf16 key past its half row", off, 0, (long long)e * D * 4 + D * 2, t);
            buffer_load(c, "staged key (bf16)", off, 8, rk_size, t);
          } else {
            buffer_load(c, "staged key", (long long)(e * D + 4 * c4) * 4, 16, rk_size, t);
          }
          buffer_load(c, "staged value", (long long)(e * D + 4 * c4) * 4, 16, rk_size, t);
          if (KDA) {
            const long long off = e >= r ? (long long)((e - r) * D + 4 * c4) * 4 : MODEL_G_COMP_OFF;
            if (e < r && off < rg_size) fail(c, "compensator G offset (close)", off, rg_size, 1LL << 32, t);
            buffer_load(c, "staged G", off, 16, rg_size, t);
          } else {
            buffer_load(c, "staged G", (long long)e * 4, 4, rg_size, t);
          }
        }
        const int nkb = (cnt + 3) >> 2;
        for (int kb = 0; kb < nkb; ++kb) {
          const int e = 4 * kb + (lane >> 4);
          in(c, "lds operand entry", e, 1, 0, ch, t);
          const int a_row = wave * 4 * RB + RB * ((lane & 15) >> 2) + (lane & 3);
          for (int q = 0; q < RB / 4; ++q) in(c, "lds key operand", a_row + 4 * q, 1, 0, D, t);
          in(c, "lds value operand", CB * (lane & 15), CB, 0, D, t);
        }
        if (m0 + ch >= E) break;
      }
    }
    if (step) {  // u = beta (v - M^T k), o = M^T q: token rows from LDS, column sums, the output
      in(c, "lds token key/query rows", i0, RB, 0, D, t);
      in(c, "lds token value row", j0, CB, 0, D, t);
      const int g = lane >> 4;
      for (int sum = 0; sum < 2; ++sum) {
        if (CB == 8) in(c, "lds column partials", j0 + 2 * g, 2, 0, D, t);
        else if (CB == 4) in(c, "lds column partials", j0 + g, 1, 0, D, t);
        else in(c, "lds column partials", j0 + (g >> 1), 1, 0, D, t);
        for (int bb = 0; bb < CB; ++bb) in(c, "lds column read", j0 + bb, 1, 0, D, t);
      }
      split_store(c, "token output store", (hD + j0) * 4, CB, ti, 0, z.o, t);
    }
    for (int l = 0; l < r; ++l) {
      if (RB == 16) {  // kappa's row partials and totals (D = 128)
        for (int k = 0; k < 4; ++k) in(c, "lds kappa partials", (long long)ti * PR + tj * PX + 4 * k, 4, 0, 8LL * PR, t);
        for (int q = 0; q < 16; ++q) in(c, "lds kappa partial read", (long long)ti * PR + q * PX + tj, 1, (long long)ti * PR, (long long)ti * PR + PR, t);
        in(c, "lds kappa total", (long long)ti * 16 + tj, 1, 0, 8 * 16, t);
        for (int k = 0; k < 4; ++k) in(c, "lds kappa totals read", (long long)ti * 16 + 4 * k, 4, 0, 8 * 16, t);
      }
      if (!dense && warm) in(c, "warm start value", ((erow + l) * D + j0) * 4, CB * 4, 0, z.eu, t);
      const int g = lane >> 4;
      if (CB == 8) in(c, "lds column partials", j0 + 2 * g, 2, 0, D, t);
      else if (CB == 4) in(c, "lds column partials", j0 + g, 1, 0, D, t);
      else in(c, "lds column partials", j0 + (g >> 1), 1, 0, D, t);
      for (int bb = 0; bb < CB; ++bb) in(c, "lds column read", j0 + bb, 1, 0, D, t);
      split_store(c, "compensator key store", ((erow + l) * D + i0) * 4, RB, tj, 0, z.ek, t);
      split_store(c, "compensator value store", ((erow + l) * D + j0) * 4, CB, ti, 0, z.eu, t);
      if (KDA) split_store(c, "compensator G store", ((erow + l) * D + i0) * 4, RB, tj, 0, z.eg, t);
      if (!KDA && t == 0) in(c, "compensator G store", (erow + l) * 4, 4, 0, z.eg, t);
    }
    for (int bb = 0; bb < CB; ++bb) in(c, "residual export", ((hD + j0 + bb) * D + i0) * 4, RB * 4, 0, (long long)c.BH * D * D * 4, t);
    const int NV = CB >= 4 ? CB / 4 : 1;
    if (CB >= 4) {
      const int jg = j0 + (lane >> 4) * NV;
      in(c, "lds column maxima", jg, NV, 0, D, t);
    } else {
      for (int bb = 0; bb < CB; ++bb) in(c, "lds column maxima", j0 + bb, 1, 0, D, t);
    }
    const long long head = bh * HB;
    for (int bb = 0; bb < CB; ++bb) {
      const int j = j0 + bb;
      if (BITS == 6) {
        in(c, "6-bit hi code store", head + (long long)j * (D / 2) + i0 / 2, RB / 2, head, head + (long long)D * D / 2, t);
        const int NJ = D / 16;
        const long long w = (long long)D * D / 2 + 4LL * (((j & 15) * NJ + i0 / 16) * NJ + (j >> 4));
        if (ti % (16 / RB) == 0) in(c, "6-bit lo word store", head + w, 4, head + (long long)D * D / 2, head + HB, t);
      } else {
        in(c, "code store", head + (long long)j * (D * BITS / 8) + i0 * BITS / 8, RB * BITS / 8, head, head + HB, t);
      }
    }
    if (RB == 16) in(c, "row scale store", (hD + i0 + tj) * 4, 4, 0, z.s, t);
    else split_store(c, "row scale store", (hD + i0) * 4, RB, tj, 0, z.s, t);
    if (CB >= 4) {
      if (wave == 0)
        for (int m = 0; m < NV; ++m) in(c, "column scale store", (hD + j0 + (lane >> 4) * NV + m) * 4, 4, 0, z.c, t);
    } else if (ti == 0) {
      in(c, "column scale store", (hD + j0) * 4, CB * 4, 0, z.c, t);
    }
    if (t == 0) in(c, "length store", bh * 4, 4, 0, z.blen, t);
  }
}

}  // namespace

// FP32-state baseline: one workgroup of 2D threads per head over a [d_v][d_k]
// fp32 state; D/16 lanes share a value column and lane li holds float4 pieces
// (D/16) w + li, w < 4, of columns grp + NG c. Every piece lies inside its own
// head's state and every float4 of the head is held by exactly one thread.
void baseline(const Cfg& c) {
  const int D = c.D, NT = 2 * D, LPC = D / 16, NG = NT / LPC, CPT = D / NG;
  const long long head = 4LL * D * D, lo = head * c.bh, hi = lo + head;
  static int held[128 * 128 / 4];
  for (int x = 0; x < D * D / 4; ++x) held[x] = 0;
  for (int t = 0; t < NT; ++t) {
    const int grp = t / LPC, li = t % LPC;
    for (int cc = 0; cc < CPT; ++cc) {
      const long long j = grp + NG * cc;
      in(c, "baseline v/o column", 4LL * (c.bh * (long long)D + j), 4, 4LL * c.bh * D, 4LL * (c.bh + 1) * D, t);
      for (int w = 0; w < 4; ++w) {
        const long long piece = j * (D / 4) + LPC * w + li + MODEL_BL_PIECE_OFF;  // float4 index inside the head
        in(c, "baseline state piece", lo + 16 * piece, 16, lo, hi, t);
        ++held[piece];
      }
    }
    for (int w = 0; w < 4; ++w) in(c, "baseline lds k/q/decay", 16LL * (LPC * w + li), 16, 0, 4LL * D, t);
    if (t < D) in(c, "baseline lds fill", 4LL * t, 4, 0, 4LL * D, t);
  }
  for (int x = 0; x < D * D / 4; ++x) {
    ++checks;
    if (held[x] != 1) fail(c, "baseline state coverage (pieces held once)", x, held[x], 1, -1);
  }
}

int main() {
  const int dims[] = {32, 64, 128}, bits[] = {8, 6, 4};
  const int wmaxes[] = {1, 2, 3, 4, 7, 8, 15, 16, 17, 20, 23, 24, 25, 31, 32, 33, 47, 48, 49, 63, 64};
  const int BH = 3;
  long long configs = 0;
  for (int D : dims)
    for (int BITS : bits)
      for (int KDA = 0; KDA < 2; ++KDA)
        for (int r = 0; r <= 8; ++r)
          for (int w_max : wmaxes)
            for (int bh = 0; bh < BH; bh += BH - 1) {
              for (int BF16 = 0; BF16 < 2; ++BF16)
                for (int n = 0; n < w_max; ++n) {  // decode: buf_len < w_max
                  decode_step(Cfg{D, BITS, KDA, BF16, r, w_max, n, bh, BH});
                  ++configs;
                }
              for (int BF16 = 0; BF16 < 2; ++BF16)  // (bf16: the buffered keys are bf16)
                for (int n = 0; n <= w_max; ++n)      // close: buf_len <= w_max
                  for (int warm = 0; warm < 2; ++warm) {
                    close_kernel(Cfg{D, BITS, KDA, BF16, r, w_max, n, bh, BH}, false, warm);
                    ++configs;
                  }
              close_kernel(Cfg{D, BITS, KDA, 0, r, w_max, 0, bh, BH}, true, false);  // encode
              ++configs;
              for (int BF16 = 0; BF16 < 2; ++BF16)
                for (int n = 0; n < w_max; ++n) {  // the window's last token, then the close
                  close_kernel(Cfg{D, BITS, KDA, BF16, r, w_max, n, bh, BH}, false, false, true);
                  ++configs;
                }
            }
  for (int D : dims)
    for (int bh = 0; bh < BH; ++bh) {
      baseline(Cfg{D, 0, 0, 0, 0, 0, 0, bh, BH});
      ++configs;
    }
  std::printf("bounds model: %lld launch configurations, %lld access checks, all inside their buffers\n", configs,
              checks);
  return 0;
}
