/*
 * leapquant.h -- C ABI of the LeapQuant decode path for delta-rule linear
 * attention (Gated DeltaNet with scalar decay, Kimi Delta Attention with
 * per-key-channel decay) on AMD MI355X (gfx950).
 *
 * Method: "LeapQuant: Efficient Linear Attention with Accurate Recurrent State
 * Quantization" (original abstract) and the wink.run article "Linear attention
 * has to move state every token it generates; LeapQuant compresses it to 8-bit
 * without losing accuracy" (paragraphs on per-window quantization, compensator
 * tokens and residual smoothing). Recurrences: Gated Delta Networks (Yang et
 * al., ICLR 2025) and Kimi Delta Attention (Kimi Linear report, 2025).
 *
 * Per (sequence b, head h) -- a "head" below -- the recurrent state
 * S in R^{d_k x d_v} (row i = key channel, column j = value channel) is held as
 * a window-start residual diag(s) C diag(c) (symmetric 8-, 6- or 4-bit codes C with
 * per-key-row smoothing scales s and per-value-column scales c), fixed for a
 * window, plus a list of fp32 rank-one entries (k_e, u_e, G_e):
 *   S = exp(G) (.) diag(s) C diag(c) + sum_e exp(G - G_e) (.) k_e u_e^T
 * where G is the cumulative log-decay since the window start and (.) scales
 * key rows. The first r entries are the compensator tokens (unit keys, G_e = 0:
 * they sit at window position 0 and take the same update path as tokens);
 * the next n are the window's buffered tokens, G_e = G at that token.
 *
 * Conventions for every entry point:
 *  - Every pointer is a DEVICE pointer unless marked (host). The caller
 *    allocates and frees all memory; the library allocates nothing and keeps
 *    no mutable global state.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). Work
 *    is enqueued asynchronously; the library never synchronises.
 *  - Arguments are validated on the host before anything is enqueued. A
 *    rejected call returns a negative LQ_ERR_* code and enqueues nothing.
 *    Launch failures return LQ_ERR_LAUNCH. Faults inside a kernel surface at
 *    the caller's next synchronisation.
 *  - batch * heads == 0 is a valid empty call: it returns LQ_OK and enqueues
 *    nothing.
 *  - Layouts are dense and row-major in the order written; "head index"
 *    bh = b * heads + h. State buffers, dense states and o must be 16-byte
 *    aligned; q, k, v 16-byte (fp32) or 8-byte (bf16); g, beta, buf_len, err
 *    and close lists 4-byte (LQ_ERR_ALIGN otherwise).
 *  - Supported shapes (build-time limit): d_k == d_v in {32, 64, 128}.
 */
#ifndef LEAPQUANT_H
#define LEAPQUANT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define LQ_OK 0
#define LQ_ERR_NULL (-1)   /* a required pointer is NULL */
#define LQ_ERR_SHAPE (-2)  /* unsupported batch/heads/d_k/d_v */
#define LQ_ERR_BITS (-3)   /* bits not 4, 6 or 8 */
#define LQ_ERR_CONFIG (-4) /* w_max, n_comp, power_iters, flags or close list out of range */
#define LQ_ERR_LAUNCH (-5) /* the HIP launch failed */
#define LQ_ERR_ALIGN (-6)  /* a buffer is not aligned as the conventions above require */

/* activation dtypes for q, k, v */
#define LQ_ACT_F32 0
#define LQ_ACT_BF16 1

/* bits of the device error word lq_state.err */
#define LQ_DEVERR_BUFFER_FULL 1 /* decode_step met a head whose buffer held w_max entries */
#define LQ_DEVERR_BAD_SEQ 2     /* window_close met a sequence id outside [0, batch) */
#define LQ_DEVERR_BAD_LEN 4     /* a head's buf_len was outside [0, w_max]; the head was skipped */

/* Problem shape and method parameters (host struct, passed by pointer). */
typedef struct lq_dims {
  int32_t batch;             /* B sequences, >= 0 */
  int32_t heads;             /* H heads per sequence, >= 0 */
  int32_t d_k, d_v;          /* key / value head dims; equal, in {32, 64, 128} */
  int32_t w_max;             /* buffer capacity per head, 1..64 (>= every window length used) */
  int32_t n_comp;            /* r compensators, 0..8 */
  int32_t bits;              /* 8, 6 or 4 */
  int32_t decay_per_channel; /* 0: GDN, g is [B][H]; 1: KDA, g is [B][H][d_k] */
  int32_t act_dtype;         /* LQ_ACT_F32 or LQ_ACT_BF16 for q, k, v */
  int32_t smoothing;         /* 1: per-key-row smoothing scales; 0: s == 1 */
  int32_t power_iters;       /* T power iterations per compensator, 1..64 */
  int32_t warm_start;        /* 0: every close starts the power method from the fixed
                                SplitMix64 vectors; 1: a close starts compensator l from
                                the head's current compensator value u_l (the window that
                                is closing), falling back to the fixed vector where u_l is
                                zero. A variant, not on the pages; encode always starts
                                from the fixed vectors. */
} lq_dims;

/* The LeapQuant state of all B*H heads (device buffers owned by the caller).
   Entry arrays hold r + w_max entries per head: entries 0..r-1 are the
   compensators, entries r..r+n-1 the buffered tokens (n = buf_len). */
typedef struct lq_state {
  void* codes;       /* codes in [-Q, Q], Q = 2^(bits-1) - 1; per head
                        (d = d_k = d_v, value column j, key channel i):
                        8 bits: int8 [d_v][d_k], two's complement;
                        4 bits: [d_v][d_k/2] bytes, channel 2m in the low
                        nibble and 2m+1 in the high nibble of byte m;
                        6 bits: 3*d*d/4 bytes in two planes, code = 4*hi + lo:
                        first d*d/2 bytes: hi = code >> 2 (arithmetic, in
                        [-8, 7]) in the 4-bit layout; then d*d/16 little-endian
                        32-bit words W[j % 16][i / 16][j / 16], word holding
                        lo = code & 3 of channels 16*(i/16) .. +15 of column
                        j, channel c = i % 16 at bits 8*(p%4) + 2*(p/4) with
                        p = c/2 for even c and 8 + c/2 for odd c. */
  float* row_scale;  /* s [B*H][d_k] key-row smoothing scales */
  float* col_scale;  /* c [B*H][d_v] value-column scales */
  float* ent_k;      /* [B*H][r + w_max][d_k] entry keys (compensator keys are unit vectors).
                        With act_dtype LQ_ACT_BF16 a buffered token's key row (entries r..)
                        holds its bf16 key k_t, exactly as given, in the row's first
                        d_k * 2 bytes (little-endian bf16, channel order); the rest of that
                        row is unused. Compensator rows are fp32 either way. A state is
                        therefore used with one act_dtype while its buffer holds tokens
                        (at a window boundary the buffer is empty and either may follow). */
  float* ent_u;      /* [B*H][r + w_max][d_v] entry values u_e */
  float* ent_g;      /* [B*H][r + w_max] (GDN) or [B*H][r + w_max][d_k] (KDA): G_e, the
                        cumulative log-decay since the window start (0 for compensators;
                        the KDA kernels take that value and do not read those rows) */
  int32_t* buf_len;  /* [B*H] buffered tokens n per head */
  int32_t* err;      /* [1] device error word (LQ_DEVERR_* bits), may be NULL */
} lq_state;

/* Number of device buffers in lq_state whose sizes lq_state_sizes reports,
   in the field order above: codes, row_scale, col_scale, ent_k, ent_u,
   ent_g, buf_len, err. */
#define LQ_STATE_NBUF 8

/* Host-only helper: bytes needed for each lq_state buffer (err: 4 bytes).
   bytes_out (host) receives LQ_STATE_NBUF sizes. Validates dims. */
int lq_state_sizes(const lq_dims* dims, size_t* bytes_out);

/* Encode fp32 dense states into LeapQuant form: compensator extraction by a
   T-step power method with deflation (start vectors from SplitMix64), key-row
   smoothing, symmetric quantisation with per-value-column scales; writes the
   compensators as entries 0..r-1 and empties every buffer (buf_len = 0).
   Same arithmetic as a window close with no entries. Sources: LeapQuant
   abstract (compensator tokens, smoothing) and the wink.run article's
   compensator and smoothing paragraphs.
   S: fp32 [B*H][d_v][d_k] (element (j, i) = S[i][j], i.e. S transposed).
   dbg_residual: NULL, or fp32 [B*H][d_v][d_k] receiving the residual after
   the compensators are removed and before smoothing/rounding. */
int leapquant_encode(const lq_dims* dims, const float* S, const lq_state* st,
                     float* dbg_residual, void* stream);

/* One decode token for every head. Source: the wink.run article, paragraph on
   per-window quantization (the low-bit state stays frozen for a window and
   each token's update is kept in a full-precision buffer), and the
   compensator-token paragraph (compensators are updates of the same shape as
   a token's, read on the same path); LeapQuant abstract. Per head, with
   G_t = G_{t-1} + g_t (G_{t-1} = G of the last entry, 0 if there is none):
     y^x = c (.) C^T (s (.) exp(G_t) (.) x) + sum_e u_e (k_e . (exp(G_t - G_e) (.) x)),
     u_t = beta_t (v_t - y^k),  o_t = y^q + (k_t . q_t) u_t,
   with entries e = 0..r+n-1 of the head (compensators included), then appends
   (k_t, u_t, G_t) as entry r+n (k_t at the activation width, see lq_state.ent_k)
   and increments buf_len.
   q, k: [B][H][d_k]; v: [B][H][d_v] (fp32 or bf16 per act_dtype);
   g: fp32 [B][H] (GDN) or [B][H][d_k] (KDA), the log-decay (alpha = exp(g));
   beta: fp32 [B][H]; o: fp32 [B][H][d_v] (output).
   Precondition: every head has buf_len < w_max. A head with a full buffer is
   left unchanged (its o is not written) and LQ_DEVERR_BUFFER_FULL is or-ed
   into *st->err when err is not NULL. */
int leapquant_decode_step(const lq_dims* dims, const lq_state* st, const void* q, const void* k,
                          const void* v, const float* g, const float* beta, float* o,
                          void* stream);

/* leapquant_decode_step for a state whose every head holds n buffered tokens,
   0 <= n < w_max: the caller's window schedule knows the position (every
   sequence's windows aligned, as when they start together and share W; the
   wink.run article, per-window quantization). The same step, bit for bit; the
   kernel needs no head's buffer length before it issues the entry-row loads,
   so every load goes out in the order the arithmetic uses it. Arguments as
   leapquant_decode_step. Returns LQ_ERR_CONFIG for n outside [0, w_max). A
   head whose stored buf_len differs from n is left unchanged (its o is not
   written) and LQ_DEVERR_BAD_LEN is or-ed into *st->err when err is not
   NULL. */
int leapquant_decode_step_at(const lq_dims* dims, const lq_state* st, int32_t n, const void* q,
                             const void* k, const void* v, const float* g, const float* beta,
                             float* o, void* stream);

/* Window close for a list of sequences (all heads of each): fold the entries
   into the dense state S = exp(G_n) (.) diag(s) C diag(c) + sum_e exp(G_n - G_e) (.) k_e u_e^T
   (G_n = G of the last entry), re-extract the compensators into entries
   0..r-1, re-smooth, requantise, and empty the buffer (buf_len = 0).
   A partly filled buffer is legal (a partial window). Sources: LeapQuant
   abstract (one requantization per window; compensators and smoothing).
   seq_ids: int32 [n_seq] distinct sequence ids in [0, B), or NULL for all B
   sequences (n_seq is then ignored). An id outside [0, B) is skipped and
   LQ_DEVERR_BAD_SEQ is or-ed into *st->err. Duplicated ids race.
   dbg_residual: NULL or fp32 [B*H][d_v][d_k]; rows of closed sequences get
   the pre-quantisation residual. */
int leapquant_window_close(const lq_dims* dims, const lq_state* st, const int32_t* seq_ids,
                           int32_t n_seq, float* dbg_residual, void* stream);

/* The window's last decode token and its window close in one pass, for a
   state whose every head holds n buffered tokens, 0 <= n < w_max, and whose
   every sequence closes after this token (aligned windows; the wink.run
   article, per-window quantization: the state is requantized once per window,
   after the window's last token). Per head the result is that of
   leapquant_decode_step_at(n) followed by leapquant_window_close of every
   sequence, up to fp32 rounding: the token's step is taken on the folded
   fp32 state instead of the codes plus the buffer, with G_t = G_n + g_t,
     S = decay of the folded state to G_t,  u_t = beta_t (v_t - S^T k_t),
     S += k_t u_t^T,  o_t = S^T q_t,
   and the token is not appended (the close empties the buffer). Then the
   compensators, smoothing and codes as leapquant_window_close. Arguments as
   leapquant_decode_step_at (o is written); dbg_residual as
   leapquant_window_close (NULL, or fp32 [B*H][d_v][d_k]). Returns
   LQ_ERR_CONFIG for n outside [0, w_max). A head whose stored buf_len differs
   from n is left unchanged (its o is not written) and LQ_DEVERR_BAD_LEN is
   or-ed into *st->err when err is not NULL. */
int leapquant_decode_close_at(const lq_dims* dims, const lq_state* st, int32_t n, const void* q,
                              const void* k, const void* v, const float* g, const float* beta,
                              float* o, float* dbg_residual, void* stream);

/* FP32-state baseline: one exact decode token of the gated delta rule with the
   state kept in fp32 (no quantisation), the full-precision state that the
   LeapQuant abstract and the wink.run article's results table and speed
   paragraph compare against (gated delta rule: Gated DeltaNet; per-channel
   decay: Kimi Delta Attention). Decay first:
     S' = alpha (.)_rows S,  u = beta (v - S'^T k),  S = S' + k u^T,  o = S^T q.
   S: fp32 [B*H][d_v][d_k] (transposed, in/out). Other arguments as
   leapquant_decode_step. Only batch, heads, d_k, d_v, decay_per_channel and
   act_dtype of dims are used. */
int gdn_decode_fp32_baseline(const lq_dims* dims, float* S, const void* q, const void* k,
                             const void* v, const float* g, const float* beta, float* o,
                             void* stream);

/* Prefill handoff: the exact gated delta rule (decay first, as
   gdn_decode_fp32_baseline) over n_tokens prompt tokens with the fp32 state
   held on chip, then, when st is not NULL, the encode of the final state
   into st (as leapquant_encode: compensators, smoothing, quantization, empty
   buffer), so that decoding starts from the prompt. The pages quantize the
   state per window of decoded tokens (wink.run article, per-window
   quantization; LeapQuant abstract); the prompt runs at full precision and
   is quantized once, at the handoff. At d_k = 128 the prompt is evaluated
   in chunks of 16 tokens (the same recurrence reassociated into matrix
   products), so results agree with the token-by-token form to fp32 rounding.
   S: fp32 [B*H][d_v][d_k] (transposed), the state before the prompt on
   entry and after it on return. Tokens are time-major: q, k: [n_tokens][B][H]
   [d_k]; v: [n_tokens][B][H][d_v] (fp32 or bf16 per act_dtype); g: fp32
   [n_tokens][B][H] (GDN) or [n_tokens][B][H][d_k] (KDA), the log-decay;
   beta: fp32 [n_tokens][B][H]; o: fp32 [n_tokens][B][H][d_v] (output).
   n_tokens >= 0 (0: encode only). The method fields of dims (w_max, n_comp,
   bits, smoothing, power_iters) are validated only when st is not NULL. */
int leapquant_prefill(const lq_dims* dims, float* S, int32_t n_tokens, const void* q,
                      const void* k, const void* v, const float* g, const float* beta,
                      float* o, const lq_state* st, void* stream);

/* Prefix-cache snapshots. At a window boundary the buffer is empty and a
   head's state is its codes, scales and compensators (LeapQuant abstract;
   wink.run article, prefix caching and memory paragraphs), which is all a
   snapshot keeps. One record per head, in this order: codes
   (d_k*d_v*bits/8 bytes, the layout of lq_state.codes), row scales (4*d_k),
   column scales (4*d_v), compensator keys (4*r*d_k), compensator values
   (4*r*d_v). snap: [n_seq][H][record] (or [B][H][record] when seq_ids is
   NULL), 16-byte aligned, caller-owned. */

/* Host-only: bytes of one head's snapshot record. */
int lq_snapshot_bytes(const lq_dims* dims, size_t* bytes_per_head);

/* Copy the state of the listed sequences (NULL: all) into snap. Every listed
   head must be at a window boundary (buf_len == 0); a head that is not is
   skipped, its record left as it was, and LQ_DEVERR_BAD_LEN is or-ed into
   *st->err. Ids outside [0, B) set LQ_DEVERR_BAD_SEQ. */
int leapquant_snapshot(const lq_dims* dims, const lq_state* st, const int32_t* seq_ids,
                       int32_t n_seq, void* snap, void* stream);

/* Write snapshot records back into the listed sequences: codes, scales and
   compensators, compensator G = 0, buf_len = 0 (a window start). The
   records of snap are taken in the same order as seq_ids. */
int leapquant_restore(const lq_dims* dims, const lq_state* st, const int32_t* seq_ids,
                      int32_t n_seq, const void* snap, void* stream);

/* Dense window-start state Shat_0 = sum_{e<r} k_e u_e^T + diag(s) C diag(c)
   (compensators plus residual) of every head into S_out: fp32
   [B*H][d_v][d_k] (transposed). Source: the wink.run article's
   compensator-token and residual-smoothing paragraphs (the state is the
   rank-one compensators plus the smoothed, quantized residual). Reads the
   codes, the scales and entries 0..r-1 only (the buffered entries are not
   part of Shat_0); writes nothing but S_out. Test helper. */
int leapquant_dequantize(const lq_dims* dims, const lq_state* st, float* S_out, void* stream);

/* Host-only: sequences whose window ends with decode token `step` (0-based),
   i.e. (win_off[b] + step + 1) % win_len[b] == 0, written in increasing order
   to out_ids (host, capacity batch). win_len (host) [batch] window lengths
   >= 1; win_off (host) [batch] start positions inside the first window, in
   [0, win_len[b]). Returns the count, or a negative LQ_ERR_* code. */
int32_t lq_close_list(const int32_t* win_len, const int32_t* win_off, int32_t batch, int64_t step,
                      int32_t* out_ids);

/* Host-only: static text for a status code. */
const char* lq_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* LEAPQUANT_H */
