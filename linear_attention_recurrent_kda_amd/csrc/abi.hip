// C ABI of the LeapQuant decode library: host-side validation, then one
// asynchronous launch on the caller's stream. Nothing here allocates,
// synchronises or keeps state; a rejected call enqueues nothing and makes no
// HIP call at all.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "leapquant.h"
#include "lq_launch.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_dims(const lq_dims* d, bool method) {
  if (!d) return LQ_ERR_NULL;
  if (d->batch < 0 || d->heads < 0) return LQ_ERR_SHAPE;
  if (int64_t(d->batch) * int64_t(d->heads) > int64_t(INT32_MAX)) return LQ_ERR_SHAPE;
  if (d->d_k != d->d_v) return LQ_ERR_SHAPE;
  if (d->d_k != 32 && d->d_k != 64 && d->d_k != 128) return LQ_ERR_SHAPE;
  if (d->decay_per_channel != 0 && d->decay_per_channel != 1) return LQ_ERR_CONFIG;
  if (d->act_dtype != LQ_ACT_F32 && d->act_dtype != LQ_ACT_BF16) return LQ_ERR_CONFIG;
  if (method) {
    if (d->bits != 8 && d->bits != 6 && d->bits != 4) return LQ_ERR_BITS;
    if (d->w_max < 1 || d->w_max > 64) return LQ_ERR_CONFIG;
    if (d->n_comp < 0 || d->n_comp > 8) return LQ_ERR_CONFIG;
    if (d->power_iters < 1 || d->power_iters > 64) return LQ_ERR_CONFIG;
    if (d->smoothing != 0 && d->smoothing != 1) return LQ_ERR_CONFIG;
    if (d->warm_start != 0 && d->warm_start != 1) return LQ_ERR_CONFIG;
  }
  return LQ_OK;
}

// buffers: 0 = codes/scales/entries, 1 = + buf_len
int check_state(const lq_dims* d, const lq_state* st, int buffers) {
  if (!st) return LQ_ERR_NULL;
  if (!st->codes || !st->row_scale || !st->col_scale) return LQ_ERR_NULL;
  if (!st->ent_k || !st->ent_u || !st->ent_g) return LQ_ERR_NULL;
  if (buffers >= 1 && !st->buf_len) return LQ_ERR_NULL;
  const void* a16[] = {st->codes, st->row_scale, st->col_scale, st->ent_k, st->ent_u, st->ent_g};
  for (const void* p : a16)
    if (!aligned(p, 16)) return LQ_ERR_ALIGN;
  if ((st->buf_len && !aligned(st->buf_len, 4)) || (st->err && !aligned(st->err, 4))) return LQ_ERR_ALIGN;
  return LQ_OK;
}

int check_acts(const lq_dims* d, const void* q, const void* k, const void* v, const float* g,
               const float* beta, const float* o) {
  if (!q || !k || !v || !g || !beta || !o) return LQ_ERR_NULL;
  // value rows and outputs move four channels per access
  const uintptr_t ea = d->act_dtype == LQ_ACT_BF16 ? 8 : 16;
  if (!aligned(q, ea) || !aligned(k, ea) || !aligned(v, ea)) return LQ_ERR_ALIGN;
  if (!aligned(g, 4) || !aligned(beta, 4) || !aligned(o, 16)) return LQ_ERR_ALIGN;
  return LQ_OK;
}

bool empty(const lq_dims* d) { return d->batch == 0 || d->heads == 0; }

lq::StepArgs step_args(const lq_dims* d, const lq_state* st) {
  lq::StepArgs a{};
  a.codes = st->codes;
  a.s = st->row_scale;
  a.c = st->col_scale;
  a.ek = st->ent_k;
  a.eu = st->ent_u;
  a.eg = st->ent_g;
  a.blen = st->buf_len;
  a.err = st->err;
  a.r = d->n_comp;
  a.w_max = d->w_max;
  a.n_at = -1;
  return a;
}

lq::CloseArgs close_args(const lq_dims* d, const lq_state* st) {
  lq::CloseArgs a{};
  a.codes = st->codes;
  a.s = st->row_scale;
  a.c = st->col_scale;
  a.ek = st->ent_k;
  a.eu = st->ent_u;
  a.eg = st->ent_g;
  a.blen = st->buf_len;
  a.err = st->err;
  a.batch = d->batch;
  a.heads = d->heads;
  a.r = d->n_comp;
  a.w_max = d->w_max;
  a.T = d->power_iters;
  a.smoothing = d->smoothing;
  a.warm = d->warm_start;
  return a;
}

int launched(hipError_t e) { return e == hipSuccess ? LQ_OK : LQ_ERR_LAUNCH; }

}  // namespace

extern "C" {

int lq_state_sizes(const lq_dims* d, size_t* out) {
  int rc = check_dims(d, true);
  if (rc) return rc;
  if (!out) return LQ_ERR_NULL;
  const size_t BH = size_t(d->batch) * size_t(d->heads), D = size_t(d->d_k);
  const size_t NE = size_t(d->w_max) + size_t(d->n_comp);  // entries per head
  out[0] = BH * D * D * size_t(d->bits) / 8;
  out[1] = BH * D * 4;
  out[2] = BH * D * 4;
  out[3] = BH * NE * D * 4;
  out[4] = BH * NE * D * 4;
  out[5] = BH * NE * (d->decay_per_channel ? D : 1) * 4;
  out[6] = BH * 4;
  out[7] = 4;
  return LQ_OK;
}

int leapquant_encode(const lq_dims* d, const float* S, const lq_state* st, float* dbg, void* stream) {
  int rc = check_dims(d, true);
  if (rc) return rc;
  if (empty(d)) return LQ_OK;
  if ((rc = check_state(d, st, 1))) return rc;
  if (!S) return LQ_ERR_NULL;
  if (!aligned(S, 16) || (dbg && !aligned(dbg, 16))) return LQ_ERR_ALIGN;
  lq::CloseArgs a = close_args(d, st);
  a.S = S;
  a.dbg = dbg;
  return launched(lq::launch_close(*d, a, d->batch * d->heads, static_cast<hipStream_t>(stream)));
}

int leapquant_decode_step(const lq_dims* d, const lq_state* st, const void* q, const void* k,
                          const void* v, const float* g, const float* beta, float* o, void* stream) {
  int rc = check_dims(d, true);
  if (rc) return rc;
  if (empty(d)) return LQ_OK;
  if ((rc = check_state(d, st, 1))) return rc;
  if ((rc = check_acts(d, q, k, v, g, beta, o))) return rc;
  lq::StepArgs a = step_args(d, st);
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.o = o;
  return launched(lq::launch_decode_step(*d, a, static_cast<hipStream_t>(stream)));
}

int leapquant_decode_step_at(const lq_dims* d, const lq_state* st, int32_t n, const void* q, const void* k,
                             const void* v, const float* g, const float* beta, float* o, void* stream) {
  int rc = check_dims(d, true);
  if (rc) return rc;
  if (n < 0 || n >= d->w_max) return LQ_ERR_CONFIG;
  if (empty(d)) return LQ_OK;
  if ((rc = check_state(d, st, 1))) return rc;
  if ((rc = check_acts(d, q, k, v, g, beta, o))) return rc;
  lq::StepArgs a = step_args(d, st);
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.o = o;
  a.n_at = n;
  return launched(lq::launch_decode_step(*d, a, static_cast<hipStream_t>(stream)));
}

int leapquant_decode_close_at(const lq_dims* d, const lq_state* st, int32_t n, const void* q, const void* k,
                              const void* v, const float* g, const float* beta, float* o, float* dbg,
                              void* stream) {
  int rc = check_dims(d, true);
  if (rc) return rc;
  if (n < 0 || n >= d->w_max) return LQ_ERR_CONFIG;
  if (empty(d)) return LQ_OK;
  if ((rc = check_state(d, st, 1))) return rc;
  if ((rc = check_acts(d, q, k, v, g, beta, o))) return rc;
  if (dbg && !aligned(dbg, 16)) return LQ_ERR_ALIGN;
  lq::CloseArgs a = close_args(d, st);
  a.dbg = dbg;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.o = o;
  a.n_at = n;
  return launched(lq::launch_close(*d, a, d->batch * d->heads, static_cast<hipStream_t>(stream)));
}

int leapquant_window_close(const lq_dims* d, const lq_state* st, const int32_t* seq_ids, int32_t n_seq,
                           float* dbg, void* stream) {
  int rc = check_dims(d, true);
  if (rc) return rc;
  if (seq_ids && (n_seq < 0 || n_seq > d->batch)) return LQ_ERR_CONFIG;
  if (empty(d) || (seq_ids && n_seq == 0)) return LQ_OK;
  if ((rc = check_state(d, st, 1))) return rc;
  if (dbg && !aligned(dbg, 16)) return LQ_ERR_ALIGN;
  if (seq_ids && !aligned(seq_ids, 4)) return LQ_ERR_ALIGN;
  lq::CloseArgs a = close_args(d, st);
  a.seq_ids = seq_ids;
  a.dbg = dbg;
  const int n_blocks = (seq_ids ? n_seq : d->batch) * d->heads;
  return launched(lq::launch_close(*d, a, n_blocks, static_cast<hipStream_t>(stream)));
}

int gdn_decode_fp32_baseline(const lq_dims* d, float* S, const void* q, const void* k, const void* v,
                             const float* g, const float* beta, float* o, void* stream) {
  int rc = check_dims(d, false);
  if (rc) return rc;
  if (empty(d)) return LQ_OK;
  if (!S) return LQ_ERR_NULL;
  if (!aligned(S, 16)) return LQ_ERR_ALIGN;
  if ((rc = check_acts(d, q, k, v, g, beta, o))) return rc;
  lq::BaselineArgs a{S, q, k, v, g, beta, o};
  return launched(lq::launch_baseline(*d, a, static_cast<hipStream_t>(stream)));
}

int leapquant_prefill(const lq_dims* d, float* S, int32_t n_tokens, const void* q, const void* k,
                      const void* v, const float* g, const float* beta, float* o, const lq_state* st,
                      void* stream) {
  int rc = check_dims(d, st != nullptr);
  if (rc) return rc;
  if (n_tokens < 0) return LQ_ERR_CONFIG;
  if (empty(d)) return LQ_OK;
  if (!S) return LQ_ERR_NULL;
  if (!aligned(S, 16)) return LQ_ERR_ALIGN;
  if (n_tokens > 0 && (rc = check_acts(d, q, k, v, g, beta, o))) return rc;
  if (st && (rc = check_state(d, st, 1))) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (n_tokens > 0) {
    lq::PrefillArgs a{S, q, k, v, g, beta, o, n_tokens, d->batch * d->heads};
    if ((rc = launched(lq::launch_prefill(*d, a, s)))) return rc;
  }
  if (!st) return LQ_OK;
  lq::CloseArgs a = close_args(d, st);  // the handoff: encode the prompt's final state
  a.S = S;
  return launched(lq::launch_close(*d, a, d->batch * d->heads, s));
}

int lq_snapshot_bytes(const lq_dims* d, size_t* bytes_per_head) {
  int rc = check_dims(d, true);
  if (rc) return rc;
  if (!bytes_per_head) return LQ_ERR_NULL;
  const size_t D = size_t(d->d_k);
  *bytes_per_head = D * D * size_t(d->bits) / 8 + 2 * 4 * D + 2 * 4 * size_t(d->n_comp) * D;
  return LQ_OK;
}

namespace {

int snapshot_call(const lq_dims* d, const lq_state* st, const int32_t* seq_ids, int32_t n_seq, const void* snap,
                  bool save, void* stream) {
  int rc = check_dims(d, true);
  if (rc) return rc;
  if (seq_ids && (n_seq < 0 || n_seq > d->batch)) return LQ_ERR_CONFIG;
  if (empty(d) || (seq_ids && n_seq == 0)) return LQ_OK;
  if ((rc = check_state(d, st, 1))) return rc;
  if (!snap) return LQ_ERR_NULL;
  if (!aligned(snap, 16) || (seq_ids && !aligned(seq_ids, 4))) return LQ_ERR_ALIGN;
  lq::SnapshotArgs a{};
  a.codes = st->codes;
  a.s = st->row_scale;
  a.c = st->col_scale;
  a.ek = st->ent_k;
  a.eu = st->ent_u;
  a.eg = st->ent_g;
  a.blen = st->buf_len;
  a.err = st->err;
  a.seq_ids = seq_ids;
  a.snap = const_cast<void*>(snap);
  lq_snapshot_bytes(d, &a.record_bytes);
  a.batch = d->batch;
  a.heads = d->heads;
  a.d = d->d_k;
  a.r = d->n_comp;
  a.w_max = d->w_max;
  a.bits = d->bits;
  a.kda = d->decay_per_channel;
  const int n_blocks = (seq_ids ? n_seq : d->batch) * d->heads;
  return launched(lq::launch_snapshot(a, n_blocks, save, static_cast<hipStream_t>(stream)));
}

}  // namespace

int leapquant_snapshot(const lq_dims* d, const lq_state* st, const int32_t* seq_ids, int32_t n_seq, void* snap,
                       void* stream) {
  return snapshot_call(d, st, seq_ids, n_seq, snap, true, stream);
}

int leapquant_restore(const lq_dims* d, const lq_state* st, const int32_t* seq_ids, int32_t n_seq,
                      const void* snap, void* stream) {
  return snapshot_call(d, st, seq_ids, n_seq, snap, false, stream);
}

int leapquant_dequantize(const lq_dims* d, const lq_state* st, float* S_out, void* stream) {
  int rc = check_dims(d, true);
  if (rc) return rc;
  if (empty(d)) return LQ_OK;
  if ((rc = check_state(d, st, 0))) return rc;
  if (!S_out) return LQ_ERR_NULL;
  if (!aligned(S_out, 16)) return LQ_ERR_ALIGN;
  return launched(lq::launch_dequantize(*d, *st, S_out, static_cast<hipStream_t>(stream)));
}

int32_t lq_close_list(const int32_t* win_len, const int32_t* win_off, int32_t batch, int64_t step,
                      int32_t* out_ids) {
  if (batch < 0 || step < 0) return LQ_ERR_CONFIG;
  if (batch == 0) return 0;
  if (!win_len || !win_off || !out_ids) return LQ_ERR_NULL;
  for (int32_t b = 0; b < batch; ++b)
    if (win_len[b] < 1 || win_off[b] < 0 || win_off[b] >= win_len[b]) return LQ_ERR_CONFIG;
  int32_t n = 0;
  for (int32_t b = 0; b < batch; ++b)
    if ((int64_t(win_off[b]) + step + 1) % int64_t(win_len[b]) == 0) out_ids[n++] = b;
  return n;
}

const char* lq_status_string(int status) {
  switch (status) {
    case LQ_OK: return "ok";
    case LQ_ERR_NULL: return "a required pointer is NULL";
    case LQ_ERR_SHAPE: return "unsupported shape (d_k == d_v in {32, 64, 128}, batch, heads >= 0)";
    case LQ_ERR_BITS: return "bits must be 4, 6 or 8";
    case LQ_ERR_CONFIG: return "parameter out of range (w_max, n_comp, power_iters, flags, token or close list)";
    case LQ_ERR_LAUNCH: return "HIP kernel launch failed";
    case LQ_ERR_ALIGN: return "buffer not aligned (16 bytes for state buffers and dense states)";
    default: return "unknown status";
  }
}

}  // extern "C"
