// Host-side kernel launchers (internal). Arguments are already validated by
// the C ABI layer; each launcher enqueues on `stream` and returns hipError_t
// of the launch.
#pragma once

#include <hip/hip_runtime.h>

#include "leapquant.h"

namespace lq {

// Kernel-side view of the state plus the per-call activations.
struct StepArgs {
  const void* codes;
  const float* s;
  const float* c;
  float* ek;  // entry keys   [BH][r + w_max][D]
  float* eu;  // entry values [BH][r + w_max][D]
  float* eg;  // entry G      [BH][r + w_max] or [BH][r + w_max][D]
  int32_t* blen;
  int32_t* err;
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  float* o;
  int r;
  int w_max;
  int n_at;  // -1: read each head's buffer length; >= 0: every head holds n_at tokens
};

struct CloseArgs {
  const float* S;          // dense input (encode) or NULL (close)
  void* codes;
  float* s;
  float* c;
  float* ek;
  float* eu;
  float* eg;
  int32_t* blen;
  int32_t* err;
  const int32_t* seq_ids;  // NULL: all sequences
  float* dbg;              // NULL or residual output
  int batch;
  int heads;
  int r;
  int w_max;
  int T;
  int smoothing;
  int warm;                // start compensator l from the current entry l's value (close only)
  // one decode token taken first (NULL q: none): every head holds n_at tokens
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  float* o;
  int n_at;
};

struct BaselineArgs {
  float* S;
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  float* o;
};

struct PrefillArgs {
  float* S;  // [BH][D][D] fp32, value-column major (in/out)
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  float* o;
  int n_tokens;
  int n_heads;
};

struct SnapshotArgs {
  void* codes;
  float* s;
  float* c;
  float* ek;
  float* eu;
  float* eg;
  int32_t* blen;
  int32_t* err;
  const int32_t* seq_ids;  // NULL: all sequences
  void* snap;              // [n_seq][heads][record_bytes]
  size_t record_bytes;
  int batch;
  int heads;
  int d;
  int r;
  int w_max;
  int bits;
  int kda;
};

hipError_t launch_snapshot(const SnapshotArgs& a, int n_blocks, bool save, hipStream_t stream);
hipError_t launch_prefill(const lq_dims& d, const PrefillArgs& a, hipStream_t stream);
hipError_t launch_decode_step(const lq_dims& d, const StepArgs& a, hipStream_t stream);
hipError_t launch_close(const lq_dims& d, const CloseArgs& a, int n_blocks, hipStream_t stream);
hipError_t launch_baseline(const lq_dims& d, const BaselineArgs& a, hipStream_t stream);
hipError_t launch_dequantize(const lq_dims& d, const lq_state& st, float* out, hipStream_t stream);

}  // namespace lq
