// Prefix-cache snapshots of the LeapQuant state (gfx950). The state is
// compact at a window boundary (wink.run article, prefix caching and memory
// paragraphs; LeapQuant abstract): the buffer is empty, so a head is fully
// described by its codes, its two scale vectors and its r compensators.
// Snapshot and restore copy exactly that, one workgroup per head, in 16-byte
// pieces, with non-temporal loads and stores (each byte is moved once).
//
// Record of one head, in this order (bytes): codes D*D*bits/8, row scales 4D,
// column scales 4D, compensator keys 4rD, compensator values 4rD. Every
// piece is a multiple of 16 bytes for the supported shapes.
#include "lq_common.h"
#include "lq_launch.h"

namespace lq {

namespace {

__device__ __forceinline__ void copy16(const void* src, void* dst, size_t bytes) {
  typedef unsigned int u4 __attribute__((ext_vector_type(4)));
  const u4* s = static_cast<const u4*>(src);
  u4* d = static_cast<u4*>(dst);
  for (size_t i = threadIdx.x; i < bytes / 16; i += blockDim.x)
    __builtin_nontemporal_store(__builtin_nontemporal_load(s + i), d + i);
}

template <bool SAVE>
__global__ void __launch_bounds__(256) snapshot_kernel(SnapshotArgs a) {
  const int H = a.heads, D = a.d, r = a.r;
  int b = blockIdx.x / H;
  const int h = blockIdx.x % H;
  const int slot = b;  // record index of this sequence in the snapshot
  if (a.seq_ids) b = a.seq_ids[b];
  if (b < 0 || b >= a.batch) {
    if (threadIdx.x == 0 && a.err) atomicOr(a.err, LQ_DEVERR_BAD_SEQ);
    return;
  }
  const size_t bh = size_t(b) * H + h;
  const size_t code_bytes = size_t(D) * D * a.bits / 8;
  const size_t vec = size_t(D) * 4, comp = size_t(r) * D * 4;
  const size_t ne = size_t(r) + a.w_max;  // entries per head
  uint8_t* rec = static_cast<uint8_t*>(a.snap) + (size_t(slot) * H + h) * a.record_bytes;
  uint8_t* codes = static_cast<uint8_t*>(a.codes) + bh * code_bytes;
  uint8_t* s = reinterpret_cast<uint8_t*>(a.s + bh * D);
  uint8_t* c = reinterpret_cast<uint8_t*>(a.c + bh * D);
  uint8_t* ek = reinterpret_cast<uint8_t*>(a.ek + bh * ne * D);
  uint8_t* eu = reinterpret_cast<uint8_t*>(a.eu + bh * ne * D);
  if constexpr (SAVE) {
    const int n = __builtin_amdgcn_readfirstlane(a.blen[bh]);
    if (n != 0) {  // not at a window boundary: nothing is written for this head
      if (threadIdx.x == 0 && a.err) atomicOr(a.err, LQ_DEVERR_BAD_LEN);
      return;
    }
    copy16(codes, rec, code_bytes);
    copy16(s, rec + code_bytes, vec);
    copy16(c, rec + code_bytes + vec, vec);
    copy16(ek, rec + code_bytes + 2 * vec, comp);
    copy16(eu, rec + code_bytes + 2 * vec + comp, comp);
  } else {
    copy16(rec, codes, code_bytes);
    copy16(rec + code_bytes, s, vec);
    copy16(rec + code_bytes + vec, c, vec);
    copy16(rec + code_bytes + 2 * vec, ek, comp);
    copy16(rec + code_bytes + 2 * vec + comp, eu, comp);
    // compensators sit at window position 0 (G = 0); the buffer starts empty
    const size_t gl = a.kda ? size_t(D) : 1;
    for (size_t i = threadIdx.x; i < size_t(r) * gl; i += blockDim.x) a.eg[bh * ne * gl + i] = 0.f;
    if (threadIdx.x == 0) a.blen[bh] = 0;
  }
}

}  // namespace

hipError_t launch_snapshot(const SnapshotArgs& a, int n_blocks, bool save, hipStream_t stream) {
  if (save) hipLaunchKernelGGL((snapshot_kernel<true>), dim3(n_blocks), dim3(256), 0, stream, a);
  else hipLaunchKernelGGL((snapshot_kernel<false>), dim3(n_blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace lq
