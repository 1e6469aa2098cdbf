// Context cache update after a block is committed.
//
// What it computes: Nemotron-TwoTower (gist.science explainer), Technical Summary >
// Generation Process (once a block is committed, the context tower updates its states with
// the new clean tokens) and the snilld.dk TwoTower article, "Blockwise generering i
// praksis" (the context tower then updates its caches, once per block): the new key and
// value rows of one attention layer, [B, S, Hkv, D], are written at positions
// ctx_len[b] .. ctx_len[b]+S-1 of that layer's cache [B, Lmax, Hkv, D], and ctx_len[b]
// grows by S when asked (the last layer of a step). A sequence whose block does not fit is
// left as it is and flagged.
//
// How: per sequence the S new rows of a tensor are one contiguous run of S*Hkv*D elements,
// and so is their destination; one workgroup per sequence copies both runs with 16-byte
// accesses (4-byte ones when the run or a base is not 16-byte aligned), non-temporal, as
// the rows are not read again in this step. All threads read ctx_len[b] before the barrier
// after which one thread may bump it.
#include "tt_internal.h"

namespace tt {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int NT = 256;

template <typename V>
__device__ __forceinline__ void copy_run(const char* src, char* dst, size_t bytes) {
  const size_t n = bytes / sizeof(V);
  const V* s = reinterpret_cast<const V*>(src);
  V* d = reinterpret_cast<V*>(dst);
  for (size_t i = threadIdx.x; i < n; i += NT) __builtin_nontemporal_store(__builtin_nontemporal_load(s + i), d + i);
}

__global__ __launch_bounds__(NT) void ctx_append_kernel(AppendArgs a) {
  const int b = blockIdx.x;
  const int n = a.ctx_len[b];
  __syncthreads();  // every thread has read ctx_len[b] before it may change
  const bool fits = n >= 0 && (long long)n + a.S <= a.Lmax;
  if (threadIdx.x == 0 && a.skipped) a.skipped[b] = fits ? 0 : 1;
  if (!fits) return;
  const size_t run = (size_t)a.S * a.row_bytes;
  const size_t src = (size_t)b * run;
  const size_t dst = ((size_t)b * a.Lmax + n) * a.row_bytes;
  const char* kn = static_cast<const char*>(a.k_new);
  const char* vn = static_cast<const char*>(a.v_new);
  char* kc = static_cast<char*>(a.k_ctx);
  char* vc = static_cast<char*>(a.v_ctx);
  if (a.vec16) {
    copy_run<u32x4>(kn + src, kc + dst, run);
    copy_run<u32x4>(vn + src, vc + dst, run);
  } else if (a.elt == 4) {
    copy_run<uint32_t>(kn + src, kc + dst, run);
    copy_run<uint32_t>(vn + src, vc + dst, run);
  } else {
    copy_run<uint16_t>(kn + src, kc + dst, run);
    copy_run<uint16_t>(vn + src, vc + dst, run);
  }
  if (a.bump && threadIdx.x == 0) a.ctx_len[b] = n + a.S;
}

}  // namespace

hipError_t launch_ctx_append(const AppendArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(ctx_append_kernel, dim3(a.B), dim3(NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace tt
