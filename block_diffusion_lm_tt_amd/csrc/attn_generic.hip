// Denoiser block attention for the shapes the MFMA kernel does not take: fp32 inputs, or
// a head dim other than 128. Same definition (Nemotron-TwoTower, gist.science explainer,
// Technical Summary > Generation Process): one softmax over [context keys ; block keys],
// no mask inside the block, scale 1/sqrt(D), query head h reads KV head h / G.
//
// One workgroup of 256 threads per query row (b, i, h). Keys are visited in slices of
// 256 (one key per thread: fp32 dot product over D), the slice's weights go through LDS,
// and thread d < D accumulates the value column d with an fp32 online softmax. Accurate
// expf throughout; this path is about coverage, not speed.
#include "tt_internal.h"

namespace tt {
namespace {

constexpr int NT = 256;

template <typename T>
__device__ __forceinline__ float ld(const T* p, size_t i);
template <>
__device__ __forceinline__ float ld<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t* p, size_t i) {
  return __uint_as_float(((uint32_t)p[i]) << 16);
}

template <typename T>
__device__ __forceinline__ void st(T* p, size_t i, float v);
template <>
__device__ __forceinline__ void st<float>(float* p, size_t i, float v) { p[i] = v; }
template <>
__device__ __forceinline__ void st<uint16_t>(uint16_t* p, size_t i, float v) {
  p[i] = __builtin_bit_cast(uint16_t, (__bf16)v);
}

__device__ __forceinline__ float block_max(float v, float* red) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const float r = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return r;
}

__device__ __forceinline__ float block_sum(float v, float* red) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const float r = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return r;
}

template <typename T>
__global__ __launch_bounds__(NT) void attn_generic_kernel(AttnArgs a) {
  __shared__ float qs[256];
  __shared__ float ps[NT];
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const int row = blockIdx.x;  // ((b*S + i)*Hq + h)
  const int h = row % a.Hq;
  const int bi = row / a.Hq;
  const int b = bi / a.S;
  const int g = h / a.G;
  const int D = a.D;
  const T* q = static_cast<const T*>(a.q);
  const T* kc = static_cast<const T*>(a.k_ctx);
  const T* vc = static_cast<const T*>(a.v_ctx);
  const T* kb = static_cast<const T*>(a.k_blk);
  const T* vb = static_cast<const T*>(a.v_blk);
  int nctx = a.ctx_len[b];
  nctx = nctx < 0 ? 0 : (nctx > a.Lmax ? a.Lmax : nctx);
  const int n = nctx + a.S;
  const float scale = 1.0f / sqrtf((float)D);
  for (int d = tid; d < D; d += NT) qs[d] = ld(q, (size_t)row * D + d);
  __syncthreads();

  float m = -INFINITY, l = 0.0f, acc = 0.0f;
  for (int j0 = 0; j0 < n; j0 += NT) {
    const int j = j0 + tid;
    float s = -INFINITY;
    if (j < n) {
      const T* kp;
      size_t off;
      if (j < nctx) {
        kp = kc;
        off = (((size_t)b * a.Lmax + j) * a.Hkv + g) * D;
      } else {
        kp = kb;
        off = (((size_t)b * a.S + (j - nctx)) * a.Hkv + g) * D;
      }
      float dot = 0.0f;
      for (int d = 0; d < D; ++d) dot = fmaf(qs[d], ld(kp, off + d), dot);
      s = dot * scale;
    }
    const float mn = fmaxf(m, block_max(s, red));
    const float alpha = expf(m - mn);  // m = -inf on the first slice -> 0
    const float p = (j < n) ? expf(s - mn) : 0.0f;
    ps[tid] = p;
    const float psum = block_sum(p, red);  // also orders the ps[] writes before the reads
    l = l * alpha + psum;
    m = mn;
    if (tid < D) {
      float part = 0.0f;
      const int cnt = min(NT, n - j0);
      for (int jj = 0; jj < cnt; ++jj) {
        const int jk = j0 + jj;
        const T* vp;
        size_t off;
        if (jk < nctx) {
          vp = vc;
          off = (((size_t)b * a.Lmax + jk) * a.Hkv + g) * D;
        } else {
          vp = vb;
          off = (((size_t)b * a.S + (jk - nctx)) * a.Hkv + g) * D;
        }
        part = fmaf(ps[jj], ld(vp, off + tid), part);
      }
      acc = acc * alpha + part;
    }
    __syncthreads();  // ps[] is rewritten by the next slice
  }
  if (tid < D) st(static_cast<T*>(a.o), (size_t)row * D + tid, acc / l);
}

}  // namespace

hipError_t launch_attn_generic(const AttnArgs& a, int dtype, hipStream_t s) {
  const int rows = a.B * a.S * a.Hq;
  if (dtype == TT_F32)
    hipLaunchKernelGGL(attn_generic_kernel<float>, dim3(rows), dim3(NT), 0, s, a);
  else
    hipLaunchKernelGGL(attn_generic_kernel<uint16_t>, dim3(rows), dim3(NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace tt
