// adaLN-single time modulation of one denoiser layer.
//
// What it computes: Nemotron-TwoTower (gist.science explainer), Technical Summary > Training
// and Conditioning > Time Conditioning (the denoiser is conditioned on the diffusion timestep
// through adaptive layer normalization) and the snilld.dk TwoTower article, "Hvad TwoTower
// aendrer teknisk" (every layer is time-modulated by a small adaLN-single block). One shared
// set of vectors per sequence (shift, scale, gate) = t_mod[b], plus the layer's own offsets
// table = (shift, scale, gate):
//   adaln_modulate:  y = LN(x) * (1 + scale) + shift     (LN: no affine terms, eps inside
//                                                           the root), before the mixer
//   adaln_gate:      out = x + gate * f                   (the mixer's output f joins the
//                                                           residual stream)
//
// How: both are HBM-bound row passes. The modulation takes one workgroup of 256 threads per
// row: each thread holds its share of the row in registers (16-byte pieces, consecutive
// pieces on consecutive threads, when the row width is a multiple of a piece and every base
// is 16-byte aligned; else single elements strided by 256), the mean and then the variance of
// the deviations are reduced in fp32 (wave shuffles, then LDS), and the modulated row is
// written once. The gated residual is element-wise, one thread per 16-byte piece (or per
// element).
#include "tt_internal.h"

namespace tt {
namespace {

constexpr int NT = 256;

template <typename T> __device__ __forceinline__ float ldf(const T* p, size_t i);
template <> __device__ __forceinline__ float ldf<float>(const float* p, size_t i) { return p[i]; }
template <> __device__ __forceinline__ float ldf<uint16_t>(const uint16_t* p, size_t i) {
  return __uint_as_float(((uint32_t)p[i]) << 16);
}
template <typename T> __device__ __forceinline__ void stf(T* p, size_t i, float v);
template <> __device__ __forceinline__ void stf<float>(float* p, size_t i, float v) { p[i] = v; }
template <> __device__ __forceinline__ void stf<uint16_t>(uint16_t* p, size_t i, float v) {
  p[i] = __builtin_bit_cast(uint16_t, (__bf16)v);
}

__device__ __forceinline__ float block_sum(float v, float* red) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// J: elements per thread (d <= 256 J)
template <typename T, int J>
__global__ __launch_bounds__(NT) void adaln_modulate_kernel(AdalnArgs a) {
  __shared__ float red[4];
  const int row = blockIdx.x, tid = threadIdx.x;
  const int b = row / a.S;
  const T* x = static_cast<const T*>(a.x) + (size_t)row * a.d;
  float v[J];
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int k = tid + j * NT;
    v[j] = k < a.d ? ldf(x, k) : 0.0f;
    s += v[j];
  }
  const float mean = block_sum(s, red) / (float)a.d;
  float q = 0.0f;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int k = tid + j * NT;
    const float e = k < a.d ? v[j] - mean : 0.0f;
    q = fmaf(e, e, q);
  }
  const float var = block_sum(q, red) / (float)a.d;
  const float rstd = 1.0f / sqrtf(var + a.eps);
  const float* tm = a.t_mod + (size_t)b * 3 * a.d;
  T* y = static_cast<T*>(a.y) + (size_t)row * a.d;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int k = tid + j * NT;
    if (k < a.d) {
      const float shift = tm[k] + a.table[k];
      const float scale = tm[a.d + k] + a.table[a.d + k];
      stf(y, k, fmaf((v[j] - mean) * rstd, 1.0f + scale, shift));
    }
  }
}

template <typename T>
__global__ __launch_bounds__(NT) void adaln_gate_kernel(AdalnArgs a) {
  const size_t i = (size_t)blockIdx.x * NT + threadIdx.x;
  const size_t n = (size_t)a.B * a.S * a.d;
  if (i >= n) return;
  const size_t row = i / a.d;
  const int k = (int)(i - row * a.d);
  const int b = (int)(row / a.S);
  const float gate = a.t_mod[((size_t)b * 3 + 2) * a.d + k] + a.table[2 * a.d + k];
  const float r = fmaf(gate, ldf(static_cast<const T*>(a.f), i), ldf(static_cast<const T*>(a.x), i));
  stf(static_cast<T*>(a.y), i, r);
}

// 16-byte pieces: VE elements of T
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
template <typename T> struct Piece { static constexpr int VE = 16 / sizeof(T); };

template <typename T>
__device__ __forceinline__ void unpack(const u32x4& r, float (&v)[Piece<T>::VE]);
template <>
__device__ __forceinline__ void unpack<uint16_t>(const u32x4& r, float (&v)[8]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    v[2 * k] = __uint_as_float(r[k] << 16);
    v[2 * k + 1] = __uint_as_float(r[k] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void unpack<float>(const u32x4& r, float (&v)[4]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) v[k] = __uint_as_float(r[k]);
}
template <typename T>
__device__ __forceinline__ u32x4 pack(const float (&v)[Piece<T>::VE]);
template <>
__device__ __forceinline__ u32x4 pack<uint16_t>(const float (&v)[8]) {
  u32x4 r;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t lo = __builtin_bit_cast(uint16_t, (__bf16)v[2 * k]);
    const uint32_t hi = __builtin_bit_cast(uint16_t, (__bf16)v[2 * k + 1]);
    r[k] = lo | (hi << 16);
  }
  return r;
}
template <>
__device__ __forceinline__ u32x4 pack<float>(const float (&v)[4]) {
  u32x4 r;
#pragma unroll
  for (int k = 0; k < 4; ++k) r[k] = __float_as_uint(v[k]);
  return r;
}

// JP: pieces per thread (d <= 256 JP VE)
template <typename T, int JP>
__global__ __launch_bounds__(NT) void adaln_modulate_vec_kernel(AdalnArgs a) {
  constexpr int VE = Piece<T>::VE;
  __shared__ float red[4];
  const int row = blockIdx.x, tid = threadIdx.x;
  const int b = row / a.S;
  const int np = a.d / VE;  // pieces per row
  const u32x4* x = reinterpret_cast<const u32x4*>(static_cast<const T*>(a.x) + (size_t)row * a.d);
  float v[JP][VE];
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < JP; ++j) {
    const int c = tid + j * NT;
    if (c < np) {
      unpack<T>(x[c], v[j]);
    } else {
#pragma unroll
      for (int k = 0; k < VE; ++k) v[j][k] = 0.0f;
    }
#pragma unroll
    for (int k = 0; k < VE; ++k) s += v[j][k];
  }
  const float mean = block_sum(s, red) / (float)a.d;
  float q = 0.0f;
#pragma unroll
  for (int j = 0; j < JP; ++j) {
    if (tid + j * NT < np) {
#pragma unroll
      for (int k = 0; k < VE; ++k) {
        const float e = v[j][k] - mean;
        q = fmaf(e, e, q);
      }
    }
  }
  const float var = block_sum(q, red) / (float)a.d;
  const float rstd = 1.0f / sqrtf(var + a.eps);
  const float* tm = a.t_mod + (size_t)b * 3 * a.d;
  u32x4* y = reinterpret_cast<u32x4*>(static_cast<T*>(a.y) + (size_t)row * a.d);
#pragma unroll
  for (int j = 0; j < JP; ++j) {
    const int c = tid + j * NT;
    if (c < np) {
      float o[VE];
#pragma unroll
      for (int k = 0; k < VE; ++k) {
        const int e = c * VE + k;
        const float shift = tm[e] + a.table[e];
        const float scale = tm[a.d + e] + a.table[a.d + e];
        o[k] = fmaf((v[j][k] - mean) * rstd, 1.0f + scale, shift);
      }
      y[c] = pack<T>(o);
    }
  }
}

template <typename T>
__global__ __launch_bounds__(NT) void adaln_gate_vec_kernel(AdalnArgs a) {
  constexpr int VE = Piece<T>::VE;
  const size_t i = (size_t)blockIdx.x * NT + threadIdx.x;  // piece
  const size_t n = (size_t)a.B * a.S * a.d / VE;
  if (i >= n) return;
  const size_t e0 = i * VE;
  const size_t row = e0 / a.d;
  const int k0 = (int)(e0 - row * a.d);
  const int b = (int)(row / a.S);
  float xv[VE], fv[VE], o[VE];
  unpack<T>(reinterpret_cast<const u32x4*>(a.x)[i], xv);
  unpack<T>(reinterpret_cast<const u32x4*>(a.f)[i], fv);
  const float* g = a.t_mod + ((size_t)b * 3 + 2) * a.d + k0;
  const float* gt = a.table + 2 * a.d + k0;
#pragma unroll
  for (int k = 0; k < VE; ++k) o[k] = fmaf(g[k] + gt[k], fv[k], xv[k]);
  reinterpret_cast<u32x4*>(a.y)[i] = pack<T>(o);
}

template <typename T>
bool vec_ok(const AdalnArgs& a, bool with_f) {
  constexpr int VE = Piece<T>::VE;
  uintptr_t bases = (uintptr_t)a.x | (uintptr_t)a.y | (uintptr_t)a.t_mod | (uintptr_t)a.table;
  if (with_f) bases |= (uintptr_t)a.f;
  return a.d % VE == 0 && bases % 16 == 0;
}

template <typename T>
hipError_t modulate_t(const AdalnArgs& a, hipStream_t s) {
  constexpr int VE = Piece<T>::VE;
  if (vec_ok<T>(a, false)) {
    const int JP = (a.d / VE + NT - 1) / NT;
    const dim3 grid(a.B * a.S), block(NT);
    if (JP <= 1) hipLaunchKernelGGL((adaln_modulate_vec_kernel<T, 1>), grid, block, 0, s, a);
    else if (JP <= 2) hipLaunchKernelGGL((adaln_modulate_vec_kernel<T, 2>), grid, block, 0, s, a);
    else if (JP <= 4) hipLaunchKernelGGL((adaln_modulate_vec_kernel<T, 4>), grid, block, 0, s, a);
    else if (JP <= 8) hipLaunchKernelGGL((adaln_modulate_vec_kernel<T, 8>), grid, block, 0, s, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
  }
  const int J = (a.d + NT - 1) / NT;
  const dim3 grid(a.B * a.S), block(NT);
  if (J <= 4) hipLaunchKernelGGL((adaln_modulate_kernel<T, 4>), grid, block, 0, s, a);
  else if (J <= 8) hipLaunchKernelGGL((adaln_modulate_kernel<T, 8>), grid, block, 0, s, a);
  else if (J <= 16) hipLaunchKernelGGL((adaln_modulate_kernel<T, 16>), grid, block, 0, s, a);
  else if (J <= 32) hipLaunchKernelGGL((adaln_modulate_kernel<T, 32>), grid, block, 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

hipError_t launch_adaln_modulate(const AdalnArgs& a, int dtype, hipStream_t s) {
  return dtype == TT_BF16 ? modulate_t<uint16_t>(a, s) : modulate_t<float>(a, s);
}

hipError_t launch_adaln_gate(const AdalnArgs& a, int dtype, hipStream_t s) {
  const size_t n = (size_t)a.B * a.S * a.d;
  if (dtype == TT_BF16 ? vec_ok<uint16_t>(a, true) : vec_ok<float>(a, true)) {
    const size_t np = n / (dtype == TT_BF16 ? 8 : 4);
    const dim3 grid((unsigned)((np + NT - 1) / NT)), block(NT);
    if (dtype == TT_BF16)
      hipLaunchKernelGGL(adaln_gate_vec_kernel<uint16_t>, grid, block, 0, s, a);
    else
      hipLaunchKernelGGL(adaln_gate_vec_kernel<float>, grid, block, 0, s, a);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((n + NT - 1) / NT)), block(NT);
  if (dtype == TT_BF16)
    hipLaunchKernelGGL(adaln_gate_kernel<uint16_t>, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(adaln_gate_kernel<float>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace tt
