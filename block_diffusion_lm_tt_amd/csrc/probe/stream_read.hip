// Measurement probe, not part of the decoding path: plain HBM streaming reads, the ceiling the
// benchmark sets its kernels' bandwidth beside. Two forms over a grid-strided range:
//  - registers: every thread keeps eight 16-byte non-temporal loads in flight (consumed only
//    after all eight are issued) and folds what it read into one word per workgroup, so that
//    no load can be dropped;
//  - LDS-DMA: every wave copies 16-byte pieces straight into LDS (global_load_lds_dwordx4,
//    the attention kernel's way of streaming its context), eight per thread in flight.
// And the matrix cores' bf16 rate (v_mfma_f32_32x32x16_bf16 back to back, at the end).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int NTH = 256;
constexpr int U = 8;  // loads in flight per thread

__global__ __launch_bounds__(NTH) void stream_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                          uint32_t* __restrict__ sink) {
  __shared__ uint32_t red[NTH / 64];
  const size_t stride = (size_t)gridDim.x * NTH;
  size_t i = (size_t)blockIdx.x * NTH + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int k = 0; k < U; ++k) v[k] = __builtin_nontemporal_load(src + i + k * stride);
#pragma unroll
    for (int k = 0; k < U; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

__global__ __launch_bounds__(NTH) void stream_read_lds_kernel(const u32x4* __restrict__ src, size_t n16,
                                                              uint32_t* __restrict__ sink) {
  __shared__ u32x4 buf[U * NTH];  // 32 KB: stage k of wave w at buf[k * NTH + 64 w]
  const int w = threadIdx.x >> 6;
  const size_t stride = (size_t)gridDim.x * NTH;
  size_t i = (size_t)blockIdx.x * NTH + threadIdx.x;
  uint32_t acc = 0;
  // every lane of a wave takes the same trip count (the range end is checked for the wave's
  // last lane), so the copies are issued by whole waves
  const size_t wave_last = (size_t)blockIdx.x * NTH + 64 * w + 63;
  size_t j = wave_last;
  for (; j + (U - 1) * stride < n16; j += U * stride, i += U * stride) {
#pragma unroll
    for (int k = 0; k < U; ++k)
      __builtin_amdgcn_global_load_lds((const void*)(src + i + k * stride),
                                       (__attribute__((address_space(3))) void*)(&buf[k * NTH + 64 * w]), 16, 0,
                                       0);
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  __syncthreads();
  const u32x4 v = buf[threadIdx.x];
  acc ^= v.x ^ v.y ^ v.z ^ v.w;
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x] = acc;
}

}  // namespace

// The same read through LDS: pieces land in LDS by DMA and are not otherwise used.
extern "C" int ttprobe_stream_read_lds(const void* src, size_t bytes, uint32_t* sink, int blocks,
                                       hipStream_t stream) {
  if (!src || !sink || blocks < 1 || bytes % 16 != 0 || (uintptr_t)src % 16 != 0) return -1;
  hipLaunchKernelGGL(stream_read_lds_kernel, dim3(blocks), dim3(NTH), 0, stream, static_cast<const u32x4*>(src),
                     bytes / 16, sink);
  return (int)hipGetLastError();
}

// Reads `bytes` (a multiple of 16) from the device buffer `src` with `blocks` workgroups of 256
// threads on `stream`; `sink` (device, `blocks` words) receives one word per workgroup.
// Returns 0, or a hipError_t value on a launch failure, or -1 on bad arguments.
extern "C" int ttprobe_stream_read(const void* src, size_t bytes, uint32_t* sink, int blocks,
                                   hipStream_t stream) {
  if (!src || !sink || blocks < 1 || bytes % 16 != 0 || (uintptr_t)src % 16 != 0) return -1;
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(NTH), 0, stream, static_cast<const u32x4*>(src),
                     bytes / 16, sink);
  return (int)hipGetLastError();
}

// ---- matrix-core rate: v_mfma_f32_32x32x16_bf16 back to back -----------------------------
// Each wave runs four independent accumulation chains (so a product never waits for the
// previous one's result), `iters` rounds of four products, and writes one value so that no
// product can be dropped.
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void mfma_rate_kernel(int iters, float* sink) {
  bf16x8 a, b;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    a[k] = (__bf16)(0.001f * (threadIdx.x + k));
    b[k] = (__bf16)(0.002f * (threadIdx.x - k));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) s += c0[k] + c1[k] + c2[k] + c3[k];
  if (s == 12345.0f) sink[blockIdx.x] = s;  // practically never: keeps the products live
}

}  // namespace

// blocks workgroups of four waves (one per SIMD of a CU when blocks = 256 per CU count),
// each wave 4 * iters products of 32 x 32 x 16 (32768 flop each). Returns 0 or a HIP error.
extern "C" int ttprobe_mfma_rate(int blocks, int iters, float* sink, hipStream_t stream) {
  if (blocks < 1 || iters < 1 || !sink) return -1;
  hipLaunchKernelGGL(mfma_rate_kernel, dim3(blocks), dim3(256), 0, stream, iters, sink);
  return (int)hipGetLastError();
}
