// The denoiser's Mamba-2 layer over one block, started from the state seeded by the context
// tower.
//
// What it computes: snilld.dk TwoTower article, "Hvad TwoTower aendrer teknisk" (the
// denoiser's Mamba-2 states are seeded directly from the context tower) and Nemotron-TwoTower
// (gist.science explainer), Technical Summary > Methodology > Architecture (the context tower
// produces layer-aligned KV caches and Mamba states) and ablations (Mamba stays causal). Per
// sequence b and head h, the Mamba-2 selective state-space recurrence over the block's S
// positions, from the seeded state h0[b,h] (P x N):
//   delta_t = softplus(dt + dt_bias[h]),  a_t = exp(-exp(A_log[h]) delta_t)
//   state_t = a_t state_{t-1} + delta_t x_t B_t^T,   y_t = state_t C_t + D[h] x_t
// and, when asked, the state after the block (the context tower's own state update over a
// committed block is the same computation).
//
// How: one workgroup of 256 threads per (sequence, head). The seeded state (P x N fp32) is the
// stream that bounds the kernel: each thread loads its P x N / 256 share (one row p, a run of
// N / (256 / P) columns) with 16-byte loads issued first, while the block's B, C, x and step
// sizes are staged in LDS. The recurrence is evaluated in its unrolled (chunked) form, chunks
// of up to 16 positions: with L_t the cumulative log decay inside the chunk,
//   y_t = e^{L_t} (state C_t) + sum_{s<=t} e^{L_t - L_s} delta_s (C_t . B_s) x_s + D x_t,
//   state' = e^{L_last} state + sum_s e^{L_last - L_s} delta_s x_s B_s^T
// The readout state C_t is the bulk of the arithmetic (P x N x chunk FMAs, fp32 VALU); the
// within-chunk matrix M_ts = e^{L_t - L_s} delta_s (C_t . B_s) is computed once per chunk and
// shared by the P rows; the state update runs only between chunks or for the returned state.
#include "tt_internal.h"

namespace tt {
namespace {

constexpr int NT = 256;
constexpr int CH = kMambaChunk;   // positions per chunk (16)

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

__device__ __forceinline__ float softplus(float z) { return z > 20.0f ? z : log1pf(expf(z)); }

// NPT: state columns per thread (N / (256 / P)), a compile-time bound on the registers
template <typename T, int NPT>
__global__ __launch_bounds__(NT) void mamba2_scan_kernel(MambaArgs a) {
  __shared__ float sC[CH][kMambaMaxN];
  __shared__ float sB[CH][kMambaMaxN];
  __shared__ float sX[CH][kMambaMaxP];
  __shared__ float sM[CH][CH];
  __shared__ float sL[CH], sDelta[CH];
  const int tid = threadIdx.x;
  const int bh = blockIdx.x;
  const int b = bh / a.H, h = bh - b * a.H;
  const int g = h / (a.H / a.G);
  const int tpr = NT / a.P;            // threads per state row (a power of 2, <= 64)
  const int p = tid / tpr, nq = tid - p * tpr;
  const int n0 = nq * NPT;             // this thread's columns [n0, n0 + NPT)
  const bool active = p < a.P;         // (every thread is a row's when P divides 256)

  // the seeded state: this thread's run of one row, 16-byte loads first
  float st[NPT];
  const float* h0 = a.h0 + ((size_t)b * a.H + h) * a.P * a.N + (size_t)p * a.N + n0;
  if (active) {
#pragma unroll
    for (int k = 0; k < NPT; k += 4) {
      const float4 v = *reinterpret_cast<const float4*>(h0 + k);
      st[k] = v.x;
      st[k + 1] = v.y;
      st[k + 2] = v.z;
      st[k + 3] = v.w;
    }
  }
  const float A = -expf(a.A_log[h]);
  const float bias = a.dt_bias[h];
  const float Dh = a.Dskip[h];
  const T* X = static_cast<const T*>(a.x);
  const T* Bm = static_cast<const T*>(a.Bm);
  const T* Cm = static_cast<const T*>(a.Cm);
  T* Y = static_cast<T*>(a.y);

  for (int t0 = 0; t0 < a.S; t0 += CH) {
    const int lc = min(CH, a.S - t0);
    __syncthreads();  // the previous chunk's LDS reads are done
    // stage the chunk: B, C (group g), x (head h), step sizes and cumulative log decay
    for (int i = tid; i < lc * a.N; i += NT) {
      const int t = i / a.N, n = i - t * a.N;
      const size_t o = (((size_t)b * a.S + t0 + t) * a.G + g) * a.N + n;
      sB[t][n] = ldf(Bm, o);
      sC[t][n] = ldf(Cm, o);
    }
    for (int i = tid; i < lc * a.P; i += NT) {
      const int t = i / a.P, q = i - t * a.P;
      sX[t][q] = ldf(X, (((size_t)b * a.S + t0 + t) * a.H + h) * a.P + q);
    }
    if (tid < 64) {
      const float d = tid < lc ? softplus(a.dt[((size_t)b * a.S + t0 + tid) * a.H + h] + bias) : 0.0f;
      float l = d * A;  // inclusive prefix sum over the chunk (a wave scan)
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(l, off, 64);
        if (tid >= off) l += y;
      }
      if (tid < lc) {
        sDelta[tid] = d;
        sL[tid] = l;
      }
    }
    __syncthreads();
    // the within-chunk matrix, s <= t
    for (int i = tid; i < lc * lc; i += NT) {
      const int t = i / lc, s = i - t * lc;
      float m = 0.0f;
      if (s <= t) {
        float cb = 0.0f;
        for (int n = 0; n < a.N; ++n) cb = fmaf(sC[t][n], sB[s][n], cb);
        m = expf(sL[t] - sL[s]) * sDelta[s] * cb;
      }
      sM[t][s] = m;
    }
    // the readout of the state carried into the chunk: this thread's partial of state C_t
    float yr[CH];
#pragma unroll
    for (int t = 0; t < CH; ++t) {
      float acc = 0.0f;
      if (t < lc) {
#pragma unroll
        for (int k = 0; k < NPT; ++k) acc = fmaf(st[k], sC[t][n0 + k], acc);
      }
      yr[t] = acc;
    }
    // the row's partials meet across its tpr threads (consecutive lanes)
    for (int off = 1; off < tpr; off <<= 1)
#pragma unroll
      for (int t = 0; t < CH; ++t) yr[t] += __shfl_xor(yr[t], off, 64);
    __syncthreads();  // sM complete
    // outputs: thread nq of a row writes the positions t = nq, nq + tpr, ...
    if (active) {
#pragma unroll
      for (int t = 0; t < CH; ++t) {
        if (t >= lc || (t % tpr) != nq) continue;
        float v = expf(sL[t]) * yr[t] + Dh * sX[t][p];
        for (int s = 0; s <= t; ++s) v = fmaf(sM[t][s], sX[s][p], v);
        stf(Y, (((size_t)b * a.S + t0 + t) * a.H + h) * a.P + p, v);
      }
    }
    // the state after the chunk, when another chunk follows or the caller wants it
    if (t0 + lc < a.S || a.h_out) {
      const float last = sL[lc - 1];
      const float keep = expf(last);
#pragma unroll
      for (int k = 0; k < NPT; ++k) st[k] *= keep;
      for (int s = 0; s < lc; ++s) {
        const float w = expf(last - sL[s]) * sDelta[s] * sX[s][p];
#pragma unroll
        for (int k = 0; k < NPT; ++k) st[k] = fmaf(w, sB[s][n0 + k], st[k]);
      }
    }
  }
  if (a.h_out && active) {
    float* ho = a.h_out + ((size_t)b * a.H + h) * a.P * a.N + (size_t)p * a.N + n0;
#pragma unroll
    for (int k = 0; k < NPT; k += 4) *reinterpret_cast<float4*>(ho + k) = float4{st[k], st[k + 1], st[k + 2], st[k + 3]};
  }
}

template <typename T>
hipError_t launch_t(const MambaArgs& a, hipStream_t s) {
  const int npt = a.N / (NT / a.P);
  dim3 grid(a.B * a.H), block(NT);
  switch (npt) {
    case 4: hipLaunchKernelGGL((mamba2_scan_kernel<T, 4>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((mamba2_scan_kernel<T, 8>), grid, block, 0, s, a); break;
    case 16: hipLaunchKernelGGL((mamba2_scan_kernel<T, 16>), grid, block, 0, s, a); break;
    case 32: hipLaunchKernelGGL((mamba2_scan_kernel<T, 32>), grid, block, 0, s, a); break;
    case 64: hipLaunchKernelGGL((mamba2_scan_kernel<T, 64>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool mamba_shape_supported(int P, int N) {
  if (P < 4 || P > kMambaMaxP || (P & (P - 1)) != 0) return false;  // 256 / P threads per row
  if (N > kMambaMaxN) return false;
  const int tpr = 256 / P;
  if (N % tpr != 0) return false;
  const int npt = N / tpr;
  return npt == 4 || npt == 8 || npt == 16 || npt == 32 || npt == 64;
}

hipError_t launch_mamba2_scan(const MambaArgs& a, int dtype, hipStream_t s) {
  return dtype == TT_BF16 ? launch_t<uint16_t>(a, s) : launch_t<float>(a, s);
}

}  // namespace tt
