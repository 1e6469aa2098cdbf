// Confidence-threshold commit (confidence unmasking) of one denoising step.
//
// What it computes: Nemotron-TwoTower (gist.science explainer), Technical Summary >
// Training and Conditioning > Sampling, and the snilld.dk TwoTower article, "Blockwise
// generering i praksis". For each masked position: token = lowest index of the row max,
// Z = sum_v exp(l_v - max), conf = 1/Z, committed = conf > gamma; a sequence with masked
// positions and no commit commits its most confident masked position (lowest i on ties).
//
// How: the work is one pass over the masked rows' logits, so it is HBM bound.
//  1. commit_reduce: one workgroup per (masked row, 8192-element vocabulary chunk). Each
//     thread loads its 32 (bf16) or 16 (fp32) elements with 16-byte loads, keeps them in
//     registers, finds its max and lowest argmax, and the workgroup merges them (wave
//     shuffles + LDS, lowest index on ties). A second pass over the registers sums
//     exp2((x - max) * log2 e) in fp32 per thread and in fp64 across threads.
//  2. commit_merge: one workgroup per sequence merges the chunks in fp64, estimates Z and
//     takes every decision whose margin is safe. The estimate's relative error is below
//     1e-5 (fp32 exp2 of an exactly formed difference, <= 32 terms per fp32 partial), so a
//     decision is taken only outside a relative band of 1e-4 around the threshold, and
//     fallback candidates are all positions within 4e-4 of the best estimate. Positions in
//     a band are flagged.
//  3. commit_recheck: flagged rows only -- Z recomputed over the full row with fp64 exp.
//  4. commit_finalize: sequences with flagged rows decide with the fp64 values (conf =
//     1/Z > gamma, evaluated in fp64 as in exact arithmetic) and apply the fallback.
#include "tt_internal.h"

namespace tt {
namespace {

constexpr int NT = 256;
constexpr int LOADS = 4;  // 16-byte loads per thread per chunk
constexpr float kLog2e = 1.4426950408889634f;
constexpr double kBand = 1e-4;       // threshold band (relative)
constexpr double kFallBand = 4e-4;   // fallback candidate band (relative)

template <typename T> struct Vec;
template <> struct Vec<uint16_t> { static constexpr int N = 8; };
template <> struct Vec<float> { static constexpr int N = 4; };

__device__ __forceinline__ float to_f(uint16_t x) { return __uint_as_float(((uint32_t)x) << 16); }
__device__ __forceinline__ float to_f(float x) { return x; }

// (m, tok) merge: larger value wins, equal values -> lower index
__device__ __forceinline__ void argmax_merge(float& m, int& tok, float m2, int tok2) {
  if (m2 > m || (m2 == m && tok2 < tok)) {
    m = m2;
    tok = tok2;
  }
}

template <typename T>
__global__ __launch_bounds__(NT) void commit_reduce_kernel(CommitArgs a) {
  constexpr int VE = Vec<T>::N;
  constexpr int EPT = VE * LOADS;
  __shared__ float sm_m[4];
  __shared__ int sm_t[4];
  __shared__ double sm_z[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const long long blk = blockIdx.x;
  const int row = (int)(blk / a.n_chunks);
  const int ch = (int)(blk - (long long)row * a.n_chunks);
  if (!a.mask[row]) return;
  const T* base = static_cast<const T*>(a.logits) + (size_t)row * a.V;
  const int begin = ch * a.chunk_elems;
  const int end = min(a.V, begin + a.chunk_elems);

  float x[EPT];
#pragma unroll
  for (int ld = 0; ld < LOADS; ++ld) {
    const int i0 = begin + (ld * NT + tid) * VE;
    const T* p = base + i0;
    if (i0 + VE <= end && ((reinterpret_cast<uintptr_t>(p) & 15) == 0)) {
      const uint4 v = *reinterpret_cast<const uint4*>(p);
      const T* e = reinterpret_cast<const T*>(&v);
#pragma unroll
      for (int k = 0; k < VE; ++k) x[ld * VE + k] = to_f(e[k]);
    } else {
#pragma unroll
      for (int k = 0; k < VE; ++k) x[ld * VE + k] = (i0 + k < end) ? to_f(p[k]) : -INFINITY;
    }
  }
  // thread max / lowest argmax (elements are visited in increasing index order)
  float m = -INFINITY;
  int tok = 0x7fffffff;
#pragma unroll
  for (int ld = 0; ld < LOADS; ++ld)
#pragma unroll
    for (int k = 0; k < VE; ++k) {
      const float v = x[ld * VE + k];
      if (v > m) {
        m = v;
        tok = begin + (ld * NT + tid) * VE + k;
      }
    }
  for (int off = 32; off > 0; off >>= 1) {
    const float m2 = __shfl_xor(m, off, 64);
    const int t2 = __shfl_xor(tok, off, 64);
    argmax_merge(m, tok, m2, t2);
  }
  if (lane == 0) {
    sm_m[w] = m;
    sm_t[w] = tok;
  }
  __syncthreads();
  float M = sm_m[0];
  int TOK = sm_t[0];
  for (int k = 1; k < 4; ++k) argmax_merge(M, TOK, sm_m[k], sm_t[k]);

  float zf = 0.0f;
#pragma unroll
  for (int i = 0; i < EPT; ++i) zf += exp2f((x[i] - M) * kLog2e);  // -inf -> 0
  double z = (double)zf;
  for (int off = 32; off > 0; off >>= 1) z += __shfl_xor(z, off, 64);
  if (lane == 0) sm_z[w] = z;
  __syncthreads();
  if (tid == 0) {
    CommitChunk c;
    c.m = M;
    c.tok = TOK;
    c.z = (sm_z[0] + sm_z[1]) + (sm_z[2] + sm_z[3]);
    a.chunks[(size_t)row * a.n_chunks + ch] = c;
  }
}

// Workgroup-wide helpers for the per-sequence kernels (blockDim.x = multiple of 64, <= 1024).
__device__ __forceinline__ double block_min_d(double v, double* red) {
  for (int off = 32; off > 0; off >>= 1) v = fmin(v, __shfl_xor(v, off, 64));
  const int nw = blockDim.x >> 6;
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double r = red[0];
  for (int k = 1; k < nw; ++k) r = fmin(r, red[k]);
  __syncthreads();
  return r;
}

__global__ void commit_merge_kernel(CommitArgs a) {
  __shared__ double red[16];
  const int b = blockIdx.x, i = threadIdx.x;
  const bool in = i < a.S;
  const size_t row = (size_t)b * a.S + i;
  const bool masked = in && a.mask[row];
  float M = -INFINITY;
  int tok = 0x7fffffff;
  double Z = INFINITY;
  bool sure = false, band = false;
  if (masked) {
    const CommitChunk* c = a.chunks + row * a.n_chunks;
    for (int k = 0; k < a.n_chunks; ++k) argmax_merge(M, tok, c[k].m, c[k].tok);
    Z = 0.0;
    for (int k = 0; k < a.n_chunks; ++k) Z += c[k].z * exp((double)c[k].m - (double)M);
    const double zg = Z * (double)a.gamma;
    band = fabs(zg - 1.0) <= kBand;
    sure = !band && zg < 1.0;
  }
  const bool any_sure = __syncthreads_or(sure);
  const bool any_masked = __syncthreads_or(masked);
  bool cand = false;
  if (!any_sure && any_masked) {
    const double zmin = block_min_d(masked ? Z : INFINITY, red);
    cand = masked && Z <= zmin * (1.0 + kFallBand);
  }
  const bool flag = band || cand;
  const bool any_flag = __syncthreads_or(flag);
  if (in) {
    CommitRow r;
    r.m = M;
    r.tok = tok;
    r.z_est = Z;
    r.z_exact = 0.0;
    r.flag = flag ? 1 : 0;
    r.decided = sure ? 1 : 0;
    a.rows[row] = r;
  }
  if (!any_flag) {
    // every decision is safe; with no sure commit there would have been a flagged candidate
    if (in) {
      a.token_id[row] = masked ? tok : -1;
      a.committed[row] = sure ? 1 : 0;
      if (a.conf) a.conf[row] = masked ? (float)(1.0 / Z) : 0.0f;
    }
    if (i == 0) a.seq_done[b] = 1;
  } else if (i == 0) {
    a.seq_done[b] = 0;
  }
}

template <typename T>
__global__ __launch_bounds__(NT) void commit_recheck_kernel(CommitArgs a) {
  __shared__ double red[4];
  const size_t row = blockIdx.x;
  const int b = (int)(row / a.S);
  if (a.seq_done[b] || !a.mask[row] || !a.rows[row].flag) return;
  const T* base = static_cast<const T*>(a.logits) + row * a.V;
  const double M = (double)a.rows[row].m;
  double z = 0.0;
  for (int v = threadIdx.x; v < a.V; v += NT) z += exp((double)to_f(base[v]) - M);
  for (int off = 32; off > 0; off >>= 1) z += __shfl_xor(z, off, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = z;
  __syncthreads();
  if (threadIdx.x == 0) a.rows[row].z_exact = (red[0] + red[1]) + (red[2] + red[3]);
}

__global__ void commit_finalize_kernel(CommitArgs a) {
  __shared__ double red[16];
  const int b = blockIdx.x, i = threadIdx.x;
  if (a.seq_done[b]) return;
  const bool in = i < a.S;
  const size_t row = (size_t)b * a.S + i;
  const bool masked = in && a.mask[row];
  double conf = -1.0;
  bool c = false;
  int tok = -1;
  if (masked) {
    const CommitRow r = a.rows[row];
    tok = r.tok;
    if (r.flag) {
      conf = 1.0 / r.z_exact;
      c = conf > (double)a.gamma;
    } else {
      conf = 1.0 / r.z_est;
      c = r.decided != 0;
    }
  }
  const bool any_c = __syncthreads_or(c);
  const bool any_masked = __syncthreads_or(masked);
  if (!any_c && any_masked) {
    // most confident masked position, lowest i on ties: minimise (-conf, i)
    const double best = -block_min_d(masked ? -conf : INFINITY, red);
    const bool at_best = masked && conf == best;
    // lowest i attaining the best value
    __shared__ int first;
    if (i == 0) first = 0x7fffffff;
    __syncthreads();
    if (at_best) atomicMin(&first, i);
    __syncthreads();
    c = (i == first);
  }
  if (in) {
    a.token_id[row] = masked ? tok : -1;
    a.committed[row] = c ? 1 : 0;
    if (a.conf) a.conf[row] = masked ? (float)conf : 0.0f;
  }
}

}  // namespace

int commit_chunk_elems(int dtype) { return NT * LOADS * (dtype == TT_BF16 ? 8 : 4); }

hipError_t launch_commit(const CommitArgs& a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  const long long nblk = (long long)a.B * a.S * a.n_chunks;
  const int seq_threads = ((a.S + 63) / 64) * 64;
  if (ev0) (void)hipEventRecord(ev0, s);
  if (a.dtype == TT_BF16)
    hipLaunchKernelGGL(commit_reduce_kernel<uint16_t>, dim3((unsigned)nblk), dim3(NT), 0, s, a);
  else
    hipLaunchKernelGGL(commit_reduce_kernel<float>, dim3((unsigned)nblk), dim3(NT), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ev1) (void)hipEventRecord(ev1, s);
  hipLaunchKernelGGL(commit_merge_kernel, dim3(a.B), dim3(seq_threads), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.dtype == TT_BF16)
    hipLaunchKernelGGL(commit_recheck_kernel<uint16_t>, dim3(a.B * a.S), dim3(NT), 0, s, a);
  else
    hipLaunchKernelGGL(commit_recheck_kernel<float>, dim3(a.B * a.S), dim3(NT), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(commit_finalize_kernel, dim3(a.B), dim3(seq_threads), 0, s, a);
  return hipGetLastError();
}

}  // namespace tt
