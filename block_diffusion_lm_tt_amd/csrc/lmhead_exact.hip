// Exact mode of the fused LM head + commit: the rows whose token or decision the fp32 logits
// cannot settle are recomputed in fp64 from the hidden and head rows, so that every integer
// output is the exact-arithmetic one (up to margins below fp64 rounding).
//
// What it computes: the same rule as the fused call (Nemotron-TwoTower, gist.science
// explainer, Technical Summary > Training and Conditioning > Sampling): token = lowest v of
// the row max of l = h W^T, conf = 1/Z with Z = sum_v exp(l_v - max), committed = conf >
// gamma, and the fallback to the most confident masked position (lowest i on ties) of a
// sequence that commits nothing.
//
// How. The fused kernels leave, per masked row, the fp32-logit estimates (max M, token,
// Z) and the runner-up logit M2; the merge bounds every fp32 logit's distance to the exact
// one by eps (a multiple of the row's ||h||_2 and a bound on the head rows' norms). Then:
//  1. lmhead_flag (one workgroup per sequence): the token is settled unless M - M2 <= 2 eps;
//     conf* lies within a factor exp(+-(2 eps + 1e-4)) of the estimate, so the threshold test
//     is settled outside that band, and the fallback winner is settled when a single
//     position's interval reaches the largest lower bound. Rows that are not settled are
//     listed; for each it records which 256-entry vocabulary tiles must be recomputed: every
//     tile for a row whose decision is open, only the tiles whose fp32 max reaches M - 2 eps
//     for a row whose token alone is open (the exact argmax cannot lie elsewhere). Settled
//     outputs are written here.
//  2. lmhead_exact (one workgroup per vocabulary tile, each lane one head row): the listed
//     rows that need the tile, eight at a time: fp64 dot products (each bf16 product exact,
//     fp64 sums), then per row the tile's exact max, lowest argmax and sum of exp in fp64.
//     A tile no listed row needs costs one load of the counter and of its flags.
//  3. lmhead_final (one workgroup per sequence with a listed row): merges each listed row's
//     exact tile records, writes its token and confidence, decides its threshold test in
//     fp64 and, when the fallback was left open, picks the winner among the listed rows (the
//     only ones that can hold the largest confidence).
#include "tt_internal.h"

namespace tt {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int FT = 256;              // threads of the per-sequence kernels
constexpr int kMaxS = 1024;
constexpr double kZBand = 1e-4;      // the fp32 evaluation of Z, relative (about 1e-5)
constexpr int EXB = 16;              // listed rows per pass of the exact kernel (a pass reads
                                     // the tile's head rows once: more rows, fewer passes)
constexpr int KB = 128;              // features per LDS block of the exact kernel

__device__ __forceinline__ double bf(uint16_t x) { return (double)__uint_as_float(((uint32_t)x) << 16); }

template <typename V>
__device__ __forceinline__ V block_reduce(V v, V* red, V (*op)(V, V)) {
  for (int off = 32; off > 0; off >>= 1) v = op(v, __shfl_xor(v, off, 64));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  V r = red[0];
  for (int k = 1; k < FT / 64; ++k) r = op(r, red[k]);
  __syncthreads();
  return r;
}
__device__ double dmax(double a, double b) { return fmax(a, b); }
__device__ double dsum(double a, double b) { return a + b; }
__device__ int imin(int a, int b) { return min(a, b); }
__device__ int isum(int a, int b) { return a + b; }

// seq_state: -2 = no fallback (some position commits for certain, or none is masked);
// -1 = the fallback is open (decided from exact values); p >= 0 = position p is the settled
// fallback winner.
__global__ __launch_bounds__(FT) void lmhead_flag_kernel(LmExactArgs a) {
  __shared__ double s_lo[kMaxS], s_hi[kMaxS];
  __shared__ uint8_t s_dec[kMaxS];  // 0 no, 1 yes, 2 open; 255 unmasked
  __shared__ uint8_t s_tok[kMaxS];  // token open
  __shared__ double redd[FT / 64];
  __shared__ int redi[FT / 64];
  const int b = blockIdx.x, tid = threadIdx.x;
  const double g = (double)a.gamma;
  int yes = 0, open = 0;
  for (int i = tid; i < a.S; i += FT) {
    const size_t r = (size_t)b * a.S + i;
    a.flags[r] = -1;
    if (!a.mask[r]) {
      s_dec[i] = 255;
      s_tok[i] = 0;
      s_lo[i] = s_hi[i] = -1.0;
      a.token_id[r] = -1;
      a.committed[r] = 0;
      if (a.conf) a.conf[r] = 0.0f;
      continue;
    }
    const CommitChunk c = a.merged[r];
    const double m2 = a.rowx[2 * r], eps = a.rowx[2 * r + 1];
    const double conf = 1.0 / c.z;
    const double w = 2.0 * eps + log1p(kZBand);  // half-width of the interval of ln conf*
    s_lo[i] = conf * exp(-w);
    s_hi[i] = conf * exp(w);
    s_tok[i] = (m2 != -INFINITY && (double)c.m - m2 <= 2.0 * eps) ? 1 : 0;
    int d;
    if (g <= 0.0) d = 1;                    // conf* > 0
    else if (g >= 1.0) d = 0;               // conf* <= 1
    else {
      const double lz = log(c.z * g);       // ln(gamma / conf)
      d = fabs(lz) <= w ? 2 : (lz < 0.0 ? 1 : 0);
    }
    s_dec[i] = (uint8_t)d;
    yes |= d == 1;
    open |= d == 2;
    a.token_id[r] = c.tok;
    a.committed[r] = d == 1;
    if (a.conf) a.conf[r] = (float)conf;
  }
  yes = __syncthreads_or(yes);
  open = __syncthreads_or(open);
  int state = -2;
  if (!yes) {
    double lo = -1.0;
    for (int i = tid; i < a.S; i += FT)
      if (s_dec[i] != 255) lo = fmax(lo, s_lo[i]);
    const double maxlo = block_reduce<double>(lo, redd, dmax);
    if (maxlo >= 0.0) {  // some position is masked
      int nc = 0, first = 0x7fffffff;
      for (int i = tid; i < a.S; i += FT)
        if (s_dec[i] != 255 && s_hi[i] >= maxlo) {
          ++nc;
          first = min(first, i);
        }
      nc = block_reduce<int>(nc, redi, isum);
      first = block_reduce<int>(first, redi, imin);
      if (!open && nc == 1) {
        state = first;
        if (tid == 0) a.committed[(size_t)b * a.S + first] = 1;
      } else {
        state = -1;
        for (int i = tid; i < a.S; i += FT)
          if (s_dec[i] != 255 && s_hi[i] >= maxlo) s_dec[i] = 2;  // the candidates: exact values needed
      }
    }
  }
  if (tid == 0) a.seq_state[b] = state;
  __syncthreads();
  // list the rows left open, then mark the tiles each needs (the whole workgroup per row)
  __shared__ int s_slot[kMaxS];
  for (int i = tid; i < a.S; i += FT) {
    s_slot[i] = -1;
    if (s_dec[i] == 255 || (s_dec[i] != 2 && !s_tok[i])) continue;
    const size_t r = (size_t)b * a.S + i;
    const int slot = atomicAdd(a.count, 1);
    a.flags[r] = slot;
    a.list[slot] = (int)r;
    s_slot[i] = slot;
  }
  __syncthreads();
  for (int i = 0; i < a.S; ++i) {
    const int slot = s_slot[i];
    if (slot < 0) continue;
    const size_t r = (size_t)b * a.S + i;
    uint8_t* need = a.need + (size_t)slot * a.NVT;
    if (s_dec[i] == 2) {
      for (int t = tid; t < a.NVT; t += FT) need[t] = 1;
    } else {
      const CommitChunk* ch = a.chunks + r * a.NVT;
      const double lim = (double)a.merged[r].m - 2.0 * a.rowx[2 * r + 1];
      for (int t = tid; t < a.NVT; t += FT) need[t] = (double)ch[t].m >= lim;
    }
  }
}

// One workgroup per 256-entry vocabulary tile; lane v of the tile accumulates, for up to EXB
// listed rows at a time, sum_k h[k] w_v[k] in fp64 (hidden features staged in LDS as fp64,
// read by broadcast), then each row's tile record is reduced over the workgroup.
static_assert(EXB * KB * 8 + EXB * 256 * 8 <= 160 * 1024 - 4096, "exact kernel LDS");
__global__ __launch_bounds__(256) void lmhead_exact_kernel(LmExactArgs a) {
  __shared__ double hs[EXB][KB];
  __shared__ double lg[EXB][256];
  __shared__ int rows[EXB], slots[EXB];
  __shared__ int nsel;
  __shared__ double redd[4];
  __shared__ int redi[4];
  const int vt = blockIdx.x, tid = threadIdx.x;
  const int F = *a.count;
  if (F == 0) return;
  const int v = vt * 256 + tid;
  const uint16_t* W = static_cast<const uint16_t*>(a.weight);
  const uint16_t* Hd = static_cast<const uint16_t*>(a.hidden);
  const uint16_t* wrow = W + (size_t)min(v, a.V - 1) * a.K;
  int f0 = 0;
  while (true) {
    // the next listed rows that need this tile
    if (tid == 0) {
      int n = 0;
      for (; f0 < F && n < EXB; ++f0)
        if (a.need[(size_t)f0 * a.NVT + vt]) {
          slots[n] = f0;
          rows[n] = a.list[f0];
          ++n;
        }
      nsel = n;
    }
    __syncthreads();
    const int nf = nsel;
    if (nf == 0) break;
    double acc[EXB];
#pragma unroll
    for (int j = 0; j < EXB; ++j) acc[j] = 0.0;
    for (int k0 = 0; k0 < a.K; k0 += KB) {
      const int kn = min(KB, a.K - k0);
      __syncthreads();
      for (int e = tid; e < EXB * KB; e += 256) {
        const int j = e / KB, k = e - j * KB;
        hs[j][k] = (j < nf && k < kn) ? bf(Hd[(size_t)rows[j] * a.K + k0 + k]) : 0.0;
      }
      __syncthreads();
      for (int k = 0; k < kn; k += 8) {
        const u32x4 wv = *reinterpret_cast<const u32x4*>(wrow + k0 + k);
        const uint16_t* we = reinterpret_cast<const uint16_t*>(&wv);
        double wd[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) wd[u] = bf(we[u]);
#pragma unroll
        for (int j = 0; j < EXB; ++j) {
          if (j < nf) {
#pragma unroll
            for (int u = 0; u < 8; ++u) acc[j] = fma(hs[j][k + u], wd[u], acc[j]);
          }
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < EXB; ++j) lg[j][tid] = v < a.V ? acc[j] : -INFINITY;
    __syncthreads();
    for (int j = 0; j < nf; ++j) {
      const double x = lg[j][tid];
      const double M = block_reduce<double>(x, redd, dmax);
      const int tk = block_reduce<int>(x == M ? v : 0x7fffffff, redi, imin);
      const double z = block_reduce<double>(x == -INFINITY ? 0.0 : exp(x - M), redd, dsum);
      if (tid == 0) {
        ExactChunk e;
        e.m = M;
        e.tok = tk;
        e.pad = 0;
        e.z = z;
        a.exact[(size_t)slots[j] * a.NVT + vt] = e;
      }
    }
    __syncthreads();
  }
}

// merge of exact tile records (the tiles a row needed; larger max wins, equal maxima keep the
// lower index, z moves to the common max)
__device__ __forceinline__ void exact_merge(double& m, int& tok, double& z, double m2, int t2, double z2) {
  if (m2 == -INFINITY) return;
  if (m == -INFINITY) {
    m = m2;
    tok = t2;
    z = z2;
    return;
  }
  const double M = fmax(m, m2);
  z = z * exp(m - M) + z2 * exp(m2 - M);
  if (m2 > m || (m2 == m && t2 < tok)) tok = t2;
  m = M;
}

__global__ __launch_bounds__(FT) void lmhead_final_kernel(LmExactArgs a) {
  __shared__ double redd[FT / 64], redz[FT / 64];
  __shared__ int redi[FT / 64];
  __shared__ double s_conf[kMaxS];  // exact confidence of a wholly recomputed row, else -1
  const int b = blockIdx.x, tid = threadIdx.x;
  int any = 0;
  for (int i = tid; i < a.S; i += FT) {
    any |= a.flags[(size_t)b * a.S + i] >= 0;
    s_conf[i] = -1.0;
  }
  if (!__syncthreads_or(any)) return;
  const int state = a.seq_state[b];
  const double g = (double)a.gamma;
  for (int i = 0; i < a.S; ++i) {  // (uniform loop: every thread reads the same slot)
    const size_t r = (size_t)b * a.S + i;
    const int slot = a.flags[r];
    if (slot < 0) continue;
    const uint8_t* need = a.need + (size_t)slot * a.NVT;
    const ExactChunk* ex = a.exact + (size_t)slot * a.NVT;
    double m = -INFINITY, z = 0.0;
    int tok = 0x7fffffff, all = 1;
    for (int t = tid; t < a.NVT; t += FT) {
      if (need[t]) exact_merge(m, tok, z, ex[t].m, ex[t].tok, ex[t].z);
      else all = 0;
    }
    all = __syncthreads_and(all);
    for (int off = 32; off > 0; off >>= 1) {
      const double m2 = __shfl_xor(m, off, 64);
      const int t2 = __shfl_xor(tok, off, 64);
      const double z2 = __shfl_xor(z, off, 64);
      exact_merge(m, tok, z, m2, t2, z2);
    }
    if ((tid & 63) == 0) {
      redd[tid >> 6] = m;
      redi[tid >> 6] = tok;
      redz[tid >> 6] = z;
    }
    __syncthreads();
    if (tid == 0) {
      double M = redd[0], Z = redz[0];
      int T = redi[0];
      for (int w = 1; w < FT / 64; ++w) exact_merge(M, T, Z, redd[w], redi[w], redz[w]);
      a.token_id[r] = T;
      // a row recomputed for its token alone (some of its tiles) keeps its settled decision
      // and confidence estimate
      if (all) {
        const double conf = 1.0 / Z;
        if (a.conf) a.conf[r] = (float)conf;
        const int d = (g <= 0.0) ? 1 : (g >= 1.0 ? 0 : (conf > g ? 1 : 0));
        a.committed[r] = (uint8_t)(d || i == state);
        s_conf[i] = conf;
      }
    }
    __syncthreads();
  }
  if (state == -1 && tid == 0) {
    // no certain commit: unless a recomputed row commits, the fallback winner is the largest
    // exact confidence among the wholly recomputed rows (every position that can hold the
    // largest confidence was recomputed), lowest position on ties
    int yes = 0;
    for (int i = 0; i < a.S; ++i) {
      const size_t r = (size_t)b * a.S + i;
      yes |= a.mask[r] && a.committed[r];
    }
    if (!yes) {
      double best = -1.0;
      int bi = -1;
      for (int i = 0; i < a.S; ++i)
        if (s_conf[i] > best) {
          best = s_conf[i];
          bi = i;
        }
      if (bi >= 0) a.committed[(size_t)b * a.S + bi] = 1;
    }
  }
}

// ---- the weight bound: out = max_v ||w_v||_2, rounded up to fp32 --------------------------
__global__ void zero_kernel(float* out) { *out = 0.0f; }

__global__ __launch_bounds__(256) void weight_bound_kernel(const uint16_t* W, int V, int K, float* out) {
  __shared__ double red[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  double best = 0.0;
  for (int v = blockIdx.x * 4 + w; v < V; v += gridDim.x * 4) {
    const uint16_t* row = W + (size_t)v * K;
    double s = 0.0;  // exact squares, fp64 sums
    if (K % 8 == 0 && (reinterpret_cast<uintptr_t>(W) & 15) == 0) {
      for (int k = lane * 8; k < K; k += 512) {
        const u32x4 q = *reinterpret_cast<const u32x4*>(row + k);
        const uint16_t* e = reinterpret_cast<const uint16_t*>(&q);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const double x = bf(e[u]);
          s = fma(x, x, s);
        }
      }
    } else {
      for (int k = lane; k < K; k += 64) {
        const double x = bf(row[k]);
        s = fma(x, x, s);
      }
    }
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    best = fmax(best, s);
  }
  if (lane == 0) red[w] = best;
  __syncthreads();
  if (tid == 0) {
    const double m = fmax(fmax(red[0], red[1]), fmax(red[2], red[3]));
    // sqrt of an fp64 sum of at most 2^20 terms, inflated to cover its rounding, then
    // rounded up to fp32; non-negative floats order like their bit patterns
    const float f = __double2float_ru(sqrt(m) * (1.0 + 1e-9));
    atomicMax(reinterpret_cast<unsigned int*>(out), __float_as_uint(f));
  }
}

}  // namespace

hipError_t launch_lmhead_flag(const LmExactArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(lmhead_flag_kernel, dim3(a.B), dim3(FT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_lmhead_exact(const LmExactArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(lmhead_exact_kernel, dim3(a.NVT), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_lmhead_final(const LmExactArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(lmhead_final_kernel, dim3(a.B), dim3(FT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_lmhead_weight_bound(const void* weight, int V, int K, float* out, hipStream_t s) {
  hipLaunchKernelGGL(zero_kernel, dim3(1), dim3(1), 0, s, out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(weight_bound_kernel, dim3(1024), dim3(256), 0, s, static_cast<const uint16_t*>(weight), V, K,
                     out);
  return hipGetLastError();
}

}  // namespace tt
