// Confidence-threshold commit (confidence unmasking) of one denoising step.
//
// What it computes: Nemotron-TwoTower (gist.science explainer), Technical Summary >
// Training and Conditioning > Sampling, and the snilld.dk TwoTower article, "Blockwise
// generering i praksis". For each masked position: token = lowest index of the row max,
// Z = sum_v exp(l_v - max), conf = 1/Z, committed = conf > gamma; a sequence with masked
// positions and no commit commits its most confident masked position (lowest i on ties).
//
// How: the work is one pass over the masked rows' logits, so it is HBM bound. Two launches,
// with no communication between workgroups inside a launch:
//  1. commit_reduce: one workgroup per (masked row, vocabulary chunk). Each thread issues its
//     eight 16-byte non-temporal loads at once and consumes them in element order with an
//     online max, lowest argmax and sum of exp2((x - m) * log2 e) relative to its running
//     max m (rescaled when m grows); the workgroup merges (max, argmax) (wave shuffles +
//     LDS, lowest index on ties) and sums the threads' partials, moved to the chunk max, in
//     fp64. Unmasked rows exit at once and are never read.
//  2. commit_decide: one workgroup per sequence. It merges each masked row's chunks in chunk
//     order in one pass (all of a row's record loads in flight, online max / lowest argmax /
//     fp64 sum rescaled by fp32 factors), giving the row's token and an estimate of Z whose
//     relative error is below 1e-5 (per fp32 partial: 64 terms, each exp2 of a scaled
//     difference to the running max, and at most 9 rescalings; about 7e-6 in the worst
//     case). A threshold decision is taken on the estimate only outside a relative band of
//     1e-4; the fallback is taken on the estimate only when its winner leads every other
//     position by more than 4e-4. Positions inside a band are recomputed by the same
//     workgroup over the full row with fp64 exp and decided on those values (conf = 1/Z >
//     gamma, in fp64 as in exact arithmetic), so every integer output is the
//     exact-arithmetic decision except for margins below fp64 rounding. Called behind the
//     fused LM head (no logits in memory), the same kernel decides on the chunk estimates
//     alone, without the bands.
//  Folding step 2 into step 1 (the last-arriving workgroup of a sequence deciding) was built
//  and measured slower: the arrival counters are device-scope atomics on one word per
//  sequence, about 80 per word here, and they serialize (49.6 us per call against 25).
#include <mutex>

#include "tt_internal.h"

namespace tt {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int NT = 256;
constexpr int LOADS = 8;  // 16-byte loads per thread per chunk
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

// ---- per-sequence decision (by one workgroup of NTH threads) ---------------------------

template <int NTH>
__device__ __forceinline__ double dblock_max(double v, double* red) {
  for (int off = 32; off > 0; off >>= 1) v = fmax(v, __shfl_xor(v, off, 64));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double r = red[0];
  for (int k = 1; k < NTH / 64; ++k) r = fmax(r, red[k]);
  return r;
}

template <int NTH>
__device__ __forceinline__ double dblock_sum(double v, double* red) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double r = red[0];
  for (int k = 1; k < NTH / 64; ++k) r += red[k];
  return r;
}

template <int NTH>
__device__ __forceinline__ int iblock_min(int v, int* red) {
  for (int off = 32; off > 0; off >>= 1) v = min(v, __shfl_xor(v, off, 64));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  int r = red[0];
  for (int k = 1; k < NTH / 64; ++k) r = min(r, red[k]);
  return r;
}

template <int NTH>
__device__ __forceinline__ int iblock_sum(int v, int* red) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  int r = red[0];
  for (int k = 1; k < NTH / 64; ++k) r += red[k];
  return r;
}

// fp64 Z of one row, by the whole workgroup (fixed reduction order: deterministic)
template <typename T, int NTH>
__device__ double row_z_fp64(const T* row, int V, double M, double* red) {
  double z = 0.0;
  for (int v = threadIdx.x; v < V; v += NTH) z += exp((double)to_f(row[v]) - M);
  return dblock_sum<NTH>(z, red);
}

struct DecideSmem {
  double redd[16];
  int redi[16];
  int nl;
  float Mf;
  int flagged[1024];
};

// Decide sequence b from its rows' chunk records: tokens, confidences, the gamma rule with
// the fallback, and the fp64 recheck of the rows inside a band (when a.logits is given).
// Writes the outputs of the masked rows, and of the unmasked rows too when write_unmasked.
template <typename T, int NTH, int MAXP>
__device__ void decide_sequence(const CommitArgs& a, int b, bool write_unmasked, DecideSmem& sh) {
  // MAXP: positions per thread (S <= NTH * MAXP)
  const int tid = threadIdx.x;
  const T* logits = static_cast<const T*>(a.logits);
  bool msk[MAXP];
  float mm[MAXP];
  double zz[MAXP];
  int tk[MAXP], fl[MAXP], dec[MAXP];
  int any_c = 0, nflag = 0, nmask = 0;
  const bool exact = a.logits != nullptr;  // else: no logits to recompute from
  // the mask bytes and the first eight chunk records of every position are loaded together
  // (records of unmasked rows are read and ignored), so that one round trip serves both
  uint8_t mraw[MAXP];
  unsigned long long r0[MAXP][8], z0[MAXP][8];
#pragma unroll
  for (int p = 0; p < MAXP; ++p) {
    const size_t row = (size_t)b * a.S + min(tid + p * NTH, a.S - 1);
    mraw[p] = a.mask[row];
    const unsigned long long* c = reinterpret_cast<const unsigned long long*>(a.chunks + row * a.n_chunks);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = min(j, a.n_chunks - 1);
      r0[p][j] = c[2 * k];
      z0[p][j] = c[2 * k + 1];
    }
  }
#pragma unroll
  for (int p = 0; p < MAXP; ++p) {
    const int i = tid + p * NTH;
    const size_t row = (size_t)b * a.S + i;
    msk[p] = i < a.S && mraw[p];
    mm[p] = -INFINITY;
    zz[p] = 1.0;
    tk[p] = -1;
    fl[p] = dec[p] = 0;
    if (write_unmasked && i < a.S && !msk[p]) {
      a.token_id[row] = -1;
      a.committed[row] = 0;
      if (a.conf) a.conf[row] = 0.0f;
    }
    if (!msk[p]) continue;
    ++nmask;
    // merge the row's chunk records (written by the previous launch), eight at a time with
    // all loads in flight, by an online max / lowest argmax / rescaled fp64 sum in chunk
    // order (the rescale factors in fp32: relative error ~1e-7 on an estimate decided
    // outside 1e-4)
    const unsigned long long* c = reinterpret_cast<const unsigned long long*>(a.chunks + row * a.n_chunks);
    float M = -INFINITY;
    int tok = 0x7fffffff;
    double Z = 0.0;
    for (int k0 = 0; k0 < a.n_chunks; k0 += 8) {
      unsigned long long r[8], zb[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int k = min(k0 + j, a.n_chunks - 1);
        r[j] = k0 == 0 ? r0[p][j] : c[2 * k];
        zb[j] = k0 == 0 ? z0[p][j] : c[2 * k + 1];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (k0 + j >= a.n_chunks) break;
        const float mk = __uint_as_float((uint32_t)r[j]);
        const double zk = __longlong_as_double((long long)zb[j]);
        const float mn = fmaxf(M, mk);
        if (mk > M || (mk == M && (int)(uint32_t)(r[j] >> 32) < tok)) tok = (int)(uint32_t)(r[j] >> 32);
        Z = Z * (double)__builtin_amdgcn_exp2f((M - mn) * kLog2e) + zk * (double)__builtin_amdgcn_exp2f((mk - mn) * kLog2e);
        M = mn;
      }
    }
    mm[p] = M;
    tk[p] = tok;
    zz[p] = Z;
    const double zg = Z * (double)a.gamma;
    if (exact && fabs(zg - 1.0) <= kBand) {
      fl[p] = 1;
      ++nflag;
    } else {
      dec[p] = zg < 1.0;
    }
    any_c |= dec[p];
  }
  any_c = __syncthreads_or(any_c);
  nmask = iblock_sum<NTH>(nmask, sh.redi);
  int nflag_tot = iblock_sum<NTH>(nflag, sh.redi);
  // fallback on the estimates when it is unambiguous; otherwise flag every candidate
  bool fallback_pending = false;
  if (!any_c && nmask > 0) {
    double my = -1.0;
#pragma unroll
    for (int p = 0; p < MAXP; ++p)
      if (msk[p]) my = fmax(my, 1.0 / zz[p]);
    const double best = dblock_max<NTH>(my, sh.redd);
    int mi = 0x7fffffff;
#pragma unroll
    for (int p = 0; p < MAXP; ++p)
      if (msk[p] && 1.0 / zz[p] == best) mi = min(mi, tid + p * NTH);
    const int bi = iblock_min<NTH>(mi, sh.redi);
    double my2 = -1.0;
#pragma unroll
    for (int p = 0; p < MAXP; ++p)
      if (msk[p] && tid + p * NTH != bi) my2 = fmax(my2, 1.0 / zz[p]);
    const double second = dblock_max<NTH>(my2, sh.redd);
    if (exact && (nflag_tot > 0 || (second >= 0.0 && best <= second * (1.0 + kFallBand)))) {
      fallback_pending = true;
#pragma unroll
      for (int p = 0; p < MAXP; ++p)
        if (msk[p] && fl[p] == 0 && (1.0 / zz[p]) * (1.0 + kFallBand) >= best) {
          fl[p] = 1;
          ++nflag;
        }
      nflag_tot = iblock_sum<NTH>(nflag, sh.redi);
    } else {
#pragma unroll
      for (int p = 0; p < MAXP; ++p)
        if (tid + p * NTH == bi) dec[p] = 1;
    }
  }
  if (nflag_tot > 0) {
    // fp64 recomputation of every flagged row by the whole workgroup
    if (tid == 0) sh.nl = 0;
    __syncthreads();
#pragma unroll
    for (int p = 0; p < MAXP; ++p)
      if (fl[p]) sh.flagged[atomicAdd(&sh.nl, 1)] = tid + p * NTH;
    __syncthreads();
    const int n = sh.nl;
    for (int f = 0; f < n; ++f) {
      const int i = sh.flagged[f];
      const size_t row = (size_t)b * a.S + i;
      if ((i % NTH) == tid) sh.Mf = mm[i / NTH];
      __syncthreads();
      const double z = row_z_fp64<T, NTH>(logits + row * a.V, a.V, (double)sh.Mf, sh.redd);
      if ((i % NTH) == tid) zz[i / NTH] = z;
      __syncthreads();
    }
    any_c = 0;
#pragma unroll
    for (int p = 0; p < MAXP; ++p) {
      if (!msk[p]) continue;
      if (fl[p]) dec[p] = (1.0 / zz[p]) > (double)a.gamma;  // band rows decided exactly
      any_c |= dec[p];
    }
    any_c = __syncthreads_or(any_c);
    if (!any_c && (fallback_pending || nmask > 0)) {
      // most confident masked position (flagged rows carry exact values; every other row
      // is outside the candidate band), lowest position on ties
      double my = -1.0;
#pragma unroll
      for (int p = 0; p < MAXP; ++p)
        if (msk[p]) my = fmax(my, 1.0 / zz[p]);
      const double best = dblock_max<NTH>(my, sh.redd);
      int mi = 0x7fffffff;
#pragma unroll
      for (int p = 0; p < MAXP; ++p)
        if (msk[p] && 1.0 / zz[p] == best) mi = min(mi, tid + p * NTH);
      const int bi = iblock_min<NTH>(mi, sh.redi);
#pragma unroll
      for (int p = 0; p < MAXP; ++p)
        if (tid + p * NTH == bi) dec[p] = 1;
    }
  }
#pragma unroll
  for (int p = 0; p < MAXP; ++p) {
    if (!msk[p]) continue;
    const size_t row = (size_t)b * a.S + tid + p * NTH;
    a.token_id[row] = tk[p];
    a.committed[row] = dec[p] ? 1 : 0;
    if (a.conf) a.conf[row] = (float)(1.0 / zz[p]);
  }
}

// ---- step 1: per-chunk reduction ------------------------------------------------------

template <typename T>
__global__ __launch_bounds__(NT) void commit_reduce_kernel(CommitArgs a) {
  constexpr int VE = Vec<T>::N;
  __shared__ float sm_m[4];
  __shared__ int sm_t[4];
  __shared__ double sm_z[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int blk = blockIdx.x;
  const int row = blk / a.n_chunks;
  const int ch = blk - row * a.n_chunks;
  if (!a.mask[row]) return;  // an unmasked row is never read
  const T* base = static_cast<const T*>(a.logits) + (size_t)row * a.V;
  const int begin = ch * a.chunk_elems;
  const int end = min(a.V, begin + a.chunk_elems);

  // All of the thread's 16-byte loads are issued first; each is consumed as it lands, in
  // increasing element order, by an online max / lowest argmax / rescaled sum (few live
  // registers, so many workgroups per CU and many loads in flight). A chunk that is not
  // whole (the row's last) or not 16-byte aligned takes element loads instead.
  float m = -INFINITY, sf = 0.0f;  // sf = sum of exp2((x - m) log2 e) over the elements seen
  int tok = 0x7fffffff;
  auto consume = [&](const float (&v)[VE], int i0) {
    float mb = v[0];
    int kb = 0;
#pragma unroll
    for (int k = 1; k < VE; ++k)
      if (v[k] > mb) {
        mb = v[k];
        kb = k;
      }
    if (mb > m) tok = i0 + kb;  // strict: an equal later value keeps the lower index
    const float mn = fmaxf(m, mb);
    sf *= (m == mn) ? 1.0f : __builtin_amdgcn_exp2f((m - mn) * kLog2e);  // exp2(-inf) = 0
    if (mn != -INFINITY) {
#pragma unroll
      for (int k = 0; k < VE; ++k) sf += __builtin_amdgcn_exp2f((v[k] - mn) * kLog2e);  // -inf -> 0
    }
    m = mn;
  };
  const bool whole = begin + a.chunk_elems <= end && ((reinterpret_cast<uintptr_t>(base + begin) & 15) == 0);
  if (whole) {
    u32x4 raw[LOADS];
#pragma unroll
    for (int ld = 0; ld < LOADS; ++ld)
      raw[ld] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + begin + (ld * NT + tid) * VE));
#pragma unroll
    for (int ld = 0; ld < LOADS; ++ld) {
      const T* e = reinterpret_cast<const T*>(&raw[ld]);
      float v[VE];
#pragma unroll
      for (int k = 0; k < VE; ++k) v[k] = to_f(e[k]);
      consume(v, begin + (ld * NT + tid) * VE);
    }
  } else {
    for (int ld = 0; ld < LOADS; ++ld) {
      const int i0 = begin + (ld * NT + tid) * VE;
      float v[VE];
#pragma unroll
      for (int k = 0; k < VE; ++k) v[k] = (i0 + k < end) ? to_f(base[i0 + k]) : -INFINITY;
      consume(v, i0);
    }
  }
  const float mt = m;  // this thread's max: its sum is relative to it
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

  // the thread's sum moved to the chunk max (mt <= M; a thread that saw only -inf adds 0)
  const float zf = mt == -INFINITY ? 0.0f : sf * __builtin_amdgcn_exp2f((mt - M) * kLog2e);
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

// ---- step 2: per-sequence decision -----------------------------------------------------

// one workgroup per sequence: a single wave for blocks of up to 64 positions, else 512 threads
template <typename T, int NTH, int MAXP>
__global__ __launch_bounds__(NTH) void commit_decide_kernel(CommitArgs a) {
  __shared__ DecideSmem dsm;
  decide_sequence<T, NTH, MAXP>(a, blockIdx.x, true, dsm);
}

}  // namespace

template <typename T>
hipError_t launch_decide_t(const CommitArgs& a, hipStream_t s) {
  if (a.S <= 64)
    hipLaunchKernelGGL((commit_decide_kernel<T, 64, 1>), dim3(a.B), dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL((commit_decide_kernel<T, 512, 2>), dim3(a.B), dim3(512), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_commit_decide(const CommitArgs& a, hipStream_t s) { return launch_decide_t<uint16_t>(a, s); }

int commit_chunk_elems(int dtype) { return NT * LOADS * (dtype == TT_BF16 ? 8 : 4); }

// ---- scratch of the allocation-free commit entry point ---------------------------------
// One array per GPU, held until the process ends; every allocation-free commit call on a GPU
// uses that GPU's copy (calls that overlap on one GPU race on it). In host code the array's
// name is only a stand-in: its device address is looked up once per device and kept.
static __device__ __align__(256) unsigned char scratch[kCommitScratchBytes];

hipError_t commit_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_commit(const CommitArgs& a, hipStream_t s, hipEvent_t ev_reduce_end) {
  const long long nblk = (long long)a.B * a.S * a.n_chunks;
  if (a.dtype == TT_BF16)
    hipLaunchKernelGGL(commit_reduce_kernel<uint16_t>, dim3((unsigned)nblk), dim3(NT), 0, s, a);
  else
    hipLaunchKernelGGL(commit_reduce_kernel<float>, dim3((unsigned)nblk), dim3(NT), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ev_reduce_end) (void)hipEventRecord(ev_reduce_end, s);
  return a.dtype == TT_BF16 ? launch_decide_t<uint16_t>(a, s) : launch_decide_t<float>(a, s);
}

}  // namespace tt
