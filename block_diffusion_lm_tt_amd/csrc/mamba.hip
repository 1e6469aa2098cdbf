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
// How (bf16, P a multiple of 16 up to 128, N = 32, 64 or 128, 16-byte aligned inputs): one
// workgroup per (sequence, head), P / 16 waves, wave w owning the state rows p in
// [16w, 16w + 16). The seeded state (P x N fp32) is the stream that bounds the kernel; it is
// loaded straight into matrix-core accumulator tiles (16 state columns x 16 rows each) and
// stays there. The recurrence is evaluated in its unrolled (chunked) form, chunks of up to 16
// positions: with L_t the cumulative log decay inside the chunk,
//   y_t = e^{L_t} (state C_t) + sum_{s<=t} e^{L_t - L_s} delta_s (C_t . B_s) x_s + D x_t,
//   state' = e^{L_last} state + sum_s e^{L_last - L_s} delta_s x_s B_s^T
// and every product is a v_mfma_f32_16x16x{32,16}_bf16: the chunk's C_t . B_s (exact bf16
// inputs), the readout state C_t, the within-chunk sum (with D on the diagonal), the state
// update. fp32 operands (the state, the decay-weighted within-chunk matrix, the weighted
// inputs) enter as a pair of bf16 values hi + lo, hi the rounded value and lo the rounded
// remainder, which carries 16 of fp32's 24 significand bits: each term's error stays within
// 2^-17 of its magnitude, accumulated in fp32.
//
// Otherwise (fp32 inputs, other widths, unaligned bases): one workgroup of 256 threads per
// (sequence, head) on the vector ALUs; each thread holds a run of one state row in registers,
// the readout state C_t is P x N x chunk FMAs, the within-chunk matrix is computed once per
// chunk and shared by the P rows, and the state update runs only between chunks or for the
// returned state.
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

// ---- matrix-core path --------------------------------------------------------------------

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ short bf16_bits(float v) { return __builtin_bit_cast(short, (__bf16)v); }
__device__ __forceinline__ float bits_f32(short b) { return __uint_as_float(((uint32_t)(uint16_t)b) << 16); }

// v = hi + lo + r with hi, lo bf16 (rounded to nearest) and |r| <= 2^-17 |v|
__device__ __forceinline__ void split_bf16(float v, short& hi, short& lo) {
  hi = bf16_bits(v);
  lo = bf16_bits(v - bits_f32(hi));
}

// LDS of one chunk: B and C rows (bf16, rows of N padded by 16 bytes), B transposed [n][s]
// and x transposed [p][s] (rows of 16 positions padded to 20)
template <int NW, int NM>
struct alignas(16) MmaSmem {
  static constexpr int N = 32 * NM, P = 16 * NW;
  static constexpr int RB = N + 8;   // bf16 elements per B / C row
  static constexpr int RT = 20;      // bf16 elements per transposed row
  uint16_t sB[CH * RB];
  uint16_t sC[CH * RB];
  uint16_t sBT[N * RT];
  uint16_t sXT[P * RT];
};

// state column of accumulator row r of tile T: tiles 2m and 2m + 1 hold the columns
// 32m + 8 (r / 4) + (r % 4) and the same + 4, so that lane group g's eight readout slots are the
// contiguous columns 32m + 8g .. 32m + 8g + 7
__device__ __forceinline__ int tile_col(int T, int r) { return 32 * (T >> 1) + 8 * (r >> 2) + 4 * (T & 1) + (r & 3); }

// One chunk's inputs in registers: this thread's 16-byte pieces of the B and C rows and of
// the x rows (zero past the chunk end), and lane c's step input dt (position c).
template <int NW, int NM>
struct ChunkRegs {
  static constexpr int NTH = 64 * NW, N = 32 * NM, P = 16 * NW;
  static constexpr int NBC = 2 * CH * (N / 8);      // B and C pieces per chunk
  static constexpr int NX = CH * (P / 8);           // x pieces per chunk
  static constexpr int KB = (NBC + NTH - 1) / NTH;  // per thread
  static constexpr int KX = (NX + NTH - 1) / NTH;
  uint4 bc[KB];
  uint4 x[KX];
  float dt;
};

// The loads are unconditional (indexes clamped into the chunk) so that they all issue before
// the first wait; what lies past the chunk end is zeroed when the pieces are stored.
template <int NW, int NM>
__device__ __forceinline__ void chunk_load(ChunkRegs<NW, NM>& r, const MambaArgs& a, int b, int h, int grp,
                                           int t0, int lc, int tid, int c) {
  using R = ChunkRegs<NW, NM>;
  const uint16_t* Bm = static_cast<const uint16_t*>(a.Bm);
  const uint16_t* Cm = static_cast<const uint16_t*>(a.Cm);
  const uint16_t* X = static_cast<const uint16_t*>(a.x);
#pragma unroll
  for (int k = 0; k < R::KB; ++k) {
    const int i = min(tid + k * R::NTH, R::NBC - 1);
    const int which = i / (CH * (R::N / 8));
    const int j = i - which * (CH * (R::N / 8));
    const int s = min(j / (R::N / 8), lc - 1), q = j % (R::N / 8);
    r.bc[k] = *reinterpret_cast<const uint4*>((which ? Cm : Bm) +
                                              (((size_t)b * a.S + t0 + s) * a.G + grp) * R::N + 8 * q);
  }
#pragma unroll
  for (int k = 0; k < R::KX; ++k) {
    const int i = min(tid + k * R::NTH, R::NX - 1);
    const int s = min(i / (R::P / 8), lc - 1), q = i % (R::P / 8);
    r.x[k] = *reinterpret_cast<const uint4*>(X + (((size_t)b * a.S + t0 + s) * a.H + h) * R::P + 8 * q);
  }
  r.dt = a.dt[((size_t)b * a.S + t0 + min(c, lc - 1)) * a.H + h];
}

template <int NW, int NM>
__device__ __forceinline__ void chunk_store(const ChunkRegs<NW, NM>& r, MmaSmem<NW, NM>& sm, int tid, int lc,
                                            bool update) {
  using R = ChunkRegs<NW, NM>;
  using Sm = MmaSmem<NW, NM>;
  const uint4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int k = 0; k < R::KB; ++k) {
    const int i = tid + k * R::NTH;
    if (i >= R::NBC) break;
    const int which = i / (CH * (R::N / 8));
    const int j = i - which * (CH * (R::N / 8));
    const int s = j / (R::N / 8), q = j % (R::N / 8);
    const uint4 v = s < lc ? r.bc[k] : zero;
    *reinterpret_cast<uint4*>((which ? sm.sC : sm.sB) + s * Sm::RB + 8 * q) = v;
    if (!which && update) {
      const uint16_t* e = reinterpret_cast<const uint16_t*>(&v);
#pragma unroll
      for (int u = 0; u < 8; ++u) sm.sBT[(8 * q + u) * Sm::RT + s] = e[u];
    }
  }
#pragma unroll
  for (int k = 0; k < R::KX; ++k) {
    const int i = tid + k * R::NTH;
    if (i >= R::NX) break;
    const int s = i / (R::P / 8), q = i % (R::P / 8);
    const uint4 v = s < lc ? r.x[k] : zero;
    const uint16_t* e = reinterpret_cast<const uint16_t*>(&v);
#pragma unroll
    for (int u = 0; u < 8; ++u) sm.sXT[(8 * q + u) * Sm::RT + s] = e[u];
  }
}

// (at least four waves per SIMD: within 128 registers, four workgroups of four waves per CU
// keep their state loads in flight; the compiler fits the headline shape without spills)
template <int NW, int NM>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(4, 8))) void mamba2_scan_mfma_kernel(MambaArgs a) {
  constexpr int N = 32 * NM, P = 16 * NW, NT2 = 2 * NM;
  using Sm = MmaSmem<NW, NM>;
  __shared__ Sm sm;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = lane & 15, g = lane >> 4;   // accumulator column / operand row, lane group
  const int bh = blockIdx.x;
  const int b = bh / a.H, h = bh - b * a.H;
  const int grp = h / (a.H / a.G);
  const int S = a.S, H = a.H;
  uint16_t* Y = static_cast<uint16_t*>(a.y);
  const bool want_state = a.h_out != nullptr;
  const int p = 16 * w + c;                 // this lane's state row (accumulator column)

  // every load of the first chunk is issued before any is used: the chunk's B, C, x and dt
  // first, then the seeded state (lane (p, g) takes the columns 32m + 8g .. + 7 of row p as two
  // 16-byte loads), which is not needed until the readout
  ChunkRegs<NW, NM> cr;
  int lc = min(CH, S);
  chunk_load(cr, a, b, h, grp, 0, lc, tid, c);
  f32x4 st[NT2];  // the state: st[T][i] = state[p][tile_col(T, 4g + i)]
  {
    const float* h0 = a.h0 + ((size_t)bh * P + p) * N + 8 * g;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const float4 u = *reinterpret_cast<const float4*>(h0 + 32 * m);
      const float4 v = *reinterpret_cast<const float4*>(h0 + 32 * m + 4);
      st[2 * m] = f32x4{u.x, u.y, u.z, u.w};
      st[2 * m + 1] = f32x4{v.x, v.y, v.z, v.w};
    }
  }
  const float A = -expf(a.A_log[h]);
  const float bias = a.dt_bias[h];
  const float Dh = a.Dskip[h];

  for (int t0 = 0;;) {
    const bool update = t0 + lc < S || want_state;
    chunk_store(cr, sm, tid, lc, update);
    // step sizes and cumulative log decay of the chunk, replicated in each group of 16 lanes
    // (lane c holds position c)
    const float dl = c < lc ? softplus(cr.dt + bias) : 0.0f;
    float L = dl * A;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const float u = __shfl_up(L, off, 16);
      if (c >= off) L += u;
    }
    const float Llast = __shfl(L, lc - 1, 16);
    float Ls[4], ds[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      Ls[i] = __shfl(L, 4 * g + i, 16);
      ds[i] = __shfl(dl, 4 * g + i, 16);
    }
    __syncthreads();

    // CB^T[s][t] = B_s . C_t: lane holds t = c, s = 4g + i
    f32x4 cb = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const bf16x8 av = *reinterpret_cast<const bf16x8*>(sm.sB + c * Sm::RB + 32 * m + 8 * g);
      const bf16x8 bv = *reinterpret_cast<const bf16x8*>(sm.sC + c * Sm::RB + 32 * m + 8 * g);
      cb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, cb, 0, 0, 0);
    }
    // the within-chunk matrix M[t][s] (s <= t), D on its diagonal, as hi + lo operands
    s16x4 mhi, mlo;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = 4 * g + i;
      float v = s <= c ? expf(L - Ls[i]) * ds[i] * cb[i] : 0.0f;
      if (s == c) v += Dh;
      short hs, ls;
      split_bf16(v, hs, ls);
      mhi[i] = hs;
      mlo[i] = ls;
    }
    // readout of the carried state: Y^T[t][p] = sum_n C_t[n] state[p][n]; lane holds p, t = 4g + i
    f32x4 yacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const bf16x8 av = *reinterpret_cast<const bf16x8*>(sm.sC + c * Sm::RB + 32 * m + 8 * g);
      bf16x8 bhi, blo;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float v = st[2 * m + (k >> 2)][k & 3];
        short hs, ls;
        split_bf16(v, hs, ls);
        bhi[k] = __builtin_bit_cast(__bf16, hs);
        blo[k] = __builtin_bit_cast(__bf16, ls);
      }
      yacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bhi, yacc, 0, 0, 0);
      yacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, blo, yacc, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) yacc[i] *= expf(Ls[i]);
    // + sum_s M[t][s] x_s[p] (x exact in bf16)
    const s16x4 xv = *reinterpret_cast<const s16x4*>(sm.sXT + p * Sm::RT + 4 * g);
    yacc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(mhi, xv, yacc, 0, 0, 0);
    yacc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(mlo, xv, yacc, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 4 * g + i;
      if (t < lc) Y[(((size_t)b * S + t0 + t) * H + h) * P + p] = (uint16_t)bf16_bits(yacc[i]);
    }
    if (update) {
      // state <- e^{L_last} state + sum_s B_s[n] (w_s x_s[p]), w_s = e^{L_last - L_s} delta_s
      s16x4 whi, wlo;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = expf(Llast - Ls[i]) * ds[i] * bits_f32(xv[i]);
        short hs, ls;
        split_bf16(v, hs, ls);
        whi[i] = hs;
        wlo[i] = ls;
      }
      const float keep = expf(Llast);
#pragma unroll
      for (int T = 0; T < NT2; ++T) {
        st[T] *= keep;
        const s16x4 bt = *reinterpret_cast<const s16x4*>(sm.sBT + tile_col(T, c) * Sm::RT + 4 * g);
        st[T] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(bt, whi, st[T], 0, 0, 0);
        st[T] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(bt, wlo, st[T], 0, 0, 0);
      }
    }
    t0 += CH;
    if (t0 >= S) break;
    lc = min(CH, S - t0);
    chunk_load(cr, a, b, h, grp, t0, lc, tid, c);
    __syncthreads();  // the chunk's LDS reads are done before the next one is stored
  }
  if (want_state) {
    float* ho = a.h_out + ((size_t)bh * P + p) * N + 8 * g;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      *reinterpret_cast<float4*>(ho + 32 * m) = float4{st[2 * m][0], st[2 * m][1], st[2 * m][2], st[2 * m][3]};
      *reinterpret_cast<float4*>(ho + 32 * m + 4) =
          float4{st[2 * m + 1][0], st[2 * m + 1][1], st[2 * m + 1][2], st[2 * m + 1][3]};
    }
  }
}

// ---- vector-ALU path ----------------------------------------------------------------------

// NPT: state columns per thread (N / (256 / P)), a compile-time bound on the registers
template <typename T, int NPT>
__global__ __launch_bounds__(NT) void mamba2_scan_kernel(MambaArgs a) {
  // rows padded by one word: the chunk matrix reads 16 rows of B (and 4 of C) at one column
  __shared__ float sC[CH][kMambaMaxN + 1];
  __shared__ float sB[CH][kMambaMaxN + 1];
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

template <int NW>
hipError_t launch_mfma_nw(const MambaArgs& a, hipStream_t s) {
  const dim3 grid(a.B * a.H), block(64 * NW);
  switch (a.N) {
    case 32: hipLaunchKernelGGL((mamba2_scan_mfma_kernel<NW, 1>), grid, block, 0, s, a); break;
    case 64: hipLaunchKernelGGL((mamba2_scan_mfma_kernel<NW, 2>), grid, block, 0, s, a); break;
    case 128: hipLaunchKernelGGL((mamba2_scan_mfma_kernel<NW, 4>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

bool mfma_path(const MambaArgs& a, int dtype) {
  if (dtype != TT_BF16 || (a.P != 16 && a.P != 32 && a.P != 64 && a.P != 128)) return false;
  if (a.N != 32 && a.N != 64 && a.N != 128) return false;
  const uintptr_t bases = (uintptr_t)a.x | (uintptr_t)a.Bm | (uintptr_t)a.Cm;
  return bases % 16 == 0;
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
  if (mfma_path(a, dtype)) {
    switch (a.P) {
      case 16: return launch_mfma_nw<1>(a, s);
      case 32: return launch_mfma_nw<2>(a, s);
      case 64: return launch_mfma_nw<4>(a, s);
      default: return launch_mfma_nw<8>(a, s);
    }
  }
  return dtype == TT_BF16 ? launch_t<uint16_t>(a, s) : launch_t<float>(a, s);
}

}  // namespace tt
