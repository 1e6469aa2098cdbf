// LM head fused with the commit's vocabulary reduction, bf16, on gfx950 MFMA.
//
// What it computes: Nemotron-TwoTower (gist.science explainer), Technical Summary > Training
// and Conditioning > Sampling -- every still-masked position of the block is predicted at
// once from the denoiser's output, and confidence decides which are committed (the snilld.dk
// TwoTower article, "Blockwise generering i praksis"). Here the prediction's last step, the
// LM head, is computed and reduced in one pass: for every masked position (b,i) with hidden
// state h[b,i,0:K] and every vocabulary entry v with head row w[v,0:K],
//   l[b,i,v] = sum_k h[b,i,k] * w[v,k]      (bf16 inputs, fp32 accumulation)
// and, per 256-entry vocabulary chunk, the chunk max, the lowest index attaining it and
// sum_v exp(l_v - chunk max). The logits never reach memory. The commit's decide step then
// merges the chunks of each row (token, Z, conf = 1/Z) and applies the gamma rule.
//
// How (MI355X design):
//  * One workgroup = 256 head rows (a vocabulary tile) x 128 masked hidden rows (a row
//    group), 8 waves of 64 x 64, each wave a 2 x 2 block of v_mfma_f32_32x32x16_bf16 with
//    the head rows on the M side and the hidden rows on the N side (C^T = W H^T): both
//    operands are 16-byte row-major reads of K-contiguous rows. fp32 accumulators stay in
//    registers for the whole K loop.
//  * K runs in stages of 64 features (32 KB of head rows + 16 KB of hidden rows). The
//    loads run four stages ahead into registers (six 16-byte loads per lane per stage,
//    96 VGPRs in flight, about 2 us of matrix work: HBM latency under load is well past
//    what a three-stage LDS ring of 48 KB stages covers); each stage then goes from
//    registers into one of two LDS buffers (ds_write_b128, 1 KB per wave per load); one
//    barrier per stage. Each 128-byte LDS row holds its eight 16-byte chunks permuted by
//    slot = chunk ^ ((row/2)%8) (applied on the global side), so the 16 lanes of one
//    ds_read_b128 pass (16 consecutive rows, one chunk) hit 16 distinct bank groups.
//  * The masked rows are compacted inside the kernel (a ballot scan of the mask by every
//    workgroup), so the launch needs no host synchronisation; a row group past the number
//    of masked rows exits at once, and the last group pads with its first row (results
//    discarded).
//  * The row groups of one vocabulary tile are consecutive workgroups of one XCD (workgroup
//    id % 8 is its XCD), so they run together and the tile's head rows come from HBM once
//    and from that XCD's L2 for the others.
//  * Epilogue: each lane holds 32 logits of one row; a lane scans them in increasing
//    vocabulary order (max, lowest argmax), sums exp relative to its max, merges with the
//    lane holding the row's other 32 (lanes l, l^32), and the four waves of a row merge
//    through LDS in vocabulary order into the chunk record (z widened to fp64). A second
//    launch merges each masked row's chunk records (one workgroup per row) into one.
#include "tt_internal.h"

namespace tt {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4 gu32x4;  // global memory: no flat loads

constexpr int VT = kLmVocabPerWg;     // 256 head rows per workgroup
constexpr int RT = kLmRowsPerWg;      // 128 hidden rows per workgroup
constexpr int KS = kLmFeaturesPerStage;  // 64 features per stage
constexpr int ROWB = KS * 2;          // 128-byte LDS rows
constexpr int WTB = VT * ROWB;        // 32 KB of head rows per stage
constexpr int HTB = RT * ROWB;        // 16 KB of hidden rows per stage
constexpr int STB = WTB + HTB;        // 48 KB per stage
constexpr int NSTG = 2;               // LDS buffers
constexpr int NW = 8;
constexpr int NTHR = NW * 64;
constexpr int WDMA = WTB / 1024 / NW;  // 4 loads of head rows per lane per stage
constexpr int HDMA = HTB / 1024 / NW;  // 2 loads of hidden rows per lane per stage
constexpr int NCP = WDMA + HDMA;      // 16-byte loads per lane per stage
constexpr int P = 4;                  // stages held in registers (loads in flight)
constexpr float kLog2e = 1.4426950408889634f;

static_assert(RT == 2 * 64 && VT == 4 * 64, "waves: 2 row blocks x 4 vocabulary blocks of 64");
static_assert(ROWB * 8 == 1024, "one 16-byte load per lane = 8 LDS rows");
static_assert(NSTG * STB <= 160 * 1024 - 8 * 1024, "buffers and epilogue fit the LDS");

__shared__ __attribute__((aligned(1024))) char g_lds[NSTG * STB];
__shared__ int g_rows[RT];
__shared__ int g_wcnt[NW];

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const char*>((uintptr_t)((hi << 32) | lo));
}

// (m, tok, z) merge of two partials over disjoint vocabulary sets: larger max wins, equal
// maxima keep the lower index; z moves to the common max. An empty partial has m = -inf.
// The runner-up r (the largest value after the max, counting a repeated max) of a union of
// two sets is the largest of the two runners-up and the smaller maximum.
__device__ __forceinline__ void part_merge(float& m, int& tok, float& z, float& r, float m2, int tok2, float z2,
                                           float r2) {
  if (m2 == -INFINITY) return;
  if (m == -INFINITY) {
    m = m2;
    tok = tok2;
    z = z2;
    r = r2;
    return;
  }
  const float M = fmaxf(m, m2);
  z = z * exp2f((m - M) * kLog2e) + z2 * exp2f((m2 - M) * kLog2e);
  r = fmaxf(fmaxf(r, r2), fminf(m, m2));
  if (m2 > m || (m2 == m && tok2 < tok)) tok = tok2;
  m = M;
}

// STRAIGHT: K is a multiple of 64*P with at least 2P stages (the straight-line schedule).
template <bool STRAIGHT>
__global__ __launch_bounds__(NTHR, 1) void lmhead_reduce_kernel(LmHeadArgs a) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int id = blockIdx.x;
  const int xcd = id & 7, kk = id >> 3;
  const int rg = __builtin_amdgcn_readfirstlane(kk % a.NRG);
  const int vt = __builtin_amdgcn_readfirstlane((kk / a.NRG) * 8 + xcd);
  if (vt >= a.NVT) return;

  // ---- this row group's masked rows (ballot scan of the mask, in position order)
  const int BS = a.B * a.S;
  int total = 0;
  for (int p0 = 0; p0 < BS; p0 += NTHR) {
    const int p = p0 + tid;
    const bool m = p < BS && a.mask[p] != 0;
    const uint64_t bal = __ballot(m);
    const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
    if (lane == 0) g_wcnt[wave] = __popcll(bal);
    __syncthreads();
    int before = total, chunk = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int c = g_wcnt[w];
      before += w < wave ? c : 0;
      chunk += c;
    }
    const int idx = before + below - rg * RT;
    if (m && idx >= 0 && idx < RT) g_rows[idx] = p;
    total += chunk;
    __syncthreads();
  }
  const int nrows = __builtin_amdgcn_readfirstlane(min(RT, total - rg * RT));
  if (nrows <= 0) return;
  if (tid < RT && tid >= nrows) g_rows[tid] = g_rows[0];
  __syncthreads();

  // ---- load offsets (fixed per lane; the stage moves the scalar bases by 128 bytes)
  const size_t rowb = (size_t)a.K * 2;
  uint32_t woff[WDMA], hoff[HDMA];
#pragma unroll
  for (int i = 0; i < WDMA; ++i) {
    const int row = (wave * WDMA + i) * 8 + (lane >> 3);
    const int vrow = min(vt * VT + row, a.V - 1) - vt * VT;  // rows past V read the last row
    woff[i] = (uint32_t)((size_t)vrow * rowb) + ((((lane & 7) ^ swz(row))) << 4);
  }
#pragma unroll
  for (int j = 0; j < HDMA; ++j) {
    const int row = (wave * HDMA + j) * 8 + (lane >> 3);
    hoff[j] = (uint32_t)((size_t)g_rows[row] * rowb) + ((((lane & 7) ^ swz(row))) << 4);
  }
  const char* wbase = uniform_ptr(static_cast<const char*>(a.weight) + (size_t)vt * VT * rowb);
  const char* hbase = uniform_ptr(static_cast<const char*>(a.hidden));

  // stage s of this wave: 16 bytes per lane per copy, held in registers until written to LDS
  auto gload = [&](int s, u32x4 (&r)[NCP]) {
    const char* wb = wbase + (size_t)s * ROWB;
    const char* hb = hbase + (size_t)s * ROWB;
#pragma unroll
    for (int i = 0; i < WDMA; ++i) r[i] = *(gu32x4*)(wb + woff[i]);
#pragma unroll
    for (int j = 0; j < HDMA; ++j) r[WDMA + j] = *(gu32x4*)(hb + hoff[j]);
  };
  // this wave's part of a stage into LDS buffer q: copy i lands at rows (wave*WDMA+i)*8..
  auto lwrite = [&](int q, const u32x4 (&r)[NCP]) {
    char* ls = g_lds + q * STB + lane * 16;
#pragma unroll
    for (int i = 0; i < WDMA; ++i) *reinterpret_cast<u32x4*>(ls + (wave * WDMA + i) * 1024) = r[i];
#pragma unroll
    for (int j = 0; j < HDMA; ++j) *reinterpret_cast<u32x4*>(ls + WTB + (wave * HDMA + j) * 1024) = r[WDMA + j];
  };

  // ---- operand read offsets: wave (wr, wv) holds rows wr*64.. and vocabulary wv*64..
  const int wr = wave & 1, wv = wave >> 1;
  const int lr = lane & 31, lh = lane >> 5;
  int offA[KS / 16], offB[KS / 16];
  {
    const int ra = wv * 64 + lr, rb = wr * 64 + lr;  // +32 for the second block: same swizzle
#pragma unroll
    for (int ks = 0; ks < KS / 16; ++ks) {
      offA[ks] = ra * ROWB + (((2 * ks + lh) ^ swz(ra)) << 4);
      offB[ks] = WTB + rb * ROWB + (((2 * ks + lh) ^ swz(rb)) << 4);
    }
  }

  f32x16 acc[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.0f;

  // ---- K loop. Before iteration s, LDS buffer s%2 holds stage s (written, not yet
  // published) and registers rb[(s+1)%P], ... hold stages s+1 .. s+P (loads in flight).
  // Iteration s: barrier (stage s visible; every wave done with stage s-1's buffer), the
  // products of stage s, then stage s+1 from registers into the other buffer and the loads
  // of stage s+1+P into the registers it frees.
  const int NS = a.K / KS;
  u32x4 rb[P][NCP];
  gload(0, rb[0]);
  lwrite(0, rb[0]);
#pragma unroll
  for (int p = 1; p <= P; ++p)
    if (STRAIGHT || p < NS) gload(p, rb[p % P]);  // (straight: NS >= 2P, no guard)
  auto iter = [&](int s, u32x4 (&rnext)[NCP], bool write_next, bool load_ahead) {
    __syncthreads();
    const char* st = g_lds + (s & 1) * STB;
    // operands of step ks+1 are read while the products of step ks run
    bf16x8 op[2][4];
    auto ld = [&](int ks, bf16x8 (&o)[4]) {
      o[0] = *reinterpret_cast<const bf16x8*>(st + offA[ks]);
      o[1] = *reinterpret_cast<const bf16x8*>(st + offA[ks] + 32 * ROWB);
      o[2] = *reinterpret_cast<const bf16x8*>(st + offB[ks]);
      o[3] = *reinterpret_cast<const bf16x8*>(st + offB[ks] + 32 * ROWB);
    };
    ld(0, op[0]);
#pragma unroll
    for (int ks = 0; ks < KS / 16; ++ks) {
      if (ks + 1 < KS / 16) ld(ks + 1, op[(ks + 1) & 1]);
      const bf16x8(&o)[4] = op[ks & 1];
      acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o[0], o[2], acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o[0], o[3], acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o[1], o[2], acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o[1], o[3], acc[1][1], 0, 0, 0);
    }
    if (write_next) {
      lwrite((s + 1) & 1, rnext);
      if (load_ahead) gload(s + 1 + P, rnext);
    }
  };
  if constexpr (STRAIGHT) {
    // straight-line blocks of P stages (static register buffers, every load and write
    // unconditional in the loop, so each wait covers exactly the stage it needs): loads
    // stop after stage NS-1 (second-to-last block), writes after stage NS-1 (last block)
    int s = 0;
    for (; s < NS - 2 * P; s += P) {
#pragma unroll
      for (int u = 0; u < P; ++u) iter(s + u, rb[(u + 1) % P], true, true);
    }
#pragma unroll
    for (int u = 0; u < P; ++u) iter(s + u, rb[(u + 1) % P], true, u < P - 1);
    s += P;
#pragma unroll
    for (int u = 0; u < P; ++u) iter(s + u, rb[(u + 1) % P], u < P - 1, false);
  } else {
    // any other K: the same schedule with run-time guards (the compiler then waits for every
    // load in flight before each write)
    for (int s = 0; s < NS; s += P) {
#pragma unroll
      for (int u = 0; u < P; ++u)
        if (s + u < NS) iter(s + u, rb[(u + 1) % P], s + u + 1 < NS, s + u + 1 + P < NS);
    }
  }
  __syncthreads();  // the buffers are reused for the epilogue's partials

  // ---- epilogue. acc[mb][nb][i]: row wr*64 + nb*32 + lr, vocabulary entry
  // vt*256 + wv*64 + mb*32 + 8*(i/4) + 4*lh + i%4 (increasing in (mb, i)).
  float* pm = reinterpret_cast<float*>(g_lds);
  int* pt = reinterpret_cast<int*>(g_lds + RT * 4 * 4);
  float* pz = reinterpret_cast<float*>(g_lds + RT * 4 * 8);
  float* pr = reinterpret_cast<float*>(g_lds + RT * 4 * 12);
  const int v0 = vt * VT + wv * 64 + 4 * lh;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    float m = -INFINITY, rr = -INFINITY;  // max and runner-up
    int tok = 0x7fffffff;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int v = v0 + mb * 32 + 8 * (i >> 2) + (i & 3);
        const float x = acc[mb][nb][i];
        if (v < a.V) {
          if (x > m) {
            rr = m;
            m = x;
            tok = v;
          } else {
            rr = fmaxf(rr, x);
          }
        }
      }
    // exp of (x - m): the difference first, so the max term is exactly 1 and each exponent's
    // rounding is relative to x - m (a scaled m would carry the rounding of m * log2 e)
    float z = 0.0f;
    if (m != -INFINITY) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int v = v0 + mb * 32 + 8 * (i >> 2) + (i & 3);
          if (v < a.V) z += exp2f((acc[mb][nb][i] - m) * kLog2e);
        }
    }
    const float m2 = __shfl_xor(m, 32);
    const int t2 = __shfl_xor(tok, 32);
    const float z2 = __shfl_xor(z, 32);
    const float r2 = __shfl_xor(rr, 32);
    part_merge(m, tok, z, rr, m2, t2, z2, r2);
    if (lh == 0) {
      const int r = wr * 64 + nb * 32 + lr;
      pm[r * 4 + wv] = m;
      pt[r * 4 + wv] = tok;
      pz[r * 4 + wv] = z;
      pr[r * 4 + wv] = rr;
    }
  }
  __syncthreads();
  if (tid < nrows) {
    float m = pm[tid * 4], rr = pr[tid * 4];
    int tok = pt[tid * 4];
    double z = pz[tid * 4];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const float m2 = pm[tid * 4 + w];
      if (m2 == -INFINITY) continue;
      const double z2 = pz[tid * 4 + w];
      const float r2 = pr[tid * 4 + w];
      if (m == -INFINITY) {
        m = m2;
        tok = pt[tid * 4 + w];
        z = z2;
        rr = r2;
        continue;
      }
      const float M = fmaxf(m, m2);
      z = z * exp((double)m - (double)M) + z2 * exp((double)m2 - (double)M);
      rr = fmaxf(fmaxf(rr, r2), fminf(m, m2));
      if (m2 > m) tok = pt[tid * 4 + w];  // equal maxima keep the earlier (lower) block
      m = M;
    }
    CommitChunk c;
    c.m = m;
    c.tok = tok;
    c.z = z;
    const size_t at = (size_t)g_rows[tid] * a.NVT + vt;
    a.chunks[at] = c;
    a.runner[at] = rr;
  }
}

// Merge of a masked row's NVT chunk records into one (the decide step then reads one record
// per row): 256 threads, each merges its chunks (k = t, t + 256, ...) in fp64, then the
// workgroup merges the threads' partials; larger max wins, equal maxima keep the lower index
// (an order-free rule), z moves to the common max in fp64. The row's runner-up logit is
// merged alongside. In exact mode (a weight bound is given) the workgroup also bounds the
// error of the row's fp32 logits: each is a sum of K exact bf16 products accumulated in fp32
// in some order, so it lies within 2 K 2^-24 sum_k |h_k w_vk| (a factor 2 covers a rounding
// that is not to nearest) <= 2 K 2^-24 ||h||_2 max_v ||w_v||_2 of the exact value.
constexpr int MT = 256;

__device__ __forceinline__ void merge_d(float& m, int& tok, double& z, float& r, float m2, int tok2, double z2,
                                        float r2) {
  if (m2 == -INFINITY) return;
  if (m == -INFINITY) {
    m = m2;
    tok = tok2;
    z = z2;
    r = r2;
    return;
  }
  const float M = fmaxf(m, m2);
  z = z * exp((double)m - (double)M) + z2 * exp((double)m2 - (double)M);
  r = fmaxf(fmaxf(r, r2), fminf(m, m2));
  if (m2 > m || (m2 == m && tok2 < tok)) tok = tok2;
  m = M;
}

__global__ __launch_bounds__(MT) void lmhead_merge_kernel(LmHeadArgs a) {
  __shared__ float sm[MT / 64], sr[MT / 64];
  __shared__ int st[MT / 64];
  __shared__ double sz[MT / 64], sh[MT / 64];
  const int row = blockIdx.x, tid = threadIdx.x;
  if (row == 0 && tid == 0 && a.count) *a.count = 0;  // the flag step's counter
  if (!a.mask[row]) return;
  const CommitChunk* c = a.chunks + (size_t)row * a.NVT;
  const float* rc = a.runner + (size_t)row * a.NVT;
  float m = -INFINITY, r = -INFINITY;
  int tok = 0x7fffffff;
  double z = 0.0;
  for (int k = tid; k < a.NVT; k += MT) merge_d(m, tok, z, r, c[k].m, c[k].tok, c[k].z, rc[k]);
  // (exact mode) ||h||_2^2 of the row, in fp64 (each square of a bf16 value is exact)
  double hh = 0.0;
  if (a.w_bound) {
    const uint16_t* h = static_cast<const uint16_t*>(a.hidden) + (size_t)row * a.K;
    for (int k = tid; k < a.K; k += MT) {
      const double x = (double)__uint_as_float(((uint32_t)h[k]) << 16);
      hh = fma(x, x, hh);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float m2 = __shfl_xor(m, off);
    const int t2 = __shfl_xor(tok, off);
    const double z2 = __shfl_xor(z, off);
    const float r2 = __shfl_xor(r, off);
    merge_d(m, tok, z, r, m2, t2, z2, r2);
    hh += __shfl_xor(hh, off);
  }
  if ((tid & 63) == 0) {
    sm[tid >> 6] = m;
    st[tid >> 6] = tok;
    sz[tid >> 6] = z;
    sr[tid >> 6] = r;
    sh[tid >> 6] = hh;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < MT / 64; ++w) merge_d(m, tok, z, r, sm[w], st[w], sz[w], sr[w]);
    CommitChunk rec;
    rec.m = m;
    rec.tok = tok;
    rec.z = z;
    a.merged[row] = rec;
    if (a.w_bound) {
      const double hn = sqrt((sh[0] + sh[1]) + (sh[2] + sh[3]));
      // the bound's own rounding (a few fp64 operations) is covered by the factor 1 + 1e-12
      const double eps = 2.0 * (double)a.K * 0x1p-24 * hn * (double)*a.w_bound * (1.0 + 1e-12);
      a.rowx[2 * (size_t)row] = (double)r;
      a.rowx[2 * (size_t)row + 1] = eps;
    }
  }
}

}  // namespace

hipError_t launch_lmhead_reduce(const LmHeadArgs& a, hipStream_t s) {
  const int groups = (a.NVT + 7) / 8;
  const int NS = a.K / KS;
  if (NS % P == 0 && NS >= 2 * P)
    hipLaunchKernelGGL(lmhead_reduce_kernel<true>, dim3(8 * a.NRG * groups), dim3(NTHR), 0, s, a);
  else
    hipLaunchKernelGGL(lmhead_reduce_kernel<false>, dim3(8 * a.NRG * groups), dim3(NTHR), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_lmhead_merge(const LmHeadArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(lmhead_merge_kernel, dim3(a.B * a.S), dim3(MT), 0, s, a);
  return hipGetLastError();
}

}  // namespace tt
