// Denoiser block attention, bf16, head dim 128, on gfx950 MFMA.
//
// What it computes: Nemotron-TwoTower (gist.science explainer), Technical Summary >
// Methodology > Architecture and > Generation Process -- every block query of sequence b
// and query head h attends, in ONE softmax, to the frozen context tower's same-layer keys
// k_ctx[b, 0:ctx_len[b], g] followed by the block's own keys k_blk[b, 0:S, g] (no mask
// inside the block), g = h / G. Values likewise; scale 1/sqrt(D).
//
// How (MI355X design):
//  * A unit is one (sequence b, KV head g). All G*S query rows of a unit read the same
//    keys, so they are packed as the N side of the MFMAs: S^T = K Q^T and O^T += V^T P^T
//    with v_mfma_f32_32x32x16_bf16. Each wave owns 32 query rows, a workgroup 128, and a
//    unit with more rows is covered by NQ workgroups (a "cluster") placed on one XCD so
//    that the cluster's key stream is fetched from HBM once and shared through that XCD's
//    L2.
//  * Keys of a unit are the concatenation [context ; block]; the key sequence is cut in
//    64-key tiles. All tiles of all units form one global list that is split evenly over
//    the clusters of a persistent grid (the plan is computed in-kernel from ctx_len).
//    A cluster range that covers a whole unit writes the final output; a unit cut by a
//    range boundary leaves per-piece partials (running max, sum, unnormalised O) that the
//    combine kernel merges with a log-sum-exp rescale.
//  * K and V tiles are staged HBM -> registers -> LDS (double-buffered, one barrier per
//    tile) in the same row-major layout, 16-byte chunks XOR-swizzled by row so that the
//    K operand reads (ds_read_b128) and the transposing V operand reads
//    (ds_read_b64_tr_b16) are bank-conflict free. The score accumulator layout of the
//    first MFMA is consumed directly as the P operand of the second (no shuffles): the
//    V^T operand is read in the matching key order.
//  * Online softmax in the log2 domain; row max reduced across the two lane halves with
//    v_permlane32_swap; the running max is only moved (and O rescaled) when a tile's max
//    exceeds it by more than 2^8, which leaves the result unchanged and skips most
//    rescales.
//  * Context rows at or past ctx_len are never loaded; keys past ctx_len+S in the last
//    tile are zero-filled and masked to -inf.
#include "tt_internal.h"

namespace tt {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int KT = kAttnKeysPerTile;          // 64 keys per tile
constexpr int D = kAttnMfmaD;                 // 128
constexpr int ROWB = D * 2;                   // 256 bytes per key row
constexpr int TILEB = KT * ROWB;              // 16 KB per tensor per tile
constexpr int RWG = kAttnRowsPerWg;           // 128 query rows per workgroup
constexpr int NTHR = kAttnWaves * 64;         // 256 threads
constexpr int CHUNKS_PER_THREAD = KT * (D / 8) / NTHR;  // 4 x 16-byte chunks per tensor
constexpr float kLazy = 8.0f;                 // log2 headroom before the running max moves

static_assert(CHUNKS_PER_THREAD * NTHR == KT * (D / 8), "tile split");

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * ROWB + ((chunk ^ (row & 15)) << 4);
}

__device__ __forceinline__ float lane_pair_max(float v) {
  // lanes l and l^32 hold the same query column; the swap hands each lane both halves
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float lane_pair_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ int clamp_ctx(const int32_t* ctx_len, int b, int Lmax) {
  int n = ctx_len[b];
  return n < 0 ? 0 : (n > Lmax ? Lmax : n);
}

// Exclusive prefix sums over sequences of (tiles per unit * Hkv) into P[0..B]; P[B] = total.
__device__ void build_plan(int* P, int* wsum, const int32_t* ctx_len, int B, int S, int Hkv,
                           int Lmax) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int per = (B + NTHR - 1) / NTHR;
  const int b0 = tid * per;
  int local = 0;
  for (int k = 0; k < per; ++k) {
    const int b = b0 + k;
    if (b < B) local += ((clamp_ctx(ctx_len, b, Lmax) + S + KT - 1) / KT) * Hkv;
  }
  int x = local;
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  int before = 0;
  for (int k = 0; k < w; ++k) before += wsum[k];
  int run = before + x - local;
  for (int k = 0; k < per; ++k) {
    const int b = b0 + k;
    if (b < B) {
      P[b] = run;
      run += ((clamp_ctx(ctx_len, b, Lmax) + S + KT - 1) / KT) * Hkv;
    }
  }
  if (tid == 0) P[B] = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  __syncthreads();
}

struct TileSrc {
  const uint16_t* kc;
  const uint16_t* vc;
  const uint16_t* kb;
  const uint16_t* vb;
  int b, g, nctx, nvalid, S, Hkv, Lmax;
};

// Global loads of one K and one V tile (4 + 4 chunks of 16 bytes per thread).
__device__ __forceinline__ void load_tile(const TileSrc& s, int t, u32x4 (&kr)[CHUNKS_PER_THREAD],
                                          u32x4 (&vr)[CHUNKS_PER_THREAD]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int r = 0; r < CHUNKS_PER_THREAD; ++r) {
    const int id = tid + r * NTHR;
    const int row = id >> 4, c = id & 15;
    const int key = t * KT + row;
    const uint16_t *kp, *vp;
    if (key < s.nctx) {
      const size_t off = ((size_t)(s.b * s.Lmax + key) * s.Hkv + s.g) * D + c * 8;
      kp = s.kc + off;
      vp = s.vc + off;
    } else if (key < s.nvalid) {
      const size_t off = ((size_t)(s.b * s.S + (key - s.nctx)) * s.Hkv + s.g) * D + c * 8;
      kp = s.kb + off;
      vp = s.vb + off;
    } else {
      kp = vp = nullptr;
    }
    if (kp) {
      kr[r] = *reinterpret_cast<const u32x4*>(kp);
      vr[r] = *reinterpret_cast<const u32x4*>(vp);
    } else {
      kr[r] = u32x4{0, 0, 0, 0};
      vr[r] = u32x4{0, 0, 0, 0};
    }
  }
}

__device__ __forceinline__ void store_tile(char* kbuf, char* vbuf, const u32x4 (&kr)[CHUNKS_PER_THREAD],
                                           const u32x4 (&vr)[CHUNKS_PER_THREAD]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int r = 0; r < CHUNKS_PER_THREAD; ++r) {
    const int id = tid + r * NTHR;
    const int row = id >> 4, c = id & 15;
    *reinterpret_cast<u32x4*>(kbuf + swz(row, c)) = kr[r];
    *reinterpret_cast<u32x4*>(vbuf + swz(row, c)) = vr[r];
  }
}

__global__ __launch_bounds__(NTHR, 1) void attn_mfma_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[4 * TILEB];  // K0 V0 K1 V1
  __shared__ int wsum[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, lh = lane >> 5;
  const int id = blockIdx.x;
  const int xcd = id & 7, kk = id >> 3;
  const int cluster = (kk / a.NQ) * 8 + xcd;
  const int qs = kk % a.NQ;

  // ---- plan: tile prefix sums in LDS, then this cluster's range of the global tile list
  int* P = reinterpret_cast<int*>(smem);
  build_plan(P, wsum, a.ctx_len, a.B, a.S, a.Hkv, a.Lmax);
  const int T = P[a.B];
  if (id == 0)
    for (int b = tid; b <= a.B; b += NTHR) a.plan[b] = P[b];
  const int t0 = (int)(((long long)cluster * T) / a.NC);
  const int t1 = (int)(((long long)(cluster + 1) * T) / a.NC);
  int bcur = 0;
  {
    int lo = 0, hi = a.B - 1;  // largest b with P[b] <= t0
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (P[mid] <= t0) lo = mid; else hi = mid - 1;
    }
    bcur = lo;
  }
  int pb = P[bcur];
  __syncthreads();  // P lives in the tile buffers; done with it
  if (t0 >= t1) return;

  const uint16_t* Q = static_cast<const uint16_t*>(a.q);
  uint16_t* O = static_cast<uint16_t*>(a.o);
  const int G = a.G, S = a.S, rows_unit = G * S;

  TileSrc src;
  src.kc = static_cast<const uint16_t*>(a.k_ctx);
  src.vc = static_cast<const uint16_t*>(a.v_ctx);
  src.kb = static_cast<const uint16_t*>(a.k_blk);
  src.vb = static_cast<const uint16_t*>(a.v_blk);
  src.S = S;
  src.Hkv = a.Hkv;
  src.Lmax = a.Lmax;

  int t = t0;
  bool first_seg = true;
  int nctx = clamp_ctx(a.ctx_len, bcur, a.Lmax);
  int nt = (nctx + S + KT - 1) / KT;
  while (t < t1) {
    while (t >= pb + nt * a.Hkv) {  // advance to the sequence holding tile t
      pb += nt * a.Hkv;
      ++bcur;
      nctx = clamp_ctx(a.ctx_len, bcur, a.Lmax);
      nt = (nctx + S + KT - 1) / KT;
    }
    const int g = (t - pb) / nt;
    const int ta = (t - pb) - g * nt;                  // first local tile of the segment
    const int ustart = pb + g * nt;
    const int te = min(nt, t1 - ustart);               // one past the last local tile
    const bool whole = (ta == 0 && te == nt);
    const int slot = first_seg ? 0 : 1;
    first_seg = false;
    t = ustart + te;

    src.b = bcur;
    src.g = g;
    src.nctx = nctx;
    src.nvalid = nctx + S;

    // ---- this wave's 32 query rows: row r of the unit is (head-in-group r / S, position r % S)
    const int r = qs * RWG + wave * 32 + lr;
    const bool rvalid = r < rows_unit;
    const int hl = rvalid ? r / S : 0, pos = rvalid ? r - hl * S : 0;
    const size_t qoff = (((size_t)bcur * S + pos) * a.Hq + (size_t)g * G + hl) * D;
    bf16x8 qreg[D / 16];
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
      u32x4 v = rvalid ? *reinterpret_cast<const u32x4*>(Q + qoff + ds * 16 + lh * 8) : u32x4{0, 0, 0, 0};
      qreg[ds] = __builtin_bit_cast(bf16x8, v);
    }

    f32x16 oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int k = 0; k < 16; ++k) oacc[db][k] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f;

    u32x4 kr[CHUNKS_PER_THREAD], vr[CHUNKS_PER_THREAD];
    load_tile(src, ta, kr, vr);
    store_tile(smem, smem + TILEB, kr, vr);
    __syncthreads();

    for (int tt = ta; tt < te; ++tt) {
      const int cur = (tt - ta) & 1;
      const bool more = tt + 1 < te;
      if (more) load_tile(src, tt + 1, kr, vr);
      const char* Kb = smem + cur * 2 * TILEB;
      const char* Vb = Kb + TILEB;

      // S^T[key][query] = K Q^T over two 32-key blocks
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int k = 0; k < 16; ++k) sacc[kb][k] = 0.0f;
        const int row = kb * 32 + lr;
#pragma unroll
        for (int ds = 0; ds < D / 16; ++ds) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(Kb + swz(row, 2 * ds + lh));
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[ds], sacc[kb], 0, 0, 0);
        }
      }
      if (tt == nt - 1) {  // keys past ctx_len + S in the unit's last tile
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int k = 0; k < 16; ++k) {
            const int key = tt * KT + kb * 32 + 8 * (k >> 2) + 4 * lh + (k & 3);
            if (key >= src.nvalid) sacc[kb][k] = -INFINITY;
          }
      }
      float mx = sacc[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int k = 0; k < 16; ++k) mx = fmaxf(mx, sacc[kb][k]);
      mx = lane_pair_max(mx) * a.scale_log2;
      if (__any(mx > m_run + kLazy)) {
        const float mn = fmaxf(m_run, mx);
        const float alpha = exp2f(m_run - mn);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int k = 0; k < 16; ++k) oacc[db][k] *= alpha;
        l_run *= alpha;
        m_run = mn;
      }
      // P = exp2(s*scale_log2 - m) packed as the B operand of the PV products:
      // key-step ks = 2*kb + k/8 holds the 8 values k%8 of accumulator half k/8
      bf16x8 pb8[4];
      float psum = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const float p = exp2f(sacc[kb][k] * a.scale_log2 - m_run);
          psum += p;
          pb8[2 * kb + (k >> 3)][k & 7] = (__bf16)p;
        }
      l_run += psum;

      // O^T[d][query] += V^T P^T ; the V^T operand is read transposed from the row-major
      // tile: lane i of each 16-lane group receives d = base + i for 4 keys per read
      const int grp2 = (lane >> 4) & 1, j = lane & 15;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int vrow = ks * 16 + 4 * lh + (j >> 2);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const int d = db * 32 + grp2 * 16 + 4 * (j & 3);
          const int boff = (d & 7) * 2;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4*)(Vb + swz(vrow, d >> 3) + boff));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4*)(Vb + swz(vrow + 8, d >> 3) + boff));
          const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
          const bf16x8 va = __builtin_bit_cast(bf16x8, u32x4{lo2[0], lo2[1], hi2[0], hi2[1]});
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb8[ks], oacc[db], 0, 0, 0);
        }
      }

      if (more) store_tile(smem + (cur ^ 1) * 2 * TILEB, smem + (cur ^ 1) * 2 * TILEB + TILEB, kr, vr);
      __syncthreads();
    }

    // ---- epilogue
    const float lt = lane_pair_sum(l_run);
    if (whole) {
      if (rvalid) {
        const float inv = 1.0f / lt;
        uint16_t* orow = O + qoff;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            bf16x4 v;
#pragma unroll
            for (int k = 0; k < 4; ++k) v[k] = (__bf16)(oacc[db][q4 * 4 + k] * inv);
            const int d = db * 32 + 8 * q4 + 4 * lh;
            *reinterpret_cast<u32x2*>(orow + d) = __builtin_bit_cast(u32x2, v);
          }
      }
    } else {
      float* base = a.part + ((size_t)(cluster * 2 + slot) * a.NQ + qs) * (size_t)(RWG * (D + 2));
      const int rw = wave * 32 + lr;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d = db * 32 + 8 * q4 + 4 * lh;
          float4 v = make_float4(oacc[db][q4 * 4 + 0], oacc[db][q4 * 4 + 1], oacc[db][q4 * 4 + 2],
                                 oacc[db][q4 * 4 + 3]);
          *reinterpret_cast<float4*>(base + (size_t)rw * D + d) = v;
        }
      if (lh == 0) {
        base[RWG * D + rw] = m_run;
        base[RWG * D + RWG + rw] = lt;
      }
    }
  }
}

// Merge the partials of every unit that a cluster boundary cut. One workgroup covers 8 query
// rows of one unit (32 threads x 4 head-dim values per row).
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  const int u = blockIdx.x;
  const int b = u / a.Hkv, g = u - b * a.Hkv;
  const int rows_unit = a.G * a.S;
  const int r = blockIdx.y * 8 + (threadIdx.x >> 5);
  const int d = (threadIdx.x & 31) * 4;
  const int T = a.plan[a.B];
  const int pb = a.plan[b];
  const int nt = (a.plan[b + 1] - pb) / a.Hkv;
  const int start = pb + g * nt, end = start + nt;
  // cluster c owns [c*T/NC, (c+1)*T/NC); the one holding tile x is ceil((x+1)*NC/T) - 1
  const int c_first = (int)((((long long)start + 1) * a.NC + T - 1) / T) - 1;
  const int c_last = (int)((((long long)end) * a.NC + T - 1) / T) - 1;
  if (c_first == c_last) return;  // one cluster saw the whole unit and wrote it already
  if (r >= rows_unit) return;
  const int qsl = r / RWG, rw = r - qsl * RWG;
  float M = -INFINITY;
  for (int c = c_first; c <= c_last; ++c) {
    const int r0 = (int)(((long long)c * T) / a.NC);
    if (r0 == (int)(((long long)(c + 1) * T) / a.NC)) continue;  // empty range (T < NC)
    const int slot = (start <= r0) ? 0 : 1;
    const float* base = a.part + ((size_t)(c * 2 + slot) * a.NQ + qsl) * (size_t)(RWG * (D + 2));
    M = fmaxf(M, base[RWG * D + rw]);
  }
  float L = 0.0f, o0 = 0.0f, o1 = 0.0f, o2 = 0.0f, o3 = 0.0f;
  for (int c = c_first; c <= c_last; ++c) {
    const int r0 = (int)(((long long)c * T) / a.NC);
    if (r0 == (int)(((long long)(c + 1) * T) / a.NC)) continue;
    const int slot = (start <= r0) ? 0 : 1;
    const float* base = a.part + ((size_t)(c * 2 + slot) * a.NQ + qsl) * (size_t)(RWG * (D + 2));
    const float w = exp2f(base[RWG * D + rw] - M);
    L += w * base[RWG * D + RWG + rw];
    const float4 v = *reinterpret_cast<const float4*>(base + (size_t)rw * D + d);
    o0 += w * v.x;
    o1 += w * v.y;
    o2 += w * v.z;
    o3 += w * v.w;
  }
  const float inv = 1.0f / L;
  const int hl = r / a.S, pos = r - hl * a.S;
  uint16_t* orow = static_cast<uint16_t*>(a.o) +
                   (((size_t)b * a.S + pos) * a.Hq + (size_t)g * a.G + hl) * D + d;
  bf16x4 v;
  v[0] = (__bf16)(o0 * inv);
  v[1] = (__bf16)(o1 * inv);
  v[2] = (__bf16)(o2 * inv);
  v[3] = (__bf16)(o3 * inv);
  *reinterpret_cast<u32x2*>(orow) = __builtin_bit_cast(u32x2, v);
}

}  // namespace

hipError_t launch_attn_mfma(const AttnArgs& a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  if (ev0) (void)hipEventRecord(ev0, s);
  hipLaunchKernelGGL(attn_mfma_kernel, dim3(a.NC * a.NQ), dim3(NTHR), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ev1) (void)hipEventRecord(ev1, s);
  const int rows_unit = a.G * a.S;
  hipLaunchKernelGGL(attn_combine_kernel, dim3(a.B * a.Hkv, (rows_unit + 7) / 8), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace tt
