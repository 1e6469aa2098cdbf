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
//    with v_mfma_f32_32x32x16_bf16. Each of the 4 waves of a workgroup owns 64 query rows
//    (two 32-column MFMA blocks, so every K/V operand read from LDS feeds two products);
//    256 rows per workgroup, one workgroup per CU. A unit with more rows is covered by NQ
//    workgroups (a "cluster") placed on one XCD so that its key stream is fetched from
//    HBM once and shared through that XCD's L2.
//  * Keys of a unit are the concatenation [context ; block]; the key sequence is cut in
//    64-key tiles. All tiles of all units form one global list that is split evenly over
//    the clusters of a persistent grid (the plan is computed in-kernel from ctx_len).
//    A cluster range that covers a whole unit writes the final output; a unit cut by a
//    range boundary leaves per-piece partials (running max and sum in fp32, normalised O
//    in bf16) that the combine kernel merges with a log-sum-exp rescale.
//  * K and V tiles go HBM -> LDS directly (global_load_lds_dwordx4, no staging registers)
//    into a ring of 8 stages of 16 KB (32-key tiles): up to seven tiles, ~112 KB of reads,
//    are in flight per CU while one is computed; one barrier per tile, explicit vmcnt waits.
//    Each 256-byte LDS row holds its 16-byte chunks permuted by slot = chunk ^ f(row),
//    f(row) = 2*(row%8) + (row/8)%2 (the permutation is applied on the global side of
//    the copy). With it the K operand reads (ds_read_b128, 16 rows per phase) and the
//    transposing V operand reads (ds_read_b64_tr_b16, 4 rows x 2 chunks per phase) are
//    bank-conflict free; per-lane read offsets are precomputed, the row block and key
//    step are immediate offsets.
//  * The score accumulator layout of the first MFMA is consumed directly as the P operand
//    of the second (no shuffles): the V^T operand is read in the matching key order.
//  * Online softmax in the log2 domain; row max reduced across the two lane halves with
//    v_permlane32_swap; the running max is only moved (and O rescaled) when a tile's max
//    exceeds it by more than 2^8, which leaves the result unchanged and skips most
//    rescales. Only the unit's last tile carries the key mask (a wave-uniform branch).
//    Keys past ctx_len + S read the block's last row (finite data) and are masked to -inf.
//  * Built with IEEE mode off (no NaN reaches this kernel: padding is never read and the
//    masked scores are -inf), so the row max is a plain v_max3 chain without the NaN
//    quieting that IEEE mode adds to every operand.
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
constexpr int ROWB = D * 2;                   // 256-byte LDS rows
constexpr int TB = KT * ROWB;                 // 16 KB per tensor tile
constexpr int STAGEB = 2 * TB;                // K tile then V tile
constexpr int NW = kAttnWaves;                // 4 waves
constexpr int NTHR = NW * 64;                 // 256 threads
constexpr int RPW = kAttnRowsPerWave;         // 64 query rows per wave
constexpr int NB = RPW / 32;                  // 2 MFMA column blocks per wave
constexpr int RWG = kAttnRowsPerWg;           // 256 query rows per workgroup
constexpr int DMA_PER_TENSOR = TB / 1024 / NW;  // 2 one-KB copies per wave per tensor
constexpr int DMA_PER_TILE = 2 * DMA_PER_TENSOR;
constexpr int NSTAGE = 8;                     // LDS ring: up to 7 tiles in flight
constexpr float kLazy = 8.0f;                 // log2 headroom before the running max moves

static_assert(NSTAGE * STAGEB >= (kMaxB + 1) * 4, "tile plan must fit in the ring");
static_assert(NB == 2, "two column blocks per wave");

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__shared__ __attribute__((aligned(1024))) char g_ring[NSTAGE * STAGEB];

__device__ __forceinline__ int swz(int row) { return ((row & 7) << 1) | ((row >> 3) & 1); }

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

// the same value, held in a scalar register (b is wave-uniform at every call site below)
__device__ __forceinline__ int clamp_ctx_u(const int32_t* ctx_len, int b, int Lmax) {
  return __builtin_amdgcn_readfirstlane(clamp_ctx(ctx_len, b, Lmax));
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
  int before = 0, total = 0;
  for (int k = 0; k < NW; ++k) {
    before += (k < w) ? wsum[k] : 0;
    total += wsum[k];
  }
  int run = before + x - local;
  for (int k = 0; k < per; ++k) {
    const int b = b0 + k;
    if (b < B) {
      P[b] = run;
      run += ((clamp_ctx(ctx_len, b, Lmax) + S + KT - 1) / KT) * Hkv;
    }
  }
  if (tid == 0) P[B] = total;
  __syncthreads();
}

// Source rows of one unit for the tile copies. This lane copies, for i = 0..1, the 16-byte
// chunk c_i of tile row 8*wave + 4*i + lane/16 (c_i = (lane%16) ^ f(row)).
struct TileSrc {
  const char* kc;   // k_ctx row 0 of this unit (bytes; row stride rs)
  const char* vc;
  const char* kb;   // k_blk row 0 of this unit
  const char* vb;
  size_t rs;        // Hkv * D * 2 bytes
  int nctx, S;
  int coff[DMA_PER_TENSOR];  // c_i * 16
};

// One 16-byte-per-lane global -> LDS copy (global_load_lds_dwordx4): lane i's 16 bytes land
// at LDS byte lds + 16 i. Written as asm so that the compiler's own wait insertion does not
// treat every later LDS read as dependent on it (it would wait for all copies in flight);
// completion is awaited explicitly (vmcnt) before the barrier that publishes a stage. The
// copy has no register result; its address registers are consumed at issue.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds)
               : "memory", "m0");
}

// Issue the DMA copies of tile t into stage st: key j < ctx_len reads context row j, else
// block row j - ctx_len; keys past ctx_len + S read the last block row (finite data whose
// scores are masked). One wave-uniform LDS destination per copy (1 KB = 4 rows).
__device__ __forceinline__ void issue_tile(const TileSrc& s, int t, char* st) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < DMA_PER_TENSOR; ++i) {
    const int row = (KT / NW) * w + 4 * i;
    const int key = t * KT + row + (lane >> 4);
    const bool in_ctx = key < s.nctx;
    const int idx = in_ctx ? key : min(key - s.nctx, s.S - 1);
    const size_t off = (size_t)idx * s.rs + s.coff[i];
    const char* kp = (in_ctx ? s.kc : s.kb) + off;
    const char* vp = (in_ctx ? s.vc : s.vb) + off;
    const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(st + row * ROWB));
    dma16(kp, lds);
    dma16(vp, lds + TB);
  }
}

// wait until at most n vector-memory operations of this wave are outstanding (n <= 63)
#define TT_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0x70 | 0xF00)

__device__ __forceinline__ void wait_tiles_after(int n_after) {
  // n_after: tiles whose copies were issued after the one to be consumed (0..NSTAGE-2)
  switch (n_after) {
    case 0: TT_WAIT_VM(0); break;
    case 1: TT_WAIT_VM(1 * DMA_PER_TILE); break;
    case 2: TT_WAIT_VM(2 * DMA_PER_TILE); break;
    case 3: TT_WAIT_VM(3 * DMA_PER_TILE); break;
    case 4: TT_WAIT_VM(4 * DMA_PER_TILE); break;
    case 5: TT_WAIT_VM(5 * DMA_PER_TILE); break;
    default: TT_WAIT_VM(6 * DMA_PER_TILE); break;
  }
}
static_assert(NSTAGE - 2 == 6, "wait table covers NSTAGE - 2 tiles after");

__device__ __forceinline__ bf16x8 ld_k(const char* p) { return *reinterpret_cast<const bf16x8*>(p); }

__device__ __forceinline__ bf16x8 ld_v(const char* lo_p, const char* hi_p) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lo_p));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(hi_p));
  const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
  return __builtin_bit_cast(bf16x8, u32x4{lo2[0], lo2[1], hi2[0], hi2[1]});
}

struct WaveState {
  f32x16 oacc[D / 32][NB];
  float m_run[NB], l_run[NB];
};

struct LaneOffsets {
  int k[D / 16];          // K operand, d-step ds: row lr, chunk (2 ds + lh) ^ f(lr)
  int v[D / 32][2];       // V^T operand, head-dim block db, row half (+0 / +8)
};

// One 32-key tile for this wave's 64 query rows (two column blocks). mask: the unit's
// last tile (wave-uniform).
__device__ __forceinline__ void compute_tile(const char* st, const LaneOffsets& lo,
                                             const bf16x8 (&qreg)[NB][D / 16], WaveState& w,
                                             float scale_log2, int key0, int nvalid, int lh,
                                             bool mask) {
  // S^T[key][query] = K Q^T for the column blocks nb; each K operand feeds both column
  // blocks; operands are read two d-steps ahead
  f32x16 s[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int k = 0; k < 16; ++k) s[nb][k] = 0.0f;
  constexpr int NDS = D / 16;
  bf16x8 ka[NDS];
  ka[0] = ld_k(st + lo.k[0]);
  ka[1] = ld_k(st + lo.k[1]);
#pragma unroll
  for (int ds = 0; ds < NDS; ++ds) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      s[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ds], qreg[nb][ds], s[nb], 0, 0, 0);
    if (ds + 2 < NDS) ka[ds + 2] = ld_k(st + lo.k[ds + 2]);
  }
  if (mask) {  // keys past ctx_len + S; lim is opaque so the compares stay in this branch
    int lim = nvalid - key0 - 4 * lh;
    asm volatile("" : "+v"(lim));
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int o = 8 * (k >> 2) + (k & 3);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        if (o >= lim) s[nb][k] = -INFINITY;
    }
  }
  // per column block: running max, lazy rescale, P = exp2(s*scale_log2 - m) packed as the
  // B operand of the PV products (key-step ks = k/8 holds the values k%8)
  bf16x8 pb[NB][2];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float mx = s[nb][0];
#pragma unroll
    for (int k = 1; k < 16; ++k) mx = __builtin_fmaxf(mx, s[nb][k]);
    mx = lane_pair_max(mx) * scale_log2;
    if (__any(mx > w.m_run[nb] + kLazy)) {
      const float mn = fmaxf(w.m_run[nb], mx);
      const float alpha = __builtin_amdgcn_exp2f(w.m_run[nb] - mn);
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int k = 0; k < 16; ++k) w.oacc[db][nb][k] *= alpha;
      w.l_run[nb] *= alpha;
      w.m_run[nb] = mn;
    }
    float psum = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float p = __builtin_amdgcn_exp2f(s[nb][k] * scale_log2 - w.m_run[nb]);
      psum += p;
      pb[nb][k >> 3][k & 7] = (__bf16)p;
    }
    w.l_run[nb] += psum;
  }
  // O^T[d][query] += V^T P^T; each V operand feeds both column blocks
  const char* vt = st + TB;
  bf16x8 va = ld_v(vt + lo.v[0][0], vt + lo.v[0][1]);
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int nks = (db + 1 < D / 32) ? ks : ks + 1;
      const int ndb = (db + 1 < D / 32) ? db + 1 : 0;
      bf16x8 vn = va;
      if (nks < 2) vn = ld_v(vt + lo.v[ndb][0] + nks * 16 * ROWB, vt + lo.v[ndb][1] + nks * 16 * ROWB);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        w.oacc[db][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[nb][ks], w.oacc[db][nb], 0, 0, 0);
      va = vn;
    }
}

// Partial slot of one (cluster, segment, query slice): O/l as bf16 [RWG][D], then m, l fp32.
constexpr size_t kPartBytes = (size_t)RWG * D * 2 + (size_t)RWG * 8;

__device__ __forceinline__ char* part_slot(const AttnArgs& a, int cluster, int slot, int qsl) {
  return reinterpret_cast<char*>(a.part) + ((size_t)(cluster * 2 + slot) * a.NQ + qsl) * kPartBytes;
}

__global__ __launch_bounds__(NTHR, 1) void attn_mfma_kernel(AttnArgs a) {
  __shared__ int wsum[NW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, lh = lane >> 5;
  const int id = blockIdx.x;
  const int xcd = id & 7, kk = id >> 3;
  const int cluster = (kk / a.NQ) * 8 + xcd;
  const int qs = kk % a.NQ;

  // ---- plan: tile prefix sums in LDS, then this cluster's range of the global tile list
  int* P = reinterpret_cast<int*>(g_ring);
  build_plan(P, wsum, a.ctx_len, a.B, a.S, a.Hkv, a.Lmax);
  const int T = __builtin_amdgcn_readfirstlane(P[a.B]);
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
  int pb = __builtin_amdgcn_readfirstlane(P[bcur]);
  bcur = __builtin_amdgcn_readfirstlane(bcur);
  __syncthreads();  // P lives in the ring; done with it
  if (t0 >= t1) return;

  const uint16_t* Q = static_cast<const uint16_t*>(a.q);
  uint16_t* O = static_cast<uint16_t*>(a.o);
  const int G = a.G, S = a.S, rows_unit = G * S;

  // this lane's LDS read offsets within a stage
  LaneOffsets lo;
  {
    const int fk = swz(lr);
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) lo.k[ds] = lr * ROWB + (((2 * ds + lh) ^ fk) << 4);
    const int j = lane & 15, grp2 = (lane >> 4) & 1;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 4 * lh + (j >> 2) + 8 * h;
      const int fv = swz(row);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int c = 4 * db + 2 * grp2 + ((j & 3) >> 1);
        lo.v[db][h] = row * ROWB + ((c ^ fv) << 4) + (j & 1) * 8;
      }
    }
  }

  int t = t0;
  bool first_seg = true;
  int nctx = clamp_ctx_u(a.ctx_len, bcur, a.Lmax);
  int nt = (nctx + S + KT - 1) / KT;
  while (t < t1) {
    while (t >= pb + nt * a.Hkv) {  // advance to the sequence holding tile t
      pb += nt * a.Hkv;
      ++bcur;
      nctx = clamp_ctx_u(a.ctx_len, bcur, a.Lmax);
      nt = (nctx + S + KT - 1) / KT;
    }
    const int g = __builtin_amdgcn_readfirstlane((t - pb) / nt);
    const int ta = __builtin_amdgcn_readfirstlane((t - pb) - g * nt);  // first local tile
    const int ustart = pb + g * nt;
    const int te = __builtin_amdgcn_readfirstlane(min(nt, t1 - ustart));  // one past the last
    const bool whole = (ta == 0 && te == nt);
    const int slot = first_seg ? 0 : 1;
    first_seg = false;
    t = ustart + te;
    const int nvalid = nctx + S;

    TileSrc src;
    {
      const size_t rsb = (size_t)a.Hkv * D * 2;
      src.rs = rsb;
      src.kc = static_cast<const char*>(a.k_ctx) + ((size_t)bcur * a.Lmax * a.Hkv + g) * D * 2;
      src.vc = static_cast<const char*>(a.v_ctx) + ((size_t)bcur * a.Lmax * a.Hkv + g) * D * 2;
      src.kb = static_cast<const char*>(a.k_blk) + ((size_t)bcur * S * a.Hkv + g) * D * 2;
      src.vb = static_cast<const char*>(a.v_blk) + ((size_t)bcur * S * a.Hkv + g) * D * 2;
      src.nctx = nctx;
      src.S = S;
#pragma unroll
      for (int i = 0; i < DMA_PER_TENSOR; ++i)
        src.coff[i] = (((lane & 15) ^ swz(((KT / NW) * wave + 4 * i + (lane >> 4)) & 15)) << 4);
    }

    // prologue: the first NSTAGE-1 tiles of the segment in flight
    for (int k = 0; k < NSTAGE - 1 && ta + k < te; ++k) issue_tile(src, ta + k, g_ring + k * STAGEB);

    // ---- this wave's query rows: row r of the unit is (head-in-group r / S, position r % S)
    bf16x8 qreg[NB][D / 16];
    size_t qoff[NB];
    bool rvalid[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int r = qs * RWG + wave * RPW + nb * 32 + lr;
      rvalid[nb] = r < rows_unit;
      const int hl = rvalid[nb] ? r / S : 0, pos = rvalid[nb] ? r - hl * S : 0;
      qoff[nb] = (((size_t)bcur * S + pos) * a.Hq + (size_t)g * G + hl) * D;
#pragma unroll
      for (int ds = 0; ds < D / 16; ++ds) {
        u32x4 v = rvalid[nb] ? *reinterpret_cast<const u32x4*>(Q + qoff[nb] + ds * 16 + lh * 8)
                             : u32x4{0, 0, 0, 0};
        qreg[nb][ds] = __builtin_bit_cast(bf16x8, v);
      }
    }

    // the query loads must not be left pending into the tile loop: the compiler would
    // otherwise place a wait for them inside the loop, where the copies in flight are
    // younger and the wait would drain them too
    TT_WAIT_VM(0);


    WaveState ws;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int k = 0; k < 16; ++k) ws.oacc[db][nb][k] = 0.0f;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      ws.m_run[nb] = -INFINITY;
      ws.l_run[nb] = 0.0f;
    }

    // ring of NSTAGE stages: tile ta+u lives in stage u % NSTAGE
    for (int tt = ta; tt < te; ++tt) {
      const int u = (tt - ta) & (NSTAGE - 1);
      wait_tiles_after(__builtin_amdgcn_readfirstlane(min(NSTAGE - 2, te - 1 - tt)));
      __syncthreads();
      if (tt + NSTAGE - 1 < te)
        issue_tile(src, tt + NSTAGE - 1, g_ring + ((u + NSTAGE - 1) & (NSTAGE - 1)) * STAGEB);
      compute_tile(g_ring + u * STAGEB, lo, qreg, ws, a.scale_log2, tt * KT, nvalid, lh, tt == nt - 1);
    }
    __syncthreads();  // every wave is done with the stages before the next segment's copies

    // ---- epilogue: O / l (bf16) to the output, or with m and l to a partial slot
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float lt = lane_pair_sum(ws.l_run[nb]);
      const float inv = 1.0f / lt;
      uint16_t* orow;
      if (whole) {
        orow = rvalid[nb] ? O + qoff[nb] : nullptr;
      } else {
        char* base = part_slot(a, cluster, slot, qs);
        const int rw = wave * RPW + nb * 32 + lr;
        orow = reinterpret_cast<uint16_t*>(base) + (size_t)rw * D;
        if (lh == 0) {
          float* ml = reinterpret_cast<float*>(base + (size_t)RWG * D * 2);
          ml[rw] = ws.m_run[nb];
          ml[RWG + rw] = lt;
        }
      }
      if (orow) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            bf16x4 v;
#pragma unroll
            for (int k = 0; k < 4; ++k) v[k] = (__bf16)(ws.oacc[db][nb][q4 * 4 + k] * inv);
            const int d = db * 32 + 8 * q4 + 4 * lh;
            *reinterpret_cast<u32x2*>(orow + d) = __builtin_bit_cast(u32x2, v);
          }
      }
    }
  }
}

// Merge the partials of every unit that a cluster boundary cut. One workgroup covers 8 query
// rows of one unit (32 threads x 4 head-dim values per row); one pass with a running max.
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
  float M = -INFINITY, L = 0.0f, o0 = 0.0f, o1 = 0.0f, o2 = 0.0f, o3 = 0.0f;
  for (int c = c_first; c <= c_last; ++c) {
    const int r0 = (int)(((long long)c * T) / a.NC);
    if (r0 == (int)(((long long)(c + 1) * T) / a.NC)) continue;  // empty range (T < NC)
    const int slot = (start <= r0) ? 0 : 1;
    const char* base = part_slot(a, c, slot, qsl);
    const float* ml = reinterpret_cast<const float*>(base + (size_t)RWG * D * 2);
    const float m = ml[rw], l = ml[RWG + rw];
    const u32x2 raw = *reinterpret_cast<const u32x2*>(base + ((size_t)rw * D + d) * 2);
    const bf16x4 v = __builtin_bit_cast(bf16x4, raw);
    const float mn = fmaxf(M, m);
    const float sa = __builtin_amdgcn_exp2f(M - mn);  // 0 on the first piece
    const float sb = __builtin_amdgcn_exp2f(m - mn) * l;
    L = L * sa + sb;
    o0 = o0 * sa + sb * (float)v[0];
    o1 = o1 * sa + sb * (float)v[1];
    o2 = o2 * sa + sb * (float)v[2];
    o3 = o3 * sa + sb * (float)v[3];
    M = mn;
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

size_t attn_part_bytes(int nc, int nq) { return (size_t)nc * 2 * nq * kPartBytes; }

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
