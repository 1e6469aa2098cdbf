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
//    32-key tiles. All tiles of all units form one global list that is split evenly over
//    the clusters of a persistent grid (the plan is computed in-kernel from ctx_len).
//    A cluster range that covers a whole unit writes the final output; a unit cut by a
//    range boundary leaves per-piece partials (running max and sum in fp32, normalised O
//    in bf16) that the combine kernel merges with a log-sum-exp rescale.
//  * K and V tiles go HBM -> LDS directly (global_load_lds_dwordx4, no staging registers)
//    into a ring of 8 stages of 16 KB (8 KB of keys + 8 KB of values): up to six tiles
//    are in flight per CU while two are in use; one barrier per tile, explicit vmcnt
//    waits. The query rows of a segment arrive the same way (through four of the stages)
//    so that the first tile's wait does not also wait for the rest of the prologue.
//    Each 256-byte LDS row holds its 16-byte chunks permuted by slot = chunk ^ f(row),
//    f(row) = 4*(row%4) + (row/4)%4 (the permutation is applied on the global side of
//    the copy). The K operand reads (ds_read_b128) serve 16 lanes = 16 consecutive rows
//    per pass: f is a bijection on them, so one chunk column lands on all 64 banks. The
//    transposing V operand reads (ds_read_b64_tr_b16) serve 32 lanes = 4 consecutive
//    rows x one aligned group of 4 chunks per pass: f/4 = row%4 sends the 4 rows to 4
//    different chunk groups. Both are bank-conflict free (measured with the LDS bank
//    conflict counter); per-lane read offsets are precomputed.
//  * The score accumulator layout of the first MFMA is consumed directly as the P operand
//    of the second (no shuffles): the V^T operand is read in the matching key order.
//  * Software pipeline, one wave per SIMD: while the matrix core runs the QK products of
//    tile t+1, the same wave's VALU computes the softmax of tile t (exp2, row sums, bf16
//    packing); the PV products of tile t then overlap the row maxima of tile t+1. The
//    loop is unrolled by two so that the score registers of consecutive tiles alternate
//    without copies.
//  * Online softmax in the log2 domain; row max reduced across the two lane halves with
//    v_permlane32_swap; the running max is only moved (and O rescaled) when a tile's max
//    exceeds it by more than 2^8, which leaves the result unchanged and skips most
//    rescales. Only the unit's last tile carries the key mask (a wave-uniform branch).
//    Keys past ctx_len + S read the block's last row (finite data) and are masked to -inf.
//  * The epilogue stages each wave's O tile through LDS and writes whole 256-byte rows.
//  * Built with IEEE mode off (no NaN reaches this kernel: padding is never read and the
//    masked scores are -inf), so the row max is a plain v_max3 chain without the NaN
//    quieting that IEEE mode adds to every operand.
#include "tt_internal.h"

namespace tt {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int KT = kAttnKeysPerTile;          // 32 keys per tile
constexpr int D = kAttnMfmaD;                 // 128
constexpr int ROWB = D * 2;                   // 256-byte LDS rows
constexpr int TB = KT * ROWB;                 // 8 KB per tensor tile
constexpr int STAGEB = 2 * TB;                // K tile then V tile
constexpr int NW = kAttnWaves;                // 4 waves
constexpr int NTHR = NW * 64;                 // 256 threads
constexpr int RPW = kAttnRowsPerWave;         // 64 query rows per wave
constexpr int NB = RPW / 32;                  // 2 MFMA column blocks per wave
constexpr int RWG = kAttnRowsPerWg;           // 256 query rows per workgroup
constexpr int DMA_PER_TENSOR = TB / 1024 / NW;  // 2 one-KB copies per wave per tensor
constexpr int DMA_PER_TILE = 2 * DMA_PER_TENSOR;
constexpr int DMA_Q = RPW * ROWB / 1024;      // 16 one-KB copies for a wave's query rows
constexpr int NSTAGE = 8;                     // LDS ring
constexpr int NPRO = 4;                       // tiles issued before the query rows are read
constexpr int OROWB = ROWB + 16;              // padded row of the epilogue staging
constexpr float kLazy = 8.0f;                 // log2 headroom before the running max moves

static_assert(NSTAGE * STAGEB >= (kMaxB + 1) * 4, "tile plan must fit in the ring");
static_assert(NB == 2, "two column blocks per wave");
static_assert(RPW * ROWB == STAGEB, "a wave's query rows fill one stage");
static_assert(NPRO + NW == NSTAGE, "query rows use the stages after the prologue tiles");
static_assert(NW * RPW * OROWB <= NSTAGE * STAGEB, "epilogue staging fits in the ring");

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__shared__ __attribute__((aligned(1024))) char g_ring[NSTAGE * STAGEB];

__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

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

// The same value for a wave-uniform b, read with a scalar load (through the constant
// address space: ctx_len is not written while the kernel runs). A vector load here would
// make the compiler wait on the vector-memory counter, i.e. also for the epilogue stores
// and tile copies in flight.
typedef const __attribute__((address_space(4))) int32_t c_i32;
__device__ __forceinline__ int clamp_ctx_u(const int32_t* ctx_len, int b, int Lmax) {
  const int n = ((c_i32*)(uintptr_t)ctx_len)[b];
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
  uint32_t voff[DMA_PER_TENSOR];  // (tile row of copy i of this lane) * rs + c_i * 16
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

// The same copy from a wave-uniform base (scalar registers) plus a 32-bit per-lane offset.
__device__ __forceinline__ void dma16s(const char* base, uint32_t voff, uint32_t lds) {
  // the two halves through scalar registers; readfirstlane yields a signed int, so each
  // half is taken as uint32_t before widening (a sign-extended low half would corrupt
  // the high word)
  const uint64_t v = (uint64_t)(uintptr_t)base;
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  base = reinterpret_cast<const char*>((uintptr_t)((hi << 32) | lo));
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 offset:0" ::"v"(voff),
               "s"(base), "s"(lds)
               : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)p);
}

// Issue the DMA copies of tile t into stage st: key j < ctx_len reads context row j, else
// block row j - ctx_len; keys past ctx_len + S read the last block row (finite data whose
// scores are masked). One wave-uniform LDS destination per copy (1 KB = 4 rows).
__device__ __forceinline__ void issue_tile(const TileSrc& s, int t, char* st) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if ((t + 1) * KT <= __builtin_amdgcn_readfirstlane(s.nctx)) {
    // every key in the context: scalar bases, fixed lane offsets
    const size_t toff = (size_t)t * KT * s.rs;
#pragma unroll
    for (int i = 0; i < DMA_PER_TENSOR; ++i) {
      const uint32_t lds = lds_addr(st + ((KT / NW) * w + 4 * i) * ROWB);
      dma16s(s.kc + toff, s.voff[i], lds);
      dma16s(s.vc + toff, s.voff[i], lds + TB);
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < DMA_PER_TENSOR; ++i) {
    const int row = (KT / NW) * w + 4 * i;
    const int key = t * KT + row + (lane >> 4);
    const bool in_ctx = key < s.nctx;
    const int idx = in_ctx ? key : min(key - s.nctx, s.S - 1);
    const size_t off = (size_t)idx * s.rs + s.coff[i];
    const char* kp = (in_ctx ? s.kc : s.kb) + off;
    const char* vp = (in_ctx ? s.vc : s.vb) + off;
    const uint32_t lds = lds_addr(st + row * ROWB);
    dma16(kp, lds);
    dma16(vp, lds + TB);
  }
}

// wait until at most n vector-memory operations of this wave are outstanding (n <= 63)
#define TT_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0x70 | 0xF00)
// wait until this wave's LDS reads and writes are done
#define TT_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(0xC07F)

__device__ __forceinline__ void wait_tiles_after(int n_after) {
  // n_after: tiles whose copies were issued after the one to be consumed (0..6)
  if (n_after == 5) {  // the steady state of the tile loop
    TT_WAIT_VM(5 * DMA_PER_TILE);
    return;
  }
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

constexpr int NDS = D / 16;       // K operands per tile (d-steps)
constexpr int NVO = 2 * (D / 32);  // V^T operands per tile, index i = ks * 4 + db

// K operands of one 32-key tile (one ds_read_b128 per d-step)
__device__ __forceinline__ void load_k(const char* st, const LaneOffsets& lo, bf16x8 (&ka)[NDS]) {
#pragma unroll
  for (int ds = 0; ds < NDS; ++ds) ka[ds] = ld_k(st + lo.k[ds]);
}

// V^T operands of one tile (two ds_read_b64_tr_b16 each)
__device__ __forceinline__ void load_v(const char* st, const LaneOffsets& lo, bf16x8 (&va)[NVO]) {
  const char* vt = st + TB;
#pragma unroll
  for (int i = 0; i < NVO; ++i)
    va[i] = ld_v(vt + lo.v[i % 4][0] + (i / 4) * 16 * ROWB, vt + lo.v[i % 4][1] + (i / 4) * 16 * ROWB);
}

// S^T[key][query] = K Q^T of one 32-key tile for this wave's two column blocks; each K
// operand feeds both.
__device__ __forceinline__ void qk_mfma(const bf16x8 (&ka)[NDS], const bf16x8 (&qreg)[NB][D / 16],
                                        f32x16 (&s)[NB]) {
  const f32x16 zero = {};
#pragma unroll
  for (int ds = 0; ds < NDS; ++ds)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      s[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ds], qreg[nb][ds], ds == 0 ? zero : s[nb], 0, 0, 0);
}

__device__ __forceinline__ void qk_tile(const char* st, const LaneOffsets& lo,
                                        const bf16x8 (&qreg)[NB][D / 16], f32x16 (&s)[NB]) {
  bf16x8 ka[NDS];
  load_k(st, lo, ka);
  qk_mfma(ka, qreg, s);
}

// keys at or past nvalid get -inf (the unit's last tile only)
__device__ __forceinline__ void mask_tile(f32x16 (&s)[NB], int key0, int nvalid, int lh) {
  int lim = nvalid - key0 - 4 * lh;
  asm volatile("" : "+v"(lim));  // keeps the compares inside the (rarely taken) branch
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int o = 8 * (k >> 2) + (k & 3);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      if (o >= lim) s[nb][k] = -INFINITY;
  }
}

// row max of a tile in the log2 domain (scale_log2 > 0 commutes with max)
__device__ __forceinline__ void tile_max(const f32x16 (&s)[NB], float scale_log2, float (&mx)[NB]) {
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float m = s[nb][0];
#pragma unroll
    for (int k = 1; k < 16; ++k) m = __builtin_fmaxf(m, s[nb][k]);
    mx[nb] = lane_pair_max(m) * scale_log2;
  }
}

// move the running max (and rescale O and l) where a tile's max exceeds it by > 2^kLazy
__device__ __forceinline__ void rescale(WaveState& w, const float (&mx)[NB]) {
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    if (__any(mx[nb] > w.m_run[nb] + kLazy)) {
      const float mn = fmaxf(w.m_run[nb], mx[nb]);
      const float alpha = __builtin_amdgcn_exp2f(w.m_run[nb] - mn);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        // O lives in accumulation registers; the hints keep the allocator from moving it
        // (for this rare VALU update) into the registers the tile loop needs
        asm volatile("" : "+a"(w.oacc[db][nb]));
#pragma unroll
        for (int k = 0; k < 16; ++k) w.oacc[db][nb][k] *= alpha;
        asm volatile("" : "+a"(w.oacc[db][nb]));
      }
      w.l_run[nb] *= alpha;
      w.m_run[nb] = mn;
    }
  }
}

// P = exp2(s * scale_log2 - m), packed as the B operand of the PV products (key-step
// ks = k / 8 holds the values k % 8); row sums into l
__device__ __forceinline__ void softmax_tile(const f32x16 (&s)[NB], WaveState& w, float scale_log2,
                                             bf16x8 (&pb)[NB][2]) {
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int k = 0; k < 16; ++k)
      pb[nb][k >> 3][k & 7] = (__bf16)__builtin_amdgcn_exp2f(s[nb][k] * scale_log2 - w.m_run[nb]);
    // row sums of the bf16-rounded P, i.e. of exactly the weights the PV products use,
    // two values per dot instruction
    float ps0 = 0.0f, ps1 = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x2* pp = reinterpret_cast<const bf16x2*>(&pb[nb][ks]);
      ps0 = __builtin_amdgcn_fdot2_f32_bf16(pp[0], ones, ps0, false);
      ps1 = __builtin_amdgcn_fdot2_f32_bf16(pp[1], ones, ps1, false);
      ps0 = __builtin_amdgcn_fdot2_f32_bf16(pp[2], ones, ps0, false);
      ps1 = __builtin_amdgcn_fdot2_f32_bf16(pp[3], ones, ps1, false);
    }
    w.l_run[nb] += ps0 + ps1;
  }
}

// O^T[d][query] += V^T P^T; each V operand feeds both column blocks
__device__ __forceinline__ void pv_mfma(const bf16x8 (&va)[NVO], const bf16x8 (&pb)[NB][2], WaveState& w) {
#pragma unroll
  for (int i = 0; i < NVO; ++i)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      w.oacc[i % 4][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i], pb[nb][i / 4], w.oacc[i % 4][nb], 0, 0, 0);
}

// Per-segment loop state.
struct Seg {
  TileSrc src;
  LaneOffsets lo;
  float scale_log2;
  int ta, te, nt, nvalid, lh;
};

__device__ __forceinline__ char* stage_of(const Seg& g, int t) {
  return g_ring + ((t - g.ta) & (NSTAGE - 1)) * STAGEB;
}

// One pipeline step: softmax and PV of tile t (scores in s, row max in mx); with NEXT also
// the QK products of tile t+1 into sn and its row max into mx. The segment's last step
// (NEXT false) applies the key mask when its tile is the unit's last one, and takes that
// tile's max again; the other steps are one branch-free block after the rescale check, in
// which the scheduler interleaves the two tiles' work.
template <bool NEXT>
__device__ __forceinline__ void step(const Seg& g, const bf16x8 (&qreg)[NB][D / 16], WaveState& ws,
                                     f32x16 (&s)[NB], f32x16 (&sn)[NB], float (&mx)[NB], int t) {
  if (NEXT) {
    // tile t+1 complete for every wave; tiles issued after it: up to t+6
    wait_tiles_after(__builtin_amdgcn_readfirstlane(min(5, g.te - 2 - t)));
    __syncthreads();
  } else if (__builtin_amdgcn_readfirstlane(t) == g.nt - 1) {
    mask_tile(s, t * KT, g.nvalid, g.lh);
    tile_max(s, g.scale_log2, mx);
  }
  rescale(ws, mx);

  // The step body is written in issue order; sched_barrier keeps the compiler's
  // scheduler from regrouping it. Each QK product of tile t+1 is followed by one piece of
  // the softmax of tile t and by LDS operand reads spread over the phase: the K operands
  // three d-steps ahead of their products, the V operands of tile t one per product (all
  // in registers by the PV phase). Reads spread this way keep the LDS queue short: a
  // wave stalled on a full LDS command queue cannot issue the arithmetic behind it.
  const char* kst = stage_of(g, t + 1);
  const char* vst = stage_of(g, t) + TB;
  bf16x8 ka[NDS], va[NVO];
  constexpr int KAHEAD = 3;
  if (NEXT) {
#pragma unroll
    for (int ds = 0; ds < KAHEAD; ++ds) ka[ds] = ld_k(kst + g.lo.k[ds]);
  }
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  bf16x8 pb[NB][2];
  float psum[NB][2] = {{0.0f, 0.0f}, {0.0f, 0.0f}};
  const f32x16 zero = {};
  auto piece = [&](int i) {  // scores 2*(i%8), 2*(i%8)+1 of column block i/8
    const int nb = i >> 3, k = 2 * (i & 7);
    const float p0 = __builtin_amdgcn_exp2f(s[nb][k] * g.scale_log2 - ws.m_run[nb]);
    const float p1 = __builtin_amdgcn_exp2f(s[nb][k + 1] * g.scale_log2 - ws.m_run[nb]);
    bf16x2 pp;
    pp[0] = (__bf16)p0;
    pp[1] = (__bf16)p1;
    pb[nb][k >> 3][k & 7] = pp[0];
    pb[nb][k >> 3][(k & 7) + 1] = pp[1];
    psum[nb][i & 1] = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, psum[nb][i & 1], false);
  };
  constexpr int NPC = 16, LEAD = 2;
#pragma unroll
  for (int i = 0; i < LEAD; ++i) piece(i);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < NDS * NB; ++i) {
    if (NEXT) {
      const int ds = i >> 1, nb = i & 1;
      sn[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ds], qreg[nb][ds], ds == 0 ? zero : sn[nb], 0, 0, 0);
      if (nb == 1 && ds + KAHEAD < NDS) ka[ds + KAHEAD] = ld_k(kst + g.lo.k[ds + KAHEAD]);
    }
    if (i + LEAD < NPC) piece(i + LEAD);
    if (i < NVO) va[i] = ld_v(vst + g.lo.v[i % 4][0] + (i / 4) * 16 * ROWB, vst + g.lo.v[i % 4][1] + (i / 4) * 16 * ROWB);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) ws.l_run[nb] += psum[nb][0] + psum[nb][1];

  // PV products of tile t. The scores of tile t+1 move to VGPRs in quarters (once, for
  // its max and the next step's softmax) and are reduced to row maxima in between, late
  // enough that its QK products have completed: column block 0 after PV product 4,
  // column block 1 after product 9.
  float mpart[NB];
#pragma unroll
  for (int j = 0; j < NVO * NB; ++j) {
    const int i = j >> 1, nb = j & 1;
    ws.oacc[i % 4][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i], pb[nb][i / 4], ws.oacc[i % 4][nb], 0, 0, 0);
    if (NEXT) {
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
        const int q = j - (4 + 5 * cb);  // quarter of column block cb handled after product j
        if (q >= 0 && q < 4) {
          f32x4 v = {sn[cb][4 * q], sn[cb][4 * q + 1], sn[cb][4 * q + 2], sn[cb][4 * q + 3]};
          asm volatile("" : "+v"(v));
#pragma unroll
          for (int k = 0; k < 4; ++k) sn[cb][4 * q + k] = v[k];
          const float m4 = __builtin_fmaxf(__builtin_fmaxf(v[0], v[1]), __builtin_fmaxf(v[2], v[3]));
          mpart[cb] = q == 0 ? m4 : __builtin_fmaxf(mpart[cb], m4);
        }
        if (q == 4) mx[cb] = lane_pair_max(mpart[cb]) * g.scale_log2;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // the copies of tile t+7 (its stage held tile t-1, which every wave finished before
  // this step's barrier); issued after the products so that a stalled issue of the
  // copies delays no arithmetic of this step
  if (NEXT && t + NSTAGE - 1 < g.te) issue_tile(g.src, t + NSTAGE - 1, stage_of(g, t + NSTAGE - 1));
}

// Partial slot of one (cluster, segment, query slice): O/l as bf16 [RWG][D], then m, l fp32.
constexpr size_t kPartBytes = (size_t)RWG * D * 2 + (size_t)RWG * 8;

__device__ __forceinline__ char* part_slot(const AttnArgs& a, int cluster, int slot, int qsl) {
  return reinterpret_cast<char*>(a.part) + ((size_t)(cluster * 2 + slot) * a.NQ + qsl) * kPartBytes;
}

// byte offset of query row r of unit (b, g) in q / o ([B, S, Hq, D] bf16)
__device__ __forceinline__ size_t qrow_bytes(const AttnArgs& a, int b, int g, int r) {
  const int hl = r / a.S, pos = r - hl * a.S;
  return ((((size_t)b * a.S + pos) * a.Hq + (size_t)g * a.G + hl) * D) * 2;
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

  const char* Qb = static_cast<const char*>(a.q);
  char* Ob = static_cast<char*>(a.o);
  const int G = a.G, S = a.S, rows_unit = G * S;

  Seg sg;
  sg.scale_log2 = a.scale_log2;
  sg.lh = lh;
  {
    const int fk = swz(lr);
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) sg.lo.k[ds] = lr * ROWB + (((2 * ds + lh) ^ fk) << 4);
    const int j = lane & 15, grp2 = (lane >> 4) & 1;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 4 * lh + (j >> 2) + 8 * h;
      const int fv = swz(row);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int c = 4 * db + 2 * grp2 + ((j & 3) >> 1);
        sg.lo.v[db][h] = row * ROWB + ((c ^ fv) << 4) + (j & 1) * 8;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < DMA_PER_TENSOR; ++i) {
    const int row = (KT / NW) * wave + 4 * i + (lane >> 4);
    sg.src.coff[i] = ((lane & 15) ^ swz(row & 15)) << 4;
    sg.src.voff[i] = (uint32_t)(row * a.Hkv * D * 2 + sg.src.coff[i]);
  }

  int t = t0;
  bool first_seg = true;
  int nctx = clamp_ctx_u(a.ctx_len, bcur, a.Lmax);
  int nt = (nctx + S + KT - 1) / KT;
  while (t < t1) {
    while (t >= pb + nt * a.Hkv) {  // advance to the sequence holding tile t
      pb = __builtin_amdgcn_readfirstlane(pb + nt * a.Hkv);
      bcur = __builtin_amdgcn_readfirstlane(bcur + 1);
      nctx = clamp_ctx_u(a.ctx_len, bcur, a.Lmax);
      nt = __builtin_amdgcn_readfirstlane((nctx + S + KT - 1) / KT);
    }
    const int g = __builtin_amdgcn_readfirstlane((t - pb) / nt);
    const int ta = __builtin_amdgcn_readfirstlane((t - pb) - g * nt);  // first local tile
    const int ustart = pb + g * nt;
    const int te = __builtin_amdgcn_readfirstlane(min(nt, t1 - ustart));  // one past the last
    const bool whole = (ta == 0 && te == nt);
    const int slot = first_seg ? 0 : 1;
    first_seg = false;
    t = ustart + te;
    const int n = te - ta;  // tiles in this segment (>= 1)
    // an opaque copy of the lane id: the per-lane addresses of the prologue and epilogue
    // are then computed here rather than hoisted out of the segment loop and kept live
    // (in registers the tile loop needs) across it
    int ln = lane;
    asm volatile("" : "+v"(ln));

    sg.ta = ta;
    sg.te = te;
    sg.nt = nt;
    sg.nvalid = nctx + S;
    {
      const size_t rsb = (size_t)a.Hkv * D * 2;
      sg.src.rs = rsb;
      sg.src.kc = static_cast<const char*>(a.k_ctx) + ((size_t)bcur * a.Lmax * a.Hkv + g) * D * 2;
      sg.src.vc = static_cast<const char*>(a.v_ctx) + ((size_t)bcur * a.Lmax * a.Hkv + g) * D * 2;
      sg.src.kb = static_cast<const char*>(a.k_blk) + ((size_t)bcur * S * a.Hkv + g) * D * 2;
      sg.src.vb = static_cast<const char*>(a.v_blk) + ((size_t)bcur * S * a.Hkv + g) * D * 2;
      sg.src.nctx = nctx;
      sg.src.S = S;
    }

    // ---- prologue. Query rows of this wave -> stage NPRO + wave (row j of the wave at LDS
    // row j, chunks permuted like the key tiles); row r of the unit is (head-in-group r / S,
    // position r % S); rows past the unit read its row 0 (results discarded).
    const int row0 = qs * RWG + wave * RPW;  // this wave's first unit row
    {
      char* qst = g_ring + (NPRO + wave) * STAGEB;
#pragma unroll
      for (int i = 0; i < DMA_Q; ++i) {
        const int j = 4 * i + (ln >> 4);
        const int r = row0 + j;
        const int c = (ln & 15) ^ swz(j & 15);
        dma16(Qb + qrow_bytes(a, bcur, g, r < rows_unit ? r : 0) + (c << 4), lds_addr(qst + 4 * i * ROWB));
      }
    }
    const int npro = min(n, NPRO);
    for (int k = 0; k < npro; ++k) issue_tile(sg.src, ta + k, stage_of(sg, ta + k));
    switch (npro) {  // this wave's query rows have landed
      case 1: TT_WAIT_VM(1 * DMA_PER_TILE); break;
      case 2: TT_WAIT_VM(2 * DMA_PER_TILE); break;
      case 3: TT_WAIT_VM(3 * DMA_PER_TILE); break;
      default: TT_WAIT_VM(4 * DMA_PER_TILE); break;
    }
    bf16x8 qreg[NB][D / 16];
    {
      const char* qst = g_ring + (NPRO + wave) * STAGEB;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int ds = 0; ds < D / 16; ++ds) {
          qreg[nb][ds] = ld_k(qst + nb * 32 * ROWB + sg.lo.k[ds]);
          // the query operands stay in accumulation registers (MFMA sources may be read
          // from there), leaving the VGPRs to the softmax
          asm volatile("" : "+a"(qreg[nb][ds]));
        }
    }
    TT_WAIT_LGKM0();
    __syncthreads();  // every wave has its query rows: their stages take tiles now
    for (int k = NPRO; k < min(n, NSTAGE - 1); ++k) issue_tile(sg.src, ta + k, stage_of(sg, ta + k));
    wait_tiles_after(__builtin_amdgcn_readfirstlane(min(n, NSTAGE - 1) - 1));  // tile ta
    __syncthreads();

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

    f32x16 sA[NB], sB[NB];
    float mx[NB];
    qk_tile(stage_of(sg, ta), sg.lo, qreg, sA);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) asm volatile("" : "+v"(sA[nb]));
    tile_max(sA, sg.scale_log2, mx);

    // ---- pipelined loop, unrolled by two (scores alternate between sA and sB)
    int tt = ta;
    for (; tt + 2 < te; tt += 2) {
      step<true>(sg, qreg, ws, sA, sB, mx, tt);
      step<true>(sg, qreg, ws, sB, sA, mx, tt + 1);
    }
    if (tt + 1 < te) {
      step<true>(sg, qreg, ws, sA, sB, mx, tt);
      step<false>(sg, qreg, ws, sB, sA, mx, tt + 1);
    } else {
      step<false>(sg, qreg, ws, sA, sB, mx, tt);
    }
    __syncthreads();  // every wave is done with the stages

    // ---- epilogue: O / l as bf16 through this wave's LDS staging rows, then whole rows
    // to the output, or to a partial slot with m and l
    char* ost = g_ring + wave * RPW * OROWB;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float lt = lane_pair_sum(ws.l_run[nb]);
      const float inv = 1.0f / lt;
      char* orow = ost + (nb * 32 + (ln & 31)) * OROWB;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          bf16x4 v;
#pragma unroll
          for (int k = 0; k < 4; ++k) v[k] = (__bf16)(ws.oacc[db][nb][q4 * 4 + k] * inv);
          *reinterpret_cast<u32x2*>(orow + (db * 32 + 8 * q4 + 4 * (ln >> 5)) * 2) = __builtin_bit_cast(u32x2, v);
        }
      if (!whole && ln < 32) {
        float* ml = reinterpret_cast<float*>(part_slot(a, cluster, slot, qs) + (size_t)RWG * D * 2);
        const int rw = wave * RPW + nb * 32 + ln;
        ml[rw] = ws.m_run[nb];
        ml[RWG + rw] = lt;
      }
    }
    TT_WAIT_LGKM0();
    char* pbase = whole ? nullptr : part_slot(a, cluster, slot, qs) + (size_t)wave * RPW * ROWB;
#pragma unroll 4
    for (int i = 0; i < RPW / 4; ++i) {
      const int j = 4 * i + (ln >> 4);
      const u32x4 v = *reinterpret_cast<const u32x4*>(ost + j * OROWB + (ln & 15) * 16);
      if (whole) {
        const int r = row0 + j;
        if (r < rows_unit) *reinterpret_cast<u32x4*>(Ob + qrow_bytes(a, bcur, g, r) + (ln & 15) * 16) = v;
      } else {
        *reinterpret_cast<u32x4*>(pbase + (size_t)j * ROWB + (ln & 15) * 16) = v;
      }
    }
    __syncthreads();  // the staging rows are ring stages of the next segment
  }
}

// Merge the partials of every unit that a cluster boundary cut. One workgroup covers 16
// query rows of one unit (16 threads x 8 head-dim values per row). The pieces are read
// eight at a time, all loads in flight together, then merged with a running max.
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  constexpr int PB = 8;
  const int u = blockIdx.x;
  const int b = u / a.Hkv, g = u - b * a.Hkv;
  const int rows_unit = a.G * a.S;
  const int r = blockIdx.y * 16 + (threadIdx.x >> 4);
  const int d = (threadIdx.x & 15) * 8;
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
  float M = -INFINITY, L = 0.0f, o[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) o[k] = 0.0f;
  for (int c0 = c_first; c0 <= c_last; c0 += PB) {
    float mv[PB], lv[PB];
    u32x4 ov[PB];
#pragma unroll
    for (int j = 0; j < PB; ++j) {
      const int c = c0 + j;
      const int r0 = (int)(((long long)c * T) / a.NC);
      const bool ok = c <= c_last && r0 != (int)(((long long)(c + 1) * T) / a.NC);  // non-empty
      mv[j] = -INFINITY;
      lv[j] = 0.0f;
      ov[j] = u32x4{0, 0, 0, 0};
      if (ok) {
        const int slot = (start <= r0) ? 0 : 1;
        const char* base = part_slot(a, c, slot, qsl);
        const float* ml = reinterpret_cast<const float*>(base + (size_t)RWG * D * 2);
        mv[j] = ml[rw];
        lv[j] = ml[RWG + rw];
        ov[j] = *reinterpret_cast<const u32x4*>(base + ((size_t)rw * D + d) * 2);
      }
    }
#pragma unroll
    for (int j = 0; j < PB; ++j) {
      if (lv[j] > 0.0f) {  // every stored piece has l >= 1
        const float mn = fmaxf(M, mv[j]);
        const float sa = __builtin_amdgcn_exp2f(M - mn);  // 0 on the first piece
        const float sb = __builtin_amdgcn_exp2f(mv[j] - mn) * lv[j];
        const bf16x8 v = __builtin_bit_cast(bf16x8, ov[j]);
        L = L * sa + sb;
#pragma unroll
        for (int k = 0; k < 8; ++k) o[k] = o[k] * sa + sb * (float)v[k];
        M = mn;
      }
    }
  }
  const float inv = 1.0f / L;
  bf16x8 v;
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] = (__bf16)(o[k] * inv);
  *reinterpret_cast<u32x4*>(static_cast<char*>(a.o) + qrow_bytes(a, b, g, r) + d * 2) =
      __builtin_bit_cast(u32x4, v);
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
  hipLaunchKernelGGL(attn_combine_kernel, dim3(a.B * a.Hkv, (rows_unit + 15) / 16), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace tt
