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
//    with v_mfma_f32_32x32x16_bf16. A workgroup of 8 waves covers 256 query rows, 32 per
//    wave; one workgroup per CU, two waves per SIMD. A unit with more rows is covered by
//    NQ workgroups (a "cluster") placed on one XCD so that its key stream is fetched from
//    HBM once and shared through that XCD's L2. Clusters are numbered XCD-major: the
//    clusters that hold the pieces of one cut unit sit on one XCD and share its query rows.
//  * Keys of a unit are the concatenation [context ; block]; the key sequence is cut in
//    32-key tiles. All units form one global list of positions, each unit a fixed number
//    of overhead positions (the cost of a segment, in tiles) followed by its tiles; the
//    list is split evenly over the clusters of a persistent grid (the plan is computed
//    in-kernel from ctx_len), so a cluster's tiles plus its segments' fixed costs are
//    about the same for every cluster.
//    A cluster range that covers a whole unit writes the final output; a unit cut by a
//    range boundary leaves per-piece partials (running max and sum in fp32, normalised O
//    in bf16) that the combine kernel merges with a log-sum-exp rescale. The cluster whose
//    segment ends a unit leaves the unit's merge record (none when it held the unit whole);
//    the combine's grid is one row of workgroups per unit, and it touches nothing else.
//  * K and V tiles go HBM -> LDS directly (global_load_lds_dwordx4, no staging registers)
//    into a ring of 8 stages of 16 KB (8 KB of keys + 8 KB of values): six tiles are in
//    flight per CU while two are in use; explicit vmcnt waits and one barrier per tile.
//    The query rows of a segment arrive the same way (through four of the stages).
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
//  * Two wave groups in antiphase ("ping-pong"): per tile a wave runs a matrix phase (QK
//    products of tile j, PV products of tile j-1) and a vector phase (max, exp2, row sums
//    and bf16 packing of tile j). Waves 0-3 run matrix then vector, waves 4-7 vector then
//    matrix, so each SIMD's two waves keep its matrix core and its VALU busy at the same
//    time. With 32 rows per wave everything fits in 256 VGPRs (no accumulation registers,
//    no moves between register files).
//  * A unit of fewer than 256 query rows (small G*S) leaves waves whose 32 rows all lie past
//    it: those waves copy their share of every tile, wait and meet the barriers, but skip the
//    operand reads and the arithmetic (a second instantiation; G*S a multiple of 256 runs the
//    code without the test).
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
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int KT = kAttnKeysPerTile;          // 32 keys per tile
constexpr int D = kAttnMfmaD;                 // 128
constexpr int ROWB = D * 2;                   // 256-byte LDS rows
constexpr int TB = KT * ROWB;                 // 8 KB per tensor tile
constexpr int STAGEB = 2 * TB;                // K tile then V tile
constexpr int NW = kAttnWaves;                // 8 waves
constexpr int NTHR = NW * 64;                 // 512 threads
constexpr int RPW = kAttnRowsPerWave;         // 32 query rows per wave
constexpr int RWG = kAttnRowsPerWg;           // 256 query rows per workgroup
constexpr int DMA_PER_TENSOR = TB / 1024 / NW;  // one 1-KB copy per wave per tensor
constexpr int DMA_PER_TILE = 2 * DMA_PER_TENSOR;
constexpr int DMA_Q = RPW * ROWB / 1024;      // 8 one-KB copies for a wave's query rows
constexpr int NSTAGE = 8;                     // LDS ring
constexpr int NPRO = 4;                       // tiles issued before the query rows are read
constexpr int NAHEAD = 6;                     // tiles issued ahead of the one in the QK phase
constexpr int OROWB = ROWB + 16;              // padded row of the epilogue staging
constexpr int NDS = D / 16;                   // K operands per tile (d-steps)
constexpr int NVO = 2 * (D / 32);             // V^T operands per tile, index i = ks * 4 + db
constexpr float kLazy = 8.0f;                 // log2 headroom before the running max moves

static_assert(NSTAGE * STAGEB >= (kMaxB + 1) * 4, "tile plan must fit in the ring");
static_assert(RPW == 32 && DMA_PER_TENSOR == 1, "one MFMA column block and one copy per wave");
static_assert(RPW * ROWB == TB && NW == 2 * (NSTAGE - NPRO), "query rows fill the stages after the prologue tiles");
static_assert(NW * RPW * OROWB <= NSTAGE * STAGEB, "epilogue staging fits in the ring");
static_assert(NAHEAD + 2 == NSTAGE, "two stages in use, the rest in flight");
static_assert(NSTAGE * TB == 65536, "immediate LDS offsets cover one tensor's stages");

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Work-item and workgroup ids straight from the hardware registers. (The HIP accessors are
// device-library functions; built with IEEE mode off, this file's kernels do not match
// their attributes, so the compiler would call them rather than inline them.)
__device__ __forceinline__ int tid_x() { return (int)__builtin_amdgcn_workitem_id_x(); }
__device__ __forceinline__ int bid_x() { return (int)__builtin_amdgcn_workgroup_id_x(); }
__device__ __forceinline__ int bid_y() { return (int)__builtin_amdgcn_workgroup_id_y(); }

// The ring holds the K tiles of the 8 stages in its first 64 KB and the V tiles in the
// next 64 KB, so that every LDS operand read of a stage is a fixed per-lane register plus
// an immediate offset below 64 KB. It is the kernel's only LDS variable (at address 0);
// its last 64 bytes are the plan's per-wave sums.
constexpr int VOFF = NSTAGE * TB;
__shared__ __attribute__((aligned(1024))) char g_ring[NSTAGE * STAGEB + 64];

__device__ __forceinline__ char* kst(int s) { return g_ring + s * TB; }
__device__ __forceinline__ char* vst(int s) { return g_ring + VOFF + s * TB; }

__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

// The lane id, recomputed where it is used (v_mbcnt, in an asm block that the compiler
// neither hoists nor merges), so that no register holds it across the tile loop: every
// register there is taken, and a value spilled to scratch would be reloaded behind a wait
// for all vector-memory operations, i.e. for every tile copy in flight.
__device__ __forceinline__ int fresh_lane() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
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

// The same value for a wave-uniform b, read with a scalar load (through the constant
// address space: ctx_len is not written while the kernel runs). A vector load here would
// make the compiler wait on the vector-memory counter, i.e. also for the epilogue stores
// and tile copies in flight.
typedef const __attribute__((address_space(4))) int32_t c_i32;
__device__ __forceinline__ int clamp_ctx_u(const int32_t* ctx_len, int b, int Lmax) {
  const int n = ((c_i32*)(uintptr_t)ctx_len)[b];
  return n < 0 ? 0 : (n > Lmax ? Lmax : n);
}

// Exclusive prefix sums over sequences of (positions per unit * Hkv) into P[0..B]; P[B] =
// total. A unit's positions: kAttnSegmentCost overhead positions, then its tiles.
__device__ void build_plan(int* P, int* wsum, const int32_t* ctx_len, int B, int S, int Hkv,
                           int Lmax) {
  const int tid = tid_x(), lane = tid & 63, w = tid >> 6;
  const int per = (B + NTHR - 1) / NTHR;
  const int b0 = tid * per;
  int local = 0;
  for (int k = 0; k < per; ++k) {
    const int b = b0 + k;
    if (b < B) local += ((clamp_ctx(ctx_len, b, Lmax) + S + KT - 1) / KT + kAttnSegmentCost) * Hkv;
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
      run += ((clamp_ctx(ctx_len, b, Lmax) + S + KT - 1) / KT + kAttnSegmentCost) * Hkv;
    }
  }
  if (tid == 0) P[B] = total;
  __syncthreads();
}

// Source rows of one unit for the tile copies. This lane copies the 16-byte chunk
// c = (lane%16) ^ f(row) of tile row 4*wave + lane/16 of each tensor.
struct TileSrc {
  const char* kc;   // k_ctx row 0 of this unit (bytes; row stride rs)
  const char* vc;
  const char* kb;   // k_blk row 0 of this unit
  const char* vb;
  size_t rs;        // Hkv * D * 2 bytes
  int nctx, S;
  int coff;         // c * 16
  uint32_t voff;    // (tile row of this lane) * rs + c * 16
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

// A wave-uniform pointer moved to scalar registers: the two halves through readfirstlane,
// which yields a signed int, so each half is taken as uint32_t before widening (a
// sign-extended low half would corrupt the high word).
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const char*>((uintptr_t)((hi << 32) | lo));
}

// The same copy from a wave-uniform base (scalar registers) plus a 32-bit per-lane offset.
__device__ __forceinline__ void dma16s(const char* base, uint32_t voff, uint32_t lds) {
  base = uniform_ptr(base);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 offset:0" ::"v"(voff),
               "s"(base), "s"(lds)
               : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)p);
}

// Issue this wave's copies of tile t into stage st: key j < ctx_len reads context row j,
// else block row j - ctx_len; keys past ctx_len + S read the last block row (finite data
// whose scores are masked). One wave-uniform LDS destination per copy (1 KB = 4 rows).
__device__ __forceinline__ void issue_tile(const TileSrc& s, int t, int st, int w) {
  const uint32_t ldk = lds_addr(kst(st) + 4 * w * ROWB), ldv = ldk + VOFF;
  if ((t + 1) * KT <= __builtin_amdgcn_readfirstlane(s.nctx)) {
    // every key in the context: scalar bases, fixed lane offsets
    const size_t toff = (size_t)t * KT * s.rs;
    dma16s(s.kc + toff, s.voff, ldk);
    dma16s(s.vc + toff, s.voff, ldv);
    return;
  }
  const int key = t * KT + 4 * w + (fresh_lane() >> 4);
  const bool in_ctx = key < s.nctx;
  const int idx = in_ctx ? key : min(key - s.nctx, s.S - 1);
  const size_t off = (size_t)idx * s.rs + s.coff;
  dma16((in_ctx ? s.kc : s.kb) + off, ldk);
  dma16((in_ctx ? s.vc : s.vb) + off, ldv);
}

// The steady-state copy: a scalar base (already wave-uniform, in scalar registers) plus
// the lane offset.
__device__ __forceinline__ void dma16u(const char* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 offset:0" ::"v"(voff),
               "s"(base), "s"(lds)
               : "memory", "m0");
}

// wait until at most n vector-memory operations of this wave are outstanding (n <= 63)
#define TT_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0x70 | 0xF00)
// wait until this wave's LDS reads and writes are done
#define TT_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(0xC07F)

__device__ __forceinline__ void wait_tiles_after(int n_after) {
  // n_after: tiles whose copies were issued after the one to be consumed (0..6)
  if (n_after == NAHEAD - 1) {  // the steady state of the tile loop
    TT_WAIT_VM((NAHEAD - 1) * DMA_PER_TILE);
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

struct LaneOffsets {
  int k[NDS];             // K operand, d-step ds: row lr, chunk (2 ds + lh) ^ f(lr)
  int v[D / 32][2];       // V^T operand, head-dim block db, row half (+0 / +8); + VOFF
};

// Per-wave accumulation state of one segment.
struct WaveState {
  f32x16 oacc[D / 32];    // O^T, one 32x32 block per head-dim block
  f32x16 s;               // scores S^T of the tile between its matrix and vector phases
  bf16x8 pb[2];           // P of the tile between its vector phase and the next matrix phase
  float m_run, l_run;
};

// LDS operand reads for a matrix phase: K operands of a tile (ds_read_b128 each) and the
// V^T operands of a tile (two ds_read_b64_tr_b16 each).
__device__ __forceinline__ void load_k_ops(const char* st, const LaneOffsets& lo, bf16x8 (&ka)[NDS]) {
#pragma unroll
  for (int ds = 0; ds < NDS; ++ds) ka[ds] = ld_k(st + lo.k[ds]);
}

// (st: the stage's K tile; the V^T lane offsets include the distance to its V tile)
__device__ __forceinline__ void load_v_ops(const char* st, const LaneOffsets& lo, bf16x8 (&va)[NVO]) {
#pragma unroll
  for (int i = 0; i < NVO; ++i)
    va[i] = ld_v(st + lo.v[i % 4][0] + (i / 4) * 16 * ROWB, st + lo.v[i % 4][1] + (i / 4) * 16 * ROWB);
}

// Matrix phase: QK products of one tile (if do_qk) and PV products of the previous one
// (if do_pv), from operands read during the preceding vector phase.
__device__ __forceinline__ void matrix_phase(const bf16x8 (&ka)[NDS], const bf16x8 (&va)[NVO],
                                             const bf16x8 (&qreg)[NDS], WaveState& w, bool do_qk,
                                             bool do_pv) {
  if (do_qk) {
    const f32x16 zero = {};
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds)
      w.s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ds], qreg[ds], ds == 0 ? zero : w.s, 0, 0, 0);
  }
  if (do_pv) {
#pragma unroll
    for (int i = 0; i < NVO; ++i)
      w.oacc[i % 4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i], w.pb[i / 4], w.oacc[i % 4], 0, 0, 0);
  }
}

// Vector phase of a tile: key mask (the unit's last tile only), row max, lazy rescale,
// P = exp2(s * scale_log2 - m) packed as the PV B operand (key-step ks = k / 8 holds
// the values k % 8), and the row sums of the bf16-rounded P.
__device__ __forceinline__ void vector_phase(WaveState& w, float scale_log2, bool mask, int lim0) {
  if (mask) {  // keys at or past nvalid get -inf (lim0: nvalid - the tile's first key)
    const int lim = lim0 - 4 * (fresh_lane() >> 5);
#pragma unroll
    for (int k = 0; k < 16; ++k)
      if (8 * (k >> 2) + (k & 3) >= lim) w.s[k] = -INFINITY;
  }
  // Each lane half holds 16 of the tile's 32 keys for its row. The half maxima decide
  // whether the running max may stay (every half within 2^kLazy of it, so is the row);
  // only when some lane's half exceeds it are the two halves combined (v_permlane32_swap,
  // a slow instruction) and O, l rescaled, identically in both halves.
  float m = w.s[0];
#pragma unroll
  for (int k = 1; k < 16; ++k) m = __builtin_fmaxf(m, w.s[k]);
  if (__any(m * scale_log2 > w.m_run + kLazy)) {
    const float mx = lane_pair_max(m) * scale_log2;  // scale_log2 > 0 commutes with max
    const float mn = fmaxf(w.m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(w.m_run - mn);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int k = 0; k < 16; ++k) w.oacc[db][k] *= alpha;
    w.l_run *= alpha;
    w.m_run = mn;
  }
  // P in bf16 for the PV products; the row sum in fp32 from the unrounded values (plain
  // adds: the dot instructions contend with the other wave's matrix products)
  // (the sums start from the first terms: with IEEE semantics 0 + p is not folded)
  float ps0, ps1;
#pragma unroll
  for (int k = 0; k < 16; k += 2) {
    const float p0 = __builtin_amdgcn_exp2f(w.s[k] * scale_log2 - w.m_run);
    const float p1 = __builtin_amdgcn_exp2f(w.s[k + 1] * scale_log2 - w.m_run);
    w.pb[k >> 3][k & 7] = (__bf16)p0;
    w.pb[k >> 3][(k & 7) + 1] = (__bf16)p1;
    ps0 = k == 0 ? p0 : ps0 + p0;
    ps1 = k == 0 ? p1 : ps1 + p1;
  }
  w.l_run += ps0 + ps1;
}

// The barrier between two phases; no instruction moves across it (the compiler would
// otherwise move matrix products, which touch no memory, into the neighbouring phase).
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);
}

// One tile iteration j in the steady state (j >= 1, j + NAHEAD < n, tile j + NAHEAD
// wholly in the context): every copy takes the scalar path from the running bases kp, vp
// (advanced by one tile), no key is masked, and both wave groups run the same waits.
// After the matrix phase 5 tiles of copies may stay outstanding behind tile j+1 (group 0
// needs tile j+1 at the coming barrier, group 1 needed it one barrier earlier); after the
// vector phase 4 behind tile j+2 (group 1 needs it at the coming barrier, group 0 waits
// for it half an iteration early). With U >= 0 (the stage of tile j, known at compile
// time) every LDS operand read is a lane register plus an immediate offset. A wave whose
// query rows all lie past the unit (act false) only copies, waits and meets the barriers.
template <int U>
__device__ __forceinline__ void steady_iter(int j, const char*& kp, const char*& vp, size_t tstep,
                                            uint32_t voff, uint32_t wrow, const LaneOffsets& lo,
                                            bf16x8 (&ka)[NDS], bf16x8 (&va)[NVO],
                                            const bf16x8 (&qreg)[NDS], WaveState& ws,
                                            float scale_log2, bool act) {
  const int s0 = U >= 0 ? U : (j & (NSTAGE - 1));
  const int s1 = (s0 + 1) & (NSTAGE - 1), sa = (s0 + NAHEAD) & (NSTAGE - 1);
  dma16u(kp, voff, (uint32_t)(uintptr_t)kst(sa) + wrow);
  dma16u(vp, voff, (uint32_t)(uintptr_t)vst(sa) + wrow);
  kp += tstep;
  vp += tstep;
  if (act) matrix_phase(ka, va, qreg, ws, true, true);
  TT_WAIT_VM((NAHEAD - 1) * DMA_PER_TILE);
  phase_barrier();
  if (act) {
    load_k_ops(kst(s1), lo, ka);
    load_v_ops(kst(s0), lo, va);
  }
  __builtin_amdgcn_sched_barrier(0);
  if (act) vector_phase(ws, scale_log2, false, 0);
  TT_WAIT_VM((NAHEAD - 2) * DMA_PER_TILE);
  phase_barrier();
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

// Cluster c owns positions [range_start(c), range_start(c+1)), range_start(c) =
// floor(c T / NC); cluster_of(x) is the one holding position x, ceil((x+1) NC / T) - 1.
// In double: the products are integers below 2^53 (exact) and a quotient that is not an
// integer is at least 1/max(T, NC) from one, far above the rounding error, so the floor
// and ceil are exact.
__device__ __forceinline__ int range_start(int c, int T, int NC) {
  return (int)floor((double)c * (double)T / (double)NC);
}
__device__ __forceinline__ int cluster_of(int x, int T, int NC) {
  return (int)ceil((double)(x + 1) * (double)NC / (double)T) - 1;
}

// ALL: every wave holds rows of the unit (G*S a multiple of the workgroup's 256 rows); else a
// wave whose 32 rows all lie past the unit skips the operand reads and the arithmetic.
template <bool ALL>
__global__ __launch_bounds__(NTHR, 1) void attn_mfma_kernel(AttnArgs a) {
  int* wsum = reinterpret_cast<int*>(g_ring + NSTAGE * STAGEB);

  const int tid = tid_x(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;  // 0: matrix phase first, 1: vector phase first
  const int lr = lane & 31, lh = lane >> 5;
  const int id = bid_x();
  const int xcd = id & 7, kk = id >> 3;
  // workgroup id % 8 is its XCD; clusters are numbered XCD-major, so the consecutive
  // clusters that share a cut unit also share an L2 and fetch its query rows once
  const int cluster = __builtin_amdgcn_readfirstlane(xcd * (a.NC / 8) + kk / a.NQ);
  const int qs = __builtin_amdgcn_readfirstlane(kk % a.NQ);

  // ---- plan: position prefix sums in LDS, then this cluster's range of the global list
  int* P = reinterpret_cast<int*>(g_ring);
  build_plan(P, wsum, a.ctx_len, a.B, a.S, a.Hkv, a.Lmax);
  const int T = __builtin_amdgcn_readfirstlane(P[a.B]);
  const int t0 = range_start(cluster, T, a.NC);
  const int t1 = range_start(cluster + 1, T, a.NC);
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
  if (t0 >= t1) {
    // an empty range (only when T < NC): its slot-0 piece is marked empty (l = 0) for the
    // combine, which may meet it between the first and the last piece of a cut unit
    float* ml = reinterpret_cast<float*>(part_slot(a, cluster, 0, qs) + (size_t)RWG * D * 2);
    if (tid < RWG) ml[RWG + tid] = 0.0f;
    return;
  }

  const char* Qb = static_cast<const char*>(a.q);
  char* Ob = static_cast<char*>(a.o);
  const int G = a.G, S = a.S, rows_unit = G * S;
  const bool act = ALL || __builtin_amdgcn_readfirstlane(qs * RWG + wave * RPW) < rows_unit;

  LaneOffsets lo;
  {
    const int fk = swz(lr);
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) lo.k[ds] = lr * ROWB + (((2 * ds + lh) ^ fk) << 4);
    const int j = lane & 15, grp2 = (lane >> 4) & 1;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 4 * lh + (j >> 2) + 8 * h;
      const int fv = swz(row);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int c = 4 * db + 2 * grp2 + ((j & 3) >> 1);
        lo.v[db][h] = VOFF + row * ROWB + ((c ^ fv) << 4) + (j & 1) * 8;
        // opaque, so that the compiler keeps VOFF in the register rather than in the
        // reads' offset field (which holds 16 bits)
        asm volatile("" : "+v"(lo.v[db][h]));
      }
    }
  }
  TileSrc src;
  {
    const int row = 4 * wave + (lane >> 4);
    src.coff = ((lane & 15) ^ swz(row & 15)) << 4;
    src.voff = (uint32_t)(row * a.Hkv * D * 2 + src.coff);
    src.rs = (size_t)a.Hkv * D * 2;
    src.S = S;
  }
  const float scale_log2 = a.scale_log2;

  constexpr int SC = kAttnSegmentCost;
  int t = t0;  // a position of the global list
  bool first_seg = true;
  int nctx = clamp_ctx_u(a.ctx_len, bcur, a.Lmax);
  int nt = (nctx + S + KT - 1) / KT;  // tiles per unit of sequence bcur
  while (t < t1) {
    while (t >= pb + (nt + SC) * a.Hkv) {  // advance to the sequence holding position t
      pb = __builtin_amdgcn_readfirstlane(pb + (nt + SC) * a.Hkv);
      bcur = __builtin_amdgcn_readfirstlane(bcur + 1);
      nctx = clamp_ctx_u(a.ctx_len, bcur, a.Lmax);
      nt = __builtin_amdgcn_readfirstlane((nctx + S + KT - 1) / KT);
    }
    const int g = __builtin_amdgcn_readfirstlane((t - pb) / (nt + SC));
    const int ustart = pb + g * (nt + SC);  // the unit's overhead positions, then its tiles
    const int ta = __builtin_amdgcn_readfirstlane(max(t - ustart - SC, 0));  // first local tile
    const int te = __builtin_amdgcn_readfirstlane(min(nt, t1 - ustart - SC));  // one past the last
    t = ustart + nt + SC;
    if (te <= ta) continue;  // the range ends among the unit's overhead positions
    const bool whole = (ta == 0 && te == nt);
    const int slot = first_seg ? 0 : 1;
    if (te == nt && qs == 0 && wave == 0 && fresh_lane() == 0) {
      // the unit's merge record, by the cluster whose segment ends the unit: none for a whole
      // unit; for a cut one (its last piece is always the cluster's first segment) the first
      // piece's cluster and slot and this cluster, the last piece's
      int4 r = int4{-1, 0, 0, 0};
      if (ta > 0) {
        const int cf = cluster_of(ustart + SC, T, a.NC);
        const int cs = 2 * cf + (range_start(cf, T, a.NC) < ustart ? 1 : 0);
        r = int4{bcur, g, cs, cluster};
      }
      int u = __builtin_amdgcn_readfirstlane(bcur * a.Hkv + g);
      asm volatile("" : "+s"(u));  // the address is formed here, not kept across the loop
      *reinterpret_cast<int4*>(a.rec + 4 * u) = r;
    }
    first_seg = false;
    const int n = te - ta;  // tiles in this segment (>= 1)
    const int nvalid = nctx + S;

    src.kc = static_cast<const char*>(a.k_ctx) + ((size_t)bcur * a.Lmax * a.Hkv + g) * D * 2;
    src.vc = static_cast<const char*>(a.v_ctx) + ((size_t)bcur * a.Lmax * a.Hkv + g) * D * 2;
    src.kb = static_cast<const char*>(a.k_blk) + ((size_t)bcur * S * a.Hkv + g) * D * 2;
    src.vb = static_cast<const char*>(a.v_blk) + ((size_t)bcur * S * a.Hkv + g) * D * 2;
    src.nctx = nctx;

    // ---- prologue. Query rows of this wave -> its 8 KB behind the first NPRO stages (row
    // j of the wave at LDS row j, chunks permuted like the key tiles); row r of the unit is
    // (head-in-group r / S, position r % S); rows past the unit read its row 0 (results
    // discarded).
    const int row0 = qs * RWG + wave * RPW;  // this wave's first unit row
    char* qst = g_ring + (wave >> 2) * VOFF + NPRO * TB + (wave & 3) * TB;
    uint32_t qlds = lds_addr(qst);
    asm volatile("" : "+s"(qlds));  // computed here, not hoisted into registers
    const int ln = fresh_lane();
#pragma unroll
    for (int i = 0; i < DMA_Q; ++i) {
      const int j = 4 * i + (ln >> 4);
      const int r = row0 + j;
      const int c = (ln & 15) ^ swz(j & 15);
      dma16(Qb + qrow_bytes(a, bcur, g, r < rows_unit ? r : 0) + (c << 4), qlds + 4 * i * ROWB);
    }
    const int npro = min(n, NPRO);
    for (int k = 0; k < npro; ++k) issue_tile(src, ta + k, k, wave);
    switch (npro) {  // this wave's query rows have landed
      case 1: TT_WAIT_VM(1 * DMA_PER_TILE); break;
      case 2: TT_WAIT_VM(2 * DMA_PER_TILE); break;
      case 3: TT_WAIT_VM(3 * DMA_PER_TILE); break;
      default: TT_WAIT_VM(4 * DMA_PER_TILE); break;
    }
    bf16x8 qreg[NDS];
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) qreg[ds] = ld_k(qst + lo.k[ds]);
    TT_WAIT_LGKM0();
    __syncthreads();  // every wave has its query rows: their stages take tiles now
    for (int k = NPRO; k < min(n, NAHEAD); ++k) issue_tile(src, ta + k, k, wave);
    wait_tiles_after(__builtin_amdgcn_readfirstlane(min(n, NAHEAD) - 1));  // local tile 0
    __syncthreads();

    WaveState ws;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int k = 0; k < 16; ++k) ws.oacc[db][k] = 0.0f;
    ws.m_run = -INFINITY;
    ws.l_run = 0.0f;

    // ---- tile loop, one code path for both wave groups. Iteration j: matrix phase (QK
    // products of tile j, PV products of tile j-1), barrier, vector phase (tile j; it
    // first issues the LDS reads of the next matrix phase: K of tile j+1, V of tile j, so
    // their latency passes behind its arithmetic), barrier. Group 1 passes one extra
    // barrier first, so it runs each phase while group 0 runs the other one (the barriers
    // pair group 0's k-th with group 1's (k-1)-th; each SIMD holds one wave of each group).
    // Tile j+1 is published by the barrier that starts group 0's vector phase j: before it
    // each wave waits for its own copies of that tile (group 0 after matrix phase j, group
    // 1 after vector phase j-1). A wave issues its copies of tile j+6 at the start of its
    // matrix phase j, into the stage of tile j-2, whose last reads (vector phase j-2) both
    // groups finished two barriers earlier. Local tile k uses stage k % 8. The first
    // iteration, the last ones and those whose copies need the block rows take the general
    // path below; the rest run steady_iter, eight at a time with compile-time stages.
    bf16x8 ka[NDS], va[NVO];
    if (act) load_k_ops(kst(0), lo, ka);
    if (grp == 1) {
      if (1 < n) wait_tiles_after(__builtin_amdgcn_readfirstlane(min(NAHEAD - 2, n - 2)));
      __syncthreads();
    }
    auto general_iter = [&](int j) {
      if (j + NAHEAD < n) issue_tile(src, ta + j + NAHEAD, (j + NAHEAD) & (NSTAGE - 1), wave);
      if (act) matrix_phase(ka, va, qreg, ws, j < n, j >= 1);
      if (grp == 0 && j + 1 < n) wait_tiles_after(__builtin_amdgcn_readfirstlane(min(NAHEAD - 1, n - 2 - j)));
      phase_barrier();
      if (act && j + 1 < n) load_k_ops(kst((j + 1) & (NSTAGE - 1)), lo, ka);
      if (act && j < n) load_v_ops(kst(j & (NSTAGE - 1)), lo, va);
      __builtin_amdgcn_sched_barrier(0);
      if (act && j < n) vector_phase(ws, scale_log2, ta + j == nt - 1, nvalid - (ta + j) * KT);
      if (grp == 1 && j + 2 < n) wait_tiles_after(__builtin_amdgcn_readfirstlane(min(NAHEAD - 2, n - 3 - j)));
      phase_barrier();
    };
    general_iter(0);
    int j = 1;
    // last steady iteration: its copies (tile ta + j + NAHEAD) lie wholly in the context
    const int jss = __builtin_amdgcn_readfirstlane(min(n - NAHEAD - 1, nctx / KT - ta - NAHEAD - 1));
    if (j <= jss) {
      const size_t tstep = (size_t)KT * src.rs;
      const char* kp = uniform_ptr(src.kc + (size_t)(ta + 1 + NAHEAD) * tstep);
      const char* vp = uniform_ptr(src.vc + (size_t)(ta + 1 + NAHEAD) * tstep);
      const uint32_t wrow = __builtin_amdgcn_readfirstlane(4 * wave * ROWB);
      for (; j + 7 <= jss; j += 8) {  // j % 8 == 1
        steady_iter<1>(j, kp, vp, tstep, src.voff, wrow, lo, ka, va, qreg, ws, scale_log2, act);
        steady_iter<2>(j + 1, kp, vp, tstep, src.voff, wrow, lo, ka, va, qreg, ws, scale_log2, act);
        steady_iter<3>(j + 2, kp, vp, tstep, src.voff, wrow, lo, ka, va, qreg, ws, scale_log2, act);
        steady_iter<4>(j + 3, kp, vp, tstep, src.voff, wrow, lo, ka, va, qreg, ws, scale_log2, act);
        steady_iter<5>(j + 4, kp, vp, tstep, src.voff, wrow, lo, ka, va, qreg, ws, scale_log2, act);
        steady_iter<6>(j + 5, kp, vp, tstep, src.voff, wrow, lo, ka, va, qreg, ws, scale_log2, act);
        steady_iter<7>(j + 6, kp, vp, tstep, src.voff, wrow, lo, ka, va, qreg, ws, scale_log2, act);
        steady_iter<0>(j + 7, kp, vp, tstep, src.voff, wrow, lo, ka, va, qreg, ws, scale_log2, act);
      }
      for (; j <= jss; ++j) steady_iter<-1>(j, kp, vp, tstep, src.voff, wrow, lo, ka, va, qreg, ws, scale_log2, act);
    }
    for (; j <= n; ++j) general_iter(j);
    if (grp == 0) __syncthreads();

    // ---- epilogue: O / l as bf16 through this wave's LDS staging rows, then whole rows
    // to the output, or to a partial slot with m and l
    char* ost = g_ring + wave * RPW * OROWB;
    const int ln2 = fresh_lane();
    {
      const float lt = lane_pair_sum(ws.l_run);
      const float inv = 1.0f / lt;
      char* orow = ost + (ln2 & 31) * OROWB;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          bf16x4 v;
#pragma unroll
          for (int k = 0; k < 4; ++k) v[k] = (__bf16)(ws.oacc[db][q4 * 4 + k] * inv);
          *reinterpret_cast<u32x2*>(orow + (db * 32 + 8 * q4 + 4 * (ln2 >> 5)) * 2) = __builtin_bit_cast(u32x2, v);
        }
      if (!whole && ln2 < 32) {
        float* ml = reinterpret_cast<float*>(part_slot(a, cluster, slot, qs) + (size_t)RWG * D * 2);
        const int rw = wave * RPW + ln2;
        ml[rw] = ws.m_run;
        ml[RWG + rw] = lt;
      }
    }
    TT_WAIT_LGKM0();
    char* pbase = whole ? nullptr : part_slot(a, cluster, slot, qs) + (size_t)wave * RPW * ROWB;
#pragma unroll 4
    for (int i = 0; i < RPW / 4; ++i) {
      const int j = 4 * i + (ln2 >> 4);
      const u32x4 v = *reinterpret_cast<const u32x4*>(ost + j * OROWB + (ln2 & 15) * 16);
      if (whole) {
        const int r = row0 + j;
        if (r < rows_unit) *reinterpret_cast<u32x4*>(Ob + qrow_bytes(a, bcur, g, r) + (ln2 & 15) * 16) = v;
      } else {
        *reinterpret_cast<u32x4*>(pbase + (size_t)j * ROWB + (ln2 & 15) * 16) = v;
      }
    }
    __syncthreads();  // the staging rows are ring stages of the next segment
  }
}

// Merge the partials of every unit that a cluster boundary cut. Workgroup (x, u) reads the
// merge record of unit u (none: the unit was held whole, and it exits) and covers 16 query
// rows of that unit (16 threads x 8 head-dim values per row). The pieces lie in clusters
// first .. last of the record; they are read eight at a time, all loads in flight together,
// and merged with a running max.
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  constexpr int PB = 8;
  // grid: (row chunk, unit): the row chunks of one record are consecutive workgroups, so
  // they spread over the XCDs (workgroup id % 8)
  // the record was written by the previous kernel: scalar loads, uniform arithmetic
  const c_i32* rec = (c_i32*)(uintptr_t)(a.rec + 4 * bid_y());
  const int b = rec[0];
  if (b < 0) return;
  const int g = rec[1], c_first = rec[2] >> 1, first_slot = rec[2] & 1, c_last = rec[3];
  const int rows_unit = a.G * a.S;
  const int r = bid_x() * 16 + (tid_x() >> 4);
  if (r >= rows_unit) return;
  const int d = (tid_x() & 15) * 8;
  const int qsl = r / RWG, rw = r - qsl * RWG;
  // the first piece is its cluster's second segment when that cluster's range starts
  // before the unit; every later piece is its cluster's first segment (l = 0 marks the
  // piece of an empty range). Piece c + 1 lies 2 * NQ slots after piece c.
  const size_t step = (size_t)2 * a.NQ * kPartBytes;
  const char* p0 = part_slot(a, c_first, first_slot, qsl) + ((size_t)rw * D + d) * 2;
  const char* q0 = part_slot(a, c_first, 0, qsl) + ((size_t)rw * D + d) * 2;  // pieces after the first
  const int lo_off = RWG * D * 2 - (rw * D + d) * 2;  // from the O chunk to this row's m
  float M = -INFINITY, L = 0.0f, o[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) o[k] = 0.0f;
  for (int c0 = c_first; c0 <= c_last; c0 += PB) {
    float mv[PB], lv[PB];
    u32x4 ov[PB];
#pragma unroll
    for (int j = 0; j < PB; ++j) {  // unconditional loads (of the last piece past the end)
      const int c = min(c0 + j, c_last);
      const char* po = (c == c_first ? p0 : q0 + (size_t)(c - c_first) * step);
      const float* ml = reinterpret_cast<const float*>(po + lo_off) + rw;
      mv[j] = ml[0];
      lv[j] = c0 + j <= c_last ? ml[RWG] : 0.0f;
      ov[j] = *reinterpret_cast<const u32x4*>(po);
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
  if ((a.G * a.S) % RWG == 0) hipLaunchKernelGGL(attn_mfma_kernel<true>, dim3(a.NC * a.NQ), dim3(NTHR), 0, s, a);
  else hipLaunchKernelGGL(attn_mfma_kernel<false>, dim3(a.NC * a.NQ), dim3(NTHR), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ev1) (void)hipEventRecord(ev1, s);
  const int rows_unit = a.G * a.S;
  hipLaunchKernelGGL(attn_combine_kernel, dim3((rows_unit + 15) / 16, a.B * a.Hkv), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace tt
