// Internal declarations shared by the libtt translation units (host launch helpers and
// the parameter blocks the kernels take). Not part of the C-ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "tt.h"

namespace tt {

// ---------------------------------------------------------------------------------------
// attention
// ---------------------------------------------------------------------------------------

constexpr int kAttnKeysPerTile = 32;   // keys staged in LDS per pipeline step
constexpr int kAttnMinTilesPerCluster = 8;  // a small problem takes fewer clusters (host plan)
constexpr int kAttnWaves = 8;          // waves per workgroup of the MFMA kernel
constexpr int kAttnRowsPerWave = 32;   // query rows (head-in-group x block position) per wave
constexpr int kAttnRowsPerWg = kAttnWaves * kAttnRowsPerWave;
constexpr int kAttnMfmaD = 128;        // head dim of the MFMA kernel
constexpr int kMaxB = 8191;            // largest batch (the tile plan sits in LDS)
// The fixed cost of one segment (a cluster's run over one unit: query rows in, pipeline
// fill and drain, output rows out), in tiles. The tile list is split over the clusters
// with this many extra positions in front of each unit, so that a cluster that handles
// more segments gets fewer tiles.
constexpr int kAttnSegmentCost = 12;

struct AttnArgs {
  const void* q;
  const void* k_blk;
  const void* v_blk;
  const void* k_ctx;
  const void* v_ctx;
  const int32_t* ctx_len;
  void* o;
  float* part;        // partial results per (cluster, segment, query slice)
  int32_t* rec;       // [B*Hkv][4] merge records: per unit (b, g), b = -1 for a unit one
                      // cluster holds whole, else (b, g, 2 * first piece's cluster + its slot,
                      // last piece's cluster); written by the main kernel, read by the combine
  int B, S, Hq, Hkv, G, D, Lmax;
  int NQ;             // workgroups (query slices) per (sequence, KV head) unit
  int NC;             // clusters; each owns a contiguous range of the global position list
  float scale_log2;   // log2(e) / sqrt(D)
};

hipError_t launch_attn_mfma(const AttnArgs& a, hipStream_t s, hipEvent_t ev_main0, hipEvent_t ev_main1);
hipError_t launch_attn_generic(const AttnArgs& a, int dtype, hipStream_t s);
size_t attn_part_bytes(int nc, int nq);  // partial-result workspace of the MFMA path

// ---------------------------------------------------------------------------------------
// commit
// ---------------------------------------------------------------------------------------

struct CommitChunk {   // per (row, vocabulary chunk): partial max / argmax / sum of exp
  float m;
  int32_t tok;
  double z;
};

struct CommitArgs {
  const void* logits;
  const uint8_t* mask;
  float gamma;
  int32_t* token_id;
  uint8_t* committed;
  float* conf;
  CommitChunk* chunks;     // [B*S][n_chunks]
  int B, S, V;
  int n_chunks, chunk_elems;
  int dtype;
};

// ---------------------------------------------------------------------------------------
// context cache update after a commit
// ---------------------------------------------------------------------------------------

struct AppendArgs {
  const void* k_new;
  const void* v_new;
  void* k_ctx;
  void* v_ctx;
  int32_t* ctx_len;
  uint8_t* skipped;    // may be null
  int B, S, Lmax;
  size_t row_bytes;    // Hkv * D * element size
  int elt;             // element size in bytes
  int bump;
  int vec16;           // every run and base 16-byte aligned
};

hipError_t launch_ctx_append(const AppendArgs& a, hipStream_t s);

int commit_chunk_elems(int dtype);
constexpr long long kMaxGridBlocks = 16777215;  // 256-thread workgroups: < 2^32 work-items
// the commit: the chunk reduction, then the per-sequence decision (an event may be recorded
// between the two launches)
hipError_t launch_commit(const CommitArgs& a, hipStream_t s, hipEvent_t ev_reduce_end);
// the decide step alone (a.logits == nullptr: decisions on the chunk estimates only)
hipError_t launch_commit_decide(const CommitArgs& a, hipStream_t s);
// The allocation-free commit's scratch: a static device array of this many bytes per GPU;
// commit_scratch() returns the current device's address of it (looked up on first use).
constexpr size_t kCommitScratchBytes = (size_t)4 << 20;
hipError_t commit_scratch(void** ptr);

// ---------------------------------------------------------------------------------------
// LM head fused with the commit's vocabulary reduction
// ---------------------------------------------------------------------------------------

constexpr int kLmVocabPerWg = 256;      // head rows (vocabulary entries) per workgroup = chunk
constexpr int kLmRowsPerWg = 128;       // masked hidden rows per workgroup
constexpr int kLmFeaturesPerStage = 64; // K per LDS stage (K must be a multiple)
constexpr int kLmMaxRows = 4096;        // B*S limit

struct LmHeadArgs {
  const void* hidden;   // [B*S][K] bf16
  const void* weight;   // [V][K] bf16
  const uint8_t* mask;  // [B*S]
  CommitChunk* chunks;  // [B*S][NVT]
  float* runner;        // [B*S][NVT]: the chunk's runner-up logit (a second copy of the max
                        // when it occurs twice; -inf when the chunk holds one entry)
  CommitChunk* merged;  // [B*S], one record per masked row
  double* rowx;         // [B*S][2]: the row's runner-up logit and the bound on |fp32 logit -
                        // exact logit| (exact mode; else unused)
  const float* w_bound; // device: an upper bound on max_v ||weight[v]||_2, or null (estimates only)
  int* count;           // device: flagged-row counter, zeroed by the merge (exact mode), or null
  int B, S, K, V;
  int NRG;              // row groups: ceil(B*S / 128)
  int NVT;              // vocabulary tiles: ceil(V / 256)
};

// the head + reduction kernel (chunk records), and the per-row merge of those into merged[]
hipError_t launch_lmhead_reduce(const LmHeadArgs& a, hipStream_t s);
hipError_t launch_lmhead_merge(const LmHeadArgs& a, hipStream_t s);

// ---- exact mode of the fused LM head + commit: rows whose token or decision the fp32
// logits cannot settle are recomputed in fp64 from the hidden and head rows
struct ExactChunk {  // per (flagged row, vocabulary tile): exact max, lowest argmax, sum of exp
  double m;
  int32_t tok;
  int32_t pad;
  double z;
};

struct LmExactArgs {
  const void* hidden;         // [B*S][K] bf16
  const void* weight;         // [V][K] bf16
  const uint8_t* mask;        // [B*S]
  const CommitChunk* chunks;  // [B*S][NVT] fp32-logit tile records
  const CommitChunk* merged;  // [B*S] fp32-logit estimates
  const double* rowx;         // [B*S][2] runner-up and error bound
  int* flags;                 // [B*S]: list slot of a recomputed row, else -1
  int* list;                  // [B*S] recomputed rows, in arrival order
  int* count;                 // number of recomputed rows
  int* seq_state;             // [B]: fallback state of each sequence (see lmhead_exact.hip)
  uint8_t* need;              // [B*S (list order)][NVT]: tiles to recompute
  ExactChunk* exact;          // [B*S (list order)][NVT]
  float gamma;
  int32_t* token_id;
  uint8_t* committed;
  float* conf;
  int B, S, K, V, NVT;
};

hipError_t launch_lmhead_flag(const LmExactArgs& a, hipStream_t s);
hipError_t launch_lmhead_exact(const LmExactArgs& a, hipStream_t s);
hipError_t launch_lmhead_final(const LmExactArgs& a, hipStream_t s);
// the weight bound of exact mode: out = an upper bound on max_v ||weight[v]||_2
hipError_t launch_lmhead_weight_bound(const void* weight, int V, int K, float* out, hipStream_t s);

// ---------------------------------------------------------------------------------------
// the denoiser's Mamba-2 scan from the seeded state, and adaLN-single modulation
// ---------------------------------------------------------------------------------------

constexpr int kMambaChunk = 16;   // positions per chunk of the unrolled scan
constexpr int kMambaMaxP = 128;   // head width
constexpr int kMambaMaxN = 128;   // state width

struct MambaArgs {
  const void* x;         // [B,S,H,P] dtype
  const float* dt;       // [B,S,H]
  const float* dt_bias;  // [H]
  const float* A_log;    // [H]
  const float* Dskip;    // [H]
  const void* Bm;        // [B,S,G,N] dtype
  const void* Cm;        // [B,S,G,N] dtype
  const float* h0;       // [B,H,P,N] the seeded state
  void* y;               // [B,S,H,P] dtype
  float* h_out;          // [B,H,P,N] or null
  int B, S, H, P, N, G;
};

// P a power of 2 in [4, 128], N <= 128, N / (256 / P) in {4, 8, 16, 32, 64}
bool mamba_shape_supported(int P, int N);
hipError_t launch_mamba2_scan(const MambaArgs& a, int dtype, hipStream_t s);

constexpr int kAdalnMaxD = 8192;  // row width of the modulation (32 elements per thread)

struct AdalnArgs {
  const void* x;         // [B,S,d] dtype
  const void* f;         // [B,S,d] dtype (gated residual only)
  const float* t_mod;    // [B,3,d] shift, scale, gate per sequence
  const float* table;    // [3,d] the layer's offsets
  void* y;               // [B,S,d] dtype
  int B, S, d;
  float eps;
};

hipError_t launch_adaln_modulate(const AdalnArgs& a, int dtype, hipStream_t s);
hipError_t launch_adaln_gate(const AdalnArgs& a, int dtype, hipStream_t s);

}  // namespace tt
