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
  int32_t* rec;       // [NC][4] merge records: per cluster, the cut unit whose last piece it
                      // holds (b, g, 2 * first cluster + first piece's slot, list length)
                      // or b = -1; written by the main kernel, read by the combine
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
hipError_t launch_commit(const CommitArgs& a, hipStream_t s, hipEvent_t ev_reduce0, hipEvent_t ev_reduce1);
// the decide step alone (a.logits == nullptr: decisions on the chunk estimates only)
hipError_t launch_commit_decide(const CommitArgs& a, hipStream_t s);

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
  CommitChunk* merged;  // [B*S], one record per masked row
  int B, S, K, V;
  int NRG;              // row groups: ceil(B*S / 128)
  int NVT;              // vocabulary tiles: ceil(V / 256)
};

// the head + reduction kernel (chunk records), and the per-row merge of those into merged[]
hipError_t launch_lmhead_reduce(const LmHeadArgs& a, hipStream_t s);
hipError_t launch_lmhead_merge(const LmHeadArgs& a, hipStream_t s);

}  // namespace tt
