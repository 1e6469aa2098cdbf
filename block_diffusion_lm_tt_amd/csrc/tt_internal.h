// Internal declarations shared by the libtt translation units (host launch helpers and
// the parameter blocks the kernels take). Not part of the C-ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/tt.h"

namespace tt {

// ---------------------------------------------------------------------------------------
// attention
// ---------------------------------------------------------------------------------------

constexpr int kAttnKeysPerTile = 64;   // keys staged in LDS per pipeline step
constexpr int kAttnWaves = 4;          // waves per workgroup of the MFMA kernel
constexpr int kAttnRowsPerWave = 32;   // query rows (head-in-group x block position) per wave
constexpr int kAttnRowsPerWg = kAttnWaves * kAttnRowsPerWave;
constexpr int kAttnMfmaD = 128;        // head dim of the MFMA kernel
constexpr int kMaxB = 16383;           // largest batch (the tile plan sits in LDS)

struct AttnArgs {
  const void* q;
  const void* k_blk;
  const void* v_blk;
  const void* k_ctx;
  const void* v_ctx;
  const int32_t* ctx_len;
  void* o;
  float* part;        // partial results: [n_clusters*2][NQ][rows_wg*(D+2)] fp32
  int32_t* plan;      // [B+1] tile prefix sums, written by workgroup 0 for the combine
  int B, S, Hq, Hkv, G, D, Lmax;
  int NQ;             // workgroups (query slices) per (sequence, KV head) unit
  int NC;             // clusters; each owns a contiguous range of the global tile list
  float scale_log2;   // log2(e) / sqrt(D)
};

hipError_t launch_attn_mfma(const AttnArgs& a, hipStream_t s, hipEvent_t ev_main0, hipEvent_t ev_main1);
hipError_t launch_attn_generic(const AttnArgs& a, int dtype, hipStream_t s);

// ---------------------------------------------------------------------------------------
// commit
// ---------------------------------------------------------------------------------------

struct CommitChunk {   // per (row, vocabulary chunk): partial max / argmax / sum of exp
  float m;
  int32_t tok;
  double z;
};

struct CommitRow {     // per (b, i): merged values and the decision state
  float m;
  int32_t tok;
  double z_est;        // fast estimate
  double z_exact;      // fp64 recomputation (valid when flag != 0)
  int32_t flag;        // 1 = recompute in fp64
  int32_t decided;     // 1 = committed by a sure threshold decision
};

struct CommitArgs {
  const void* logits;
  const uint8_t* mask;
  float gamma;
  int32_t* token_id;
  uint8_t* committed;
  float* conf;
  CommitChunk* chunks;  // [B*S][n_chunks]
  CommitRow* rows;      // [B*S]
  int32_t* seq_done;    // [B]
  int B, S, V;
  int n_chunks, chunk_elems;
  int dtype;
};

int commit_chunk_elems(int dtype);
hipError_t launch_commit(const CommitArgs& a, hipStream_t s, hipEvent_t ev_reduce0, hipEvent_t ev_reduce1);

}  // namespace tt
