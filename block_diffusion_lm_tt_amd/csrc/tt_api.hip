// libtt C-ABI: argument validation, workspace layout, launches and kernel timing.
// The operations themselves are documented in include/tt.h.
#include <math.h>

#include <mutex>
#include <vector>

#include "tt_internal.h"

namespace tt {
namespace {

constexpr int kCUs = 256;        // MI355X compute units
constexpr int kWgPerCU = 1;      // resident MFMA-attention workgroups per CU (register bound)
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct AttnPlan {
  bool mfma;
  int NQ, NC;
  size_t plan_bytes, part_bytes;
};

tt_status plan_attn(const tt_attn_shape* sh, AttnPlan* p) {
  if (!sh) return TT_ERR_INVALID_ARG;
  if (sh->B < 0 || sh->S < 1 || sh->Hq < 1 || sh->Hkv < 1 || sh->D < 1 || sh->Lmax < 0)
    return TT_ERR_INVALID_ARG;
  if (sh->Hq % sh->Hkv != 0) return TT_ERR_INVALID_ARG;
  if (sh->dtype != TT_F32 && sh->dtype != TT_BF16) return TT_ERR_UNSUPPORTED;
  if (sh->D > 256 || sh->S > 1024 || sh->B > kMaxB) return TT_ERR_UNSUPPORTED;
  const long long lim = 1LL << 31;
  if ((long long)sh->B * sh->S * sh->Hq * sh->D >= lim) return TT_ERR_UNSUPPORTED;
  if ((long long)sh->B * sh->Lmax * sh->Hkv * sh->D >= lim) return TT_ERR_UNSUPPORTED;
  p->mfma = sh->dtype == TT_BF16 && sh->D == kAttnMfmaD;
  const int G = sh->Hq / sh->Hkv;
  p->NQ = (G * sh->S + kAttnRowsPerWg - 1) / kAttnRowsPerWg;
  int nc = (kCUs * kWgPerCU) / p->NQ;
  // a small problem takes fewer clusters, so that its units are not cut into more pieces
  // than their work warrants: at least kAttnMinTilesPerCluster tiles per cluster when every
  // context is full (ctx_len lives on the device; Lmax bounds it)
  const long long tmax = (long long)sh->B * sh->Hkv *
                         ((sh->Lmax + sh->S + kAttnKeysPerTile - 1) / kAttnKeysPerTile);
  if (tmax / kAttnMinTilesPerCluster < nc) nc = (int)(tmax / kAttnMinTilesPerCluster);
  nc = nc / 8 * 8;
  p->NC = nc < 8 ? 8 : nc;
  if (p->mfma) {
    p->plan_bytes = align_up((size_t)sh->B * sh->Hkv * 4 * sizeof(int32_t));
    p->part_bytes = align_up(attn_part_bytes(p->NC, p->NQ));
  } else {
    p->plan_bytes = p->part_bytes = 0;
  }
  return TT_OK;
}

struct CommitPlan {
  int n_chunks, chunk_elems;
  size_t chunk_bytes;
};

tt_status plan_commit(int32_t B, int32_t S, int32_t V, int32_t dtype, CommitPlan* p) {
  if (B < 0 || S < 1 || V < 1) return TT_ERR_INVALID_ARG;
  if (dtype != TT_F32 && dtype != TT_BF16) return TT_ERR_UNSUPPORTED;
  if (S > 1024) return TT_ERR_UNSUPPORTED;
  p->chunk_elems = commit_chunk_elems(dtype);
  p->n_chunks = (V + p->chunk_elems - 1) / p->chunk_elems;
  // one workgroup per (row, chunk): the launch grid bounds the shape
  if ((long long)B * S * p->n_chunks > kMaxGridBlocks) return TT_ERR_UNSUPPORTED;
  p->chunk_bytes = align_up((size_t)B * S * p->n_chunks * sizeof(CommitChunk));
  return TT_OK;
}

struct LmPlan {
  int NRG, NVT;
  size_t chunk_bytes, runner_bytes, merged_bytes;
  // exact mode
  size_t rowx_bytes, flags_bytes, list_bytes, count_bytes, state_bytes, need_bytes, exact_bytes;
  size_t base() const { return chunk_bytes + runner_bytes + merged_bytes; }
  size_t exact_total() const {
    return base() + rowx_bytes + flags_bytes + list_bytes + count_bytes + state_bytes + need_bytes + exact_bytes;
  }
};

tt_status plan_lmhead(int32_t B, int32_t S, int32_t K, int32_t V, LmPlan* p) {
  if (B < 0 || S < 1 || K < 1 || V < 1) return TT_ERR_INVALID_ARG;
  if (S > 1024 || (long long)B * S > kLmMaxRows) return TT_ERR_UNSUPPORTED;
  if (K % kLmFeaturesPerStage != 0 || K > (1 << 20)) return TT_ERR_UNSUPPORTED;
  if ((long long)B * S * K >= (1LL << 31)) return TT_ERR_UNSUPPORTED;
  p->NRG = (B * S + kLmRowsPerWg - 1) / kLmRowsPerWg;
  p->NVT = (int)(((long long)V + kLmVocabPerWg - 1) / kLmVocabPerWg);
  const size_t rows = (size_t)B * S;
  p->chunk_bytes = align_up(rows * p->NVT * sizeof(CommitChunk));
  p->runner_bytes = align_up(rows * p->NVT * sizeof(float));
  p->merged_bytes = align_up(rows * sizeof(CommitChunk));
  p->rowx_bytes = align_up(rows * 2 * sizeof(double));
  p->flags_bytes = align_up(rows * sizeof(int));
  p->list_bytes = align_up(rows * sizeof(int));
  p->count_bytes = align_up(sizeof(int));
  p->state_bytes = align_up((size_t)B * sizeof(int));
  p->need_bytes = align_up(rows * p->NVT);
  p->exact_bytes = align_up(rows * p->NVT * sizeof(ExactChunk));
  return TT_OK;
}

// ---- timing -------------------------------------------------------------------------
constexpr int kMaxTimed = 4096;

struct Profiler {
  std::mutex mu;
  bool enabled = false;
  std::vector<hipEvent_t> attn_ev[4];   // attn start, main start, main end, attn end
  std::vector<hipEvent_t> commit_ev[3]; // commit start, reduce end, commit end
  std::vector<hipEvent_t> lm_ev[3];     // LM-head commit start, reduce end, end
  int64_t attn_calls = 0, commit_calls = 0, lm_calls = 0;
  int attn_used = 0, commit_used = 0, lm_used = 0;
};
Profiler g_prof;

hipEvent_t ev_slot(std::vector<hipEvent_t>& v, int idx) {
  while ((int)v.size() <= idx) {
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    v.push_back(e);
  }
  return v[idx];
}

}  // namespace
}  // namespace tt

using namespace tt;

extern "C" {

int32_t tt_version(void) { return (1 << 16) | 1; }

#ifndef TT_SOURCE_HASH
#error "TT_SOURCE_HASH must be defined by the build (block_diffusion_lm_tt_amd/build.py)"
#endif
const char* tt_build_id(void) { return TT_SOURCE_HASH; }

const char* tt_status_str(tt_status s) {
  switch (s) {
    case TT_OK: return "TT_OK";
    case TT_ERR_INVALID_ARG: return "TT_ERR_INVALID_ARG";
    case TT_ERR_UNSUPPORTED: return "TT_ERR_UNSUPPORTED";
    case TT_ERR_WORKSPACE: return "TT_ERR_WORKSPACE";
    case TT_ERR_HIP: return "TT_ERR_HIP";
  }
  return "TT_UNKNOWN_STATUS";
}

size_t tt_block_denoise_attn_workspace(const tt_attn_shape* shape) {
  AttnPlan p;
  if (plan_attn(shape, &p) != TT_OK) return 0;
  const size_t n = p.plan_bytes + p.part_bytes;
  return n < kAlign ? kAlign : n;
}

tt_status tt_block_denoise_attn(const tt_attn_shape* shape, const void* q, const void* k_blk,
                                const void* v_blk, const void* k_ctx, const void* v_ctx,
                                const int32_t* ctx_len, void* o, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  AttnPlan p;
  tt_status st = plan_attn(shape, &p);
  if (st != TT_OK) return st;
  if (shape->B == 0) return TT_OK;
  if (!q || !k_blk || !v_blk || !ctx_len || !o) return TT_ERR_INVALID_ARG;
  if (shape->Lmax > 0 && (!k_ctx || !v_ctx)) return TT_ERR_INVALID_ARG;
  const size_t need = tt_block_denoise_attn_workspace(shape);
  if (!workspace || workspace_bytes < need) return TT_ERR_WORKSPACE;
  // the MFMA path copies 16-byte pieces: a base off that boundary takes the element-wise path
  const uintptr_t bases = (uintptr_t)q | (uintptr_t)k_blk | (uintptr_t)v_blk | (uintptr_t)k_ctx |
                          (uintptr_t)v_ctx | (uintptr_t)o;
  const bool mfma = p.mfma && bases % 16 == 0;

  AttnArgs a;
  a.q = q;
  a.k_blk = k_blk;
  a.v_blk = v_blk;
  a.k_ctx = k_ctx;
  a.v_ctx = v_ctx;
  a.ctx_len = ctx_len;
  a.o = o;
  a.rec = static_cast<int32_t*>(workspace);
  a.part = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.plan_bytes);
  a.B = shape->B;
  a.S = shape->S;
  a.Hq = shape->Hq;
  a.Hkv = shape->Hkv;
  a.G = shape->Hq / shape->Hkv;
  a.D = shape->D;
  a.Lmax = shape->Lmax;
  a.NQ = p.NQ;
  a.NC = p.NC;
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)shape->D));

  hipEvent_t ev[4] = {nullptr, nullptr, nullptr, nullptr};
  {
    std::lock_guard<std::mutex> lk(g_prof.mu);
    if (g_prof.enabled) {
      ++g_prof.attn_calls;
      if (g_prof.attn_used < kMaxTimed) {
        for (int k = 0; k < 4; ++k) ev[k] = ev_slot(g_prof.attn_ev[k], g_prof.attn_used);
        if (ev[0] && ev[1] && ev[2] && ev[3]) ++g_prof.attn_used;
        else ev[0] = ev[1] = ev[2] = ev[3] = nullptr;
      }
    }
  }
  if (ev[0]) (void)hipEventRecord(ev[0], stream);
  hipError_t e;
  if (mfma) {
    e = launch_attn_mfma(a, stream, ev[1], ev[2]);
  } else {
    if (ev[1]) (void)hipEventRecord(ev[1], stream);
    e = launch_attn_generic(a, shape->dtype, stream);
    if (ev[2]) (void)hipEventRecord(ev[2], stream);
  }
  if (ev[3]) (void)hipEventRecord(ev[3], stream);
  return e == hipSuccess ? TT_OK : TT_ERR_HIP;
}

size_t tt_commit_workspace(int32_t B, int32_t S, int32_t V, int32_t dtype) {
  CommitPlan p;
  if (plan_commit(B, S, V, dtype, &p) != TT_OK) return 0;
  const size_t n = p.chunk_bytes;
  return n < kAlign ? kAlign : n;
}

tt_status tt_commit(int32_t B, int32_t S, int32_t V, int32_t dtype, const void* logits,
                    const uint8_t* mask, float gamma, int32_t* token_id, uint8_t* committed,
                    float* conf, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  CommitPlan p;
  tt_status st = plan_commit(B, S, V, dtype, &p);
  if (st != TT_OK) return st;
  if (isnan(gamma)) return TT_ERR_INVALID_ARG;
  if (B == 0) return TT_OK;
  if (!logits || !mask || !token_id || !committed) return TT_ERR_INVALID_ARG;
  const size_t need = tt_commit_workspace(B, S, V, dtype);
  if (!workspace || workspace_bytes < need) return TT_ERR_WORKSPACE;

  CommitArgs a;
  a.logits = logits;
  a.mask = mask;
  a.gamma = gamma;
  a.token_id = token_id;
  a.committed = committed;
  a.conf = conf;
  char* ws = static_cast<char*>(workspace);
  a.chunks = reinterpret_cast<CommitChunk*>(ws);
  a.B = B;
  a.S = S;
  a.V = V;
  a.n_chunks = p.n_chunks;
  a.chunk_elems = p.chunk_elems;
  a.dtype = dtype;

  hipEvent_t ev[3] = {nullptr, nullptr, nullptr};
  {
    std::lock_guard<std::mutex> lk(g_prof.mu);
    if (g_prof.enabled) {
      ++g_prof.commit_calls;
      if (g_prof.commit_used < kMaxTimed) {
        for (int k = 0; k < 3; ++k) ev[k] = ev_slot(g_prof.commit_ev[k], g_prof.commit_used);
        if (ev[0] && ev[1] && ev[2]) ++g_prof.commit_used;
        else ev[0] = ev[1] = ev[2] = nullptr;
      }
    }
  }
  if (ev[0]) (void)hipEventRecord(ev[0], stream);
  hipError_t e = launch_commit(a, stream, ev[1]);
  if (ev[2]) (void)hipEventRecord(ev[2], stream);
  return e == hipSuccess ? TT_OK : TT_ERR_HIP;
}

tt_status tt_commit_noalloc(int32_t B, int32_t S, int32_t V, int32_t dtype, const void* logits,
                            const uint8_t* mask, float gamma, int32_t* token_id, uint8_t* committed,
                            float* conf, hipStream_t stream) {
  CommitPlan p;
  tt_status st = plan_commit(B, S, V, dtype, &p);
  if (st != TT_OK) return st;
  if (isnan(gamma)) return TT_ERR_INVALID_ARG;
  if (B == 0) return TT_OK;
  if (!logits || !mask || !token_id || !committed) return TT_ERR_INVALID_ARG;
  if (p.chunk_bytes > kCommitScratchBytes) return TT_ERR_UNSUPPORTED;
  void* ws = nullptr;
  if (commit_scratch(&ws) != hipSuccess) return TT_ERR_HIP;

  CommitArgs a;
  a.logits = logits;
  a.mask = mask;
  a.gamma = gamma;
  a.token_id = token_id;
  a.committed = committed;
  a.conf = conf;
  a.chunks = static_cast<CommitChunk*>(ws);
  a.B = B;
  a.S = S;
  a.V = V;
  a.n_chunks = p.n_chunks;
  a.chunk_elems = p.chunk_elems;
  a.dtype = dtype;
  return launch_commit(a, stream, nullptr) == hipSuccess ? TT_OK : TT_ERR_HIP;
}

size_t tt_lmhead_commit_workspace(int32_t B, int32_t S, int32_t K, int32_t V) {
  LmPlan p;
  if (plan_lmhead(B, S, K, V, &p) != TT_OK) return 0;
  return p.base();
}

tt_status tt_lmhead_commit(int32_t B, int32_t S, int32_t K, int32_t V, const void* hidden,
                           const void* weight, const uint8_t* mask, float gamma,
                           int32_t* token_id, uint8_t* committed, float* conf, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  LmPlan p;
  tt_status st = plan_lmhead(B, S, K, V, &p);
  if (st != TT_OK) return st;
  if (isnan(gamma)) return TT_ERR_INVALID_ARG;
  if (B == 0) return TT_OK;
  if (!hidden || !weight || !mask || !token_id || !committed) return TT_ERR_INVALID_ARG;
  if (((uintptr_t)hidden | (uintptr_t)weight) % 16 != 0) return TT_ERR_UNSUPPORTED;  // 16-byte loads
  const size_t need = tt_lmhead_commit_workspace(B, S, K, V);
  if (!workspace || workspace_bytes < need) return TT_ERR_WORKSPACE;

  LmHeadArgs l;
  l.hidden = hidden;
  l.weight = weight;
  l.mask = mask;
  char* ws = static_cast<char*>(workspace);
  l.chunks = reinterpret_cast<CommitChunk*>(ws);
  l.runner = reinterpret_cast<float*>(ws + p.chunk_bytes);
  l.merged = reinterpret_cast<CommitChunk*>(ws + p.chunk_bytes + p.runner_bytes);
  l.rowx = nullptr;
  l.w_bound = nullptr;
  l.count = nullptr;
  l.B = B;
  l.S = S;
  l.K = K;
  l.V = V;
  l.NRG = p.NRG;
  l.NVT = p.NVT;

  CommitArgs c;
  c.logits = nullptr;  // decisions on the chunk estimates (the logits are never stored)
  c.mask = mask;
  c.gamma = gamma;
  c.token_id = token_id;
  c.committed = committed;
  c.conf = conf;
  c.chunks = l.merged;
  c.B = B;
  c.S = S;
  c.V = V;
  c.n_chunks = 1;
  c.chunk_elems = V;
  c.dtype = TT_BF16;

  hipEvent_t ev[3] = {nullptr, nullptr, nullptr};
  {
    std::lock_guard<std::mutex> lk(g_prof.mu);
    if (g_prof.enabled) {
      ++g_prof.lm_calls;
      if (g_prof.lm_used < kMaxTimed) {
        for (int k = 0; k < 3; ++k) ev[k] = ev_slot(g_prof.lm_ev[k], g_prof.lm_used);
        if (ev[0] && ev[1] && ev[2]) ++g_prof.lm_used;
        else ev[0] = ev[1] = ev[2] = nullptr;
      }
    }
  }
  if (ev[0]) (void)hipEventRecord(ev[0], stream);
  hipError_t e = launch_lmhead_reduce(l, stream);
  if (e != hipSuccess) return TT_ERR_HIP;
  if (ev[1]) (void)hipEventRecord(ev[1], stream);
  e = launch_lmhead_merge(l, stream);
  if (e != hipSuccess) return TT_ERR_HIP;
  e = launch_commit_decide(c, stream);
  if (ev[2]) (void)hipEventRecord(ev[2], stream);
  return e == hipSuccess ? TT_OK : TT_ERR_HIP;
}

tt_status tt_lmhead_weight_bound(const void* weight, int32_t V, int32_t K, float* bound, hipStream_t stream) {
  if (V < 0 || K < 1) return TT_ERR_INVALID_ARG;
  if ((long long)V * K >= (1LL << 40)) return TT_ERR_UNSUPPORTED;
  if (!bound || (V > 0 && !weight)) return TT_ERR_INVALID_ARG;
  return launch_lmhead_weight_bound(weight, V, K, bound, stream) == hipSuccess ? TT_OK : TT_ERR_HIP;
}

size_t tt_lmhead_commit_exact_workspace(int32_t B, int32_t S, int32_t K, int32_t V) {
  LmPlan p;
  if (plan_lmhead(B, S, K, V, &p) != TT_OK) return 0;
  return p.exact_total();
}

tt_status tt_lmhead_commit_exact(int32_t B, int32_t S, int32_t K, int32_t V, const void* hidden,
                                 const void* weight, const uint8_t* mask, float gamma, const float* w_bound,
                                 int32_t* token_id, uint8_t* committed, float* conf, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  LmPlan p;
  tt_status st = plan_lmhead(B, S, K, V, &p);
  if (st != TT_OK) return st;
  if (isnan(gamma)) return TT_ERR_INVALID_ARG;
  if (B == 0) return TT_OK;
  if (!hidden || !weight || !mask || !w_bound || !token_id || !committed) return TT_ERR_INVALID_ARG;
  if (((uintptr_t)hidden | (uintptr_t)weight) % 16 != 0) return TT_ERR_UNSUPPORTED;  // 16-byte loads
  const size_t need = tt_lmhead_commit_exact_workspace(B, S, K, V);
  if (!workspace || workspace_bytes < need) return TT_ERR_WORKSPACE;

  char* ws = static_cast<char*>(workspace);
  size_t off = 0;
  auto take = [&](size_t n) {
    char* q = ws + off;
    off += n;
    return q;
  };
  LmHeadArgs l;
  l.hidden = hidden;
  l.weight = weight;
  l.mask = mask;
  l.chunks = reinterpret_cast<CommitChunk*>(take(p.chunk_bytes));
  l.runner = reinterpret_cast<float*>(take(p.runner_bytes));
  l.merged = reinterpret_cast<CommitChunk*>(take(p.merged_bytes));
  l.rowx = reinterpret_cast<double*>(take(p.rowx_bytes));
  l.w_bound = w_bound;
  LmExactArgs x;
  x.flags = reinterpret_cast<int*>(take(p.flags_bytes));
  x.list = reinterpret_cast<int*>(take(p.list_bytes));
  x.count = reinterpret_cast<int*>(take(p.count_bytes));
  x.seq_state = reinterpret_cast<int*>(take(p.state_bytes));
  x.need = reinterpret_cast<uint8_t*>(take(p.need_bytes));
  x.exact = reinterpret_cast<ExactChunk*>(take(p.exact_bytes));
  l.count = x.count;
  l.B = B;
  l.S = S;
  l.K = K;
  l.V = V;
  l.NRG = p.NRG;
  l.NVT = p.NVT;
  x.hidden = hidden;
  x.weight = weight;
  x.mask = mask;
  x.chunks = l.chunks;
  x.merged = l.merged;
  x.rowx = l.rowx;
  x.gamma = gamma;
  x.token_id = token_id;
  x.committed = committed;
  x.conf = conf;
  x.B = B;
  x.S = S;
  x.K = K;
  x.V = V;
  x.NVT = p.NVT;

  hipError_t e = launch_lmhead_reduce(l, stream);
  if (e == hipSuccess) e = launch_lmhead_merge(l, stream);
  if (e == hipSuccess) e = launch_lmhead_flag(x, stream);
  if (e == hipSuccess) e = launch_lmhead_exact(x, stream);
  if (e == hipSuccess) e = launch_lmhead_final(x, stream);
  return e == hipSuccess ? TT_OK : TT_ERR_HIP;
}

tt_status tt_ctx_append(const tt_attn_shape* shape, const void* k_new, const void* v_new,
                        void* k_ctx, void* v_ctx, int32_t* ctx_len, int32_t bump, uint8_t* skipped,
                        hipStream_t stream) {
  if (!shape) return TT_ERR_INVALID_ARG;
  const tt_attn_shape& sh = *shape;
  if (sh.B < 0 || sh.S < 1 || sh.Hkv < 1 || sh.D < 1 || sh.Lmax < 0) return TT_ERR_INVALID_ARG;
  if (sh.dtype != TT_F32 && sh.dtype != TT_BF16) return TT_ERR_UNSUPPORTED;
  if (sh.B > kMaxB || sh.S > 1024 || sh.D > 256) return TT_ERR_UNSUPPORTED;
  if ((long long)sh.B * sh.Lmax * sh.Hkv * sh.D >= (1LL << 31)) return TT_ERR_UNSUPPORTED;
  if ((long long)sh.B * sh.S * sh.Hkv * sh.D >= (1LL << 31)) return TT_ERR_UNSUPPORTED;
  if (sh.B == 0) return TT_OK;
  if (!k_new || !v_new || !k_ctx || !v_ctx || !ctx_len) return TT_ERR_INVALID_ARG;
  AppendArgs a;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_ctx = k_ctx;
  a.v_ctx = v_ctx;
  a.ctx_len = ctx_len;
  a.skipped = skipped;
  a.B = sh.B;
  a.S = sh.S;
  a.Lmax = sh.Lmax;
  a.elt = sh.dtype == TT_F32 ? 4 : 2;
  a.row_bytes = (size_t)sh.Hkv * sh.D * a.elt;
  a.bump = bump != 0;
  const uintptr_t bases = (uintptr_t)k_new | (uintptr_t)v_new | (uintptr_t)k_ctx | (uintptr_t)v_ctx;
  a.vec16 = (a.row_bytes % 16 == 0) && (bases % 16 == 0);
  return launch_ctx_append(a, stream) == hipSuccess ? TT_OK : TT_ERR_HIP;
}

tt_status tt_mamba2_seeded_scan(const tt_mamba_shape* shape, const void* x, const float* dt,
                                const float* dt_bias, const float* A_log, const float* Dskip,
                                const void* Bm, const void* Cm, const float* h0, void* y, float* h_out,
                                hipStream_t stream) {
  if (!shape) return TT_ERR_INVALID_ARG;
  const tt_mamba_shape& sh = *shape;
  if (sh.B < 0 || sh.S < 1 || sh.H < 1 || sh.P < 1 || sh.N < 1 || sh.G < 1 || sh.H % sh.G != 0)
    return TT_ERR_INVALID_ARG;
  if (sh.dtype != TT_F32 && sh.dtype != TT_BF16) return TT_ERR_UNSUPPORTED;
  if (!mamba_shape_supported(sh.P, sh.N) || sh.S > 1024) return TT_ERR_UNSUPPORTED;
  if ((long long)sh.B * sh.H > kMaxGridBlocks) return TT_ERR_UNSUPPORTED;
  if ((long long)sh.B * sh.S * sh.H * sh.P >= (1LL << 31) || (long long)sh.B * sh.H * sh.P * sh.N >= (1LL << 31) ||
      (long long)sh.B * sh.S * sh.G * sh.N >= (1LL << 31))
    return TT_ERR_UNSUPPORTED;
  if (sh.B == 0) return TT_OK;
  if (!x || !dt || !dt_bias || !A_log || !Dskip || !Bm || !Cm || !h0 || !y) return TT_ERR_INVALID_ARG;
  if (((uintptr_t)h0 | (uintptr_t)h_out) % 16 != 0) return TT_ERR_UNSUPPORTED;  // 16-byte state loads
  MambaArgs a;
  a.x = x;
  a.dt = dt;
  a.dt_bias = dt_bias;
  a.A_log = A_log;
  a.Dskip = Dskip;
  a.Bm = Bm;
  a.Cm = Cm;
  a.h0 = h0;
  a.y = y;
  a.h_out = h_out;
  a.B = sh.B;
  a.S = sh.S;
  a.H = sh.H;
  a.P = sh.P;
  a.N = sh.N;
  a.G = sh.G;
  return launch_mamba2_scan(a, sh.dtype, stream) == hipSuccess ? TT_OK : TT_ERR_HIP;
}

static tt_status adaln_args(int32_t B, int32_t S, int32_t d, int32_t dtype, const void* x, const float* t_mod,
                            const float* table, void* y, AdalnArgs* a) {
  if (B < 0 || S < 1 || d < 1) return TT_ERR_INVALID_ARG;
  if (dtype != TT_F32 && dtype != TT_BF16) return TT_ERR_UNSUPPORTED;
  if (d > kAdalnMaxD || (long long)B * S > kMaxGridBlocks || (long long)B * S * d >= (1LL << 31))
    return TT_ERR_UNSUPPORTED;
  if (B == 0) return TT_OK;
  if (!x || !t_mod || !table || !y) return TT_ERR_INVALID_ARG;
  a->x = x;
  a->f = nullptr;
  a->t_mod = t_mod;
  a->table = table;
  a->y = y;
  a->B = B;
  a->S = S;
  a->d = d;
  a->eps = 0.0f;
  return TT_OK;
}

tt_status tt_adaln_modulate(int32_t B, int32_t S, int32_t d, int32_t dtype, const void* x, const float* t_mod,
                            const float* table, float eps, void* y, hipStream_t stream) {
  AdalnArgs a;
  if (!(eps >= 0.0f) || isinf(eps)) return TT_ERR_INVALID_ARG;
  const tt_status st = adaln_args(B, S, d, dtype, x, t_mod, table, y, &a);
  if (st != TT_OK || B == 0) return st;
  a.eps = eps;
  return launch_adaln_modulate(a, dtype, stream) == hipSuccess ? TT_OK : TT_ERR_HIP;
}

tt_status tt_adaln_gate(int32_t B, int32_t S, int32_t d, int32_t dtype, const void* x, const void* f,
                        const float* t_mod, const float* table, void* out, hipStream_t stream) {
  AdalnArgs a;
  const tt_status st = adaln_args(B, S, d, dtype, x, t_mod, table, out, &a);
  if (st != TT_OK || B == 0) return st;
  if (!f) return TT_ERR_INVALID_ARG;
  a.f = f;
  return launch_adaln_gate(a, dtype, stream) == hipSuccess ? TT_OK : TT_ERR_HIP;
}

tt_status tt_profile_enable(int32_t enable) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  g_prof.enabled = enable != 0;
  return TT_OK;
}

tt_status tt_profile_reset(void) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  g_prof.attn_calls = g_prof.commit_calls = g_prof.lm_calls = 0;
  g_prof.attn_used = g_prof.commit_used = g_prof.lm_used = 0;
  return TT_OK;
}

tt_status tt_profile_read(tt_profile_stats* out) {
  if (!out) return TT_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(g_prof.mu);
  tt_profile_stats s = {};
  float ms = 0.0f;
  for (int k = 0; k < g_prof.attn_used; ++k) {
    if (hipEventSynchronize(g_prof.attn_ev[3][k]) != hipSuccess) return TT_ERR_HIP;
    if (hipEventElapsedTime(&ms, g_prof.attn_ev[0][k], g_prof.attn_ev[3][k]) != hipSuccess) return TT_ERR_HIP;
    s.attn_total_ms += ms;
    if (hipEventElapsedTime(&ms, g_prof.attn_ev[1][k], g_prof.attn_ev[2][k]) != hipSuccess) return TT_ERR_HIP;
    s.attn_main_ms += ms;
  }
  for (int k = 0; k < g_prof.commit_used; ++k) {
    if (hipEventSynchronize(g_prof.commit_ev[2][k]) != hipSuccess) return TT_ERR_HIP;
    if (hipEventElapsedTime(&ms, g_prof.commit_ev[0][k], g_prof.commit_ev[2][k]) != hipSuccess) return TT_ERR_HIP;
    s.commit_total_ms += ms;
    if (hipEventElapsedTime(&ms, g_prof.commit_ev[0][k], g_prof.commit_ev[1][k]) != hipSuccess) return TT_ERR_HIP;
    s.commit_reduce_ms += ms;
  }
  for (int k = 0; k < g_prof.lm_used; ++k) {
    if (hipEventSynchronize(g_prof.lm_ev[2][k]) != hipSuccess) return TT_ERR_HIP;
    if (hipEventElapsedTime(&ms, g_prof.lm_ev[0][k], g_prof.lm_ev[2][k]) != hipSuccess) return TT_ERR_HIP;
    s.lm_total_ms += ms;
    if (hipEventElapsedTime(&ms, g_prof.lm_ev[0][k], g_prof.lm_ev[1][k]) != hipSuccess) return TT_ERR_HIP;
    s.lm_reduce_ms += ms;
  }
  s.attn_calls = g_prof.attn_used;
  s.commit_calls = g_prof.commit_used;
  s.lm_calls = g_prof.lm_used;
  *out = s;
  return TT_OK;
}

}  // extern "C"
