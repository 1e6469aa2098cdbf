"""The block loop of block-wise diffusion decoding on device-resident synthetic inputs.

One block of S masked positions is refined over T denoising steps; each step runs the
denoiser block attention on every layer (tt_block_denoise_attn, each layer over its own
context KV) and then the confidence commit (tt_commit) on that step's logits. Positions
committed at a step leave the masked set; at the last step every position still masked is
committed with its greedy token (the end of the block). The committed block's rows then
enter every layer's context cache (tt_ctx_append, the last layer bumping ctx_len).

Source: Nemotron-TwoTower (gist.science explainer), Technical Summary > Generation Process
(the block is refined over T steps, committed, and the context tower's caches take the
clean tokens) and the snilld.dk TwoTower article, "Blockwise generering i praksis" (several
tokens committed per step, caches updated once per block).

The loop's bookkeeping between the library calls (the still-masked set, the end-of-block
rule, the per-step counts) is the caller's policy, written here once so that the benchmark
and the parity tests run the same code. The logits of a step are seeded synthetic inputs
(no model produces them), so they do not depend on the attention outputs; the stand-in for
the context tower's rows of the committed block is the last step's block K/V of each layer.
"""
from __future__ import annotations

from typing import List, Optional

import numpy as np

from . import tensors as TZ
from . import workloads as W


class BlockLoop:
    """Device buffers of the block-loop workload ``w`` (layers > 1, steps T) on ``dev``.

    Each layer's context cache has S spare rows past Lmax (filled with NaN) so that the
    committed block's rows fit; every block starts from the workload's context lengths.
    """

    def __init__(self, w: W.Workload, dev, keep_host: bool = False):
        import torch

        from . import _lib as tt
        self.w, self.dev = w, dev
        T, L = w.steps, w.layers
        self.dt = tt.TT_BF16 if w.dtype == W.BF16 else tt.TT_F32
        self.ctx0 = torch.from_numpy(w.ctx_lens()).to(dev)
        self.ctx = self.ctx0.clone()
        self.kcs, self.vcs = [], []
        self.host_ctx_kv = [] if keep_host else None
        for l in range(L):
            x = w.attn(step=0, layer=l)
            spare = np.full((w.B, w.S, w.Hkv, w.D), W.BF16_NAN if w.dtype == W.BF16 else np.nan,
                            dtype=x.k_ctx.dtype)
            kh = np.concatenate([x.k_ctx, spare], axis=1)
            vh = np.concatenate([x.v_ctx, spare], axis=1)
            self.kcs.append(TZ.to_torch(kh, w.dtype, dev))
            self.vcs.append(TZ.to_torch(vh, w.dtype, dev))
            if keep_host:
                self.host_ctx_kv.append((kh, vh))
            del x
        self.qkv_host = [[w.block_qkv(t, l) for l in range(L)] for t in range(T)]
        self.qkv = [[tuple(TZ.to_torch(a, w.dtype, dev) for a in self.qkv_host[t][l]) for l in range(L)]
                    for t in range(T)]
        self.commits = [w.commit(step=t) for t in range(T)]
        self.logits = [TZ.commit_to_device(c, dev)[0] for c in self.commits]
        self.out = torch.empty_like(self.qkv[0][0][0])
        self.ws_a = torch.empty(max(1, tt.tt_block_denoise_attn_workspace(w.B, w.S, w.Hq, w.Hkv, w.D,
                                                                          w.Lmax + w.S, self.dt)),
                                dtype=torch.uint8, device=dev)
        self.ws_c = torch.empty(max(1, tt.tt_commit_workspace(w.B, w.S, w.V, self.dt)),
                                dtype=torch.uint8, device=dev)
        self.tok = torch.empty((w.B, w.S), dtype=torch.int32, device=dev)
        self.com = torch.empty((w.B, w.S), dtype=torch.uint8, device=dev)
        self.mask = torch.empty((w.B, w.S), dtype=torch.uint8, device=dev)
        self.counts = torch.zeros((T,), dtype=torch.int64, device=dev)
        self.ones = torch.ones((w.B, w.S), dtype=torch.uint8, device=dev)

    def run_block(self, gamma: float, record: Optional[List] = None, outs: Optional[dict] = None):
        """One block: T steps x L layers, the commits, then the cache update of every layer.

        ``record``: a list that receives, per step, device copies of (token_id, committed)
        after the end-of-block rule. ``outs``: a dict {(step, layer): None} whose entries
        receive a device copy of that attention call's output."""
        from . import _lib as tt
        w = self.w
        T, L = w.steps, w.layers
        self.mask.copy_(self.ones)
        self.ctx.copy_(self.ctx0)
        for t in range(T):
            for l in range(L):
                q, kb, vb = self.qkv[t][l]
                tt.tt_block_denoise_attn(q, kb, vb, self.kcs[l], self.vcs[l], self.ctx, out=self.out,
                                         workspace=self.ws_a)
                if outs is not None and (t, l) in outs:
                    outs[(t, l)] = self.out.clone()
            tt.tt_commit(self.logits[t], self.mask, gamma, token_id=self.tok, committed=self.com,
                         workspace=self.ws_c, want_conf=False)
            if t == T - 1:
                self.com.copy_(self.mask)  # end of the block: every position still masked commits
            if record is not None:
                record.append((self.tok.clone(), self.com.clone()))
            self.counts[t] += self.com.sum()
            self.mask.sub_(self.com)  # committed positions were masked: mask & ~committed
        for l in range(L):
            _, kb, vb = self.qkv[T - 1][l]
            tt.tt_ctx_append(kb, vb, self.kcs[l], self.vcs[l], self.ctx, bump=(l == L - 1))
