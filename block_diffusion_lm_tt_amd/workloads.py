"""Seeded synthetic inputs for the block-denoise attention and the confidence commit.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic. Both the HIP path and the CPU oracle are fed the very same
bytes from here, so a parity test compares two computations on identical inputs.

Conventions
-----------
* numpy PCG64 streams, one per tensor: ``SeedSequence([seed, tensor_id, step, layer])``.
* fp32 draws are rounded to bfloat16 with round-to-nearest-even; bf16 tensors are
  carried as ``uint16`` bit patterns (numpy has no bfloat16 type).
* Layouts (all row-major, last index fastest):
  ``q[B,S,Hq,D]``, ``k_blk/v_blk[B,S,Hkv,D]``, ``k_ctx/v_ctx[B,Lmax,Hkv,D]``,
  ``ctx_len[B]`` int32, ``logits[B,S,V]``, ``mask[B,S]`` uint8 (1 = still masked).
* Context rows ``[ctx_len[b], Lmax)`` are padding. By default they are filled with
  NaN so that any read of them shows up in the output.

The five workload specs mirror the method's deployment point (block size 16, the
gamma threshold, GQA groups of 16 query heads per KV head, 128-wide heads) as stated
on the pages "Nemotron-TwoTower: Diffusion Language Modeling with Pretrained
Autoregressive Context" (Technical Summary > Generation Process; Training and
Conditioning > Sampling) and the snilld.dk article on TwoTower (Blockwise generering
i praksis).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

F32 = "f32"
BF16 = "bf16"

# tensor ids for the per-tensor random streams
(_T_Q, _T_KB, _T_VB, _T_KC, _T_VC, _T_LEN, _T_LOGIT, _T_MASK, _T_PEAK, _T_BIAS, _T_HID, _T_HEAD, _T_MX, _T_MDT,
 _T_MPAR, _T_MB, _T_MC, _T_MH0, _T_AX, _T_AF, _T_AT) = range(21)

BF16_NAN = np.uint16(0x7FC0)


def _rng(seed: int, tensor: int, step: int = 0, layer: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor, step, layer])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to fp32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(rng: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def _encode(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == F32:
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == BF16:
        return f32_to_bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


@dataclasses.dataclass
class AttnInputs:
    B: int
    S: int
    Hq: int
    Hkv: int
    D: int
    Lmax: int
    dtype: str
    q: np.ndarray
    k_blk: np.ndarray
    v_blk: np.ndarray
    k_ctx: np.ndarray
    v_ctx: np.ndarray
    ctx_len: np.ndarray  # int32 [B]
    # planted hot keys (make_attn with hot_keys): {(b, g): context positions}, else None
    hot: Optional[dict] = None

    @property
    def ctx_kv_bytes(self) -> int:
        """Bytes of valid context K and V (the stream that bounds the kernel)."""
        elt = 4 if self.dtype == F32 else 2
        return 2 * self.Hkv * self.D * elt * int(self.ctx_len.astype(np.int64).sum())


@dataclasses.dataclass
class CommitInputs:
    B: int
    S: int
    V: int
    dtype: str
    logits: np.ndarray
    mask: np.ndarray  # uint8 [B,S]
    gamma: float

    @property
    def masked_row_bytes(self) -> int:
        elt = 4 if self.dtype == F32 else 2
        return int(self.mask.astype(np.int64).sum()) * self.V * elt


@dataclasses.dataclass
class LmHeadInputs:
    B: int
    S: int
    K: int          # d_model
    V: int
    hidden: np.ndarray  # uint16 (bf16 bits) [B,S,K]
    weight: np.ndarray  # uint16 (bf16 bits) [V,K], one row per vocabulary entry
    mask: np.ndarray    # uint8 [B,S]
    gamma: float


def make_lmhead(B: int, S: int, K: int, V: int, seed: int = 0, step: int = 0, gamma: float = 0.8,
                mask: Optional[np.ndarray] = None, sigma: float = 3.0,
                peaks: Optional[dict] = None) -> LmHeadInputs:
    """Hidden states N(0, 1) [B,S,K] and LM-head weights N(0, sigma/sqrt(K)) [V,K], both
    rounded to bf16, so that a logit has standard deviation about sigma.

    ``peaks``: ``{"p": 0.6, "low": 8.0, "high": 14.0}`` picks, independently per position
    with probability p, a random token v and a height h ~ U(low, high), and adds
    (h / |w_v|^2) * w_v to the position's hidden state (before rounding): that token's
    logit rises by about h.
    """
    wsc = float(sigma) / math.sqrt(K)
    rw = _rng(seed, _T_HEAD)
    w32 = np.empty((V, K), dtype=np.float32)
    for v0 in range(0, V, 8192):  # chunked draws keep the fp32 staging small
        w32[v0:v0 + 8192] = _normal(rw, (min(8192, V - v0), K), wsc)
    w = f32_to_bf16_bits(w32)
    del w32
    h = _normal(_rng(seed, _T_HID, step), (B, S, K))
    if peaks:
        rp = _rng(seed, _T_PEAK, step)
        hit = rp.random((B, S)) < float(peaks.get("p", 0.6))
        ids = rp.integers(0, V, size=(B, S))
        ht = rp.uniform(float(peaks.get("low", 8.0)), float(peaks.get("high", 14.0)), size=(B, S))
        for b, i in zip(*np.nonzero(hit)):
            wv = bf16_bits_to_f32(w[ids[b, i]]).astype(np.float64)
            h[b, i] += (ht[b, i] / float(wv @ wv) * wv).astype(np.float32)
    if mask is None:
        mask = np.ones((B, S), dtype=np.uint8)
    return LmHeadInputs(B, S, K, V, f32_to_bf16_bits(h), w, np.ascontiguousarray(mask, dtype=np.uint8),
                        float(np.float32(gamma)))


@dataclasses.dataclass
class MambaInputs:
    B: int
    S: int
    H: int
    P: int
    N: int
    G: int
    dtype: str
    x: np.ndarray        # [B,S,H,P] dtype
    dt: np.ndarray       # [B,S,H] fp32 (before the softplus)
    dt_bias: np.ndarray  # [H] fp32
    A_log: np.ndarray    # [H] fp32
    Dskip: np.ndarray    # [H] fp32
    Bm: np.ndarray       # [B,S,G,N] dtype
    Cm: np.ndarray       # [B,S,G,N] dtype
    h0: np.ndarray       # [B,H,P,N] fp32, the seeded state


def make_mamba(B: int, S: int, H: int, P: int, N: int, G: int, dtype: str = BF16, seed: int = 0,
               step: int = 0, layer: int = 0) -> MambaInputs:
    """Inputs of the denoiser's Mamba-2 scan from a seeded state: x ~ N(0,1) and B, C ~ N(0, 1/N)
    (so that B . C has unit variance), dt ~ N(0, 0.5), step biases placing softplus(dt_bias)
    log-uniformly in [1e-3, 1e-1], A_log = log U(1, 16), D ~ U(0.5, 1.5), and a seeded state
    ~ N(0, 0.5^2) (the context tower's state for the layer)."""
    x = _normal(_rng(seed, _T_MX, step, layer), (B, S, H, P))
    dt = _normal(_rng(seed, _T_MDT, step, layer), (B, S, H), 0.5)
    r = _rng(seed, _T_MPAR, 0, layer)
    dt0 = np.exp(r.uniform(np.log(1e-3), np.log(1e-1), H))
    dt_bias = np.log(np.expm1(dt0)).astype(np.float32)
    A_log = np.log(r.uniform(1.0, 16.0, H)).astype(np.float32)
    Dskip = r.uniform(0.5, 1.5, H).astype(np.float32)
    Bm = _normal(_rng(seed, _T_MB, step, layer), (B, S, G, N), 1.0 / math.sqrt(N))
    Cm = _normal(_rng(seed, _T_MC, step, layer), (B, S, G, N), 1.0 / math.sqrt(N))
    h0 = _normal(_rng(seed, _T_MH0, 0, layer), (B, H, P, N), 0.5)
    return MambaInputs(B, S, H, P, N, G, dtype, _encode(x, dtype), dt, dt_bias, A_log, Dskip, _encode(Bm, dtype),
                       _encode(Cm, dtype), h0)


@dataclasses.dataclass
class AdalnInputs:
    B: int
    S: int
    d: int
    dtype: str
    x: np.ndarray       # [B,S,d] dtype
    f: np.ndarray       # [B,S,d] dtype (the mixer's output, for the gated residual)
    t_mod: np.ndarray   # [B,3,d] fp32: shift, scale, gate of each sequence's timestep
    table: np.ndarray   # [3,d] fp32: the layer's offsets


def make_adaln(B: int, S: int, d: int, dtype: str = BF16, seed: int = 0, layer: int = 0) -> AdalnInputs:
    """adaLN-single inputs: rows x ~ 0.2 + N(0, 1.5^2) (a nonzero mean for the normalization
    to remove), mixer outputs f ~ N(0,1), per-sequence vectors t_mod ~ N(0, 0.5^2) and the
    layer's offsets ~ N(0, 0.1^2)."""
    x = _normal(_rng(seed, _T_AX, 0, layer), (B, S, d), 1.5) + np.float32(0.2)
    f = _normal(_rng(seed, _T_AF, 0, layer), (B, S, d))
    rt = _rng(seed, _T_AT, 0, layer)
    t_mod = (rt.standard_normal((B, 3, d)) * 0.5).astype(np.float32)
    table = (rt.standard_normal((3, d)) * 0.1).astype(np.float32)
    return AdalnInputs(B, S, d, dtype, _encode(x, dtype), _encode(f, dtype), t_mod, table)


def make_attn(B: int, S: int, Hq: int, Hkv: int, D: int, ctx_lens: Sequence[int] | np.ndarray,
              Lmax: Optional[int] = None, dtype: str = BF16, seed: int = 0, step: int = 0,
              layer: int = 0, pad_fill: str = "nan", hot_keys: Optional[dict] = None) -> AttnInputs:
    """Draw i.i.d. N(0,1) block and context Q/K/V for the given shape.

    ``hot_keys`` (optional) plants concentrated attention: ``{"frac": 0.01, "boost": 8.0,
    "bias_norm": 2.0}`` adds, per KV head g, a random unit direction u_g scaled by
    kappa = sqrt(boost*sqrt(D)) to a seeded ``frac`` of each sequence's context keys and
    to every query of that group, plus ``bias_norm * u_g`` to all context keys.
    """
    ctx = np.asarray(ctx_lens, dtype=np.int32).reshape(B)
    if Lmax is None:
        Lmax = int(ctx.max()) if B else 0
    if (ctx < 0).any() or (ctx > Lmax).any():
        raise ValueError("ctx_len out of range")
    q = _normal(_rng(seed, _T_Q, step, layer), (B, S, Hq, D))
    kb = _normal(_rng(seed, _T_KB, step, layer), (B, S, Hkv, D))
    vb = _normal(_rng(seed, _T_VB, step, layer), (B, S, Hkv, D))
    kc = np.empty((B, Lmax, Hkv, D), dtype=np.float32)
    vc = np.empty((B, Lmax, Hkv, D), dtype=np.float32)
    rk = _rng(seed, _T_KC, 0, layer)
    rv = _rng(seed, _T_VC, 0, layer)
    for b in range(B):
        n = int(ctx[b])
        kc[b, :n] = _normal(rk, (n, Hkv, D))
        vc[b, :n] = _normal(rv, (n, Hkv, D))
    hot_sets = {} if hot_keys else None
    if hot_keys:
        G = Hq // Hkv
        kappa = math.sqrt(float(hot_keys.get("boost", 8.0)) * math.sqrt(D))
        rb = _rng(seed, _T_BIAS, 0, layer)
        for g in range(Hkv):
            u = rb.standard_normal(D).astype(np.float32)
            u /= np.float32(np.linalg.norm(u))
            for b in range(B):
                n = int(ctx[b])
                kc[b, :n, g] += np.float32(hot_keys.get("bias_norm", 2.0)) * u
                nh = int(math.ceil(float(hot_keys.get("frac", 0.01)) * n))
                if nh:
                    hot = rb.choice(n, size=nh, replace=False)
                    kc[b, hot, g] += np.float32(kappa) * u
                    hot_sets[(b, g)] = np.sort(hot)
            q[:, :, g * G:(g + 1) * G] += np.float32(kappa) * u
    # padding rows
    if dtype == BF16:
        kc_e, vc_e = _encode(kc, dtype), _encode(vc, dtype)
        fillv = BF16_NAN if pad_fill == "nan" else np.uint16(0)
    else:
        kc_e, vc_e = kc, vc
        fillv = np.float32(np.nan) if pad_fill == "nan" else np.float32(0)
    for b in range(B):
        n = int(ctx[b])
        kc_e[b, n:] = fillv
        vc_e[b, n:] = fillv
    return AttnInputs(B, S, Hq, Hkv, D, Lmax, dtype, _encode(q, dtype), _encode(kb, dtype),
                      _encode(vb, dtype), kc_e, vc_e, ctx, hot_sets)


def make_block_qkv(B: int, S: int, Hq: int, Hkv: int, D: int, dtype: str = BF16, seed: int = 0,
                   step: int = 0, layer: int = 0):
    """The block's (q, k_blk, v_blk) of one (step, layer): the same draws as ``make_attn``
    (without hot keys), without drawing the context again."""
    q = _normal(_rng(seed, _T_Q, step, layer), (B, S, Hq, D))
    kb = _normal(_rng(seed, _T_KB, step, layer), (B, S, Hkv, D))
    vb = _normal(_rng(seed, _T_VB, step, layer), (B, S, Hkv, D))
    return _encode(q, dtype), _encode(kb, dtype), _encode(vb, dtype)


def make_commit(B: int, S: int, V: int, dtype: str = BF16, sigma: float = 3.0, seed: int = 0,
                step: int = 0, gamma: float = 0.8, mask: Optional[np.ndarray] = None,
                peaks: Optional[dict] = None) -> CommitInputs:
    """Logits N(0, sigma) (sigma is the standard deviation) with optional planted peaks.

    ``peaks``: ``{"mode": "half", "height": 12.0}`` plants one peak at a random vocab id in
    exactly floor(S/2) seeded positions of each sequence; ``{"mode": "bernoulli", "p": 0.6,
    "low": 8.0, "high": 14.0}`` plants, independently per position with probability p, a
    peak of height U(low, high). Peaks are added to the fp32 draw before bf16 rounding.
    """
    x = _normal(_rng(seed, _T_LOGIT, step), (B, S, V), sigma)
    if peaks:
        rp = _rng(seed, _T_PEAK, step)
        if peaks["mode"] == "half":
            for b in range(B):
                pos = rp.choice(S, size=S // 2, replace=False)
                ids = rp.integers(0, V, size=pos.size)
                x[b, pos, ids] += np.float32(peaks.get("height", 12.0))
        elif peaks["mode"] == "bernoulli":
            hit = rp.random((B, S)) < float(peaks.get("p", 0.6))
            ids = rp.integers(0, V, size=(B, S))
            h = rp.uniform(float(peaks.get("low", 8.0)), float(peaks.get("high", 14.0)), size=(B, S))
            bb, ss = np.nonzero(hit)
            x[bb, ss, ids[bb, ss]] += h[bb, ss].astype(np.float32)
        else:
            raise ValueError(peaks["mode"])
    if mask is None:
        mask = np.ones((B, S), dtype=np.uint8)
    return CommitInputs(B, S, V, dtype, _encode(x, dtype), np.ascontiguousarray(mask, dtype=np.uint8),
                        float(np.float32(gamma)))


def random_mask(B: int, S: int, kmin: int, kmax: int, seed: int, step: int = 0) -> np.ndarray:
    """Per sequence, k ~ U{kmin..kmax} positions (a seeded subset) are still masked; both
    bounds are clamped to S (a block shorter than kmin is wholly masked)."""
    r = _rng(seed, _T_MASK, step)
    m = np.zeros((B, S), dtype=np.uint8)
    lo, hi = min(kmin, S), min(kmax, S)
    for b in range(B):
        k = int(r.integers(lo, hi + 1))
        m[b, r.choice(S, size=k, replace=False)] = 1
    return m


# ----------------------------------------------------------------------------------------
# The five workloads. Sizes follow the deployment point on the pages (S=16, gamma 0.8,
# bf16) at a 30B-class GQA shape; ambiguities in their wording are settled here:
#   * N(0, s): s is the standard deviation.
#   * "half of the positions" = exactly floor(S/2) seeded positions.
#   * "60% of positions" = each position independently with probability 0.6.
#   * concentrated attention for the long-context case: see make_attn(hot_keys=...).
# ----------------------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    dtype: str
    B: int
    S: int
    Hq: int
    Hkv: int
    D: int
    Lmax: int
    V: int
    gamma: float
    layers: int = 1
    steps: int = 1

    @property
    def seed(self) -> int:
        return 1000 + self.cid

    def ctx_lens(self) -> np.ndarray:
        if self.cid == 3:
            return _rng(self.seed, _T_LEN).integers(1024, 8192 + 1, size=self.B).astype(np.int32)
        return np.full(self.B, self.Lmax, dtype=np.int32)

    def attn(self, step: int = 0, layer: int = 0, B: Optional[int] = None) -> AttnInputs:
        """Attention inputs; ``B`` < self.B takes the first B sequences (same draws order)."""
        ctx = self.ctx_lens()
        nb = self.B if B is None else B
        hot = {"frac": 0.01, "boost": 8.0, "bias_norm": 2.0} if self.cid == 4 else None
        return make_attn(nb, self.S, self.Hq, self.Hkv, self.D, ctx[:nb], Lmax=self.Lmax,
                         dtype=self.dtype, seed=self.seed, step=step, layer=layer, hot_keys=hot)

    def block_qkv(self, step: int, layer: int):
        """(q, k_blk, v_blk) of one denoising step and layer (block-loop workload)."""
        return make_block_qkv(self.B, self.S, self.Hq, self.Hkv, self.D, self.dtype, self.seed, step,
                              layer)

    def commit(self, step: int = 0, gamma: Optional[float] = None, B: Optional[int] = None,
               mask: Optional[np.ndarray] = None) -> CommitInputs:
        nb = self.B if B is None else B
        g = self.gamma if gamma is None else gamma
        if self.cid == 1:
            return make_commit(nb, self.S, self.V, F32, sigma=2.0, seed=self.seed, step=step, gamma=g,
                               mask=mask)
        if self.cid == 2:
            return make_commit(nb, self.S, self.V, BF16, 3.0, self.seed, step, g, mask,
                               {"mode": "half", "height": 12.0})
        if self.cid == 3:
            m = random_mask(self.B, self.S, 4, 16, self.seed)[:nb] if mask is None else mask
            return make_commit(nb, self.S, self.V, BF16, 3.0, self.seed, step, g, m,
                               {"mode": "bernoulli", "p": 0.6, "low": 8.0, "high": 14.0})
        if self.cid == 4:
            return make_commit(nb, self.S, self.V, BF16, 3.0, self.seed, step, g, mask)
        if self.cid == 5:
            return make_commit(nb, self.S, self.V, BF16, 3.0, self.seed, step, g, mask,
                               {"mode": "bernoulli", "p": 0.6, "low": 8.0, "high": 14.0})
        raise ValueError(self.cid)


WORKLOADS = {
    1: Workload(1, "tiny-f32 B1 ctx128 S16 Hq4 Hkv1 D64", F32, 1, 16, 4, 1, 64, 128, 1024, 0.8),
    2: Workload(2, "single-seq bf16 B1 ctx4096 S16 Hq32 Hkv2 D128", BF16, 1, 16, 32, 2, 128, 4096,
                131072, 0.8),
    3: Workload(3, "batched-serving bf16 B32 ctx U[1024,8192] S16 Hq32 Hkv2 D128", BF16, 32, 16, 32, 2,
                128, 8192, 131072, 0.8),
    4: Workload(4, "long-context bf16 B4 ctx65536 S16 Hq32 Hkv2 D128 hot1%", BF16, 4, 16, 32, 2, 128,
                65536, 131072, 0.9),
    5: Workload(5, "block-loop bf16 B16 ctx8192 S32 Hq32 Hkv2 D128 6 layers T4", BF16, 16, 32, 32, 2,
                128, 8192, 131072, 0.8, layers=6, steps=4),
}
