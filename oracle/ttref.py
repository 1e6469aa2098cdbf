"""ctypes binding of the fp64 CPU oracle (oracle/ttref.c). TEST INFRASTRUCTURE ONLY.

Arrays are numpy, host memory. bf16 tensors are uint16 bit patterns, fp32 tensors float32.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None
_DT = {"f32": 0, "bf16": 1}


def lib_path() -> str:
    return _build.LIB


def _lib():
    global _LIB
    if _LIB is None:
        path = os.environ.get("TTREF_LIB")  # the mutation tests point this at a planted-mistake build
        if path is None:
            path = _build.LIB
            if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
                _build.build()
        L = ctypes.CDLL(path)
        vp, i32 = ctypes.c_void_p, ctypes.c_int
        L.ttref_block_denoise_attn.argtypes = [i32] * 7 + [vp] * 7
        L.ttref_block_denoise_attn.restype = i32
        L.ttref_commit.argtypes = [i32, i32, i32, i32, vp, vp, ctypes.c_double, vp, vp, vp, vp]
        L.ttref_commit.restype = i32
        L.ttref_decode.argtypes = [vp, ctypes.c_size_t, i32]
        L.ttref_decode.restype = ctypes.c_double
        L.ttref_lmhead_commit.argtypes = [i32] * 4 + [vp] * 3 + [ctypes.c_double] + [vp] * 4
        L.ttref_lmhead_commit.restype = i32
        L.ttref_ctx_append.argtypes = [i32] * 6 + [vp] * 5 + [i32, vp]
        L.ttref_ctx_append.restype = i32
        L.ttref_mamba2_scan.argtypes = [i32] * 7 + [vp] * 10
        L.ttref_mamba2_scan.restype = i32
        L.ttref_adaln_modulate.argtypes = [i32] * 4 + [vp] * 3 + [ctypes.c_double, vp]
        L.ttref_adaln_modulate.restype = i32
        L.ttref_adaln_gate.argtypes = [i32] * 4 + [vp] * 5
        L.ttref_adaln_gate.restype = i32
        L.ttref_threads.argtypes = []
        L.ttref_threads.restype = i32
        _LIB = L
    return _LIB


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check_dtype(a: np.ndarray, dtype: str):
    want = np.uint16 if dtype == "bf16" else np.float32
    if a.dtype != want or not a.flags.c_contiguous:
        raise TypeError(f"expected contiguous {want} array for dtype {dtype}, got {a.dtype}")


def ttref_threads() -> int:
    """Host threads used by the oracle's parallel loops."""
    return int(_lib().ttref_threads())


def ttref_decode(a: np.ndarray, dtype: str) -> np.ndarray:
    """Widen every element with the oracle's own decode (for pinning it)."""
    _check_dtype(a, dtype)
    L = _lib()
    flat = a.reshape(-1)
    return np.array([L.ttref_decode(_ptr(flat), i, _DT[dtype]) for i in range(flat.size)])


def ttref_block_denoise_attn(B, S, Hq, Hkv, D, Lmax, dtype, q, k_blk, v_blk, k_ctx, v_ctx, ctx_len):
    """Returns out[B,S,Hq,D] float64."""
    for t in (q, k_blk, v_blk, k_ctx, v_ctx):
        _check_dtype(t, dtype)
    assert q.size == B * S * Hq * D and k_blk.size == B * S * Hkv * D and v_blk.size == k_blk.size
    assert k_ctx.size == B * Lmax * Hkv * D and v_ctx.size == k_ctx.size
    ctx = np.ascontiguousarray(ctx_len, dtype=np.int32)
    assert ctx.size == B
    out = np.zeros((B, S, Hq, D), dtype=np.float64)
    rc = _lib().ttref_block_denoise_attn(B, S, Hq, Hkv, D, Lmax, _DT[dtype], _ptr(q), _ptr(k_blk),
                                         _ptr(v_blk), _ptr(k_ctx), _ptr(v_ctx), _ptr(ctx), _ptr(out))
    if rc != 0:
        raise ValueError(f"ttref_block_denoise_attn failed with status {rc}")
    return out


def ttref_commit(B, S, V, dtype, logits, mask, gamma):
    """Returns (token_id int32[B,S], committed uint8[B,S], conf f64[B,S], Z f64[B,S])."""
    _check_dtype(logits, dtype)
    assert logits.size == B * S * V
    m = np.ascontiguousarray(mask, dtype=np.uint8)
    assert m.size == B * S
    tok = np.zeros((B, S), dtype=np.int32)
    com = np.zeros((B, S), dtype=np.uint8)
    conf = np.zeros((B, S), dtype=np.float64)
    z = np.zeros((B, S), dtype=np.float64)
    rc = _lib().ttref_commit(B, S, V, _DT[dtype], _ptr(logits), _ptr(m), float(gamma), _ptr(tok),
                             _ptr(com), _ptr(conf), _ptr(z))
    if rc != 0:
        raise ValueError(f"ttref_commit failed with status {rc}")
    return tok, com, conf, z


def ttref_lmhead_commit(B, S, K, V, hidden, weight, mask, gamma):
    """LM head then commit: hidden uint16 (bf16 bits) [B,S,K], weight uint16 [V,K].
    Returns (token_id int32[B,S], committed uint8[B,S], conf f64[B,S], Z f64[B,S])."""
    _check_dtype(hidden, "bf16")
    _check_dtype(weight, "bf16")
    assert hidden.size == B * S * K and weight.size == V * K
    m = np.ascontiguousarray(mask, dtype=np.uint8)
    assert m.size == B * S
    tok = np.zeros((B, S), dtype=np.int32)
    com = np.zeros((B, S), dtype=np.uint8)
    conf = np.zeros((B, S), dtype=np.float64)
    z = np.zeros((B, S), dtype=np.float64)
    rc = _lib().ttref_lmhead_commit(B, S, K, V, _ptr(hidden), _ptr(weight), _ptr(m), float(gamma),
                                    _ptr(tok), _ptr(com), _ptr(conf), _ptr(z))
    if rc != 0:
        raise ValueError(f"ttref_lmhead_commit failed with status {rc}")
    return tok, com, conf, z


def ttref_ctx_append(B, S, Hkv, D, Lmax, dtype, k_new, v_new, k_ctx, v_ctx, ctx_len, bump):
    """Returns (k_ctx', v_ctx', ctx_len', skipped): updated copies of the cache and lengths,
    and uint8[B] flags of the sequences whose block did not fit. The inputs are not modified."""
    for t in (k_new, v_new, k_ctx, v_ctx):
        _check_dtype(t, dtype)
    assert k_new.size == B * S * Hkv * D and v_new.size == k_new.size
    assert k_ctx.size == B * Lmax * Hkv * D and v_ctx.size == k_ctx.size
    kc, vc = np.array(k_ctx, copy=True), np.array(v_ctx, copy=True)
    ctx = np.array(ctx_len, dtype=np.int32, copy=True)
    assert ctx.size == B
    skipped = np.zeros(B, dtype=np.uint8)
    rc = _lib().ttref_ctx_append(B, S, Hkv, D, Lmax, _DT[dtype], _ptr(k_new), _ptr(v_new), _ptr(kc),
                                 _ptr(vc), _ptr(ctx), int(bool(bump)), _ptr(skipped))
    if rc != 0:
        raise ValueError(f"ttref_ctx_append failed with status {rc}")
    return kc, vc, ctx, skipped


def _f32(a, n):
    a = np.ascontiguousarray(a, dtype=np.float32)
    assert a.size == n
    return a


def ttref_mamba2_scan(B, S, H, P, N, G, dtype, x, dt, dt_bias, A_log, Dskip, Bm, Cm, h0, want_state=True):
    """Mamba-2 scan of one block from the seeded state h0. x [B,S,H,P] and Bm, Cm [B,S,G,N] in
    dtype (bf16 bits or fp32); dt [B,S,H], dt_bias, A_log, Dskip [H] and h0 [B,H,P,N] fp32.
    Returns (y f64 [B,S,H,P], h_out f64 [B,H,P,N] or None)."""
    for t in (x, Bm, Cm):
        _check_dtype(t, dtype)
    assert x.size == B * S * H * P and Bm.size == B * S * G * N and Cm.size == Bm.size
    dt, dt_bias, A_log, Dskip = _f32(dt, B * S * H), _f32(dt_bias, H), _f32(A_log, H), _f32(Dskip, H)
    h0 = _f32(h0, B * H * P * N)
    y = np.zeros((B, S, H, P), dtype=np.float64)
    hs = np.zeros((B, H, P, N), dtype=np.float64) if want_state else None
    rc = _lib().ttref_mamba2_scan(B, S, H, P, N, G, _DT[dtype], _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A_log),
                                  _ptr(Dskip), _ptr(Bm), _ptr(Cm), _ptr(h0), _ptr(y),
                                  _ptr(hs) if hs is not None else None)
    if rc != 0:
        raise ValueError(f"ttref_mamba2_scan failed with status {rc}")
    return y, hs


def ttref_adaln_modulate(B, S, d, dtype, x, t_mod, table, eps=1e-6):
    """adaLN modulation before a layer's mixer: LN(x) * (1 + scale) + shift. x [B,S,d] in dtype,
    t_mod [B,3,d] and table [3,d] fp32 (shift, scale, gate). Returns y f64 [B,S,d]."""
    _check_dtype(x, dtype)
    assert x.size == B * S * d
    t_mod, table = _f32(t_mod, B * 3 * d), _f32(table, 3 * d)
    y = np.zeros((B, S, d), dtype=np.float64)
    rc = _lib().ttref_adaln_modulate(B, S, d, _DT[dtype], _ptr(x), _ptr(t_mod), _ptr(table), float(eps), _ptr(y))
    if rc != 0:
        raise ValueError(f"ttref_adaln_modulate failed with status {rc}")
    return y


def ttref_adaln_gate(B, S, d, dtype, x, f, t_mod, table):
    """Gated residual after a layer's mixer: x + gate * f. Returns out f64 [B,S,d]."""
    _check_dtype(x, dtype)
    _check_dtype(f, dtype)
    assert x.size == B * S * d and f.size == x.size
    t_mod, table = _f32(t_mod, B * 3 * d), _f32(table, 3 * d)
    out = np.zeros((B, S, d), dtype=np.float64)
    rc = _lib().ttref_adaln_gate(B, S, d, _DT[dtype], _ptr(x), _ptr(f), _ptr(t_mod), _ptr(table), _ptr(out))
    if rc != 0:
        raise ValueError(f"ttref_adaln_gate failed with status {rc}")
    return out
