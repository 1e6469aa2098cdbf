"""ctypes binding of libtt (include/tt.h). Argument marshalling only.

Every step of the computation runs in the HIP kernels of libtt.so; this module checks
tensor dtypes, shapes, devices and contiguity, allocates outputs and workspaces with
torch (device memory plumbing), and passes raw device pointers plus the current HIP
stream to the C-ABI. There is no fallback: if libtt.so is missing or a call fails, an
exception is raised.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Tuple

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtt.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "tt.h")

TT_F32, TT_BF16 = 0, 1
STATUS = {0: "TT_OK", 1: "TT_ERR_INVALID_ARG", 2: "TT_ERR_UNSUPPORTED", 3: "TT_ERR_WORKSPACE",
          4: "TT_ERR_HIP"}


class TTError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}")
        self.status = status


class AttnShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("S", ctypes.c_int32), ("Hq", ctypes.c_int32),
                ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32), ("Lmax", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class MambaShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("S", ctypes.c_int32), ("H", ctypes.c_int32), ("P", ctypes.c_int32),
                ("N", ctypes.c_int32), ("G", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class ProfileStats(ctypes.Structure):
    _fields_ = [("attn_calls", ctypes.c_int64), ("attn_total_ms", ctypes.c_double),
                ("attn_main_ms", ctypes.c_double), ("commit_calls", ctypes.c_int64),
                ("commit_total_ms", ctypes.c_double), ("commit_reduce_ms", ctypes.c_double),
                ("lm_calls", ctypes.c_int64), ("lm_total_ms", ctypes.c_double),
                ("lm_reduce_ms", ctypes.c_double)]


_LIB = None


def lib() -> ctypes.CDLL:
    """Load libtt.so (built by block_diffusion_lm_tt_amd/build.py). Raises if it is missing."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libtt.so not found at {LIB_PATH}; build it first "
                              "(python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(LIB_PATH)
        L.tt_build_id.restype = ctypes.c_char_p
        L.tt_build_id.argtypes = []
        built = L.tt_build_id().decode()
        from .build import source_hash
        want = source_hash()
        if built != want:  # a stale library is never run
            raise ImportError(f"libtt.so at {LIB_PATH} was built from other sources (build id "
                              f"{built}, sources {want}); rebuild it "
                              "(python -c 'import __graft_entry__ as g; g.build()')")
        vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
        L.tt_version.restype = i32
        L.tt_version.argtypes = []
        L.build_id = built
        L.tt_status_str.restype = ctypes.c_char_p
        L.tt_status_str.argtypes = [i32]
        L.tt_ctx_append.restype = i32
        L.tt_ctx_append.argtypes = [ctypes.POINTER(AttnShape), vp, vp, vp, vp, vp, i32, vp, vp]
        L.tt_block_denoise_attn_workspace.restype = sz
        L.tt_block_denoise_attn_workspace.argtypes = [ctypes.POINTER(AttnShape)]
        L.tt_block_denoise_attn.restype = i32
        L.tt_block_denoise_attn.argtypes = [ctypes.POINTER(AttnShape)] + [vp] * 8 + [sz, vp]
        L.tt_commit_workspace.restype = sz
        L.tt_commit_workspace.argtypes = [i32, i32, i32, i32]
        L.tt_commit.restype = i32
        L.tt_commit.argtypes = [i32, i32, i32, i32, vp, vp, ctypes.c_float, vp, vp, vp, vp, sz, vp]
        L.tt_commit_noalloc.restype = i32
        L.tt_commit_noalloc.argtypes = [i32, i32, i32, i32, vp, vp, ctypes.c_float, vp, vp, vp, vp]
        L.tt_lmhead_commit_workspace.restype = sz
        L.tt_lmhead_commit_workspace.argtypes = [i32, i32, i32, i32]
        L.tt_lmhead_commit.restype = i32
        L.tt_lmhead_commit.argtypes = [i32, i32, i32, i32, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp, sz, vp]
        L.tt_mamba2_seeded_scan.restype = i32
        L.tt_mamba2_seeded_scan.argtypes = [ctypes.POINTER(MambaShape)] + [vp] * 10 + [vp]
        L.tt_adaln_modulate.restype = i32
        L.tt_adaln_modulate.argtypes = [i32] * 4 + [vp] * 3 + [ctypes.c_float, vp, vp]
        L.tt_adaln_gate.restype = i32
        L.tt_adaln_gate.argtypes = [i32] * 4 + [vp] * 5 + [vp]
        L.tt_lmhead_commit_exact_workspace.restype = sz
        L.tt_lmhead_commit_exact_workspace.argtypes = [i32] * 4
        L.tt_lmhead_commit_exact.restype = i32
        L.tt_lmhead_commit_exact.argtypes = [i32] * 4 + [vp, vp, vp, ctypes.c_float, vp, vp, vp, vp, vp, sz, vp]
        L.tt_lmhead_weight_bound.restype = i32
        L.tt_lmhead_weight_bound.argtypes = [vp, i32, i32, vp, vp]
        L.tt_profile_enable.restype = i32
        L.tt_profile_enable.argtypes = [i32]
        L.tt_profile_reset.restype = i32
        L.tt_profile_reset.argtypes = []
        L.tt_profile_read.restype = i32
        L.tt_profile_read.argtypes = [ctypes.POINTER(ProfileStats)]
        _LIB = L
    return _LIB


def header_symbols() -> list:
    """Names of the functions include/tt.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tt_[a-z0-9_]+)\s*\(", text)))


def _check(fn: str, status: int):
    if status != 0:
        raise TTError(fn, status)


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return TT_BF16
    if t.dtype == torch.float32:
        return TT_F32
    raise TypeError(f"unsupported dtype {t.dtype}; libtt takes bfloat16 or float32")


def _dev(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (libtt has no CPU path)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream(device, stream) -> int:
    torch = _torch()
    s = torch.cuda.current_stream(device) if stream is None else stream
    return int(s.cuda_stream)


def attn_shape(B, S, Hq, Hkv, D, Lmax, dtype_code) -> AttnShape:
    return AttnShape(B, S, Hq, Hkv, D, Lmax, dtype_code)


def tt_block_denoise_attn_workspace(B, S, Hq, Hkv, D, Lmax, dtype_code) -> int:
    sh = attn_shape(B, S, Hq, Hkv, D, Lmax, dtype_code)
    return int(lib().tt_block_denoise_attn_workspace(ctypes.byref(sh)))


def tt_commit_workspace(B, S, V, dtype_code) -> int:
    return int(lib().tt_commit_workspace(B, S, V, dtype_code))


def tt_block_denoise_attn(q, k_blk, v_blk, k_ctx, v_ctx, ctx_len, out=None, workspace=None,
                          stream=None):
    """o[B,S,Hq,D] = denoiser block attention over [context KV ; block KV] (see include/tt.h)."""
    torch = _torch()
    for name, t in (("q", q), ("k_blk", k_blk), ("v_blk", v_blk), ("k_ctx", k_ctx), ("v_ctx", v_ctx),
                    ("ctx_len", ctx_len)):
        _dev(t, name)
    B, S, Hq, D = q.shape
    Bk, Sk, Hkv, Dk = k_blk.shape
    Lmax = k_ctx.shape[1]
    if (Bk, Sk, Dk) != (B, S, D) or v_blk.shape != k_blk.shape:
        raise ValueError("k_blk/v_blk must be [B,S,Hkv,D] matching q")
    if k_ctx.shape != (B, Lmax, Hkv, D) or v_ctx.shape != k_ctx.shape:
        raise ValueError("k_ctx/v_ctx must be [B,Lmax,Hkv,D]")
    if ctx_len.dtype != torch.int32 or ctx_len.shape != (B,):
        raise ValueError("ctx_len must be int32 [B]")
    dt = _dtype_code(q)
    for t in (k_blk, v_blk, k_ctx, v_ctx):
        if t.dtype != q.dtype:
            raise TypeError("q, k and v tensors must share one dtype")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    _dev(out, "out")
    sh = attn_shape(B, S, Hq, Hkv, D, Lmax, dt)
    need = int(lib().tt_block_denoise_attn_workspace(ctypes.byref(sh)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace")
    st = lib().tt_block_denoise_attn(ctypes.byref(sh), q.data_ptr(), k_blk.data_ptr(), v_blk.data_ptr(),
                                     k_ctx.data_ptr(), v_ctx.data_ptr(), ctx_len.data_ptr(), out.data_ptr(),
                                     workspace.data_ptr(), workspace.numel(), _stream(q.device, stream))
    _check("tt_block_denoise_attn", st)
    return out


def tt_commit(logits, mask, gamma: float, token_id=None, committed=None, conf=None, workspace=None,
              stream=None, want_conf: bool = True) -> Tuple:
    """(token_id int32[B,S], committed uint8[B,S], conf float32[B,S] or None); see include/tt.h."""
    torch = _torch()
    _dev(logits, "logits")
    _dev(mask, "mask")
    B, S, V = logits.shape
    if mask.dtype != torch.uint8 or mask.shape != (B, S):
        raise ValueError("mask must be uint8 [B,S]")
    dt = _dtype_code(logits)
    dev = logits.device
    if token_id is None:
        token_id = torch.empty((B, S), dtype=torch.int32, device=dev)
    if committed is None:
        committed = torch.empty((B, S), dtype=torch.uint8, device=dev)
    if conf is None and want_conf:
        conf = torch.empty((B, S), dtype=torch.float32, device=dev)
    if token_id.dtype != torch.int32 or token_id.shape != (B, S):
        raise ValueError("token_id must be int32 [B,S]")
    if committed.dtype != torch.uint8 or committed.shape != (B, S):
        raise ValueError("committed must be uint8 [B,S]")
    _dev(token_id, "token_id")
    _dev(committed, "committed")
    if conf is not None:
        if conf.dtype != torch.float32 or conf.shape != (B, S):
            raise ValueError("conf must be float32 [B,S]")
        _dev(conf, "conf")
    need = int(lib().tt_commit_workspace(B, S, V, dt))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _dev(workspace, "workspace")
    st = lib().tt_commit(B, S, V, dt, logits.data_ptr(), mask.data_ptr(), float(gamma), token_id.data_ptr(),
                         committed.data_ptr(), conf.data_ptr() if conf is not None else None,
                         workspace.data_ptr(), workspace.numel(), _stream(dev, stream))
    _check("tt_commit", st)
    return token_id, committed, conf


def tt_lmhead_commit_workspace(B, S, K, V) -> int:
    return int(lib().tt_lmhead_commit_workspace(B, S, K, V))


def tt_lmhead_commit(hidden, weight, mask, gamma: float, token_id=None, committed=None, conf=None,
                     want_conf: bool = True, workspace=None, stream=None, w_bound=None):
    """LM head + commit (see include/tt.h): hidden bf16 [B,S,K], weight bf16 [V,K], mask uint8
    [B,S]. With w_bound (a float32 device tensor of one element, from tt_lmhead_weight_bound)
    the exact mode (tt_lmhead_commit_exact) runs. Returns (token_id int32[B,S], committed
    uint8[B,S], conf float32[B,S] or None)."""
    torch = _torch()
    _dev(hidden, "hidden")
    _dev(weight, "weight")
    _dev(mask, "mask")
    if hidden.dtype != torch.bfloat16 or weight.dtype != torch.bfloat16:
        raise TypeError("hidden and weight must be bfloat16")
    if hidden.dim() != 3 or weight.dim() != 2 or weight.shape[1] != hidden.shape[2]:
        raise ValueError("hidden must be [B,S,K] and weight [V,K]")
    B, S, K = hidden.shape
    V = weight.shape[0]
    if mask.dtype != torch.uint8 or mask.shape != (B, S):
        raise ValueError("mask must be uint8 [B,S]")
    dev = hidden.device
    if token_id is None:
        token_id = torch.empty((B, S), dtype=torch.int32, device=dev)
    if committed is None:
        committed = torch.empty((B, S), dtype=torch.uint8, device=dev)
    if conf is None and want_conf:
        conf = torch.empty((B, S), dtype=torch.float32, device=dev)
    if token_id.dtype != torch.int32 or token_id.shape != (B, S):
        raise ValueError("token_id must be int32 [B,S]")
    if committed.dtype != torch.uint8 or committed.shape != (B, S):
        raise ValueError("committed must be uint8 [B,S]")
    _dev(token_id, "token_id")
    _dev(committed, "committed")
    if conf is not None:
        if conf.dtype != torch.float32 or conf.shape != (B, S):
            raise ValueError("conf must be float32 [B,S]")
        _dev(conf, "conf")
    if w_bound is not None:
        _dev(w_bound, "w_bound")
        if w_bound.dtype != torch.float32 or w_bound.numel() != 1:
            raise ValueError("w_bound must be a float32 tensor of one element")
        need = int(lib().tt_lmhead_commit_exact_workspace(B, S, K, V))
    else:
        need = tt_lmhead_commit_workspace(B, S, K, V)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _dev(workspace, "workspace")
    cp = conf.data_ptr() if conf is not None else None
    if w_bound is not None:
        st = lib().tt_lmhead_commit_exact(B, S, K, V, hidden.data_ptr(), weight.data_ptr(), mask.data_ptr(),
                                          float(gamma), w_bound.data_ptr(), token_id.data_ptr(),
                                          committed.data_ptr(), cp, workspace.data_ptr(), workspace.numel(),
                                          _stream(dev, stream))
        _check("tt_lmhead_commit_exact", st)
    else:
        st = lib().tt_lmhead_commit(B, S, K, V, hidden.data_ptr(), weight.data_ptr(), mask.data_ptr(),
                                    float(gamma), token_id.data_ptr(), committed.data_ptr(), cp,
                                    workspace.data_ptr(), workspace.numel(), _stream(dev, stream))
        _check("tt_lmhead_commit", st)
    return token_id, committed, conf


def tt_lmhead_weight_bound(weight, bound=None, stream=None):
    """An upper bound on max_v ||weight[v]||_2 (see include/tt.h), as a float32 device tensor of
    one element: the w_bound of the exact LM head mode."""
    torch = _torch()
    _dev(weight, "weight")
    if weight.dtype != torch.bfloat16 or weight.dim() != 2:
        raise ValueError("weight must be bfloat16 [V,K]")
    if bound is None:
        bound = torch.empty((1,), dtype=torch.float32, device=weight.device)
    _dev(bound, "bound")
    V, K = weight.shape
    st = lib().tt_lmhead_weight_bound(weight.data_ptr(), V, K, bound.data_ptr(), _stream(weight.device, stream))
    _check("tt_lmhead_weight_bound", st)
    return bound


def tt_ctx_append(k_new, v_new, k_ctx, v_ctx, ctx_len, bump: bool = True, skipped=None,
                  want_skipped: bool = False, stream=None):
    """Writes the committed block's new K/V rows [B,S,Hkv,D] into the context cache at ctx_len
    (in place) and, with bump, adds S to ctx_len (see include/tt.h). Returns the uint8[B]
    skipped flags when requested (want_skipped or a skipped tensor given), else None."""
    torch = _torch()
    for name, t in (("k_new", k_new), ("v_new", v_new), ("k_ctx", k_ctx), ("v_ctx", v_ctx),
                    ("ctx_len", ctx_len)):
        _dev(t, name)
    B, S, Hkv, D = k_new.shape
    Lmax = k_ctx.shape[1]
    if v_new.shape != k_new.shape:
        raise ValueError("k_new/v_new must be [B,S,Hkv,D]")
    if k_ctx.shape != (B, Lmax, Hkv, D) or v_ctx.shape != k_ctx.shape:
        raise ValueError("k_ctx/v_ctx must be [B,Lmax,Hkv,D] matching k_new")
    if ctx_len.dtype != torch.int32 or ctx_len.shape != (B,):
        raise ValueError("ctx_len must be int32 [B]")
    dt = _dtype_code(k_new)
    for t in (v_new, k_ctx, v_ctx):
        if t.dtype != k_new.dtype:
            raise TypeError("k_new, v_new, k_ctx and v_ctx must share one dtype")
    if skipped is None and want_skipped:
        skipped = torch.empty((B,), dtype=torch.uint8, device=k_new.device)
    if skipped is not None:
        if skipped.dtype != torch.uint8 or skipped.shape != (B,):
            raise ValueError("skipped must be uint8 [B]")
        _dev(skipped, "skipped")
    sh = attn_shape(B, S, Hkv, Hkv, D, Lmax, dt)
    st = lib().tt_ctx_append(ctypes.byref(sh), k_new.data_ptr(), v_new.data_ptr(), k_ctx.data_ptr(),
                             v_ctx.data_ptr(), ctx_len.data_ptr(), 1 if bump else 0,
                             skipped.data_ptr() if skipped is not None else None,
                             _stream(k_new.device, stream))
    _check("tt_ctx_append", st)
    return skipped


def tt_mamba2_seeded_scan(x, dt, dt_bias, A_log, Dskip, Bm, Cm, h0, G: int, y=None, h_out=None,
                          want_state: bool = False, stream=None):
    """The denoiser's Mamba-2 scan over one block from the seeded state h0 (see include/tt.h).
    x [B,S,H,P] and Bm, Cm [B,S,G,N] bf16 or fp32; dt [B,S,H], dt_bias/A_log/Dskip [H], h0
    [B,H,P,N] fp32. Returns (y [B,S,H,P] in x's dtype, h_out fp32 [B,H,P,N] or None)."""
    torch = _torch()
    for name, t in (("x", x), ("dt", dt), ("dt_bias", dt_bias), ("A_log", A_log), ("Dskip", Dskip),
                    ("Bm", Bm), ("Cm", Cm), ("h0", h0)):
        _dev(t, name)
    B, S, H, P = x.shape
    N = Bm.shape[-1]
    if Bm.shape != (B, S, G, N) or Cm.shape != Bm.shape:
        raise ValueError("Bm/Cm must be [B,S,G,N]")
    if dt.shape != (B, S, H) or h0.shape != (B, H, P, N):
        raise ValueError("dt must be [B,S,H] and h0 [B,H,P,N]")
    for name, t in (("dt_bias", dt_bias), ("A_log", A_log), ("Dskip", Dskip)):
        if t.shape != (H,):
            raise ValueError(f"{name} must be [H]")
    for t in (dt, dt_bias, A_log, Dskip, h0):
        if t.dtype != torch.float32:
            raise TypeError("dt, dt_bias, A_log, Dskip and h0 must be float32")
    dt_code = _dtype_code(x)
    if Bm.dtype != x.dtype or Cm.dtype != x.dtype:
        raise TypeError("x, Bm and Cm must share one dtype")
    if y is None:
        y = torch.empty_like(x)
    _dev(y, "y")
    if h_out is None and want_state:
        h_out = torch.empty_like(h0)
    if h_out is not None:
        _dev(h_out, "h_out")
    sh = MambaShape(B, S, H, P, N, G, dt_code)
    st = lib().tt_mamba2_seeded_scan(ctypes.byref(sh), x.data_ptr(), dt.data_ptr(), dt_bias.data_ptr(),
                                     A_log.data_ptr(), Dskip.data_ptr(), Bm.data_ptr(), Cm.data_ptr(),
                                     h0.data_ptr(), y.data_ptr(), h_out.data_ptr() if h_out is not None else None,
                                     _stream(x.device, stream))
    _check("tt_mamba2_seeded_scan", st)
    return y, h_out


def _adaln_common(x, t_mod, table):
    torch = _torch()
    for name, t in (("x", x), ("t_mod", t_mod), ("table", table)):
        _dev(t, name)
    B, S, d = x.shape
    if t_mod.shape != (B, 3, d) or table.shape != (3, d):
        raise ValueError("t_mod must be [B,3,d] and table [3,d]")
    if t_mod.dtype != torch.float32 or table.dtype != torch.float32:
        raise TypeError("t_mod and table must be float32")
    return B, S, d, _dtype_code(x)


def tt_adaln_modulate(x, t_mod, table, eps: float = 1e-6, y=None, stream=None):
    """y = LN(x) * (1 + scale) + shift with adaLN-single vectors (see include/tt.h)."""
    torch = _torch()
    B, S, d, dt = _adaln_common(x, t_mod, table)
    if y is None:
        y = torch.empty_like(x)
    _dev(y, "y")
    st = lib().tt_adaln_modulate(B, S, d, dt, x.data_ptr(), t_mod.data_ptr(), table.data_ptr(), float(eps),
                                 y.data_ptr(), _stream(x.device, stream))
    _check("tt_adaln_modulate", st)
    return y


def tt_adaln_gate(x, f, t_mod, table, out=None, stream=None):
    """out = x + gate * f with adaLN-single vectors (see include/tt.h)."""
    torch = _torch()
    B, S, d, dt = _adaln_common(x, t_mod, table)
    _dev(f, "f")
    if f.shape != x.shape or f.dtype != x.dtype:
        raise ValueError("f must match x")
    if out is None:
        out = torch.empty_like(x)
    _dev(out, "out")
    st = lib().tt_adaln_gate(B, S, d, dt, x.data_ptr(), f.data_ptr(), t_mod.data_ptr(), table.data_ptr(),
                             out.data_ptr(), _stream(x.device, stream))
    _check("tt_adaln_gate", st)
    return out


def profile_enable(on: bool = True):
    _check("tt_profile_enable", lib().tt_profile_enable(1 if on else 0))


def profile_reset():
    _check("tt_profile_reset", lib().tt_profile_reset())


def profile_read() -> dict:
    s = ProfileStats()
    _check("tt_profile_read", lib().tt_profile_read(ctypes.byref(s)))
    return {k: getattr(s, k) for k, _ in ProfileStats._fields_}
