"""Move seeded host inputs (numpy, bf16 as uint16 bits) onto the GPU as torch tensors."""
from __future__ import annotations

import numpy as np

from . import workloads as W


def to_torch(a: np.ndarray, dtype: str, device):
    import torch
    if dtype == W.BF16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device)


def attn_to_device(x: W.AttnInputs, device):
    import torch
    f = lambda a: to_torch(a, x.dtype, device)  # noqa: E731
    return (f(x.q), f(x.k_blk), f(x.v_blk), f(x.k_ctx), f(x.v_ctx),
            torch.from_numpy(np.ascontiguousarray(x.ctx_len, dtype=np.int32)).to(device))


def commit_to_device(c: W.CommitInputs, device):
    import torch
    return to_torch(c.logits, c.dtype, device), torch.from_numpy(np.ascontiguousarray(c.mask)).to(device)


def lmhead_to_device(x: W.LmHeadInputs, device):
    """(hidden bf16 [B,S,K], weight bf16 [V,K], mask uint8 [B,S]) on the device."""
    import torch
    return (to_torch(x.hidden, W.BF16, device), to_torch(x.weight, W.BF16, device),
            torch.from_numpy(np.ascontiguousarray(x.mask)).to(device))


def mamba_to_device(m: W.MambaInputs, device):
    """(x, dt, dt_bias, A_log, Dskip, Bm, Cm, h0) on the device."""
    import torch
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)  # noqa: E731
    return (to_torch(m.x, m.dtype, device), f(m.dt), f(m.dt_bias), f(m.A_log), f(m.Dskip),
            to_torch(m.Bm, m.dtype, device), to_torch(m.Cm, m.dtype, device), f(m.h0))


def adaln_to_device(a: W.AdalnInputs, device):
    """(x, f, t_mod, table) on the device."""
    import torch
    f32 = lambda t: torch.from_numpy(np.ascontiguousarray(t, dtype=np.float32)).to(device)  # noqa: E731
    return to_torch(a.x, a.dtype, device), to_torch(a.f, a.dtype, device), f32(a.t_mod), f32(a.table)
