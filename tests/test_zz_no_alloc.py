"""tt_commit_noalloc (the commit without a workspace, for callers that cannot allocate)
against tt_commit, through the C-ABI: identical token_id, committed and conf, on two calls
in a row, the second on a smaller input (its static scratch keeps the first call's records)."""
import ctypes

import numpy as np
import pytest
import torch

from block_diffusion_lm_tt_amd import tensors as TZ
from block_diffusion_lm_tt_amd import workloads as W

pytestmark = pytest.mark.gpu


def _noalloc(lg, mk, gamma, dt):
    from block_diffusion_lm_tt_amd import _lib
    B, S, V = lg.shape
    tok = torch.empty((B, S), dtype=torch.int32, device=lg.device)
    com = torch.empty((B, S), dtype=torch.uint8, device=lg.device)
    conf = torch.empty((B, S), dtype=torch.float32, device=lg.device)
    st = _lib.lib().tt_commit_noalloc(B, S, V, dt, lg.data_ptr(), mk.data_ptr(), ctypes.c_float(gamma),
                                      tok.data_ptr(), com.data_ptr(), conf.data_ptr(),
                                      torch.cuda.current_stream(lg.device).cuda_stream)
    assert st == 0, _lib.STATUS.get(st, st)
    return tok, com, conf


def test_noalloc_commit_equals_the_workspace_commit():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_diffusion_lm_tt_amd as tt
    dev = torch.device("cuda:0")
    w3 = W.WORKLOADS[3]
    big = w3.commit()                                          # B=32, S=16, V=131072 bf16
    small = W.make_commit(3, 7, 1001, W.BF16, seed=9, mask=W.random_mask(3, 7, 1, 7, seed=9),
                          peaks={"mode": "bernoulli", "p": 0.5, "low": 4.0, "high": 10.0})
    for c in (big, small):
        print(f"noalloc commit B={c.B} S={c.S} V={c.V}", flush=True)
        g = float(np.float32(c.gamma if c is big else 0.3))
        lg, mk = TZ.commit_to_device(c, dev)
        t1, c1, f1 = _noalloc(lg, mk, g, 1)
        t2, c2, f2 = tt.tt_commit(lg, mk, g)
        torch.cuda.synchronize()
        assert torch.equal(t1, t2) and torch.equal(c1, c2)
        assert torch.equal(f1.view(torch.int32), f2.view(torch.int32))  # same kernels: same bits
        print(f"  identical; {int(c1.sum())} committed", flush=True)


def test_noalloc_commit_refuses_shapes_past_its_scratch():
    from block_diffusion_lm_tt_amd import _lib
    L = _lib.lib()
    # 65536 rows x 8 chunks x 16 bytes = 8 MiB of records > 4 MiB: refused before any launch
    st = L.tt_commit_noalloc(4096, 16, 131072, 1, 0x1000, 0x1000, ctypes.c_float(0.5), 0x1000, 0x1000,
                             None, None)
    assert st == 2
