"""The C-ABI library loads and exports what include/tt.h declares; host-side validation
returns the documented status codes without touching a GPU (CPU only)."""
import ctypes

import pytest

import block_diffusion_lm_tt_amd as tt
from block_diffusion_lm_tt_amd import _lib

INVALID, UNSUPPORTED, WORKSPACE = 1, 2, 3


def test_library_exports_every_declared_symbol():
    L = tt.lib()
    names = tt.header_symbols()
    assert {"tt_block_denoise_attn", "tt_commit", "tt_block_denoise_attn_workspace", "tt_commit_workspace",
            "tt_status_str", "tt_version", "tt_profile_enable", "tt_profile_reset", "tt_profile_read"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"libtt.so does not export {n}"


def test_probe_library_exports_its_probes():
    # the measurement probes the benchmark times its ceilings with (a library of their own)
    from block_diffusion_lm_tt_amd.build import PROBE_LIB
    P = ctypes.CDLL(PROBE_LIB)
    for n in ("ttprobe_stream_read", "ttprobe_stream_read_lds", "ttprobe_mfma_rate", "ttprobe_lds_read",
              "ttprobe_tile_core"):
        assert hasattr(P, n), f"libttprobe.so does not export {n}"
    # argument checks on the host, before any launch
    P.ttprobe_tile_core.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    P.ttprobe_lds_read.argtypes = P.ttprobe_tile_core.argtypes
    assert P.ttprobe_tile_core(7, 1, 1, ctypes.c_void_p(16), None) == -1
    assert P.ttprobe_tile_core(0, 0, 1, ctypes.c_void_p(16), None) == -1
    assert P.ttprobe_lds_read(2, 1, 1, ctypes.c_void_p(16), None) == -1
    assert P.ttprobe_lds_read(0, 1, 1, None, None) == -1


def test_build_id_matches_the_sources_beside_it():
    from block_diffusion_lm_tt_amd.build import source_hash
    L = tt.lib()
    bid = L.tt_build_id().decode()
    assert len(bid) == 16 and bid == source_hash()


def test_stale_library_is_refused(tmp_path, monkeypatch):
    # a library whose build id differs from the sources' hash is never loaded
    from block_diffusion_lm_tt_amd import build as B
    monkeypatch.setattr(B, "source_hash", lambda: "0" * 16)
    monkeypatch.setattr(_lib, "_LIB", None)
    with pytest.raises(ImportError, match="other sources"):
        _lib.lib()
    monkeypatch.setattr(_lib, "_LIB", None)


def test_version_and_status_strings():
    L = tt.lib()
    assert L.tt_version() >> 16 == 1
    for code, name in _lib.STATUS.items():
        assert L.tt_status_str(code).decode() == name
    assert L.tt_status_str(99).decode() == "TT_UNKNOWN_STATUS"


def _shape(**kw):
    d = dict(B=32, S=16, Hq=32, Hkv=2, D=128, Lmax=8192, dtype=_lib.TT_BF16)
    d.update(kw)
    return _lib.attn_shape(**{k: d[k] for k in ("B", "S", "Hq", "Hkv", "D", "Lmax")}, dtype_code=d["dtype"])


def test_attn_workspace_query():
    L = tt.lib()
    ok = L.tt_block_denoise_attn_workspace(ctypes.byref(_shape()))
    assert ok > 0 and ok % 256 == 0
    assert L.tt_block_denoise_attn_workspace(ctypes.byref(_shape(dtype=_lib.TT_F32, D=64))) >= 256
    assert L.tt_block_denoise_attn_workspace(ctypes.byref(_shape(Hq=30, Hkv=4))) == 0  # Hq % Hkv
    assert L.tt_block_denoise_attn_workspace(ctypes.byref(_shape(D=512))) == 0
    assert L.tt_block_denoise_attn_workspace(None) == 0


FAKE = 0x1000  # never dereferenced: every call below fails validation before any launch
FAKE16 = FAKE  # (16-byte aligned, for the alignment checks)


@pytest.mark.parametrize("kw,want", [
    (dict(S=0), INVALID), (dict(B=-1), INVALID), (dict(Hq=6, Hkv=4), INVALID), (dict(D=0), INVALID),
    (dict(Lmax=-1), INVALID), (dict(dtype=7), UNSUPPORTED), (dict(D=300), UNSUPPORTED),
    (dict(S=2048), UNSUPPORTED), (dict(B=20000), UNSUPPORTED),
    (dict(B=4096, Lmax=65536), UNSUPPORTED),  # context storage past 2^31 elements
])
def test_attn_rejects_bad_shapes(kw, want):
    L = tt.lib()
    st = L.tt_block_denoise_attn(ctypes.byref(_shape(**kw)), *([FAKE] * 8), 1 << 30, None)
    assert st == want


def test_attn_rejects_null_pointers_and_short_workspace():
    L = tt.lib()
    sh = _shape()
    need = L.tt_block_denoise_attn_workspace(ctypes.byref(sh))
    for k in range(7):
        ptrs = [FAKE] * 8
        ptrs[k] = None
        if k in (3, 4):  # k_ctx / v_ctx may only be NULL when Lmax == 0
            assert L.tt_block_denoise_attn(ctypes.byref(sh), *ptrs, need, None) == INVALID
        else:
            assert L.tt_block_denoise_attn(ctypes.byref(sh), *ptrs, need, None) == INVALID
    assert L.tt_block_denoise_attn(ctypes.byref(sh), *([FAKE] * 8), need - 1, None) == WORKSPACE
    ptrs = [FAKE] * 7 + [None]
    assert L.tt_block_denoise_attn(ctypes.byref(sh), *ptrs, need, None) == WORKSPACE
    assert L.tt_block_denoise_attn(None, *([FAKE] * 8), need, None) == INVALID


def test_attn_batch_zero_is_a_noop():
    L = tt.lib()
    assert L.tt_block_denoise_attn(ctypes.byref(_shape(B=0)), *([None] * 8), 0, None) == 0


def test_commit_validation():
    L = tt.lib()
    need = L.tt_commit_workspace(32, 16, 131072, _lib.TT_BF16)
    assert need > 0 and need % 256 == 0
    assert L.tt_commit_workspace(1, 0, 10, 1) == 0
    assert L.tt_commit_workspace(1, 2000, 10, 1) == 0
    assert L.tt_commit_workspace(1, 2, 10, 5) == 0
    args = lambda **kw: dict(dict(B=32, S=16, V=131072, dt=1, lg=FAKE, mk=FAKE, g=0.8, tok=FAKE, com=FAKE,  # noqa
                                  conf=None, ws=FAKE, n=need), **kw)
    call = lambda a: L.tt_commit(a["B"], a["S"], a["V"], a["dt"], a["lg"], a["mk"], a["g"], a["tok"],  # noqa
                                 a["com"], a["conf"], a["ws"], a["n"], None)
    assert call(args(g=float("nan"))) == INVALID
    assert call(args(S=0)) == INVALID
    assert call(args(V=0)) == INVALID
    assert call(args(B=-2)) == INVALID
    assert call(args(dt=3)) == UNSUPPORTED
    assert call(args(S=1025)) == UNSUPPORTED
    # one workgroup per (position, 16384-entry chunk): the grid bounds B*S*chunks by 2^24 - 1
    assert L.tt_commit_workspace(8191, 1024, 16384 * 3, 1) == 0
    assert call(args(B=8191, S=1024, V=16384 * 3)) == UNSUPPORTED
    assert L.tt_commit_workspace(1023, 1024, 16384 * 16, 1) > 0   # 16760832 workgroups fit
    assert L.tt_commit_workspace(1024, 1024, 16384 * 16, 1) == 0  # 2^24 do not

    for k in ("lg", "mk", "tok", "com"):
        assert call(args(**{k: None})) == INVALID
    assert call(args(n=need - 1)) == WORKSPACE
    assert call(args(ws=None)) == WORKSPACE
    assert call(args(B=0, lg=None)) == 0


def test_lmhead_commit_validation():
    L = tt.lib()
    need = L.tt_lmhead_commit_workspace(32, 16, 4096, 131072)
    # per position and 256-entry chunk a 16-byte record and a 4-byte runner-up, then 16 bytes per position
    assert need == 32 * 16 * 512 * 16 + 32 * 16 * 512 * 4 + 32 * 16 * 16
    assert L.tt_lmhead_commit_workspace(1, 1, 100, 10) == 0    # K not a multiple of 64
    assert L.tt_lmhead_commit_workspace(1, 0, 64, 10) == 0
    assert L.tt_lmhead_commit_workspace(5, 1000, 64, 10) == 0  # B*S > 4096
    args = lambda **kw: dict(dict(B=32, S=16, K=4096, V=131072, h=FAKE, w=FAKE, mk=FAKE, g=0.8,  # noqa
                                  tok=FAKE, com=FAKE, conf=None, ws=FAKE, n=need), **kw)
    call = lambda a: L.tt_lmhead_commit(a["B"], a["S"], a["K"], a["V"], a["h"], a["w"], a["mk"],  # noqa
                                        a["g"], a["tok"], a["com"], a["conf"], a["ws"], a["n"], None)
    assert call(args(g=float("nan"))) == INVALID
    for kw in (dict(S=0), dict(K=0), dict(V=0), dict(B=-1)):
        assert call(args(**kw)) == INVALID
    for kw in (dict(K=100), dict(S=1025), dict(B=300), dict(K=1 << 21)):
        assert call(args(**kw)) == UNSUPPORTED
    for k in ("h", "w", "mk", "tok", "com"):
        assert call(args(**{k: None})) == INVALID
    # 16-byte loads of the hidden states and the head's rows
    assert call(args(h=FAKE + 2)) == UNSUPPORTED
    assert call(args(w=FAKE + 8)) == UNSUPPORTED
    assert call(args(n=need - 1)) == WORKSPACE
    assert call(args(ws=None)) == WORKSPACE
    assert call(args(B=0, h=None, w=None)) == 0


def test_lmhead_exact_validation():
    L = tt.lib()
    need = L.tt_lmhead_commit_exact_workspace(32, 16, 4096, 131072)
    rows, nvt = 32 * 16, 512
    assert need == rows * nvt * (16 + 4 + 1 + 24) + rows * (16 + 16 + 4 + 4) + 256 + 32 * 4 + 128
    assert L.tt_lmhead_commit_exact_workspace(1, 1, 100, 10) == 0
    args = lambda **kw: dict(dict(B=32, S=16, K=4096, V=131072, h=FAKE, w=FAKE, mk=FAKE, g=0.8, wb=FAKE,  # noqa
                                  tok=FAKE, com=FAKE, conf=None, ws=FAKE, n=need), **kw)
    call = lambda a: L.tt_lmhead_commit_exact(a["B"], a["S"], a["K"], a["V"], a["h"], a["w"], a["mk"],  # noqa
                                              a["g"], a["wb"], a["tok"], a["com"], a["conf"], a["ws"], a["n"],
                                              None)
    assert call(args(g=float("nan"))) == INVALID
    for k in ("h", "w", "mk", "wb", "tok", "com"):
        assert call(args(**{k: None})) == INVALID
    assert call(args(K=100)) == UNSUPPORTED
    assert call(args(h=FAKE + 2)) == UNSUPPORTED
    assert call(args(n=need - 1)) == WORKSPACE
    assert call(args(B=0, h=None, w=None, wb=None)) == 0
    assert L.tt_lmhead_weight_bound(FAKE, -1, 64, FAKE, None) == INVALID
    assert L.tt_lmhead_weight_bound(FAKE, 10, 0, FAKE, None) == INVALID
    assert L.tt_lmhead_weight_bound(FAKE, 10, 64, None, None) == INVALID
    assert L.tt_lmhead_weight_bound(None, 10, 64, FAKE, None) == INVALID
    assert L.tt_lmhead_weight_bound(FAKE, 1 << 30, 1 << 20, FAKE, None) == UNSUPPORTED


@pytest.mark.parametrize("kw,want", [
    (dict(S=0), INVALID), (dict(B=-1), INVALID), (dict(Hkv=0), INVALID), (dict(D=0), INVALID),
    (dict(Lmax=-1), INVALID), (dict(dtype=7), UNSUPPORTED), (dict(D=300), UNSUPPORTED),
    (dict(S=2048), UNSUPPORTED), (dict(B=20000), UNSUPPORTED), (dict(B=4096, Lmax=65536), UNSUPPORTED),
])
def test_ctx_append_rejects_bad_shapes(kw, want):
    L = tt.lib()
    assert L.tt_ctx_append(ctypes.byref(_shape(**kw)), *([FAKE] * 5), 1, FAKE, None) == want


def test_ctx_append_null_pointers_and_empty_batch():
    L = tt.lib()
    sh = _shape()
    for k in range(5):
        ptrs = [FAKE] * 5
        ptrs[k] = None
        assert L.tt_ctx_append(ctypes.byref(sh), *ptrs, 1, None, None) == INVALID
    assert L.tt_ctx_append(None, *([FAKE] * 5), 1, None, None) == INVALID
    assert L.tt_ctx_append(ctypes.byref(_shape(B=0)), *([None] * 5), 1, None, None) == 0


def test_profile_api_without_gpu_work():
    tt.profile_enable(True)
    tt.profile_reset()
    st = tt.profile_read()
    assert st["attn_calls"] == 0 and st["commit_calls"] == 0 and st["lm_calls"] == 0
    tt.profile_enable(False)


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 1, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        tt.tt_block_denoise_attn(q, q, q, q, q, torch.zeros(1, dtype=torch.int32))


def _mshape(**kw):
    d = dict(B=32, S=16, H=128, P=64, N=128, G=8, dtype=_lib.TT_BF16)
    d.update(kw)
    return _lib.MambaShape(d["B"], d["S"], d["H"], d["P"], d["N"], d["G"], d["dtype"])


@pytest.mark.parametrize("kw,want", [
    (dict(B=-1), INVALID), (dict(S=0), INVALID), (dict(H=0), INVALID), (dict(G=3), INVALID),
    (dict(N=0), INVALID), (dict(dtype=7), UNSUPPORTED), (dict(P=4, N=16), UNSUPPORTED),
    (dict(P=48), UNSUPPORTED), (dict(P=256), UNSUPPORTED), (dict(N=256), UNSUPPORTED), (dict(N=100), UNSUPPORTED),
    (dict(S=1025), UNSUPPORTED), (dict(B=65536, H=256, G=8), UNSUPPORTED),
])
def test_mamba_scan_rejects_bad_shapes(kw, want):
    L = tt.lib()
    assert L.tt_mamba2_seeded_scan(ctypes.byref(_mshape(**kw)), *([FAKE16] * 10), None) == want


def test_mamba_scan_null_pointers_alignment_and_empty_batch():
    L = tt.lib()
    sh = _mshape()
    assert L.tt_mamba2_seeded_scan(None, *([FAKE16] * 10), None) == INVALID
    for k in range(9):  # every argument but h_out is required
        ptrs = [FAKE16] * 10
        ptrs[k] = None
        assert L.tt_mamba2_seeded_scan(ctypes.byref(sh), *ptrs, None) == INVALID
    ptrs = [FAKE16] * 10
    ptrs[7] = FAKE16 + 4  # h0 not 16-byte aligned
    assert L.tt_mamba2_seeded_scan(ctypes.byref(sh), *ptrs, None) == UNSUPPORTED
    ptrs = [FAKE16] * 10
    ptrs[9] = FAKE16 + 8  # h_out not 16-byte aligned
    assert L.tt_mamba2_seeded_scan(ctypes.byref(sh), *ptrs, None) == UNSUPPORTED
    assert L.tt_mamba2_seeded_scan(ctypes.byref(_mshape(B=0)), *([None] * 10), None) == 0


def test_adaln_validation():
    L = tt.lib()
    bf = _lib.TT_BF16
    assert L.tt_adaln_modulate(2, 3, 0, bf, FAKE16, FAKE16, FAKE16, 1e-6, FAKE16, None) == INVALID
    assert L.tt_adaln_modulate(-1, 3, 8, bf, FAKE16, FAKE16, FAKE16, 1e-6, FAKE16, None) == INVALID
    assert L.tt_adaln_modulate(2, 0, 8, bf, FAKE16, FAKE16, FAKE16, 1e-6, FAKE16, None) == INVALID
    assert L.tt_adaln_modulate(2, 3, 8, bf, FAKE16, FAKE16, FAKE16, -1.0, FAKE16, None) == INVALID
    assert L.tt_adaln_modulate(2, 3, 8, bf, FAKE16, FAKE16, FAKE16, float("nan"), FAKE16, None) == INVALID
    assert L.tt_adaln_modulate(2, 3, 8, bf, FAKE16, FAKE16, FAKE16, float("inf"), FAKE16, None) == INVALID
    assert L.tt_adaln_modulate(2, 3, 8193, bf, FAKE16, FAKE16, FAKE16, 1e-6, FAKE16, None) == UNSUPPORTED
    assert L.tt_adaln_modulate(2, 3, 8, 9, FAKE16, FAKE16, FAKE16, 1e-6, FAKE16, None) == UNSUPPORTED
    for k in range(4):
        ptrs = [FAKE16] * 4
        ptrs[k] = None
        assert L.tt_adaln_modulate(2, 3, 8, bf, *ptrs[:3], 1e-6, ptrs[3], None) == INVALID
    assert L.tt_adaln_modulate(0, 3, 8, bf, None, None, None, 1e-6, None, None) == 0
    assert L.tt_adaln_gate(2, 3, 8, bf, FAKE16, None, FAKE16, FAKE16, FAKE16, None) == INVALID
    assert L.tt_adaln_gate(2, 3, 8193, bf, *([FAKE16] * 5), None) == UNSUPPORTED
    assert L.tt_adaln_gate(0, 3, 8, bf, *([None] * 5), None) == 0
