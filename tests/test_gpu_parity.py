"""GPU parity: the HIP path (through the C-ABI) against the fp64 CPU oracle on identical inputs.

Bars: commit token_id / committed bit-exact; commit conf within 1e-5 relative; attention
max-abs error <= 1e-4 for fp32 and <= 1e-2 for bf16 (outputs widened to fp64).
"""
import math

import numpy as np
import pytest
import torch

from block_diffusion_lm_tt_amd import tensors as TZ
from block_diffusion_lm_tt_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL = {W.F32: 1e-4, W.BF16: 1e-2}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_diffusion_lm_tt_amd as tt
    tt.lib()  # the HIP library must be there: no fallback
    return torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)


def _gpu_attn(x: W.AttnInputs, dev):
    import block_diffusion_lm_tt_amd as tt
    args = TZ.attn_to_device(x, dev)
    out = tt.tt_block_denoise_attn(*args)
    torch.cuda.synchronize()
    return out.double().cpu().numpy()


def _oracle_attn(x: W.AttnInputs):
    from oracle import ttref_block_denoise_attn
    return ttref_block_denoise_attn(x.B, x.S, x.Hq, x.Hkv, x.D, x.Lmax, x.dtype, x.q, x.k_blk, x.v_blk,
                                    x.k_ctx, x.v_ctx, x.ctx_len)


def _slice_b(x: W.AttnInputs, b: int, heads=None) -> W.AttnInputs:
    """Sequence b alone (optionally one KV group's query heads), for sampled oracle checks."""
    q, kb, vb, kc, vc = x.q[b:b + 1], x.k_blk[b:b + 1], x.v_blk[b:b + 1], x.k_ctx[b:b + 1], x.v_ctx[b:b + 1]
    Hq, Hkv = x.Hq, x.Hkv
    if heads is not None:  # (g, G): the G query heads of KV head g
        g, G = heads
        q = q[:, :, g * G:(g + 1) * G]
        kb, vb, kc, vc = (t[:, :, g:g + 1] for t in (kb, vb, kc, vc))
        Hq, Hkv = G, 1
    c = np.ascontiguousarray
    return W.AttnInputs(1, x.S, Hq, Hkv, x.D, x.Lmax, x.dtype, c(q), c(kb), c(vb), c(kc), c(vc),
                        x.ctx_len[b:b + 1].copy())


def _assert_attn(got, want, dtype, what):
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - want).max()
    _say(f"{what}: max-abs err {err:.3e}")
    assert err <= TOL[dtype], f"{what}: max-abs error {err} > {TOL[dtype]}"


# ------------------------------------------------------------------------------------------------
# attention, whole outputs at oracle-friendly sizes (several tiles, ragged tails, split units)
# ------------------------------------------------------------------------------------------------

ATTN_CASES = [
    # name, B, S, Hq, Hkv, D, ctx_lens, Lmax, dtype
    ("mfma-ragged", 3, 16, 32, 2, 128, [0, 77, 300], 320, W.BF16),
    ("mfma-tiny-rows", 2, 5, 6, 2, 128, [64, 129], 200, W.BF16),
    ("mfma-S1", 4, 1, 16, 1, 128, [1, 63, 64, 65], 70, W.BF16),
    # units of fewer rows than a workgroup: the waves past the unit's rows idle
    ("mfma-S4-idle-waves", 2, 4, 32, 2, 128, [300, 45], 320, W.BF16),      # 64 rows: 6 of 8 waves idle
    ("mfma-S8-idle-waves", 2, 8, 32, 2, 128, [500, 0], 512, W.BF16),       # 128 rows
    ("mfma-S24-NQ2-idle", 2, 24, 32, 2, 128, [400, 90], 400, W.BF16),      # 384 rows: second slice half idle
    ("mfma-G32-NQ2", 2, 16, 32, 1, 128, [260, 129], 260, W.BF16),          # one KV head: 512 rows, two slices
    ("mfma-G5-S3", 3, 3, 10, 2, 128, [31, 32, 33], 40, W.BF16),            # odd group size, 15 rows
    ("mfma-ctx-full", 4, 16, 32, 2, 128, [96, 96, 96, 96], 96, W.BF16),    # every context exactly Lmax
    ("mfma-S64-NQ8", 2, 64, 32, 2, 128, [500, 31], 512, W.BF16),
    ("mfma-S32-NQ2", 3, 32, 32, 2, 128, [700, 33, 260], 704, W.BF16),
    ("mfma-S128-NQ8", 1, 128, 32, 2, 128, [900], 900, W.BF16),
    ("mfma-S1024-NQ32", 1, 1024, 8, 1, 128, [200], 200, W.BF16),      # the longest block
    ("generic-f32-S1024", 1, 1024, 2, 1, 64, [100], 100, W.F32),
    ("mfma-ctx0", 2, 16, 32, 2, 128, [0, 0], 0, W.BF16),
    ("mfma-G1", 2, 16, 4, 4, 128, [130, 7], 130, W.BF16),
    ("mfma-long-split", 1, 16, 32, 2, 128, [9000], 9000, W.BF16),
    # segments of many lengths: every remainder of the eight-tile steady-state unrolling
    ("mfma-steady-mix", 8, 16, 32, 2, 128, [230, 262, 295, 330, 361, 390, 425, 470], 480, W.BF16),
    ("generic-f32-cfg1", 1, 16, 4, 1, 64, [128], 128, W.F32),
    ("generic-bf16-D64", 2, 8, 8, 2, 64, [40, 300], 300, W.BF16),
    ("generic-f32-D80", 2, 3, 6, 3, 80, [0, 257], 260, W.F32),
    ("generic-bf16-D256", 2, 4, 4, 2, 256, [33, 150], 150, W.BF16),   # the largest head dim
    ("generic-f32-D1", 1, 2, 2, 1, 1, [5], 8, W.F32),                 # the smallest
    ("generic-f32-fp32-D128", 2, 16, 8, 2, 128, [70, 0], 80, W.F32),  # fp32 at the MFMA width
]


@pytest.mark.parametrize("case", ATTN_CASES, ids=[c[0] for c in ATTN_CASES])
def test_attn_matches_oracle(dev, case):
    name, B, S, Hq, Hkv, D, ctx, Lmax, dtype = case
    _say(f"attn case {name}")
    x = W.make_attn(B, S, Hq, Hkv, D, ctx, Lmax=Lmax, dtype=dtype, seed=100 + len(name))
    _assert_attn(_gpu_attn(x, dev), _oracle_attn(x), dtype, name)


def test_attn_padding_is_never_read(dev):
    # NaN vs finite junk in the padding rows: bit-identical outputs
    x = W.make_attn(3, 16, 32, 2, 128, [5, 200, 64], Lmax=256, dtype=W.BF16, seed=7)
    a = _gpu_attn(x, dev)
    y = W.AttnInputs(**{**x.__dict__})
    y.k_ctx, y.v_ctx = x.k_ctx.copy(), x.v_ctx.copy()
    for b in range(3):
        y.k_ctx[b, x.ctx_len[b]:] = 0x4700
        y.v_ctx[b, x.ctx_len[b]:] = 0xC700
    assert np.array_equal(a, _gpu_attn(y, dev))


def test_attn_block_permutation_equivariance(dev):
    x = W.make_attn(2, 16, 32, 2, 128, [100, 3], Lmax=100, dtype=W.BF16, seed=9)
    perm = np.random.default_rng(3).permutation(16)
    y = W.AttnInputs(**{**x.__dict__})
    y.q, y.k_blk, y.v_blk = (np.ascontiguousarray(t[:, perm]) for t in (x.q, x.k_blk, x.v_blk))
    a, b = _gpu_attn(x, dev), _gpu_attn(y, dev)
    assert np.abs(b - a[:, perm]).max() <= 1e-2


def _offset_copy(t, dev, off=1):
    """t on the device starting `off` elements past a 16-byte boundary (contiguous)."""
    buf = torch.empty(t.numel() + off, dtype=t.dtype, device=dev)
    v = buf[off:off + t.numel()].view(t.shape)
    v.copy_(t)
    return v


def test_attn_misaligned_inputs_take_the_elementwise_path(dev):
    # bases off a 16-byte boundary cannot take the MFMA path's 16-byte copies: the library
    # sends them to the element-wise kernel, with the same results
    import block_diffusion_lm_tt_amd as tt
    x = W.make_attn(2, 16, 32, 2, 128, [77, 300], Lmax=300, dtype=W.BF16, seed=21)
    _say("attn misaligned bf16 D=128")
    q, kb, vb, kc, vc, cl = TZ.attn_to_device(x, dev)
    q2, kc2 = _offset_copy(q, dev), _offset_copy(kc, dev)
    out = _offset_copy(torch.zeros_like(q), dev)
    assert q2.data_ptr() % 16 and kc2.data_ptr() % 16 and out.data_ptr() % 16
    tt.tt_block_denoise_attn(q2, kb, vb, kc2, vc, cl, out=out)
    torch.cuda.synchronize()
    _assert_attn(out.double().cpu().numpy(), _oracle_attn(x), W.BF16, "misaligned")


def test_attn_deterministic_replay(dev):
    x = W.WORKLOADS[3].attn(B=8)
    assert np.array_equal(_gpu_attn(x, dev), _gpu_attn(x, dev))


# ------------------------------------------------------------------------------------------------
# attention at the workloads' full sizes, every unit against the oracle (the block-loop
# workload's calls are checked inside its loop: test_gpu_blockloop.py)
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("cid", [1, 2, 3, 4])
def test_attn_workload_full(dev, cid):
    w = W.WORKLOADS[cid]
    _say(f"attn workload {cid}: {w.name}")
    x = w.attn()
    _assert_attn(_gpu_attn(x, dev), _oracle_attn(x), x.dtype, f"workload {cid}, every unit")


@pytest.mark.parametrize("dtype,D", [(W.BF16, 128), (W.F32, 64)])
def test_attn_ctx_len_outside_the_storage_is_clamped(dev, dtype, D):
    # ctx_len lives on the device, so the kernels clamp it to [0, Lmax]: -5 reads no context
    # row and Lmax + 100 reads all Lmax of them, exactly like 0 and Lmax
    import block_diffusion_lm_tt_amd as tt
    Lmax = 96
    x = W.make_attn(3, 16, 8, 2, D, [0, Lmax, 37], Lmax=Lmax, dtype=dtype, seed=12)
    _say(f"attn ctx_len clamp {dtype} D={D}")
    q, kb, vb, kc, vc, _ = TZ.attn_to_device(x, dev)
    wild = torch.tensor([-5, Lmax + 100, 37], dtype=torch.int32, device=dev)
    got = tt.tt_block_denoise_attn(q, kb, vb, kc, vc, wild)
    torch.cuda.synchronize()
    _assert_attn(got.double().cpu().numpy(), _oracle_attn(x), dtype, "clamped ctx_len")


# ------------------------------------------------------------------------------------------------
# commit
# ------------------------------------------------------------------------------------------------

def _gpu_commit(c: W.CommitInputs, dev, gamma=None):
    import block_diffusion_lm_tt_amd as tt
    lg, mk = TZ.commit_to_device(c, dev)
    tok, com, conf = tt.tt_commit(lg, mk, c.gamma if gamma is None else gamma)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), com.cpu().numpy(), conf.cpu().numpy()


def _oracle_commit(c: W.CommitInputs, gamma=None):
    from oracle import ttref_commit
    return ttref_commit(c.B, c.S, c.V, c.dtype, c.logits, c.mask, c.gamma if gamma is None else gamma)


def _assert_commit(c, dev, gamma=None, what=""):
    # the threshold as the C-ABI receives it (a C float) goes to both sides: one rule
    g = float(np.float32(c.gamma if gamma is None else gamma))
    tok, com, conf = _gpu_commit(c, dev, g)
    otok, ocom, oconf, oz = _oracle_commit(c, g)
    assert np.array_equal(tok, otok), f"{what}: token_id differs at {np.argwhere(tok != otok)[:5]}"
    assert np.array_equal(com, ocom), f"{what}: committed differs at {np.argwhere(com != ocom)[:5]}"
    m = c.mask.astype(bool)
    np.testing.assert_allclose(conf[m], oconf[m], rtol=1e-5, atol=0)
    assert np.all(conf[~m] == 0)
    _say(f"{what}: gamma={g} committed {int(com.sum())} of {int(m.sum())} masked")
    return com


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_commit_workload(dev, cid):
    w = W.WORKLOADS[cid]
    c = w.commit(step=0)
    gammas = [0.5, 0.8, 0.95] if cid == 5 else [c.gamma]
    for g in gammas:
        _assert_commit(c, dev, g, f"workload {cid}")


@pytest.mark.parametrize("gamma", [0.0, -1.0, 1.0, 1.5, float("inf"), float("-inf"), 0.3])
def test_commit_gamma_edges(dev, gamma):
    c = W.make_commit(6, 16, 5000, W.BF16, seed=31, mask=W.random_mask(6, 16, 0, 16, seed=31),
                      peaks={"mode": "bernoulli", "p": 0.5, "low": 2.0, "high": 12.0})
    _assert_commit(c, dev, gamma, "edges")


def test_commit_ties_and_duplicates(dev):
    V = 4096
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 8, V)).astype(np.float32) * 3
    x[0, 0] = 1.25                    # all-equal row: token 0, conf 1/V
    x[0, 1] = x[0, 2] = x[0, 3]       # duplicated rows: exact fallback tie -> lowest position
    x[1, :, 7] = 40.0                 # max tie at 7 and 4000 -> token 7
    x[1, :, 4000] = 40.0
    x[2, :] = x[2, 0]                 # whole sequence identical rows
    x[3, 5, 123] = 100.0              # one huge peak
    bits = W.f32_to_bf16_bits(x)
    mask = np.ones((4, 8), np.uint8)
    mask[0, 0] = 0
    for gamma in (0.8, 2.0, 0.0):
        _assert_commit(W.CommitInputs(4, 8, V, W.BF16, bits, mask, gamma), dev, gamma, f"ties g={gamma}")
    xf = np.ascontiguousarray(x)
    _assert_commit(W.CommitInputs(4, 8, V, W.F32, xf, mask, 2.0), dev, 2.0, "ties f32")


def test_commit_gamma_on_the_threshold(dev):
    # gamma placed one float ulp below / at / above an exact confidence forces the fp64 recheck
    c = W.make_commit(4, 16, 131072, W.BF16, seed=44, peaks={"mode": "bernoulli", "p": 0.8,
                                                             "low": 13.0, "high": 18.0})
    _, _, oconf, _ = _oracle_commit(c, 0.5)
    target = float(np.sort(oconf.ravel())[-3])
    for g in (np.nextafter(np.float32(target), np.float32(0)), np.float32(target),
              np.nextafter(np.float32(target), np.float32(1))):
        _assert_commit(c, dev, float(g), "threshold")


@pytest.mark.parametrize("B,S,V,dtype", [
    (3, 1, 1, W.BF16), (2, 7, 1001, W.BF16), (2, 7, 1001, W.F32), (1, 1000, 333, W.BF16),
    (5, 16, 8193, W.BF16), (2, 16, 16383, W.F32), (0, 16, 100, W.BF16),
])
def test_commit_shapes(dev, B, S, V, dtype):
    c = W.make_commit(B, S, V, dtype, seed=B * 1000 + S + V, mask=W.random_mask(B, S, 0, S, seed=V),
                      peaks={"mode": "bernoulli", "p": 0.4, "low": 3.0, "high": 9.0})
    if B == 0:
        import block_diffusion_lm_tt_amd as tt
        lg, mk = TZ.commit_to_device(c, dev)
        tok, com, conf = tt.tt_commit(lg, mk, 0.5)
        torch.cuda.synchronize()
        assert tok.numel() == 0
        return
    for g in (0.05, 0.5, 1.2):
        _assert_commit(c, dev, g, f"shape {B}x{S}x{V}")


def test_commit_unmasked_rows_never_read(dev):
    c = W.make_commit(2, 8, 2048, W.BF16, seed=3, mask=np.array([[1, 0] * 4, [0, 0, 0, 1, 0, 0, 0, 0]], np.uint8))
    base = _gpu_commit(c, dev, 0.4)
    junk = c.logits.copy()
    junk[c.mask == 0] = 0x7FC0  # NaN in unmasked rows
    d = W.CommitInputs(c.B, c.S, c.V, c.dtype, junk, c.mask, 0.4)
    got = _gpu_commit(d, dev, 0.4)
    for a, b in zip(base, got):
        assert np.array_equal(a, b)


# ---- context cache update after a commit: bit-exact against the oracle -------------------------

def _from_device(t, dtype):
    if dtype == W.BF16:
        return t.cpu().view(torch.int16).numpy().view(np.uint16)
    return t.cpu().numpy()


def _append_inputs(B, S, Hkv, D, Lmax, dtype, ctx, seed):
    rng = np.random.default_rng(seed)
    if dtype == W.BF16:
        mk = lambda *sh: rng.integers(0, 1 << 16, size=sh, dtype=np.uint16)  # noqa: E731 (any bits, NaN included)
    else:
        mk = lambda *sh: rng.standard_normal(sh).astype(np.float32)  # noqa: E731
    return mk(B, S, Hkv, D), mk(B, S, Hkv, D), mk(B, Lmax, Hkv, D), mk(B, Lmax, Hkv, D), \
        np.array(ctx, dtype=np.int32)


APPEND_CASES = [
    # name, B, S, Hkv, D, Lmax, dtype, ctx_len, bump
    ("bf16-edges", 7, 16, 2, 128, 64, W.BF16, [0, 1, 47, 48, 49, 64, -3], True),
    ("bf16-no-bump", 3, 16, 2, 128, 40, W.BF16, [0, 10, 24], False),
    ("f32-unaligned-rows", 4, 5, 3, 7, 30, W.F32, [0, 25, 26, 13], True),
    ("bf16-unaligned-rows", 3, 3, 1, 5, 12, W.BF16, [9, 10, 2], True),
    ("bf16-S1", 5, 1, 2, 64, 8, W.BF16, [0, 7, 8, 3, 6], True),
    ("bf16-long-blocks", 2, 256, 4, 128, 1024, W.BF16, [700, 768], True),
]


@pytest.mark.parametrize("case", APPEND_CASES, ids=[c[0] for c in APPEND_CASES])
def test_ctx_append_matches_oracle(dev, case):
    import block_diffusion_lm_tt_amd as tt
    from oracle import ttref_ctx_append
    name, B, S, Hkv, D, Lmax, dtype, ctx, bump = case
    _say(f"[ctx_append] {name}: B={B} S={S} Hkv={Hkv} D={D} Lmax={Lmax} {dtype} ctx={ctx} bump={bump}")
    kn, vn, kc, vc, cl = _append_inputs(B, S, Hkv, D, Lmax, dtype, ctx, seed=B * 31 + S)
    ek, ev, ecl, esk = ttref_ctx_append(B, S, Hkv, D, Lmax, dtype, kn, vn, kc, vc, cl, bump)
    tkn, tvn = TZ.to_torch(kn, dtype, dev), TZ.to_torch(vn, dtype, dev)
    tkc, tvc = TZ.to_torch(kc, dtype, dev), TZ.to_torch(vc, dtype, dev)
    tcl = torch.from_numpy(cl).to(dev)
    sk = tt.tt_ctx_append(tkn, tvn, tkc, tvc, tcl, bump=bump, want_skipped=True)
    torch.cuda.synchronize()
    assert np.array_equal(sk.cpu().numpy(), esk)
    assert np.array_equal(tcl.cpu().numpy(), ecl)
    assert _from_device(tkc, dtype).tobytes() == ek.tobytes()
    assert _from_device(tvc, dtype).tobytes() == ev.tobytes()


def test_ctx_append_then_attention_matches_oracle(dev):
    """The block loop's end: after the cache update (bump), attention over the grown context
    agrees with the oracle on the same updated inputs."""
    import block_diffusion_lm_tt_amd as tt
    from oracle import ttref_ctx_append
    x = W.make_attn(3, 16, 32, 2, 128, [100, 0, 300], Lmax=320, dtype=W.BF16, seed=11)
    k2, v2, c2, _ = ttref_ctx_append(x.B, x.S, x.Hkv, x.D, x.Lmax, x.dtype, x.k_blk, x.v_blk, x.k_ctx,
                                     x.v_ctx, x.ctx_len, True)
    q, kb, vb, kc, vc, cl = TZ.attn_to_device(x, dev)
    tt.tt_ctx_append(kb, vb, kc, vc, cl, bump=True)
    out = tt.tt_block_denoise_attn(q, kb, vb, kc, vc, cl)
    torch.cuda.synchronize()
    y = W.AttnInputs(x.B, x.S, x.Hq, x.Hkv, x.D, x.Lmax, x.dtype, x.q, x.k_blk, x.v_blk, k2, v2, c2)
    want = _oracle_attn(y)
    err = float(np.abs(out.double().cpu().numpy() - want).max())
    assert err <= TOL[W.BF16], err
