"""Pins for the oracle's Mamba-2 scan from a seeded state and its adaLN-single modulation.

Sources: snilld.dk TwoTower article, "Hvad TwoTower aendrer teknisk" (the denoiser's Mamba-2
states are seeded from the context tower; every layer is time-modulated by a small
adaLN-single block); gist.science explainer (English), Technical Summary > Methodology >
Architecture (the context tower produces KV caches and Mamba states), Training and
Conditioning > Time Conditioning (adaptive layer normalization on the diffusion timestep),
ablations (Mamba stays causal). The pages name the layer types; the Mamba-2 recurrence and
the adaLN form are their published definitions.

The scan is pinned to its unrolled matrix form (each output as the seeded state's decayed
readout plus a causal, decay-weighted sum over earlier inputs: a different evaluation from
the oracle's step-by-step state update), to the composition of two scans, to its limits
(no step: the state stays the seed; no memory: only the current input), to causality, to
affinity in the seed and to the head-to-group map. The modulation is pinned to a library
layer normalization, to closed forms and to the affine invariance of normalization; the
gated residual to exactly representable arithmetic.
"""
import numpy as np
import pytest
import torch

from block_diffusion_lm_tt_amd import workloads as W
from oracle import ttref_adaln_gate, ttref_adaln_modulate, ttref_mamba2_scan


def _scan_inputs(B, S, H, P, N, G, seed, dtype=W.F32):
    r = np.random.default_rng(seed)
    x = r.standard_normal((B, S, H, P)).astype(np.float32)
    Bm = (r.standard_normal((B, S, G, N)) / np.sqrt(N)).astype(np.float32)
    Cm = (r.standard_normal((B, S, G, N)) / np.sqrt(N)).astype(np.float32)
    if dtype == W.BF16:  # values that bf16 holds exactly, so both dtypes describe one input
        x, Bm, Cm = (W.bf16_bits_to_f32(W.f32_to_bf16_bits(t)) for t in (x, Bm, Cm))
    dt = (r.standard_normal((B, S, H)) - 1.0).astype(np.float32)
    dt_bias = (r.standard_normal(H) * 0.5).astype(np.float32)
    A_log = np.log(r.uniform(1.0, 8.0, H)).astype(np.float32)
    Dsk = r.uniform(0.5, 1.5, H).astype(np.float32)
    h0 = r.standard_normal((B, H, P, N)).astype(np.float32)
    return dict(x=x, dt=dt, dt_bias=dt_bias, A_log=A_log, Dskip=Dsk, Bm=Bm, Cm=Cm, h0=h0)


def _run(B, S, H, P, N, G, inp, dtype=W.F32):
    x, Bm, Cm = inp["x"], inp["Bm"], inp["Cm"]
    if dtype == W.BF16:
        x, Bm, Cm = (W.f32_to_bf16_bits(t) for t in (x, Bm, Cm))
    return ttref_mamba2_scan(B, S, H, P, N, G, dtype, x, inp["dt"], inp["dt_bias"], inp["A_log"], inp["Dskip"],
                             Bm, Cm, inp["h0"])


def _matrix_form(B, S, H, P, N, G, inp):
    """y_t = e^{L_t} (h0 C_t) + sum_{s<=t} e^{L_t - L_s} delta_s (C_t . B_s) x_s + D x_t, with
    L_t = sum_{r<=t} delta_r A (the recurrence unrolled); final state likewise."""
    x = inp["x"].astype(np.float64)
    Bm, Cm = inp["Bm"].astype(np.float64), inp["Cm"].astype(np.float64)
    h0 = inp["h0"].astype(np.float64)
    z = inp["dt"].astype(np.float64) + inp["dt_bias"].astype(np.float64)[None, None, :]
    delta = np.logaddexp(0.0, z)                                  # softplus (library form)
    A = -np.exp(inp["A_log"].astype(np.float64))
    y = np.zeros((B, S, H, P))
    hs = np.zeros((B, H, P, N))
    for b in range(B):
        for h in range(H):
            g = h // (H // G)
            L = np.cumsum(delta[b, :, h] * A[h])                   # [S]
            C, Bg = Cm[b, :, g], Bm[b, :, g]                       # [S, N]
            dec = np.exp(L[:, None] - L[None, :]) * np.tril(np.ones((S, S)))
            M = dec * (C @ Bg.T) * delta[b, None, :, h]            # [t, s]
            y[b, :, h] = np.exp(L)[:, None] * (C @ h0[b, h].T) + M @ x[b, :, h] \
                + float(inp["Dskip"][h]) * x[b, :, h]
            w = np.exp(L[-1] - L) * delta[b, :, h]                 # [S]
            hs[b, h] = np.exp(L[-1]) * h0[b, h] + (x[b, :, h] * w[:, None]).T @ Bg
    return y, hs


@pytest.mark.parametrize("shape", [(2, 5, 4, 3, 6, 2), (1, 1, 2, 4, 5, 1), (2, 16, 8, 8, 16, 4)])
def test_scan_matches_its_matrix_form(shape):
    B, S, H, P, N, G = shape
    inp = _scan_inputs(B, S, H, P, N, G, seed=sum(shape))
    y, hs = _run(B, S, H, P, N, G, inp)
    ym, hm = _matrix_form(B, S, H, P, N, G, inp)
    np.testing.assert_allclose(y, ym, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(hs, hm, rtol=1e-10, atol=1e-10)


def test_scan_composes_over_a_split_block():
    B, S, H, P, N, G = 2, 9, 4, 3, 5, 2
    inp = _scan_inputs(B, S, H, P, N, G, seed=3)
    y, hs = _run(B, S, H, P, N, G, inp)
    k = 4
    first = {n: (v[:, :k] if n in ("x", "dt", "Bm", "Cm") else v) for n, v in inp.items()}
    y1, h1 = _run(B, k, H, P, N, G, {n: np.ascontiguousarray(v) for n, v in first.items()})
    second = {n: (v[:, k:] if n in ("x", "dt", "Bm", "Cm") else v) for n, v in inp.items()}
    second["h0"] = h1.astype(np.float32)
    # the carried state is rounded to fp32 (the oracle's state input type): compare loosely
    y2, h2 = _run(B, S - k, H, P, N, G, {n: np.ascontiguousarray(v) for n, v in second.items()})
    np.testing.assert_allclose(y[:, :k], y1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(y[:, k:], y2, rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(hs, h2, rtol=1e-5, atol=1e-5)


def test_scan_without_steps_reads_out_the_seed():
    # dt -> -inf: delta = softplus(-inf) = 0, the state stays the seed: y_t = h0 C_t + D x_t
    B, S, H, P, N, G = 2, 4, 4, 3, 5, 2
    inp = _scan_inputs(B, S, H, P, N, G, seed=4)
    inp["dt"][:] = -1e4
    y, hs = _run(B, S, H, P, N, G, inp)
    g = np.arange(H) // (H // G)
    want = np.einsum("bhpn,bshn->bshp", inp["h0"].astype(np.float64), inp["Cm"][:, :, g].astype(np.float64)) \
        + inp["Dskip"].astype(np.float64)[None, None, :, None] * inp["x"].astype(np.float64)
    np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(hs, inp["h0"], rtol=0, atol=0)


def test_scan_without_memory_sees_only_the_current_input():
    # A -> -inf: a_t = 0 once delta > 0, so state_t = delta_t x_t B_t^T and
    # y_t = delta_t x_t (B_t . C_t) + D x_t, whatever the seed
    B, S, H, P, N, G = 2, 3, 2, 4, 3, 1
    inp = _scan_inputs(B, S, H, P, N, G, seed=5)
    inp["A_log"][:] = 60.0
    y, _ = _run(B, S, H, P, N, G, inp)
    delta = np.logaddexp(0.0, inp["dt"].astype(np.float64) + inp["dt_bias"].astype(np.float64)[None, None, :])
    bc = np.einsum("bsn,bsn->bs", inp["Bm"][:, :, 0].astype(np.float64), inp["Cm"][:, :, 0].astype(np.float64))
    x64 = inp["x"].astype(np.float64)
    want = (delta * bc[:, :, None])[..., None] * x64 + inp["Dskip"].astype(np.float64)[None, None, :, None] * x64
    np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-12)


def test_scan_is_causal_and_affine_in_the_seed():
    B, S, H, P, N, G = 1, 6, 2, 3, 4, 2
    inp = _scan_inputs(B, S, H, P, N, G, seed=6)
    y, _ = _run(B, S, H, P, N, G, inp)
    changed = {n: v.copy() for n, v in inp.items()}
    changed["x"][:, 3] += 5.0
    changed["Bm"][:, 3] -= 1.0
    y2, _ = _run(B, S, H, P, N, G, changed)
    assert np.array_equal(y[:, :3], y2[:, :3]) and not np.allclose(y[:, 3:], y2[:, 3:])
    # y is affine in the seed: y(2 h0) - y(h0) = y(h0) - y(0)
    z = {n: v.copy() for n, v in inp.items()}
    z["h0"][:] = 0
    d = {n: v.copy() for n, v in inp.items()}
    d["h0"] = (2 * inp["h0"]).astype(np.float32)
    y0, _ = _run(B, S, H, P, N, G, z)
    yd, _ = _run(B, S, H, P, N, G, d)
    np.testing.assert_allclose(yd - y, y - y0, rtol=1e-12, atol=1e-12)
    assert not np.allclose(y, y0)  # the seed matters


def test_scan_head_to_group_map():
    # heads h of a group read that group's B, C: with every head's own inputs equal, heads of
    # one group agree and heads of groups with different B, C do not; group of h = h // (H/G)
    B, S, H, P, N, G = 1, 4, 6, 2, 3, 3
    inp = _scan_inputs(B, S, H, P, N, G, seed=7)
    for k in ("x",):
        inp[k][:] = inp[k][:, :, :1]
    inp["dt"][:] = inp["dt"][:, :, :1]
    for k in ("dt_bias", "A_log", "Dskip"):
        inp[k][:] = inp[k][0]
    inp["h0"][:] = inp["h0"][:, :1]
    y, _ = _run(B, S, H, P, N, G, inp)
    for h in range(H):
        for h2 in range(H):
            same = h // 2 == h2 // 2
            assert np.array_equal(y[:, :, h], y[:, :, h2]) == same, (h, h2)


def test_scan_bf16_decode():
    B, S, H, P, N, G = 2, 3, 4, 3, 5, 2
    inp = _scan_inputs(B, S, H, P, N, G, seed=8, dtype=W.BF16)
    y32, h32 = _run(B, S, H, P, N, G, inp, W.F32)
    y16, h16 = _run(B, S, H, P, N, G, inp, W.BF16)
    assert np.array_equal(y32, y16) and np.array_equal(h32, h16)


def test_scan_rejects_bad_group_split():
    inp = _scan_inputs(1, 2, 3, 2, 2, 1, seed=9)
    with pytest.raises(ValueError):
        ttref_mamba2_scan(1, 2, 3, 2, 2, 2, W.F32, inp["x"], inp["dt"], inp["dt_bias"], inp["A_log"], inp["Dskip"],
                          np.zeros((1, 2, 2, 2), np.float32), np.zeros((1, 2, 2, 2), np.float32), inp["h0"])


# ---- adaLN-single ----------------------------------------------------------------------------

def _mod_inputs(B, S, d, seed):
    r = np.random.default_rng(seed)
    x = (r.standard_normal((B, S, d)) * 2 + 0.5).astype(np.float32)
    t_mod = (r.standard_normal((B, 3, d)) * 0.3).astype(np.float32)
    table = (r.standard_normal((3, d)) * 0.1).astype(np.float32)
    return x, t_mod, table


def test_modulate_matches_library_layer_norm():
    B, S, d = 2, 3, 40
    x, t_mod, table = _mod_inputs(B, S, d, 1)
    y = ttref_adaln_modulate(B, S, d, W.F32, x, t_mod, table, eps=1e-6)
    xt = torch.from_numpy(x).double()
    u = torch.nn.functional.layer_norm(xt, (d,), eps=1e-6).numpy()
    shift = (t_mod[:, 0].astype(np.float64) + table[0])[:, None, :]
    scale = (t_mod[:, 1].astype(np.float64) + table[1])[:, None, :]
    np.testing.assert_allclose(y, u * (1 + scale) + shift, rtol=1e-12, atol=1e-12)


def test_modulate_closed_forms():
    B, S, d = 2, 2, 16
    x, t_mod, table = _mod_inputs(B, S, d, 2)
    zero_t, zero_tab = np.zeros_like(t_mod), np.zeros_like(table)
    u = ttref_adaln_modulate(B, S, d, W.F32, x, zero_t, zero_tab, eps=0.0)
    np.testing.assert_allclose(u.mean(-1), 0, atol=1e-12)
    np.testing.assert_allclose((u ** 2).mean(-1), 1, rtol=1e-12)
    # a constant row normalizes to 0: the output is the shift alone
    xc = np.full((B, S, d), 3.25, np.float32)
    y = ttref_adaln_modulate(B, S, d, W.F32, xc, t_mod, table, eps=1e-6)
    np.testing.assert_allclose(y, np.broadcast_to((t_mod[:, 0].astype(np.float64) + table[0])[:, None, :], y.shape),
                               rtol=0, atol=1e-12)


def test_modulate_invariant_under_affine_rescale_and_sources_add():
    B, S, d = 1, 3, 24
    x, t_mod, table = _mod_inputs(B, S, d, 3)
    y = ttref_adaln_modulate(B, S, d, W.F32, x, t_mod, table, eps=0.0)
    x2 = (x * 4.0 - 1.5).astype(np.float32)  # exact in fp32 for these magnitudes? close enough
    y2 = ttref_adaln_modulate(B, S, d, W.F32, x2, t_mod, table, eps=0.0)
    np.testing.assert_allclose(y, y2, rtol=1e-6, atol=1e-6)
    # the shared vectors and the layer's offsets enter only through their sum
    t2 = (t_mod + table[None]).astype(np.float32)
    y3 = ttref_adaln_modulate(B, S, d, W.F32, x, t2, np.zeros_like(table), eps=0.0)
    y4 = ttref_adaln_modulate(B, S, d, W.F32, x, np.zeros_like(t_mod),
                              (t_mod[0] + table).astype(np.float32), eps=0.0)
    np.testing.assert_allclose(y, y3, rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(y, y4, rtol=1e-6, atol=1e-6)


def test_gate_exact_and_uses_the_gate_slot_only():
    B, S, d = 2, 3, 8
    r = np.random.default_rng(4)
    x = r.integers(-8, 9, (B, S, d)).astype(np.float32)
    f = (r.integers(-8, 9, (B, S, d)) * 0.5).astype(np.float32)
    t_mod = np.zeros((B, 3, d), np.float32)
    table = np.zeros((3, d), np.float32)
    t_mod[:, 2] = r.integers(-4, 5, (B, d)) * 0.25
    table[2] = r.integers(-4, 5, d) * 0.125
    t_mod[:, :2] = 1e6  # shift and scale slots must not enter the residual
    table[:2] = -7e5
    out = ttref_adaln_gate(B, S, d, W.F32, x, f, t_mod, table)
    gate = (t_mod[:, 2].astype(np.float64) + table[2])[:, None, :]
    assert np.array_equal(out, x + gate * f)
    t_mod[:, 2] = 0
    table[2] = 0
    assert np.array_equal(ttref_adaln_gate(B, S, d, W.F32, x, f, t_mod, table), x.astype(np.float64))


def test_adaln_bf16_decode():
    B, S, d = 1, 2, 32
    x, t_mod, table = _mod_inputs(B, S, d, 5)
    xb = W.f32_to_bf16_bits(x)
    xf = W.bf16_bits_to_f32(xb)
    assert np.array_equal(ttref_adaln_modulate(B, S, d, W.BF16, xb, t_mod, table),
                          ttref_adaln_modulate(B, S, d, W.F32, xf, t_mod, table))
    assert np.array_equal(ttref_adaln_gate(B, S, d, W.BF16, xb, xb, t_mod, table),
                          ttref_adaln_gate(B, S, d, W.F32, xf, xf, t_mod, table))
