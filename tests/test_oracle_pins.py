"""Pins for the fp64 CPU oracle: checks against things other than the oracle itself.

Each test pins the oracle to a library routine, a closed form, an invariant of the
method, or a hand-derived fixture under tests/golden/ (each with its citation). They are
chosen so that a plausible slip in the oracle (a dropped key set, a wrong sign, a wrong
KV-head index, a transposed operand, >= instead of >, a wrong tie rule) fails one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

from block_diffusion_lm_tt_amd import workloads as W
from oracle import ttref_block_denoise_attn, ttref_commit, ttref_ctx_append, ttref_decode, ttref_lmhead_commit

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _dec(a, dtype):
    """Library decode (torch) of bf16 bits / fp32 to float64, independent of the oracle's."""
    if dtype == W.BF16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).double()
    return torch.from_numpy(np.ascontiguousarray(a)).double()


def _attn(x: W.AttnInputs):
    return ttref_block_denoise_attn(x.B, x.S, x.Hq, x.Hkv, x.D, x.Lmax, x.dtype, x.q, x.k_blk, x.v_blk,
                                    x.k_ctx, x.v_ctx, x.ctx_len)


def _sdpa(x: W.AttnInputs):
    """torch fp64 scaled_dot_product_attention over [context keys ; block keys], GQA grouping by
    the library's own enable_gqa rule (query head h reads KV head h // (Hq/Hkv))."""
    out = torch.zeros((x.B, x.S, x.Hq, x.D), dtype=torch.float64)
    q, kb, vb = _dec(x.q, x.dtype), _dec(x.k_blk, x.dtype), _dec(x.v_blk, x.dtype)
    kc, vc = _dec(x.k_ctx, x.dtype), _dec(x.v_ctx, x.dtype)
    for b in range(x.B):
        n = int(x.ctx_len[b])
        k = torch.cat([kc[b, :n], kb[b]], 0)  # [n+S, Hkv, D]
        v = torch.cat([vc[b, :n], vb[b]], 0)
        o = torch.nn.functional.scaled_dot_product_attention(
            q[b].transpose(0, 1)[None], k.transpose(0, 1)[None], v.transpose(0, 1)[None], enable_gqa=True)
        out[b] = o[0].transpose(0, 1)
    return out.numpy()


# ------------------------------------------------------------------------------------------------
# decode
# ------------------------------------------------------------------------------------------------

def test_decode_matches_library_conversion():
    bits = np.array([0x0000, 0x8000, 0x3F80, 0xBF80, 0x0001, 0x807F, 0x7F7F, 0x7F80, 0xFF80, 0x4049,
                     0x3E20, 0xC2F6], dtype=np.uint16)
    got = ttref_decode(bits, W.BF16)
    want = _dec(bits, W.BF16).numpy()
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))
    f = np.array([1.5, -0.0, 3.4e38, 1e-45, -7.25], dtype=np.float32)
    assert np.array_equal(ttref_decode(f, W.F32), f.astype(np.float64))


def test_generator_rounding_is_rne():
    # ties to even: 1 + 2^-8 is halfway between bf16 1.0 and 1.0078125 -> rounds to 1.0 (even)
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -9], dtype=np.float32)
    got = W.f32_to_bf16_bits(x)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)


# ------------------------------------------------------------------------------------------------
# attention
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [W.F32, W.BF16])
@pytest.mark.parametrize("shape", [
    # B, S, Hq, Hkv, D, ctx_lens, Lmax
    (1, 4, 2, 1, 8, [5], 8),
    (2, 3, 6, 2, 16, [0, 7], 9),
    (3, 16, 8, 2, 32, [33, 1, 64], 70),
    (1, 1, 4, 4, 8, [3], 3),
])
def test_attn_matches_torch_sdpa(dtype, shape):
    B, S, Hq, Hkv, D, ctx, Lmax = shape
    x = W.make_attn(B, S, Hq, Hkv, D, ctx, Lmax=Lmax, dtype=dtype, seed=11)
    np.testing.assert_allclose(_attn(x), _sdpa(x), rtol=0, atol=1e-12)


def test_attn_ctx0_is_block_self_attention():
    x = W.make_attn(2, 8, 4, 2, 16, [0, 0], Lmax=4, dtype=W.BF16, seed=3)
    got = _attn(x)
    q, k, v = _dec(x.q, x.dtype), _dec(x.k_blk, x.dtype), _dec(x.v_blk, x.dtype)
    want = torch.nn.functional.scaled_dot_product_attention(
        q.transpose(1, 2), k.transpose(1, 2), v.transpose(1, 2), enable_gqa=True).transpose(1, 2)
    np.testing.assert_allclose(got, want.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("name", ["attn_joint_softmax.json", "attn_two_keys.json"])
def test_attn_golden(name):
    d = json.load(open(os.path.join(GOLDEN, name)))
    B, S, Hq, Hkv, D, Lmax = (d[k] for k in ("B", "S", "Hq", "Hkv", "D", "Lmax"))
    f = lambda key, shape: np.array(d[key], dtype=np.float64).astype(np.float32).reshape(shape)  # noqa
    out = ttref_block_denoise_attn(B, S, Hq, Hkv, D, Lmax, "f32", f("q", (B, S, Hq, D)),
                                   f("k_blk", (B, S, Hkv, D)), f("v_blk", (B, S, Hkv, D)),
                                   f("k_ctx", (B, Lmax, Hkv, D)), f("v_ctx", (B, Lmax, Hkv, D)),
                                   np.array(d["ctx_len"], dtype=np.int32))
    np.testing.assert_allclose(out, np.array(d["expected"]).reshape(B, S, Hq, D), rtol=0, atol=d["atol"])


def test_attn_closed_form_single_key():
    # ctx_len = 0 and S = 1: the only key is the query's own block key, so out = v exactly.
    x = W.make_attn(3, 1, 4, 2, 16, [0, 0, 0], Lmax=2, dtype=W.BF16, seed=5)
    out = _attn(x)
    v = _dec(x.v_blk, x.dtype).numpy()  # [B,1,Hkv,D]
    for h in range(4):
        np.testing.assert_array_equal(out[:, :, h], v[:, :, h // 2])


def test_attn_closed_form_constant_values_and_equal_keys():
    x = W.make_attn(2, 5, 4, 1, 8, [6, 2], Lmax=6, dtype=W.F32, seed=9)
    # constant V rows -> output is that constant, whatever the scores
    c = np.linspace(-2, 3, 8).astype(np.float32)
    for b in range(2):
        x.v_ctx[b, :x.ctx_len[b]] = c
    x.v_blk[:] = c
    np.testing.assert_allclose(_attn(x), np.broadcast_to(c, (2, 5, 4, 8)), rtol=0, atol=1e-12)
    # all keys equal -> uniform weights -> mean of the n = ctx_len + S value rows
    y = W.make_attn(2, 5, 4, 1, 8, [6, 2], Lmax=6, dtype=W.F32, seed=9)
    k = np.arange(8, dtype=np.float32) / 8
    for b in range(2):
        y.k_ctx[b, :y.ctx_len[b]] = k
    y.k_blk[:] = k
    out = _attn(y)
    for b in range(2):
        n = int(y.ctx_len[b])
        vals = np.concatenate([y.v_ctx[b, :n, 0], y.v_blk[b, :, 0]]).astype(np.float64)
        np.testing.assert_allclose(out[b], np.broadcast_to(vals.mean(0), (5, 4, 8)), rtol=0, atol=1e-12)


def test_attn_probabilities_match_library_softmax_and_sum_to_one():
    # One-hot value rows (D >= number of keys) make out[d] equal the weight of key d, so the
    # output is the probability row itself: it must sum to 1 and equal scipy's softmax of the
    # scaled scores (scores by a numpy matmul).
    B, S, Hq, Hkv, D, n_ctx = 1, 3, 2, 1, 16, 9
    x = W.make_attn(B, S, Hq, Hkv, D, [n_ctx], Lmax=12, dtype=W.F32, seed=21)
    n = n_ctx + S
    eye = np.eye(D, dtype=np.float32)
    x.v_ctx[0, :n_ctx, 0] = eye[:n_ctx]
    x.v_blk[0, :, 0] = eye[n_ctx:n]
    out = _attn(x)
    np.testing.assert_allclose(out.sum(-1), 1.0, rtol=0, atol=1e-14)
    assert (out >= 0).all() and np.all(out[..., n:] == 0)
    keys = np.concatenate([x.k_ctx[0, :n_ctx, 0], x.k_blk[0, :, 0]]).astype(np.float64)
    for i in range(S):
        for h in range(Hq):
            p = scipy.special.softmax(keys @ x.q[0, i, h].astype(np.float64) / math.sqrt(D))
            np.testing.assert_allclose(out[0, i, h, :n], p, rtol=0, atol=1e-14)


def test_attn_gqa_head_mapping():
    # KV head g carries constant value rows g+1; query head h must read KV head h // (Hq/Hkv).
    B, S, Hq, Hkv, D = 2, 4, 12, 3, 8
    x = W.make_attn(B, S, Hq, Hkv, D, [5, 3], Lmax=5, dtype=W.F32, seed=2)
    for g in range(Hkv):
        for b in range(B):
            x.v_ctx[b, :x.ctx_len[b], g] = g + 1
        x.v_blk[:, :, g] = g + 1
    out = _attn(x)
    for h in range(Hq):
        np.testing.assert_allclose(out[:, :, h], h // (Hq // Hkv) + 1, rtol=0, atol=1e-12)


def test_attn_block_permutation_equivariance():
    x = W.make_attn(2, 16, 8, 2, 32, [40, 7], Lmax=40, dtype=W.BF16, seed=4)
    perm = np.random.default_rng(0).permutation(16)
    y = W.AttnInputs(**{**x.__dict__})
    y.q = np.ascontiguousarray(x.q[:, perm])
    y.k_blk = np.ascontiguousarray(x.k_blk[:, perm])
    y.v_blk = np.ascontiguousarray(x.v_blk[:, perm])
    np.testing.assert_allclose(_attn(y), _attn(x)[:, perm], rtol=0, atol=1e-12)


def test_attn_context_permutation_invariance_and_padding_independence():
    x = W.make_attn(2, 4, 4, 2, 16, [30, 12], Lmax=33, dtype=W.BF16, seed=8)
    base = _attn(x)
    assert np.isfinite(base).all()  # NaN padding was never read
    y = W.AttnInputs(**{**x.__dict__})
    y.k_ctx, y.v_ctx = x.k_ctx.copy(), x.v_ctx.copy()
    rng = np.random.default_rng(1)
    for b in range(2):
        n = int(x.ctx_len[b])
        p = rng.permutation(n)
        y.k_ctx[b, :n] = x.k_ctx[b, p]
        y.v_ctx[b, :n] = x.v_ctx[b, p]
        y.k_ctx[b, n:] = 0x4700  # finite junk instead of NaN
        y.v_ctx[b, n:] = 0xC700
    np.testing.assert_allclose(_attn(y), base, rtol=0, atol=1e-12)


def test_attn_linear_in_values():
    x = W.make_attn(1, 4, 2, 1, 8, [10], Lmax=10, dtype=W.F32, seed=13)
    y = W.make_attn(1, 4, 2, 1, 8, [10], Lmax=10, dtype=W.F32, seed=14)
    for t in (x, y):  # dyadic values so that the fp32 sums below are exact
        t.v_ctx = np.round(t.v_ctx * 64) / 64
        t.v_blk = np.round(t.v_blk * 64) / 64
    z = W.AttnInputs(**{**x.__dict__})
    z.v_ctx = x.v_ctx + y.v_ctx
    z.v_blk = x.v_blk + y.v_blk
    yx = W.AttnInputs(**{**x.__dict__})
    yx.v_ctx, yx.v_blk = y.v_ctx, y.v_blk
    np.testing.assert_allclose(_attn(z), _attn(x) + _attn(yx), rtol=0, atol=1e-12)


# ------------------------------------------------------------------------------------------------
# commit
# ------------------------------------------------------------------------------------------------

def _commit(c: W.CommitInputs, gamma=None):
    return ttref_commit(c.B, c.S, c.V, c.dtype, c.logits, c.mask, c.gamma if gamma is None else gamma)


@pytest.mark.parametrize("dtype,V", [(W.F32, 1000), (W.BF16, 4096), (W.BF16, 1)])
def test_commit_matches_library_argmax_and_logsumexp(dtype, V):
    c = W.make_commit(3, 8, V, dtype, sigma=3.0, seed=17, gamma=0.3,
                      mask=(np.arange(24).reshape(3, 8) % 3 != 1).astype(np.uint8),
                      peaks={"mode": "bernoulli", "p": 0.5, "low": 4.0, "high": 9.0})
    tok, com, conf, z = _commit(c)
    x = _dec(c.logits, dtype).numpy()
    for b in range(3):
        for i in range(8):
            if not c.mask[b, i]:
                assert tok[b, i] == -1 and com[b, i] == 0 and conf[b, i] == 0
                continue
            row = x[b, i]
            assert tok[b, i] == np.argmax(row)  # numpy: first occurrence of the maximum
            lse = scipy.special.logsumexp(row)
            np.testing.assert_allclose(conf[b, i], math.exp(row.max() - lse), rtol=1e-13)
            np.testing.assert_allclose(z[b, i], math.exp(lse - row.max()), rtol=1e-13)
            np.testing.assert_allclose(conf[b, i], scipy.special.softmax(row).max(), rtol=1e-13)


@pytest.mark.parametrize("name", ["commit_small.json", "commit_strict.json"])
def test_commit_golden(name):
    d = json.load(open(os.path.join(GOLDEN, name)))
    B, S, V = d["B"], d["S"], d["V"]
    logits = np.array(d["logits"], dtype=np.float32)
    tok, com, conf, z = ttref_commit(B, S, V, "f32", logits, np.array(d["mask"], np.uint8), d["gamma"])
    assert tok.tolist() == d["expected_token_id"]
    assert com.tolist() == d["expected_committed"]
    zexp = np.array([[eval(e, {"__builtins__": {}}, {"exp": math.exp}) for e in r] for r in d["expected_Z"]])
    np.testing.assert_allclose(z, zexp, rtol=d["z_rtol"], atol=0)


def test_commit_closed_forms():
    V = 777
    logits = np.zeros((1, 3, V), dtype=np.float32)
    logits[0, 1, 500] = 100.0  # one dominant peak: conf = 1/(1+(V-1)e^-100) -> 1.0 in fp64
    logits[0, 2, :] = -3.25    # all equal, shifted: tok 0, conf 1/V
    tok, com, conf, z = ttref_commit(1, 3, V, "f32", logits, np.ones((1, 3), np.uint8), 0.9)
    assert tok.tolist() == [[0, 500, 0]]
    assert conf[0, 0] == pytest.approx(1 / V, rel=1e-14) and conf[0, 2] == pytest.approx(1 / V, rel=1e-14)
    assert conf[0, 1] == pytest.approx(1.0, abs=1e-15)
    assert com.tolist() == [[0, 1, 0]]


def test_commit_gamma_zero_commits_every_masked_position():
    c = W.make_commit(4, 16, 2048, W.BF16, seed=5, mask=W.random_mask(4, 16, 0, 16, seed=5))
    tok, com, _, _ = _commit(c, 0.0)
    assert np.array_equal(com, c.mask)
    assert np.array_equal(tok >= 0, c.mask.astype(bool))


@pytest.mark.parametrize("gamma", [1.0, 1.5, float("inf")])
def test_commit_gamma_above_one_commits_exactly_the_most_confident(gamma):
    c = W.make_commit(5, 16, 1500, W.BF16, seed=6, mask=W.random_mask(5, 16, 0, 16, seed=6),
                      peaks={"mode": "bernoulli", "p": 0.3, "low": 2.0, "high": 6.0})
    tok, com, conf, _ = _commit(c, gamma)
    for b in range(5):
        if c.mask[b].any():
            assert com[b].sum() == 1
            masked_conf = np.where(c.mask[b] == 1, conf[b], -1.0)
            assert com[b, int(np.argmax(masked_conf))] == 1
        else:
            assert com[b].sum() == 0


def test_commit_fallback_tie_goes_to_lowest_position():
    rng = np.random.default_rng(2)
    row = rng.standard_normal(64).astype(np.float32)
    flat = (0.1 * rng.standard_normal(64)).astype(np.float32)  # flatter row: lower confidence
    logits = np.stack([flat, row, row, row])[None]
    tok, com, conf, _ = ttref_commit(1, 4, 64, "f32", np.ascontiguousarray(logits),
                                     np.array([[1, 0, 1, 1]], np.uint8), 2.0)
    # position 1 is unmasked (not eligible); 2 and 3 tie exactly; the lowest (2) wins
    assert com.tolist() == [[0, 0, 1, 0]]
    assert tok[0, 1] == -1


def test_commit_monotone_in_gamma_and_unmasked_untouched():
    w = W.WORKLOADS[3]
    c = W.make_commit(8, 16, 8192, W.BF16, seed=w.seed, mask=W.random_mask(8, 16, 4, 16, seed=1),
                      peaks={"mode": "bernoulli", "p": 0.6, "low": 8.0, "high": 14.0})
    prev = None
    for g in [0.0, 0.3, 0.5, 0.8, 0.95, 0.999, 1.0]:
        tok, com, _, _ = _commit(c, g)
        assert np.all(com <= c.mask)
        assert np.all(tok[c.mask == 0] == -1)
        if prev is not None:
            assert np.all(com <= prev), f"committed set grew when gamma rose to {g}"
        prev = com


def test_commit_no_masked_positions_commits_nothing():
    c = W.make_commit(2, 8, 100, W.F32, seed=1, mask=np.zeros((2, 8), np.uint8))
    tok, com, conf, z = _commit(c, 1.5)
    assert com.sum() == 0 and np.all(tok == -1)


def test_commit_rejects_nan_gamma():
    c = W.make_commit(1, 2, 10, W.F32, seed=1)
    with pytest.raises(ValueError):
        _commit(c, float("nan"))



# ---- LM head followed by the commit ------------------------------------------------------------

def _lmhead(x: W.LmHeadInputs, gamma=None):
    return ttref_lmhead_commit(x.B, x.S, x.K, x.V, x.hidden, x.weight, x.mask,
                               x.gamma if gamma is None else gamma)


def _int_bf16(rng, shape, lo, hi):
    """Small integers as bf16 bits (exact), so that every logit is an exact integer."""
    return W.f32_to_bf16_bits(rng.integers(lo, hi + 1, size=shape).astype(np.float32))


@pytest.mark.parametrize("gamma", [0.0, 0.3, 0.8, 1.5])
def test_lmhead_on_integer_data_equals_commit_of_the_exact_logits(gamma):
    # integer hidden states and weights: numpy's int64 product gives the logits exactly, and
    # the commit of those logits (an fp32 tensor holding them exactly) must agree bit for bit
    rng = np.random.default_rng(11)
    B, S, K, V = 3, 8, 48, 300
    h = _int_bf16(rng, (B, S, K), -3, 3)
    w = _int_bf16(rng, (V, K), -2, 2)
    mask = W.random_mask(B, S, 0, S, seed=4)
    hi = W.bf16_bits_to_f32(h).astype(np.int64)
    wi = W.bf16_bits_to_f32(w).astype(np.int64)
    logits = np.einsum("bsk,vk->bsv", hi, wi).astype(np.float32)  # |l| <= 288: exact
    ref = ttref_commit(B, S, V, "f32", np.ascontiguousarray(logits), mask, gamma)
    got = ttref_lmhead_commit(B, S, K, V, h, w, mask, gamma)
    for r, g in zip(ref, got):
        assert np.array_equal(r, g)
    assert (logits.max(-1, keepdims=True) == logits).sum(-1).max() > 1  # the tie rule is exercised


def test_lmhead_matches_library_fp64_matmul_argmax_and_softmax():
    x = W.make_lmhead(2, 8, 192, 1000, seed=9, gamma=0.6, mask=W.random_mask(2, 8, 3, 8, seed=2),
                      peaks={"p": 0.5, "low": 4.0, "high": 9.0})
    tok, com, conf, z = _lmhead(x)
    h = _dec(x.hidden, W.BF16).numpy()
    w = _dec(x.weight, W.BF16).numpy()
    logits = h @ w.T  # numpy fp64 matmul of the library-decoded inputs
    for b in range(x.B):
        masked = [i for i in range(x.S) if x.mask[b, i]]
        for i in range(x.S):
            if not x.mask[b, i]:
                assert tok[b, i] == -1 and com[b, i] == 0 and conf[b, i] == 0
                continue
            row = logits[b, i]
            assert tok[b, i] == np.argmax(row)
            np.testing.assert_allclose(conf[b, i], scipy.special.softmax(row).max(), rtol=1e-12)
            np.testing.assert_allclose(z[b, i], math.exp(scipy.special.logsumexp(row) - row.max()), rtol=1e-12)
        above = [i for i in masked if conf[b, i] > x.gamma]
        want = above if above else ([max(masked, key=lambda i: conf[b, i])] if masked else [])
        assert sorted(np.nonzero(com[b])[0].tolist()) == sorted(want)


def test_lmhead_closed_form_one_hot_head():
    # head rows w_v = 2 e_v (V = K), hidden state c e_j: logits 2c at j, 0 elsewhere
    K = V = 64
    w = W.f32_to_bf16_bits(2.0 * np.eye(V, K, dtype=np.float32))
    hid = np.zeros((1, 3, K), np.float32)
    hid[0, 0, 5], hid[0, 1, 40], hid[0, 2, 63] = 1.0, 3.0, 0.5
    tok, com, conf, z = ttref_lmhead_commit(1, 3, K, V, W.f32_to_bf16_bits(hid), w,
                                            np.ones((1, 3), np.uint8), 0.5)
    assert tok.tolist() == [[5, 40, 63]]
    for i, c in enumerate([1.0, 3.0, 0.5]):
        assert conf[0, i] == pytest.approx(1.0 / (1.0 + (V - 1) * math.exp(-2.0 * c)), rel=1e-14)
    assert com.tolist() == [[0, 1, 0]]  # only 2c = 6 clears 0.5


def test_lmhead_does_not_read_unmasked_hidden_rows():
    x = W.make_lmhead(2, 6, 32, 200, seed=3, mask=np.array([[1, 0, 1, 0, 0, 1], [0, 0, 0, 0, 0, 0]], np.uint8))
    ref = _lmhead(x)
    hid = x.hidden.copy()
    hid[x.mask == 0] = W.BF16_NAN
    got = ttref_lmhead_commit(x.B, x.S, x.K, x.V, hid, x.weight, x.mask, x.gamma)
    for r, g in zip(ref, got):
        assert np.array_equal(r, g)
    assert got[1][1].sum() == 0 and np.all(got[0][1] == -1)


# ---- context cache update after a commit ------------------------------------------------------

def _append_case(B, S, Hkv, D, Lmax, dtype, ctx, seed):
    rng = np.random.default_rng(seed)
    bits = np.uint16 if dtype == W.BF16 else np.float32
    mk = (lambda *sh: rng.integers(0, 1 << 16, size=sh, dtype=np.uint16)) if dtype == W.BF16 else \
        (lambda *sh: rng.standard_normal(sh).astype(np.float32))
    kn, vn = mk(B, S, Hkv, D), mk(B, S, Hkv, D)
    kc, vc = mk(B, Lmax, Hkv, D), mk(B, Lmax, Hkv, D)
    assert kn.dtype == bits
    return kn, vn, kc, vc, np.array(ctx, dtype=np.int32)


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_append_equals_concatenation(dtype):
    """Each fitting sequence's cache is [old rows 0:n ; the block ; old rows n+S:], built here with
    numpy concatenation; the rest is untouched and flagged."""
    B, S, Hkv, D, Lmax = 6, 3, 2, 5, 9
    ctx = [0, 4, 6, 7, 9, -1]  # fits, fits, fits exactly, too long, full, negative
    kn, vn, kc, vc, cl = _append_case(B, S, Hkv, D, Lmax, dtype, ctx, seed=3)
    k2, v2, c2, skipped = ttref_ctx_append(B, S, Hkv, D, Lmax, dtype, kn, vn, kc, vc, cl, bump=1)
    for b, n in enumerate(ctx):
        fits = 0 <= n and n + S <= Lmax
        assert skipped[b] == (0 if fits else 1)
        if fits:
            ek = np.concatenate([kc[b, :n], kn[b], kc[b, n + S:]])
            ev = np.concatenate([vc[b, :n], vn[b], vc[b, n + S:]])
            assert c2[b] == n + S
        else:
            ek, ev = kc[b], vc[b]
            assert c2[b] == n
        assert ek.tobytes() == k2[b].tobytes() and ev.tobytes() == v2[b].tobytes(), f"sequence {b}"


def test_append_without_bump_keeps_lengths():
    kn, vn, kc, vc, cl = _append_case(3, 2, 1, 4, 8, W.BF16, [0, 3, 6], seed=4)
    k2, _, c2, skipped = ttref_ctx_append(3, 2, 1, 4, 8, W.BF16, kn, vn, kc, vc, cl, bump=0)
    assert np.array_equal(c2, cl) and not skipped.any()
    assert np.array_equal(k2[1, 3:5], kn[1])


def test_append_twice_equals_one_append_of_both_blocks():
    """Appending block A then block B (bumping) equals appending [A ; B] as one block of 2S."""
    B, S, Hkv, D, Lmax = 4, 3, 2, 4, 13
    ctx = [0, 2, 7, 5]
    ka, va, kc, vc, cl = _append_case(B, S, Hkv, D, Lmax, W.BF16, ctx, seed=5)
    kb, vb, _, _, _ = _append_case(B, S, Hkv, D, Lmax, W.BF16, ctx, seed=6)
    k1, v1, c1, _ = ttref_ctx_append(B, S, Hkv, D, Lmax, W.BF16, ka, va, kc, vc, cl, bump=1)
    k1, v1, c1, s1 = ttref_ctx_append(B, S, Hkv, D, Lmax, W.BF16, kb, vb, k1, v1, c1, bump=1)
    kab = np.ascontiguousarray(np.concatenate([ka, kb], axis=1))
    vab = np.ascontiguousarray(np.concatenate([va, vb], axis=1))
    k2, v2, c2, s2 = ttref_ctx_append(B, 2 * S, Hkv, D, Lmax, W.BF16, kab, vab, kc, vc, cl, bump=1)
    assert np.array_equal(s1, s2) and np.array_equal(c1, c2)
    assert np.array_equal(k1, k2) and np.array_equal(v1, v2)


def test_append_then_attention_sees_the_block_as_context():
    """After the update, attention with an empty block position set reduces to the keys
    [old context ; appended block]: torch fp64 SDPA over that concatenation agrees with the
    oracle attention run on the updated cache (S'=1 query block whose own key is appended too)."""
    B, S, Hq, Hkv, D, Lmax = 2, 4, 4, 2, 8, 12
    x = W.make_attn(B, S, Hq, Hkv, D, [3, 5], Lmax=Lmax, dtype=W.BF16, seed=7)
    k2, v2, c2, _ = ttref_ctx_append(B, S, Hkv, D, Lmax, W.BF16, x.k_blk, x.v_blk, x.k_ctx, x.v_ctx,
                                     x.ctx_len, bump=1)
    y = W.AttnInputs(B, S, Hq, Hkv, D, Lmax, W.BF16, x.q, x.k_blk, x.v_blk, k2, v2, c2)
    # keys seen by y: [ctx ; block ; block] -- the block twice. SDPA over exactly that set:
    out = torch.zeros((B, S, Hq, D), dtype=torch.float64)
    q = _dec(x.q, W.BF16)
    for b in range(B):
        n = int(c2[b])
        keys = torch.cat([_dec(k2, W.BF16)[b, :n], _dec(x.k_blk, W.BF16)[b]], 0)
        vals = torch.cat([_dec(v2, W.BF16)[b, :n], _dec(x.v_blk, W.BF16)[b]], 0)
        qq = q[b].permute(1, 0, 2)                       # [Hq, S, D]
        kk = keys.permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
        vv = vals.permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
        out[b] = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv).permute(1, 0, 2)
    got = _attn(y)
    assert np.abs(got - out.numpy()).max() < 1e-12
