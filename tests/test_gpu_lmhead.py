"""GPU parity of the fused LM head + commit (tt_lmhead_commit) against the fp64 CPU oracle.

The kernel accumulates each logit in fp32, so its logits differ from the exact ones by at
most eps_v = K * 2^-24 * sum_k |h_k w_vk| (bf16 products are exact in fp32; each of the at
most K additions rounds once, in any order). Per row, eps = max_v eps_v, computed here
exactly with a float64 matmul of |h| and |w|. From that bound:
  * token: equal to the oracle's wherever the exact top-1 margin exceeds 2 eps; elsewhere
    its exact logit lies within 2 eps of the exact maximum;
  * conf: |ln conf_gpu - ln conf| <= 2 eps + 1e-5 (1e-5: the fp32 exp sums, fp64 merge);
  * committed: a masked position whose exact conf clears gamma by more than that margin
    (either way) is decided as the oracle decides; the rest are checked for validity: the
    committed set is exactly {conf_gpu > gamma}, or, when that is empty, the single most
    confident masked position by conf_gpu (lowest position on ties).
Integer inputs make every logit exact in fp32 (eps = 0): there tokens, ties included, are
bit-exact.
"""
import math

import numpy as np
import pytest
import torch

from block_diffusion_lm_tt_amd import tensors as TZ
from block_diffusion_lm_tt_amd import workloads as W

pytestmark = pytest.mark.gpu

U = 2.0 ** -24
C3_PEAKS = {"p": 0.6, "low": 8.0, "high": 14.0}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_diffusion_lm_tt_amd as tt
    tt.lib()  # the HIP library must be there: no fallback
    return torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)


def _gpu(x: W.LmHeadInputs, dev, gamma=None):
    import block_diffusion_lm_tt_amd as tt
    h, w, m = TZ.lmhead_to_device(x, dev)
    tok, com, conf = tt.tt_lmhead_commit(h, w, m, x.gamma if gamma is None else gamma)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), com.cpu().numpy(), conf.double().cpu().numpy()


def _sub(x: W.LmHeadInputs, seqs) -> W.LmHeadInputs:
    c = np.ascontiguousarray
    return W.LmHeadInputs(len(seqs), x.S, x.K, x.V, c(x.hidden[seqs]), x.weight, c(x.mask[seqs]), x.gamma)


def _exact(x: W.LmHeadInputs, gamma, exact_logits=False):
    """Oracle outputs plus, per masked row, the exact logits (for validity checks), their
    top-2 margin and the error bound eps (0 when the inputs make every fp32 logit exact)."""
    from oracle import ttref_lmhead_commit
    tok, com, conf, _ = ttref_lmhead_commit(x.B, x.S, x.K, x.V, x.hidden, x.weight, x.mask, gamma)
    bs, ii = np.nonzero(x.mask)
    rows = {}
    if bs.size == 0:
        return tok, com, conf, rows
    hm = W.bf16_bits_to_f32(x.hidden[bs, ii]).astype(np.float64)  # [R, K] masked rows
    w = W.bf16_bits_to_f32(x.weight).astype(np.float64)             # [V, K]
    lg = hm @ w.T                           # library fp64 matmul (cross-check of the oracle)
    bound = np.abs(hm) @ np.abs(w).T        # sum_k |h_k w_vk|
    for r, (b, i) in enumerate(zip(bs, ii)):
        l = lg[r]
        eps = 0.0 if exact_logits else x.K * U * float(bound[r].max())
        top = np.sort(l)[-2:] if x.V > 1 else np.array([-np.inf, l[0]])
        rows[(int(b), int(i))] = (l, top[1] - top[0], eps)
    return tok, com, conf, rows


def _check(x: W.LmHeadInputs, got, want, gamma, what):
    tok_g, com_g, conf_g = got
    tok_o, com_o, conf_o, rows = want
    for b in range(x.B):
        for i in range(x.S):
            if not x.mask[b, i]:
                assert tok_g[b, i] == -1 and com_g[b, i] == 0 and conf_g[b, i] == 0, (what, b, i)
                continue
            l, margin, eps = rows[(b, i)]
            assert abs(l[tok_o[b, i]] - l.max()) <= 1e-9 * max(1.0, abs(l.max())), (what, "oracle token")
            if margin > 2 * eps:
                assert tok_g[b, i] == tok_o[b, i], (what, b, i, tok_g[b, i], tok_o[b, i], margin, eps)
            else:
                assert 0 <= tok_g[b, i] < x.V and l[tok_g[b, i]] >= l.max() - 2 * eps, (what, b, i)
            d = 2 * eps + 1e-5
            assert abs(math.log(conf_g[b, i]) - math.log(conf_o[b, i])) <= d, \
                (what, b, i, conf_g[b, i], conf_o[b, i], d)
        masked = [i for i in range(x.S) if x.mask[b, i]]
        # validity: the GPU's commits follow the rule on its own conf
        above = [i for i in masked if conf_g[b, i] > gamma]
        if above:
            want_set = set(above)
        elif masked:
            best = max(conf_g[b, i] for i in masked)
            want_set = {min(i for i in masked if conf_g[b, i] == best)}
        else:
            want_set = set()
        near = [i for i in masked
                if math.isfinite(gamma) and abs(conf_g[b, i] - gamma) <= 1e-6 * max(abs(gamma), 1e-30)]
        if not near:
            assert set(np.nonzero(com_g[b])[0].tolist()) == want_set, (what, b)
        # agreement with the oracle outside the error band
        sure = all(abs(math.log(conf_o[b, i]) - math.log(gamma)) > 2 * (2 * rows[(b, i)][2] + 1e-5)
                   for i in masked) if gamma > 0 and math.isfinite(gamma) else True
        if sure and masked:
            if any(conf_o[b, i] > gamma for i in masked):
                assert np.array_equal(com_g[b], com_o[b]), (what, b, com_g[b], com_o[b])
            else:  # fallback: equal when the winner is clear of the runner-up
                cs = sorted((conf_o[b, i] for i in masked), reverse=True)
                dmax = max(2 * rows[(b, i)][2] + 1e-5 for i in masked)
                if len(cs) == 1 or math.log(cs[0]) - math.log(cs[1]) > 2 * dmax:
                    assert np.array_equal(com_g[b], com_o[b]), (what, b, com_g[b], com_o[b])


def _int_case(B, S, K, V, seed, mask, hlo=-3, hhi=3, wlo=-2, whi=2, gamma=0.5):
    rng = np.random.default_rng(seed)
    f = lambda shape, lo, hi: W.f32_to_bf16_bits(rng.integers(lo, hi + 1, size=shape).astype(np.float32))  # noqa
    return W.LmHeadInputs(B, S, K, V, f((B, S, K), hlo, hhi), f((V, K), wlo, whi), mask, gamma)


INT_CASES = [
    # (id, B, S, K, V, mask kind)
    ("k64-v300-ragged", 3, 8, 64, 300, "random"),
    ("k128-v1000-rows320", 20, 16, 128, 1000, "c3"),
    ("k64-v1", 2, 4, 64, 1, "all"),
    ("k192-v257", 1, 129, 192, 257, "all"),
    ("k64-v512-none-masked", 2, 16, 64, 512, "none"),
    ("k128-v2048-rows512", 32, 16, 128, 2048, "all"),
]


def _mask(kind, B, S, seed):
    if kind == "all":
        return np.ones((B, S), np.uint8)
    if kind == "none":
        return np.zeros((B, S), np.uint8)
    if kind == "c3":
        return W.random_mask(B, S, 4, 16, seed=seed)
    return W.random_mask(B, S, 0, S, seed=seed)


@pytest.mark.parametrize("case", INT_CASES, ids=[c[0] for c in INT_CASES])
def test_lmhead_integer_data_bit_exact_tokens(dev, case):
    name, B, S, K, V, kind = case
    _say(f"[lmhead int] {name}")
    x = _int_case(B, S, K, V, seed=B * 7 + K, mask=_mask(kind, B, S, seed=K))
    got = _gpu(x, dev)
    want = _exact(x, x.gamma, exact_logits=True)  # integer sums below 2^24: exact in fp32
    assert np.array_equal(got[0], want[0]), f"{name}: tokens differ"  # exact logits: exact tokens
    _check(x, got, want, x.gamma, name)


RAND_CASES = [
    ("k192-v1000", 2, 8, 192, 1000, 0.6),
    ("k4096-v4096", 4, 16, 4096, 4096, 0.8),
    ("k1024-v33000-ragged", 3, 16, 1024, 33000, 0.8),
]


@pytest.mark.parametrize("case", RAND_CASES, ids=[c[0] for c in RAND_CASES])
def test_lmhead_random_data_within_bound(dev, case):
    name, B, S, K, V, gamma = case
    _say(f"[lmhead rand] {name}")
    x = W.make_lmhead(B, S, K, V, seed=V + K, gamma=gamma, mask=W.random_mask(B, S, 2, S, seed=3),
                      peaks=C3_PEAKS)
    _check(x, _gpu(x, dev), _exact(x, gamma), gamma, name)


@pytest.mark.parametrize("gamma", [0.0, 1.5, float("inf"), -1.0])
def test_lmhead_gamma_edges(dev, gamma):
    _say(f"[lmhead gamma] {gamma}")
    x = W.make_lmhead(3, 16, 256, 2000, seed=21, gamma=gamma, mask=W.random_mask(3, 16, 0, 16, seed=8),
                      peaks=C3_PEAKS)
    tok, com, conf = _gpu(x, dev)
    for b in range(x.B):
        n = int(x.mask[b].sum())
        if gamma <= 0:
            assert np.array_equal(com[b], x.mask[b])
        else:
            assert com[b].sum() == (1 if n else 0)
    _check(x, (tok, com, conf), _exact(x, gamma), gamma, f"gamma={gamma}")


def test_lmhead_unmasked_hidden_rows_never_read(dev):
    _say("[lmhead] unmasked rows are NaN")
    x = W.make_lmhead(2, 16, 128, 1024, seed=5, mask=W.random_mask(2, 16, 3, 10, seed=5), peaks=C3_PEAKS)
    want = _exact(x, x.gamma)
    hid = x.hidden.copy()
    hid[x.mask == 0] = W.BF16_NAN
    y = W.LmHeadInputs(x.B, x.S, x.K, x.V, hid, x.weight, x.mask, x.gamma)
    _check(y, _gpu(y, dev), want, x.gamma, "nan rows")


def test_lmhead_matches_unfused_commit_on_exact_logits(dev):
    # integer data: the LM head's logits are exact, so the fused call and tt_commit on the
    # materialised fp32 logits must agree (tokens, decisions) and conf to 1e-5
    import block_diffusion_lm_tt_amd as tt
    _say("[lmhead] fused vs unfused")
    x = _int_case(8, 16, 256, 3000, seed=4, mask=W.random_mask(8, 16, 1, 16, seed=4), gamma=0.2)
    h, w, m = TZ.lmhead_to_device(x, dev)
    logits = torch.matmul(h.float().reshape(-1, x.K), w.float().t().contiguous()).reshape(x.B, x.S, x.V)
    t1, c1, f1 = tt.tt_lmhead_commit(h, w, m, x.gamma)
    t2, c2, f2 = tt.tt_commit(logits.contiguous(), m, x.gamma)
    torch.cuda.synchronize()
    assert torch.equal(t1, t2)
    near = ((f2.double() - x.gamma).abs() <= 1e-4 * x.gamma).any()
    if not near:
        assert torch.equal(c1, c2)
    np.testing.assert_allclose(f1.double().cpu().numpy(), f2.double().cpu().numpy(), rtol=1e-5, atol=0)


def test_lmhead_full_size_sampled(dev):
    # the batched-serving commit workload behind an LM head: B=32, S=16, d_model 4096,
    # V=131072, 4..16 masked positions per sequence, peaks on 60% of positions; the whole
    # batch runs on the GPU, the oracle checks the first and the last sequence
    _say("[lmhead] full size B32 S16 K4096 V131072")
    w3 = W.WORKLOADS[3]
    x = W.make_lmhead(w3.B, w3.S, 4096, w3.V, seed=w3.seed, gamma=w3.gamma,
                      mask=W.random_mask(w3.B, w3.S, 4, 16, seed=w3.seed), peaks=C3_PEAKS)
    tok, com, conf = _gpu(x, dev)
    seqs = [0, w3.B - 1]
    y = _sub(x, seqs)
    _check(y, (tok[seqs], com[seqs], conf[seqs]), _exact(y, x.gamma), x.gamma, "full size")


def test_misaligned_operands_are_refused(dev):
    # the kernel's 16-byte loads need 16-byte aligned hidden states and head rows: an
    # operand off that boundary is refused (TT_ERR_UNSUPPORTED), nothing is launched
    import block_diffusion_lm_tt_amd as tt
    x = W.make_lmhead(1, 16, 64, 100, seed=8)
    h, w, m = TZ.lmhead_to_device(x, dev)
    buf = torch.empty(h.numel() + 1, dtype=h.dtype, device=dev)
    h2 = buf[1:].view(h.shape)
    h2.copy_(h)
    with pytest.raises(tt.TTError, match="UNSUPPORTED"):
        tt.tt_lmhead_commit(h2, w, m, 0.5)


# ---- exact mode (tt_lmhead_commit_exact): integer outputs equal the oracle's --------------

def _gpu_exact(x: W.LmHeadInputs, dev, gamma=None):
    import block_diffusion_lm_tt_amd as tt
    h, w, m = TZ.lmhead_to_device(x, dev)
    wb = tt.tt_lmhead_weight_bound(w)
    tok, com, conf = tt.tt_lmhead_commit(h, w, m, x.gamma if gamma is None else gamma, w_bound=wb)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), com.cpu().numpy(), conf.double().cpu().numpy()


def _check_exact(x: W.LmHeadInputs, got, gamma, what):
    want = _exact(x, gamma)
    tok_o, com_o = want[0], want[1]
    assert np.array_equal(got[0], tok_o), (what, "tokens", np.argwhere(got[0] != tok_o)[:5])
    assert np.array_equal(got[1], com_o), (what, "decisions", np.argwhere(got[1] != com_o)[:5])
    _check(x, got, want, gamma, what)  # confidences within the fp32 bound (exact where recomputed)


def test_lmhead_weight_bound(dev):
    import block_diffusion_lm_tt_amd as tt
    rng = np.random.default_rng(3)
    w = rng.normal(0.0, 0.05, size=(3001, 320)).astype(np.float32)
    w[1777] *= 7.0  # the largest row
    wb = W.f32_to_bf16_bits(w)
    got = float(tt.tt_lmhead_weight_bound(TZ.to_torch(wb, W.BF16, dev)).cpu()[0])
    norms = np.sqrt((W.bf16_bits_to_f32(wb).astype(np.float64) ** 2).sum(1))
    _say(f"[lmhead] weight bound {got:.9g} vs max row norm {norms.max():.9g}")
    assert norms.max() <= got <= norms.max() * (1 + 1e-6)


EXACT_RAND = [
    ("k192-v1000", 2, 8, 192, 1000, 0.6),
    ("k4096-v4096", 4, 16, 4096, 4096, 0.8),
    ("k1024-v33000-ragged", 3, 16, 1024, 33000, 0.8),
    ("k256-v2000-all-masked", 4, 16, 256, 2000, 0.05),
]


@pytest.mark.parametrize("case", EXACT_RAND, ids=[c[0] for c in EXACT_RAND])
def test_lmhead_exact_random(dev, case):
    name, B, S, K, V, gamma = case
    _say(f"[lmhead exact] {name}")
    mask = np.ones((B, S), np.uint8) if "all" in name else W.random_mask(B, S, 2, S, seed=3)
    x = W.make_lmhead(B, S, K, V, seed=V + K + 1, gamma=gamma, mask=mask, peaks=C3_PEAKS)
    _check_exact(x, _gpu_exact(x, dev), gamma, name)


@pytest.mark.parametrize("gamma", [0.0, 1.5, float("inf"), -1.0])
def test_lmhead_exact_gamma_edges(dev, gamma):
    x = W.make_lmhead(3, 16, 256, 2000, seed=21, gamma=gamma, mask=W.random_mask(3, 16, 0, 16, seed=8),
                      peaks=C3_PEAKS)
    _check_exact(x, _gpu_exact(x, dev), gamma, f"exact gamma={gamma}")


def test_lmhead_exact_integer_data(dev):
    x = _int_case(20, 16, 128, 1000, seed=147, mask=W.random_mask(20, 16, 4, 16, seed=128))
    _check_exact(x, _gpu_exact(x, dev), x.gamma, "exact integer")


def test_lmhead_exact_near_ties(dev):
    # margins far below the fp32 error bound, where the estimates cannot decide:
    #  - sequence 0: two positions whose hidden rows differ in one feature by one bf16 step
    #    (fallback between nearly equal confidences) and two identical rows (an exact tie:
    #    the lower position wins);
    #  - sequence 1: a row aimed at two head rows that differ in one feature by one bf16 step
    #    (top-2 logits nearly tied);
    #  - sequence 2: gamma set to a position's exact confidence rounded to fp32 (threshold).
    _say("[lmhead exact] near ties")
    B, S, K, V = 3, 16, 512, 3000
    x = W.make_lmhead(B, S, K, V, seed=77, gamma=0.3, mask=np.ones((B, S), np.uint8), peaks=C3_PEAKS)
    hid, wgt = x.hidden.copy(), x.weight.copy()
    hid[0, 5] = hid[0, 2]
    hid[0, 5, 17] = hid[0, 5, 17] + 1  # one bf16 step
    hid[0, 9] = hid[0, 3]
    wgt[1201] = wgt[1200]
    wgt[1201, 40] = wgt[1201, 40] + 1
    wf = W.bf16_bits_to_f32(wgt[1200]).astype(np.float64)
    hid[1, 4] = W.f32_to_bf16_bits((12.0 * wf / np.dot(wf, wf)).astype(np.float32))
    y = W.LmHeadInputs(B, S, K, V, hid, wgt, x.mask, x.gamma)
    _, _, conf_o, _ = _exact(y, 0.3)
    # for sequence 2 the gamma of the whole call cannot differ per sequence: take the row's
    # confidence as gamma for a second call on sequence 2 alone
    _check_exact(y, _gpu_exact(y, dev), 0.3, "near ties")
    z = _sub(y, [2])
    g2 = float(np.float32(conf_o[2, 7]))
    _check_exact(z, _gpu_exact(z, dev, gamma=g2), g2, "gamma at a confidence")


def test_lmhead_exact_full_size_sampled(dev):
    _say("[lmhead exact] full size B32 S16 K4096 V131072")
    w3 = W.WORKLOADS[3]
    x = W.make_lmhead(w3.B, w3.S, 4096, w3.V, seed=w3.seed, gamma=w3.gamma,
                      mask=W.random_mask(w3.B, w3.S, 4, 16, seed=w3.seed), peaks=C3_PEAKS)
    tok, com, conf = _gpu_exact(x, dev)
    seqs = [0, w3.B - 1]
    y = _sub(x, seqs)
    _check_exact(y, (tok[seqs], com[seqs], conf[seqs]), x.gamma, "exact full size")
