"""What the seeded workloads must satisfy for the parity claims to mean what they say (CPU).

* Bit-exact commits rest on fp64 decision margins: on every seeded commit row of the five
  workloads (the block loop's whole commit chain at each gamma of its sweep included), the
  oracle's margin to the threshold and to the fallback's runner-up must exceed 1e-12,
  far above the kernels' fp64 recheck error. Exceptions are printed (none expected).
  Reading: confidence above the threshold gamma decides a commit (gist.science explainer,
  Technical Summary > Training and Conditioning > Sampling).
* The long-context workload's planted hot keys (about 1% of each context) must carry most
  of the attention mass: its premise is that attention concentrates on about 1% of keys,
  which the wording of the inputs (a bias direction on every key) would not produce alone.
  The realised mass is computed in fp64 from the plain softmax over [context ; block] keys
  (gist.science explainer, Technical Summary > Methodology > Architecture) and printed.
"""
import numpy as np
import pytest

from block_diffusion_lm_tt_amd import workloads as W

from loopref import decision_margins, f32, oracle_commit_chain


def _say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("cid", [1, 2, 3, 4])
def test_commit_margins_single_step(cid):
    from oracle import ttref_commit
    w = W.WORKLOADS[cid]
    c = w.commit()
    g = f32(c.gamma)
    tok, com, conf, z = ttref_commit(c.B, c.S, c.V, c.dtype, c.logits, c.mask, g)
    thr, fb, small = decision_margins(c.mask, conf, z, g)
    _say(f"workload {cid}: {int(c.mask.sum())} masked rows, {int(com.sum())} committed; "
         f"min margins threshold {thr:.3e} fallback {fb:.3e}; below 1e-12: {small}")
    assert not small and thr > 1e-12 and fb > 1e-12


def test_commit_margins_block_loop_chain():
    w = W.WORKLOADS[5]
    commits = [w.commit(step=t) for t in range(w.steps)]
    for gamma in (0.5, 0.8, 0.95):
        g = f32(gamma)
        chain = oracle_commit_chain(commits, g)
        per_step = []
        for t, o in enumerate(chain):
            thr, fb, small = decision_margins(o["mask"], o["conf"], o["z"], g)
            per_step.append(int(o["committed"].sum()))
            _say(f"block loop gamma {g:.4f} step {t}: {int(o['mask'].sum())} masked, "
                 f"{int(o['threshold_committed'].sum())} by the rule; min margins threshold {thr:.3e} "
                 f"fallback {fb:.3e}; below 1e-12: {small}")
            assert not small and thr > 1e-12 and fb > 1e-12
        assert sum(per_step) == w.B * w.S
        _say(f"block loop gamma {g:.4f}: commits per step {per_step}")


def test_long_context_hot_keys_carry_the_attention_mass():
    w = W.WORKLOADS[4]
    x = w.attn()
    assert x.hot is not None and len(x.hot) == x.B * x.Hkv
    G = x.Hq // x.Hkv
    q = W.bf16_bits_to_f32(x.q).astype(np.float64)
    kc = W.bf16_bits_to_f32(x.k_ctx)
    kb = W.bf16_bits_to_f32(x.k_blk).astype(np.float64)
    masses = []
    for (b, g), hot in sorted(x.hot.items()):
        n = int(x.ctx_len[b])
        assert hot.size == int(np.ceil(0.01 * n))
        keys = np.concatenate([kc[b, :n, g].astype(np.float64), kb[b, :, g]], axis=0)  # [n+S, D]
        qs = q[b, :, g * G:(g + 1) * G].reshape(-1, x.D)                               # [S*G, D]
        s = qs @ keys.T / np.sqrt(x.D)
        s -= s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        m = p[:, hot].sum(axis=1)
        masses.append(m)
        _say(f"b={b} g={g}: {hot.size} hot keys of {n} ({100 * hot.size / n:.2f}%) hold "
              f"{100 * m.mean():.1f}% of the attention mass (min over queries {100 * m.min():.1f}%)")
    allm = np.concatenate(masses)
    _say(f"hot-set attention mass over all {allm.size} query rows: mean {allm.mean():.4f}, "
         f"min {allm.min():.4f}")
    assert allm.mean() > 0.8 and allm.min() > 0.5
