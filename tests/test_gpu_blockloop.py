"""GPU parity of the whole block loop (B=16, S=32, ctx 8192, 6 layers, T=4 steps, bf16).

The loop runs exactly as the benchmark runs it (block_diffusion_lm_tt_amd/blockloop.py):
attention on every layer, the commit on each step's logits with the still-masked set
evolving, the end-of-block commit at the last step, and the context cache update of every
layer. The oracle replays the same chain on the same inputs: its own evolving masks, the
forced final commit, then ttref_ctx_append layer by layer. Bars: token_id and committed
bit-identical at every step, identical commits per step and ctx_len, caches bit-identical;
attention max-abs <= 1e-2 against the oracle on every unit of the calls checked.
"""
import numpy as np
import pytest
import torch

from block_diffusion_lm_tt_amd import workloads as W

from loopref import decision_margins, f32, oracle_commit_chain

pytestmark = pytest.mark.gpu

W5 = W.WORKLOADS[5]


def _say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def loop():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_diffusion_lm_tt_amd as tt
    from block_diffusion_lm_tt_amd.blockloop import BlockLoop
    tt.lib()
    _say(f"[blockloop] generating {W5.name}")
    return BlockLoop(W5, torch.device("cuda:0"), keep_host=True)


@pytest.mark.parametrize("gamma", [0.5, 0.8, 0.95])
def test_block_loop_commits_match_oracle(loop, gamma):
    g = f32(gamma)
    _say(f"[blockloop] commit chain gamma={g}")
    rec = []
    loop.counts.zero_()
    loop.run_block(g, record=rec)
    torch.cuda.synchronize()
    want = oracle_commit_chain(loop.commits, g)
    counts = loop.counts.cpu().numpy()
    for t, ((tok, com), o) in enumerate(zip(rec, want)):
        tok, com = tok.cpu().numpy(), com.cpu().numpy()
        masked = o["mask"].astype(bool)
        assert np.array_equal(tok, o["token_id"]), f"step {t}: token_id differs"
        assert np.array_equal(com, o["committed"]), f"step {t}: committed differs at {np.argwhere(com != o['committed'])[:5]}"
        assert counts[t] == int(o["committed"].sum()), f"step {t}: commit count {counts[t]} != {o['committed'].sum()}"
        thr, fb, small = decision_margins(o["mask"], o["conf"], o["z"], g)
        _say(f"  step {t}: {int(masked.sum())} masked, {int(com.sum())} committed "
             f"({int(o['threshold_committed'].sum())} by the rule); margins threshold {thr:.3e} "
             f"fallback {fb:.3e}; exceptions {small}")
    # every position is committed by the end of the block and ctx_len grew by S
    assert int(sum(o["committed"].sum() for o in want)) == W5.B * W5.S
    assert np.array_equal(loop.ctx.cpu().numpy(), W5.ctx_lens() + W5.S)


def test_block_loop_cache_update_matches_oracle(loop):
    from oracle import ttref_ctx_append
    loop.run_block(f32(0.8))
    torch.cuda.synchronize()
    ctx = W5.ctx_lens().astype(np.int32)
    Lx = W5.Lmax + W5.S
    for l in range(W5.layers):
        _say(f"[blockloop] cache update layer {l}")
        kh, vh = loop.host_ctx_kv[l]
        _, kb, vb = loop.qkv_host[W5.steps - 1][l]
        ek, ev, c2, sk = ttref_ctx_append(W5.B, W5.S, W5.Hkv, W5.D, Lx, W5.dtype, kb, vb, kh, vh, ctx,
                                          l == W5.layers - 1)
        assert not sk.any()
        got_k = loop.kcs[l].cpu().view(torch.int16).numpy().view(np.uint16)
        got_v = loop.vcs[l].cpu().view(torch.int16).numpy().view(np.uint16)
        assert got_k.tobytes() == ek.tobytes(), f"layer {l}: k cache differs"
        assert got_v.tobytes() == ev.tobytes(), f"layer {l}: v cache differs"
        ctx = c2
    assert np.array_equal(loop.ctx.cpu().numpy(), ctx)


def _checked_calls():
    rng = np.random.default_rng(W5.seed)
    later = list(zip(rng.integers(1, W5.steps, 3).tolist(), rng.integers(0, W5.layers, 3).tolist()))
    return [(0, l) for l in range(W5.layers)] + sorted(set(later))


@pytest.fixture(scope="module")
def loop_outs(loop):
    outs = {k: None for k in _checked_calls()}
    loop.run_block(f32(0.8), outs=outs)
    torch.cuda.synchronize()
    return {k: v.double().cpu().numpy() for k, v in outs.items()}


@pytest.mark.parametrize("call", _checked_calls(), ids=lambda c: f"t{c[0]}l{c[1]}")
def test_block_loop_attention_matches_oracle(loop, loop_outs, call):
    from oracle import ttref_block_denoise_attn
    t, l = call
    _say(f"[blockloop] attention step {t} layer {l}, every unit")
    kh, vh = loop.host_ctx_kv[l]
    q, kb, vb = loop.qkv_host[t][l]
    want = ttref_block_denoise_attn(W5.B, W5.S, W5.Hq, W5.Hkv, W5.D, W5.Lmax + W5.S, W5.dtype, q, kb, vb,
                                    kh, vh, W5.ctx_lens())
    got = loop_outs[call]
    assert np.isfinite(got).all()
    err = float(np.abs(got - want).max())
    _say(f"  max-abs err {err:.3e}")
    assert err <= 1e-2
