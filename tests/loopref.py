"""The block loop's commit chain replayed with the fp64 oracle (test helper, no pytest tests).

Nemotron-TwoTower (gist.science explainer), Technical Summary > Generation Process and
Training and Conditioning > Sampling; snilld.dk TwoTower article, "Blockwise generering i
praksis": a block starts with every position masked; each step commits the masked
positions whose confidence is above gamma (or the single most confident one); committed
positions leave the masked set; the last of the T steps commits every position still
masked (the end of the block, a harness policy).
"""
from __future__ import annotations

import numpy as np


def f32(gamma: float) -> float:
    """The threshold as the C-ABI receives it (a C float), widened back to double, so that
    the oracle and the kernels apply one and the same rule."""
    return float(np.float32(gamma))


def oracle_commit_chain(commits, gamma: float):
    """commits: the T steps' CommitInputs (their masks are ignored: the chain evolves its own).
    Returns per step a dict with the oracle's token_id, committed (after the end-of-block
    rule), conf, Z and the mask the step started from."""
    from oracle import ttref_commit
    T = len(commits)
    B, S = commits[0].B, commits[0].S
    mask = np.ones((B, S), np.uint8)
    out = []
    for t, c in enumerate(commits):
        tok, com, conf, z = ttref_commit(c.B, c.S, c.V, c.dtype, c.logits, mask, gamma)
        threshold_com = com.copy()
        if t == T - 1:
            com = mask.copy()
        out.append({"token_id": tok, "committed": com, "threshold_committed": threshold_com,
                    "conf": conf, "z": z, "mask": mask.copy()})
        mask = (mask & (1 - com)).astype(np.uint8)
    return out


def decision_margins(mask, conf, z, gamma: float):
    """The fp64 margins that bit-exact integer decisions rest on, for one commit call.

    threshold: per masked row, |Z * gamma - 1| (the relative distance of conf = 1/Z from
    gamma). fallback: per sequence that commits nothing by threshold, the relative gap
    (conf_best - conf_second) / conf_best between its two most confident masked positions;
    an exact tie (equal Z) is decided by position and counts as infinite margin.
    Returns (min threshold margin, min fallback margin, list of (b, i, kind, margin) below
    1e-12)."""
    m = mask.astype(bool)
    thr = np.abs(z[m] * gamma - 1.0) if m.any() else np.array([np.inf])
    small = []
    for b, i in zip(*np.nonzero(m & (np.abs(z * gamma - 1.0) < 1e-12))):
        small.append((int(b), int(i), "threshold", float(abs(z[b, i] * gamma - 1.0))))
    fb = [np.inf]
    for b in range(mask.shape[0]):
        rows = np.nonzero(m[b])[0]
        if rows.size < 2 or (conf[b, rows] > gamma).any():
            continue
        order = np.argsort(-conf[b, rows], kind="stable")
        c1, c2 = conf[b, rows[order[0]]], conf[b, rows[order[1]]]
        if z[b, rows[order[0]]] == z[b, rows[order[1]]]:
            continue
        gap = (c1 - c2) / c1
        fb.append(gap)
        if gap < 1e-12:
            small.append((b, int(rows[order[0]]), "fallback", float(gap)))
    return float(thr.min()), float(min(fb)), small
