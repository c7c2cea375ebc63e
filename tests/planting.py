"""Inputs whose integer results are unique by construction (test
infrastructure; uses only the oracle and the seeded generators).

* ``planted_head``: lm_head inputs where every hidden row has one planted
  maximum logit at least ``margin`` above its runner-up.  For row r a seeded
  target id v_r is chosen; the 4-bit codes of lm_head row v_r are stepped by
  +-1 along sign(normed[r, k]) (k in a seeded order, codes kept in 0..15),
  updating every row's logit of column v_r exactly, until v_r leads row r by
  the margin.  The result is then re-checked with the oracle's own logits.
* ``router_margin_ok`` / ``head_margin``: margin gates for the MoE router and
  for argmax rows.
"""
from __future__ import annotations

import numpy as np

import oracle
from mtp_speculative_draft_amd import synth


def head_margin(logits_row: np.ndarray) -> float:
    top = np.partition(logits_row.astype(np.float64), -2)[-2:]
    return float(top[1] - top[0])


def planted_head(x: np.ndarray, gamma: np.ndarray, lm: synth.Q4, eps: float, margin: float = 0.5, seed: int = 7):
    """Returns (lm_planted, targets, normed, logits) with logits from the oracle."""
    g = np.random.default_rng(seed)
    m = x.shape[0]
    normed = oracle.rmsnorm(x, gamma, eps)
    base = oracle.gemv4(lm, normed).astype(np.float64)  # [m, V]
    V = lm.n
    targets = g.choice(V, size=m, replace=False)
    codes = synth.unpack_q4_codes(lm.codes[targets])  # [m, K] rows being planted
    cur = base.copy()
    nd = normed.astype(np.float64)
    for r in range(m):
        v = int(targets[r])
        row = codes[r].astype(np.int64)
        order = g.permutation(lm.k)
        others = np.delete(cur[r], v)
        need = float(others.max()) + margin
        sign = np.sign(nd[r])
        i = 0
        while cur[r, v] < need:
            k = int(order[i % lm.k])
            i += 1
            step = int(sign[k])
            if step == 0 or not (0 <= row[k] + step <= 15):
                if i > 40 * lm.k:
                    raise RuntimeError("planting did not converge")
                continue
            row[k] += step
            s = float(lm.scales[v, k // 32])
            cur[:, v] += s * step * nd[:, k]
        codes[r] = row.astype(np.uint8)
    planted = synth.Q4(lm.codes.copy(), lm.scales, lm.biases)
    planted.codes[targets] = synth.pack_q4(codes)
    # exact re-check: only the planted rows changed
    sub = synth.Q4(planted.codes[targets], lm.scales[targets], lm.biases[targets])
    logits = base.astype(np.float32).copy()
    logits[:, targets] = oracle.gemv4(sub, normed)
    for r in range(m):
        row = logits[r].astype(np.float64)
        v = int(targets[r])
        assert int(np.argmax(row)) == v
        assert row[v] - np.max(np.delete(row, v)) >= margin - 1e-6
    return planted, targets.astype(np.int32), normed, logits


def router_margin_ok(router_logits: np.ndarray, top_k: int, margin: float) -> bool:
    for row in router_logits.astype(np.float64):
        s = np.sort(row)[::-1]
        if s[top_k - 1] - s[top_k] < margin:
            return False
    return True
