"""The ungated delta-rule loop in the form the pages give it.

TEST INFRASTRUCTURE ONLY.  "Kimi K3 深度拆解" (chenxutan.com), section 4.2
"线性注意力与 Delta Rule", describes a single-head loop over tokens with a
[d, d_v] state that starts at zero; for each token it first erases the old
memory along k (S minus beta times the outer product of k with k^T S), then
writes beta times the outer product of k and v, then reads q @ S.  There is no
forget gate.  It is restated here in numpy (with an optional initial state) so
that the gated oracle can be checked against it at g = 0.
"""
from __future__ import annotations

import numpy as np


def delta_rule(q, k, v, beta, S0=None):
    """q, k: [T, d]; v: [T, d_v]; beta: [T].  Returns (outputs [T, d_v], S)."""
    q, k, v, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, beta))
    S = np.zeros((q.shape[1], v.shape[1])) if S0 is None else np.array(S0, dtype=np.float64)
    outs = []
    for t in range(q.shape[0]):
        S = S - beta[t] * np.outer(k[t], k[t] @ S)   # erase along k_t
        S = S + beta[t] * np.outer(k[t], v[t])       # write k_t v_t^T
        outs.append(q[t] @ S)                        # read the updated state
    return np.array(outs), S
