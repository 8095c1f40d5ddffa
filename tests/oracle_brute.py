"""Per-element loops for tiny inputs: an independent second statement of
explicit MLA, used only to pin the fp64 oracle.

Everything is plain Python scalars and loops: no numpy linear algebra, no
shared helper with ``oracle/``. The sample holding a position is found by a
linear scan over the sample boundaries (the oracle uses a binary search).
"""

import math


def sample_start(p, cu):
    if cu is None:
        return 0
    start = None
    for k in range(len(cu) - 1):
        if cu[k] <= p < cu[k + 1]:
            start = cu[k]
    assert start is not None, "position outside the packed range"
    return int(start)


def brute_forward(q, c_kv, k_rope, W_UK, W_UV, q_offset=0, cu=None, scale=None,
                  positions=None):
    """q[i][h][d], c_kv[t][c], k_rope[t][r], W_UK[c][h*dn+d], W_UV[c][h*dv+d]
    as nested lists (or arrays indexed element by element). Row i sits at
    positions[i] if given, else at q_offset + i."""
    S_loc, n_h, d_qk = len(q), len(q[0]), len(q[0][0])
    S, d_c = len(c_kv), len(c_kv[0])
    d_rope = len(k_rope[0])
    d_nope = d_qk - d_rope
    d_v = len(W_UV[0]) // n_h
    if scale is None:
        scale = 1.0 / math.sqrt(d_qk)
    out = [[[0.0] * d_v for _ in range(n_h)] for _ in range(S_loc)]
    lse = [[0.0] * n_h for _ in range(S_loc)]
    for h in range(n_h):
        Kfull = []
        Vfull = []
        for t in range(S):
            kn = [sum(float(c_kv[t][c]) * float(W_UK[c][h * d_nope + d]) for c in range(d_c))
                  for d in range(d_nope)]
            Kfull.append(kn + [float(k_rope[t][r]) for r in range(d_rope)])
            Vfull.append([sum(float(c_kv[t][c]) * float(W_UV[c][h * d_v + d]) for c in range(d_c))
                          for d in range(d_v)])
        for i in range(S_loc):
            p = q_offset + i if positions is None else int(positions[i])
            lo = sample_start(p, cu)
            js = list(range(lo, p + 1))
            s = [scale * sum(float(q[i][h][d]) * Kfull[j][d] for d in range(d_qk)) for j in js]
            m = max(s)
            z = sum(math.exp(x - m) for x in s)
            L = m + math.log(z)
            lse[i][h] = L
            for d in range(d_v):
                out[i][h][d] = sum(math.exp(s[a] - L) * Vfull[j][d] for a, j in enumerate(js))
    return out, lse


def brute_visible_pairs(S_loc, q_offset, cu=None):
    n = 0
    for i in range(S_loc):
        p = q_offset + i
        for j in range(0, p + 1):
            if sample_start(j, cu) == sample_start(p, cu):
                n += 1
    return n
