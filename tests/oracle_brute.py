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


class MacCounter(dict):
    """Multiply-adds performed, by product: every inner loop below that
    multiplies two numbers and adds the result counts one under its name."""

    def add(self, name, n):
        self[name] = self.get(name, 0) + n


def _dot(a, b, counter=None, name=None):
    if counter is not None:
        counter.add(name, len(a))
    return sum(float(x) * float(y) for x, y in zip(a, b))


def _dims(q, c_kv, k_rope, W_UV):
    S_loc, n_h, d_qk = len(q), len(q[0]), len(q[0][0])
    d_c = len(c_kv[0])
    d_rope = len(k_rope[0])
    return S_loc, n_h, d_qk, d_c, d_rope, d_qk - d_rope, len(W_UV[0]) // n_h


def _needed_keys(S_loc, q_offset, cu, positions):
    """[first, last] latent rows any local row sees, by scanning the rows."""
    ps = [q_offset + i if positions is None else int(positions[i]) for i in range(S_loc)]
    return min(sample_start(p, cu) for p in ps), max(ps)


def _rebuild(c_kv, k_rope, W_UK, W_UV, h, t, d_c, d_nope, d_v, d_rope, counter):
    """K row (nope | rope) and V row of key t for head h."""
    col = lambda W, d, w: [W[c][h * w + d] for c in range(d_c)]  # noqa: E731
    kn = [_dot(c_kv[t], col(W_UK, d, d_nope), counter, "rebuild_K") for d in range(d_nope)]
    v = [_dot(c_kv[t], col(W_UV, d, d_v), counter, "rebuild_V") for d in range(d_v)]
    return kn + [float(k_rope[t][r]) for r in range(d_rope)], v


def brute_forward(q, c_kv, k_rope, W_UK, W_UV, q_offset=0, cu=None, scale=None,
                  positions=None, counter=None):
    """q[i][h][d], c_kv[t][c], k_rope[t][r], W_UK[c][h*dn+d], W_UV[c][h*dv+d]
    as nested lists (or arrays indexed element by element). Row i sits at
    positions[i] if given, else at q_offset + i. `counter` (a MacCounter)
    receives the multiply-adds of each product."""
    S_loc, n_h, d_qk, d_c, d_rope, d_nope, d_v = _dims(q, c_kv, k_rope, W_UV)
    if scale is None:
        scale = 1.0 / math.sqrt(d_qk)
    out = [[[0.0] * d_v for _ in range(n_h)] for _ in range(S_loc)]
    lse = [[0.0] * n_h for _ in range(S_loc)]
    if S_loc == 0:
        return out, lse
    k_first, k_last = _needed_keys(S_loc, q_offset, cu, positions)
    for h in range(n_h):
        Kfull, Vfull = {}, {}
        for t in range(k_first, k_last + 1):
            Kfull[t], Vfull[t] = _rebuild(c_kv, k_rope, W_UK, W_UV, h, t, d_c, d_nope, d_v,
                                          d_rope, counter)
        for i in range(S_loc):
            p = q_offset + i if positions is None else int(positions[i])
            lo = sample_start(p, cu)
            js = list(range(lo, p + 1))
            s = [scale * _dot(q[i][h], Kfull[j], counter, "score") for j in js]
            m = max(s)
            z = sum(math.exp(x - m) for x in s)
            L = m + math.log(z)
            lse[i][h] = L
            w = [math.exp(x - L) for x in s]
            for d in range(d_v):
                out[i][h][d] = _dot(w, [Vfull[j][d] for j in js], counter, "PV")
    return out, lse


def brute_backward(dout, q, c_kv, k_rope, W_UK, W_UV, out, q_offset=0, cu=None, scale=None,
                   positions=None, counter=None):
    """Gradients of sum(out * dout) by the chain rule, element by element:
    (dq, dc_kv, dk_rope, dW_UK, dW_UV) as nested lists. `out` is the forward
    output (as the backward receives it); the scores are recomputed from q
    and the rebuilt keys. `counter` receives the multiply-adds of each
    product, the rebuild of K and V included under its own names."""
    S_loc, n_h, d_qk, d_c, d_rope, d_nope, d_v = _dims(q, c_kv, k_rope, W_UV)
    S = len(c_kv)
    if scale is None:
        scale = 1.0 / math.sqrt(d_qk)
    dq = [[[0.0] * d_qk for _ in range(n_h)] for _ in range(S_loc)]
    dc = [[0.0] * d_c for _ in range(S)]
    dkr = [[0.0] * d_rope for _ in range(S)]
    dWk = [[0.0] * (n_h * d_nope) for _ in range(d_c)]
    dWv = [[0.0] * (n_h * d_v) for _ in range(d_c)]
    if S_loc == 0:
        return dq, dc, dkr, dWk, dWv
    k_first, k_last = _needed_keys(S_loc, q_offset, cu, positions)
    for h in range(n_h):
        Kfull, Vfull = {}, {}
        for t in range(k_first, k_last + 1):
            Kfull[t], Vfull[t] = _rebuild(c_kv, k_rope, W_UK, W_UV, h, t, d_c, d_nope, d_v,
                                          d_rope, counter)
        dK = {t: [0.0] * d_qk for t in Kfull}
        dV = {t: [0.0] * d_v for t in Vfull}
        for i in range(S_loc):
            p = q_offset + i if positions is None else int(positions[i])
            js = list(range(sample_start(p, cu), p + 1))
            s = [scale * _dot(q[i][h], Kfull[j], counter, "score") for j in js]
            m = max(s)
            L = m + math.log(sum(math.exp(x - m) for x in s))
            D = _dot(dout[i][h], out[i][h], counter, "D")
            for a, j in enumerate(js):
                P = math.exp(s[a] - L)
                dP = _dot(dout[i][h], Vfull[j], counter, "dP")
                dS = P * (dP - D)
                for d in range(d_v):
                    dV[j][d] += P * float(dout[i][h][d])
                counter is not None and counter.add("dV", d_v)
                for d in range(d_qk):
                    dq[i][h][d] += scale * dS * Kfull[j][d]
                    dK[j][d] += scale * dS * float(q[i][h][d])
                counter is not None and counter.add("dq", d_qk)
                counter is not None and counter.add("dK", d_qk)
        for t in Kfull:
            for r in range(d_rope):
                dkr[t][r] += dK[t][d_nope + r]
            for c in range(d_c):
                dc[t][c] += _dot(dK[t][:d_nope], [W_UK[c][h * d_nope + d] for d in range(d_nope)],
                                 counter, "dc_kv")
                dc[t][c] += _dot(dV[t], [W_UV[c][h * d_v + d] for d in range(d_v)], counter, "dc_kv")
                for d in range(d_nope):
                    dWk[c][h * d_nope + d] += float(c_kv[t][c]) * dK[t][d]
                for d in range(d_v):
                    dWv[c][h * d_v + d] += float(c_kv[t][c]) * dV[t][d]
                counter is not None and counter.add("dW", d_nope + d_v)
    return dq, dc, dkr, dWk, dWv


def brute_visible_pairs(S_loc, q_offset, cu=None):
    n = 0
    for i in range(S_loc):
        p = q_offset + i
        for j in range(0, p + 1):
            if sample_start(j, cu) == sample_start(p, cu):
                n += 1
    return n
