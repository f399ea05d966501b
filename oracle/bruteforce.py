"""Pure-Python scalar-loop evaluation of the block for tiny shapes.

TEST INFRASTRUCTURE ONLY (part of the oracle).  It writes every sum out as an
explicit loop over Python floats (math module only, no numpy arithmetic) so
that it can cross-check ``oracle.reference`` element by element on the toy
shapes (d_model=16, 8 query heads, 2 KV heads, head_dim=2 as in the worked
example of [L3] §4.1).  Page tags as in the package docstring.
"""

import math


def _tolist(a):
    return a.tolist() if hasattr(a, "tolist") else a


def rmsnorm_row(x, gamma, eps):
    # [RN] "How it works": x / sqrt(mean(x^2) + eps) * g
    s = 0.0
    for xi in x:
        s += xi * xi
    inv = 1.0 / math.sqrt(s / len(x) + eps)
    return [x[i] * inv * gamma[i] for i in range(len(x))]


def matvec(w, x):
    # y_o = sum_i W[o][i] x_i  (weights stored [out, in])
    out = []
    for row in w:
        acc = 0.0
        for i, xi in enumerate(x):
            acc += row[i] * xi
        out.append(acc)
    return out


def rope_head(vec, m, theta):
    # pair (2k, 2k+1) rotated by m * theta^(-2k/hd)  ([LA] §3)
    hd = len(vec)
    out = list(vec)
    for kk in range(hd // 2):
        ang = m * theta ** (-2.0 * kk / hd)
        c, s = math.cos(ang), math.sin(ang)
        a, b = vec[2 * kk], vec[2 * kk + 1]
        out[2 * kk] = a * c - b * s
        out[2 * kk + 1] = a * s + b * c
    return out


def attend(qv, keys, vals):
    # softmax(q.k_j / sqrt(hd)) weighted sum of v_j  ([L3] §4.5)
    hd = len(qv)
    sc = []
    for kv in keys:
        d = 0.0
        for i in range(hd):
            d += qv[i] * kv[i]
        sc.append(d / math.sqrt(hd))
    mx = max(sc)
    e = [math.exp(s - mx) for s in sc]
    z = sum(e)
    out = [0.0] * hd
    for j, vv in enumerate(vals):
        p = e[j] / z
        for i in range(hd):
            out[i] += p * vv[i]
    return out


def silu(z):
    return z / (1.0 + math.exp(-z))


def block_forward(x, w, positions, theta, eps, n_q, n_kv):
    """x [B][T][d] nested lists (or arrays), w as in oracle.reference,
    positions [B][T].  Cache-less causal prefill; returns y as nested lists."""
    x = _tolist(x)
    W = {kname: _tolist(v) for kname, v in w.items()}
    positions = _tolist(positions)
    B, T = len(x), len(x[0])
    hd = len(W["wq"]) // n_q
    r = n_q // n_kv
    y = []
    for b in range(B):
        qs, ks, vs = [], [], []
        for t in range(T):
            a = rmsnorm_row(x[b][t], W["attn_norm"], eps)
            q = matvec(W["wq"], a)
            k = matvec(W["wk"], a)
            v = matvec(W["wv"], a)
            m = positions[b][t]
            qs.append([rope_head(q[h * hd:(h + 1) * hd], m, theta) for h in range(n_q)])
            ks.append([rope_head(k[g * hd:(g + 1) * hd], m, theta) for g in range(n_kv)])
            vs.append([v[g * hd:(g + 1) * hd] for g in range(n_kv)])
        yb = []
        for t in range(T):
            o = []
            for h in range(n_q):
                g = h // r
                o += attend(qs[t][h], [ks[j][g] for j in range(t + 1)],
                            [vs[j][g] for j in range(t + 1)])
            ao = matvec(W["wo"], o)
            hrow = [x[b][t][i] + ao[i] for i in range(len(ao))]
            f = rmsnorm_row(hrow, W["ffn_norm"], eps)
            gate = matvec(W["w_gate"], f)
            up = matvec(W["w_up"], f)
            mact = [silu(gate[i]) * up[i] for i in range(len(gate))]
            dn = matvec(W["w_down"], mact)
            yb.append([hrow[i] + dn[i] for i in range(len(dn))])
        y.append(yb)
    return y
