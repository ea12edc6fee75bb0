"""Scalar brute-force evaluation of pair-biased attention (tiny sizes only).

Independent of ``oracle/``: plain Python floats, explicit loops, math.fsum,
math.exp.  Used to pin the fp64 reference.  Every quantity is computed from
its definition (LayerNorm with biased variance, linear maps y = x @ W,
logits q.k/sqrt(d) + bias, softmax over kept keys, sigmoid gate, output map).
"""
import math


def _ln(x, gamma, beta, eps):
    c = len(x)
    mu = math.fsum(x) / c
    var = math.fsum((t - mu) * (t - mu) for t in x) / c
    inv = 1.0 / math.sqrt(var + eps)
    return [(x[n] - mu) * inv * gamma[n] + beta[n] for n in range(c)]


def _matvec(x, W):
    """y[o] = sum_n x[n] W[n][o]."""
    return [math.fsum(x[n] * W[n][o] for n in range(len(x))) for o in range(len(W[0]))]


def _sig(t):
    return 1.0 / (1.0 + math.exp(-t))


def _lst(a):
    return a.tolist() if hasattr(a, "tolist") else a


def _unpack(p):
    return {k: _lst(v) for k, v in p.items() if k != "eps"}, float(p.get("eps", 1e-5))


def _attend(qv, keys, vals, biases, keep, d):
    """One query against a list of keys: returns sum_k w_k v_k (list of d)."""
    idx = [k for k in range(len(keys)) if keep[k]]
    if not idx:
        return [0.0] * d
    scale = 1.0 / math.sqrt(d)
    logits = {k: math.fsum(qv[t] * keys[k][t] for t in range(d)) * scale + biases[k] for k in idx}
    mx = max(logits.values())
    e = {k: math.exp(logits[k] - mx) for k in idx}
    tot = math.fsum(e.values())
    return [math.fsum(e[k] / tot * vals[k][t] for k in idx) for t in range(d)]


def _project_all(x, P, H):
    """LN + q/k/v/gpre for one feature vector; returns dict of lists."""
    xh = _ln(x, P["ln_gamma"], P["ln_beta"], P["_eps"])
    return {"xh": xh, "q": _matvec(xh, P["w_q"]), "k": _matvec(xh, P["w_k"]),
            "v": _matvec(xh, P["w_v"]), "g": _matvec(xh, P["w_g"])}


def _finish(o_cat, g_pre, P):
    g = [_sig(g_pre[n] + P["b_g"][n]) for n in range(len(g_pre))]
    y = _matvec([g[n] * o_cat[n] for n in range(len(o_cat))], P["w_o"])
    return [y[n] + P["b_o"][n] for n in range(len(y))]


def _bias_scalar(x, P, h, prefix):
    xh = _ln(x, P[prefix + "_gamma"], P[prefix + "_beta"], P["_eps"])
    return math.fsum(xh[n] * P["w_b"][n][h] for n in range(len(xh)))


def tri(z, mask, p, H, orientation):
    """Full [I][I][c] output of triangle attention, START (0) or END (1)."""
    P, eps = _unpack(p)
    P["_eps"] = eps
    z = _lst(z)
    I = len(z)
    c = len(z[0][0])
    hd = len(P["w_q"][0])
    d = hd // H
    keepM = [[1] * I for _ in range(I)] if mask is None else _lst(mask)
    pr = [[_project_all(z[a][b], P, H) for b in range(I)] for a in range(I)]
    Bz = [[[_bias_scalar(z[a][b], P, h, "ln") for h in range(H)] for b in range(I)] for a in range(I)]
    out = [[None] * I for _ in range(I)]
    for a in range(I):
        for b in range(I):
            o_cat = []
            for h in range(H):
                sl = slice(h * d, (h + 1) * d)
                if orientation == 0:   # row a, query b, keys (a, k)
                    qv = pr[a][b]["q"][sl]
                    keys = [pr[a][k]["k"][sl] for k in range(I)]
                    vals = [pr[a][k]["v"][sl] for k in range(I)]
                    biases = [Bz[b][k][h] for k in range(I)]
                    keep = [keepM[a][k] != 0 for k in range(I)]
                else:                  # column b, query a, keys (k, b)
                    qv = pr[a][b]["q"][sl]
                    keys = [pr[k][b]["k"][sl] for k in range(I)]
                    vals = [pr[k][b]["v"][sl] for k in range(I)]
                    biases = [Bz[k][a][h] for k in range(I)]
                    keep = [keepM[k][b] != 0 for k in range(I)]
                o_cat += _attend(qv, keys, vals, biases, keep, d)
            out[a][b] = _finish(o_cat, pr[a][b]["g"], P)
    return out


def msa(m, z, mask, p, H):
    """Full [S][I][c_m] output of MSA row attention with pair bias."""
    P, eps = _unpack(p)
    P["_eps"] = eps
    m = _lst(m)
    z = _lst(z)
    S, I = len(m), len(m[0])
    hd = len(P["w_q"][0])
    d = hd // H
    keepM = [[1] * I for _ in range(S)] if mask is None else _lst(mask)
    Bz = [[[_bias_scalar(z[i][j], P, h, "lnz") for h in range(H)] for j in range(I)] for i in range(I)]
    out = [[None] * I for _ in range(S)]
    for s in range(S):
        pr = [_project_all(m[s][i], P, H) for i in range(I)]
        for i in range(I):
            o_cat = []
            for h in range(H):
                sl = slice(h * d, (h + 1) * d)
                o_cat += _attend(pr[i]["q"][sl], [pr[j]["k"][sl] for j in range(I)],
                                 [pr[j]["v"][sl] for j in range(I)], [Bz[i][j][h] for j in range(I)],
                                 [keepM[s][j] != 0 for j in range(I)], d)
            out[s][i] = _finish(o_cat, pr[i]["g"], P)
    return out


def partial(q_pairs, kv_pairs, bias, mask, p, H):
    """One key shard: per-head o = sum_k w_k v_k over the shard's kept keys
    and lse = ln sum_k exp(logit_k) (explicit loops).  q_pairs [R][Jq][c],
    kv_pairs [R][Kn][c], bias [H][Jq][Kn], mask [R][Kn] or None.  Returns
    (o [R][Jq][H*d], lse [R][H][Jq]); a query with no kept key gets o = 0 and
    lse = -inf."""
    P, eps = _unpack(p)
    P["_eps"] = eps
    qp, kp, bias = _lst(q_pairs), _lst(kv_pairs), _lst(bias)
    R, Jq, Kn = len(qp), len(qp[0]), len(kp[0])
    hd = len(P["w_q"][0])
    d = hd // H
    keepM = [[1] * Kn for _ in range(R)] if mask is None else _lst(mask)
    o = [[None] * Jq for _ in range(R)]
    lse = [[[None] * Jq for _ in range(H)] for _ in range(R)]
    for r in range(R):
        pq = [_project_all(qp[r][j], P, H) for j in range(Jq)]
        pk = [_project_all(kp[r][k], P, H) for k in range(Kn)]
        for j in range(Jq):
            o_cat = []
            for h in range(H):
                sl = slice(h * d, (h + 1) * d)
                keep = [keepM[r][k] != 0 for k in range(Kn)]
                o_cat += _attend(pq[j]["q"][sl], [pk[k]["k"][sl] for k in range(Kn)],
                                 [pk[k]["v"][sl] for k in range(Kn)], bias[h][j], keep, d)
                idx = [k for k in range(Kn) if keep[k]]
                if idx:
                    lg = [math.fsum(pq[j]["q"][sl][t] * pk[k]["k"][sl][t] for t in range(d)) / math.sqrt(d)
                          + bias[h][j][k] for k in idx]
                    mx = max(lg)
                    lse[r][h][j] = mx + math.log(math.fsum(math.exp(t - mx) for t in lg))
                else:
                    lse[r][h][j] = -math.inf
            o[r][j] = o_cat
    return o, lse
