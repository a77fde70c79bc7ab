"""Scalar brute-force statement of the decoder block, for tiny shapes.

TEST INFRASTRUCTURE ONLY (see oracle/block.py).  This is a second, separate
writing of the same block with explicit Python loops over every index and
the ``math`` module only; it shares no code with oracle/block.py so that a
slip in one (a transposed operand, a wrong head index, a dropped term) shows
up as a disagreement.  It follows the same pages and readings as
oracle/block.py; see that module's docstring for the sources.
"""
from __future__ import annotations

import math


def _dot(u, w):
    s = 0.0
    for a, b in zip(u, w):
        s += a * b
    return s


def _matvec(W, x):
    """W stored [out][in]; returns y[o] = sum_i W[o][i] x[i]."""
    return [_dot(row, x) for row in W]


def _rmsnorm(x, g, eps):
    ms = 0.0
    for v in x:
        ms += v * v
    ms /= len(x)
    r = 1.0 / math.sqrt(ms + eps)
    return [g[i] * x[i] * r for i in range(len(x))]


def _rope_one(u, pos, theta):
    hd = len(u)
    half = hd // 2
    out = [0.0] * hd
    for i in range(half):
        ang = pos * theta ** (-(2.0 * i) / hd)
        c, s = math.cos(ang), math.sin(ang)
        out[i] = u[i] * c - u[i + half] * s
        out[i + half] = u[i + half] * c + u[i] * s
    return out


def _sig(z):
    return 1.0 / (1.0 + math.exp(-z))


def _softplus(z):
    return math.log(1.0 + math.exp(z))


def _act(kind, z, cfg, W):
    if kind == "relu2":
        return max(z, 0.0) ** 2
    if kind == "xielu":
        beta = cfg["xielu_beta"]
        ap = _softplus(float(W["xielu_alpha_p"]))
        an = beta + _softplus(float(W["xielu_alpha_n"]))
        if z > 0:
            return ap * z * z + beta * z
        return an * (math.expm1(min(z, cfg["xielu_eps"])) - z) + beta * z
    raise ValueError(kind)


def _swiglu(m, Wg, Wu, Wd):
    gate = _matvec(Wg, m)
    up = _matvec(Wu, m)
    n = [gate[j] * _sig(gate[j]) * up[j] for j in range(len(gate))]
    return _matvec(Wd, n)


def _bf16(v):
    if v == 0.0:
        return 0.0
    m, e = math.frexp(v)
    q = m * 256.0
    r = math.floor(q)
    d = q - r
    if d > 0.5 or (d == 0.5 and (int(r) % 2 == 1)):
        r += 1
    return math.ldexp(r, e - 8)


def _f32(v):
    import struct
    return struct.unpack("f", struct.pack("f", v))[0]


def block(x, mask, W, cfg):
    """x: list of S rows (lists of H floats) for one sequence; mask: list of
    S ints or None.  W: dict of nested lists / floats.  Returns the
    layer_output rows and a few interior values, as lists."""
    S = len(x)
    H = len(x[0])
    nh, nkv, hd = cfg["nh"], cfg["nkv"], cfg["hd"]
    g = nh // nkv
    eps = cfg["eps"]
    L = lambda name: [list(map(float, r)) for r in W[name]]  # noqa: E731
    vec = lambda name: [float(v) for v in W[name]]  # noqa: E731

    a = [_rmsnorm(x[s], vec("w_in_norm"), eps) for s in range(S)]
    q = [[None] * nh for _ in range(S)]
    k = [[None] * nkv for _ in range(S)]
    v = [[None] * nkv for _ in range(S)]
    Wq, Wk, Wv, Wo = L("wq"), L("wk"), L("wv"), L("wo")
    for s in range(S):
        qf = _matvec(Wq, a[s])
        kf = _matvec(Wk, a[s])
        vf = _matvec(Wv, a[s])
        for h in range(nh):
            u = qf[h * hd:(h + 1) * hd]
            if cfg["qk_norm"]:
                u = _rmsnorm(u, vec("w_q_norm"), eps)
            if cfg["use_rope"]:
                u = _rope_one(u, s, cfg["theta"])
            q[s][h] = u
        for h in range(nkv):
            u = kf[h * hd:(h + 1) * hd]
            if cfg["qk_norm"]:
                u = _rmsnorm(u, vec("w_k_norm"), eps)
            if cfg["use_rope"]:
                u = _rope_one(u, s, cfg["theta"])
            k[s][h] = u
            v[s][h] = vf[h * hd:(h + 1) * hd]

    W_win = cfg["window"]
    layer_mid, mlp_in, out, head_outs = [], [], [], []
    for i in range(S):
        heads = []
        for h in range(nh):
            kvh = h // g
            sc = []
            for j in range(S):
                ok = j <= i
                if mask is not None and mask[j] == 0:
                    ok = False
                if W_win and W_win > 0 and not (i - j < W_win):
                    ok = False
                if ok:
                    sc.append((j, _dot(q[i][h], k[j][kvh]) / math.sqrt(hd)))
            if not sc:
                heads.append([0.0] * hd)
                continue
            mx = max(t for _, t in sc)
            ws = [(j, math.exp(t - mx)) for j, t in sc]
            z = sum(w for _, w in ws)
            o = [0.0] * hd
            for j, w in ws:
                for d in range(hd):
                    o[d] += (w / z) * v[j][kvh][d]
            heads.append(o)
        head_outs.append(heads)
        premix = []
        G = cfg["head_gate"]
        gl = _matvec(L("w_head_gate"), a[i]) if G else None
        for h in range(nh):
            for d in range(hd):
                val = heads[h][d]
                if G == nh:
                    val *= _sig(gl[h])
                elif G:
                    val *= _sig(gl[h * hd + d])
                premix.append(val)
        att = _matvec(Wo, premix)
        if cfg["sandwich"]:
            att = _rmsnorm(att, vec("w_post_attn_norm"), eps)
        mid = [x[i][c] + att[c] for c in range(H)]
        layer_mid.append(mid)
        m = _rmsnorm(mid, vec("w_mlp_norm"), eps)
        mlp_in.append(m)
        kind = cfg["mlp"]
        if kind == "swiglu":
            y = _swiglu(m, L("w_gate"), L("w_up"), L("w_down"))
        elif kind in ("relu2", "xielu"):
            up = _matvec(L("w_up"), m)
            n = [_act(kind, z, cfg, W) for z in up]
            y = _matvec(L("w_down"), n)
        elif kind == "moe":
            E = len(W["w_router"])
            logits = _matvec(L("w_router"), m)
            if cfg["dtype"] == "bf16":
                logits = [_bf16(t) for t in logits]
            sg = [_sig(t) for t in logits]
            biased = [_f32(_f32(sg[e]) + _f32(float(W["expert_bias"][e])))
                      for e in range(E)]
            chosen = []
            for _ in range(cfg["top_k"]):
                best = None
                for e in range(E):
                    if e in chosen:
                        continue
                    if best is None or biased[e] > biased[best]:
                        best = e
                chosen.append(best)
            tot = sum(sg[e] for e in chosen)
            y = [0.0] * H
            for e in chosen:
                w = sg[e] / tot * cfg["route_scale"]
                ye = _swiglu(m, [list(map(float, r)) for r in W["w_e_gate"][e]],
                             [list(map(float, r)) for r in W["w_e_up"][e]],
                             [list(map(float, r)) for r in W["w_e_down"][e]])
                for c in range(H):
                    y[c] += w * ye[c]
            ys = _swiglu(m, L("w_sh_gate"), L("w_sh_up"), L("w_sh_down"))
            y = [y[c] + ys[c] for c in range(H)]
        else:
            raise ValueError(kind)
        if cfg["sandwich"]:
            y = _rmsnorm(y, vec("w_post_mlp_norm"), eps)
        out.append([mid[c] + y[c] for c in range(H)])
    return {"layer_output": out, "layer_mid": layer_mid, "mlp_input": mlp_in,
            "attention_norm_output": a, "attention_head_outputs": head_outs}
