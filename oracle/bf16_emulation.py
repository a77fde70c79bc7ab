"""The block evaluated in float64 but rounded to bfloat16 exactly where a
bf16-operand implementation must round: the normed stream a, q/k/v after
the q/k norm and rotary, the attention probabilities fed to the P.V
product, the gated head outputs (o_proj operand), the MLP operand m, the
MLP neurons, the mixture's weighted slot outputs, and y.  The residual
stream stays unrounded, as in libblock.

TEST INFRASTRUCTURE ONLY, like the rest of this package: its distance from
the exact oracle is the floor that no bf16-operand implementation can beat
by more than chance, and the GPU's error is judged against it.  It reuses
the oracle's step functions and adds only the roundings.

Every function takes the rounding as ``rnd`` (default: round to nearest
bfloat16, ties to even).  ``dithered(rng)`` returns a rounding with the
same error law at a random position inside the bf16 grid: x -> RNE(c x) / c
with c = 2^u, u ~ U[0, 1) drawn per element.  Two implementations that
round at the same points but not at the same values (another accumulation
order, another softmax scale) draw their rounding errors like two such
samples; the spread of the largest error over many samples is what the
GPU tests allow between the GPU and this emulation.
"""
from __future__ import annotations

import numpy as np

from oracle import block as ob

r16 = ob.round_bf16


def dithered(rng):
    """A bf16 rounding at a random position of the grid (see the module
    docstring); rng is a numpy Generator."""
    def rnd(x):
        x = np.asarray(x, np.float64)
        c = np.exp2(rng.random(x.shape))
        return r16(x * c) / c
    return rnd


def attention_sublayer_bf16(x, a, key_mask, W, cfg, rows=None, rnd=r16):
    S = x.shape[0]
    rows = np.arange(S) if rows is None else np.asarray(rows)
    kmax = int(rows.max()) + 1
    pos = np.arange(kmax)
    q, k, v = ob.qkv_heads(a[:kmax], W, cfg, pos)
    q, k, v = rnd(q[:, rows]), rnd(k), rnd(v)
    nh, nkv, hd = cfg["nh"], cfg["nkv"], cfg["hd"]
    g = nh // nkv
    vis = ob.visibility(rows, pos, None if key_mask is None else key_mask[:kmax],
                        cfg["window"])
    R = len(rows)
    out = np.zeros((R, nh, hd))
    for h in range(nh):
        s = np.where(vis, q[h] @ k[h // g].T / np.sqrt(hd), -np.inf)
        m = np.max(s, -1, keepdims=True)
        m = np.where(np.isfinite(m), m, 0.0)
        p = np.exp(s - m)
        l = p.sum(-1, keepdims=True)
        out[:, h] = np.where(l > 0, (rnd(p) @ v[h // g]) / np.where(l > 0, l, 1), 0)
    G = cfg["head_gate"]
    premix = out.reshape(R, nh * hd)
    if G:
        gl = ob.sigmoid(ob.linear(a[rows], W["w_head_gate"]))
        premix = (out * gl[:, :, None]).reshape(R, -1) if G == nh else premix * gl
    o = ob.linear(rnd(premix), W["wo"])
    att = ob.rms_norm(o, W["w_post_attn_norm"], cfg["eps"]) if cfg["sandwich"] else o
    return {"attention_output": att, "layer_mid": np.asarray(x)[rows] + att}


def mlp_sublayer_bf16(mid, m, W, cfg, router_logits=None, rnd=r16):
    """The MLP from its bf16 operand m (rounded to nearest here if it is not
    one already: a GPU tap passes through unchanged)."""
    kind = cfg["mlp"]
    m = r16(m)
    if kind == "swiglu":
        n = rnd(ob.silu(ob.linear(m, W["w_gate"])) * ob.linear(m, W["w_up"]))
        raw = ob.linear(n, W["w_down"])
    elif kind == "relu2":
        raw = ob.linear(rnd(ob.relu2(ob.linear(m, W["w_up"]))), W["w_down"])
    elif kind == "xielu":
        n = ob.xielu(ob.linear(m, W["w_up"]), W["xielu_alpha_p"], W["xielu_alpha_n"],
                     cfg["xielu_beta"], cfg["xielu_eps"])
        raw = ob.linear(rnd(n), W["w_down"])
    else:
        if router_logits is None:
            router_logits = ob.linear(m, W["w_router"])
        _, idx, w = ob.route(router_logits, W["expert_bias"], cfg["top_k"],
                             cfg["route_scale"], cfg["dtype"])
        raw = np.zeros_like(mid)
        for e in np.unique(idx):
            rows, slots = np.nonzero(idx == e)
            n = rnd(ob.silu(ob.linear(m[rows], W["w_e_gate"][e])) *
                    ob.linear(m[rows], W["w_e_up"][e]))
            y = rnd(w[rows, slots][:, None] * ob.linear(n, W["w_e_down"][e]))
            np.add.at(raw, rows, y)
        if cfg["n_shared"]:
            n = rnd(ob.silu(ob.linear(m, W["w_sh_gate"])) * ob.linear(m, W["w_sh_up"]))
            raw = raw + ob.linear(n, W["w_sh_down"])
    mo = ob.rms_norm(raw, W["w_post_mlp_norm"], cfg["eps"]) if cfg["sandwich"] else raw
    out = {"mlp_output": mo, "layer_output": np.asarray(mid) + mo}
    if kind == "moe":
        out["expert_indices"] = idx
    return out


def block_bf16(x, key_mask, W, cfg, rows=None, rnd=r16):
    x = np.asarray(x, np.float64)
    S = x.shape[0]
    rows = np.arange(S) if rows is None else np.asarray(rows)
    kmax = int(rows.max()) + 1
    a = rnd(ob.rms_norm(x[:kmax], W["w_in_norm"], cfg["eps"]))
    att = attention_sublayer_bf16(x[:kmax], a, key_mask, W, cfg, rows, rnd)
    mid = att["layer_mid"]
    m = rnd(ob.mlp_norm(mid, W, cfg))
    out = mlp_sublayer_bf16(mid, m, W, cfg, rnd=rnd)
    out.update(att)
    return out
