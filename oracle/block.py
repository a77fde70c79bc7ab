"""fp64 CPU oracle of one Llama-family decoder block (forward pass).

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product
path (libblock and its Python binding) never imports, links or runs it, and
this module imports nothing from the product path.

Every function works in float64 NumPy on the exact fp64 images of the stored
inputs.  The block is a finite composition of plain definitions (norms,
matrix products, rotations, a softmax, pointwise activations, a top-k), so
the oracle is those definitions written out, one function per step, with no
blocking, fusion or reordering beyond what a step's own definition states.
The one rounding it performs is the router's cast of its logits to the
model's dtype, because the afmoe page states that the choice of experts is
made from those rounded logits.

Sources (the pages these functions follow):
  [llama]   safebydesign granite sheet "LlamaForCausalLM 32L-4096d",
            section "Implementing it" (the block as pseudo-code).
  [arcee]   nnterp encyclopedia, arcee page, section 03 "The Notes".
  [afmoe]   nnterp encyclopedia, afmoe page, section 03 "The Notes".
  [apertus] nnterp encyclopedia, apertus page, section 03 "The Notes".
  [support] the section 02 "support()" tables of the three nnterp pages,
            which name each value and its layout.

Readings taken where the pages are silent (each one is listed with its
reason in the design notes):
  * RMSNorm is g * x / sqrt(mean(x^2) + eps) (eps inside the root, the gain
    multiplies).
  * RoPE is the rotate-half form: pairs (i, i + hd/2), angle s * theta^(-2i/hd),
    positions 0..S-1 of each sequence.
  * attention_mask masks keys only; a query row whose every key is masked
    yields probabilities 0 and output 0.
  * sliding window W: key j is visible to query i iff i - W < j <= i.
  * top-k ties go to the lower expert index; slots are in descending biased
    score.
  * the per-head sigmoid gate (G = num_heads columns) scales every channel of
    its head; the per-channel gate (G = num_heads * head_dim) scales one
    channel each.

Parity unpinned (no number on the pages fixes them; the tests pin every
other property of these steps): the rotate-half pairing of ``rope`` as
against an interleaved one, and which of the two head-gate widths the real
afmoe model uses.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


# --------------------------------------------------------------------------
# elementary steps
# --------------------------------------------------------------------------

def rms_norm(x, g, eps):
    """RMSNorm over the last axis: g * x / sqrt(mean(x^2) + eps).

    [llama] applies the layer's input norm with eps 1e-5 but prints no
    formula; [afmoe] section 03 remarks that the norm ignores the scale of
    its input (up to eps).  This is the reading stated in the module
    docstring.
    """
    x = np.asarray(x, F64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return np.asarray(g, F64) * (x / np.sqrt(ms + eps))


def linear(x, w):
    """A bias-free Linear: x @ w.T with w in [out_features, in_features].

    [llama] multiplies the stream by the transposed projection matrices;
    the module printouts of the nnterp pages list every projection without
    a bias.
    """
    return np.asarray(x, F64) @ np.asarray(w, F64).T


def rope_cos_sin(positions, hd, theta):
    """Angles of the plain rotary embedding: phi[s, i] = s * theta^(-2i/hd).

    [llama] rotates q and k with base 10000 after the projections.  Returns
    cos, sin of shape [len(positions), hd/2].
    """
    i = np.arange(hd // 2, dtype=F64)
    inv_freq = theta ** (-2.0 * i / hd)
    phi = np.asarray(positions, F64)[:, None] * inv_freq[None, :]
    return np.cos(phi), np.sin(phi)


def rope(u, cos, sin):
    """Rotate-half RoPE on u[..., S, hd] with per-position cos/sin [S, hd/2].

    (u_i, u_{i+hd/2}) -> (u_i cos - u_{i+hd/2} sin, u_{i+hd/2} cos + u_i sin).
    """
    u = np.asarray(u, F64)
    half = u.shape[-1] // 2
    lo, hi = u[..., :half], u[..., half:]
    return np.concatenate([lo * cos - hi * sin, hi * cos + lo * sin], axis=-1)


def visibility(q_pos, k_pos, key_mask, window):
    """Boolean [len(q_pos), len(k_pos)]: may query q_pos[a] read key k_pos[b]?

    Causal ([llama] masks the softmax causally), restricted to real keys
    (the [support] tables mark padding with zeros in attention_mask) and,
    when window > 0, to the ``window`` most recent positions, the query's
    own included ([afmoe] section 03 on the sliding-window blocks).
    """
    qp = np.asarray(q_pos)[:, None]
    kp = np.asarray(k_pos)[None, :]
    vis = kp <= qp
    if key_mask is not None:
        vis = vis & (np.asarray(key_mask)[None, :] != 0)
    if window and window > 0:
        vis = vis & (qp - kp < window)
    return vis


def softmax_rows(scores):
    """Row softmax over the last axis; -inf entries get probability 0.

    A row that is -inf everywhere returns all zeros (reading: nothing is
    visible, so nothing is mixed in).
    """
    s = np.asarray(scores, F64)
    m = np.max(s, axis=-1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m)
    z = np.sum(e, axis=-1, keepdims=True)
    return np.where(z > 0, e / np.where(z > 0, z, 1.0), 0.0)


def attention(q, k, v, q_pos, k_pos, key_mask, window):
    """Grouped-query softmax attention for one sequence.

    q [nh, Sq, hd], k [nkv, Sk, hd], v [nkv, Sk, hd].  Query head h reads
    KV head h // (nh // nkv), the grouping the [arcee] and [apertus] notes
    describe (each KV head serves a run of consecutive query heads).
    [llama]: scores are q.k scaled by 1/sqrt(head_dim), masked causally,
    softmaxed over keys, and the probabilities weight the values.

    Returns (head_out [Sq, nh, hd], scores [nh, Sq, Sk] masked with -inf,
    probs [nh, Sq, Sk]).
    """
    nh, _, hd = q.shape
    nkv = k.shape[0]
    g = nh // nkv
    vis = visibility(q_pos, k_pos, key_mask, window)
    scores = np.empty((nh, q.shape[1], k.shape[1]), F64)
    for h in range(nh):
        raw = q[h] @ k[h // g].T / np.sqrt(F64(hd))
        scores[h] = np.where(vis, raw, -np.inf)
    probs = softmax_rows(scores)
    out = np.empty((q.shape[1], nh, hd), F64)
    for h in range(nh):
        out[:, h, :] = probs[h] @ v[h // g]
    return out, scores, probs


def silu(z):
    """silu(z) = z / (1 + e^-z), the gate activation of [llama]'s MLP."""
    z = np.asarray(z, F64)
    return z / (1.0 + np.exp(-z))


def sigmoid(z):
    z = np.asarray(z, F64)
    return 1.0 / (1.0 + np.exp(-z))


def relu2(z):
    """Squared ReLU of the [arcee] MLP: max(z, 0)^2, exactly zero below zero."""
    z = np.asarray(z, F64)
    r = np.maximum(z, 0.0)
    return r * r


def softplus(z):
    z = np.asarray(z, F64)
    return np.log1p(np.exp(-np.abs(z))) + np.maximum(z, 0.0)


def xielu(z, alpha_p_raw, alpha_n_raw, beta=0.5, eps=-1e-6):
    """xIELU, the activation of the ungated [apertus] MLP (section 03).

    alpha_p = softplus(raw_p), alpha_n = beta + softplus(raw_n);
    z > 0 : alpha_p z^2 + beta z;
    z <= 0: alpha_n (expm1(min(z, eps)) - z) + beta z.
    """
    z = np.asarray(z, F64)
    ap = softplus(alpha_p_raw)
    an = beta + softplus(alpha_n_raw)
    pos = ap * z * z + beta * z
    neg = an * (np.expm1(np.minimum(z, eps)) - z) + beta * z
    return np.where(z > 0, pos, neg)


def round_bf16(x):
    """Round float64 values to the nearest bfloat16 (ties to even).

    bfloat16 keeps 8 significant bits: with x = m * 2^e and m in [0.5, 1),
    the result is rint(m * 2^8) * 2^(e-8); np.rint rounds half to even.
    """
    x = np.asarray(x, F64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def round_f32(x):
    return np.asarray(x, F64).astype(np.float32).astype(F64)


# --------------------------------------------------------------------------
# MLPs
# --------------------------------------------------------------------------

def swiglu_mlp(m, w_gate, w_up, w_down):
    """[llama] gated MLP: down( silu(gate(m)) * up(m) )."""
    n = silu(linear(m, w_gate)) * linear(m, w_up)
    return linear(n, w_down), n


def relu2_mlp(m, w_up, w_down):
    """[arcee] ungated MLP: down( relu(up(m))^2 )."""
    n = relu2(linear(m, w_up))
    return linear(n, w_down), n


def xielu_mlp(m, w_up, w_down, alpha_p_raw, alpha_n_raw, beta, eps):
    """[apertus] ungated MLP: down( xielu(up(m)) )."""
    n = xielu(linear(m, w_up), alpha_p_raw, alpha_n_raw, beta, eps)
    return linear(n, w_down), n


def route(logits, bias, top_k, route_scale, model_dtype):
    """The sigmoid router of the [afmoe] notes (section 03, on the router).

    logits: router.gate's output.  The page states the logits are in the
    model's dtype and are cast to float32 before the sigmoid and the bias
    add, so the choice is taken in float32: s32 = fp32(sigmoid(l)),
    c = fp32(s32 + bias), top_k of c in descending order (ties: lower
    expert index first).  The weights are the chosen unbiased sigmoids,
    renormalised to sum to one and multiplied by route_scale.

    Returns (rounded logits [T, E], indices [T, k] int64, weights [T, k]).
    """
    l = np.asarray(logits, F64)
    if model_dtype == "bf16":
        l = round_bf16(l)
    s = sigmoid(l)
    s32 = s.astype(np.float32)
    c32 = (s32 + np.asarray(bias, np.float32)).astype(np.float32)
    E = l.shape[-1]
    # descending by value, ascending by index on ties: stable sort of -c
    order = np.argsort(-c32.astype(F64), axis=-1, kind="stable")
    idx = order[:, :top_k]
    chosen = np.take_along_axis(s, idx, axis=-1)
    w = chosen / np.sum(chosen, axis=-1, keepdims=True) * route_scale
    assert idx.max(initial=0) < E
    return l, idx, w


def moe_mlp(m, W, cfg, logits=None):
    """Sigmoid-routed mixture plus shared expert ([afmoe] notes).

    routed = sum over slots of w_slot * E_{idx_slot}(m) with the SwiGLU
    expert E_e; shared = the shared SwiGLU expert on every token; the
    mixture returns routed + shared (the [afmoe] notes identify that sum
    with the MLP's output).  ``logits`` may be given to force the router's input
    (a tap of the implementation under test); otherwise the oracle computes
    them.
    """
    if logits is None:
        logits = linear(m, W["w_router"])
    l, idx, w = route(logits, W["expert_bias"], cfg["top_k"],
                      cfg["route_scale"], cfg["dtype"])
    T = m.shape[0]
    H = m.shape[1]
    expert_outputs = np.zeros((T, cfg["top_k"], H), F64)
    for e in np.unique(idx):
        rows, slots = np.nonzero(idx == e)
        y, _ = swiglu_mlp(m[rows], W["w_e_gate"][e], W["w_e_up"][e],
                          W["w_e_down"][e])
        expert_outputs[rows, slots, :] = w[rows, slots][:, None] * y
    routed = np.sum(expert_outputs, axis=1)
    shared, _ = swiglu_mlp(m, W["w_sh_gate"], W["w_sh_up"], W["w_sh_down"])
    return {
        "router_logits": l,
        "expert_indices": idx,
        "expert_weights": w,
        "expert_outputs": expert_outputs,
        "routed_output": routed,
        "shared_expert_output": shared,
        "mlp_raw": routed + shared,
    }


def mlp_forward(m, W, cfg, router_logits=None):
    """The block's MLP on the normed stream m [T, H] -> dict of values.

    ``mlp_raw`` is mlp.output (before any post-MLP norm).
    """
    kind = cfg["mlp"]
    if kind == "swiglu":
        y, n = swiglu_mlp(m, W["w_gate"], W["w_up"], W["w_down"])
        # [support] mlp_activation is act_fn's output: silu of the gate
        # projection on a gated MLP
        return {"mlp_raw": y, "mlp_neurons": n,
                "mlp_activation": silu(linear(m, W["w_gate"]))}
    if kind == "relu2":
        y, n = relu2_mlp(m, W["w_up"], W["w_down"])
        return {"mlp_raw": y, "mlp_neurons": n, "mlp_activation": n}
    if kind == "xielu":
        y, n = xielu_mlp(m, W["w_up"], W["w_down"], W["xielu_alpha_p"],
                         W["xielu_alpha_n"], cfg["xielu_beta"],
                         cfg["xielu_eps"])
        # ungated: the activation is what the down projection receives
        return {"mlp_raw": y, "mlp_neurons": n, "mlp_activation": n}
    if kind == "moe":
        return moe_mlp(m, W, cfg, router_logits)
    raise ValueError(kind)


# --------------------------------------------------------------------------
# the two sublayers
# --------------------------------------------------------------------------

def qkv_heads(a, W, cfg, positions):
    """Project a [n, H] to per-head q [nh, n, hd], k, v [nkv, n, hd].

    Optional per-head q/k RMSNorm ahead of the rotary ([apertus] section 03:
    each head's query and key are normalised, one gain vector shared by all
    heads), then RoPE unless the block is a full (global) afmoe block
    ([afmoe] section 03: only the sliding-window blocks rotate).
    """
    nh, nkv, hd = cfg["nh"], cfg["nkv"], cfg["hd"]
    n = a.shape[0]
    q = linear(a, W["wq"]).reshape(n, nh, hd).transpose(1, 0, 2)
    k = linear(a, W["wk"]).reshape(n, nkv, hd).transpose(1, 0, 2)
    v = linear(a, W["wv"]).reshape(n, nkv, hd).transpose(1, 0, 2)
    if cfg["qk_norm"]:
        q = rms_norm(q, W["w_q_norm"], cfg["eps"])
        k = rms_norm(k, W["w_k_norm"], cfg["eps"])
    if cfg["use_rope"]:
        cos, sin = rope_cos_sin(positions, hd, cfg["theta"])
        q = rope(q, cos, sin)
        k = rope(k, cos, sin)
    return q, k, v


def attention_sublayer(x, a, key_mask, W, cfg, rows=None):
    """Attention half of one sequence's block, evaluated at query ``rows``.

    x: layer_input [S, H]; a: attention_norm_output [S, H] (the normed
    stream the projections read); key_mask: attention_mask [S] or None.
    Only keys at positions <= max(rows) are projected (later keys are
    invisible to every requested row).

    Returns a dict of the [support] values at ``rows``: attention_queries
    [nh, R, hd], attention_keys and attention_values [nkv, K, hd] (K = the
    keys up to max(rows)), attention_scores [nh, R, K],
    attention_probabilities, attention_head_outputs [R, nh, hd],
    attention_premix, attention_output, layer_mid.
    """
    S = x.shape[0]
    rows = np.arange(S) if rows is None else np.asarray(rows)
    kmax = int(rows.max()) + 1
    k_pos = np.arange(kmax)
    _, k, v = qkv_heads(a[:kmax], W, cfg, k_pos)
    q, _, _ = qkv_heads(a[rows], W, cfg, rows)
    km = None if key_mask is None else np.asarray(key_mask)[:kmax]
    head_out, scores, probs = attention(q, k, v, rows, k_pos, km,
                                        cfg["window"])
    nh, hd = cfg["nh"], cfg["hd"]
    R = len(rows)
    premix = head_out.reshape(R, nh * hd)
    gate = cfg["head_gate"]
    if gate:
        # [afmoe] section 03: the heads' outputs are scaled by the sigmoid
        # of a gate projected from the attention's input, ahead of o_proj.
        gl = sigmoid(linear(a[rows], W["w_head_gate"]))
        if gate == nh:
            premix = (head_out * gl[:, :, None]).reshape(R, nh * hd)
        elif gate == nh * hd:
            premix = premix * gl
        else:
            raise ValueError("head gate width must be nh or nh*hd")
    o = linear(premix, W["wo"])
    if cfg["sandwich"]:
        # [afmoe] sandwich norm: the attention's output is normed before
        # it joins the residual stream
        attn_out = rms_norm(o, W["w_post_attn_norm"], cfg["eps"])
    else:
        attn_out = o
    mid = np.asarray(x, F64)[rows] + attn_out
    return {
        "attention_queries": q,
        "attention_keys": k,
        "attention_values": v,
        "attention_scores": scores,
        "attention_probabilities": probs,
        "attention_head_outputs": head_out,
        "attention_premix": premix,
        "attention_output": attn_out,
        "layer_mid": mid,
    }


def mlp_norm(mid, W, cfg):
    """The normed stream entering the MLP (mlp_input).

    Llama/arcee/apertus: post_attention_layernorm (feedforward_layernorm on
    apertus); afmoe: pre_mlp_layernorm.  Both weights arrive as w_mlp_norm.
    """
    return rms_norm(mid, W["w_mlp_norm"], cfg["eps"])


def mlp_sublayer(mid, m, W, cfg, router_logits=None):
    """MLP half at the given tokens: mid = layer_mid, m = mlp_input.

    Returns the MLP values plus mlp_output (what is added to the stream) and
    layer_output.
    """
    out = mlp_forward(m, W, cfg, router_logits)
    if cfg["sandwich"]:
        mlp_output = rms_norm(out["mlp_raw"], W["w_post_mlp_norm"], cfg["eps"])
    else:
        mlp_output = out["mlp_raw"]
    out["mlp_output"] = mlp_output
    out["layer_output"] = np.asarray(mid, F64) + mlp_output
    return out


def block_forward(x, key_mask, W, cfg, rows=None):
    """The whole block for one sequence x [S, H], evaluated at ``rows``.

    Returns every named value: layer_input, attention_norm_output (at rows),
    the attention values, layer_mid, mlp_input, the MLP values,
    layer_output.
    """
    x = np.asarray(x, F64)
    S = x.shape[0]
    rows = np.arange(S) if rows is None else np.asarray(rows)
    kmax = int(rows.max()) + 1
    a = rms_norm(x[:kmax], W["w_in_norm"], cfg["eps"])
    att = attention_sublayer(x[:kmax], a, key_mask, W, cfg, rows)
    mid = att["layer_mid"]
    m = mlp_norm(mid, W, cfg)
    mo = mlp_sublayer(mid, m, W, cfg)
    # [support] mlp_norm_output is the norm's output and mlp_input what the
    # MLP is called with: the same tensor in these blocks
    res = {"layer_input": x[rows], "attention_norm_output": a[rows],
           "mlp_input": m, "mlp_norm_output": m}
    res.update(att)
    res.update(mo)
    return res
