"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test names the passage it rests on.  None of them re-types the oracle's
own formula: they check printed values, identities the pages print,
invariants, special cases and a separate brute-force statement.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import block as ob
from oracle import brute
from transformer_decoder_block_amd import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def tiny(mlp="swiglu", **kw):
    base = dict(name="tiny", dtype="f32", B=2, S=7, H=16, nh=4, nkv=2, hd=4,
                mlp=mlp, I=12, seed=99)
    if mlp == "moe":
        base.update(E=5, top_k=2, I_e=6, n_shared=1, route_scale=2.826)
    base.update(kw)
    return synth.Workload(**base)


def inputs(w):
    W = synth.weights_f64(w, synth.make_weights(w))
    x = synth.to_f64(synth.make_x(w), w.dtype)
    mask = synth.make_mask(w)
    return x, mask, W


def fwd(w, x, mask, W, b=0, rows=None):
    return ob.block_forward(x[b], None if mask is None else mask[b], W,
                            w.as_dict(), rows)


def to_lists(W):
    return {k: (v.tolist() if isinstance(v, np.ndarray) else v)
            for k, v in W.items()}


# ---------------------------------------------------------------- brute force

BRUTE_CASES = [
    tiny("swiglu"),
    tiny("relu2", pad=3),
    tiny("xielu", qk_norm=True),
    tiny("moe", qk_norm=True, sandwich=True, window=3, head_gate=4),
    tiny("moe", qk_norm=True, sandwich=True, window=0, head_gate=16,
         use_rope=False, dtype="bf16"),
    tiny("swiglu", sandwich=True, qk_norm=True, head_gate=4, use_rope=False),
    tiny("swiglu", nh=4, nkv=1, hd=4, window=2, pad=2),
]


@pytest.mark.parametrize("w", BRUTE_CASES, ids=lambda w: f"{w.mlp}-{w.dtype}")
def test_forward_matches_brute_force(w):
    """The vectorised oracle and the scalar-loop statement agree to ~1e-12
    on every family and feature flag (a transposed operand, a wrong head
    map or a dropped term in either would show here)."""
    x, mask, W = inputs(w)
    WL = to_lists(W)
    for b in range(w.B):
        r = fwd(w, x, mask, W, b)
        rb = brute.block(x[b].tolist(), None if mask is None else
                         mask[b].tolist(), WL, w.as_dict())
        for key in ("layer_output", "layer_mid", "mlp_input",
                    "attention_norm_output"):
            got = np.asarray(rb[key])
            ref = r[key]
            assert np.max(np.abs(got - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref))), key
        ho = np.asarray(rb["attention_head_outputs"])
        assert np.max(np.abs(ho - r["attention_head_outputs"])) <= 1e-12


def test_rows_subset_matches_full():
    """Evaluating at a subset of query rows equals the full evaluation there."""
    w = tiny("moe", qk_norm=True, sandwich=True, window=3, head_gate=4, S=9)
    x, mask, W = inputs(w)
    full = fwd(w, x, mask, W)
    rows = np.array([0, 4, 5])
    part = fwd(w, x, mask, W, rows=rows)
    np.testing.assert_allclose(part["layer_output"], full["layer_output"][rows],
                               rtol=0, atol=1e-13)


# ------------------------------------------------------------- residual ids

@pytest.mark.parametrize("w", [tiny("swiglu"), tiny("relu2"),
                               tiny("xielu", qk_norm=True),
                               tiny("moe", sandwich=True, head_gate=4, qk_norm=True)],
                         ids=lambda w: w.mlp)
def test_residual_identity(w):
    """layer_input + attention_output + mlp_output == layer_output (the
    identity stated in section 01 of the arcee, afmoe and apertus pages;
    exact in float32 there, so exact in float64 here)."""
    x, mask, W = inputs(w)
    r = fwd(w, x, mask, W)
    lhs = r["layer_input"] + r["attention_output"] + r["mlp_output"]
    assert np.array_equal(lhs, r["layer_output"])


def test_routed_plus_shared_is_mlp_output():
    """afmoe notes, section 03: the routed and shared outputs add up to the
    MLP's output."""
    w = tiny("moe", sandwich=True, head_gate=4, qk_norm=True)
    x, mask, W = inputs(w)
    r = fwd(w, x, mask, W)
    assert np.array_equal(r["routed_output"] + r["shared_expert_output"],
                          r["mlp_raw"])
    # and the post-MLP norm's output is what the block adds
    np.testing.assert_allclose(
        r["mlp_output"], ob.rms_norm(r["mlp_raw"], W["w_post_mlp_norm"], w.eps),
        rtol=0, atol=0)


# ------------------------------------------------------------------ RMSNorm

def test_rmsnorm_scale_invariant_up_to_eps():
    """afmoe notes, section 03: scaling the norm's input does not change its
    output, up to eps."""
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 64))
    g = rng.standard_normal(64)
    for lam in (3.0, 1e3):
        a = ob.rms_norm(x, g, 0.0)
        b = ob.rms_norm(lam * x, g, 0.0)
        np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-13)
    # with eps > 0 the invariance is broken by an amount that shrinks with scale
    d_small = np.max(np.abs(ob.rms_norm(1e-3 * x, g, 1e-5) - ob.rms_norm(x, g, 0.0)))
    d_big = np.max(np.abs(ob.rms_norm(1e3 * x, g, 1e-5) - ob.rms_norm(x, g, 0.0)))
    assert d_small > 1e-3 and d_big < 1e-10


def test_rmsnorm_unit_rms_and_gain_per_channel():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((4, 32)) * 7
    y = ob.rms_norm(x, np.ones(32), 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, -1)), 1.0, rtol=1e-14)
    g = rng.standard_normal(32)
    np.testing.assert_allclose(ob.rms_norm(x, g, 0.0), y * g, rtol=1e-14)


# -------------------------------------------------------------------- RoPE

def test_rope_identity_at_position_zero():
    """apertus notes: at position 0 the rotation is the identity."""
    rng = np.random.default_rng(2)
    u = rng.standard_normal((3, 1, 64))
    cos, sin = ob.rope_cos_sin(np.array([0]), 64, 10000.0)
    assert np.array_equal(ob.rope(u, cos, sin), u)


def test_rope_is_a_rotation_and_relative():
    rng = np.random.default_rng(3)
    hd = 16
    q = rng.standard_normal(hd)
    k = rng.standard_normal(hd)

    def rot(u, p):
        c, s = ob.rope_cos_sin(np.array([p]), hd, 10000.0)
        return ob.rope(u[None, :], c, s)[0]

    # norm preserved
    assert abs(np.linalg.norm(rot(q, 37)) - np.linalg.norm(q)) < 1e-12
    # the score depends on the positions only through their difference
    s1 = rot(q, 10) @ rot(k, 3)
    s2 = rot(q, 107) @ rot(k, 100)
    assert abs(s1 - s2) < 1e-11
    assert abs(s1 - rot(q, 7) @ k) < 1e-11
    # and it does depend on the difference
    assert abs(s1 - rot(q, 11) @ rot(k, 3)) > 1e-3


# --------------------------------------------------------------- attention

def _attn_case(S=9, nh=4, nkv=2, hd=8, seed=4):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((nh, S, hd))
    k = rng.standard_normal((nkv, S, hd))
    v = rng.standard_normal((nkv, S, hd))
    return q, k, v


def test_softmax_rows_sum_to_one():
    q, k, v = _attn_case()
    pos = np.arange(9)
    mask = np.array([1, 1, 1, 1, 1, 1, 0, 0, 1])
    _, sc, p = ob.attention(q, k, v, pos, pos, mask, 4)
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=0, atol=1e-14)
    assert np.all(p[np.isneginf(sc)] == 0)
    assert np.all(p[~np.isneginf(sc)] > 0)


def test_attention_single_token_returns_v_and_zero_query_averages():
    q, k, v = _attn_case(S=1)
    out, _, _ = ob.attention(q, k, v, np.arange(1), np.arange(1), None, 0)
    for h in range(4):
        np.testing.assert_allclose(out[0, h], v[h // 2, 0], rtol=0, atol=1e-15)
    q, k, v = _attn_case()
    q[:] = 0
    pos = np.arange(9)
    out, _, _ = ob.attention(q, k, v, pos, pos, None, 3)
    for i in range(9):
        lo = max(0, i - 3 + 1)
        np.testing.assert_allclose(out[i, 1], v[0, lo:i + 1].mean(0), atol=1e-14)
        np.testing.assert_allclose(out[i, 3], v[1, lo:i + 1].mean(0), atol=1e-14)


def test_fully_masked_row_is_zero():
    q, k, v = _attn_case()
    pos = np.arange(9)
    mask = np.zeros(9, int)
    mask[5:] = 1
    out, _, p = ob.attention(q, k, v, pos, pos, mask, 0)
    assert np.all(out[:5] == 0) and np.all(p[:, :5] == 0)
    assert np.all(np.abs(out[5:]) > 0)


@pytest.mark.parametrize("w", [tiny("swiglu", S=10), tiny("moe", S=10, window=4,
                                sandwich=True, qk_norm=True, head_gate=4)],
                         ids=["llama", "afmoe"])
def test_causality(w):
    """Perturbing tokens t >= t0 leaves every earlier output bitwise unchanged
    (the llama sheet's causal mask)."""
    x, mask, W = inputs(w)
    r0 = fwd(w, x, mask, W)
    x2 = x.copy()
    x2[0, 6:] += np.random.default_rng(5).standard_normal(x2[0, 6:].shape)
    r1 = fwd(w, x2, mask, W)
    assert np.array_equal(r0["layer_output"][:6], r1["layer_output"][:6])
    assert not np.allclose(r0["layer_output"][6:], r1["layer_output"][6:])


def test_window_edge():
    """With window W, query i reads keys i-W+1..i: perturbing key i-W leaves
    row i unchanged, perturbing key i-W+1 changes it."""
    w = tiny("swiglu", S=12, window=4)
    x, mask, W = inputs(w)
    r0 = fwd(w, x, mask, W)
    i = 10
    for j, changes in ((i - 4, False), (i - 3, True)):
        x2 = x.copy()
        x2[0, j] *= -1.5
        r1 = fwd(w, x2, mask, W)
        same = np.array_equal(r0["layer_output"][i], r1["layer_output"][i])
        assert same != changes, (j, changes)


def test_padding_invariance():
    """Padded keys (attention_mask 0) do not reach any row: changing the
    padded tokens leaves every other row bitwise unchanged."""
    w = tiny("relu2", S=10, pad=4)
    x, mask, W = inputs(w)
    b = w.B - 1
    assert mask[b, -4:].sum() == 0
    r0 = fwd(w, x, mask, W, b)
    x2 = x.copy()
    x2[b, -4:] = 3.0
    r1 = fwd(w, x2, mask, W, b)
    assert np.array_equal(r0["layer_output"][:6], r1["layer_output"][:6])


def test_gqa_head_map():
    """arcee notes: an edit to key/value head j reaches query heads g*j ..
    g*j+g-1 and no others."""
    w = tiny("swiglu", nh=6, nkv=2, hd=4, H=24)
    x, mask, W = inputs(w)
    r0 = fwd(w, x, mask, W)
    W2 = dict(W)
    W2["wv"] = W["wv"].copy()
    j = 1
    W2["wv"][j * 4:(j + 1) * 4] *= 2.0
    r1 = fwd(w, x, mask, W2)
    d = np.abs(r0["attention_head_outputs"] - r1["attention_head_outputs"]).max(axis=(0, 2))
    assert np.all(d[:3] == 0) and np.all(d[3:] > 0)


def test_qk_norm_renormalises_head_scale():
    """apertus notes: scaling one head's slice of q_proj's output is
    renormalised away by the per-head q norm."""
    w = tiny("xielu", qk_norm=True)
    x, mask, W = inputs(w)
    W = dict(W)
    W["wq"] = W["wq"] * 30.0      # make the attention pattern non-uniform
    W["wk"] = W["wk"] * 30.0
    r0 = fwd(w, x, mask, W)
    W2 = dict(W)
    W2["wq"] = W["wq"].copy()
    W2["wq"][4:8] *= 2.0
    r1 = fwd(w, x, mask, W2)
    assert np.max(np.abs(r0["layer_output"] - r1["layer_output"])) < 1e-5
    # without the norm the same edit is visible
    W3 = dict(W2)
    r2 = ob.block_forward(x[0], None, W3, dict(w.as_dict(), qk_norm=False))
    r3 = ob.block_forward(x[0], None, W, dict(w.as_dict(), qk_norm=False))
    assert np.max(np.abs(r2["layer_output"] - r3["layer_output"])) > 1e-3


def test_head_gate():
    """afmoe notes: o_proj's input is the ungated heads times sigmoid(gate);
    a zero gate projection halves every head."""
    w = tiny("moe", sandwich=True, qk_norm=True, head_gate=4)
    x, mask, W = inputs(w)
    W0 = dict(W)
    W0["w_head_gate"] = np.zeros_like(W["w_head_gate"])
    r = fwd(w, x, mask, W0)
    np.testing.assert_allclose(r["attention_premix"],
                               0.5 * r["attention_head_outputs"].reshape(7, -1),
                               rtol=0, atol=0)
    # per-channel gate: the gate column h*hd+d scales channel d of head h only
    w2 = w.replace(head_gate=16)
    W2 = synth.weights_f64(w2, synth.make_weights(w2))
    r2 = fwd(w2, x, mask, W2)
    a = r2["attention_norm_output"]
    gl = 1 / (1 + np.exp(-(a @ W2["w_head_gate"].T)))
    np.testing.assert_allclose(r2["attention_premix"],
                               r2["attention_head_outputs"].reshape(7, -1) * gl,
                               rtol=1e-15, atol=0)


def test_global_block_queries_are_q_norm_output():
    """afmoe notes: on a full block (no rotary) attention_queries is
    q_norm's output unchanged, so scores equal q_norm(q).k_norm(k)/sqrt(hd)."""
    w = tiny("swiglu", sandwich=True, qk_norm=True, head_gate=4, use_rope=False)
    x, mask, W = inputs(w)
    r = fwd(w, x, mask, W)
    a = r["attention_norm_output"]
    qn = ob.rms_norm((a @ W["wq"].T).reshape(7, 4, 4), W["w_q_norm"], w.eps)
    kn = ob.rms_norm((a @ W["wk"].T).reshape(7, 2, 4), W["w_k_norm"], w.eps)
    s = qn[:, 1] @ kn[:, 0].T / 2.0
    vis = np.tril(np.ones((7, 7), bool))
    np.testing.assert_allclose(r["attention_scores"][1][vis], s[vis], atol=1e-14)


# -------------------------------------------------------------- activations

def test_relu2_exact_zeros():
    """arcee notes, section 03: the activations equal the squared ReLU of the
    up projection exactly, so every negative pre-activation gives 0."""
    w = tiny("relu2")
    x, mask, W = inputs(w)
    r = fwd(w, x, mask, W)
    pre = r["mlp_input"] @ W["w_up"].T
    acts = r["mlp_neurons"]
    assert np.array_equal(acts == 0, pre <= 0)
    assert np.array_equal(acts, np.where(pre > 0, pre, 0.0) ** 2)


def test_xielu_printed_values():
    """apertus notes, section 03 (the xIELU negative branch): block
    8 prints -0.107 at -1, 1.78 at -5, 10.3 at -20 and a minimum of -0.14
    near -0.63.  One effective alpha_n (solved from the value at -20) must
    reproduce all of them through the raw (pre-softplus) parameterisation."""
    g = json.load(open(os.path.join(GOLD, "xielu_apertus_block8.json")))
    beta = g["beta"]
    # f(-20) = an*(expm1(-20)+20) - 10  =>  an
    an = (10.3 + 10.0) / (math.expm1(-20.0) + 20.0)
    raw_n = math.log(math.expm1(an - beta))     # inverse of beta+softplus
    for p in g["printed"]:
        y = float(ob.xielu(p["x"], 0.0, raw_n, beta, -1e-6))
        assert round(y, p["digits"]) == pytest.approx(p["y"], abs=1e-9), p
    xs = np.linspace(-3, 0, 300001)
    ys = ob.xielu(xs, 0.0, raw_n, beta, -1e-6)
    i = int(np.argmin(ys))
    mn = g["printed_minimum"]
    assert round(float(ys[i]), mn["y_digits"]) == pytest.approx(mn["y"])
    assert round(float(xs[i]), mn["x_digits"]) == pytest.approx(mn["x"])
    # the negative branch grows like (alpha_n - beta)|x|
    big = float(ob.xielu(-1e4, 0.0, raw_n, beta, -1e-6))
    assert big / 1e4 == pytest.approx(an - beta, rel=1e-3)


def test_xielu_positive_branch_and_continuity():
    ap_raw = 0.7
    ap = math.log1p(math.exp(ap_raw))
    for z in (1e-3, 0.5, 3.0):
        assert float(ob.xielu(z, ap_raw, 0.6, 0.5, -1e-6)) == pytest.approx(
            ap * z * z + 0.5 * z, rel=1e-14)
    # near zero both branches tend to 0
    assert abs(float(ob.xielu(1e-9, 0.9, 0.9))) < 1e-8
    assert abs(float(ob.xielu(-1e-9, 0.9, 0.9))) < 1e-5


# ------------------------------------------------------------------- router

def test_router_weights_sum_to_route_scale_and_page_identity():
    """afmoe notes: w == chosen / chosen.sum() * route_scale, summing to
    route_scale at every token (2.826 on Nano/Mini, 2.448 on Large)."""
    g = json.load(open(os.path.join(GOLD, "afmoe_router.json")))
    rng = np.random.default_rng(6)
    for c in g["cases"]:
        E, k, rs = c["num_experts"], c["top_k"], c["route_scale"]
        logits = rng.standard_normal((50, E))
        bias = rng.standard_normal(E).astype(np.float32) * 0.1
        l, idx, w = ob.route(logits, bias, k, rs, "bf16")
        np.testing.assert_allclose(w.sum(-1), rs, rtol=1e-14)
        chosen = (1 / (1 + np.exp(-l)))[np.arange(50)[:, None], idx]
        np.testing.assert_allclose(w, chosen / chosen.sum(-1, keepdims=True) * rs,
                                   rtol=1e-14)
        assert np.all([len(set(r)) == k for r in idx.tolist()])


def test_router_bias_moves_only_the_choice():
    """afmoe notes: a written expert_bias moves only the choice."""
    rng = np.random.default_rng(7)
    logits = rng.standard_normal((40, 16))
    bias = np.zeros(16, np.float32)
    _, idx0, w0 = ob.route(logits, bias, 4, 2.826, "f32")
    # force expert 5 in everywhere with a large bias
    b2 = bias.copy()
    b2[5] = 10.0
    l, idx1, w1 = ob.route(logits, b2, 4, 2.826, "f32")
    assert np.all(idx1[:, 0] == 5)
    s = 1 / (1 + np.exp(-l))
    ch = s[np.arange(40)[:, None], idx1]
    np.testing.assert_allclose(w1, ch / ch.sum(-1, keepdims=True) * 2.826, rtol=1e-14)
    # a bias that keeps the same choice keeps the same weights
    b3 = np.full(16, 0.25, np.float32)
    _, idx3, w3 = ob.route(logits, b3, 4, 2.826, "f32")
    assert np.array_equal(idx3, idx0) and np.array_equal(w3, w0)


def test_router_topk_brute_force_and_ties():
    rng = np.random.default_rng(8)
    logits = rng.integers(-3, 3, (60, 12)).astype(float) * 0.5  # many ties
    bias = np.zeros(12, np.float32)
    _, idx, _ = ob.route(logits, bias, 5, 1.0, "f32")
    for t in range(60):
        c = np.float32(1 / (1 + np.exp(-logits[t])))
        chosen = []
        for _ in range(5):
            best = max((e for e in range(12) if e not in chosen),
                       key=lambda e: (c[e], -e))
            chosen.append(best)
        assert chosen == idx[t].tolist()


def test_router_logits_rounded_to_model_dtype():
    """afmoe notes: router_logits are in the model's dtype.  The oracle's
    bf16 rounding agrees with torch's float32 -> bfloat16 cast (nearest,
    ties to even) on float32-representable inputs, including exact ties."""
    rng = np.random.default_rng(9)
    v = rng.standard_normal(20000).astype(np.float32) * 5
    ties = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 3 * 2 ** -9],
                    np.float32)
    v = np.concatenate([v, ties])
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ob.round_bf16(v.astype(np.float64)), ref)


def test_moe_single_expert_reduces_to_dense_swiglu():
    """E = 1, k = 1, route_scale = 1 and a zero shared expert: the mixture is
    the dense SwiGLU MLP of that expert's weights."""
    w = tiny("moe", E=1, top_k=1, route_scale=1.0)
    x, mask, W = inputs(w)
    W = dict(W)
    W["w_sh_down"] = np.zeros_like(W["w_sh_down"])
    m = np.random.default_rng(10).standard_normal((9, w.H))
    r = ob.mlp_forward(m, W, dict(w.as_dict(), dtype="f32"))
    y, _ = ob.swiglu_mlp(m, W["w_e_gate"][0], W["w_e_up"][0], W["w_e_down"][0])
    np.testing.assert_allclose(r["mlp_raw"], y, rtol=1e-14, atol=1e-15)


def test_expert_ablation_locality():
    """afmoe notes, 'Ablating an expert': routed_output changes on exactly
    the tokens that chose the expert."""
    w = tiny("moe", E=6, top_k=2, S=12)
    x, mask, W = inputs(w)
    m = np.random.default_rng(11).standard_normal((40, w.H))
    W = dict(W)
    W["w_router"] = W["w_router"] * 50.0   # let the choice vary by token
    cfg = w.as_dict()
    r0 = ob.mlp_forward(m, W, cfg)
    e = int(r0["expert_indices"][0, 0])
    W2 = dict(W)
    W2["w_e_down"] = W["w_e_down"].copy()
    W2["w_e_down"][e] = 0
    r1 = ob.mlp_forward(m, W2, cfg)
    chose = np.any(r0["expert_indices"] == e, axis=1)
    changed = np.any(r0["routed_output"] != r1["routed_output"], axis=1)
    assert np.array_equal(chose, changed) and chose.any() and not chose.all()
