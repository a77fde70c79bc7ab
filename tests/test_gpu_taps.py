"""GPU parity of the interior taps: the per-head queries, keys and values,
the attention probabilities, the head outputs before and after the head
gate, the MLP's activation and neurons and the mixture's per-slot, routed and shared
outputs, each against the fp64 oracle through the C ABI.

Bars:
  * float32 workloads, end to end from layer_input: max|err| / RMS(ref)
    <= 1e-4 on every tap (probabilities: elementwise, below).
  * bfloat16 workloads, stagewise: every tap is compared with the oracle
    fed the GPU's own taps of that stage's operands, so each comparison
    sees one stage's rounding only: max|err| / RMS(ref) <= 2e-2.  The head
    outputs and the gated premix, whose size varies from row to row, and the
    MLP neurons, whose distribution is heavy-tailed, are held elementwise to
    the bound of their bf16 roundings (check_rounded and the head check).
  * probabilities (float32 softmax of float32 scores of the stored q, k):
    |err| <= 1e-3 |ref| + 1e-6 elementwise.  The score of a pair carries at
    most hd float32 roundings of products no larger than |q||k| / sqrt(hd),
    about 1e-4 absolute at these sizes, which is the relative error of its
    exponential; masked entries must be exactly 0.
  * sums the block forms in float32 from stored values (routed_output from
    the slots, mlp_output from routed + shared): 1e-4 of RMS.
"""
import numpy as np
import pytest
import torch

from oracle import block as ob
from transformer_decoder_block_amd import synth
from tests.blockrun import Run, rel_err

pytestmark = pytest.mark.gpu

SMALL_BF16 = list(synth.SMALL.values())
SMALL_F32 = [synth.f32_variant(w) for w in SMALL_BF16]

F32_BAR = 1e-4
BF16_BAR = 2e-2
SUM_BAR = 1e-4

ATTN_TAPS = ["attention_queries", "attention_keys", "attention_values",
             "attention_probabilities", "attention_head_outputs",
             "attention_premix"]


def interior_taps(w):
    t = ["attention_norm_output", "layer_mid", "mlp_input", "mlp_norm_output",
         "attention_output", "mlp_output"] + ATTN_TAPS
    if w.mlp == "moe":
        t += ["router_logits", "expert_indices", "expert_weights", "expert_outputs",
              "routed_output"]
        if w.n_shared:
            t.append("shared_expert_output")
    else:
        t += ["mlp_neurons", "mlp_activation"]
    return t


def check_probs(got, ref):
    zero = ref == 0
    assert np.all(got[zero] == 0), "probability outside the visible set"
    assert np.all(np.abs(got - ref) <= 1e-3 * np.abs(ref) + 1e-6), \
        float(np.max(np.abs(got - ref) / (np.abs(ref) + 1e-6)))


def check_rounded(got, ref, roundings):
    """Elementwise: each bf16 rounding adds at most 2^-9 |value|; checked
    with a factor 2, plus 1e-3 RMS(ref) for float32 accumulation."""
    rms = np.sqrt(np.mean(ref ** 2))
    bound = roundings * 2.0 ** -8 * np.abs(ref) + 1e-3 * rms
    assert np.all(np.abs(got - ref) <= bound), float(np.max(np.abs(got - ref) - bound))


def post_norm(v, W, cfg, name):
    return ob.rms_norm(v, W[name], cfg["eps"]) if cfg["sandwich"] else v


@pytest.mark.parametrize("w", SMALL_F32, ids=lambda w: w.name)
def test_f32_interior_taps(w):
    run = Run(w)
    out = run.forward(interior_taps(w))
    x64, W, cfg = run.x64(), run.W64, w.as_dict()
    assert np.array_equal(out["mlp_norm_output"], out["mlp_input"])
    for b in range(w.B):
        mk = None if run.mask is None else run.mask[b]
        r = ob.block_forward(x64[b], mk, W, cfg)
        assert rel_err(out["mlp_norm_output"][b], r["mlp_norm_output"]) <= F32_BAR
        for name in ("attention_queries", "attention_keys", "attention_values",
                     "attention_head_outputs", "attention_premix"):
            assert rel_err(out[name][b], r[name]) <= F32_BAR, name
        check_probs(out["attention_probabilities"][b], r["attention_probabilities"])
        if w.mlp != "moe":
            assert rel_err(out["mlp_neurons"][b], r["mlp_neurons"]) <= F32_BAR
            assert rel_err(out["mlp_activation"][b], r["mlp_activation"]) <= F32_BAR
            continue
        # a token whose choice differs at a float32 tie is left out (the
        # end-to-end test bounds how many there are)
        keep = np.all(np.sort(out["expert_indices"][b], -1)
                      == np.sort(r["expert_indices"], -1), -1)
        assert keep.sum() >= w.S - max(1, w.S // 100)
        assert rel_err(out["expert_outputs"][b][keep], r["expert_outputs"][keep]) <= F32_BAR
        assert rel_err(out["routed_output"][b][keep], r["routed_output"][keep]) <= F32_BAR
        if w.n_shared:
            assert rel_err(out["shared_expert_output"][b], r["shared_expert_output"]) <= F32_BAR


@pytest.mark.parametrize("w", SMALL_BF16, ids=lambda w: w.name)
def test_bf16_interior_taps_stagewise(w):
    run = Run(w)
    out = run.forward(interior_taps(w))
    x64, W, cfg = run.x64(), run.W64, w.as_dict()
    S, nh, hd = w.S, w.nh, w.hd
    pos = np.arange(S)
    # the norm's output is the operand the MLP is called with
    assert np.array_equal(out["mlp_norm_output"], out["mlp_input"])
    for b in range(w.B):
        mk = None if run.mask is None else run.mask[b]
        a_tap = out["attention_norm_output"][b]
        # q, k, v from the GPU's normed stream
        q, k, v = ob.qkv_heads(a_tap, W, cfg, pos)
        q_t, k_t, v_t = (out["attention_queries"][b], out["attention_keys"][b],
                         out["attention_values"][b])
        assert rel_err(q_t, q) <= BF16_BAR
        assert rel_err(k_t, k) <= BF16_BAR
        assert rel_err(v_t, v) <= BF16_BAR
        # softmax and mixing from the GPU's stored q, k, v
        head_out, _, probs = ob.attention(q_t, k_t, v_t, pos, pos, mk, w.window)
        check_probs(out["attention_probabilities"][b], probs)
        ho_t = out["attention_head_outputs"][b]
        # each probability enters the bf16 product rounded to bf16 and the
        # result is rounded to bf16 once: |err| <= 2^-9 (|ref| + sum p|v|),
        # checked with a factor 2 for the float32 sums
        spv, _, _ = ob.attention(q_t, k_t, np.abs(v_t), pos, pos, mk, w.window)
        assert np.all(np.abs(ho_t - head_out) <= 2.0 ** -8 * (np.abs(head_out) + spv) + 1e-6)
        # head gate from the GPU's head outputs
        pm_t = out["attention_premix"][b]
        if w.head_gate:
            gl = ob.sigmoid(ob.linear(a_tap, W["w_head_gate"]))
            ref = (ho_t * gl[:, :, None]).reshape(S, nh * hd) if w.head_gate == nh \
                else ho_t.reshape(S, nh * hd) * gl
            # the GPU gates the float32 head output and rounds once; the
            # reference gates the head-output tap (itself rounded once)
            check_rounded(pm_t, ref, 2)
        else:
            assert np.array_equal(pm_t, ho_t.reshape(S, nh * hd))
        # o_proj (and the sandwich norm) from the GPU's premix
        ao = post_norm(ob.linear(pm_t, W["wo"]), W, cfg, "w_post_attn_norm")
        assert rel_err(out["attention_output"][b], ao) <= BF16_BAR
        # MLP from the GPU's mlp_input
        m_tap = out["mlp_input"][b]
        if w.mlp != "moe":
            n_t = out["mlp_neurons"][b]
            mref = ob.mlp_forward(m_tap, W, cfg)
            # a product of two projections is heavy-tailed: the one bf16
            # rounding of each neuron (and of each activation) is checked
            # elementwise
            check_rounded(n_t, mref["mlp_neurons"], 1)
            check_rounded(out["mlp_activation"][b], mref["mlp_activation"], 1)
            mo = post_norm(ob.linear(n_t, W["w_down"]), W, cfg, "w_post_mlp_norm")
            assert rel_err(out["mlp_output"][b], mo) <= BF16_BAR
            continue
        mres = ob.mlp_forward(m_tap, W, cfg, out["router_logits"][b])
        assert np.array_equal(out["expert_indices"][b], mres["expert_indices"])
        eo_t = out["expert_outputs"][b]
        assert rel_err(eo_t, mres["expert_outputs"]) <= BF16_BAR
        routed_t = out["routed_output"][b]
        assert rel_err(routed_t, eo_t.sum(axis=1)) <= SUM_BAR
        raw = routed_t
        if w.n_shared:
            sh_t = out["shared_expert_output"][b]
            assert rel_err(sh_t, mres["shared_expert_output"]) <= BF16_BAR
            raw = routed_t + sh_t
        mo = post_norm(raw, W, cfg, "w_post_mlp_norm")
        assert rel_err(out["mlp_output"][b], mo) <= SUM_BAR


@pytest.mark.parametrize("name", ["llama_small", "afmoe_small", "arcee_small"])
def test_interior_taps_leave_output_unchanged(name):
    """Asking for every interior tap runs extra kernels on the same stream;
    the block's output must be bit-identical to a call without taps."""
    w = synth.SMALL[name]
    run = Run(w)
    plain = run.forward()["y_raw"].clone()
    tapped = run.forward(interior_taps(w))["y_raw"]
    assert torch.equal(plain.view(torch.int16), tapped.view(torch.int16))


def all_taps(w):
    return ["layer_input", "attention_scores", "layer_output"] + interior_taps(w)


@pytest.mark.parametrize("w", SMALL_BF16 + SMALL_F32[:2], ids=lambda w: w.name)
def test_tap_canaries_small(w):
    """Every tap and y between canary words: no kernel writes past either
    end of a caller's buffer, and the output is the same as without taps."""
    run = Run(w)
    plain = run.forward()["y_raw"].clone()
    out = run.forward(all_taps(w), guard=True)
    assert torch.equal(plain.view(torch.uint8), out["y_raw"].view(torch.uint8))


@pytest.mark.parametrize("name", ["llama7b_bf16", "afmoe_bf16"])
def test_tap_canaries_full_size(name):
    """The same at full size, where the GEMMs take their largest tiles, the
    K-split tail and the persistent grid."""
    w = synth.WORKLOADS[name]
    run = Run(w)
    run.forward(all_taps(w), guard=True, on_device=True)
