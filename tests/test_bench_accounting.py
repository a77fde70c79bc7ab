"""The work bench.py divides measured times by, checked against closed forms.

* visible (query, key) pairs: causal rows see i + 1 keys; a window of W
  caps that at W; key padding on a tail removes the padded keys from every
  row after them.
* a dense block's forward FLOPs are 2 x (its weight count) x tokens for the
  projections plus 4 hd per visible pair per head for q k^T and p v.
"""
import pytest

import bench
from transformer_decoder_block_amd import synth


def causal_pairs(S, W=0, real=None):
    """Sum over rows of the visible keys, in closed form."""
    real = S if real is None else real  # keys at >= real are padding
    if W <= 0:
        # rows < real see i + 1 keys; later rows see the `real` unpadded keys
        return real * (real + 1) // 2 + (S - real) * real
    assert real == S
    return W * (W + 1) // 2 + (S - W) * W if S > W else S * (S + 1) // 2


@pytest.mark.parametrize("name", ["tiny_llama_f32", "llama7b_bf16", "arcee_gqa_bf16",
                                  "apertus_bf16", "afmoe_bf16"])
def test_visible_pairs_closed_form(name):
    w = synth.WORKLOADS[name]
    mask = synth.make_mask(w)
    expect = 0
    for b in range(w.B):
        real = w.S
        if mask is not None:
            row = mask[b]
            # the workloads pad a tail of the sequence (or nothing)
            real = int(row.sum())
            assert row[:real].all() and not row[real:].any()
        expect += causal_pairs(w.S, w.window, real)
    assert bench.visible_pairs(w, mask) == expect


def test_dense_flops_are_two_per_weight_per_token():
    w = synth.WORKLOADS["llama7b_bf16"]
    mask = synth.make_mask(w)
    H, I, hd = w.H, w.I, w.hd
    weights = H * (w.nh + 2 * w.nkv) * hd + w.nh * hd * H + 3 * H * I
    attn = 4 * hd * w.nh * bench.visible_pairs(w, mask)
    assert bench.total_flops(bench.kernel_work(w, mask)) == 2 * weights * w.T + attn
    # 419.6 MFLOP per token at this shape
    assert round((2 * weights * w.T + attn) / w.T / 1e6, 1) == 419.6


def test_moe_flops_count_chosen_experts_only():
    w = synth.WORKLOADS["afmoe_bf16"]
    mask = synth.make_mask(w)
    work = bench.kernel_work(w, mask)
    per_token_expert = 2 * 3 * w.H * w.I_e          # gate, up, down of one expert
    assert work["gemm_expert_up"][1] + work["gemm_expert_down"][1] == \
        w.T * w.top_k * per_token_expert
    assert work["gemm_router"][1] == 2 * w.T * w.H * w.E
