"""Every-element GPU parity of GEMMs whose last round runs as 256 x 128 tiles.

A persistent 256 x 256 launch whose last round would fill at most half of
the CUs, with that round made of whole tile columns, runs those columns as
a second launch of 256 x 128 tiles (the Arcee o_proj and the Apertus up
projection at their full sizes take it).  These shapes send the o_proj,
up and down GEMMs of a block through it, with a ragged last M tile, a
ragged last N tile inside the half-width columns and a K that is not a
multiple of the 64-wide stage.  Each GEMM is checked on every element
against the fp64 product of the GPU's own input tap (granite sheet
"LlamaForCausalLM 32L-4096d", section "Implementing it": o_proj with the
residual, the gated MLP, down with the residual; arcee page, section 03,
squared ReLU; apertus page, section 03, xIELU; afmoe page, section 03, the
sandwich norms):

  * plain float32 results (layer_mid, the raw products) within the
    worst-case float32 summation error of any order, K 2^-24 sum |a b|,
    plus one float32 rounding;
  * bf16 results (the neurons, y) within that plus one bf16 rounding;
  * results through a norm in float32 within 1e-4 of their RMS.

The first forward asks only for taps that are copies of buffers the block
computes anyway, so the GEMMs keep their staged epilogues; the second asks
for the raw products, which take the per-element epilogue.
"""
import numpy as np
import pytest

from oracle import block as ob
from transformer_decoder_block_amd import synth
from tests.blockrun import Run, rel_err
from tests.test_gpu_parity import F32_BAR

pytestmark = pytest.mark.gpu

CUS = 256  # compute units of the MI355X


def case(name, B, S, H, I, mlp, **kw):
    return synth.Workload(name, "bf16", B=B, S=S, H=H, nh=8, nkv=4, hd=128, mlp=mlp, I=I,
                          seed=71, **kw)


CASES = [
    # T = 4000 (16 M tiles, the last 160 rows); o_proj and down: 17 N tiles,
    # the 17th (248 columns) as two 128-wide tiles; up: 20 tiles of 128
    # neurons, the last four (504 neurons) as eight 64-neuron tiles; down's
    # K = 2552 ends in a 56-wide stage
    case("tail_swiglu", 2, 2000, 4344, 2552, "swiglu"),
    # up: 18 N tiles of 256, the 18th holding 248 columns
    case("tail_relu2", 1, 4096, 4352, 4600, "relu2"),
    # o_proj stores float32 for the sandwich norm; up 17 N tiles
    case("tail_xielu_sandwich", 4, 1024, 4352, 4352, "xielu", sandwich=True,
         qk_norm=True),
]


def persistent_tail(M, N, n_per):
    """True when the 256 x 256 launch of an M x N product ends in a round of
    whole tile columns that fills at most half of the CUs."""
    num_m, num_n = (M + 255) // 256, (N + n_per - 1) // n_per
    tiles = num_m * num_n
    rem = tiles % CUS
    return tiles > CUS and 0 < rem <= CUS // 2 and rem % num_m == 0


def sum_bound(a, b):
    """K 2^-24 (|a| |b|^T): the float32 error of any summation order of
    exact products."""
    return a.shape[1] * 2.0 ** -24 * (np.abs(a) @ np.abs(b).T)


def check_product(got, ref, bound, bf16=False, what=""):
    """|got - ref| <= bound + one rounding of the result (float32, or bf16
    with a factor 2 of slack)."""
    r = 2.0 ** -8 if bf16 else 2.0 ** -23
    err = np.abs(got - ref) - (bound + r * np.abs(ref) + 1e-30)
    bad = err > 0
    assert not bad.any(), (what, int(bad.sum()), float(err.max()))


def act_ref(w, m, W):
    """The neurons (the down projection's operand) and their float32-sum
    bound, from the GPU's MLP input."""
    cfg = w.as_dict()
    ref = ob.mlp_forward(m, W, cfg)["mlp_neurons"]
    if w.mlp == "swiglu":
        bound = None  # a product of two projections: checked with check_rounded
    else:
        z = ob.linear(m, W["w_up"])
        sb = sum_bound(m, W["w_up"])
        # |act(z + e) - act(z)| for |e| <= sb: relu2 at most (2|z| + sb) sb;
        # xielu's slope is 2 alpha_p z + beta above 0 and at most
        # alpha_n + beta below, alpha_p, alpha_n <= softplus(1) + beta < 2
        slope = 2 * np.abs(z) + sb if w.mlp == "relu2" else 4 * np.abs(z) + 3
        bound = slope * sb
    return ref, bound


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_tail_tiles_every_element(w):
    T, H, I = w.T, w.H, w.I
    up_per = 128 if w.mlp == "swiglu" else 256
    assert persistent_tail(T, H, 256), "o_proj must take the tail launch"
    assert persistent_tail(T, H, 256), "down must take the tail launch"
    assert persistent_tail(T, I, up_per), "up must take the tail launch"
    print(f"[tail] {w.name}: T={T} H={H} I={I} mlp={w.mlp} sandwich={w.sandwich}",
          flush=True)
    run = Run(w)
    W, cfg = run.W64, w.as_dict()
    x64 = run.x64().reshape(T, H)

    # staged epilogues: only copies of the block's own buffers are asked for
    out = run.forward(["attention_premix", "layer_mid", "mlp_input", "mlp_neurons"])
    pm = out["attention_premix"].reshape(T, -1)
    mid = out["layer_mid"].reshape(T, H)
    m = out["mlp_input"].reshape(T, H)
    neur = out["mlp_neurons"].reshape(T, I)
    o = ob.linear(pm, W["wo"])
    if w.sandwich:
        assert rel_err(mid - x64, ob.rms_norm(o, W["w_post_attn_norm"], w.eps)) <= F32_BAR
    else:
        check_product(mid, x64 + o, sum_bound(pm, W["wo"]), what="layer_mid")
    ref_n, bound_n = act_ref(w, m, W)
    if bound_n is None:
        rms = np.sqrt(np.mean(ref_n ** 2))
        bad = np.abs(neur - ref_n) > 2.0 ** -8 * np.abs(ref_n) + 1e-3 * rms
        assert not bad.any(), ("mlp_neurons", int(bad.sum()))
    else:
        check_product(neur, ref_n, bound_n, bf16=True, what="mlp_neurons")
    d = ob.linear(neur, W["w_down"])
    y = out["y"].reshape(T, H)
    if w.sandwich:
        ref_y = mid + ob.rms_norm(d, W["w_post_mlp_norm"], w.eps)
        rms = np.sqrt(np.mean(ref_y ** 2))
        bad = np.abs(y - ref_y) > 2.0 ** -8 * np.abs(ref_y) + F32_BAR * rms
        assert not bad.any(), ("y", int(bad.sum()))
    else:
        check_product(y, mid + d, sum_bound(neur, W["w_down"]), bf16=True, what="y")
    print(f"[tail] {w.name}: staged epilogues every element", flush=True)

    # the raw products (the per-element epilogue of the residual GEMMs)
    out2 = run.forward(["attention_output", "mlp_output", "layer_mid", "layer_output"])
    ao = out2["attention_output"].reshape(T, H)
    mo = out2["mlp_output"].reshape(T, H)
    if w.sandwich:
        assert rel_err(ao, ob.rms_norm(o, W["w_post_attn_norm"], w.eps)) <= F32_BAR
        assert rel_err(mo, ob.rms_norm(d, W["w_post_mlp_norm"], w.eps)) <= F32_BAR
    else:
        check_product(ao, o, sum_bound(pm, W["wo"]), what="attention_output")
        check_product(mo, d, sum_bound(neur, W["w_down"]), what="mlp_output")
    # the two forwards computed the same block
    assert np.array_equal(out2["layer_mid"], out["layer_mid"])
    assert np.array_equal(out2["y"], out["y"])
    print(f"[tail] {w.name}: raw products every element", flush=True)
