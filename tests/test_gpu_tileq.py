"""Every-element GPU parity of the 256 x 256 Q/K/V tile that the full-size
workloads run.

The fused Q/K/V GEMM switches to its large tile (64 x 128 wave tiles, whole
heads per wave) once the grid holds at least 256 tiles of 256 x 256; the
small parity shapes never reach it.  These shapes do, at head widths 128
and 64, with hidden 256 so that the fp64 oracle evaluates every token:

  * stage A (the attention-input norm) on every row;
  * the per-head queries, keys and values (after the q/k norm and the
    rotary) on every element, against the oracle fed the GPU's own normed
    stream, each held to its one bf16 rounding (granite sheet
    "LlamaForCausalLM 32L-4096d", section "Implementing it"; apertus page,
    section 03: per-head norm ahead of the rotary);
  * the head outputs on every element, against the oracle's attention from
    the GPU's own q, k, v (so K/V placement is checked key by key: two of
    the cases scale the queries so that most rows put nearly all their
    weight on one key, where a misplaced K or V row moves the output by
    the size of v itself);
  * stage C (layer_mid) on every row of every sequence, from the GPU's own
    q, k, v taps (head gate, o_proj, residual) and from its normed stream.

Where the grid's last round would fill at most half of the CUs, that round
runs as 256 x 128 tiles (8 waves of 32 x 128) in a launch of its own; two
cases reach it.  The cases cover a ragged last M tile, sequences that start inside a tile,
sequence lengths that are not multiples of the 8- and 16-key groups of the
transposed value store, the head-gate columns in a partial last N tile, a
window, and GQA groups of 2, 4 and 6.
"""
import numpy as np
import pytest
import torch

from oracle import bf16_emulation as em
from oracle import block as ob
from transformer_decoder_block_amd import synth
from tests.blockrun import Run, rel_err
from tests.test_gpu_parity import BF16_BAR, check_floor

pytestmark = pytest.mark.gpu


def case(name, B, S, nh, nkv, hd, sharp=0, **kw):
    base = dict(H=256, mlp="swiglu", I=256, seed=60)
    base.update(kw)
    return (synth.Workload(name, "bf16", B=B, S=S, nh=nh, nkv=nkv, hd=hd, **base), sharp)


CASES = [
    # 16 x 16 tiles; the second sequence starts at row 2000, inside M tile 7
    case("tileq_hd128_g2", 2, 2000, 16, 8, 128),
    # 17 x 17 tiles: ragged last M tile (rows 4096-4099), gate columns in
    # the last N tile, q/k norm, window; S = 1025, so every sequence but the
    # first starts inside an M tile and inside a 16-key group
    case("tileq_hd64_gate", 4, 1025, 32, 16, 64, qk_norm=True, sandwich=True,
         head_gate=32, window=300),
    # 16 x 18 tiles (the last two columns as 256 x 128 tiles), q/k norm
    # with the query gain scaled 16x (sharp
    # attention); S % 8 = 5, so 8-key groups straddle two sequences
    case("tileq_hd128_g4_sharp", 3, 1365, 24, 6, 128, sharp=16, qk_norm=True,
         mlp="xielu"),
    # 16 x 16 tiles, hd 64, GQA 6, wq scaled 128x (sharp attention)
    case("tileq_hd64_g6_sharp", 4, 1024, 48, 8, 64, sharp=128),
    # 16 x 20 tiles: the last round (64 tiles, the last four columns) runs
    # as 256 x 128 tiles, which hold the k heads (q/k norm, rotary) and the
    # v heads
    case("tileq_tail_hd128", 4, 1024, 32, 4, 128, qk_norm=True),
    # 16 x 21 tiles, the last five columns as 256 x 128 tiles: k, v and the
    # head-gate columns, a ragged last M tile, S % 16 = 1 (V^T stores that
    # straddle sequences), a window
    case("tileq_tail_hd64_gate", 2, 2001, 64, 8, 64, head_gate=64, window=500),
]


def tiles_q(w):
    n = (w.nh + 2 * w.nkv) * w.hd + w.head_gate
    return ((w.T + 255) // 256) * ((n + 255) // 256)


def check_rounded(got, ref, roundings=1):
    """|got - ref| <= roundings * 2^-8 |ref| + 1e-3 RMS(ref), every element:
    one bf16 rounding costs at most 2^-9 |value| (a factor 2 of slack), and
    float32 accumulation far less than 1e-3 of the RMS."""
    rms = np.sqrt(np.mean(ref ** 2))
    bound = roundings * 2.0 ** -8 * np.abs(ref) + 1e-3 * rms
    bad = np.abs(got - ref) > bound
    assert not bad.any(), (int(bad.sum()), float(np.max(np.abs(got - ref) - bound)))


@pytest.mark.parametrize("w,sharp", CASES, ids=[c[0].name for c in CASES])
def test_tileq_every_element(w, sharp):
    assert tiles_q(w) >= 256, "the shape must reach the large Q/K/V tile"
    print(f"[tileq] {w.name}: B={w.B} S={w.S} nh={w.nh} nkv={w.nkv} hd={w.hd} "
          f"tiles={tiles_q(w)} sharp={sharp}", flush=True)
    run = Run(w)
    W = run.W64
    if sharp:
        # an exact power-of-two scale on the device weights and the oracle's
        key = "w_q_norm" if w.qk_norm else "wq"
        run.Wd[key].mul_(sharp)
        W = dict(W)
        W[key] = W[key] * sharp
    taps = ["attention_norm_output", "attention_queries", "attention_keys",
            "attention_values", "attention_head_outputs", "layer_mid"]
    out = run.forward(taps)
    check_case(w, sharp, W, out, run.x64(), run.mask)


def check_case(w, sharp, W, out, x64, mask):
    """The comparisons of one case, given its taps as float64 arrays."""
    cfg = w.as_dict()
    S = w.S
    pos = np.arange(S)
    for b in range(w.B):
        mk = None if mask is None else mask[b]
        a_tap = out["attention_norm_output"][b]
        # stage A, every row: one bf16 rounding of the norm
        ref_a = ob.rms_norm(x64[b], W["w_in_norm"], w.eps)
        check_rounded(a_tap, ref_a)
        # q, k, v on every element, from the GPU's normed stream
        q, k, v = ob.qkv_heads(a_tap, W, cfg, pos)
        q_t, k_t, v_t = (out["attention_queries"][b], out["attention_keys"][b],
                         out["attention_values"][b])
        check_rounded(q_t, q)
        check_rounded(k_t, k)
        check_rounded(v_t, v)
        # head outputs on every element, from the GPU's stored q, k, v: each
        # probability enters the bf16 product rounded once and the output is
        # rounded once, |err| <= 2^-9 (|ref| + sum_j p_j |v_j|), checked with
        # a factor 2 for the float32 scores and sums.  One query head at a
        # time, so the oracle's score matrices stay small.
        ho_t = out["attention_head_outputs"][b]
        ho_all = np.empty_like(ho_t)
        g = w.nh // w.nkv
        for h in range(w.nh):
            kv = h // g
            ho, _, probs = ob.attention(q_t[h:h + 1], k_t[kv:kv + 1], v_t[kv:kv + 1],
                                        pos, pos, mk, w.window)
            spv = probs[0] @ np.abs(v_t[kv])
            err = np.abs(ho_t[:, h] - ho[:, 0]) - (2.0 ** -8 * (np.abs(ho[:, 0]) + spv)
                                                   + 1e-6)
            assert np.all(err <= 0), (b, h, int((err > 0).sum()), float(err.max()))
            ho_all[:, h] = ho[:, 0]
        # stage C on every row from the GPU's q, k, v: head gate, o_proj,
        # (post-norm,) residual
        premix = ho_all.reshape(S, w.nh * w.hd)
        if w.head_gate:
            gl = ob.sigmoid(ob.linear(a_tap, W["w_head_gate"]))
            premix = (ho_all * gl[:, :, None]).reshape(S, -1) if w.head_gate == w.nh \
                else premix * gl
        o = ob.linear(premix, W["wo"])
        if w.sandwich:
            o = ob.rms_norm(o, W["w_post_attn_norm"], w.eps)
        mid_t = out["layer_mid"][b]
        e_qkv = rel_err(mid_t, x64[b] + o)
        # stage C on every row from the GPU's normed stream (the workloads'
        # stagewise protocol), in blocks of query rows; where the queries
        # are scaled for sharp attention, the bf16 rounding of q and k moves
        # the scores by up to 2^-9 of their size, and the bar is the bf16
        # floor of this comparison times its derived factor
        ref_mid = np.empty_like(mid_t)
        emu_mid = np.empty_like(mid_t)
        for r0 in range(0, S, 512):
            rows = np.arange(r0, min(S, r0 + 512))
            ref_mid[rows] = ob.attention_sublayer(x64[b], a_tap, mk, W, cfg,
                                                  rows)["layer_mid"]
            if sharp:
                emu_mid[rows] = em.attention_sublayer_bf16(x64[b], a_tap, mk, W, cfg,
                                                           rows)["layer_mid"]
        e = rel_err(mid_t, ref_mid)
        print(f"[tileq] {w.name} b={b}: layer_mid max|err|/RMS from q/k/v taps "
              f"{e_qkv:.4g}, from attention_norm_output {e:.4g}", flush=True)
        assert e_qkv <= BF16_BAR
        if sharp:
            check_floor(f"{w.name} b={b} layer_mid", "attention_output", e,
                        rel_err(emu_mid, ref_mid))
        else:
            assert e <= BF16_BAR
