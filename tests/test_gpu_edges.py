"""GPU parity on the degenerate and boundary cases of the block, through the
C ABI, against the fp64 oracle (bars as in test_gpu_parity.py):

  * one token per sequence, and lengths that are not multiples of the 8-
    and 16-key groups of the transposed value store;
  * hidden and MLP widths that are multiples of 8 but not of any tile
    (ragged K and N edges in every GEMM);
  * attention masks with left padding and holes, including query rows that
    see no key at all (their attention output is 0);
  * a window of one key (each query sees itself only) and a window longer
    than the sequence (identical to full causal);
  * exact ties among the router's biased scores (the lower expert index
    wins, slots in descending score order);
  * a sliding window with 128-wide heads, and the float32 path at 2048
    tokens and hidden 2048;
  * the widest hidden size the library accepts (8192) and the largest
    expert count (256).
"""
import numpy as np
import pytest
import torch

from oracle import block as ob
from transformer_decoder_block_amd import synth
from oracle import bf16_emulation as em
from tests.blockrun import Run, dev, rel_err
from tests.test_gpu_parity import BF16_BAR, F32_BAR, check_floor, check_scores, near_tie

pytestmark = pytest.mark.gpu

TAPS = ["layer_input", "attention_norm_output", "attention_scores", "layer_mid",
        "mlp_input", "layer_output", "attention_output", "mlp_output"]
MOE_TAPS = ["router_logits", "expert_indices", "expert_weights"]


def llama(name, dtype, B, S, H=256, nh=4, nkv=2, hd=64, I=344, **kw):
    return synth.Workload(name, dtype, B=B, S=S, H=H, nh=nh, nkv=nkv, hd=hd,
                          mlp="swiglu", I=I, seed=kw.pop("seed", 40), **kw)


def afmoe(name, dtype, B, S, E=8, top_k=2, **kw):
    base = dict(H=256, nh=4, nkv=2, hd=64, mlp="moe", qk_norm=True, sandwich=True,
                window=32, head_gate=4, E=E, top_k=top_k, I_e=96, n_shared=1,
                route_scale=2.826, seed=41)
    base.update(kw)
    return synth.Workload(name, dtype, B=B, S=S, **base)


def taps_for(w):
    return TAPS + (MOE_TAPS if w.mlp == "moe" else [])


def check_f32(run, mask=None):
    """End to end from layer_input, every tap, at the float32 bar."""
    w = run.w
    md = None if mask is None else torch.from_numpy(mask).cuda()
    out = run.forward(taps_for(w), mask=md)
    x64, W, cfg = run.x64(), run.W64, w.as_dict()
    for b in range(w.B):
        mk = None if mask is None else mask[b]
        r = ob.block_forward(x64[b], mk, W, cfg)
        keep = np.ones(w.S, bool)
        if w.mlp == "moe":
            gi = np.sort(out["expert_indices"][b], -1)
            diff = np.any(gi != np.sort(r["expert_indices"], -1), -1)
            assert np.all(near_tie(r["router_logits"], W["expert_bias"], w.top_k)[diff])
            keep = ~diff
        for name in ("attention_norm_output", "layer_mid", "mlp_input", "attention_output"):
            assert rel_err(out[name][b], r[name]) <= F32_BAR, (name, b)
        for name in ("mlp_output", "layer_output"):
            assert rel_err(out[name][b][keep], r[name][keep]) <= F32_BAR, (name, b)
        check_scores(out["attention_scores"][b], r["attention_scores"], F32_BAR)
    return out


def check_bf16(run, mask=None):
    """Stagewise, each stage fed the GPU's own tap of its input."""
    w = run.w
    md = None if mask is None else torch.from_numpy(mask).cuda()
    out = run.forward(taps_for(w), mask=md)
    x64, W, cfg = run.x64(), run.W64, w.as_dict()
    lo = torch.from_numpy(out["layer_output"].astype(np.float32)).to(torch.bfloat16)
    assert torch.equal(lo.view(torch.int16), out["y_raw"].cpu().view(torch.int16))
    for b in range(w.B):
        mk = None if mask is None else mask[b]
        a_tap = out["attention_norm_output"][b]
        assert rel_err(a_tap, ob.rms_norm(x64[b], W["w_in_norm"], w.eps)) <= BF16_BAR
        att = ob.attention_sublayer(x64[b], a_tap, mk, W, cfg)
        check_scores(out["attention_scores"][b], att["attention_scores"], BF16_BAR)
        assert rel_err(out["layer_mid"][b], att["layer_mid"]) <= BF16_BAR
        fl = rel_err(em.attention_sublayer_bf16(x64[b], a_tap, mk, W, cfg)["attention_output"],
                     att["attention_output"])
        check_floor(f"{w.name} b={b}", "attention_output",
                    rel_err(out["attention_output"][b], att["attention_output"]), fl)
        mid_tap, m_tap = out["layer_mid"][b], out["mlp_input"][b]
        assert rel_err(m_tap, ob.mlp_norm(mid_tap, W, cfg)) <= BF16_BAR
        logits = None
        if w.mlp == "moe":
            logits = out["router_logits"][b]
            # the router GEMM itself (its K tail included), from the GPU's
            # own MLP input; the choice below is then made from its logits
            assert rel_err(logits, ob.linear(m_tap, W["w_router"])) <= BF16_BAR
            _, idx, wts = ob.route(logits, W["expert_bias"], w.top_k, w.route_scale, "bf16")
            assert np.array_equal(out["expert_indices"][b], idx)
            np.testing.assert_allclose(out["expert_weights"][b], wts, rtol=2e-6, atol=1e-7)
        mo = ob.mlp_sublayer(mid_tap, m_tap, W, cfg, router_logits=logits)
        assert rel_err(out["layer_output"][b], mo["layer_output"]) <= BF16_BAR
    return out


CHECK = {"f32": check_f32, "bf16": check_bf16}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("S", [1, 7, 13, 72])
def test_short_and_ragged_sequences(dtype, S):
    CHECK[dtype](Run(llama(f"llama_s{S}", dtype, B=2, S=S)))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,nh,nkv,hd", [(1, 8, 8, 64), (2, 8, 8, 128), (3, 16, 8, 64),
                                         (2, 6, 3, 64)])
def test_attention_block_order(dtype, B, nh, nkv, hd):
    """The attention launch deals the blocks of an XCD heaviest query block
    first across its (batch, KV head) groups when the groups divide over the
    8 XCDs (8, 16 and 24 groups here, one or two query heads each), and per
    group otherwise (6 groups).  A mapping that ran a block twice or not at
    all would leave rows wrong: every row of every tap is checked."""
    CHECK[dtype](Run(llama(f"llama_order_{B}_{nh}_{nkv}_{hd}", dtype, B=B, S=300, nh=nh,
                           nkv=nkv, hd=hd, seed=44)))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_token_moe(dtype):
    CHECK[dtype](Run(afmoe("afmoe_s1", dtype, B=3, S=1)))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ragged_widths(dtype):
    # hidden 264 and MLP width 200: K and N tails in every GEMM and the norms
    CHECK[dtype](Run(llama("llama_ragged", dtype, B=2, S=45, H=264, I=200)))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("H", [264, 1064])
def test_ragged_hidden_moe(dtype, H):
    """The mixture block at hidden sizes that no router stage divides: the
    router GEMM's last K stage is partial (8 or 40 of its 256 columns), and
    each of its loads tests its own columns against K."""
    CHECK[dtype](Run(afmoe(f"afmoe_h{H}", dtype, B=2, S=45, H=H, I_e=200)))


def holes_mask(B, S, seed=7):
    """Sequence 0: about a fifth of the keys masked at random; sequence 1:
    the first 9 tokens masked (left padding: query rows 0..8 see no key)."""
    rng = np.random.default_rng(seed)
    m = np.ones((B, S), np.int32)
    m[0] = (rng.random(S) > 0.2).astype(np.int32)
    m[1, :9] = 0
    return m


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("family", ["llama", "afmoe"])
def test_left_padding_and_holes(dtype, family):
    S = 150
    w = llama("llama_holes", dtype, B=2, S=S) if family == "llama" else \
        afmoe("afmoe_holes", dtype, B=2, S=S)
    run = Run(w)
    mask = holes_mask(2, S)
    out = CHECK[dtype](run, mask)
    # query rows that see no key: no attention output at all
    assert np.all(out["attention_output"][1, :9] == 0.0)
    assert np.all(np.isneginf(out["attention_scores"][1, :, :9]))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_window_of_one(dtype):
    w = llama("llama_w1", dtype, B=2, S=100, window=1)
    CHECK[dtype](Run(w))


def test_window_longer_than_sequence_is_causal():
    w = llama("llama_wlong", "bf16", B=2, S=130)
    causal = Run(w).forward(["layer_output"])
    longw = Run(w.replace(window=1000)).forward(["layer_output"])
    assert np.array_equal(causal["y"], longw["y"])
    assert np.array_equal(causal["layer_output"], longw["layer_output"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_router_exact_ties(dtype):
    """Experts 0-3 share one router row and one bias, as do 4-5: their
    biased scores tie exactly for every token."""
    w = afmoe("afmoe_ties", dtype, B=2, S=64, E=8, top_k=3)
    run = Run(w)
    for grp in ((0, 1, 2, 3), (4, 5)):
        for e in grp[1:]:
            run.Wst["w_router"][e] = run.Wst["w_router"][grp[0]]
            run.Wst["expert_bias"][e] = run.Wst["expert_bias"][grp[0]]
    # same device buffers (the handle keeps their addresses), new contents
    run.Wd["w_router"].copy_(dev(run.Wst["w_router"], w.dtype))
    run.Wd["expert_bias"].copy_(dev(run.Wst["expert_bias"], "f32"))
    run._W64 = None
    out = run.forward(["router_logits", "expert_indices", "expert_weights"])
    W = run.W64
    for b in range(w.B):
        lg = out["router_logits"][b]
        assert np.array_equal(lg[:, 0], lg[:, 3]) and np.array_equal(lg[:, 4], lg[:, 5])
        _, idx, wts = ob.route(lg, W["expert_bias"], w.top_k, w.route_scale, w.dtype)
        assert np.array_equal(out["expert_indices"][b], idx)
        np.testing.assert_allclose(out["expert_weights"][b], wts, rtol=2e-6, atol=1e-7)
        # a tied group is taken lowest index first, in consecutive slots
        for t in range(w.S):
            sel = list(idx[t])
            for grp in ((0, 1, 2, 3), (4, 5)):
                got = [e for e in sel if e in grp]
                assert got == sorted(got)
                assert got == list(grp[:len(got)])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_widest_hidden(dtype):
    w = llama("llama_h8192", dtype, B=1, S=40, H=8192, nh=64, nkv=8, hd=128, I=256)
    CHECK[dtype](Run(w))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_most_experts(dtype):
    w = afmoe("afmoe_e256", dtype, B=1, S=96, E=256, top_k=8, I_e=32, window=0,
              head_gate=0)
    CHECK[dtype](Run(w))


def test_split_tail_tiles():
    """o_proj at 4352 tokens x 4096 outputs, K = 64 heads x 128 = 8192, is
    272 tiles of 256 x 256 with 128 K stages on a 256-CU part: its last 16
    tiles (rows 4096-4351) run as two K halves summed by the fixup.  Every
    row of those tiles, and rows of the whole tiles around them, match the
    oracle on layer_mid, and y is still the rounding of the float32
    layer_output.  The Q/K/V GEMM of this shape (17 x 40 tiles) runs the
    large Q/K/V tile: its queries, keys and values are checked on every
    element."""
    from tests.blockrun import host
    from tests.test_gpu_tileq import check_rounded
    w = llama("llama_split", "bf16", B=1, S=4352, H=4096, nh=64, nkv=8, hd=128, I=512)
    run = Run(w)
    d = run.forward(["attention_norm_output", "layer_mid", "layer_output",
                     "attention_queries", "attention_keys", "attention_values"],
                    on_device=True)
    lo = d["layer_output"].to(torch.bfloat16).view(torch.int16)
    assert torch.equal(lo, d["y_raw"].view(torch.int16))
    x64, W, cfg = run.x64(), run.W64, w.as_dict()
    a_tap = host(d["attention_norm_output"][0])
    # q, k, v of every token from the GPU's normed stream
    q, k, v = ob.qkv_heads(a_tap, W, cfg, np.arange(w.S))
    check_rounded(host(d["attention_queries"][0]), q)
    check_rounded(host(d["attention_keys"][0]), k)
    check_rounded(host(d["attention_values"][0]), v)
    del q, k, v
    # every row of the split tiles, plus rows of whole tiles
    rows = np.concatenate([np.array([0, 1, 255, 256, 2047, 3839, 4094, 4095]),
                           np.arange(4096, 4352)])
    mid = host(d["layer_mid"][0][torch.from_numpy(rows).cuda()])
    for part in np.array_split(np.arange(len(rows)), 4):
        att = ob.attention_sublayer(x64[0], a_tap, None, W, cfg, rows[part])
        assert rel_err(mid[part], att["layer_mid"]) <= BF16_BAR


def test_staged_epilogue_ragged_columns():
    """Hidden 1064 (a multiple of 8, not of 64) at 13312 tokens: o_proj and
    the down projection are 52 x 5 tiles of 256 x 256 and run persistent.
    In the last column of tiles, the waves whose 64 columns pass the hidden
    size take the per-quad epilogue while the others stage their rows
    through LDS.  layer_mid and layer_output match the oracle on every
    column of rows in the first, middle and last row tiles, and y is the
    rounding of the float32 layer_output."""
    from tests.blockrun import host
    w = llama("llama_h1064", "bf16", B=1, S=13312, H=1064, nh=8, nkv=2, hd=128, I=512)
    run = Run(w)
    d = run.forward(["attention_norm_output", "layer_mid", "mlp_input", "layer_output"],
                    on_device=True)
    lo = d["layer_output"].to(torch.bfloat16).view(torch.int16)
    assert torch.equal(lo, d["y_raw"].view(torch.int16))
    x64, W, cfg = run.x64(), run.W64, w.as_dict()
    a_tap = host(d["attention_norm_output"][0])
    rows = np.array([0, 1, 127, 255, 256, 6655, 6656, 6700, 13055, 13056, 13200, 13311])
    sel = torch.from_numpy(rows).cuda()
    mid = host(d["layer_mid"][0][sel])
    att = ob.attention_sublayer(x64[0], a_tap, None, W, cfg, rows)
    assert rel_err(mid, att["layer_mid"]) <= BF16_BAR
    m_t = host(d["mlp_input"][0][sel])
    mo = ob.mlp_sublayer(mid, m_t, W, cfg)
    assert rel_err(host(d["layer_output"][0][sel]), mo["layer_output"]) <= BF16_BAR


def test_staged_epilogue_ragged_columns_moe():
    """The AFMoE block at hidden 1064 and 13312 tokens: o_proj and the
    shared expert's down projection (float32 outputs, 52 x 5 tiles) and the
    routed experts' down projection (bf16 slot outputs in expert order,
    grouped) all run persistent with a last column of tiles whose waves
    partly pass the hidden size.  layer_mid and layer_output match the
    oracle on every column of the sampled rows, the experts routed from the
    GPU's own logits."""
    from tests.blockrun import host
    w = afmoe("afmoe_h1064", "bf16", B=1, S=13312, E=16, top_k=4, H=1064, nh=8, nkv=2,
              hd=128, window=2048, head_gate=8, I_e=256)
    run = Run(w)
    d = run.forward(["attention_norm_output", "layer_mid", "mlp_input", "layer_output",
                     "router_logits"], on_device=True)
    lo = d["layer_output"].to(torch.bfloat16).view(torch.int16)
    assert torch.equal(lo, d["y_raw"].view(torch.int16))
    x64, W, cfg = run.x64(), run.W64, w.as_dict()
    a_tap = host(d["attention_norm_output"][0])
    rows = np.array([0, 1, 255, 256, 6655, 6656, 13055, 13056, 13311])
    sel = torch.from_numpy(rows).cuda()
    mid = host(d["layer_mid"][0][sel])
    att = ob.attention_sublayer(x64[0], a_tap, None, W, cfg, rows)
    assert rel_err(mid, att["layer_mid"]) <= BF16_BAR
    m_t = host(d["mlp_input"][0][sel])
    logits = host(d["router_logits"][0][sel])
    mo = ob.mlp_sublayer(mid, m_t, W, cfg, router_logits=logits)
    assert rel_err(host(d["layer_output"][0][sel]), mo["layer_output"]) <= BF16_BAR


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_trinity_nano_moe_shape(dtype):
    """The afmoe page's Nano shape: 128 routed experts of width 256, top 8,
    hidden 1024, one shared expert (narrow experts: a harder grouped GEMM)."""
    w = afmoe("afmoe_nano", dtype, B=2, S=96, E=128, top_k=8, H=1024, nh=8, nkv=2,
              hd=128, I_e=256, window=0, head_gate=8)
    CHECK[dtype](Run(w))


def test_stack_of_blocks_on_one_handle():
    """A stack: the float32 output of block 1 is the input of block 2 (other
    weights), both on one handle and one workspace, against the oracle
    applied twice."""
    w1 = llama("llama_stack", "f32", B=2, S=70, seed=50)
    w2 = w1.replace(seed=51)
    r1, r2 = Run(w1), Run(w2)
    y1 = r1.forward(["layer_output"])
    x2 = r1.forward(on_device=True)["y_raw"]
    # block 2 on block 1's handle: same shapes, block 2's weights
    from transformer_decoder_block_amd import binding as L
    y = torch.empty_like(x2)
    io = L.blk_io(x=x2.data_ptr(), attention_mask=None, batch=w1.B, seq=w1.S, y=y.data_ptr())
    st = L.blk_forward(r1.block.h, io, r2.block.w, None,
                       torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == L.BLK_OK, L.blk_last_error()
    from tests.blockrun import host
    cfg = w1.as_dict()
    for b in range(w1.B):
        h1 = ob.block_forward(r1.x64()[b], None, r1.W64, cfg)["layer_output"]
        assert rel_err(y1["layer_output"][b], h1) <= F32_BAR
        h2 = ob.block_forward(h1, None, r2.W64, cfg)["layer_output"]
        assert rel_err(host(y[b]), h2) <= F32_BAR


def _mask_ptr(run):
    return None if run.maskd is None else run.maskd.data_ptr()


def _layers_call(handle_run, runs, x, y):
    """blk_forward_layers on handle_run's handle with the weights of runs
    (and handle_run's padding mask, if any)."""
    from transformer_decoder_block_amd import binding as L
    w = handle_run.w
    io = L.blk_io(x=x.data_ptr(), attention_mask=_mask_ptr(handle_run), batch=w.B, seq=w.S,
                  y=y.data_ptr())
    layers = [r.block.w for r in runs]
    st = L.blk_forward_layers(handle_run.block.h, io, layers,
                              torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return st


def _one_by_one(handle_run, runs, x):
    """The same stack as successive blk_forward calls on one handle."""
    from transformer_decoder_block_amd import binding as L
    w = handle_run.w
    cur = x
    for r in runs:
        y = torch.empty_like(x)
        io = L.blk_io(x=cur.data_ptr(), attention_mask=_mask_ptr(handle_run), batch=w.B,
                      seq=w.S, y=y.data_ptr())
        st = L.blk_forward(handle_run.block.h, io, r.block.w, None,
                           torch.cuda.current_stream().cuda_stream)
        assert st == L.BLK_OK, L.blk_last_error()
        cur = y
    torch.cuda.synchronize()
    return cur


def test_forward_layers_f32_against_the_oracle_chain():
    """Three blocks with their own weights in one call (the model loop):
    the same bits as three blk_forward calls, and within the float32 bar of
    the oracle applied layer after layer."""
    from transformer_decoder_block_amd import binding as L
    from tests.blockrun import host
    w = llama("llama_layers", "f32", B=2, S=45, seed=60)
    runs = [Run(w.replace(seed=60 + i)) for i in range(3)]
    y = torch.empty_like(runs[0].xd)
    assert _layers_call(runs[0], runs, runs[0].xd, y) == L.BLK_OK, L.blk_last_error()
    assert torch.equal(y, _one_by_one(runs[0], runs, runs[0].xd))
    cfg = w.as_dict()
    for b in range(w.B):
        h = runs[0].x64()[b]
        for r in runs:
            h = ob.block_forward(h, None, r.W64, cfg)["layer_output"]
        assert rel_err(host(y[b]), h) <= F32_BAR


@pytest.mark.parametrize("n", [1, 2])
def test_forward_layers_bf16_matches_single_calls(n):
    """bf16 stacks of one and two layers (two: the first layer's output goes
    through the handle's buffer) give the bits of successive blk_forward
    calls, whose parity the other tests establish."""
    from transformer_decoder_block_amd import binding as L
    w = afmoe("afmoe_layers", "bf16", B=2, S=40, seed=61)
    runs = [Run(w.replace(seed=61 + i)) for i in range(n)]
    y = torch.empty_like(runs[0].xd)
    assert _layers_call(runs[0], runs, runs[0].xd, y) == L.BLK_OK, L.blk_last_error()
    assert torch.equal(y, _one_by_one(runs[0], runs, runs[0].xd))


def test_forward_layers_mask_applies_to_every_layer():
    """A padded batch through a three-layer bf16 stack: the same bits as
    three single calls with the same mask, and a stack with the mask
    differs from one without it in the padded sequence only."""
    from transformer_decoder_block_amd import binding as L
    w = llama("llama_layers_pad", "bf16", B=2, S=48, pad=9, seed=64)
    runs = [Run(w.replace(seed=64 + i)) for i in range(3)]
    assert runs[0].maskd is not None
    y = torch.empty_like(runs[0].xd)
    assert _layers_call(runs[0], runs, runs[0].xd, y) == L.BLK_OK, L.blk_last_error()
    assert torch.equal(y, _one_by_one(runs[0], runs, runs[0].xd))
    # without the mask the unpadded first sequence is unchanged, the
    # padded second one is not
    saved, runs[0].maskd = runs[0].maskd, None
    y_nomask = torch.empty_like(y)
    assert _layers_call(runs[0], runs, runs[0].xd, y_nomask) == L.BLK_OK
    runs[0].maskd = saved
    assert torch.equal(y[0], y_nomask[0])
    assert not torch.equal(y[1], y_nomask[1])


def test_forward_layers_errors_enqueue_nothing():
    """n_layers < 1, a NULL layer, and a misaligned weight of a later layer
    are refused before anything runs: y keeps its contents."""
    import ctypes as C
    from transformer_decoder_block_amd import binding as L
    w = llama("llama_layers_err", "bf16", B=1, S=16, seed=62)
    r0, r1 = Run(w), Run(w.replace(seed=63))
    y = torch.full_like(r0.xd, 7.0)
    io = L.blk_io(x=r0.xd.data_ptr(), attention_mask=None, batch=w.B, seq=w.S,
                  y=y.data_ptr())
    lib = L.load()
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    arr = (C.POINTER(L.blk_weights) * 2)(C.pointer(r0.block.w), C.pointer(r1.block.w))
    assert lib.blk_forward_layers(r0.block.h, C.byref(io), arr, 0, stream) == L.BLK_E_CONFIG
    arr[1] = C.POINTER(L.blk_weights)()
    assert lib.blk_forward_layers(r0.block.h, C.byref(io), arr, 2, stream) == L.BLK_E_NULL
    bad = L.blk_weights()
    C.memmove(C.addressof(bad), C.addressof(r1.block.w), C.sizeof(bad))
    bad.wq = r1.block.w.wq + 2
    arr[1] = C.pointer(bad)
    assert lib.blk_forward_layers(r0.block.h, C.byref(io), arr, 2, stream) == L.BLK_E_ALIGN
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_small_grid_k_split(dtype):
    """40 tokens, hidden 1024, MLP width 2000: o_proj, the up projection
    (SwiGLU pairs in the fixup) and the down projection (ragged K = 2000)
    each fill a handful of tiles with >= 16 K stages, so every tile runs as
    several K parts added by the fixup in a fixed order."""
    w = llama("llama_ksplit", dtype, B=1, S=40, H=1024, nh=8, nkv=2, hd=128, I=2000,
              seed=45)
    CHECK[dtype](Run(w))


def test_persistent_gemm_single_stage_tiles():
    """The MLP up projection at 4096 tokens and width 2104 is 16 x 17 = 272
    tiles of 256 x 256 with a single K stage (hidden 64): the persistent
    launch gives 16 of the 256 workgroups a second tile, whose first (and
    only) stage is loaded during the first tile's only stage."""
    w = llama("llama_pers", "bf16", B=1, S=4096, H=64, nh=1, nkv=1, hd=64, I=2104)
    check_bf16(Run(w))


def test_persistent_grouped_gemm():
    """Expert gate/up at 4096 (token, slot) pairs and expert width 2048 is
    at least 16 x 16 tiles of 256 x 256: the grouped GEMM runs persistent,
    its tiles found through the per-expert prefix sums."""
    w = afmoe("afmoe_pers", "bf16", B=1, S=512, E=8, top_k=8, I_e=2048, window=0,
              head_gate=0)
    check_bf16(Run(w))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_window_at_head_dim_128(dtype):
    """A sliding window with 128-wide heads and grouped queries (the
    windowed workloads use 64-wide heads): window edges fall inside key
    tiles and inside a workgroup's query block."""
    w = llama("llama_w_hd128", dtype, B=2, S=333, H=512, nh=4, nkv=2, hd=128, I=512,
              window=100, seed=44)
    CHECK[dtype](Run(w))


def test_f32_at_larger_size():
    """The float32 path beyond the small shapes: 2048 tokens, hidden 2048,
    16 heads of 128 and MLP width 5504, end to end at the float32 bar on
    sampled rows (first and last tokens, tile edges, random rows)."""
    w = llama("llama_f32_big", "f32", B=1, S=2048, H=2048, nh=16, nkv=4, hd=128, I=5504,
              seed=45)
    run = Run(w)
    out = run.forward(["layer_mid", "layer_output", "attention_norm_output"])
    rows = np.array(sorted({0, 1, 63, 64, 127, 128, 1023, 1024, 2046, 2047} |
                           set(np.random.default_rng(7).integers(0, 2048, 6).tolist())))
    r = ob.block_forward(run.x64()[0], None, run.W64, w.as_dict(), rows)
    assert rel_err(out["attention_norm_output"][0][rows], r["attention_norm_output"]) <= F32_BAR
    assert rel_err(out["layer_mid"][0][rows], r["layer_mid"]) <= F32_BAR
    assert rel_err(out["layer_output"][0][rows], r["layer_output"]) <= F32_BAR
    assert rel_err(out["y"][0][rows], r["layer_output"]) <= F32_BAR


def test_create_reports_oom_and_recovers():
    """A workspace larger than the free device memory: blk_create returns
    BLK_E_OOM with a message and no handle, and the library (and the
    device) work normally once the memory is back.  The condition is made
    from the host: all but 2 GiB of the device is held by a plain tensor."""
    from transformer_decoder_block_amd import binding as L
    w = synth.WORKLOADS["llama7b_bf16"]
    cfg = L.make_config(w, max_batch=4, max_seq=16384)  # ~6.5 GB of workspace
    torch.cuda.empty_cache()
    free, _ = torch.cuda.mem_get_info()
    hog = torch.empty(free - (2 << 30), dtype=torch.uint8, device="cuda")
    try:
        st, h = L.blk_create(cfg)
        assert st == L.BLK_E_OOM, L.blk_status_str(st)
        assert not h
        assert "hipMalloc" in L.blk_last_error()
    finally:
        del hog
        torch.cuda.empty_cache()
    st, h = L.blk_create(cfg)
    assert st == L.BLK_OK, L.blk_last_error()
    L.blk_destroy(h)
    run = Run(synth.SMALL["llama_small"])
    out = run.forward(["layer_output"])
    assert np.isfinite(out["y"]).all()
