"""Capture of a forward in a HIP graph.

blk_forward without taps only enqueues kernels on the caller's stream (no
memset, copy, allocation or synchronisation), so a caller may capture it
into a graph and replay it.  Each test captures on torch's capture stream,
replays several times with eager work and synchronisations in between, and
checks every replay bit for bit against the eager result.
"""
import pytest
import torch

from tests.blockrun import Run
from tests.test_gpu_edges import afmoe, llama
from transformer_decoder_block_amd import binding as L

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _replays_match(run, capture, y, eager):
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        capture()
    torch.cuda.synchronize()
    for i in range(REPLAYS):
        y.fill_(float("nan"))
        # eager work between replays, as a program would do
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager), f"replay {i}"
        del junk


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forward_in_a_graph(dtype):
    """A padded llama block (dense GEMMs, attention with a mask) and its
    eager result."""
    w = llama("llama_graph", dtype, B=2, S=77, pad=11, seed=70)
    run = Run(w)
    eager = run.forward(on_device=True)["y_raw"].clone()
    y = torch.empty_like(eager)

    def capture():
        run.block.forward(run.xd, y, run.maskd, None)

    _replays_match(run, capture, y, eager)


def test_moe_forward_in_a_graph():
    """The mixture: router, top-k, the dispatch's counts and scans, the
    grouped GEMMs and the combine, all recorded as kernels."""
    w = afmoe("afmoe_graph", "bf16", B=2, S=64, seed=71)
    run = Run(w)
    eager = run.forward(on_device=True)["y_raw"].clone()
    y = torch.empty_like(eager)

    def capture():
        run.block.forward(run.xd, y, run.maskd, None)

    _replays_match(run, capture, y, eager)


def test_stack_in_a_graph():
    """blk_forward_layers (two layers through the handle's buffer)."""
    w = llama("llama_graph_stack", "bf16", B=1, S=50, seed=72)
    runs = [Run(w), Run(w.replace(seed=73))]
    h = runs[0]
    y = torch.empty_like(h.xd)
    io = L.blk_io(x=h.xd.data_ptr(), attention_mask=None, batch=w.B, seq=w.S,
                  y=y.data_ptr())
    layers = [r.block.w for r in runs]
    st = L.blk_forward_layers(h.block.h, io, layers, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == L.BLK_OK, L.blk_last_error()
    eager = y.clone()

    def capture():
        s = L.blk_forward_layers(h.block.h, io, layers,
                                 torch.cuda.current_stream().cuda_stream)
        assert s == L.BLK_OK, L.blk_last_error()

    _replays_match(h, capture, y, eager)
