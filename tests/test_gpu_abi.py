"""Forward-time validation of the C ABI: every error is returned before
any launch, so the output buffer is left untouched."""
import ctypes as C

import pytest
import torch

from transformer_decoder_block_amd import binding as L
from transformer_decoder_block_amd import synth
from tests.blockrun import Run

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def run():
    return Run(synth.SMALL["llama_small"])


def call(run, x=None, y=None, B=None, S=None, weights=None, taps=None):
    w = run.w
    x = run.xd if x is None else x
    io = L.blk_io(x=x if isinstance(x, int) else x.data_ptr(), attention_mask=None,
                  batch=w.B if B is None else B, seq=w.S if S is None else S,
                  y=y if isinstance(y, int) else y.data_ptr())
    st = L.blk_forward(run.block.h, io, weights or run.block.w, taps,
                       torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return st


def sentinel(run):
    return torch.full((run.w.B, run.w.S, run.w.H), 7.0, dtype=torch.bfloat16, device="cuda")


def test_ok_then_errors_leave_y_untouched(run):
    y = sentinel(run)
    assert call(run, y=y) == L.BLK_OK
    assert not torch.all(y == 7.0)
    cases = []
    y = sentinel(run)
    cases.append((call(run, y=y, B=run.w.B + 1), L.BLK_E_SHAPE))
    cases.append((call(run, y=y, S=run.w.S + 1), L.BLK_E_SHAPE))
    cases.append((call(run, y=y, S=0), L.BLK_E_SHAPE))
    cases.append((call(run, x=run.xd.data_ptr() + 2, y=y), L.BLK_E_ALIGN))
    cases.append((call(run, x=run.xd, y=run.xd), L.BLK_E_CONFIG))
    w = L.blk_weights()
    C.memmove(C.addressof(w), C.addressof(run.block.w), C.sizeof(w))
    w.wk = None
    cases.append((call(run, y=y, weights=w), L.BLK_E_NULL))
    w.wk = run.block.w.wk
    w.w_down = run.block.w.w_down + 2
    cases.append((call(run, y=y, weights=w), L.BLK_E_ALIGN))
    t = L.blk_taps()
    buf = torch.empty((run.w.B, run.w.S, run.w.H), dtype=torch.float32, device="cuda")
    t.layer_mid = L.blk_tap(ptr=buf.data_ptr(), dtype=L.BLK_BF16)
    cases.append((call(run, y=y, taps=t), L.BLK_E_DTYPE))
    t = L.blk_taps()
    t.router_logits = L.blk_tap(ptr=buf.data_ptr(), dtype=L.BLK_BF16)
    cases.append((call(run, y=y, taps=t), L.BLK_E_CONFIG))
    for got, want in cases:
        assert got == want, (L.blk_status_str(got), L.blk_status_str(want), L.blk_last_error())
    assert torch.all(y == 7.0)


def test_profile_spans(run):
    assert L.blk_profile_begin(run.block.h, 3) == L.BLK_OK
    for _ in range(2):
        run.forward()
    prof = L.blk_profile_end(run.block.h)
    names = [p[0] for p in prof]
    assert names == ["rmsnorm_in", "gemm_qkv", "attention", "gemm_o", "rmsnorm_mlp",
                     "gemm_up", "gemm_down"]
    assert all(p[2] == 2 and p[1] > 0 for p in prof)
    assert L.blk_profile_end(run.block.h) is None


def test_two_handles_on_two_streams():
    """Each handle owns its workspace, so handles on different streams may
    run at the same time: a dense and a mixture block, and a second handle
    of the dense configuration with other weights, each enqueued eight times
    on its own stream without a synchronisation in between, give outputs bit
    for bit equal to their one-at-a-time forwards."""
    runs = [Run(synth.SMALL["llama_small"]), Run(synth.SMALL["afmoe_small"]),
            Run(synth.SMALL["llama_small"].replace(seed=77))]
    ref = [r.forward()["y_raw"].clone() for r in runs]
    streams = [torch.cuda.Stream() for _ in runs]
    ys = [torch.full_like(t, float("nan")) for t in ref]
    torch.cuda.synchronize()
    for _ in range(8):
        for r, s, y in zip(runs, streams, ys):
            r.block.forward(r.xd, y, r.maskd, None, stream=s)
    torch.cuda.synchronize()
    for r, y, y0 in zip(runs, ys, ref):
        assert torch.equal(y.view(torch.int16), y0.view(torch.int16)), r.w.name
