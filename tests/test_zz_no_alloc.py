"""blk_forward_noalloc, the forward that allocates nothing, against
blk_forward on the same inputs through the C ABI: two calls in a row (the
second with a smaller batch and sequence, so the scratch array still holds
the first call's larger contents), a padded batch, the MoE path, the float32
path, and a size that does not fit, which is refused before anything is
enqueued.  Bars as in test_gpu_parity.py (float32 1e-4, bf16 2e-2 of the
RMS); the two entry points run the same kernels, so the outputs are
expected to be bit-identical, and whether they are is printed."""
import numpy as np
import pytest
import torch

from transformer_decoder_block_amd import binding as L
from transformer_decoder_block_amd import synth
from tests.blockrun import Run, host, rel_err

pytestmark = pytest.mark.gpu

BAR = {"f32": 1e-4, "bf16": 2e-2}
CASES = ["tiny_llama_f32", "llama_small", "arcee_small", "apertus_small", "afmoe_small"]


def workload(name):
    return synth.WORKLOADS.get(name) or synth.SMALL[name]


def noalloc(run, x, mask, taps=None):
    w = run.w
    B, S = int(x.shape[0]), int(x.shape[1])
    y = torch.full((B, S, w.H), float("nan"), dtype=run.tdt, device="cuda")
    io = L.blk_io(x=x.data_ptr(), attention_mask=None if mask is None else mask.data_ptr(),
                  batch=B, seq=S, y=y.data_ptr())
    st = L.blk_forward_noalloc(run.block.cfg, io, run.block.w, taps,
                               torch.cuda.current_stream().cuda_stream)
    assert st == L.BLK_OK, (L.blk_status_str(st), L.blk_last_error())
    torch.cuda.synchronize()
    return y


def compare(tag, dtype, got, ref):
    same = torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got,
                       ref.view(torch.int16) if ref.dtype == torch.bfloat16 else ref)
    e = rel_err(host(got), host(ref))
    print(f"[noalloc] {tag}: max|err|/RMS vs blk_forward {e:.3g}, bit-identical {same}",
          flush=True)
    assert e <= BAR[dtype], (tag, e)


@pytest.mark.parametrize("name", CASES)
def test_noalloc_matches_blk_forward_twice(name):
    w = workload(name)
    run = Run(w)
    # call 1: the whole batch
    ref1 = run.forward(on_device=True)["y_raw"].clone()
    got1 = noalloc(run, run.xd, run.maskd)
    compare(f"{name} call 1 ({w.B}x{w.S})", w.dtype, got1, ref1)
    # call 2, right after: one sequence, a shorter length
    S2 = max(1, w.S // 2 + 3)
    x2 = run.xd[-1:, :S2].contiguous()
    m2 = None if run.maskd is None else run.maskd[-1:, :S2].contiguous()
    ref2 = run.forward(x=x2, mask=m2, on_device=True)["y_raw"].clone()
    got2 = noalloc(run, x2, m2)
    compare(f"{name} call 2 (1x{S2})", w.dtype, got2, ref2)


def test_noalloc_taps_and_refusal():
    w = synth.SMALL["afmoe_small"]
    run = Run(w)
    ref = run.forward(["layer_mid", "expert_indices"], on_device=True)
    taps = L.blk_taps()
    mid = torch.empty((w.B, w.S, w.H), dtype=torch.float32, device="cuda")
    idx = torch.empty((w.B, w.S, w.top_k), dtype=torch.int32, device="cuda")
    taps.layer_mid = L.blk_tap(ptr=mid.data_ptr(), dtype=L.BLK_F32)
    taps.expert_indices = L.blk_tap(ptr=idx.data_ptr(), dtype=L.BLK_I32)
    y = noalloc(run, run.xd, run.maskd, taps)
    compare("afmoe_small with taps", "bf16", y, ref["y_raw"])
    assert torch.equal(idx, ref["expert_indices"])
    assert rel_err(host(mid), host(ref["layer_mid"])) <= 1e-6
    # a batch and sequence whose workspace exceeds the scratch array: refused
    # before any launch, y untouched
    y = torch.full((w.B, w.S, w.H), 7.0, dtype=torch.bfloat16, device="cuda")
    io = L.blk_io(x=run.xd.data_ptr(), attention_mask=None, batch=64, seq=8192,
                  y=y.data_ptr())
    st = L.blk_forward_noalloc(run.block.cfg, io, run.block.w, None,
                               torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == L.BLK_E_SHAPE, L.blk_status_str(st)
    assert "bytes of workspace" in L.blk_last_error()
    assert torch.all(y == 7.0)
    # and a call that fits still works after the refusal
    y = noalloc(run, run.xd, run.maskd)
    compare("afmoe_small after a refusal", "bf16", y, ref["y_raw"])
