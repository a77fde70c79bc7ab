"""Helpers shared by the GPU tests: move a seeded workload to the device,
run libblock through its C ABI with taps, and bring the taps back as the
exact float64 images of what the kernels wrote."""
from __future__ import annotations

import numpy as np
import torch

from transformer_decoder_block_amd import binding as L
from transformer_decoder_block_amd import synth


def dev(a, dtype):
    """Stored numpy array -> device tensor (bf16 from its bit patterns)."""
    if isinstance(a, float):
        return a
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    """Device tensor -> float64 numpy (exact)."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        u = t.view(torch.int16).cpu().numpy().view(np.uint16)
        return synth.bf16_bits_to_f64(u)
    return t.cpu().numpy().astype(np.float64)


class Run:
    """Inputs of one workload on host and device, plus a libblock handle."""

    def __init__(self, w: synth.Workload, max_batch=None, max_seq=None):
        self.w = w
        self.Wst = synth.make_weights(w)
        self.xst = synth.make_x(w)
        self.mask = synth.make_mask(w)
        self.tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        self.mdt = L.BLK_BF16 if w.dtype == "bf16" else L.BLK_F32
        self.Wd = {k: dev(v, w.dtype) for k, v in self.Wst.items()}
        self.xd = dev(self.xst, w.dtype)
        self.maskd = None if self.mask is None else torch.from_numpy(self.mask).cuda()
        self.block = L.Block(L.make_config(w, max_batch, max_seq), self.Wd)
        self._W64 = None

    @property
    def W64(self):
        if self._W64 is None:
            self._W64 = synth.weights_f64(self.w, self.Wst)
        return self._W64

    def x64(self):
        return synth.to_f64(self.xst, self.w.dtype)

    def forward(self, taps=(), x=None, mask="same", on_device=False, guard=False):
        """Run once; returns dict of float64 numpy arrays (y and taps), or
        of the device tensors themselves when on_device.  With guard, y and
        every tap sit between GUARD canary elements on each side, which must
        be unchanged after the call (else AssertionError naming the buffer)."""
        w = self.w
        x = self.xd if x is None else x
        B, S = int(x.shape[0]), int(x.shape[1])
        m = self.maskd if isinstance(mask, str) else mask
        guarded = {}
        if guard:
            y = guarded_empty((B, S, w.H), self.tdt, "y", guarded)
        else:
            y = torch.empty((B, S, w.H), dtype=self.tdt, device="cuda")
        shapes = {
            "layer_input": ((B, S, w.H), self.tdt, self.mdt),
            "attention_norm_output": ((B, S, w.H), self.tdt, self.mdt),
            "attention_scores": ((B, w.nh, S, S), torch.float32, L.BLK_F32),
            "layer_mid": ((B, S, w.H), torch.float32, L.BLK_F32),
            "mlp_input": ((B, S, w.H), self.tdt, self.mdt),
            "layer_output": ((B, S, w.H), torch.float32, L.BLK_F32),
            "attention_output": ((B, S, w.H), torch.float32, L.BLK_F32),
            "mlp_output": ((B, S, w.H), torch.float32, L.BLK_F32),
            "router_logits": ((B, S, w.E), self.tdt, self.mdt),
            "expert_indices": ((B, S, w.top_k), torch.int32, L.BLK_I32),
            "expert_weights": ((B, S, w.top_k), torch.float32, L.BLK_F32),
            "attention_queries": ((B, w.nh, S, w.hd), self.tdt, self.mdt),
            "attention_keys": ((B, w.nkv, S, w.hd), self.tdt, self.mdt),
            "attention_values": ((B, w.nkv, S, w.hd), self.tdt, self.mdt),
            "attention_probabilities": ((B, w.nh, S, S), torch.float32, L.BLK_F32),
            "attention_head_outputs": ((B, S, w.nh, w.hd), self.tdt, self.mdt),
            "attention_premix": ((B, S, w.nh * w.hd), self.tdt, self.mdt),
            "mlp_neurons": ((B, S, w.I), self.tdt, self.mdt),
            "mlp_activation": ((B, S, w.I), self.tdt, self.mdt),
            "mlp_norm_output": ((B, S, w.H), self.tdt, self.mdt),
            "expert_outputs": ((B, S, w.top_k, w.H), self.tdt, self.mdt),
            "routed_output": ((B, S, w.H), torch.float32, L.BLK_F32),
            "shared_expert_output": ((B, S, w.H), torch.float32, L.BLK_F32),
        }
        tapt = {}
        for n in taps:
            shp, tdt, bdt = shapes[n]
            if guard:
                tapt[n] = (guarded_empty(shp, tdt, n, guarded), bdt)
            else:
                tapt[n] = (torch.full(shp, float("nan"), dtype=tdt, device="cuda")
                           if tdt != torch.int32 else
                           torch.full(shp, -1, dtype=tdt, device="cuda"), bdt)
        self.block.forward(x, y, m, tapt)
        torch.cuda.synchronize()
        if guard:
            check_guards(guarded)
        if on_device:
            out = {n: t for n, (t, _) in tapt.items()}
            out["y_raw"] = y
            return out
        out = {"y": host(y), "y_raw": y}
        for n, (t, _) in tapt.items():
            out[n] = t.cpu().numpy() if t.dtype == torch.int32 else host(t)
        return out


# Canary words around output buffers: GUARD elements on each side (a
# multiple of 16 bytes for every element size, so the buffer itself stays
# 16-byte aligned), filled with a NaN pattern no kernel computes.
GUARD = 64
_CANARY = {torch.float32: (torch.int32, 0x7FA5A5A5), torch.bfloat16: (torch.int16, 0x7FA5),
           torch.int32: (torch.int32, 0x5A5A5A5A)}


def guarded_empty(shape, dtype, name, registry):
    """A contiguous device tensor of `shape` inside a buffer with GUARD
    canary elements before and after it; the buffer is kept in registry."""
    n = 1
    for d in shape:
        n *= d
    idt, word = _CANARY[dtype]
    buf = torch.full((n + 2 * GUARD,), word, dtype=idt, device="cuda")
    registry[name] = (buf, n, word)
    return buf.view(dtype)[GUARD:GUARD + n].view(shape)


def check_guards(registry):
    """Every canary word is still in place."""
    bad = []
    for name, (buf, n, word) in registry.items():
        head, tail = buf[:GUARD], buf[GUARD + n:]
        if not (bool((head == word).all()) and bool((tail == word).all())):
            bad.append(name)
    assert not bad, f"writes past the ends of: {bad}"


def rel_err(got, ref):
    """max |got - ref| / RMS(ref), over finite reference entries."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    fin = np.isfinite(ref)
    rms = np.sqrt(np.mean(ref[fin] ** 2))
    return float(np.max(np.abs(got[fin] - ref[fin])) / rms)
