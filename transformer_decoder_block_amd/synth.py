"""Seeded synthetic inputs and the named workloads of the block.

This module holds shapes and random numbers only: no step of the block's
arithmetic lives here.  Both the HIP path's callers (tests, bench) and the
oracle's callers take their inputs from it, so the two sides see the same
bytes.

Recipe (every tensor):
  * generator: ``numpy.random.default_rng([seed, tensor_index, chunk])``,
    tensor_index from TENSOR_ORDER; a tensor is drawn flattened (row-major)
    in consecutive chunks of 2^20 elements, chunk = the chunk's index (the
    chunks are independent streams, so they are drawn in parallel);
  * z = standard normal drawn as float32; value = fp32(mean + std * z)
    (computed in float64, rounded once to float32); for bf16 workloads the
    stored value is that float32 rounded to bfloat16 (nearest, ties to even);
  * distributions (std, not variance): projection/router/expert weights
    N(0, 0.02); residual input N(0, 1); norm gains N(1, 0.05), or exactly 1
    where a workload says so; expert selection bias N(0, 0.1) stored in
    float32; the two xIELU raw scalars U[0.5, 1);
  * attention_mask: all ones, except that on the second half of the batch
    (b >= B - B//2) the last ``pad`` positions are 0.
"""
from __future__ import annotations

import dataclasses
import os
from dataclasses import dataclass, field

import numpy as np

TENSOR_ORDER = [
    "x", "w_in_norm", "w_post_attn_norm", "w_mlp_norm", "w_post_mlp_norm",
    "w_q_norm", "w_k_norm", "wq", "wk", "wv", "w_head_gate", "wo",
    "w_router", "expert_bias", "w_gate", "w_up", "w_down",
    "w_e_gate", "w_e_up", "w_e_down", "w_sh_gate", "w_sh_up", "w_sh_down",
    "xielu_alpha_p", "xielu_alpha_n",
]


@dataclass
class Workload:
    """Shape and feature flags of one block workload."""
    name: str
    dtype: str            # "f32" or "bf16"
    B: int
    S: int
    H: int
    nh: int
    nkv: int
    hd: int
    mlp: str              # "swiglu" | "relu2" | "xielu" | "moe"
    I: int = 0            # dense MLP width
    eps: float = 1e-5
    theta: float = 10000.0
    qk_norm: bool = False
    sandwich: bool = False
    window: int = 0       # 0 = full causal
    head_gate: int = 0    # 0, nh (per head) or nh*hd (per channel)
    use_rope: bool = True
    E: int = 0
    top_k: int = 0
    I_e: int = 0
    n_shared: int = 0
    route_scale: float = 1.0
    xielu_beta: float = 0.5
    xielu_eps: float = -1e-6
    pad: int = 0          # trailing padded tokens on the second half of the batch
    unit_gains: bool = False
    seed: int = 0

    @property
    def T(self):
        return self.B * self.S

    @property
    def I_sh(self):
        return self.I_e * self.n_shared

    def as_dict(self):
        return dataclasses.asdict(self)

    def replace(self, **kw):
        return dataclasses.replace(self, **kw)


# The five workloads of the block, in the order they are named.
WORKLOADS = {
    "tiny_llama_f32": Workload(
        "tiny_llama_f32", "f32", B=1, S=64, H=256, nh=4, nkv=2, hd=64,
        mlp="swiglu", I=688, unit_gains=True, seed=1),
    "llama7b_bf16": Workload(
        "llama7b_bf16", "bf16", B=4, S=2048, H=4096, nh=32, nkv=32, hd=128,
        mlp="swiglu", I=10928, seed=2),
    "arcee_gqa_bf16": Workload(
        "arcee_gqa_bf16", "bf16", B=4, S=4096, H=2560, nh=20, nkv=4, hd=128,
        mlp="relu2", I=18432, pad=256, seed=3),
    "apertus_bf16": Workload(
        "apertus_bf16", "bf16", B=2, S=4096, H=4096, nh=32, nkv=8, hd=128,
        mlp="xielu", I=21504, qk_norm=True, seed=4),
    "afmoe_bf16": Workload(
        "afmoe_bf16", "bf16", B=2, S=8192, H=2048, nh=32, nkv=4, hd=64,
        mlp="moe", qk_norm=True, sandwich=True, window=2048, head_gate=32,
        E=64, top_k=8, I_e=1024, n_shared=1, route_scale=2.826, seed=5),
}

# The NEXT rows at full size, on the afmoe page's Nano shapes (hidden 1024,
# 8 query heads over 2 of 128, a per-channel head gate 1024 -> 1024, q/k
# norms, sandwich norms), at the token count of the AFMoE workload:
#   * the mixture block (128 routed experts of width 256, 8 per token, one
#     shared expert), a sliding-window block with the rotary;
#   * the same block as a global one (whole causal prefix, no rotary);
#   * a dense-first block (a dense SwiGLU of width 3072).
NEXT = {
    "trinity_nano_moe_bf16": Workload(
        "trinity_nano_moe_bf16", "bf16", B=2, S=8192, H=1024, nh=8, nkv=2, hd=128,
        mlp="moe", qk_norm=True, sandwich=True, window=2048, head_gate=1024,
        E=128, top_k=8, I_e=256, n_shared=1, route_scale=2.826, seed=7),
    "trinity_nano_global_bf16": Workload(
        "trinity_nano_global_bf16", "bf16", B=2, S=8192, H=1024, nh=8, nkv=2,
        hd=128, mlp="moe", qk_norm=True, sandwich=True, window=0, use_rope=False,
        head_gate=1024, E=128, top_k=8, I_e=256, n_shared=1, route_scale=2.826,
        seed=8),
    "trinity_nano_dense_bf16": Workload(
        "trinity_nano_dense_bf16", "bf16", B=2, S=8192, H=1024, nh=8, nkv=2,
        hd=128, mlp="swiglu", I=3072, qk_norm=True, sandwich=True, window=2048,
        head_gate=1024, seed=9),
}


def workload(name: str) -> Workload:
    """A named workload: the five of the block, or a NEXT-row shape."""
    if name in WORKLOADS:
        return WORKLOADS[name]
    if name in NEXT:
        return NEXT[name]
    raise KeyError(f"unknown workload {name}")


# Small shapes of every family that the oracle finishes in seconds; each
# spans several GEMM/attention tiles and ends in a ragged tail.
SMALL = {
    "llama_small": Workload(
        "llama_small", "bf16", B=2, S=200, H=384, nh=6, nkv=2, hd=64,
        mlp="swiglu", I=688, seed=11),
    "arcee_small": Workload(
        "arcee_small", "bf16", B=2, S=300, H=320, nh=5, nkv=1, hd=64,
        mlp="relu2", I=1000, pad=37, seed=12),
    "apertus_small": Workload(
        "apertus_small", "bf16", B=2, S=260, H=512, nh=4, nkv=2, hd=128,
        mlp="xielu", I=1040, qk_norm=True, seed=13),
    "afmoe_small": Workload(
        "afmoe_small", "bf16", B=2, S=300, H=256, nh=8, nkv=2, hd=64,
        mlp="moe", qk_norm=True, sandwich=True, window=64, head_gate=8,
        E=8, top_k=2, I_e=192, n_shared=1, route_scale=2.826, seed=14),
    "afmoe_global_dense_small": Workload(
        "afmoe_global_dense_small", "bf16", B=2, S=150, H=256, nh=4, nkv=2,
        hd=64, mlp="swiglu", I=520, qk_norm=True, sandwich=True, window=0,
        head_gate=4, use_rope=False, seed=15),
    "afmoe_channel_gate_small": Workload(
        "afmoe_channel_gate_small", "bf16", B=1, S=130, H=256, nh=4, nkv=1,
        hd=64, mlp="moe", qk_norm=True, sandwich=True, window=48,
        head_gate=256, E=16, top_k=8, I_e=256, n_shared=1,
        route_scale=2.826, seed=16),
}


def f32_variant(w: Workload) -> Workload:
    return w.replace(name=w.name + "_f32", dtype="f32")


# --------------------------------------------------------------------------
# storage formats
# --------------------------------------------------------------------------

def f32_to_bf16_bits(a):
    """float32 array -> uint16 bfloat16 bit patterns (nearest, ties even)."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (r >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f64(b):
    b = np.ascontiguousarray(b, np.uint16)
    out = np.empty(b.shape, np.float64)
    fb, fo = b.reshape(-1), out.reshape(-1)

    def conv(c):
        lo, hi = c * CHUNK, min(fb.size, (c + 1) * CHUNK)
        u = fb[lo:hi].astype(np.uint32) << np.uint32(16)
        fo[lo:hi] = u.view(np.float32)

    n = (fb.size + CHUNK - 1) // CHUNK
    if n <= 1:
        conv(0) if fb.size else None
    else:
        list(_pool().map(conv, range(n)))
    return out


def to_f64(a, dtype):
    """The exact float64 image of a stored array."""
    if dtype == "bf16" and a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return np.asarray(a, np.float64)


CHUNK = 1 << 20
_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        from concurrent.futures import ThreadPoolExecutor
        n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else 4
        _POOL = ThreadPoolExecutor(max(1, min(16, n)))
    return _POOL


def _normal_stored(seed, idx, shape, mean, std, dtype):
    """The stored values of one N(mean, std) tensor (see the module recipe)."""
    n = int(np.prod(shape))
    out = np.empty(n, np.uint16 if dtype == "bf16" else np.float32)

    def fill(c):
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        rng = np.random.default_rng([seed, idx, c])
        z = rng.standard_normal(hi - lo, dtype=np.float32)
        v = (z.astype(np.float64) * std + mean).astype(np.float32)
        out[lo:hi] = f32_to_bf16_bits(v) if dtype == "bf16" else v

    list(_pool().map(fill, range((n + CHUNK - 1) // CHUNK)))
    return out.reshape(shape)


def _store(v32, dtype):
    return f32_to_bf16_bits(v32) if dtype == "bf16" else v32


def weight_shapes(w: Workload):
    """Name -> shape of every weight the workload uses ([out, in] layout)."""
    H, nh, nkv, hd = w.H, w.nh, w.nkv, w.hd
    s = {
        "w_in_norm": (H,), "w_mlp_norm": (H,),
        "wq": (nh * hd, H), "wk": (nkv * hd, H), "wv": (nkv * hd, H),
        "wo": (H, nh * hd),
    }
    if w.sandwich:
        s["w_post_attn_norm"] = (H,)
        s["w_post_mlp_norm"] = (H,)
    if w.qk_norm:
        s["w_q_norm"] = (hd,)
        s["w_k_norm"] = (hd,)
    if w.head_gate:
        s["w_head_gate"] = (w.head_gate, H)
    if w.mlp == "swiglu":
        s.update(w_gate=(w.I, H), w_up=(w.I, H), w_down=(H, w.I))
    elif w.mlp in ("relu2", "xielu"):
        s.update(w_up=(w.I, H), w_down=(H, w.I))
    elif w.mlp == "moe":
        s.update(w_router=(w.E, H), expert_bias=(w.E,),
                 w_e_gate=(w.E, w.I_e, H), w_e_up=(w.E, w.I_e, H),
                 w_e_down=(w.E, H, w.I_e),
                 w_sh_gate=(w.I_sh, H), w_sh_up=(w.I_sh, H),
                 w_sh_down=(H, w.I_sh))
    if w.mlp == "xielu":
        s.update(xielu_alpha_p=(), xielu_alpha_n=())
    return s


def make_weights(w: Workload):
    """Dict name -> stored array (uint16 bf16 bits or float32; expert_bias is
    always float32; the xIELU raw scalars are Python floats)."""
    out = {}
    for name, shape in weight_shapes(w).items():
        idx = TENSOR_ORDER.index(name)
        if name in ("xielu_alpha_p", "xielu_alpha_n"):
            rng = np.random.default_rng([w.seed, idx, 0])
            out[name] = float(np.float32(rng.uniform(0.5, 1.0)))
            continue
        if name == "expert_bias":
            out[name] = _normal_stored(w.seed, idx, shape, 0.0, 0.1, "f32")
            continue
        if name.startswith("w_") and name.endswith("norm"):
            if w.unit_gains:
                out[name] = _store(np.ones(shape, np.float32), w.dtype)
            else:
                out[name] = _normal_stored(w.seed, idx, shape, 1.0, 0.05, w.dtype)
            continue
        out[name] = _normal_stored(w.seed, idx, shape, 0.0, 0.02, w.dtype)
    return out


def make_x(w: Workload):
    """layer_input [B, S, H] in storage format."""
    idx = TENSOR_ORDER.index("x")
    return _normal_stored(w.seed, idx, (w.B, w.S, w.H), 0.0, 1.0, w.dtype)


def make_mask(w: Workload):
    """attention_mask [B, S] int32, or None when nothing is padded."""
    if not w.pad:
        return None
    m = np.ones((w.B, w.S), np.int32)
    m[w.B - w.B // 2:, w.S - w.pad:] = 0
    return m


def weights_f64(w: Workload, W):
    """The float64 images of every stored weight, as the oracle takes them."""
    out = {}
    for k, v in W.items():
        if isinstance(v, float):
            out[k] = v
        elif k == "expert_bias":
            out[k] = np.asarray(v, np.float64)
        else:
            out[k] = to_f64(v, w.dtype)
    return out
