"""ctypes binding of libblock (include/libblock.h), argument marshalling only.

The names mirror the C ABI: ``blk_create``, ``blk_forward``,
``blk_forward_layers``, ``blk_forward_noalloc``, ``blk_destroy``,
``blk_status_str``, ``blk_last_error``, ``blk_abi_version``,
``blk_workspace_bytes``, and the structs ``blk_config``, ``blk_weights``,
``blk_tap``, ``blk_taps``, ``blk_io``.  ``Block`` is a small convenience
wrapper that fills those structs from torch tensors (PyTorch supplies device
memory and the stream; every step of the block runs in libblock's kernels).

Loading fails loudly if libblock.so has not been built: there is no other
implementation behind these names.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libblock.so")

BLK_OK, BLK_E_NULL, BLK_E_CONFIG, BLK_E_SHAPE, BLK_E_ALIGN, BLK_E_DTYPE, \
    BLK_E_OOM, BLK_E_HIP = range(8)
BLK_F32, BLK_BF16, BLK_I32 = 0, 1, 2
BLK_MLP_SWIGLU, BLK_MLP_RELU2, BLK_MLP_XIELU, BLK_MLP_MOE = 0, 1, 2, 3
MLP_KIND = {"swiglu": BLK_MLP_SWIGLU, "relu2": BLK_MLP_RELU2,
            "xielu": BLK_MLP_XIELU, "moe": BLK_MLP_MOE}


class blk_config(C.Structure):
    _fields_ = [
        ("dtype", C.c_int32), ("hidden", C.c_int32), ("num_heads", C.c_int32),
        ("num_kv_heads", C.c_int32), ("head_dim", C.c_int32),
        ("mlp_kind", C.c_int32), ("intermediate", C.c_int32),
        ("rms_eps", C.c_float), ("rope_theta", C.c_float),
        ("use_rope", C.c_int32), ("qk_norm", C.c_int32),
        ("sandwich_norm", C.c_int32), ("sliding_window", C.c_int32),
        ("head_gate_dim", C.c_int32), ("num_experts", C.c_int32),
        ("top_k", C.c_int32), ("moe_intermediate", C.c_int32),
        ("num_shared_experts", C.c_int32), ("route_scale", C.c_float),
        ("xielu_beta", C.c_float), ("xielu_eps", C.c_float),
        ("max_batch", C.c_int32), ("max_seq", C.c_int32),
    ]


WEIGHT_FIELDS = [
    "w_in_norm", "w_post_attn_norm", "w_mlp_norm", "w_post_mlp_norm",
    "wq", "wk", "wv", "wo", "w_q_norm", "w_k_norm", "w_head_gate",
    "w_gate", "w_up", "w_down",
]
WEIGHT_FIELDS_2 = ["w_router", "expert_bias", "w_e_gate", "w_e_up", "w_e_down",
                   "w_sh_gate", "w_sh_up", "w_sh_down"]


class blk_weights(C.Structure):
    _fields_ = ([(n, C.c_void_p) for n in WEIGHT_FIELDS]
                + [("xielu_alpha_p_raw", C.c_double),
                   ("xielu_alpha_n_raw", C.c_double)]
                + [(n, C.c_void_p) for n in WEIGHT_FIELDS_2])


class blk_tap(C.Structure):
    _fields_ = [("ptr", C.c_void_p), ("dtype", C.c_int32)]


TAP_NAMES = ["layer_input", "attention_norm_output", "attention_scores",
             "layer_mid", "mlp_input", "layer_output", "attention_output",
             "mlp_output", "router_logits", "expert_indices", "expert_weights",
             "attention_queries", "attention_keys", "attention_values",
             "attention_probabilities", "attention_head_outputs", "attention_premix",
             "mlp_neurons", "expert_outputs", "routed_output", "shared_expert_output",
             "mlp_activation", "mlp_norm_output"]

ABI_VERSION = 6  # the BLK_ABI_VERSION these structs mirror


class blk_taps(C.Structure):
    _fields_ = [(n, blk_tap) for n in TAP_NAMES]


class blk_io(C.Structure):
    _fields_ = [("x", C.c_void_p), ("attention_mask", C.c_void_p),
                ("batch", C.c_int32), ("seq", C.c_int32), ("y", C.c_void_p)]


class blk_handle(C.Structure):
    pass


_lib = None


def load():
    """Load libblock.so (built in-tree); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m transformer_decoder_block_amd.build`")
    lib = C.CDLL(LIB_PATH, mode=os.RTLD_NOW)  # unresolved symbols fail here
    lib.blk_abi_version.restype = C.c_int32
    if lib.blk_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{LIB_PATH} has ABI {lib.blk_abi_version()}, the binding "
                           f"mirrors {ABI_VERSION}: rebuild it")
    H = C.POINTER(blk_handle)
    lib.blk_create.argtypes = [C.POINTER(blk_config), C.POINTER(H)]
    lib.blk_create.restype = C.c_int
    lib.blk_forward.argtypes = [H, C.POINTER(blk_io), C.POINTER(blk_weights),
                                C.POINTER(blk_taps), C.c_void_p]
    lib.blk_forward.restype = C.c_int
    lib.blk_forward_layers.argtypes = [H, C.POINTER(blk_io), C.POINTER(C.POINTER(blk_weights)),
                                       C.c_int32, C.c_void_p]
    lib.blk_forward_layers.restype = C.c_int
    lib.blk_forward_noalloc.argtypes = [C.POINTER(blk_config), C.POINTER(blk_io),
                                        C.POINTER(blk_weights), C.POINTER(blk_taps),
                                        C.c_void_p]
    lib.blk_forward_noalloc.restype = C.c_int
    lib.blk_destroy.argtypes = [H]
    lib.blk_destroy.restype = None
    lib.blk_status_str.argtypes = [C.c_int]
    lib.blk_status_str.restype = C.c_char_p
    lib.blk_last_error.argtypes = []
    lib.blk_last_error.restype = C.c_char_p
    lib.blk_abi_version.argtypes = []
    lib.blk_abi_version.restype = C.c_int32
    lib.blk_workspace_bytes.argtypes = [H]
    lib.blk_workspace_bytes.restype = C.c_size_t
    lib.blk_profile_begin.argtypes = [H, C.c_int32]
    lib.blk_profile_begin.restype = C.c_int
    lib.blk_profile_end.argtypes = [H, C.c_int32, C.POINTER(C.c_char_p),
                                    C.POINTER(C.c_double), C.POINTER(C.c_int32)]
    lib.blk_profile_end.restype = C.c_int32
    _lib = lib
    return lib


def blk_create(cfg: blk_config):
    """Returns (status, handle)."""
    lib = load()
    h = C.POINTER(blk_handle)()
    st = lib.blk_create(C.byref(cfg), C.byref(h))
    return st, h


def blk_forward(h, io: blk_io, w: blk_weights, taps, stream: int):
    lib = load()
    return lib.blk_forward(h, C.byref(io), C.byref(w),
                           C.byref(taps) if taps is not None else None,
                           C.c_void_p(stream))


def blk_forward_noalloc(cfg: blk_config, io: blk_io, w: blk_weights, taps, stream: int):
    lib = load()
    return lib.blk_forward_noalloc(C.byref(cfg), C.byref(io), C.byref(w),
                                   C.byref(taps) if taps is not None else None,
                                   C.c_void_p(stream))


def blk_forward_layers(h, io: blk_io, layers, stream: int):
    """layers: a sequence of blk_weights, the first layer first."""
    lib = load()
    arr = (C.POINTER(blk_weights) * len(layers))(*[C.pointer(w) for w in layers])
    return lib.blk_forward_layers(h, C.byref(io), arr, len(layers), C.c_void_p(stream))


def blk_destroy(h):
    load().blk_destroy(h)


def blk_status_str(s: int) -> str:
    return load().blk_status_str(s).decode()


def blk_last_error() -> str:
    return load().blk_last_error().decode()


def blk_abi_version() -> int:
    return load().blk_abi_version()


def blk_workspace_bytes(h) -> int:
    return load().blk_workspace_bytes(h)


def blk_profile_begin(h, max_forwards: int) -> int:
    return load().blk_profile_begin(h, max_forwards)


def blk_profile_end(h, max_entries: int = 32):
    """Returns [(name, total_ms, forwards)] or None if profiling was off."""
    names = (C.c_char_p * max_entries)()
    tot = (C.c_double * max_entries)()
    calls = (C.c_int32 * max_entries)()
    n = load().blk_profile_end(h, max_entries, names, tot, calls)
    if n < 0:
        return None
    return [(names[i].decode(), tot[i], calls[i]) for i in range(n)]


class BlockError(RuntimeError):
    def __init__(self, status, detail):
        super().__init__(f"{blk_status_str(status)}: {detail}")
        self.status = status


def make_config(w, max_batch=None, max_seq=None) -> blk_config:
    """blk_config from a workload description (synth.Workload or dict)."""
    d = w if isinstance(w, dict) else w.as_dict()
    return blk_config(
        dtype=BLK_BF16 if d["dtype"] == "bf16" else BLK_F32,
        hidden=d["H"], num_heads=d["nh"], num_kv_heads=d["nkv"],
        head_dim=d["hd"], mlp_kind=MLP_KIND[d["mlp"]],
        intermediate=d.get("I", 0), rms_eps=d["eps"], rope_theta=d["theta"],
        use_rope=int(d["use_rope"]), qk_norm=int(d["qk_norm"]),
        sandwich_norm=int(d["sandwich"]), sliding_window=d["window"],
        head_gate_dim=d["head_gate"], num_experts=d.get("E", 0),
        top_k=d.get("top_k", 0), moe_intermediate=d.get("I_e", 0),
        num_shared_experts=d.get("n_shared", 0),
        route_scale=d.get("route_scale", 1.0),
        xielu_beta=d.get("xielu_beta", 0.5), xielu_eps=d.get("xielu_eps", -1e-6),
        max_batch=max_batch or d["B"], max_seq=max_seq or d["S"])


def _ptr(t):
    return None if t is None else t.data_ptr()


def weight_shapes(cfg: blk_config) -> dict:
    """Shape of every weight the configuration reads (name -> tuple)."""
    H, nh, nkv, hd = cfg.hidden, cfg.num_heads, cfg.num_kv_heads, cfg.head_dim
    s = {"w_in_norm": (H,), "w_mlp_norm": (H,), "wq": (nh * hd, H),
         "wk": (nkv * hd, H), "wv": (nkv * hd, H), "wo": (H, nh * hd)}
    if cfg.sandwich_norm:
        s["w_post_attn_norm"] = (H,)
        s["w_post_mlp_norm"] = (H,)
    if cfg.qk_norm:
        s["w_q_norm"] = (hd,)
        s["w_k_norm"] = (hd,)
    if cfg.head_gate_dim:
        s["w_head_gate"] = (cfg.head_gate_dim, H)
    I, k = cfg.intermediate, cfg.mlp_kind
    if k == BLK_MLP_SWIGLU:
        s["w_gate"] = (I, H)
    if k in (BLK_MLP_SWIGLU, BLK_MLP_RELU2, BLK_MLP_XIELU):
        s["w_up"] = (I, H)
        s["w_down"] = (H, I)
    if k == BLK_MLP_MOE:
        E, Ie, Ish = cfg.num_experts, cfg.moe_intermediate, \
            cfg.moe_intermediate * cfg.num_shared_experts
        s.update({"w_router": (E, H), "expert_bias": (E,), "w_e_gate": (E, Ie, H),
                  "w_e_up": (E, Ie, H), "w_e_down": (E, H, Ie)})
        if Ish:
            s.update({"w_sh_gate": (Ish, H), "w_sh_up": (Ish, H), "w_sh_down": (H, Ish)})
    return s


def tap_shapes(cfg: blk_config, B: int, S: int) -> dict:
    """Shape and blk dtype of every tap of a (B, S) call (name -> (shape, dtype))."""
    H, nh, nkv, hd, md = cfg.hidden, cfg.num_heads, cfg.num_kv_heads, cfg.head_dim, cfg.dtype
    I = cfg.intermediate
    E, k = cfg.num_experts, cfg.top_k
    return {
        "layer_input": ((B, S, H), md), "attention_norm_output": ((B, S, H), md),
        "attention_scores": ((B, nh, S, S), BLK_F32), "layer_mid": ((B, S, H), BLK_F32),
        "mlp_input": ((B, S, H), md), "layer_output": ((B, S, H), BLK_F32),
        "attention_output": ((B, S, H), BLK_F32), "mlp_output": ((B, S, H), BLK_F32),
        "router_logits": ((B, S, E), md), "expert_indices": ((B, S, k), BLK_I32),
        "expert_weights": ((B, S, k), BLK_F32),
        "attention_queries": ((B, nh, S, hd), md), "attention_keys": ((B, nkv, S, hd), md),
        "attention_values": ((B, nkv, S, hd), md),
        "attention_probabilities": ((B, nh, S, S), BLK_F32),
        "attention_head_outputs": ((B, S, nh, hd), md),
        "attention_premix": ((B, S, nh * hd), md), "mlp_neurons": ((B, S, I), md),
        "mlp_activation": ((B, S, I), md), "mlp_norm_output": ((B, S, H), md),
        "expert_outputs": ((B, S, k, H), md), "routed_output": ((B, S, H), BLK_F32),
        "shared_expert_output": ((B, S, H), BLK_F32),
    }


def _torch_dtype(blk_dt):
    import torch
    return {BLK_F32: torch.float32, BLK_BF16: torch.bfloat16, BLK_I32: torch.int32}[blk_dt]


def check_tensor(name, t, shape, blk_dt):
    """A contiguous device tensor of exactly this shape and dtype, else BlockError
    (the C ABI sees bare pointers and cannot check any of it)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise BlockError(BLK_E_NULL, f"{name} must be a torch tensor")
    if t.dtype != _torch_dtype(blk_dt):
        raise BlockError(BLK_E_DTYPE, f"{name} has dtype {t.dtype}, expected "
                                      f"{_torch_dtype(blk_dt)}")
    # the same element count in another shape ([B, S, nh, hd] for
    # [B, S, nh * hd]) addresses the same bytes
    if tuple(t.shape) != tuple(shape) and t.numel() != _numel(shape):
        raise BlockError(BLK_E_SHAPE, f"{name} has shape {tuple(t.shape)}, expected {shape}")
    if not t.is_contiguous():
        raise BlockError(BLK_E_SHAPE, f"{name} must be contiguous")
    if not t.is_cuda:
        raise BlockError(BLK_E_NULL, f"{name} must be a device tensor")


def _numel(shape):
    n = 1
    for d in shape:
        n *= d
    return n


class Block:
    """One libblock handle plus the device weights it is called with."""

    def __init__(self, cfg: blk_config, weights: dict):
        st, h = blk_create(cfg)
        if st != BLK_OK:
            raise BlockError(st, blk_last_error())
        self.cfg = cfg
        self.h = h
        self.keep = dict(weights)   # keep tensors alive
        need = weight_shapes(cfg)
        wdt = {n: cfg.dtype for n in need}
        wdt["expert_bias"] = BLK_F32
        for n, shp in need.items():
            if weights.get(n) is None:
                self.close()
                raise BlockError(BLK_E_NULL, f"weight {n} is missing")
            try:
                check_tensor(f"weight {n}", weights[n], shp, wdt[n])
            except BlockError:
                self.close()
                raise
        w = blk_weights()
        for n in WEIGHT_FIELDS + WEIGHT_FIELDS_2:
            t = weights.get(n)
            setattr(w, n, _ptr(t) if t is not None else None)
        w.xielu_alpha_p_raw = float(weights.get("xielu_alpha_p", 0.0))
        w.xielu_alpha_n_raw = float(weights.get("xielu_alpha_n", 0.0))
        self.w = w

    @property
    def workspace_bytes(self):
        return blk_workspace_bytes(self.h)

    def forward(self, x, y, mask=None, taps=None, stream=None):
        """x, y: [B, S, H] device tensors; mask [B, S] int32 or None; taps:
        dict name -> (tensor, blk dtype).  Enqueues on `stream` (torch
        stream or raw handle; default: torch's current stream)."""
        import torch
        if x.dim() != 3:
            raise BlockError(BLK_E_SHAPE, f"x must be [B, S, hidden], got {tuple(x.shape)}")
        B, S = int(x.shape[0]), int(x.shape[1])
        c = self.cfg
        if not (1 <= B <= c.max_batch and 1 <= S <= c.max_seq):
            raise BlockError(BLK_E_SHAPE, f"(B, S) = ({B}, {S}) outside "
                                          f"[1, {c.max_batch}] x [1, {c.max_seq}]")
        check_tensor("x", x, (B, S, c.hidden), c.dtype)
        check_tensor("y", y, (B, S, c.hidden), c.dtype)
        if mask is not None:
            check_tensor("attention_mask", mask, (B, S), BLK_I32)
        if taps:
            shapes = tap_shapes(c, B, S)
            for name, (t, dt) in taps.items():
                if name not in shapes:
                    raise BlockError(BLK_E_CONFIG, f"unknown tap {name}")
                shp, want = shapes[name]
                if dt != want:
                    raise BlockError(BLK_E_DTYPE, f"tap {name} must be requested as {want}")
                check_tensor(f"tap {name}", t, shp, want)
        io = blk_io(x=x.data_ptr(), attention_mask=_ptr(mask), batch=B, seq=S,
                    y=y.data_ptr())
        tp = None
        if taps:
            tp = blk_taps()
            for name, (t, dt) in taps.items():
                setattr(tp, name, blk_tap(ptr=t.data_ptr(), dtype=dt))
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        elif not isinstance(stream, int):
            stream = stream.cuda_stream
        st = blk_forward(self.h, io, self.w, tp, stream)
        if st != BLK_OK:
            raise BlockError(st, blk_last_error())

    def close(self):
        if self.h:
            blk_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
