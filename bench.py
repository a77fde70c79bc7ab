"""Decoder-block prefill throughput of libblock on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--layers N] [--taps none|all]

A step is one forward pass of the whole block (every kernel of the path)
over one batch of seeded synthetic input already resident in HBM.  The
default workload is the Llama-7B-shape block (batch 4 x seq 2048, hidden
4096, 32/32 heads of 128, SwiGLU width 10928, bf16 operands, float32
accumulation).  Prints one JSON line.

--layers N times a stack of N blocks (each with its own weights) on one
handle, one blk_forward_layers call per step; --taps all requests every
tap the block has in each step (the materialising path of the interior
values).  --workload also takes the NEXT-row shapes of synth.NEXT.

Per-kernel times come from HIP events that libblock records on its own
stream inside the timed steps (blk_profile_begin/end); the roofline object
reports the dominant kernel's algorithmic FLOP rate against the bf16 dense
MFMA peak.  cpu_baseline times the fp64 CPU oracle on a bounded sample of
the same workload on this host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "block prefill tokens/s at Llama-7B shape bf16, 1 MI355X; % MFMA peak"
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # dense MFMA, MI355X
PEAK_HBM_GBS = 8000.0


def visible_pairs(w, mask):
    """Number of (query, key) pairs attention must evaluate: causal, inside
    the window, key not padded; summed over the batch (per head)."""
    import numpy as np
    tot = 0
    for b in range(w.B):
        real = np.ones(w.S, bool) if mask is None else mask[b] != 0
        for i in range(w.S):
            lo = 0 if w.window <= 0 else max(0, i - w.window + 1)
            tot += int(real[lo:i + 1].sum()) if mask is not None else (i - lo + 1)
    return tot


def kernel_work(w, mask):
    """Algorithmic FLOPs (MFMA kernels) or HBM bytes (row kernels) of one
    launch of each kernel of the block, by profile name."""
    T, H, nh, nkv, hd = w.T, w.H, w.nh, w.nkv, w.hd
    es = 2 if w.dtype == "bf16" else 4
    f = {}
    f["gemm_qkv"] = ("flop", 2.0 * T * H * ((nh + 2 * nkv) * hd + w.head_gate))
    f["attention"] = ("flop", 4.0 * hd * nh * visible_pairs(w, mask))
    f["gemm_o"] = ("flop", 2.0 * T * nh * hd * H)
    if w.mlp == "swiglu":
        f["gemm_up"] = ("flop", 2.0 * T * H * 2 * w.I)
        f["gemm_down"] = ("flop", 2.0 * T * w.I * H)
    elif w.mlp in ("relu2", "xielu"):
        f["gemm_up"] = ("flop", 2.0 * T * H * w.I)
        f["gemm_down"] = ("flop", 2.0 * T * w.I * H)
    else:
        k = w.top_k
        f["gemm_router"] = ("flop", 2.0 * T * H * w.E)
        f["gemm_router_topk"] = ("flop", 2.0 * T * H * w.E)
        f["gemm_expert_up"] = ("flop", 2.0 * T * k * H * 2 * w.I_e)
        f["gemm_expert_down"] = ("flop", 2.0 * T * k * w.I_e * H)
        if w.n_shared:
            f["gemm_shared_up"] = ("flop", 2.0 * T * H * 2 * w.I_sh)
            f["gemm_shared_down"] = ("flop", 2.0 * T * w.I_sh * H)
        f["combine"] = ("byte", T * H * (k * es + 4 + 4 + es) + H * es)
        f["topk"] = ("byte", T * w.E * es + T * k * 8)
    f["rmsnorm_in"] = ("byte", 2.0 * T * H * es + H * es)
    f["rmsnorm_mlp"] = ("byte", T * H * (4 + es) + H * es)
    f["norm_add_norm"] = ("byte", T * H * (4 + es + 4 + es) + 2 * H * es)
    f["post_mlp_norm"] = ("byte", T * H * (4 + 4 + es) + H * es)
    return f


def csrc_hash():
    """Short digest of the kernel sources; HBM counter figures taken from
    an older build no longer describe the kernels and are not reported."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "transformer_decoder_block_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the FETCH_SIZE/WRITE_SIZE
    counter summary kept in profiles/, or None when there is none for this
    workload or the kernels have changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    for line in open(path):
        line = line.strip()
        if line.startswith("traffic-json:"):
            rec = json.loads(line[len("traffic-json:"):])
            if rec.get("csrc_sha256_16") != csrc_hash():
                return None
            return rec["traffic_bytes"].get(kernel)
    return None


def total_flops(work):
    return sum(v for kind, v in work.values() if kind == "flop")


def cpu_baseline(w, budget_s=12.0):
    """The fp64 oracle on a bounded sample of the same workload: the first R
    tokens of the first nb sequences (each token's attention over its own
    causal prefix), grown (R x4 up to the whole sequence, then nb x2 up to
    the whole batch) until one run takes about budget_s seconds."""
    from threadpoolctl import threadpool_info
    from oracle import block as ob
    from transformer_decoder_block_amd import synth
    cfg = w.as_dict()
    R, nb = min(64, w.S), 1
    while True:
        w2 = w.replace(B=nb, S=R, pad=0 if nb == 1 else w.pad)
        W = synth.weights_f64(w2, synth.make_weights(w2))
        x = synth.to_f64(synth.make_x(w2), w.dtype)
        mask = synth.make_mask(w2)
        t0 = time.perf_counter()
        for b in range(nb):
            ob.block_forward(x[b], None if mask is None else mask[b], W, cfg)
        dt = time.perf_counter() - t0
        if dt > budget_s or (R >= w.S and nb >= w.B):
            break
        scale = budget_s / max(dt, 1e-3)
        if R < w.S:
            R = min(w.S, R * 4)
        else:
            nb = min(w.B, nb * 2 if scale >= 2 else nb + 1)
    # a whole workload that finishes in well under a second (the tiny
    # shapes) is run again until the timing spans about a second
    reps = 1
    if dt < 1.0:
        reps = int(min(1000, max(1, 1.0 / max(dt, 1e-4))))
        t0 = time.perf_counter()
        for _ in range(reps):
            for b in range(nb):
                ob.block_forward(x[b], None if mask is None else mask[b], W, cfg)
        dt = time.perf_counter() - t0
    info = threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    blas = ", ".join(sorted({f"{i.get('internal_api', '?')} {i.get('version', '')}".strip()
                             for i in info if i.get("user_api") == "blas"})) or "unknown"
    tokens = R * nb * reps
    runs = f", {reps} runs" if reps > 1 else ""
    return {"value": tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {R} tokens of {nb} of the {w.B} sequences ({w.name} shapes and "
                      f"weights), fp64 NumPy{runs}, {dt:.2f} s",
            "cpu_model": cpu_model(), "blas": blas}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama7b_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--layers", type=int, default=1,
                    help="time a stack of this many blocks (each with its own "
                         "weights) in one blk_forward_layers call per step")
    ap.add_argument("--taps", choices=["none", "all"], default="none",
                    help="all: request every tap the block has in each step")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="after the timed steps, copy this many MiB device to device "
                         "once (a kernel of known traffic for HBM counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs the block on one GPU; "
                          "--gpus must be 1 (no multi-GPU path)"}))
        sys.exit(2)

    import numpy as np
    import torch
    from transformer_decoder_block_amd import binding as L
    from transformer_decoder_block_amd import synth

    w = synth.workload(args.workload)
    if args.layers < 1 or (args.layers > 1 and args.taps != "none"):
        print(json.dumps({"error": "--layers must be >= 1, and taps are per single block"}))
        sys.exit(2)
    Wst = synth.make_weights(w)
    xst = synth.make_x(w)
    mask = synth.make_mask(w)

    def dev(a):
        if isinstance(a, float):
            return a
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    Wd = {k: dev(v) for k, v in Wst.items()}
    x = dev(xst)
    maskd = None if mask is None else torch.from_numpy(mask).cuda()
    y = torch.empty_like(x)
    blk = L.Block(L.make_config(w), Wd)
    # a stack: layers 2..N get weights of their own (other seeds)
    extra = [L.Block(L.make_config(w),
                     {k: dev(v) for k, v in synth.make_weights(
                         w.replace(seed=w.seed + 1000 * l)).items()})
             for l in range(1, args.layers)]
    io = L.blk_io(x=x.data_ptr(), attention_mask=maskd.data_ptr() if maskd is not None else None,
                  batch=w.B, seq=w.S, y=y.data_ptr())
    taps = None
    if args.taps == "all":
        shapes = L.tap_shapes(blk.cfg, w.B, w.S)
        names = ["layer_input", "attention_norm_output", "attention_scores", "layer_mid",
                 "mlp_input", "layer_output", "attention_output", "mlp_output",
                 "attention_queries", "attention_keys", "attention_values",
                 "attention_probabilities", "attention_head_outputs", "attention_premix",
                 "mlp_norm_output"]
        if w.mlp == "moe":
            names += ["router_logits", "expert_indices", "expert_weights", "expert_outputs",
                      "routed_output"] + (["shared_expert_output"] if w.n_shared else [])
        else:
            names += ["mlp_neurons", "mlp_activation"]
        tdt = {L.BLK_F32: torch.float32, L.BLK_BF16: torch.bfloat16, L.BLK_I32: torch.int32}
        taps = {n: (torch.empty(shapes[n][0], dtype=tdt[shapes[n][1]], device="cuda"),
                    shapes[n][1]) for n in names}
    stream = torch.cuda.Stream()

    def step():
        if args.layers > 1:
            st = L.blk_forward_layers(blk.h, io, [blk.w] + [e.w for e in extra],
                                      stream.cuda_stream)
            if st != L.BLK_OK:
                raise RuntimeError(L.blk_last_error())
        else:
            blk.forward(x, y, maskd, taps, stream=stream)

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step()
    torch.cuda.synchronize()

    # timed region: K steps on one stream, per-kernel events recorded inside
    # by the library, plus one event pair per step on the same stream
    L.blk_profile_begin(blk.h, args.steps * args.layers)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    prof = L.blk_profile_end(blk.h) or []
    ms_step = wall * 1e3 / args.steps
    step_ms = np.array([a.elapsed_time(b) for a, b in ev])
    if args.calib_copy_mb:
        n = args.calib_copy_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    work = kernel_work(w, mask)
    flops = total_flops(work) * args.layers
    per_kernel = {}
    for name, tot_ms, calls in prof:
        avg = tot_ms / max(1, calls)
        ent = {"ms": round(avg, 4)}
        if name in work:
            kind, amount = work[name]
            if kind == "flop":
                ent["tflops"] = round(amount / (avg * 1e-3) / 1e12, 1)
            else:
                ent["gbs"] = round(amount / (avg * 1e-3) / 1e9, 1)
        per_kernel[name] = ent
    flop_kernels = [(n, e) for n, e in per_kernel.items() if "tflops" in e]
    dom_name, dom = max(flop_kernels, key=lambda t: t[1]["ms"])
    peak = PEAK_TFLOPS[w.dtype]
    roof = {"bound": "mfma", "achieved": dom["tflops"], "peak": peak,
            "unit": "TFLOP/s", "frac": round(dom["tflops"] / peak, 4),
            "traffic": measured_traffic(w.name, dom_name), "kernel": dom_name,
            "flop_per_launch": work[dom_name][1]}
    if w.dtype == "bf16":
        # context only (frac is against the published peak): a loop of
        # register-only bf16 MFMAs on every SIMD of this chip, no memory
        # traffic, reached 2.1-2.3 PFLOP/s at the clock such a load holds
        roof["measured_mfma_loop_tflops"] = [2100, 2300]
    tokens = w.T
    value = tokens / (ms_step * 1e-3)
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "ms_per_block": round(ms_step / args.layers, 4),
        "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "seq": w.S, "hidden": w.H,
                   "heads": w.nh, "kv_heads": w.nkv, "head_dim": w.hd,
                   "mlp": w.mlp, "intermediate": w.I or w.I_e,
                   "parallelism": "none (1 GPU)", "layers": args.layers,
                   "taps": args.taps},
        # per-step device time (HIP events on the stream, K steps)
        "step_ms": {"median": round(float(np.median(step_ms)), 4),
                    "p10": round(float(np.quantile(step_ms, 0.1)), 4),
                    "p90": round(float(np.quantile(step_ms, 0.9)), 4),
                    "n": int(len(step_ms))},
        # the whole block's algorithmic FLOP rate and its share of the
        # dense MFMA peak (the metric's "% MFMA peak"); roofline below is
        # the dominant kernel alone
        "block_tflops": round(flops / (ms_step * 1e-3) / 1e12, 1),
        "block_frac_of_peak": round(flops / (ms_step * 1e-3) / 1e12 / peak, 4),
        "block_frac_of_peak_median_step": round(
            flops / (float(np.median(step_ms)) * 1e-3) / 1e12 / peak, 4),
        "gflop_per_step": round(flops / 1e9, 1),
        "roofline": roof,
        "kernels": per_kernel,
    }
    if not args.no_cpu_baseline and args.layers == 1 and args.taps == "none":
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
