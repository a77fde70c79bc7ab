"""Writes floor_factor.json: how far above the bf16 floor the GPU's error may
sit before the parity tests call it a fault.

The bf16 floor of a comparison is the error, against the exact fp64 oracle,
of the same computation rounded to bfloat16 at the points where a
bf16-operand path must round (oracle/bf16_emulation.py).  The GPU rounds at
those points too, but at slightly different values (float32 accumulation in
another order, the flash softmax's running scale), so its rounding errors
are another sample of the same law, and its largest error lands near, not
on, the emulation's.

To size that spread, each comparison the tests gate this way is repeated
with K dithered roundings (each rounding moved to a random position of the
bf16 grid, oracle.bf16_emulation.dithered): K independent samples of a
bf16 path with the same rounding points.  For every workload, sequence and
compared value the ratio (largest error of a sample) / (floor) is recorded;
the factor of each compared value (attention_output, mlp_output, the
end-to-end y) is the largest ratio seen for it over every workload and
sequence, rounded up to the next 0.05.  A GPU path is at least as correlated with the emulation as a
dithered sample is (most of its roundings see the same value), so this
bounds it from above; a real fault (a wrong row, a dropped term) moves the
error by far more.

Inputs: the seeded small bf16 workloads (transformer_decoder_block_amd.
synth.SMALL), every sequence; the normed stream the attention is fed is
the emulation's own.  Only the oracle and the input generator are called.

    python tests/golden/floor_factor.py [--samples K]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import bf16_emulation as em  # noqa: E402
from oracle import block as ob  # noqa: E402
from transformer_decoder_block_amd import synth  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "floor_factor.json")


def rel_err(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    return float(np.max(np.abs(got - ref)) / np.sqrt(np.mean(ref ** 2)))


def same_sets(*idx):
    ok = np.ones(idx[0].shape[0], bool)
    for i in idx[1:]:
        ok &= np.all(np.sort(i, -1) == np.sort(idx[0], -1), -1)
    return ok


def errors(x, mk, W, cfg, r, rnd):
    """The three floored comparisons of the GPU tests for one rounding."""
    # the stage inputs are bf16 operands (on the GPU: its own taps), so they
    # are rounded to nearest; the roundings inside each stage are `rnd`
    a = em.r16(ob.rms_norm(x, W["w_in_norm"], cfg["eps"]))
    att_ref = ob.attention_sublayer(x, a, mk, W, cfg)
    att = em.attention_sublayer_bf16(x, a, mk, W, cfg, rnd=rnd)
    mid = att_ref["layer_mid"]
    m = em.r16(ob.mlp_norm(mid, W, cfg))
    mo_ref = ob.mlp_sublayer(mid, m, W, cfg)
    logits = mo_ref.get("router_logits")
    mo = em.mlp_sublayer_bf16(mid, m, W, cfg, logits, rnd=rnd)
    emu = em.block_bf16(x, mk, W, cfg, rnd=rnd)
    keep = np.ones(x.shape[0], bool)
    if cfg["mlp"] == "moe":
        keep = same_sets(r["expert_indices"], emu["expert_indices"])
    return {
        "attention_output": rel_err(att["attention_output"], att_ref["attention_output"]),
        "mlp_output": rel_err(mo["mlp_output"], mo_ref["mlp_output"]),
        "end_to_end_y": rel_err(rnd(emu["layer_output"][keep]), r["layer_output"][keep]),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--samples", type=int, default=40)
    args = ap.parse_args()
    cases = []
    worst = {}
    for w in synth.SMALL.values():
        W = synth.weights_f64(w, synth.make_weights(w))
        x64 = synth.to_f64(synth.make_x(w), w.dtype)
        mask = synth.make_mask(w)
        cfg = w.as_dict()
        for b in range(w.B):
            mk = None if mask is None else mask[b]
            r = ob.block_forward(x64[b], mk, W, cfg)
            floor = errors(x64[b], mk, W, cfg, r, em.r16)
            rng = np.random.default_rng([7100, list(synth.SMALL).index(w.name), b])
            samples = [errors(x64[b], mk, W, cfg, r, em.dithered(rng))
                       for _ in range(args.samples)]
            for key, f in floor.items():
                ratios = np.array([s[key] for s in samples]) / f
                worst[key] = max(worst.get(key, 0.0), float(ratios.max()))
                cases.append({"workload": w.name, "sequence": b, "value": key,
                              "floor": round(f, 6),
                              "ratio_max": round(float(ratios.max()), 4),
                              "ratio_p99": round(float(np.quantile(ratios, 0.99)), 4),
                              "ratio_median": round(float(np.median(ratios)), 4)})
                print(f"{w.name} b={b} {key}: floor {f:.4g}, sample/floor median "
                      f"{np.median(ratios):.3f} max {ratios.max():.3f}", flush=True)
    factors = {k: round(math.ceil(v / 0.05) * 0.05, 2) for k, v in worst.items()}
    rec = {"floor_factor": factors, "largest_ratio": {k: round(v, 4) for k, v in worst.items()},
           "samples_per_case": args.samples,
           "script": "tests/golden/floor_factor.py", "cases": cases}
    with open(OUT, "w") as fh:
        json.dump(rec, fh, indent=1)
    print("floor factors", factors)


if __name__ == "__main__":
    main()
