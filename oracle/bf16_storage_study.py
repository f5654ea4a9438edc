"""Storage-point study of the 12-layer stacked model (the diagnostic mode in
``oracle.bf16_storage``), run on the CPU.

TEST INFRASTRUCTURE ONLY: it imports only ``oracle`` and ``synth``.

    python -m oracle.bf16_storage_study ref  DIR
        exact fp64 forward + backward (no storage point rounded; identical to
        oracle.gpt_forward/gpt_backward); saves the logits and every gradient
        to DIR as fp32 .npy (about 11 GB at the full size)
    python -m oracle.bf16_storage_study emu  DIR  POINTS  [--delta o|o32|p] [--ds-center]
                                       [--p-fwd-form normalised|unnormalised] [--json OUT]
        the same model with the comma-separated storage points rounded to
        bf16 (``all`` = every point, ``all-X-Y`` = every point except X and
        Y); prints max|err|/max|ref| of the logits, the table gradient and
        every parameter gradient of every layer against DIR's reference, and
        with ``--json`` also writes them, with the options and the command,
        to OUT

The inputs are the stacked-model workload's seeded draws (``synth.gpt_inputs``
with workload seed 5: 12 layers, H = 4096, 8 heads of 512, MLP 16384, V =
50257 split over 2 shards, b = 1, s = 2048; LayerNorm gamma = 1, beta = 0),
the same bits the GPU parity test feeds the library.  ``--small`` runs the
2-layer, H = 256 model of the small GPU test instead (seed 51, random
LayerNorm parameters).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402
from oracle import bf16_storage as B  # noqa: E402
from oracle.tp_oracle import partition  # noqa: E402

FULL = dict(w=5, L=12, b=1, s=2048, H=4096, heads=8, d=512, f=16384, V=50257, n=2, ln_random=False)
SMALL = dict(w=51, L=2, b=2, s=64, H=256, heads=4, d=64, f=1024, V=1000, n=2, ln_random=True)


def load_inputs(c):
    vr = [partition(c["V"], c["n"], r)[1] for r in range(c["n"])]
    ids, E, layers, dL = synth.gpt_inputs(c["w"], c["L"], c["b"] * c["s"], c["H"], c["heads"] * c["d"], c["f"],
                                          c["V"], vr, c["ln_random"])
    # bf16 values are exact in fp32: keep the weights in fp32 (half the
    # memory); the emulation widens them to fp64 per product
    f32 = lambda t: synth.bf16_bits_to_f32(t.store) if t.dtype == "bf16" else t.store.astype(np.float32)
    Ef = f32(E)
    lay = [{k: f32(t) for k, t in lw.items()} for lw in layers]
    dLf = [f32(t) for t in dL]
    return ids, Ef, lay, dLf


def grad_names(c):
    names = [f"logits{r}" for r in range(c["n"])] + ["dE"]
    for li in range(c["L"]):
        names += [f"L{li}.{k}" for k in ("WQ", "WK", "WV", "WO", "A", "B", "g1", "b1", "g2", "b2")]
    return names


def run(c, rnd, sink):
    """Forward + backward; ``sink(name, array)`` receives every output."""
    ids, E, layers, dL = load_inputs(c)
    t0 = time.time()
    logits, cache = B.gpt_forward(ids, E, layers, c["b"], c["s"], c["heads"], c["d"], c["n"], rnd)
    for r, lg in enumerate(logits):
        sink(f"logits{r}", lg)
    del logits
    print(f"  forward {time.time() - t0:.0f} s", flush=True)
    for key, val in B.gpt_backward_layers(ids, E, layers, cache, dL, c["b"], c["s"], c["heads"], c["d"], c["n"],
                                          rnd):
        if key == "dE":
            sink("dE", val)
        else:
            for k, g in val.items():
                sink(f"L{key}.{k}", g)
            print(f"  layer {key} backward done {time.time() - t0:.0f} s", flush=True)


def parse_points(spec):
    if spec in ("", "none"):
        return []
    if spec.startswith("all"):
        drop = set(spec.split("-")[1:])
        return [p for p in B.POINTS if p not in drop]
    return spec.split(",")


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("mode", choices=["ref", "emu"])
    ap.add_argument("dir")
    ap.add_argument("points", nargs="?", default="none")
    ap.add_argument("--delta", default="o", choices=["o", "o32", "p"])
    ap.add_argument("--ds-center", action="store_true")
    ap.add_argument("--p-fwd-form", default="normalised", choices=["normalised", "unnormalised"])
    ap.add_argument("--json", default=None)
    ap.add_argument("--small", action="store_true")
    a = ap.parse_args(argv)
    c = SMALL if a.small else FULL
    os.makedirs(a.dir, exist_ok=True)
    if a.mode == "ref":
        def sink(name, arr):
            np.save(os.path.join(a.dir, name + ".npy"), np.asarray(arr, dtype=np.float32))
        run(c, B.Rounding(), sink)
        return
    pts = parse_points(a.points)
    rnd = B.Rounding(pts, delta=a.delta, ds_center=a.ds_center, p_fwd_form=a.p_fwd_form)
    errs = {}

    def sink(name, arr):
        ref = np.load(os.path.join(a.dir, name + ".npy")).astype(np.float64)
        den = np.max(np.abs(ref))
        errs[name] = float(np.max(np.abs(np.asarray(arr, dtype=np.float64) - ref)) / (den if den > 0 else 1.0))
        print(f"  {name} {errs[name]:.3e}", flush=True)

    print(f"points={sorted(pts)} delta={a.delta} ds_center={a.ds_center} p_fwd_form={a.p_fwd_form}", flush=True)
    run(c, rnd, sink)
    grads = {k: v for k, v in errs.items() if not k.startswith("logits")}
    worst = max(grads, key=grads.get)
    over = sorted(k for k, v in grads.items() if v > 1e-2)
    summary = {"points": sorted(pts), "delta": a.delta, "ds_center": a.ds_center, "p_fwd_form": a.p_fwd_form,
               "worst": [worst, grads[worst]], "over_1e-2": len(over),
               "mean": float(np.mean(list(grads.values()))),
               "logits": max(v for k, v in errs.items() if k.startswith("logits")), "errors": errs}
    print("SUMMARY " + json.dumps({k: v for k, v in summary.items() if k != "errors"}), flush=True)
    print("OVER " + " ".join(f"{k}={grads[k]:.2e}" for k in over), flush=True)
    if a.json:
        args = list(argv if argv is not None else sys.argv[1:])
        args[args.index(a.dir)] = "DIR"
        small = " --small" if a.small else ""
        cmd = (f"python -m oracle.bf16_storage_study ref DIR{small} && "
               "python -m oracle.bf16_storage_study " + " ".join(args))
        with open(a.json, "w") as f:
            what = ("max|err|/max|ref| of the logits and of every gradient of the stacked model (page "
                    "'5-megatron', section 训练一般流程: two LayerNorms per layer, tied embedding; split as on "
                    "page 'Megtron张量/模型并行', sections MLP层 / Self-Attention层) computed by "
                    "oracle.bf16_storage with the listed storage points rounded to bf16, against the same "
                    "model in fp64 (oracle.gpt_forward / gpt_backward)")
            json.dump(dict(summary, model="small" if a.small else "full", command=cmd, what=what), f, indent=1,
                      sort_keys=True, ensure_ascii=False)
            f.write("\n")


if __name__ == "__main__":
    main()
