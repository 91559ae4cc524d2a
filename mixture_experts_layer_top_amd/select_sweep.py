"""Tile-selection sweep: the device's per-expert choice against each family forced, over a grid of
batch sizes and routing skews, on DeepSeek-V3-shaped layers (d = 7168, f = 2048, E = 256, k = 8).

    python -m mixture_experts_layer_top_amd.select_sweep [--T 1,4,16,...] [--eeff 8,32,...]
                                                         [--steps N] [--out FILE]

Skew is set by its effective expert count ("Decoding the Skew ...", Abstract: kernels are chosen
from the live routing histogram; skew is modelled with Dirichlet draws): each target count fixes
the Dirichlet concentration through the closed-form expected entropy (inputs.alpha_for_eeff), and
the table reports the count measured on the routed histogram as well.  Every configuration is
timed the same way: a 512 MiB read flushes L2 and the MALL before each step, HIP events on the
library's stream bracket the layer, and the median over the steps is kept.  The last column prices
a static token-count bucket (the dispatch the pages contrast with a distribution-aware one): at
most 8 rows per expert on average (T*k/E <= 8) -> every expert on the streaming tiles, else every
expert on MFMA tiles.  Prints a markdown table (and writes it to --out).
"""
from __future__ import annotations

import argparse
import statistics
import sys

import numpy as np
import torch

from . import inputs as I
from . import moe


def _time_layer(layer, logits, x, steps, scratch):
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    for _ in range(3):
        layer(logits, x)
    ts = []
    for _ in range(steps):
        scratch.view(torch.int64).sum()
        e0.record()
        layer(logits, x)
        e1.record()
        e1.synchronize()
        ts.append(e0.elapsed_time(e1))
    return statistics.median(ts)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--T", default="1,4,16,64,256")
    ap.add_argument("--eeff", default="8,32,128,224")
    ap.add_argument("--steps", type=int, default=15)
    ap.add_argument("--out", default=None)
    args = ap.parse_args(argv)
    if not torch.cuda.is_available():
        print("select_sweep needs a GPU", file=sys.stderr)
        return 1
    Ts = [int(v) for v in args.T.split(",")]
    targets = [float(v) for v in args.eeff.split(",")]
    base = I.DSV3
    W = I.gen_weights(base, "cuda")
    ew = moe.ExpertWeights(gate=W["gate"], up=W["up"], down=W["down"])
    scratch = torch.ones(512 << 20, dtype=torch.uint8, device="cuda")
    rows = ["| T | E_eff target | alpha | E_eff routed | n_active | device ms | stream ms | MFMA ms "
            "| device / best | static bucket / device |", "|---|---|---|---|---|---|---|---|---|---|"]
    print(rows[0]); print(rows[1], flush=True)
    for T in Ts:
        for tgt in targets:
            alpha = I.alpha_for_eeff(base.E, tgt)
            p = I.Problem(f"sweep_T{T}_e{tgt:g}", base.cfg_index, T=T, d=base.d, f=base.f, E=base.E,
                          k=base.k, routing="dirichlet", alpha=alpha)
            logits = torch.from_numpy(I.gen_logits(p)).cuda()
            x = torch.from_numpy(I.gen_x(p).view(np.int16)).cuda()
            ms = {}
            counts = None
            for name, cfg in (("device", moe.CONFIG_AUTO), ("stream", 0), ("mfma", 1)):
                layer = moe.Layer(ew, T, base.E, base.k, config=cfg)
                if counts is None:
                    keep = {"counts": torch.zeros(base.E, dtype=torch.int32, device="cuda")}
                    layer(logits, x, keep)
                    counts = keep["counts"].cpu().numpy()
                ms[name] = _time_layer(layer, logits, x, args.steps, scratch)
                del layer
            best = min(ms["stream"], ms["mfma"])
            static = ms["stream"] if T * base.k / base.E <= 8 else ms["mfma"]
            line = (f"| {T} | {tgt:g} | {alpha:.4g} | {I.effective_experts(counts):.1f} | "
                    f"{int((counts > 0).sum())} | {ms['device']:.3f} | {ms['stream']:.3f} | "
                    f"{ms['mfma']:.3f} | {ms['device'] / best:.3f} | {static / ms['device']:.3f} |")
            rows.append(line)
            print(line, flush=True)
    if args.out:
        with open(args.out, "w") as fh:
            fh.write("\n".join(rows) + "\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
