#!/usr/bin/env python3
"""Benchmark of the fused MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--T T] [--alpha A]
    python bench.py --select-sweep [--sweep-T 1,4,16,64,256] [--sweep-eeff 8,32,128,224]

One step = one call of the whole layer (route -> permute -> [fp8 activation quantisation] ->
tile selection -> gate/up GEMM + SwiGLU -> down GEMM -> combine) on one batch of synthetic inputs
already resident in HBM.  The default workload is the largest one that fits one GPU, the
Kimi-K2-shaped prefill layer (T=8192, d=7168, f=2048, E=384, k=8, Dirichlet(0.3) routing, bf16).
Before every step a 512 MiB read evicts L2 and the MALL; HIP events on the library's stream bracket
each step, and the per-step median is the reported time.  Prints one JSON line with tokens/s, the
roofline of the dominant kernel (timed with HIP events on the stream the library launches on) and
the CPU oracle's throughput on a bounded sample of the same workload.

--select-sweep instead times the device's tile-family choice against each family forced, over a
grid of batch sizes and routing skews on DeepSeek-V3-shaped layers, and prints a markdown table.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import statistics
import sys
import time
from dataclasses import replace

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + % HBM peak (decode) / % MFMA peak (prefill), 1 GPU"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # dense MFMA bf16
PEAK_FP8_TFLOPS = 5000.0       # dense MFMA fp8


def workload(args):
    from mixture_experts_layer_top_amd import inputs as I
    name = args.config
    if name == "tiny":
        return I.TINY
    if name in ("mixtral_prefill", "kimi_prefill"):
        base = I.MIXTRAL if name == "mixtral_prefill" else I.KIMI
        if args.T and args.T != base.T:
            return replace(base, T=args.T, name=f"{base.name}_T{args.T}")
        return base
    if name == "dsv3_decode":
        return I.dsv3_point(args.T or 256, args.alpha if args.alpha is not None else 1.0)
    if name == "fp8_dsv3_decode":
        return I.fp8_point(args.T or 128)
    if name in ("mxfp4_dsv3_decode", "mxfp4a8_dsv3_decode"):
        base = I.MXFP4 if name == "mxfp4_dsv3_decode" else I.MXFP4_A8
        T = args.T or base.T
        return replace(base, T=T, name=f"{base.name}_T{T}")
    raise SystemExit(f"unknown --config {name}")


class HipEvents:
    """hipEvent_t handles through the HIP runtime torch already loaded (same soname)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(e.value)
        return out

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


def algorithmic(p, n_active: int):
    """FLOPs and bytes the layer must move (only experts with rows count; intermediates such as
    the permuted rows, h and y are implementation overhead and are not credited)."""
    wb = {"fp8": 1, "mxfp4": 0.5}.get(p.wdtype, 2)
    sh_f = p.shared_f if p.shared else 0
    flop_gu = 4.0 * p.d * (p.f * p.T * p.k + sh_f * p.T)
    flop_dn = 2.0 * p.d * (p.f * p.T * p.k + sh_f * p.T)
    w_gu = n_active * 2.0 * p.f * p.d * wb + (2.0 * sh_f * p.d * wb if p.shared else 0.0)
    w_dn = n_active * 1.0 * p.f * p.d * wb + (1.0 * sh_f * p.d * wb if p.shared else 0.0)
    if p.wdtype == "mxfp4":  # one E8M0 byte per 32 weights
        w_gu += n_active * 2 * p.f * p.d / 32
        w_dn += n_active * p.f * p.d / 32
    if p.wdtype == "fp8":
        w_gu += (n_active * 2 * p.f * p.d + (2 * sh_f * p.d if p.shared else 0)) / (128 * 128) * 4
        w_dn += (n_active * p.f * p.d + (sh_f * p.d if p.shared else 0)) / (128 * 128) * 4
    x_bytes = p.T * p.d * 2.0
    # gate/up reads the activations as bf16, or as MXFP8 codes plus one scale byte per 32
    x_gu = p.T * p.d * (1 + 1 / 32) if p.act_mx8 else x_bytes
    out_bytes = p.T * p.d * 2.0
    logit_bytes = p.T * p.E * 4.0
    return dict(flop=flop_gu + flop_dn, flop_gu=flop_gu, flop_dn=flop_dn,
                bytes=w_gu + w_dn + x_bytes + out_bytes + logit_bytes,
                bytes_gu=w_gu + x_gu, bytes_dn=w_dn + out_bytes)


TRAFFIC_SOURCES = ("mixture_experts_layer_top_amd/csrc/gemm_bf16.hip",
                   "mixture_experts_layer_top_amd/csrc/common.h",
                   "mixture_experts_layer_top_amd/csrc/kernels.h",
                   "mixture_experts_layer_top_amd/csrc/select_dev.h")


def profiled_traffic(workload: str):
    """HBM bytes per launch of the gate/up GEMM from the committed rocprofv3 counter summary
    (profiles/gate_up_gemm_<workload>_traffic.md), or None if there is none or the kernel sources
    changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"gate_up_gemm_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(("-", "|", "#", "`")):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        h.update(open(os.path.join(ROOT, rel), "rb").read())
    if fields.get("kernel_source_sha256_16") != h.hexdigest()[:16]:
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(p, logits, x, W, sample_tokens: int):
    """The CPU oracle as it stands, timed on the first `sample_tokens` tokens of the same inputs
    (routing, permutation, experts and combine are row-wise, so this is the same workload at a
    smaller batch).  Weight bytes are copied to host memory before the clock starts."""
    import numpy as np
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = len(os.sched_getaffinity(0))
    S = min(sample_tokens, p.T)
    L = logits[:S]
    xs = x[:S]
    ids, _ = O.route(L, p.k)
    needed = sorted(set(int(e) for e in np.unique(ids)))
    host = {}
    for e in needed:
        host[e] = {n: W[n][e].cpu().numpy() for n in ("gate", "up", "down")}
        if p.wdtype in ("fp8", "mxfp4"):
            host[e].update({"s_" + n: W["s_" + n][e].cpu().numpy() for n in ("gate", "up", "down")})
    sh = None
    if p.shared:
        sh = {n: W["sh_" + n].cpu().numpy() for n in ("gate", "up", "down")}
        if p.wdtype == "fp8":
            sh.update({"s_" + n: W["s_sh_" + n].cpu().numpy() for n in ("gate", "up", "down")})
    t0 = time.perf_counter()
    O.moe_layer(L, xs, p.k, lambda e: host[e], (lambda: sh) if sh else None,
                act="fp8" if p.wdtype == "fp8" else "mxfp8" if p.act_mx8 else "bf16")
    dt = time.perf_counter() - t0
    return {"value": S / dt, "unit": "tokens/s", "cores": blas_threads, "kind": "oracle",
            "sample": f"first {S} of {p.T} tokens of {p.name} ({len(needed)} experts), "
                      f"float64 numpy/OpenBLAS, {dt:.1f} s"}


def select_control(args, p, ew, d_logits, d_x, flush, auto_ms):
    """Time the layer with every expert forced onto one tile family.  A static rule keyed on the
    batch alone (average rows per expert T*k/E against the streaming threshold) would pick one of
    the two for the whole batch; the device-side selection picks per expert and per GEMM."""
    import torch
    from mixture_experts_layer_top_amd import moe
    res = {"auto_ms": round(auto_ms, 4)}
    n = max(3, args.steps // 2)
    for name, cfg in (("stream_ms", moe.CONFIG_STREAM), ("mfma_ms", moe.CONFIG_MFMA)):
        lay = moe.Layer(ew, p.T, p.E, p.k, config=cfg)
        lay(d_logits, d_x)
        torch.cuda.synchronize()
        if args.flush:
            ts = []
            for _ in range(n):
                flush(0)
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                lay(d_logits, d_x)
                b.record()
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b))
            res[name] = round(statistics.median(ts), 4)
        else:
            t0 = time.perf_counter()
            for _ in range(n):
                lay(d_logits, d_x)
            torch.cuda.synchronize()
            res[name] = round((time.perf_counter() - t0) * 1e3 / n, 4)
    per_expert = p.T * p.k / p.E
    static = "stream_ms" if per_expert <= 8 else "mfma_ms"
    res["static_rule"] = f"T*k/E = {per_expert:g} -> {static[:-3]}"
    res["static_ms"] = res[static]
    res["auto_vs_static"] = round(res[static] / auto_ms, 3)
    res["auto_vs_best_forced"] = round(min(res["stream_ms"], res["mfma_ms"]) / auto_ms, 3)
    return res


def vendor_dense(args, p, gu_ms, dn_ms, alg):
    """The vendor library's dense bf16 GEMMs (hipBLASLt through torch.matmul) with the same FLOPs
    as the layer's two grouped GEMMs, for context: all T*k routed rows against one weight matrix,
    without grouping, gather, SwiGLU or the combine.  Same timing protocol as the layer (events
    around each call after a cache flush with --flush, else wall clock over the calls).  A dense GEMM
    reads one weight matrix where the grouped one streams every active expert's, so each entry also
    gives the time those algorithmic bytes take at peak HBM bandwidth: the comparison means most
    where that floor is well below the dense GEMM's time (prefill with few experts)."""
    import torch
    M = p.T * p.k
    res = {"note": "torch.matmul bf16 (vendor library), dense, same FLOPs as each grouped GEMM"}
    n = max(5, args.steps)
    flush_buf = torch.empty(512 << 20, dtype=torch.uint8, device="cuda") if args.flush else None
    for name, (K, N), ours, nbytes in (("gate_up", (p.d, 2 * p.f), gu_ms, alg["bytes_gu"]),
                                       ("down", (p.f, p.d), dn_ms, alg["bytes_dn"])):
        a = torch.randn(M, K, device="cuda", dtype=torch.bfloat16)
        b = torch.randn(K, N, device="cuda", dtype=torch.bfloat16)
        for _ in range(3):
            c = a @ b
        torch.cuda.synchronize()
        if flush_buf is not None:
            ts = []
            for _ in range(n):
                flush_buf.view(torch.int64).sum()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                c = a @ b
                e1.record()
                e1.synchronize()
                ts.append(e0.elapsed_time(e1))
            ms = statistics.median(ts)
        else:
            t0 = time.perf_counter()
            for _ in range(n):
                c = a @ b
            torch.cuda.synchronize()
            ms = (time.perf_counter() - t0) * 1e3 / n
        del a, b, c
        res[name] = {"shape_MxNxK": f"{M}x{N}x{K}", "ms": round(ms, 4),
                     "tflops": round(2.0 * M * N * K / (ms * 1e-3) / 1e12, 1),
                     "this_layer_kernel_ms": round(ours, 4), "layer_kernel_over_vendor": round(ours / ms, 3),
                     "grouped_bytes_hbm_floor_ms": round(nbytes / (PEAK_HBM_GBS * 1e9) * 1e3, 4)}
    res["kernel_ms_source"] = ("gate_up: HIP events around every second step's gate/up launches; "
                               "down: the phase-traced steps (each phase event adds ~5 us)")
    return res


def select_sweep(args) -> int:
    """The device's per-expert tile choice against each family forced, over a grid of batch sizes
    and routing skews, on DeepSeek-V3-shaped layers (d = 7168, f = 2048, E = 256, k = 8).

    Skew is set by its effective expert count ("Decoding the Skew ...", Abstract: kernels are
    chosen from the live routing histogram; skew is modelled with Dirichlet draws): each target
    count fixes the Dirichlet concentration through the closed-form expected entropy
    (inputs.alpha_for_eeff), and the table reports the count measured on the routed histogram as
    well.  Each configuration: 3 warm-up calls, then --steps calls, each after a 512 MiB read that
    evicts L2 and the MALL, HIP events around the layer, median.  The last column prices a static
    token-count bucket (the dispatch the pages contrast with a distribution-aware one): T*k/E <= 8
    -> every expert on the streaming tiles, else every expert on MFMA tiles."""
    import numpy as np
    import torch
    from mixture_experts_layer_top_amd import inputs as I
    from mixture_experts_layer_top_amd import moe
    Ts = [int(v) for v in args.sweep_T.split(",")]
    targets = [float(v) for v in args.sweep_eeff.split(",")]
    base = I.DSV3
    W = I.gen_weights(base, "cuda")
    ew = moe.ExpertWeights(gate=W["gate"], up=W["up"], down=W["down"])
    scratch = torch.ones(512 << 20, dtype=torch.uint8, device="cuda")

    def time_layer(layer, logits, x):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        for _ in range(3):
            layer(logits, x)
        ts = []
        for _ in range(args.steps):
            scratch.view(torch.int64).sum()
            e0.record()
            layer(logits, x)
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        return statistics.median(ts)

    print("| T | E_eff target | alpha | E_eff routed | n_active | device ms | stream ms | MFMA ms "
          "| device / best | static bucket / device |")
    print("|---|---|---|---|---|---|---|---|---|---|", flush=True)
    for T in Ts:
        for tgt in targets:
            alpha = I.alpha_for_eeff(base.E, tgt)
            p = I.Problem(f"sweep_T{T}_e{tgt:g}", base.cfg_index, T=T, d=base.d, f=base.f, E=base.E,
                          k=base.k, routing="dirichlet", alpha=alpha)
            logits = torch.from_numpy(I.gen_logits(p)).cuda()
            x = torch.from_numpy(I.gen_x(p).view(np.int16)).cuda()
            ms, counts = {}, None
            for name, cfg in (("device", moe.CONFIG_AUTO), ("stream", 0), ("mfma", 1)):
                layer = moe.Layer(ew, T, base.E, base.k, config=cfg)
                if counts is None:
                    kept = {"counts": torch.zeros(base.E, dtype=torch.int32, device="cuda")}
                    layer(logits, x, kept)
                    counts = kept["counts"].cpu().numpy()
                ms[name] = time_layer(layer, logits, x)
                del layer
            best = min(ms["stream"], ms["mfma"])
            static = ms["stream"] if T * base.k / base.E <= 8 else ms["mfma"]
            print(f"| {T} | {tgt:g} | {alpha:.4g} | {I.effective_experts(counts):.1f} | "
                  f"{int((counts > 0).sum())} | {ms['device']:.3f} | {ms['stream']:.3f} | "
                  f"{ms['mfma']:.3f} | {ms['device'] / best:.3f} | {static / ms['device']:.3f} |",
                  flush=True)
    return 0


def _policy_table_text(table, command, note):
    rows = ",\n".join("    {" + ", ".join(str(v) for v in r) + "}" for r in table)
    return f"""// Policy table of the device-side selection: kPolicyTable[T bucket][effective-expert bucket] is the
// index of the policy (select_policy.h) the selection applies.  Written by bench.py --tune-select:
//   {command}
// {note}
#pragma once

namespace moe {{

constexpr unsigned char kPolicyTable[kTBuckets][kEeffBuckets] = {{
{rows},
}};

}}  // namespace moe
"""


def tune_select(args) -> int:
    """Offline tuning of the selection policy table ("Decoding the Skew ...", Abstract: the live
    routing histogram is matched to distributions tuned offline).  For each sweep point (a layer
    shape, a batch size and a Dirichlet concentration set from a target effective expert count)
    every policy is timed with its config forced (16 + i), besides the automatic choice and a
    static token-count bucket, under the flushed protocol (a 512 MiB read before each step, HIP
    events around the layer, median).  The point falls in the table cell of its T and its routed
    histogram's effective expert count (the values the device computes); each cell takes the
    policy with the lowest mean time relative to the point's best.  Cells with no point copy the
    nearest measured cell of their T row (else policy 0).  Prints the per-point markdown table;
    --table-out writes the header."""
    import math
    import numpy as np
    import torch
    from dataclasses import replace as dc_replace
    from mixture_experts_layer_top_amd import inputs as I
    from mixture_experts_layer_top_amd import moe
    scratch = torch.ones(512 << 20, dtype=torch.uint8, device="cuda")

    def time_layer(layer, logits, x, steps, warm=3, each=False):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(warm):
            layer(logits, x)
        ts = []
        for _ in range(steps):
            scratch.view(torch.int64).sum()
            e0.record()
            layer(logits, x)
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        return ts if each else statistics.median(ts)

    def t_bucket(T):
        for i, lim in enumerate((1, 2, 4, 8, 16, 32, 64, 128, 256, 1024)):
            if T <= lim:
                return i
        return 10

    def e_bucket(e):
        for i, lim in enumerate((6, 12, 24, 48, 96, 192)):
            if e <= lim:
                return i
        return 6

    points = []
    base = I.DSV3
    for T in [int(v) for v in args.sweep_T.split(",")]:
        for tgt in [float(v) for v in args.sweep_eeff.split(",")]:
            if tgt >= base.E or tgt <= 1:
                continue
            alpha = I.alpha_for_eeff(base.E, tgt)
            points.append(I.Problem(f"tune_T{T}_e{tgt:g}", base.cfg_index, T=T, d=base.d, f=base.f,
                                    E=base.E, k=base.k, routing="dirichlet", alpha=alpha))
    if args.tune_prefill:
        points += [dc_replace(I.MIXTRAL, T=T, name=f"mixtral_T{T}") for T in (512, 2048, 4096)]
        points += [I.KIMI]
    weights = {}
    n_pol = moe.NUM_POLICIES
    table_score, table_count = {}, {}
    print("| workload | T | E_eff routed | cell | auto (ms) | " +
          " | ".join(f"P{i}" for i in range(n_pol)) + " | static bucket | best |")
    print("|---|---|---|---|---|" + "---|" * n_pol + "---|---|", flush=True)
    for p in points:
        key = (p.cfg_index, p.d, p.f, p.E)
        if key not in weights:
            weights.clear()
            torch.cuda.empty_cache()
            W = I.gen_weights(p, "cuda")
            weights[key] = moe.ExpertWeights(gate=W["gate"], up=W["up"], down=W["down"])
        ew = weights[key]
        logits = torch.from_numpy(I.gen_logits(p)).cuda()
        x = torch.from_numpy(I.gen_x(p).view(np.int16)).cuda()
        steps = args.steps if p.T <= 256 else max(5, args.steps // 3)
        auto = moe.Layer(ew, p.T, p.E, p.k)
        kept = {"counts": torch.zeros(p.E, dtype=torch.int32, device="cuda")}
        auto(logits, x, kept)
        counts = kept["counts"].cpu().numpy()
        eeff = I.effective_experts(counts)
        static_cfg = moe.CONFIG_STREAM if p.T * p.k / p.E <= 8 else moe.CONFIG_MFMA
        confs = [moe.Layer(ew, p.T, p.E, p.k, config=moe.CONFIG_POLICY0 + i) for i in range(n_pol)]
        confs += [auto, moe.Layer(ew, p.T, p.E, p.k, config=static_cfg)]
        # interleaved: rounds of a few steps per configuration, the order rotated (and reversed
        # every other round), so no configuration always runs first after a pause; the median
        # over all of a configuration's steps
        samples = [[] for _ in confs]
        rounds = 4
        for r in range(rounds):
            order = list(range(len(confs)))
            order = order[r % len(order):] + order[:r % len(order)]
            if r % 2:
                order.reverse()
            for c in order:
                samples[c] += time_layer(confs[c], logits, x, max(1, steps // rounds), warm=1, each=True)
        med = [statistics.median(v) for v in samples]
        ms, ms_auto, ms_static = med[:n_pol], med[n_pol], med[n_pol + 1]
        del confs, auto
        best = min(ms)
        cell = (t_bucket(p.T), e_bucket(eeff))
        sc = table_score.setdefault(cell, [0.0] * n_pol)
        table_count[cell] = table_count.get(cell, 0) + 1
        for i in range(n_pol):
            sc[i] += math.log(ms[i] / best)
        print(f"| {p.name} | {p.T} | {eeff:.1f} | {cell} | {ms_auto:.3f} | " +
              " | ".join(f"{v:.3f}" for v in ms) + f" | {ms_static:.3f} | P{ms.index(best)} |",
              flush=True)
    # a cell leaves policy 0 (the hand rules) only for a mean gain above the margin
    table = [[0] * 7 for _ in range(11)]
    measured = {}
    for c, v in table_score.items():
        mean = [t / table_count[c] for t in v]
        i = int(np.argmin(mean))
        measured[c] = i if mean[0] - mean[i] > math.log(1.0 + args.tune_margin) else 0
    for tb in range(11):
        row = {eb: pol for (t, eb), pol in measured.items() if t == tb}
        for eb in range(7):
            if eb in row:
                table[tb][eb] = row[eb]
            elif row:
                table[tb][eb] = row[min(row, key=lambda r: (abs(r - eb), r))]
    print("\ncells measured (T bucket, E_eff bucket) -> policy:",
          {f"{c}": p_ for c, p_ in sorted(measured.items())}, flush=True)
    if args.table_out:
        argv, skip = [], False
        for a in sys.argv[1:]:  # the command without the output path
            if skip or a.startswith("--table-out"):
                skip = a == "--table-out"
                continue
            argv.append(a)
        cmd = " ".join(["python bench.py"] + argv + ["--table-out <file>"])
        note = (f"A cell leaves policy 0 only for a mean gain above {100 * args.tune_margin:g}%; cells "
                "with no sweep point copy the nearest measured cell of their T row; rows with none "
                "hold policy 0.")
        with open(args.table_out, "w") as fh:
            fh.write(_policy_table_text(table, cmd, note))
        print(f"wrote {args.table_out}", flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="kimi_prefill",
                    choices=["mixtral_prefill", "tiny", "kimi_prefill", "dsv3_decode", "fp8_dsv3_decode",
                             "mxfp4_dsv3_decode", "mxfp4a8_dsv3_decode"])
    ap.add_argument("--T", type=int, default=None, help="tokens (overrides the workload's batch)")
    ap.add_argument("--alpha", type=float, default=None, help="Dirichlet concentration (dsv3_decode)")
    ap.add_argument("--tile-config", type=int, default=-1, help="-1 auto, 0 stream, 1 mfma")
    ap.add_argument("--no-flush", dest="flush", action="store_false",
                    help="do not sweep a 512 MiB buffer before every step (by default L2 and the "
                         "MALL are evicted and the value comes from the per-step events' median)")
    ap.add_argument("--flush-mode", choices=["read", "write"], default="read",
                    help="read: sum the buffer (evicts with clean lines); write: overwrite it (the "
                         "dirty lines are then written back while the layer runs)")
    ap.add_argument("--cpu-sample", type=int, default=None, help="tokens for the CPU oracle leg")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for HBM byte-counter calibration)")
    ap.add_argument("--graph", action="store_true",
                    help="also time replays of one layer call captured in a HIP graph")
    ap.add_argument("--vendor-dense", action="store_true",
                    help="also time the vendor library's dense bf16 GEMMs of the same FLOPs as the "
                         "layer's two grouped GEMMs (context for the MFMA kernels)")
    ap.add_argument("--select-control", action="store_true",
                    help="also time the layer with every expert forced onto one tile family (the "
                         "control arms of the device-side selection), same protocol, fewer steps")
    ap.add_argument("--select-sweep", action="store_true",
                    help="only run the tile-selection sweep over --sweep-T x --sweep-eeff (markdown "
                         "table, no JSON line)")
    ap.add_argument("--tune-select", action="store_true",
                    help="only run the selection-policy tuner over --sweep-T x --sweep-eeff (and, with "
                         "--tune-prefill, prefill shapes) and print its table")
    ap.add_argument("--tune-prefill", action="store_true")
    ap.add_argument("--tune-margin", type=float, default=0.02,
                    help="--tune-select: smallest mean gain over policy 0 that changes a cell")
    ap.add_argument("--table-out", default=None, help="--tune-select: write the policy table header here")
    ap.add_argument("--sweep-T", default="1,4,16,64,256")
    ap.add_argument("--sweep-eeff", default="8,32,128,224",
                    help="target effective expert counts (each fixes a Dirichlet concentration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(experts would shard across GPUs with an all-to-all dispatch; not built).",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch
    from mixture_experts_layer_top_amd import inputs as I
    from mixture_experts_layer_top_amd import moe

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    if args.select_sweep:
        return select_sweep(args)
    if args.tune_select:
        return tune_select(args)
    p = workload(args)
    print(f"[bench] workload {p.name}: T={p.T} d={p.d} f={p.f} E={p.E} k={p.k} {p.wdtype}"
          f"{' +shared' if p.shared else ''}", file=sys.stderr, flush=True)
    t_gen = time.perf_counter()
    logits = I.gen_logits(p)
    x = I.gen_x(p)
    W = I.gen_weights(p, "cuda")
    d_logits = torch.from_numpy(logits).cuda()
    d_x = torch.from_numpy(x.view(np.int16)).cuda()
    kw = dict(gate=W["gate"], up=W["up"], down=W["down"])
    if p.wdtype == "fp8":  # the library's tiled weight layout (made once, untimed)
        kw.update({n: moe.fp8_tile(W[n]) for n in ("gate", "up", "down")})
        kw.update(s_gate=W["s_gate"], s_up=W["s_up"], s_down=W["s_down"])
    if p.wdtype == "mxfp4":  # the library's tiled weight layout (made once, untimed)
        kw.update({n: moe.mxfp4_tile(W[n]) for n in ("gate", "up", "down")})
        kw.update(e_gate=W["s_gate"], e_up=W["s_up"], e_down=W["s_down"], act_mx8=p.act_mx8)
    if p.shared:
        kw.update(sh_gate=W["sh_gate"], sh_up=W["sh_up"], sh_down=W["sh_down"])
        if p.wdtype == "fp8":
            kw.update({n: moe.fp8_tile(W[n]) for n in ("sh_gate", "sh_up", "sh_down")})
            kw.update(s_sh_gate=W["s_sh_gate"], s_sh_up=W["s_sh_up"], s_sh_down=W["s_sh_down"])
    ew = moe.ExpertWeights(**kw)
    layer = moe.Layer(ew, p.T, p.E, p.k, config=args.tile_config)
    counts = torch.zeros(p.E, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    print(f"[bench] inputs ready in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)

    hip = HipEvents()
    K, Wm = args.steps, args.warmup
    evs = [hip.create(moe.TRACE_EVENTS) for _ in range(K)]
    scratch = torch.ones(512 << 20, dtype=torch.uint8, device="cuda") if args.flush else None

    def flush(i):
        if scratch is None:
            return
        if args.flush_mode == "write":
            scratch.fill_(i & 0xFF)
        else:
            scratch.view(torch.int64).sum()

    for i in range(Wm):
        layer(d_logits, d_x, keep={"counts": counts} if i == 0 else None)
    torch.cuda.synchronize()
    if Wm == 0:
        layer(d_logits, d_x, keep={"counts": counts})
        torch.cuda.synchronize()

    # Timed region: K steps, each after the cache flush.  Every timing event costs GPU time (a few
    # microseconds, which matters at decode sizes), so at decode sizes odd steps record only the
    # two events around the dominant kernel (the gate/up GEMM, for the roofline) and even steps only
    # the layer's first and last event (for the per-step times); prefill steps (T >= 512, where
    # they are noise) record all four, and with K = 1 the one step records all four.
    GU0, GU1, LAST = 4, 5, moe.TRACE_EVENTS - 1
    every = p.T >= 512 or K == 1
    def keep(i):
        gu = every or i % 2 == 1
        ends = every or i % 2 == 0
        return ({GU0, GU1} if gu else set()) | ({0, LAST} if ends else set())
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        flush(i)
        k_i = keep(i)
        layer.traced(d_logits, d_x, [e if j in k_i else None for j, e in enumerate(evs[i])])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gu_launch_ms = [hip.elapsed_ms(evs[i][GU0], evs[i][GU1]) for i in range(K) if GU0 in keep(i)]
    step_ms = [hip.elapsed_ms(evs[i][0], evs[i][LAST]) for i in range(K) if 0 in keep(i)]

    # Phase breakdown (not timed): a few more steps with every phase boundary recorded.
    phases = {name: [] for name in moe.TRACE_PHASES}
    for i in range(min(K, 5)):
        flush(i)
        layer.traced(d_logits, d_x, evs[i])
    torch.cuda.synchronize()
    for i in range(min(K, 5)):
        for j, name in enumerate(moe.TRACE_PHASES):
            phases[name].append(hip.elapsed_ms(evs[i][j], evs[i][j + 1]))
    for e in evs:
        hip.destroy(e)

    # HIP-graph replay (optional): one layer call captured on a side stream's capture, replayed K
    # times with the same flush protocol; the library launches no allocation, memset or host sync,
    # so the whole call is capturable.
    graph = None
    if args.graph:
        static_logits, static_x = d_logits.clone(), d_x.clone()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            layer(static_logits, static_x)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            layer(static_logits, static_x)
        torch.cuda.synchronize()
        for _ in range(Wm):
            g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        rep_ms = []
        t0 = time.perf_counter()
        for i in range(K):
            flush(i)
            e0.record()
            g.replay()
            e1.record()
            if args.flush:
                e1.synchronize()
                rep_ms.append(e0.elapsed_time(e1))
        torch.cuda.synchronize()
        g_wall = time.perf_counter() - t0
        g_ms = statistics.median(rep_ms) if args.flush else g_wall * 1e3 / K
        graph = {"ms_per_step": round(g_ms, 4), "tokens_per_s": round(p.T / (g_ms * 1e-3), 1),
                 "timing": "median of events around each replay" if args.flush
                 else "wall clock over the replays"}
        del g

    n_active = int((counts.cpu() > 0).sum())
    alg = algorithmic(p, n_active)
    ms_per_step = statistics.median(step_ms)
    q = statistics.quantiles(step_ms, n=10) if len(step_ms) >= 2 else [step_ms[0]] * 9
    step_spread = {"p10_ms": round(q[0], 4), "p50_ms": round(ms_per_step, 4), "p90_ms": round(q[8], 4),
                   "samples": len(step_ms), "wall_ms_per_step_incl_flush": round(wall * 1e3 / K, 4)}
    if args.flush:
        timing = ("median of per-step HIP events around the layer; a 512 MiB read "
                  f"({args.flush_mode}) evicts L2 and the MALL before each step")
    else:
        timing = "median of per-step HIP events around the layer, no cache flush"
    value = p.T / (ms_per_step * 1e-3)

    # (mxfp4 x mxfp8 products run at the fp8 rate: the doubled fp4/fp6 rate needs both operands
    # narrow; mxfp4 weights with bf16 activations are expanded to bf16 products)
    peak_flops = PEAK_FP8_TFLOPS if p.wdtype == "fp8" or p.act_mx8 else PEAK_BF16_TFLOPS
    # the dominant kernel's bound: whichever of its algorithmic flops and bytes takes longer at peak
    prefill = alg["flop_gu"] / (peak_flops * 1e12) > alg["bytes_gu"] / (PEAK_HBM_GBS * 1e9)
    gu_ms = statistics.mean(gu_launch_ms)
    if prefill:
        achieved = alg["flop_gu"] / (gu_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak_flops,
                "unit": "TFLOP/s", "frac": round(achieved / peak_flops, 4)}
    else:
        achieved = alg["bytes_gu"] / (gu_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}
    traffic = profiled_traffic(p.name)
    single = p.T == 1 and p.wdtype == "bf16" and not p.shared and p.d <= 8192 and args.tile_config != 1
    roof.update({"kernel": "gate/up grouped GEMM + SwiGLU" + (
                     " with the token's routing fused in (single-token decode kernel)" if single
                     else " (both tile families)"),
                 "avg_launch_ms": round(gu_ms, 4),
                 "traffic": traffic, "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE + "
                 "WRITE_SIZE, calibrated on a 1 GiB copy)" if traffic else None,
                 "algorithmic_per_launch": alg["flop_gu"] if prefill else alg["bytes_gu"]})

    layer_s = ms_per_step * 1e-3
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("mxfp4 weights, mxfp8 activations" if p.act_mx8 else
                  {"fp8": "fp8", "mxfp4": "mxfp4 weights, bf16 activations"}.get(p.wdtype, "bf16")),
        "data": "synthetic",
        "config": {"workload": p.name, "T": p.T, "d_model": p.d, "d_ff": p.f, "experts": p.E,
                   "top_k": p.k, "routing": p.routing + (f"(alpha={p.alpha:g})" if p.routing == "dirichlet" else ""),
                   "shared_expert_d_ff": p.shared_f if p.shared else 0, "n_active": n_active,
                   "tile_config": args.tile_config},
        "roofline": roof,
        "layer": {"mfma_frac": round(alg["flop"] / layer_s / 1e12 / peak_flops, 4),
                  "hbm_frac": round(alg["bytes"] / layer_s / 1e9 / PEAK_HBM_GBS, 4),
                  "phase_ms": {k: round(statistics.mean(v), 4) for k, v in phases.items()},
                  "phase_note": "separate untimed steps with every phase boundary recorded (each "
                                "timing event adds ~5 us of GPU time)",
                  "timing": timing},
    }
    out["layer"]["step_ms"] = step_spread
    if graph:
        out["graph_replay"] = graph
    if args.vendor_dense and p.wdtype == "bf16":
        out["vendor_dense"] = vendor_dense(args, p, gu_ms, statistics.mean(phases["down"]), alg)
    if args.select_control and p.wdtype == "bf16":
        out["select_control"] = select_control(args, p, ew, d_logits, d_x, flush, ms_per_step)
    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
    if not args.no_cpu_baseline:
        sample = args.cpu_sample or {"mixtral_prefill": 4096, "kimi_prefill": 256}.get(p.name, p.T)
        print(f"[bench] CPU oracle on {sample} tokens ...", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(p, logits, x, W, sample)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
