"""Token-count sweep of the MoE layer on one MI355X.

    python sweep.py [--tokens 1-64,192,768,4097] [--steps 200] [--warmup 20] [--skewed]
                    [--dtype bf16|fp8|mxfp4] [--paths default,gemv,mfma,grp,nogrp,nodgrp]

For every T, one step is one moe_forward over T synthetic tokens with the decode shapes (H 2048,
256 experts, top-8, expert and shared intermediate 512; bf16, FP8 or MXFP4 expert weights), timed as in bench.py: cold weights
(each step takes the next of several independent weight sets), activations resident in HBM,
K steps between two synchronisations. Printed per T: the kernel plan, wall microseconds per
step, tokens/s, the distinct experts touched (U, from the library's own routing), the step's
algorithmic HBM bytes and their rate against the 8 TB/s peak, and each kernel's mean duration
(events recorded by the kernel dispatches themselves). The plan changes at the routing and
expert-group boundaries (T = 16, 64), which the table places against the measured times.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def parse_tokens(spec):
    out = []
    for part in spec.split(","):
        if "-" in part:
            a, b = part.split("-")
            out.extend(range(int(a), int(b) + 1))
        else:
            out.append(int(part))
    return sorted(set(out))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--tokens", default="1-64,192,768,4097")
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sets", type=int, default=6)
    ap.add_argument("--pool", type=int, default=8)
    ap.add_argument("--skewed", action="store_true",
                    help="per-expert router bias ~ N(0, 2) (the verify workload's routing)")
    ap.add_argument("--dtype", default="bf16", choices=("bf16", "fp8", "mxfp4"),
                    help="expert weight format (bf16 activations and router throughout)")
    ap.add_argument("--paths", default="default",
                    help="comma list of expert paths to time per T: default (the library's "
                         "plan), gemv (vector-ALU decode gate/up), mfma (matrix-core decode "
                         "gate/up), grp (the expert-stationary gate/up from T = 65), nogrp "
                         "(never the expert-stationary kernels), nodgrp (the expert-stationary "
                         "gate/up but never its down product)")
    args = ap.parse_args()
    import torch
    from sparse_moe_routing_amd import binding, inputs
    if not torch.cuda.is_available():
        print("sweep.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    binding.load()
    Ts = parse_tokens(args.tokens)
    base = inputs.BY_NAME[("verify_skewed_t192" if args.skewed else "decode_b1_t4") +
                          ("" if args.dtype == "bf16" else "_" + args.dtype)]
    w = dataclasses.replace(base, name="sweep", tokens=max(Ts))
    H = w.hidden
    sets = bench.make_sets(w, args.sets, torch)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(78)
    pool = [torch.randn((w.tokens, H), generator=gen, device="cuda").to(torch.bfloat16)
            for _ in range(args.pool)]
    stream = torch.cuda.current_stream()
    # contexts over the same weight sets per path: the plan boundaries are read from
    # MOE_GEMV_MAX_TOKENS (vector-ALU gate/up up to that T), MOE_GRP_MIN_TOKENS (the
    # expert-stationary gate/up from that T) and MOE_DOWN_GRP_MIN_TOKENS (its down product from
    # that T) when a context is created
    knobs = {"default": {}, "gemv": {"MOE_GEMV_MAX_TOKENS": "64"},
             "mfma": {"MOE_GEMV_MAX_TOKENS": "0"}, "grp": {"MOE_GRP_MIN_TOKENS": "65"},
             "nogrp": {"MOE_GRP_MIN_TOKENS": "0"}, "nodgrp": {"MOE_DOWN_GRP_MIN_TOKENS": "0"}}
    path_sets = {}
    for name in args.paths.split(","):
        saved = {k: os.environ.pop(k, None)
                 for k in ("MOE_GEMV_MAX_TOKENS", "MOE_GRP_MIN_TOKENS", "MOE_DOWN_GRP_MIN_TOKENS")}
        os.environ.update(knobs[name])
        path_sets[name] = [(binding.MoeLayer(H, w.num_experts, w.inter, w.shared_inter, w.tokens,
                                             w.dtype, t), t) for _, t in sets]
        for k, v in saved.items():
            os.environ.pop(k, None)
            if v is not None:
                os.environ[k] = v
    rows = []
    for T, path in [(T, path) for T in Ts for path in path_sets]:
        sets = path_sets[path]
        wt = dataclasses.replace(w, tokens=T)
        m0 = sets[0][0]
        ws = m0.workspace(T)
        y = torch.empty((T, H), dtype=torch.float32, device="cuda")
        plan = m0.plan(T)
        xs = [x[:T] for x in pool]
        U = {}
        for si, (m, _) in enumerate(sets):
            for pi, x in enumerate(xs):
                _, ids, _, _ = m.route(x=x, want_logits=False, ws=ws)
                U[(si, pi)] = int(torch.unique(ids).numel())

        def combo(i):
            return i % len(sets), (i // len(sets) + i) % len(xs)

        for i in range(args.warmup):
            si, pi = combo(i)
            sets[si][0].forward(xs[pi], y=y, ws=ws, stream=stream)
        used = [combo(args.warmup + i) for i in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for si, pi in used:
            sets[si][0].forward(xs[pi], y=y, ws=ws, stream=stream)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        us = el * 1e6 / args.steps
        events = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * len(plan))]
                  for _ in range(args.steps)]
        for evs in events:
            for e in evs:
                e.record(stream)
        torch.cuda.synchronize()
        for i, (si, pi) in enumerate(used):
            sets[si][0].forward(xs[pi], y=y, ws=ws, events=events[i], stream=stream)
        torch.cuda.synchronize()
        per_kernel = {name: float(np.mean([ev[2 * k].elapsed_time(ev[2 * k + 1]) for ev in events]))
                      * 1e3 for k, name in enumerate(plan)}
        mean_U = float(np.mean([U[c] for c in used]))
        step_b = float(np.mean([bench.step_bytes(wt, U[c]) for c in used]))
        row = {"T": T, "path": path, "plan": plan, "us_per_step": us, "tokens_per_s": T / (us * 1e-6),
               "mean_U": mean_U, "step_bytes": step_b, "gbs": step_b / (us * 1e-6) / 1e9,
               "hbm_frac": step_b / (us * 1e-6) / 1e9 / bench.HBM_PEAK_GBS,
               "per_kernel_us": per_kernel}
        rows.append(row)
        print(json.dumps(row), flush=True)
        del ws, y
    print("\n| T | plan | us/step | tokens/s | U | MB/step | GB/s | % of 8 TB/s | kernels (us) |")
    print("|---|---|---|---|---|---|---|---|---|")
    for r in rows:
        ks = ", ".join(f"{k} {v:.1f}" for k, v in r["per_kernel_us"].items())
        print(f"| {r['T']} | {'+'.join(r['plan'][-2:] if len(r['plan']) > 2 else r['plan'])} | "
              f"{r['us_per_step']:.1f} | "
              f"{r['tokens_per_s'] / 1e3:.1f} k | {r['mean_U']:.1f} | {r['step_bytes'] / 1e6:.1f} | "
              f"{r['gbs']:.0f} | {100 * r['hbm_frac']:.1f} | {ks} |")


if __name__ == "__main__":
    main()
