"""Benchmark of the sparse MoE layer on one MI355X: tokens/s of the whole hot path.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode_b1_t4]

A step is one moe_forward over one batch of T synthetic tokens: router logits, top-8 selection
with softmax and shared gate, bucketing, the expert gate/up/down stage and the weighted combine.
Inputs are resident in HBM before the timed region. To time cold weights (the 256 MB Infinity
Cache would hold a whole T=4 working set), each step uses the next of several independent weight
sets and the next activation batch of a pool, so consecutive steps share no expert bytes.

Printed: one JSON line with the metric for --workload (default: the T=4 decode round), its
dominant kernel's roofline (algorithmic bytes per launch over its event-timed average duration)
and the oracle's CPU throughput on a bounded sample of the same workload (all threads and one).
The metric is quoted at T=4, 32 and 192, so the same line carries `sub_results` for the T=32
decode round and the skewed T=192 verify round, each timed the same way after the main one.
Next to the 8 TB/s specification each result reports `read_ceiling_gbs`: this GPU's measured rate
for reading the step's byte count once, cold (the calibration kernel of libmoe_probe.so, built
next to libmoe.so), and the step's HBM rate as a fraction of it.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="decode_b1_t4")
    ap.add_argument("--sets", type=int, default=6, help="independent weight sets (cold cache)")
    ap.add_argument("--pool", type=int, default=16, help="activation batches in the pool")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sub", action="store_true",
                    help="time only --workload (not the T=32 and skewed T=192 rounds as well)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    return ap.parse_args()


def make_sets(w, n_sets, torch):
    """Weight sets drawn on the GPU with the workload's shapes and scales (bench only)."""
    from sparse_moe_routing_amd import binding
    H, E, I, Is = w.hidden, w.num_experts, w.inter, w.shared_inter
    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16  # x and router (fp8: bf16)
    gen = torch.Generator(device="cuda")
    layers = []
    for s in range(n_sets):
        gen.manual_seed(10_000 + s)

        def draw(shape, scale):
            return (torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32)
                    * scale).to(dt)

        def draw_w(shape, scale):
            """An expert weight block; fp8: per-row E4M3 codes (uint8) and fp32 row scales;
            mxfp4: random packed E2M1 codes with E8M0 scale bytes near what the input quantizer
            gives for these scales (amax of 32 normal draws ~2.5 sigma, over 6: 2^-7 .. 2^-5)."""
            if w.dtype == "mxfp4":
                rows, cols = shape[:-1], shape[-1]
                codes = torch.randint(0, 256, (*rows, cols // 2), generator=gen, device="cuda",
                                      dtype=torch.uint8)
                sb = torch.randint(118, 123, (*rows, cols // 32), generator=gen, device="cuda",
                                   dtype=torch.uint8)
                return codes, sb
            if w.dtype != "fp8":
                return draw(shape, scale), None
            v = torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32) * scale
            rs = v.abs().amax(dim=-1).clamp_min(1e-30) / 448.0
            q = (v / rs.unsqueeze(-1)).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
            return q.view(torch.uint8), rs.contiguous()

        gu, gus = draw_w((E, 2 * I, H), H ** -0.5)
        dn, dns = draw_w((E, H, I), I ** -0.5)
        sgu, sgus = draw_w((2 * Is, H), H ** -0.5)
        sdn, sdns = draw_w((H, Is), Is ** -0.5)
        t = {"router_w": draw((E + 1, H), H ** -0.5), "router_bias": None,
             "gate_up": gu, "down": dn, "shared_gate_up": sgu, "shared_down": sdn,
             "gate_up_scale": gus, "down_scale": dns, "shared_gate_up_scale": sgus,
             "shared_down_scale": sdns}
        if w.bias_std > 0:
            b = torch.zeros(E + 1, device="cuda")
            b[:E] = torch.randn(E, generator=gen, device="cuda") * w.bias_std
            t["router_bias"] = b
        m = binding.MoeLayer(H, E, I, Is, w.tokens, w.dtype, t)
        layers.append((m, t))
    return layers


def sizes(w):
    """(activation bytes, expert weight bytes, row-scale bytes) per element / row."""
    if w.dtype == "fp8":
        return 2, 1, 4
    if w.dtype == "mxfp4":  # half a byte of code plus a scale byte per 32 weights
        return 2, 0.5 + 1 / 32, 0
    esz = 2 if w.dtype == "bf16" else 4
    return esz, esz, 0


def step_bytes(w, U):
    """Algorithmic HBM bytes of one step: router, shared expert, the U distinct routed experts
    touched (each read once, with their row scales for fp8), x in and y out."""
    esz, wsz, ssz = sizes(w)
    H, I, Is, E, T = w.hidden, w.inter, w.shared_inter, w.num_experts, w.tokens
    return (esz * (E + 1) * H + 3 * wsz * H * Is + ssz * (2 * Is + H) +
            U * (3 * wsz * H * I + ssz * (2 * I + H)) + esz * T * H + 4 * T * H)


def kernel_bytes(w, U, name):
    """Algorithmic bytes of one launch of an expert-stage kernel: the weights it must read (the U
    distinct routed experts touched, each once, and the shared expert) plus the activations it
    must read or write. Intermediates (h, partial sums, routing tables) are not counted."""
    esz, wsz, ssz = sizes(w)
    H, I, Is, T = w.hidden, w.inter, w.shared_inter, w.tokens
    name = {"gateup_wide": "gateup", "gateup_big": "gateup", "gateup_grp": "gateup", "gateup_gemv": "gateup",
            "down_wide": "down", "down_big": "down", "down_grp": "down", "down_rows": "down"}.get(name, name)
    if name == "gateup":
        return 2 * wsz * H * Is + 2 * ssz * Is + U * (2 * wsz * H * I + 2 * ssz * I) + esz * T * H
    if name == "down":
        return wsz * H * Is + ssz * H + U * (wsz * H * I + ssz * H) + 4 * T * H
    if name == "expert":
        return 3 * esz * H * Is + U * 3 * esz * H * I + esz * T * H
    if name == "decode":  # the single launch does the whole step
        return step_bytes(w, U)
    raise KeyError(name)


def kernel_sources_hash():
    """sha256[:16] over the HIP sources, as recorded with the committed counter summaries."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "sparse_moe_routing_amd", "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def counter_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from profiles/pmc_<workload>.txt (FETCH_SIZE + WRITE_SIZE,
    each scaled by what the counter reads for a plain 256 MiB copy), or None when there is no
    summary or the kernels have changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"pmc_{workload}.txt")
    if not os.path.exists(path):
        return None
    sha = None
    mib = None
    for line in open(path):
        parts = line.split()
        if len(parts) == 2 and parts[0] == "kernel_sources_sha16":
            sha = parts[1]
        if len(parts) >= 6 and parts[0] == "kernel" and parts[1] == f"{kernel}_kernel":
            mib = float(parts[-1])
    if sha != kernel_sources_hash() or mib is None:
        return None
    return mib * 2 ** 20


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, m_t, seconds):
    """The oracle (untuned) on the host: route + forward of fresh token batches of the workload's
    shapes, timed on every thread the process may use (OpenMP over tokens, so each batch holds
    at least one token per thread) and on one thread, about `seconds` each."""
    import oracle as oracle_mod
    import torch
    orc = oracle_mod.default()

    def host(a):
        if a is None:
            return None
        if a.dtype == torch.bfloat16:
            return a.view(torch.int16).cpu().numpy().view(np.uint16)
        return a.cpu().numpy()

    layer = {"num_experts": w.num_experts, "inter": w.inter, "shared_inter": w.shared_inter,
             "dtype": w.dtype}
    for k in ("router_w", "router_bias", "gate_up", "down", "shared_gate_up", "shared_down",
              "gate_up_scale", "down_scale", "shared_gate_up_scale", "shared_down_scale"):
        layer[k] = host(m_t.get(k))
    from sparse_moe_routing_amd import inputs
    try:
        allowed = len(os.sched_getaffinity(0))
    except AttributeError:
        allowed = os.cpu_count() or 1
    default_threads = orc.num_threads()  # OMP_NUM_THREADS, else the cores the process may use

    def run(threads, secs):
        orc.set_num_threads(threads)
        T = max(w.tokens, threads) if w.tokens <= 64 else 64
        T = (T + threads - 1) // threads * threads
        tokens = rounds = 0
        t0 = time.perf_counter()
        while True:
            layer["x"] = inputs.draw_x(w, T, seed=900 + rounds)
            z = orc.logits(layer["x"], layer["router_w"], layer["router_bias"])
            ids, wt, g = orc.select(z, w.num_experts, w.shared_inter > 0)
            orc.forward(layer, ids, wt, g)
            tokens += T
            rounds += 1
            el = time.perf_counter() - t0
            if el >= secs:
                break
        return tokens / el, rounds, T, el

    v_all, r_all, T_all, el_all = run(default_threads, seconds)
    v_one, r_one, T_one, el_one = run(1, max(2.0, seconds / 3))
    orc.set_num_threads(default_threads)
    return {"value": v_all, "unit": "tokens/s", "cores": default_threads, "kind": "oracle",
            "sample": f"{r_all} batches of {T_all} tokens of the {w.name} shapes (fresh x per "
                      f"batch, weight set 0), fp64 route+forward, {el_all:.1f} s on "
                      f"{default_threads} threads",
            "nproc": os.cpu_count(), "cpus_allowed": allowed, "cpu_model": _cpu_model(),
            "one_core": {"value": v_one, "unit": "tokens/s", "cores": 1,
                         "sample": f"{r_one} batches of {T_one} tokens, {el_one:.1f} s"}}


def read_ceiling(torch, nbytes, steps, stream):
    """This GPU's streaming-read rate for the step's byte count (GB/s), or None without the
    calibration library: libmoe_probe.so's kernel reads `nbytes` once per launch (grid-stride,
    16-byte non-temporal loads, one 512-thread block per compute unit), cycling over six such
    regions so that every read is cold as the weight sets are, `steps` launches back to back
    after five warm-up ones, synchronized on both sides - the same clock as the step's value."""
    import ctypes
    path = os.path.join(ROOT, "sparse_moe_routing_amd", "libmoe_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.moe_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p,
                                   ctypes.c_void_p]
    lib.moe_probe_read.restype = ctypes.c_int
    n = int(nbytes) // 256 * 256
    regions = 6
    buf = torch.ones(regions * n // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    blocks = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    s = ctypes.c_void_p(stream.cuda_stream)

    def launch(i):
        rc = lib.moe_probe_read(ctypes.c_void_p(buf.data_ptr() + (i % regions) * n), n, blocks,
                                ctypes.c_void_p(sink.data_ptr()), s)
        if rc:
            raise RuntimeError(f"moe_probe_read failed ({rc})")

    for i in range(5):
        launch(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        launch(5 + i)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    del buf
    return n / dt / 1e9


def measure(w, args, torch, log_prefix):
    """Warm-up, then K timed steps of plain moe_forward calls (wall clock, synchronized on both
    sides), then the same K steps once more with per-kernel events. Returns (result dict, the
    layer tensors of weight set 0)."""
    T, H = w.tokens, w.hidden
    log(f"[{log_prefix}] workload {w.name}: T={T} H={H} E={w.num_experts} I={w.inter} "
        f"Is={w.shared_inter} dtype={w.dtype}; {args.sets} weight sets, pool {args.pool}")
    sets = make_sets(w, args.sets, torch)
    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16  # x (fp8 workloads: bf16)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(77)
    pool = [torch.randn((T, H), generator=gen, device="cuda").to(dt) for _ in range(args.pool)]
    m0 = sets[0][0]
    ws = m0.workspace(T)
    y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    plan = m0.plan(T)
    n_ev = 2 * len(plan)  # each kernel's own start and end
    # distinct experts per (set, batch) pair, from the library's own routing (outside timing)
    U = {}
    for si, (m, _) in enumerate(sets):
        for pi, x in enumerate(pool):
            _, ids, _, _ = m.route(x=x, want_logits=False)
            U[(si, pi)] = int(torch.unique(ids).numel())
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def combo(i):
        return i % len(sets), (i // len(sets) + i) % len(pool)

    log(f"[{log_prefix}] plan {plan}; warmup {args.warmup}")
    for i in range(args.warmup):
        si, pi = combo(i)
        sets[si][0].forward(pool[pi], y=y, ws=ws)
    torch.cuda.synchronize()

    # timed region: K steps of plain moe_forward calls, synchronized on both sides
    used = [combo(args.warmup + i) for i in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for si, pi in used:
        sets[si][0].forward(pool[pi], y=y, ws=ws, stream=stream)
    t_enq = time.perf_counter()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    ms_per_step = elapsed * 1e3 / args.steps
    value = args.steps * T / elapsed

    # per-kernel durations: the same K steps again, each kernel launched with a start and a stop
    # event that its dispatch records (moe_forward_timed); not part of `value`
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
              for _ in range(args.steps)]
    for evs in events:  # torch creates the HIP event on its first record
        for e in evs:
            e.record(stream)
    torch.cuda.synchronize()
    for i, (si, pi) in enumerate(used):
        sets[si][0].forward(pool[pi], y=y, ws=ws, events=events[i], stream=stream)
    torch.cuda.synchronize()
    per_kernel = {name: [] for name in plan}
    step_ms = []
    for ev in events:
        for k, name in enumerate(plan):
            per_kernel[name].append(ev[2 * k].elapsed_time(ev[2 * k + 1]))
        step_ms.append(ev[0].elapsed_time(ev[-1]))
    mean_U = float(np.mean([U[c] for c in used]))
    stage = {}
    for name in ("gateup", "down", "gateup_wide", "gateup_big", "gateup_grp", "gateup_gemv", "down_wide",
                 "down_big", "down_grp", "down_rows", "expert"):
        if name in per_kernel:
            us = float(np.mean(per_kernel[name])) * 1e3
            b = float(np.mean([kernel_bytes(w, U[c], name) for c in used]))
            stage[name] = {"us": us, "bytes": b, "gbs": b / (us * 1e-6) / 1e9}
    dom = max(stage, key=lambda k: stage[k]["us"])  # the dominant kernel
    achieved = stage[dom]["gbs"]
    step_b = float(np.mean([step_bytes(w, U[c]) for c in used]))
    gpu_step_us = float(np.median(step_ms)) * 1e3
    ceiling = read_ceiling(torch, step_b, args.steps, stream)
    log(f"[{log_prefix}] per-kernel mean us: " + ", ".join(
        f"{k}={np.mean(v) * 1e3:.2f}" for k, v in per_kernel.items()))
    log(f"[{log_prefix}] wall {ms_per_step * 1e3:.2f} us/step (host enqueue "
        f"{(t_enq - t0) * 1e6 / args.steps:.1f} us/step), event-timed step median "
        f"{gpu_step_us:.2f} us, mean U {mean_U:.1f}, step bytes {step_b / 1e6:.1f} MB -> "
        f"{step_b / (ms_per_step * 1e-3) / 1e9:.0f} GB/s wall")
    if ceiling is not None:
        log(f"[{log_prefix}] streaming-read ceiling for {step_b / 1e6:.1f} MB cold: {ceiling:.0f} GB/s "
            f"-> the step at {step_b / (ms_per_step * 1e-3) / 1e9 / ceiling * 100:.1f} % of it")
    res = {
        "value": value, "unit": "tokens/s", "ms_per_step": ms_per_step, "dtype": w.dtype,
        "config": {"workload": w.name, "tokens": T, "hidden": H, "experts": w.num_experts,
                   "top_k": 8, "inter": w.inter, "shared_inter": w.shared_inter,
                   "router_bias_std": w.bias_std, "weight_sets": len(sets),
                   "x_pool": len(pool)},
        "hbm_gbs_step": step_b / (ms_per_step * 1e-3) / 1e9,
        "hbm_frac_step": step_b / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "step_bytes": step_b,
        "mean_distinct_experts": mean_U,
        "host_enqueue_us_per_step": (t_enq - t0) * 1e6 / args.steps,
        "event_step_us_median": gpu_step_us,
        "event_step_us_p10_p90": [float(np.percentile(step_ms, 10)) * 1e3,
                                  float(np.percentile(step_ms, 90)) * 1e3],
        "read_ceiling_gbs": ceiling,
        "hbm_frac_of_read_ceiling": (None if ceiling is None else
                                     step_b / (ms_per_step * 1e-3) / 1e9 / ceiling),
        "per_kernel_us": {k: float(np.mean(v)) * 1e3 for k, v in per_kernel.items()},
        "expert_stage_gbs": {k: v["gbs"] for k, v in stage.items()},
        "roofline": {"scope": "kernel", "kernel": dom, "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": counter_traffic(w.name, dom),
                     "algorithmic_bytes": stage[dom]["bytes"], "launch_us": stage[dom]["us"]},
    }
    keep = sets[0][1]
    for m, _ in sets:
        m.close()
    del sets, pool, ws, y, events
    return res, keep


SUB_WORKLOADS = ("decode_b8_t32", "verify_skewed_t192")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the library has no "
              "multi-GPU path (expert parallelism is a design, not code)", file=sys.stderr)
        sys.exit(2)
    import torch
    from sparse_moe_routing_amd import binding, inputs
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    binding.load()
    w = inputs.BY_NAME[args.workload]
    main_res, set0 = measure(w, args, torch, "bench")
    subs = {}
    if not args.no_sub:
        for name in SUB_WORKLOADS:
            if name == w.name:
                continue
            sub_w = inputs.BY_NAME[name]
            r, _ = measure(sub_w, args, torch, "sub")
            subs[name] = r
            torch.cuda.empty_cache()
    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20) // 4
        a = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy of {args.calib_copy_mib} MiB done (3 launches)")
    result = {
        "metric": "MoE-layer tokens/s + achieved HBM GB/s (% of peak) at T=4, 32, 192",
        "value": main_res["value"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": main_res["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
    }
    for k in ("config", "hbm_gbs_step", "hbm_frac_step", "read_ceiling_gbs",
              "hbm_frac_of_read_ceiling", "step_bytes", "mean_distinct_experts",
              "host_enqueue_us_per_step", "event_step_us_median", "event_step_us_p10_p90",
              "per_kernel_us", "expert_stage_gbs", "roofline"):
        result[k] = main_res[k]
    if subs:
        result["sub_results"] = subs
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline (oracle, ~{args.cpu_seconds:.0f} s on all threads, then one)")
        result["cpu_baseline"] = cpu_baseline(w, set0, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
