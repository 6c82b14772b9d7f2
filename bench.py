"""Benchmark of the small-batch NVFP4 MoE decode layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload flint_b1]

A step is one MoE layer call (router GEMV + routing, gate/up GEMV with
SiLU*up, down GEMV with weighted combine, all in one kernel launch) over one
batch of seeded synthetic tokens.  Weights stay cold: the layer is copied into L distinct device slots
(47 by default, one per MoE layer of the Flint model) and step i uses slot
i % L with its own input, so the touched bytes of a cycle (~631 MB at batch
1) exceed the 256 MB Infinity Cache plus the 32 MB of L2.

The timed region replays a HIP graph of the K steps (captured once, after W
eager warm-up steps and one untimed replay), bracketed by
torch.cuda.synchronize() and HIP events on the stream the kernels run on.
A step is one launch and the replayed launches run back to back, so the
region's time per step is the kernel's average launch duration, from which
the roofline figure is computed.  A second timed region runs the same K
steps eagerly with the library's profiling events around each launch (a
cross-check that also times the event packets and the dispatch).

Prints one JSON line.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=470)
    p.add_argument("--warmup", type=int, default=94)
    p.add_argument("--workload", default="flint_b1")
    p.add_argument("--slots", type=int, default=47)
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle CPU baseline")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--no-graph", action="store_true")
    p.add_argument("--calib-copy-mb", type=int, default=1024,
                   help="size of a plain device copy run once after timing (HBM counter calibration)")
    return p.parse_args()


def algorithmic_bytes(wl, d_routed: float, batch: int) -> dict:
    """Bytes one layer step must move (selected experts deduplicated)."""
    H, I = wl.hidden, wl.inter
    def expert(wtype):
        if wtype == "nvfp4":
            return {"w13": 2 * I * H // 2 + 2 * I * H // 16 + 4, "w2": H * I // 2 + H * I // 16 + 4}
        return {"w13": 2 * I * H * 2, "w2": H * I * 2}
    r, s = expert(wl.routed_wtype), expert(wl.shared_wtype)
    er = wl.n_routed + (wl.n_shared if wl.route == "sink" else 0)
    router = er * H * 2
    x_io = batch * H * 2
    k1 = router + wl.n_shared * s["w13"] + x_io
    k2 = d_routed * r["w13"] + x_io
    k3 = d_routed * r["w2"] + wl.n_shared * s["w2"] + x_io
    total = router + d_routed * (r["w13"] + r["w2"]) + wl.n_shared * (s["w13"] + s["w2"]) + 2 * x_io
    return {"k1": k1, "k2": k2, "k3": k3, "total": total}


def cpu_baseline(layer, xs, budget_s: float, algo_total: float) -> dict:
    """The oracle as it stands, on host cores, over a bounded sample of the
    workload's steps (inputs of the first slots)."""
    import oracle
    from threadpoolctl import threadpool_info

    class Cached:                     # experts generated once, outside the timed loop
        def __init__(self, base):
            self._b, self._r, self._s = base, {}, {}

        def __getattr__(self, n):
            return getattr(self._b, n)

        def routed_expert(self, e):
            if e not in self._r:
                self._r[e] = self._b.routed_expert(e)
            return self._r[e]

        def shared_expert(self, s):
            if s not in self._s:
                self._s[s] = self._b.shared_expert(s)
            return self._s[s]

    lay = Cached(layer)
    n = 0
    for x in xs[:4]:                  # populate the expert cache (untimed)
        oracle.moe_layer(lay, x)
    t0 = time.perf_counter()
    while True:
        oracle.moe_layer(lay, xs[n % len(xs)])
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 10 * len(xs):
            break
    per = el / n
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": algo_total / per / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} layer-steps (inputs of {min(n, len(xs))} slots) of the same workload in "
                      f"{el:.1f} s; {per * 1e3:.1f} ms per layer-step; expert generation excluded",
            "ms_per_step": per * 1e3}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (this build has no "
              "multi-GPU path: the layer would shard by splitting each expert's intermediate "
              "dimension across GPUs, see DESIGN.md)", file=sys.stderr)
        sys.exit(2)
    import torch
    from quantized_expert_gemv_amd import binding as B
    from quantized_expert_gemv_amd.device_layer import DeviceLayer, bits_to_bf16_tensor
    from quantized_expert_gemv_amd.synth import WORKLOADS, SynthLayer

    wl = WORKLOADS[args.workload]
    batch = wl.batch
    L = args.slots
    dev_name = torch.cuda.get_device_name(0)
    print(f"[bench] {wl.description}; {L} cold slots; device {dev_name}", file=sys.stderr, flush=True)
    layer = SynthLayer(wl)
    dev = DeviceLayer(layer, max_batch=batch)
    base = dev.buffers()
    slots = [base] + [{k: (v.clone() if v is not None else None) for k, v in base.items()} for _ in range(L - 1)]
    xs_bits = [layer.x(step=s) for s in range(L)]
    xs = [bits_to_bf16_tensor(x, dev.device) for x in xs_bits]
    outs = [torch.empty((batch, wl.hidden), dtype=torch.bfloat16, device=dev.device) for _ in range(L)]
    torch.cuda.synchronize()
    print(f"[bench] slots ready: {sum(v.numel() for v in base.values() if v is not None) * L / 1e9:.1f} GB "
          "resident", file=sys.stderr, flush=True)

    def step(i, stream=None):
        s = i % L
        dev(xs[s], out=outs[s], bufs=slots[s], stream=stream)

    # distinct routed experts per slot
    d_per_slot = []
    for s in range(L):
        step(s)
        ids, _, _ = dev.routing(batch)
        d_per_slot.append(len(set(ids.cpu().numpy().ravel().tolist())))
    K, W = args.steps, args.warmup
    d_avg = float(np.mean([d_per_slot[i % L] for i in range(K)]))
    algo = algorithmic_bytes(wl, d_avg, batch)

    for i in range(W):
        step(i)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    mode = "eager"
    if not args.no_graph:
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                for i in range(K):
                    step(W + i)
        stream.wait_stream(cap)
        g.replay()                       # untimed first replay
        torch.cuda.synchronize()
        mode = "hipgraph"
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    if mode == "hipgraph":
        g.replay()
    else:
        for i in range(K):
            step(W + i)
    ev1.record(stream)
    torch.cuda.synchronize()
    total_ms = ev0.elapsed_time(ev1)
    us_step = total_ms * 1e3 / K
    print(f"[bench] timed {K} steps ({mode}): {us_step:.2f} us/step", file=sys.stderr, flush=True)

    # second timed region: eager, with events around each launch
    n_ev = 2 * K
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    for e in evs:
        e.record(stream)                # materialise the underlying HIP events
    torch.cuda.synchronize()
    ev_ptrs = (B.C.c_void_p * n_ev)(*[e.cuda_event for e in evs])
    B.moe_layer_set_profiling(dev.handle, ev_ptrs, n_ev)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(W + i)
    torch.cuda.synchronize()
    eager_wall = time.perf_counter() - t0
    B.moe_layer_set_profiling(dev.handle, None, 0)
    d = np.array([evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(K)])
    kern = {"layer_kernel_us": float(d.mean() * 1e3), "layer_kernel_us_p50": float(np.median(d) * 1e3),
            "eager_us_per_step": eager_wall * 1e6 / K}
    print(f"[bench] layer kernel (eager, events): {kern}", file=sys.stderr, flush=True)
    flags = dev.error()
    if flags:
        raise SystemExit(f"[bench] the layer kernel reported error bits {flags:#x}")

    # plain copy of known size, for HBM counter calibration under rocprofv3 --pmc
    if args.calib_copy_mb > 0:
        n = args.calib_copy_mb * (1 << 20)
        a = torch.empty(n, dtype=torch.uint8, device=dev.device)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    gbs = algo["total"] / (us_step * 1e-6) / 1e9
    roof = None
    if kern is not None:
        # A layer step is one launch and graph-replayed launches run back to
        # back (no gaps in rocprofv3's kernel trace), so the timed region's
        # events give the average launch duration.  The eager per-launch
        # events (kernels.layer_kernel_us) also time the event packets and
        # the dispatch, and stay a cross-check.
        k_us = us_step if mode == "hipgraph" else kern["layer_kernel_us"]
        achieved = algo["total"] / (k_us * 1e-6) / 1e9
        traffic = None
        tf = os.path.join(ROOT, "profiles", f"traffic_{args.workload}.json")
        if os.path.exists(tf):
            with open(tf) as fh:
                t = json.load(fh)
            from quantized_expert_gemv_amd.profiling import src_digest
            if t.get("src_digest") == src_digest():
                traffic = t.get("dominant_bytes_per_launch")
        roof = {"bound": "hbm", "kernel": "k_fused_layer", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "algorithmic_bytes_per_launch": int(round(algo["total"])),
                "launch_us": round(k_us, 3),
                "launch_us_source": ("events around the graph-replayed timed region / launches"
                                     if mode == "hipgraph" else "events around each eager launch")}

    cpu = None
    if not args.no_cpu:
        print("[bench] oracle cpu baseline ...", file=sys.stderr, flush=True)
        cpu = cpu_baseline(layer, xs_bits, args.cpu_seconds, algo["total"])

    line = {
        "metric": "MoE layer us/step + achieved HBM GB/s, NVFP4 W4A16 H=2048 E=256 top-6",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(us_step / 1e3, 6), "us_per_step": round(us_step, 3),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "nvfp4-w/bf16-a/f32-acc" if wl.routed_wtype == "nvfp4" else "bf16-w/bf16-a/f32-acc",
        "data": "synthetic (seeded; no checkpoint)",
        "config": {"workload": wl.description, "hidden": wl.hidden, "inter": wl.inter,
                   "n_routed": wl.n_routed, "top_k": wl.top_k, "n_shared": wl.n_shared, "batch": batch,
                   "cold_slots": L, "timing": mode, "distinct_routed_per_step": d_avg,
                   "algorithmic_bytes_per_step": int(round(algo["total"])), "device": dev_name},
        "kernels": kern, "roofline": roof, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
