"""Benchmark of the small-batch NVFP4 MoE decode layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload flint_b1] [--extra flint_b8] [--all]

A step is one MoE layer call (router GEMV + routing, gate/up GEMV with
SiLU*up, down GEMV with weighted combine, all in one kernel launch) over one
batch of seeded synthetic tokens.  Weights stay cold: the layer is copied
into L distinct device slots (47 by default, one per MoE layer of the Flint
model) and step i uses slot i % L with its own input.  One cycle over the
slots (~631 MB at batch 1) exceeds the 256 MB Infinity Cache plus the 32 MB
of L2, and a 1 GiB read pass runs before the timed region.

Before the first workload, 0.5 s of untimed read passes (--gpu-warmup-ms)
let the GPU's clocks settle under load.

Timed region: W eager warm-up steps and one untimed launch of each graph
below (a graph's first launch also uploads it); then, after the read pass, one
untimed replay of a graph of the L steps 0 .. L-1 and right behind it a HIP
graph of exactly the K steps (W + i) % L, replayed once between HIP events on
the stream the kernels run on.  The untimed cycle leaves the page translations
and caches as a running model leaves them; each timed step's weights were
last touched about L - W steps (over 500 MB of other weights) earlier, so
they come from HBM whatever K is.  A step is one launch and replayed launches run
back to back, so the region's time per step is the layer kernel's average
launch duration (the roofline figure uses it).  Also reported:
  * replays: a graph of one full cycle of L steps replayed R times, each
    replay between events: p10 / p50 / p90 of elapsed / L;
  * eager: the library's profiling events around each of L eager launches
    (they also time the event packets and the dispatch);
  * the measured HBM read-stream ceiling (4 GiB read once, best of 3) and
    the per-launch floor (an empty 256-workgroup kernel, 200 launches in a
    graph);
  * the fp64 oracle on the host's cores at 1 thread and at all threads.
Other workloads (--extra, default: Flint b8, the 2-bit planes at b1 and b8,
BF16 experts at b1 and b8, the expert-sink layer at b4, a 16-layer chain in
one launch, the dense QKV GEMV at batch 1 and 8, and the prefill of 1024 and
8192 tokens with NVFP4 and with 2-bit routed experts) are measured the same
way and reported under "configs" in the same JSON line.

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
SLOTS = {"tiny": 1024, "sink_b4": 4, "flint_chain16_b1": 48}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=470)
    p.add_argument("--warmup", type=int, default=94)
    p.add_argument("--workload", default="flint_b1")
    p.add_argument("--extra", default="flint_b8,flint_2bit_b1,flint_2bit_b8,flint_bf16_b1,flint_bf16_b8,sink_b4,"
                                      "flint_chain16_b1,dense_qkv_b1,dense_qkv_b8,flint_prefill_t1024,flint_prefill_t8192,"
                                      "flint_2bit_prefill_t1024,flint_2bit_prefill_t8192",
                   help="comma-separated extra workloads ('' for none)")
    p.add_argument("--all", action="store_true", help="also the tiny workload")
    p.add_argument("--slots", type=int, default=47)
    p.add_argument("--gpu-warmup-ms", type=int, default=500,
                   help="untimed read passes before the first measurement (0: none)")
    p.add_argument("--replays", type=int, default=8)
    p.add_argument("--cpu-seconds", type=float, default=16.0, help="budget of the oracle CPU baseline")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--calib-copy-mb", type=int, default=1024,
                   help="size of a plain device copy run once after timing (HBM counter calibration)")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic_bytes(wl, d_routed: float, batch: int) -> dict:
    """Bytes one layer step must move (selected experts deduplicated)."""
    H, I = wl.hidden, wl.inter

    def expert(wtype):
        if wtype == "2bit":
            return {"w13": 2 * I * H // 4 + 2 * I * H // 16 + 4, "w2": H * I // 4 + H * I // 16 + 4}
        if wtype == "nvfp4":
            return {"w13": 2 * I * H // 2 + 2 * I * H // 16 + 4, "w2": H * I // 2 + H * I // 16 + 4}
        return {"w13": 2 * I * H * 2, "w2": H * I * 2}
    r, s = expert(wl.routed_wtype), expert(wl.shared_wtype)
    er = wl.n_routed + (wl.n_shared if wl.route == "sink" else 0)
    router = er * H * 2
    x_io = batch * H * 2
    gamma = H * 2 if wl.prenorm else 0
    total = router + d_routed * (r["w13"] + r["w2"]) + wl.n_shared * (s["w13"] + s["w2"]) + 2 * x_io + gamma
    return {"router": router, "routed": d_routed * (r["w13"] + r["w2"]),
            "shared": wl.n_shared * (s["w13"] + s["w2"]), "total": total}


def cpu_info() -> dict:
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count()
    return {"nproc": avail, "cpu_count": os.cpu_count(), "model": model}


def cpu_baseline(layer, xs, budget_s: float, algo_total: float) -> dict:
    """The oracle as it stands, on host cores, over a bounded sample of the
    workload's steps (inputs of the first slots), at 1 thread and at all."""
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits

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
    for x in xs[:4]:                  # populate the expert cache (untimed)
        oracle.moe_layer(lay, x)

    def run(seconds):
        n, t0 = 0, time.perf_counter()
        while True:
            oracle.moe_layer(lay, xs[n % len(xs)])
            n += 1
            el = time.perf_counter() - t0
            if el >= seconds or n >= 10 * len(xs):
                return n, el

    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    n_all, el_all = run(budget_s / 2)
    with threadpool_limits(1):
        n_one, el_one = run(budget_s / 2)
    per_all, per_one = el_all / n_all, el_one / n_one
    info = cpu_info()
    return {"value": algo_total / per_all / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n_all} layer-steps (inputs of {min(n_all, len(xs))} slots) of the same workload in "
                      f"{el_all:.1f} s at {threads} BLAS threads, {n_one} in {el_one:.1f} s at 1 thread; "
                      "expert generation excluded",
            "ms_per_step": per_all * 1e3, "ms_per_step_1thread": per_one * 1e3,
            "value_1thread": algo_total / per_one / 1e9, "threads": int(threads), **info}


def measure(name: str, K: int, W: int, L: int, R: int, flush) -> dict:
    """Cold-weight timing of one workload; returns its record and the layer."""
    import torch
    from quantized_expert_gemv_amd import binding as B
    from quantized_expert_gemv_amd.device_layer import DeviceLayer, bits_to_bf16_tensor
    from quantized_expert_gemv_amd.synth import WORKLOADS, SynthLayer

    wl = WORKLOADS[name]
    batch = wl.batch
    log(f"{wl.description}; {L} cold slots")
    layer = SynthLayer(wl)
    dev = DeviceLayer(layer, max_batch=batch)
    # the kernel the calls run: the kernels dedicated to the Flint shape where the layer has them
    dedicated = dev.set_path("auto") == "dedicated"
    kernel = ("k_b1_layer" if batch == 1 else "k_b8_layer") if dedicated else "k_fused_layer"
    base = dev.buffers()
    slots = [base] + [{k: (v.clone() if v is not None else None) for k, v in base.items()} for _ in range(L - 1)]
    xs_bits = [layer.x(step=s) for s in range(L)]
    xs = [bits_to_bf16_tensor(x, dev.device) for x in xs_bits]
    outs = [torch.empty((batch, wl.hidden), dtype=torch.bfloat16, device=dev.device) for _ in range(L)]
    torch.cuda.synchronize()
    resident = sum(v.numel() for v in base.values() if v is not None) * L
    log(f"slots ready: {resident / 1e9:.1f} GB resident")

    def step(i):
        s = i % L
        dev(xs[s], out=outs[s], bufs=slots[s])

    d_per_slot = []
    for s in range(L):                    # distinct routed experts per slot
        step(s)
        ids, _, _ = dev.routing(batch)
        d_per_slot.append(len(set(ids.cpu().numpy().ravel().tolist())))
    d_timed = float(np.mean([d_per_slot[(W + i) % L] for i in range(K)]))
    algo = algorithmic_bytes(wl, d_timed, batch)

    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def capture(first, n):
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                for i in range(n):
                    step(first + i)
        stream.wait_stream(cap)
        torch.cuda.synchronize()
        return g

    gK = capture(W, K)
    gL = capture(0, L)
    gK.replay()                   # each graph's first launch uploads it: keep that out of the timed region
    gL.replay()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    flush()
    gL.replay()                   # one untimed cycle over the slots, then the timed steps right behind it
    ev0.record(stream)
    gK.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    us_step = ev0.elapsed_time(ev1) * 1e3 / K
    del gK
    log(f"timed {K} steps (hipgraph, cold): {us_step:.3f} us/step")

    gL.replay()
    torch.cuda.synchronize()
    per = []
    for _ in range(R):
        ev0.record(stream)
        gL.replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        per.append(ev0.elapsed_time(ev1) * 1e3 / L)
    del gL
    per = np.array(per)
    replays = {"n": R, "steps_per_replay": L, "p10_us": float(np.percentile(per, 10)),
               "p50_us": float(np.percentile(per, 50)), "p90_us": float(np.percentile(per, 90))}
    log(f"replays of {L} steps: {replays}")

    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * L)]
    for e in evs:
        e.record(stream)                  # materialise the underlying HIP events
    torch.cuda.synchronize()
    ev_ptrs = (B.C.c_void_p * (2 * L))(*[e.cuda_event for e in evs])
    B.moe_layer_set_profiling(dev.handle, ev_ptrs, 2 * L)
    for i in range(L):
        step(i)
    torch.cuda.synchronize()
    B.moe_layer_set_profiling(dev.handle, None, 0)
    d = np.array([evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(L)]) * 1e3
    eager = {"mean_us": float(d.mean()), "p10_us": float(np.percentile(d, 10)), "p50_us": float(np.median(d))}
    flags = dev.error()
    if flags:
        raise SystemExit(f"[bench] the layer kernel reported error bits {flags:#x} on {name}")

    gbs = algo["total"] / (us_step * 1e-6) / 1e9
    rec = {"workload": wl.description, "batch": batch, "kernel": kernel,
           "us_per_step": round(us_step, 3), "gbs": round(gbs, 1),
           "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "cold_slots": L, "timing": "hipgraph, cold",
           "distinct_routed_per_step": d_timed, "algorithmic_bytes_per_step": int(round(algo["total"])),
           "bytes_breakdown": {k: int(round(v)) for k, v in algo.items()},
           "replays": replays, "eager_per_launch": eager, "resident_gb": round(resident / 1e9, 2)}
    del slots, xs, outs, base
    dev.close()
    del dev
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec, layer, xs_bits


# Dense NVFP4 GEMVs of a Flint-shaped decode step (hidden 2048, 32 query and 4
# KV heads of 64): the fused QKV projection.  name -> (rows, cols, batch)
DENSE = {"dense_qkv_b1": (2560, 2048, 1), "dense_qkv_b8": (2560, 2048, 8)}


def measure_dense(name: str, K: int, W: int, L: int, R: int, flush) -> dict:
    """Cold-weight timing of the dense GEMV on L device copies of one matrix."""
    import torch
    from quantized_expert_gemv_amd import binding as B
    rows, cols, batch = DENSE[name]
    log(f"dense NVFP4 GEMV {rows}x{cols}, batch {batch}; {L} cold slots")
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    scales = rng.integers(0x30, 0x41, size=(rows, cols // 16), dtype=np.uint8)
    cr, sr = B.moe_pack_dense(codes, scales, 0.37)
    dev = torch.device("cuda")
    slots = [(torch.from_numpy(cr).to(dev), torch.from_numpy(sr).to(dev)) for _ in range(L)]
    f = rng.standard_normal((batch, cols)).astype(np.float32).view(np.uint32).astype(np.uint64)
    xb = ((f + 0x7FFF + ((f >> 16) & 1)) >> 16).astype(np.uint16)
    x = torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16)
    ys = [torch.empty((batch, rows), dtype=torch.bfloat16, device=dev) for _ in range(L)]
    stream = torch.cuda.current_stream()

    def step(i):
        c, sc = slots[i % L]
        B.moe_dense_gemv(rows, cols, c, sc, x, ys[i % L], batch)

    for i in range(W):
        step(i)
    torch.cuda.synchronize()

    def capture(first, n):
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                for i in range(n):
                    step(first + i)
        stream.wait_stream(cap)
        torch.cuda.synchronize()
        return g

    gK = capture(W, K)
    gL = capture(0, L)
    gK.replay()                   # each graph's first launch uploads it: keep that out of the timed region
    gL.replay()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    flush()
    gL.replay()                   # one untimed cycle over the slots, then the timed steps right behind it
    ev0.record(stream)
    gK.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / K
    del gK
    gL.replay()
    torch.cuda.synchronize()
    per = []
    for _ in range(R):
        ev0.record(stream)
        gL.replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        per.append(ev0.elapsed_time(ev1) * 1e3 / L)
    del gL
    per = np.array(per)
    lay_bytes = cr.nbytes + sr.nbytes + x.numel() * 2 + batch * rows * 2
    algo = lay_bytes
    gbs = algo / (us * 1e-6) / 1e9
    log(f"timed {K} GEMVs (hipgraph, cold): {us:.3f} us each, {gbs:.0f} GB/s")
    del slots, ys
    torch.cuda.empty_cache()
    return {"workload": f"dense NVFP4 GEMV [{rows}x{cols}] (fused QKV of a Flint-shaped layer), b{batch}",
            "kernel": "k_dense_gemv", "batch": batch, "us_per_step": round(us, 3), "gbs": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "cold_slots": L, "timing": "hipgraph, cold",
            "algorithmic_bytes_per_step": int(lay_bytes),
            "replays": {"n": R, "steps_per_replay": L, "p10_us": float(np.percentile(per, 10)),
                        "p50_us": float(np.percentile(per, 50)), "p90_us": float(np.percentile(per, 90))}}


# Layer chains: one moe_decode_chain launch runs n pre-norm residual layers of
# the Flint shape at batch 1.  name -> n
CHAIN = {"flint_chain16_b1": 16}


def measure_chain(name: str, K: int, W: int, L: int, R: int, flush) -> dict:
    """Cold-weight timing of an n-layer chain: L device slots (a multiple of n),
    chain step j runs the n consecutive slots of group j % (L / n)."""
    import torch
    from quantized_expert_gemv_amd import binding as B
    from quantized_expert_gemv_amd.device_layer import DeviceLayer, bits_to_bf16_tensor
    from quantized_expert_gemv_amd.synth import WORKLOADS, SynthLayer

    n = CHAIN[name]
    L = max(n, L - L % n)
    groups = L // n
    wl = WORKLOADS["flint_chain"]
    log(f"{n}-layer chain of: {wl.description}; {L} cold slots")
    layer = SynthLayer(wl)
    dev = DeviceLayer(layer, max_batch=1)
    if dev.set_path("auto") != "dedicated":
        dev.close()
        return {"workload": f"{n}-layer chain", "skipped": "the chain needs the batch-1 kernel of the Flint shape"}
    base = dev.buffers()
    slots = [base] + [{k: (v.clone() if v is not None else None) for k, v in base.items()} for _ in range(L - 1)]
    xs = [bits_to_bf16_tensor(layer.x(step=j), dev.device) for j in range(groups)]
    outs = [torch.empty((1, wl.hidden), dtype=torch.bfloat16, device=dev.device) for _ in range(groups)]
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def step(i):
        j = i % groups
        sl = slots[j * n:(j + 1) * n]
        B.moe_decode_chain([dev.handle] * n, xs[j], [b["router_w"] for b in sl], [b["expert_packed"] for b in sl],
                           [b["scales"] for b in sl], [b["shared_w"] for b in sl], outs[j], 1)

    for i in range(W):
        step(i)
    torch.cuda.synchronize()

    def capture(first, m):
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                for i in range(m):
                    step(first + i)
        stream.wait_stream(cap)
        torch.cuda.synchronize()
        return g

    Kc = max(1, K // n)                   # about K layers in the timed region
    gK = capture(W, Kc)
    gL = capture(0, groups)
    gK.replay()                   # each graph's first launch uploads it: keep that out of the timed region
    gL.replay()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    flush()
    gL.replay()                   # one untimed cycle over the slots, then the timed chains right behind it
    ev0.record(stream)
    gK.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    us_chain = ev0.elapsed_time(ev1) * 1e3 / Kc
    del gK
    gL.replay()
    torch.cuda.synchronize()
    per = []
    for _ in range(R):
        ev0.record(stream)
        gL.replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        per.append(ev0.elapsed_time(ev1) * 1e3 / groups)
    del gL
    per = np.array(per)
    # the same layers launched one by one (the single-layer kernel), for comparison
    ys = [torch.empty((1, wl.hidden), dtype=torch.bfloat16, device=dev.device) for _ in range(L)]

    def single(i):
        s = i % L
        j = s // n
        dev(xs[j] if s % n == 0 else ys[s - 1], out=ys[s], bufs=slots[s])

    for i in range(L):
        single(i)
    torch.cuda.synchronize()
    gS = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        with torch.cuda.graph(gS, stream=cap):
            for i in range(L):
                single(i)
    stream.wait_stream(cap)
    torch.cuda.synchronize()
    gS.replay()
    torch.cuda.synchronize()
    per_s = []
    for _ in range(R):
        ev0.record(stream)
        gS.replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        per_s.append(ev0.elapsed_time(ev1) * 1e3 / L)
    del gS
    # the chain's output equals the layers' one by one
    same = all(torch.equal(outs[j].view(torch.int16), ys[(j + 1) * n - 1].view(torch.int16)) for j in range(groups))
    singles_us = float(np.median(per_s))
    log(f"same layers one launch each: {singles_us:.3f} us/layer; chain output equal to them: {same}")
    flags = dev.error()
    if flags:
        raise SystemExit(f"[bench] the chain kernel reported error bits {flags:#x}")
    if not same:
        raise SystemExit("[bench] the chain's output differs from its layers run one by one")
    lay = algorithmic_bytes(wl, float(wl.top_k), 1)
    x_io = wl.hidden * 2
    algo = n * (lay["total"] - 2 * x_io) + 2 * x_io     # x read once and the last output written once
    gbs = algo / (us_chain * 1e-6) / 1e9
    log(f"timed {Kc} chains of {n} (hipgraph, cold): {us_chain:.3f} us/chain, {us_chain / n:.3f} us/layer, "
        f"{gbs:.0f} GB/s")
    del slots, xs, outs, base, ys
    dev.close()
    del dev
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return {"workload": f"{n}-layer chain, one launch: {wl.description}", "kernel": "k_b1_layer", "batch": 1,
            "layers_per_launch": n, "us_per_launch": round(us_chain, 3), "us_per_layer": round(us_chain / n, 3),
            "gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "cold_slots": L,
            "timing": "hipgraph, cold", "launches_timed": Kc, "algorithmic_bytes_per_launch": int(round(algo)),
            "replays": {"n": R, "launches_per_replay": groups, "p10_us": float(np.percentile(per, 10)),
                        "p50_us": float(np.percentile(per, 50)), "p90_us": float(np.percentile(per, 90))},
            "one_launch_per_layer_us": round(singles_us, 3),
            "one_launch_per_layer_timing": f"graph of the same {L} layers, one launch each, replayed {R} times, p50"}


# Prefill of T tokens through the Flint-shaped NVFP4 layer (moe_prefill_layer:
# grouped GEMMs on the matrix cores).  name -> T
PREFILL = {"flint_prefill_t1024": ("flint_b1", 1024), "flint_prefill_t8192": ("flint_b1", 8192),
           "flint_2bit_prefill_t1024": ("flint_2bit_b1", 1024), "flint_2bit_prefill_t8192": ("flint_2bit_b1", 8192)}
MFMA_BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 matrix peak


def measure_prefill(name: str, K: int, W: int, R: int, flush) -> dict:
    """Prefill calls over two device copies of the layer (a call touches every
    expert: ~453 MB, above the 256 MB Infinity Cache), timed as a graph of K
    calls between HIP events after the read pass."""
    import torch
    from quantized_expert_gemv_amd import binding as B
    from quantized_expert_gemv_amd.device_layer import DeviceLayer, bits_to_bf16_tensor
    from quantized_expert_gemv_amd.synth import WORKLOADS, SynthLayer

    wname, T = PREFILL[name]
    wl = WORKLOADS[wname]
    log(f"prefill of {T} tokens: {wl.description}")
    layer = SynthLayer(wl)
    dev = DeviceLayer(layer, max_batch=1)
    base = dev.buffers()
    slots = [base, {k: (v.clone() if v is not None else None) for k, v in base.items()}]
    xs = [bits_to_bf16_tensor(layer.x(step=j, batch=T), dev.device) for j in range(2)]
    outs = [torch.empty((T, wl.hidden), dtype=torch.bfloat16, device=dev.device) for _ in range(2)]
    need = B.moe_prefill_workspace_bytes(dev.handle, T)
    ws = torch.empty(need, dtype=torch.uint8, device=dev.device)
    ids = torch.empty((T, wl.top_k), dtype=torch.int32, device=dev.device)
    stream = torch.cuda.current_stream()

    def step(i, routing=False):
        j = i % 2
        b = slots[j]
        B.moe_prefill_layer(dev.handle, xs[j], b["router_w"], b["expert_packed"], b["scales"], b["shared_w"],
                            outs[j], T, ws, need, ids if routing else None, None, None)

    distinct = []
    for j in range(2):
        step(j, routing=True)
        torch.cuda.synchronize()
        distinct.append(len(set(ids.cpu().numpy().ravel().tolist())))
    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            for i in range(K):
                step(i)
    stream.wait_stream(cap)
    torch.cuda.synchronize()
    g.replay()                        # the graph's first launch uploads it
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    per = []
    for _ in range(R):
        torch.cuda.synchronize()
        flush()                       # queued ahead of the timed calls: they start as it ends
        ev0.record(stream)
        g.replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        per.append(ev0.elapsed_time(ev1) * 1e3 / K)
    del g
    us = float(np.median(per))
    H, I, E, k, S = wl.hidden, wl.inter, wl.n_routed, wl.top_k, wl.n_shared
    d = float(np.mean(distinct))
    lay = algorithmic_bytes(wl, d, T)
    flops = 2.0 * T * E * H + 2.0 * T * (k + S) * (2 * I * H + H * I)
    gbs = lay["total"] / (us * 1e-6) / 1e9
    tfs = flops / (us * 1e-6) / 1e12
    bound = "mfma" if flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) > lay["total"] / (HBM_PEAK_GBS * 1e9) else "hbm"
    frac = tfs / MFMA_BF16_PEAK_TFLOPS if bound == "mfma" else gbs / HBM_PEAK_GBS
    log(f"prefill T={T}: {us:.1f} us/call, {T / (us * 1e-6):.3g} tokens/s, {tfs:.1f} TFLOP/s, {gbs:.0f} GB/s "
        f"({bound}-bound roofline frac {frac:.3f})")
    del slots, xs, outs, ws, base
    dev.close()
    del dev
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return {"workload": f"prefill of {T} tokens, {wl.description.replace(', b1', '')}", "tokens": T,
            "kernels": "k_pf_logits, k_pf_topk, k_pf_count, k_pf_place, k_pf_gateup, k_pf_down, k_pf_combine",
            "us_per_call": round(us, 2), "tokens_per_s": round(T / (us * 1e-6), 1), "tflops": round(tfs, 2),
            "gbs": round(gbs, 1), "bound": bound, "roofline_frac": round(frac, 4),
            "flops_per_call": flops, "algorithmic_bytes_per_call": int(round(lay["total"])),
            "distinct_routed": d, "timing": f"graph of {K} calls over 2 weight copies, after the read pass, "
                                            f"p50 of {R} replays", "workspace_bytes": need}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the layer runs on one GPU "
              "(sharding it over several, tensor-parallel inside the experts with one all-reduce of the "
              "output, is a design, not built)", file=sys.stderr)
        sys.exit(2)
    import torch
    from quantized_expert_gemv_amd import binding as B
    from quantized_expert_gemv_amd.synth import WORKLOADS

    dev_name = torch.cuda.get_device_name(0)
    log(f"device {dev_name}")
    flush_buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    B.moe_bench_fill(flush_buf, 0x5a5a5a5a)
    flush_sink = torch.zeros(16, dtype=torch.int32, device="cuda")

    def flush():
        # a 1 GiB read pass: it evicts the weights from the L2s and the
        # Infinity Cache and, unlike a write pass, leaves no dirty lines whose
        # write-back would run during the timed steps
        B.moe_bench_read_stream(flush_buf, flush_sink)

    # the GPU's clocks settle under load: read passes for a while before the
    # first measurement, so that it is taken at the same clocks as the later
    # ones (untimed, like the warm-up steps)
    if args.gpu_warmup_ms > 0:
        t_end = time.perf_counter() + args.gpu_warmup_ms * 1e-3
        while time.perf_counter() < t_end:
            flush()
            torch.cuda.synchronize()

    K, W = args.steps, args.warmup
    head, layer, xs_bits = measure(args.workload, K, W, SLOTS.get(args.workload, args.slots), args.replays, flush)
    extras = [n for n in args.extra.split(",") if n]
    if args.all:
        extras += [n for n in ("tiny",) if n not in extras]
    configs = {}
    for n in extras:
        if n in DENSE:
            configs[n] = measure_dense(n, K, W, args.slots, args.replays, flush)
            continue
        if n in PREFILL:
            configs[n] = measure_prefill(n, max(2, min(K, 20)), 2, args.replays, flush)
            continue
        if n in CHAIN:
            configs[n] = measure_chain(n, K, W, SLOTS.get(n, args.slots), args.replays, flush)
            continue
        if n == args.workload or n not in WORKLOADS:
            continue
        rec, _, _ = measure(n, K, W, SLOTS.get(n, args.slots), args.replays, flush)
        configs[n] = rec

    # measured HBM read-stream ceiling and per-launch floor
    sink = torch.zeros(16, dtype=torch.int32, device="cuda")
    big = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")
    B.moe_bench_fill(big, 0x01020304)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = 1e9
    for _ in range(3):
        flush()
        e0.record()
        B.moe_bench_read_stream(big, sink)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    ceiling = big.numel() / (best * 1e-3) / 1e9
    del big
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            for _ in range(200):
                B.moe_bench_empty(256)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    floor_us = e0.elapsed_time(e1) * 1e3 / 200
    log(f"HBM read-stream ceiling {ceiling:.0f} GB/s; empty-launch floor {floor_us:.3f} us")

    # plain copy of known size, for HBM counter calibration under rocprofv3 --pmc
    if args.calib_copy_mb > 0:
        n = args.calib_copy_mb * (1 << 20)
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    us_step = head["us_per_step"]
    achieved = head["gbs"]
    traffic = None
    tf = os.path.join(ROOT, "profiles", f"traffic_{args.workload}.json")
    if os.path.exists(tf):
        with open(tf) as fh:
            t = json.load(fh)
        from quantized_expert_gemv_amd.profiling import src_digest
        if t.get("src_digest") == src_digest():
            traffic = t.get("dominant_bytes_per_launch")
    roof = {"bound": "hbm", "kernel": head["kernel"], "achieved": achieved, "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "algorithmic_bytes_per_launch": head["algorithmic_bytes_per_step"],
            "launch_us": us_step,
            "launch_us_source": "events around a graph of the K timed launches (back to back, cold) / K",
            "measured_read_ceiling_gbs": round(ceiling, 1),
            "frac_of_measured_ceiling": round(achieved / ceiling, 4),
            "empty_launch_floor_us": round(floor_us, 3)}

    cpu = None
    if not args.no_cpu:
        log("oracle cpu baseline ...")
        cpu = cpu_baseline(layer, xs_bits, args.cpu_seconds, head["algorithmic_bytes_per_step"])

    wl = WORKLOADS[args.workload]
    line = {
        "metric": "MoE layer us/step + achieved HBM GB/s, NVFP4 W4A16 H=2048 E=256 top-6",
        "value": achieved, "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(us_step / 1e3, 6), "us_per_step": us_step, "hbm_frac": head["hbm_frac"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "nvfp4-w/bf16-a/f32-acc" if wl.routed_wtype == "nvfp4" else "bf16-w/bf16-a/f32-acc",
        "data": "synthetic (seeded; no checkpoint)",
        "config": {"workload": wl.description, "hidden": wl.hidden, "inter": wl.inter, "n_routed": wl.n_routed,
                   "top_k": wl.top_k, "n_shared": wl.n_shared, "batch": wl.batch, "cold_slots": head["cold_slots"],
                   "timing": head["timing"], "distinct_routed_per_step": head["distinct_routed_per_step"],
                   "algorithmic_bytes_per_step": head["algorithmic_bytes_per_step"], "device": dev_name},
        "replays": head["replays"], "eager_per_launch": head["eager_per_launch"],
        "roofline": roof, "cpu_baseline": cpu, "configs": configs,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
