"""Benchmark of one MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode] [--only]

A step is one colibri_moe_layer_forward (quantise, route, union dispatch,
gate/up + SiLU + requant, down, combine) over one batch of synthetic tokens
already resident in HBM.  The headline workload (--workload, default the
S = 1 decode layer: H = 6144, 256 experts of I = 2048, top-8, packed int4,
plus a shared expert) is timed for K steps; unless --only is given, the other
four workloads (tiny S = 8 int8, verify S = 4 int8, prefill S = 512 int4,
skewed S = 2048 int2) follow with their own step counts.  To keep the 256 MB
last-level cache from serving weights that a real model would have evicted,
consecutive steps rotate over several copies of the layer at distinct
addresses and over distinct token batches.

Prints one JSON line: the headline throughput (routed tokens/s per layer)
with a roofline object for its dominant kernel (timed with HIP events
recorded by the library between its stages on the benchmark's stream); per
workload, tokens/s with its HBM, int8 matrix-core and VALU-fold rooflines and
the binding one; the device's measured read-stream and int8 MFMA rates
beside the published peaks; and per workload a CPU baseline (the oracle,
single-threaded, pinned to one CPU, on a bounded sample of the batch).

    python bench.py --tier [--tier-fractions 1,0.5,0.25]

instead runs the layer with its routed experts in pinned host memory behind
an HBM slot bank (colibri_tier_forward) and prints decode tokens/s, expert
hit rate and host-to-device traffic per resident fraction, for uniform and
for Zipf-skewed routing.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
INT8_PEAK_TOPS = 5000.0      # MI355X dense int8 MFMA, published (TOPS)
BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published (TFLOP/s)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=0, help="timed steps (0: per-workload default)")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode")
    ap.add_argument("--copies", type=int, default=0,
                    help="layer copies rotated across steps (0: the workload's default: 16 for tiny and decode, "
                         "4 for verify, 2 for prefill and skewed)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", action="store_true", help="time only --workload (default: all five configs)")
    ap.add_argument("--tier", action="store_true",
                    help="tiered-residency sweep instead of the resident layer: routed experts in "
                         "pinned host memory behind an HBM slot bank (prints its own JSON line)")
    ap.add_argument("--tier-fractions", default="1,0.75,0.5,0.25,0.125",
                    help="resident fractions n_slots / n_experts of the sweep")
    ap.add_argument("--tier-stack", action="store_true",
                    help="tiered layer stack with and without router look-ahead prefetch (prints its "
                         "own JSON line)")
    ap.add_argument("--stack-layers", type=int, default=4)
    ap.add_argument("--group", type=int, default=0,
                    help="group-wise weight scales: one fp32 scale per this many columns (0: per row)")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="also run one elementwise fp32 copy of this many MiB (a known-size kernel "
                         "for scaling hardware byte counters)")
    return ap.parse_args()


def scales_per_row(w, K):
    """fp32 weight scales per row of a matrix with K columns."""
    return K // w.group if w.group else 1


def expert_bytes(w):
    """Packed weights plus scales of one expert (gate, up, down)."""
    H, I, b = w.hidden, w.inter, w.bits
    return 3 * H * I * b // 8 + (2 * I * scales_per_row(w, H) + H * scales_per_row(w, I)) * 4


def stage_bytes(w, n_units_touched, S):
    """Algorithmic HBM bytes of each stage for one step (n_units_touched =
    distinct routed experts + the shared expert)."""
    H, I, E, k, b = w.hidden, w.inter, w.n_experts, w.top_k, w.bits
    gu = n_units_touched * (2 * I * H * b // 8 + 2 * I * scales_per_row(w, H) * 4)
    dn = n_units_touched * (H * I * b // 8 + H * scales_per_row(w, I) * 4)
    return {
        "route": E * H * 4 + E * 4 + S * H * 4,
        "gate_up": gu,
        "down": dn,
        "combine": S * H * 4,
    }


HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


def _hip_runtime():
    """The HIP runtime this process already uses (torch's)."""
    import ctypes
    path = None
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64.so" in line:
                path = line.split()[-1]
                break
    lib = ctypes.CDLL(path or "libamdhip64.so")
    lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
    lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
    lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    return lib


class TimingEvents:
    """HIP events for stage timing only, created without the system-scope
    fence on record (a fenced event writes back and invalidates the caches,
    which adds microseconds to every stage it brackets)."""

    def __init__(self, n):
        import ctypes
        self._ct = ctypes
        self.lib = _hip_runtime()
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            rc = self.lib.hipEventCreateWithFlags(ctypes.byref(e), HIP_EVENT_DISABLE_SYSTEM_FENCE)
            if rc != 0:
                raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
            self.ev.append(e.value)

    def record(self, i, stream):
        rc = self.lib.hipEventRecord(self.ev[i], self._ct.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, i, j):
        t = self._ct.c_float()
        rc = self.lib.hipEventElapsedTime(self._ct.byref(t), self.ev[i], self.ev[j])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return t.value

    def close(self):
        for e in self.ev:
            self.lib.hipEventDestroy(e)
        self.ev = []


TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "decode_gate_up_traffic.json")


def measured_traffic(w, stage):
    """HBM bytes per launch of the stage's kernel from the committed counter
    runs, or None when no record matches (other workload or stage, or the
    kernel sources changed since the counters were taken)."""
    import hashlib
    if not os.path.exists(TRAFFIC_RECORD):
        return None
    with open(TRAFFIC_RECORD) as f:
        rec = json.load(f)
    if rec.get("workload") != w.name or stage != "gate_up" or w.group:
        return None
    h = hashlib.sha256()
    for src in rec["sources"]:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    return rec["traffic_bytes_per_launch"] if h.hexdigest() == rec["sources_sha256"] else None


def stage_kernel(w, stage):
    """The kernel(s) one FFN stage launches for this workload."""
    if w.S == 1:
        return {"gate_up": f"ffn_gate_up_decode<{w.bits}> (top-k selection + gate/up GEMV)",
                "down": f"ffn_down_combine_decode<{w.bits}> (down GEMV + weighted combine)"}[stage]
    if w.S <= 8:  # small batches stay on the GEMV kernels
        return f"ffn_{stage}_rows<{w.bits}>"
    if w.S * w.top_k >= 8 * w.n_experts:  # 8 or more pairs per expert: every expert on the matrix cores
        return f"ffn_{stage}_mfma<{w.bits}>"
    return f"ffn_{stage}_rows<{w.bits}> + ffn_{stage}_mfma<{w.bits}>"


def run_workload(qre, synth, torch, w, steps, warmup, copies, timed_stages=True, cpu_tokens=0):
    import numpy as np
    dev_layers = []
    base = synth.make_layer(w, device="cuda")

    def qb(b):
        return qre.QBank(b.storage, b.scale_storage, b.bits, b.group)

    def mk(L):
        sh = [qb(L.sh_gate), qb(L.sh_up), qb(L.sh_down)] if w.has_shared else None
        return qre.MoELayer(w.hidden, w.inter, w.n_experts, w.top_k, w.rsf, L.router_w, L.bias,
                            qb(L.gate), qb(L.up), qb(L.down), sh)
    dev_layers.append((mk(base), base))
    for c in range(1, copies):
        clone = synth.Layer(w, base.router_w.clone(), base.bias.clone(),
                            *[None if b is None else synth.Bank(b.n_mat, b.rows, b.K, b.bits, [], [],
                                                                b.storage.clone(), b.scale_storage.clone())
                              for b in (base.gate, base.up, base.down, base.sh_gate, base.sh_up, base.sh_down)])
        dev_layers.append((mk(clone), clone))
    n_batches = max(copies, 16) if w.S <= 8 else 2
    xs = [synth.activations(w, tag=f"/bench{i}").cuda() for i in range(n_batches)]
    out = torch.empty_like(xs[0])
    ws = dev_layers[0][0].workspace(w.S)
    torch.cuda.synchronize()

    def step(i):
        qre.moe_layer_forward(dev_layers[i % copies][0], xs[i % n_batches], out, ws)

    # A 256 MiB device copy right before each timed pass: the GPU is busy
    # with it while the host queues the first steps, so every timed window
    # opens with work already queued (the first launch's host latency stays
    # outside it, which matters when only a few steps are timed), and the
    # last-level cache holds none of the layer's weights when it opens.
    spacer = [torch.empty(64 << 20, dtype=torch.float32, device="cuda") for _ in range(2)]

    def settle():
        spacer[1].copy_(spacer[0])

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    settle()
    t_start.record(stream)
    for i in range(steps):
        step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    gpu_ms = t_start.elapsed_time(t_end)

    res = {"steps": steps, "gpu_ms": gpu_ms, "wall_s": wall}
    # per-step distribution: a start / end event around every step
    pev = TimingEvents(2 * steps)
    torch.cuda.synchronize()
    settle()
    for i in range(steps):
        pev.record(2 * i, stream)
        step(i)
        pev.record(2 * i + 1, stream)
    torch.cuda.synchronize()
    per_step = sorted(pev.elapsed_ms(2 * i, 2 * i + 1) for i in range(steps))
    pev.close()
    res["step_ms_quantiles"] = {q: per_step[min(steps - 1, int(f * steps))]
                                for q, f in (("p10", 0.1), ("median", 0.5), ("p90", 0.9))}
    if timed_stages:
        # same steps again through the staged entry point: per-stage durations
        n_ev = qre.COLI_N_STAGE_EVENTS
        tev = TimingEvents(steps * n_ev)
        torch.cuda.synchronize()
        settle()
        for i in range(steps):
            qre.moe_layer_forward_staged(dev_layers[i % copies][0], xs[i % n_batches], out, ws,
                                         tev.ev[i * n_ev:(i + 1) * n_ev])
        torch.cuda.synchronize()
        per = {s: 0.0 for s in qre.STAGES}
        for i in range(steps):
            for j, s in enumerate(qre.STAGES):
                per[s] += tev.elapsed_ms(i * n_ev + j, i * n_ev + j + 1)
        tev.close()
        res["stage_ms"] = {s: v / steps for s, v in per.items()}
    # union size of each batch (for algorithmic bytes)
    uniq = []
    for x in xs:
        ids, _ = qre.route(dev_layers[0][0], x)
        uniq.append(len(set(ids.cpu().numpy().reshape(-1).tolist())))
    res["mean_unique_experts"] = float(np.mean([uniq[i % n_batches] for i in range(steps)]))
    del dev_layers, ws, spacer
    torch.cuda.empty_cache()
    if cpu_tokens:
        xall = torch.cat(xs)  # the rotated batches: S = 1 decode draws its sample from several
        res["cpu_baseline"] = cpu_baseline(synth, w, base, xall, min(cpu_tokens, xall.shape[0]))
    del base, xs
    torch.cuda.empty_cache()
    return res


PCIE_PEAK_GBS = 63.0  # PCIe 5.0 x16, one direction after 128b/130b encoding


def h2d_probe(torch, nbytes, reps=3):
    """Copy-engine rate of pinned host -> HBM transfers of nbytes."""
    src = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    rate = reps * nbytes / (time.perf_counter() - t0) / 1e9
    del src, dst
    return rate


def tier_graph_rate(torch, tier, xs, out, ws, S, replays=20):
    """Per-token time of tier.forward replayed from a captured graph."""
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            for x in xs:
                tier.forward(x, out, ws)
    torch.cuda.synchronize()
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (replays * len(xs))
    del g
    return {"graph_ms_per_step": ms, "graph_tokens_per_s": 1000.0 * S / ms}


def run_tier(qre, synth, torch, w, fractions, steps):
    """Decode through colibri_tier_forward at several resident fractions, for
    uniform routing (the workload's normal bias) and for Zipf-skewed expert
    popularity (the skewed workload's bias recipe on the same weights)."""
    import numpy as np
    base = synth.make_layer(w, device="cuda")
    E = w.n_experts

    def pinned(t):
        p = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
        p.copy_(t)
        return p

    def host_bank(b):
        return qre.QBank(pinned(b.storage), pinned(b.scale_storage), b.bits)

    def dev_bank(b):
        return qre.QBank(b.storage, b.scale_storage, b.bits)
    routed = [host_bank(b) for b in (base.gate, base.up, base.down)]
    shared = [dev_bank(b) for b in (base.sh_gate, base.sh_up, base.sh_down)] if w.has_shared else None
    biases = {"uniform": base.bias,
              "zipf": synth.router_bias(synth.scaled(w, bias_kind="zipf")).to("cuda")}
    for b in (base.gate, base.up, base.down):
        b.storage = b.scale_storage = None
        b.data, b.scale = [], []
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    probe = h2d_probe(torch, 16 * expert_bytes(w))
    xs = [synth.activations(w, tag=f"/tier{i}").cuda() for i in range(512)]
    out = torch.empty_like(xs[0])
    sweep = []
    for kind, bias in biases.items():
        layer = qre.MoELayer(w.hidden, w.inter, E, w.top_k, w.rsf, base.router_w, bias, *routed, shared)
        for f in fractions:
            n_slots = max(1, min(E, int(round(f * E))))
            tier = qre.TieredLayer(layer, n_slots)
            ws = tier.workspace(w.S)
            if n_slots == E:
                tier.pin(list(range(E)))  # everything resident: no misses at all
            warm = max(64, 4 * n_slots // max(1, w.top_k))
            for i in range(warm):
                tier.forward(xs[i % len(xs)], out, ws)
            torch.cuda.synchronize()
            s0 = tier.stats()
            t0 = time.perf_counter()
            for i in range(steps):
                tier.forward(xs[(warm + i) % len(xs)], out, ws)
            torch.cuda.synchronize()
            t = time.perf_counter() - t0
            s1 = tier.stats()
            hits, misses = s1["hits"] - s0["hits"], s1["misses"] - s0["misses"]
            moved = misses * expert_bytes(w)
            point = {"routing": kind, "resident_fraction": n_slots / E, "n_slots": n_slots,
                     "tokens_per_s": steps * w.S / t, "ms_per_step": 1000.0 * t / steps,
                     "expert_hit_rate": hits / max(1, hits + misses),
                     "expert_loads_per_step": misses / steps,
                     "passes_per_step": (s1["passes"] - s0["passes"]) / steps,
                     "h2d_GBps": moved / t / 1e9}
            if n_slots == E:
                # The hit path without the host: 16 forwards over 16 distinct
                # tokens captured in one graph (nothing misses, so replaying
                # the same tokens changes no rate), replayed and timed on the GPU.
                point.update(tier_graph_rate(torch, tier, xs[:16], out, ws, w.S))
            sweep.append(point)
            tier.close()
            del ws
    return {"h2d_probe_GBps": probe, "sweep": sweep}


def run_tier_stack(qre, synth, torch, w, n_layers, steps):
    """Verify steps through a stack of n_layers tiered layers (one shared
    pinned store of routed experts, a router per layer), one
    colibri_tier_verify_step per step.  Synthetic residual stream: layer
    l + 1's input is x_l + sigma * z_l.  With look-ahead, layer l + 1's
    experts are predicted from x_l inside the step.  Measured per (S,
    routing, resident fraction, sigma, look-ahead): positions/s, expert hit
    rate, loads, and the draft-union statistics (distinct experts per layer
    and step, and the share of them the previous step also used)."""
    import numpy as np
    base = synth.make_layer(w, device="cuda")
    E, H = w.n_experts, w.hidden

    def pinned(t):
        p = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
        p.copy_(t)
        return p
    routed = [qre.QBank(pinned(b.storage), pinned(b.scale_storage), b.bits) for b in (base.gate, base.up, base.down)]
    shared = [qre.QBank(b.storage, b.scale_storage, b.bits) for b in (base.sh_gate, base.sh_up, base.sh_down)]
    for b in (base.gate, base.up, base.down):
        b.storage = b.scale_storage = None
        b.data, b.scale = [], []
    torch.cuda.empty_cache()
    routers = []
    for l in range(n_layers):
        wl = synth.scaled(w, layer=f"{w.layer}/stack{l}")
        routers.append(synth.router_weights(wl).cuda())
    biases = {"uniform": [synth.router_bias(synth.scaled(w, layer=f"{w.layer}/stack{l}")).cuda()
                          for l in range(n_layers)],
              "zipf": [synth.router_bias(synth.scaled(w, layer=f"{w.layer}/stack{l}", bias_kind="zipf")).cuda()
                       for l in range(n_layers)]}
    gen = torch.Generator(device="cuda")
    nw = (E + 31) // 32
    out = []
    for S in (1, 4):
        for sigma in (0.5, 1.0):
            gen.manual_seed(1234 + S)
            n_tok = steps + 64
            xs = [torch.randn(n_tok, S, H, device="cuda", generator=gen)]
            for l in range(1, n_layers):
                xs.append(xs[-1] + sigma * torch.randn(n_tok, S, H, device="cuda", generator=gen))
            X = torch.stack(xs, dim=1).contiguous()  # [n_tok][n_layers][S][H]
            del xs
            for kind in ("uniform", "zipf"):
                layers = [qre.MoELayer(H, w.inter, E, w.top_k, w.rsf, routers[l], biases[kind][l], *routed, shared)
                          for l in range(n_layers)]
                # recall of the look-ahead prediction over the timed steps
                hit = tot = 0
                for l in range(n_layers - 1):
                    pred, _ = qre.route(layers[l + 1], X[64:, l].reshape(-1, H).contiguous())
                    act, _ = qre.route(layers[l + 1], X[64:, l + 1].reshape(-1, H).contiguous())
                    pr, ac = pred.cpu().numpy(), act.cpu().numpy()
                    for t in range(0, len(ac), S):
                        a = set(ac[t:t + S].reshape(-1).tolist())
                        b = set(pr[t:t + S].reshape(-1).tolist())
                        hit += len(a & b)
                        tot += len(a)
                recall = hit / max(1, tot)
                for f in (0.5, 0.75):
                    n_slots = int(round(f * E))
                    rate = {}
                    for look in (False, True):
                        tiers = [qre.TieredLayer(layers[l], n_slots) for l in range(n_layers)]
                        ws = tiers[0].workspace(S)
                        o = torch.empty(n_layers, S, H, device="cuda")
                        mask = torch.zeros(n_layers, nw, dtype=torch.int32, device="cuda")
                        st = torch.zeros(n_tok, n_layers, 2, dtype=torch.int32, device="cuda")
                        for i in range(64):
                            qre.tier_verify_step(tiers, X[i], o, ws, mask, st[i], lookahead=look)
                        torch.cuda.synchronize()
                        s0 = [t.stats() for t in tiers]
                        t0 = time.perf_counter()
                        for i in range(64, 64 + steps):
                            qre.tier_verify_step(tiers, X[i], o, ws, mask, st[i], lookahead=look)
                        torch.cuda.synchronize()
                        dt = time.perf_counter() - t0
                        s1 = [t.stats() for t in tiers]
                        d = {k: sum(b[k] - a[k] for a, b in zip(s0, s1))
                             for k in ("hits", "misses", "prefetch_loads")}
                        u = st[64:64 + steps].cpu().numpy().astype(np.float64)
                        union, reuse = u[..., 0], u[..., 1]
                        rate[look] = steps * S / dt
                        out.append({"S": S, "sigma": sigma, "routing": kind, "resident_fraction": f,
                                    "lookahead": look, "recall": recall,
                                    "tokens_per_s": rate[look],
                                    "ms_per_layer": 1000.0 * dt / (steps * n_layers),
                                    "expert_hit_rate": d["hits"] / max(1, d["hits"] + d["misses"]),
                                    "loads_per_token_layer": (d["misses"] + d["prefetch_loads"]) / (steps * S * n_layers),
                                    "prefetch_loads_per_token_layer": d["prefetch_loads"] / (steps * S * n_layers),
                                    "union_per_layer_step": float(union.mean()),
                                    "union_per_position": float(union.mean() / S),
                                    "reuse_of_previous_step": float(reuse.sum() / max(1.0, union.sum())),
                                    **({"speedup_vs_no_lookahead": rate[True] / rate[False]} if look else {})})
                        print(f"stack S={S} sigma={sigma} {kind} f={f} lookahead={look}: "
                              f"{out[-1]['tokens_per_s']:.0f} positions/s, union {out[-1]['union_per_layer_step']:.1f}",
                              file=sys.stderr, flush=True)
                        for t in tiers:
                            t.close()
                        del tiers, ws
            del X
    return out


def cpu_info():
    """Host CPU model, logical CPUs and physical cores (from /proc/cpuinfo)."""
    model, cores = None, set()
    phys = core = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                k, _, v = line.partition(":")
                k, v = k.strip(), v.strip()
                if k == "model name" and model is None:
                    model = v
                elif k == "physical id":
                    phys = v
                elif k == "core id":
                    core = v
                elif not k and phys is not None and core is not None:
                    cores.add((phys, core))
                    phys = core = None
        if phys is not None and core is not None:
            cores.add((phys, core))
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(), "nproc_allowed": len(os.sched_getaffinity(0)),
            "physical_cores": len(cores) or None}


def cpu_baseline(synth, w, Lg, x, n_tokens):
    """The oracle, as it stands, on n_tokens tokens of the workload's batch x,
    single-threaded, with this thread pinned to one CPU (the experts it needs
    are copied from the device layer Lg; their generation is not timed)."""
    import oracle
    import numpy as np
    xs = x[:n_tokens].cpu().numpy()
    router_w, bias = Lg.router_w.cpu(), Lg.bias.cpu()
    ids, _, _ = oracle.route(xs, router_w, bias, w.top_k, w.rsf)
    needed = set(ids.reshape(-1).tolist())

    def sub(b):
        return synth.Bank(b.n_mat, b.rows, b.K, b.bits,
                          [b.storage[m].cpu() if m in needed else None for m in range(b.n_mat)],
                          [b.scale_storage[m].cpu() if m in needed else None for m in range(b.n_mat)],
                          group=b.group)

    def full(b):
        return None if b is None else synth.Bank(1, b.rows, b.K, b.bits, [b.storage[0].cpu()],
                                                 [b.scale_storage[0].cpu()], group=b.group)
    L = synth.Layer(w, router_w, bias, sub(Lg.gate), sub(Lg.up), sub(Lg.down),
                    full(Lg.sh_gate), full(Lg.sh_up), full(Lg.sh_down))
    Lh = oracle.LayerHandle(L)
    old = os.sched_getaffinity(0)
    cpu = max(old)
    os.sched_setaffinity(0, {cpu})
    try:
        t0 = time.perf_counter()
        oracle.layer_forward(Lh, xs)
        t = time.perf_counter() - t0
    finally:
        os.sched_setaffinity(0, old)
    ops = n_tokens * layer_ops(w)
    info = cpu_info()
    return {"value": n_tokens / t, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "GOPs": ops / t / 1e9, "pinned_cpu": cpu, **info,
            "sample": f"{n_tokens} tokens of the {w.name} batches through the single-threaded C "
                      f"oracle (full layer per token: router, {w.top_k} routed experts"
                      + (" + shared expert" if w.has_shared else "") + f", combine), {t:.2f} s on one CPU"}


def layer_ops(w):
    """int8 multiply-add operations of one token's routed and shared experts (2 per MAC)."""
    return 2 * (w.top_k + (1 if w.has_shared else 0)) * 3 * w.hidden * w.inter


def fold_triples(w):
    """(token, row, block) fp32 folds of one token: one fma per triple."""
    n = w.top_k + (1 if w.has_shared else 0)
    return n * (2 * w.inter * w.hidden // 32 + w.hidden * w.inter // 32)


VALU_PEAK_LANE_OPS = 256 * 64 * 2.4e9  # lane operations per second (non-packed fp32)


def device_peaks(torch, qre_probes):
    """Achievable rates of this device: a 1 GiB nontemporal read stream and
    int8 matrix-core loops (K = 32, the form the layer uses, and K = 64)."""
    import ctypes
    import synth
    st = torch.cuda.current_stream().cuda_stream
    sink = torch.zeros(8192, dtype=torch.int32, device="cuda")
    buf = torch.ones(1 << 28, dtype=torch.int32, device="cuda")  # 1 GiB
    nbytes = buf.numel() * 4
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    read = {}
    for blocked in (0, 1):
        for blocks in (512, 1024, 2048, 4096, 8192):
            args = (ctypes.c_void_p(buf.data_ptr()), nbytes, blocks, blocked, ctypes.c_void_p(sink.data_ptr()),
                    ctypes.c_void_p(st))
            assert qre_probes.colibri_probe_read(*args) == 0
            e0.record()
            reps = 5
            for _ in range(reps):
                qre_probes.colibri_probe_read(*args)
            e1.record()
            torch.cuda.synchronize()
            read[("blocked" if blocked else "grid_stride", blocks)] = \
                reps * nbytes / (e0.elapsed_time(e1) / 1000.0) / 1e9
    best = max(read, key=read.get)
    del buf
    # the one-token kernels' weight read pattern alone, at the decode layer's
    # sizes: gate+up and down of top_k + 1 experts, 16 rows per wave, 16
    # copies rotated past the caches
    wd = synth.WORKLOADS["decode"]
    u = wd.top_k + (1 if wd.has_shared else 0)
    pattern = {}
    for name, rows, rowbytes in (("gate_up", 2 * wd.inter * u, wd.hidden * wd.bits // 8),
                                 ("down", wd.hidden * u, wd.inter * wd.bits // 8)):
        ni, waves = rowbytes // 512, rows // 16
        nbytes = waves * 16 * rowbytes
        copies = torch.ones(16 * nbytes // 4, dtype=torch.int32, device="cuda")
        bases = [copies.data_ptr() + c * nbytes for c in range(16)]
        for c in range(16):
            assert qre_probes.colibri_probe_rows(ctypes.c_void_p(bases[c]), ni, waves, 1,
                                                 ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(st)) == 0
        reps = 64
        e0.record()
        for r in range(reps):
            qre_probes.colibri_probe_rows(ctypes.c_void_p(bases[r % 16]), ni, waves, 1,
                                          ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(st))
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1000.0 / reps
        pattern[name] = {"bytes": nbytes, "us": us, "GBps": nbytes / us / 1e3}
        del copies
    # the matrix-core kernels' weight read pattern alone (64 rows per
    # workgroup, 128 bytes of each row per step, two steps in flight, a
    # barrier per step), at the prefill layer's sizes: every expert once
    wp = synth.WORKLOADS["prefill"]
    u = wp.n_experts + (1 if wp.has_shared else 0)
    tile = {}
    for name, rows, rowbytes in (("gate_up", 2 * wp.inter * u, wp.hidden * wp.bits // 8),
                                 ("down", wp.hidden * u, wp.inter * wp.bits // 8)):
        nbytes = rows * rowbytes
        tb = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda")
        tsink = torch.zeros(rows // 64, dtype=torch.int32, device="cuda")
        args = (ctypes.c_void_p(tb.data_ptr()), rowbytes, rows, 128, 0, 0, ctypes.c_void_p(tsink.data_ptr()),
                ctypes.c_void_p(st))
        assert qre_probes.colibri_probe_tile(*args) == 0
        reps = 5
        e0.record()
        for _ in range(reps):
            qre_probes.colibri_probe_tile(*args)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1000.0 / reps
        tile[name] = {"bytes": nbytes, "us": us, "GBps": nbytes / us / 1e3}
        del tb, tsink
    mfma = {}
    for k in (32, 64):
        blocks, iters = 1024, 4096
        qre_probes.colibri_probe_mfma_i8(k, 64, blocks, ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(st))
        e0.record()
        assert qre_probes.colibri_probe_mfma_i8(k, iters, blocks, ctypes.c_void_p(sink.data_ptr()),
                                                ctypes.c_void_p(st)) == 0
        e1.record()
        torch.cuda.synchronize()
        ops = blocks * 4 * iters * 8 * 16 * 16 * k * 2
        mfma[k] = ops / (e0.elapsed_time(e1) / 1000.0) / 1e12
    blocks, iters = 1024, 4096
    qre_probes.colibri_probe_mfma_bf16(64, blocks, ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(st))
    e0.record()
    assert qre_probes.colibri_probe_mfma_bf16(iters, blocks, ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(st)) == 0
    e1.record()
    torch.cuda.synchronize()
    bf16_k32 = blocks * 4 * iters * 8 * 16 * 16 * 32 * 2 / (e0.elapsed_time(e1) / 1000.0) / 1e12
    return {"hbm_read_stream_GBps": read[best], "read_stream_best": f"{best[0]}, {best[1]} workgroups",
            "int8_mfma_k32_TOPS": mfma[32], "int8_mfma_k64_TOPS": mfma[64], "bf16_mfma_k32_TFLOPS": bf16_k32,
            "decode_read_pattern": pattern, "prefill_read_pattern": tile,
            "spec": {"hbm_GBps": HBM_PEAK_GBS, "int8_mfma_TOPS": INT8_PEAK_TOPS, "bf16_mfma_TFLOPS": BF16_PEAK_TFLOPS,
                     "valu_lane_ops_per_s": VALU_PEAK_LANE_OPS},
            "how": "read stream: 1 GiB read once per launch with 16-byte nontemporal loads, best of grid-stride and "
                   "blocked layouts over 512..8192 workgroups; matrix cores: 1024 workgroups of 4 waves, 8 "
                   "independent int8 (K = 32 and 64) or bf16 (16x16x32) MFMA chains per wave; decode read pattern: the one-token kernels' weight "
                   "loads (items of 2 rows x 512 B, chunk-major, 16 rows per wave) with no arithmetic, at the "
                   "decode layer's gate+up and down sizes, one launch each, 16 copies rotated; prefill read pattern: "
                   "the matrix-core kernels' weight loads (64 rows per workgroup, 128 bytes of each row per step, "
                   "two steps in flight, a barrier per step) with no arithmetic, over every expert of the prefill "
                   "layer's gate+up and down"}


def load_probes():
    import ctypes
    path = os.path.join(ROOT, "quantized_routed_expert_sigmoid_amd", "libcolibri_probes.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m quantized_routed_expert_sigmoid_amd.build`")
    L = ctypes.CDLL(path)
    L.colibri_probe_rows.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                     ctypes.c_void_p]
    L.colibri_probe_tile.argtypes = [ctypes.c_void_p] + [ctypes.c_int32] * 5 + [ctypes.c_void_p, ctypes.c_void_p]
    L.colibri_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_void_p, ctypes.c_void_p]
    L.colibri_probe_mfma_i8.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                        ctypes.c_void_p]
    L.colibri_probe_mfma_bf16.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    L.colibri_probe_mfma_bf16_block.argtypes = [ctypes.c_void_p] * 5
    return L


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library runs the layer on one MI355X; it has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)
    import torch
    import quantized_routed_expert_sigmoid_amd as qre
    import synth
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    qre.lib()
    if args.calibration_copy_mib:
        n = args.calibration_copy_mib * (1 << 20) // 4
        src = torch.ones(n, device="cuda")
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)  # reads and writes n * 4 bytes
        torch.cuda.synchronize()
        del src, dst
    w = synth.WORKLOADS[args.workload]
    if args.group:
        w = synth.scaled(w, group=args.group)
    if args.tier_stack:
        steps = args.steps or 100
        r = run_tier_stack(qre, synth, torch, w, args.stack_layers, steps)
        print(json.dumps({
            "metric": "tiered layer-stack verify positions/sec with and without router look-ahead prefetch "
                      "(one colibri_tier_verify_step per step), with draft-union statistics",
            "unit": "tokens/s", "n_gpus": 1, "steps": steps, "higher_is_better": True, "dtype": "int8",
            "data": "synthetic (seeded weights; residual stream x_l+1 = x_l + sigma * z_l; no checkpoint)",
            "config": {"workload": f"{args.stack_layers} layers of H={w.hidden} I={w.inter} E={w.n_experts} "
                                   f"top-{w.top_k} int{w.bits}, one shared pinned expert store, a router per "
                                   "layer", "expert_bytes": expert_bytes(w)},
            "stack": r}), flush=True)
        return
    if args.tier:
        fr = [float(v) for v in args.tier_fractions.split(",")]
        steps = args.steps or 300
        r = run_tier(qre, synth, torch, w, fr, steps)
        print(json.dumps({
            "metric": "tiered decode tokens/sec per MoE layer vs HBM-resident expert fraction",
            "unit": "tokens/s", "n_gpus": 1, "steps": steps, "higher_is_better": True, "dtype": "int8",
            "data": "synthetic (seeded SplitMix64 weights and activations; no checkpoint)",
            "config": {"workload": f"{w.name}: MoE layer H={w.hidden} I={w.inter} E={w.n_experts} "
                                   f"top-{w.top_k} int{w.bits}, routed experts in pinned host memory, "
                                   f"S={w.S}", "expert_bytes": expert_bytes(w)},
            "roofline": {"bound": "pcie", "unit": "GB/s", "peak": PCIE_PEAK_GBS,
                         "copy_engine_probe": r["h2d_probe_GBps"]},
            "sweep": r["sweep"]}), flush=True)
        return
    configs = [args.workload] if args.only else ["decode", "tiny", "verify", "prefill", "skewed"]
    if args.workload not in configs:
        configs.insert(0, args.workload)
    per = {}
    probes = load_probes()
    peaks = device_peaks(torch, probes)
    for name in configs:
        wc = synth.WORKLOADS[name]
        if args.group:
            wc = synth.scaled(wc, group=args.group)
        steps, warmup, copies = (args.steps, args.warmup, args.copies) if name == args.workload else \
            DEFAULTS[name]
        steps = steps or DEFAULTS[name][0]
        copies = copies or DEFAULTS[name][2]
        print(f"bench: {name} S={wc.S} int{wc.bits}: {steps} steps over {copies} layer copies",
              file=sys.stderr, flush=True)
        cpu_n = 0 if args.no_cpu_baseline else CPU_TOKENS[name]
        res = run_workload(qre, synth, torch, wc, steps, warmup, copies, cpu_tokens=cpu_n)
        per[name] = config_summary(wc, res, peaks, copies)
    w = synth.WORKLOADS[args.workload] if not args.group else synth.scaled(synth.WORKLOADS[args.workload],
                                                                              group=args.group)
    head = per[args.workload]
    res_h = head.pop("_res")
    stage_ms = res_h["stage_ms"]
    U = res_h["mean_unique_experts"] + (1 if w.has_shared else 0)
    sb = stage_bytes(w, U, w.S)
    dom = max(("gate_up", "down"), key=lambda st: stage_ms[st])
    achieved = sb[dom] / (stage_ms[dom] / 1000.0) / 1e9
    line = {
        "metric": "routed tokens/sec per MoE layer (S=1 decode, S=512 prefill); % HBM BW / % int8 MFMA",
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": head["steps"],
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "step_ms_quantiles": head["step_ms_quantiles"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic (seeded SplitMix64 weights and activations; no checkpoint)",
        "config": {"workload": head["workload"], "S": w.S, "weights": f"int{w.bits}",
                   "layer_copies_rotated": head["layer_copies_rotated"], "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": stage_kernel(w, dom), "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(w, dom), "algorithmic_bytes": sb[dom],
                     "frac_of_measured_read_stream": achieved / peaks["hbm_read_stream_GBps"]},
        "layer": head["rooflines"],
        "stage_ms": head["stage_ms"],
        "device_peaks": peaks,
        "configs": {CONFIG_IDS[n]: {k: v for k, v in per[n].items() if k != "_res"} for n in configs},
    }
    if "cpu_baseline" in head:
        line["cpu_baseline"] = head["cpu_baseline"]
    print(json.dumps(line), flush=True)


CONFIG_IDS = {"tiny": "C1_tiny", "decode": "C2_decode", "prefill": "C3_prefill", "verify": "C4_verify",
              "skewed": "C5_skewed"}
# steps, warmup, layer copies rotated per workload (batches whose weights fit
# the 256 MB last-level cache rotate enough copies that the cache cannot
# serve them)
DEFAULTS = {"tiny": (2000, 50, 16), "decode": (2000, 20, 16), "verify": (500, 20, 4), "prefill": (30, 20, 2),
            "skewed": (20, 20, 2)}
CPU_TOKENS = {"tiny": 128, "decode": 8, "verify": 4, "prefill": 8, "skewed": 8}


def config_summary(w, res, peaks, copies):
    """Throughput of one workload and its rooflines: HBM (algorithmic bytes:
    the touched experts, router, x and out), int8 matrix cores (2 per MAC of
    every routed and shared expert row), VALU (one fp32 fold per token, row
    and block); `binding` names the bound the workload meets first."""
    steps = res["steps"]
    ms = res["gpu_ms"] / steps
    t = ms / 1000.0
    U = res["mean_unique_experts"] + (1 if w.has_shared else 0)
    sb = stage_bytes(w, U, w.S)
    layer_bytes = U * expert_bytes(w) + sb["route"] + sb["combine"]
    ops = w.S * layer_ops(w)
    triples = w.S * fold_triples(w)
    bounds = {"hbm": layer_bytes / (HBM_PEAK_GBS * 1e9), "int8_mfma": ops / (INT8_PEAK_TOPS * 1e12),
              "valu_fold": triples / VALU_PEAK_LANE_OPS}
    binding = max(bounds, key=bounds.get)
    if bounds[binding] < 10e-6:
        binding = "latency"  # every bound below 10 us: launches and round trips dominate
    stage_ms = dict(res["stage_ms"])
    extra = {}
    if w.S == 1:
        # one token: the selection runs inside gate/up and the combine inside
        # down, so those two stages are empty; what they show is the cost of
        # the event pair
        extra["event_pair_overhead_ms"] = 0.5 * (stage_ms.pop("dispatch") + stage_ms.pop("combine"))
        stage_ms["gate_up_with_selection"] = stage_ms.pop("gate_up")
        stage_ms["down_with_combine"] = stage_ms.pop("down")
    if w.name == "prefill" and peaks.get("prefill_read_pattern"):
        # the matrix-core weight read pattern over every expert: the floor of
        # each FFN stage when all 257 experts are touched
        pat = peaks["prefill_read_pattern"]
        extra["read_pattern_floor_ms"] = {k: v["us"] / 1000.0 for k, v in pat.items()}
        extra["stage_frac_of_read_pattern"] = {k: pat[k]["us"] / 1000.0 / stage_ms[k] for k in ("gate_up", "down")}
    if w.S == 1:
        pat = peaks.get("decode_read_pattern", {})
        if w.name == "decode" and pat:
            # the same weight bytes read in the same pattern by a kernel that
            # does nothing else: the launch-inclusive floor of each stage
            extra["read_pattern_floor_ms"] = {k: v["us"] / 1000.0 for k, v in pat.items()}
            extra["stage_frac_of_read_pattern"] = {
                "gate_up": pat["gate_up"]["us"] / 1000.0 / stage_ms["gate_up_with_selection"],
                "down": pat["down"]["us"] / 1000.0 / stage_ms["down_with_combine"]}
    return {
        "workload": f"{w.name}: MoE layer H={w.hidden} I={w.inter} E={w.n_experts} top-{w.top_k} int{w.bits} "
                    "weights" + (f" with one scale per {w.group} columns" if w.group else "")
                    + (" + shared expert" if w.has_shared else "") + f", S={w.S}",
        "value": w.S / t, "unit": "tokens/s", "ms_per_step": ms, "us_per_step": 1000.0 * ms, "steps": steps,
        "layer_copies_rotated": copies, "step_ms_quantiles": res["step_ms_quantiles"],
        "unique_routed_experts": res["mean_unique_experts"],
        "rooflines": {
            "hbm": {"algorithmic_bytes": layer_bytes, "achieved_GBps": layer_bytes / t / 1e9,
                    "frac": layer_bytes / t / 1e9 / HBM_PEAK_GBS,
                    "frac_of_measured_read_stream": layer_bytes / t / 1e9 / peaks["hbm_read_stream_GBps"],
                    "time_at_peak_ms": 1000.0 * bounds["hbm"]},
            "int8_mfma": {"ops": ops, "achieved_TOPS": ops / t / 1e12, "frac": ops / t / 1e12 / INT8_PEAK_TOPS,
                          "frac_of_measured_k32": ops / t / 1e12 / peaks["int8_mfma_k32_TOPS"],
                          "time_at_peak_ms": 1000.0 * bounds["int8_mfma"]},
            "valu_fold": {"fold_triples": triples, "frac": triples / t / VALU_PEAK_LANE_OPS,
                          "time_at_peak_ms": 1000.0 * bounds["valu_fold"],
                          "note": "one lane operation per (token, row, block) fold at 256 CUs x 64 lanes x 2.4 GHz"},
            "binding": binding},
        "stage_ms": stage_ms, **extra,
        **({"cpu_baseline": res["cpu_baseline"]} if "cpu_baseline" in res else {}),
        "_res": res,
    }


if __name__ == "__main__":
    main()
