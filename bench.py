#!/usr/bin/env python3
"""Benchmark of the PISA hot path on one MI355X.

One step = pisa_precompute + pisa_route + pisa_attention (exact-or-approximate
mode) over one batch of seeded synthetic inputs already resident in HBM, on
the video-DiT-L workload (batch 1, 40 heads, L = 32768 on a 16x32x64 latent
grid, head dim 128, block 128, top-k 32 of 256 blocks = 12.5% density, bf16).

Prints ONE JSON line.  `value` is the algorithmic TFLOP/s of the whole step;
`ms_per_step` its latency; `roofline` describes the fused attention kernel
(the dominant one) against the bf16 MFMA peak; `phases` splits the step by
kernel (HIP events on the launch stream); `dense` is the same kernel run with
every block exact, `sdpa` torch's fused dense attention on the same tensors
(context only, never part of the library); `step_event_ms` gives p10 / p50 /
p90 of the timed steps (HIP events) and `cold_step_ms` the same for steps run
after a 512 MB scratch write (caches flushed); `density_sweep` re-routes the same
inputs at top-k 128 / 64 / 32 / 16 of 256 blocks and times both modes; `orders`
times the zeroth-order and the per-block first-order treatments of the
unselected blocks on the same inputs; `route_attention_fused` times the
routing-and-attention call (its automatic form, and the in-kernel routing form
forced) against the two calls it replaces;
`secondary` holds the other workloads: the small video one (whole steps), the
short image one (whole steps, dense comparator) and the multimodal one with its
fixed text/image block mask (PISA and keep-or-drop, dense comparator);
`roofline.attainable` is the MFMA rate
the chip sustains for the exact phase's per-chunk instruction mix on random
operands, and its streaming HBM read rate (libpisa_probe), beside the published
peaks; `cpu_baseline` is the
fp64 oracle on a bounded sample.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 4|3] [--mode approx|drop]
                    [--no-cpu-baseline] [--no-dense] [--no-sweep] [--no-orders]
                    [--no-cold] [--no-probe] [--copy-calibration]
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0               # MI355X HBM3E


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def flops(w, k):
    """Algorithmic FLOPs of one step's calls (2 per multiply-add)."""
    bh, L, d, B, nb = w.batch * w.heads, w.seq_len, w.head_dim, w.block, w.nb
    exact = bh * nb * 4 * B * (k * B) * d                 # QK^T and PV over k exact blocks
    approx = bh * L * (4 * d * (nb - k) + 2 * d * d)      # centroid logits + sigma sums + q Hbar
    stats = 2 * bh * nb * 2 * B * d * d                   # K_j^T V_j, two passes
    route = bh * nb * nb * 2 * d                          # pooled-q . kbar (fp64)
    zeroth = bh * L * 4 * d * (nb - k)                     # approx without the q Hbar term
    first_blocks = bh * L * 2 * d * d * (nb - k)          # q H_j for every unselected block
    return {"exact": exact, "approx": approx, "attention": exact + approx, "stats": stats,
            "route": route, "step": exact + approx + stats + route,
            "attention_zeroth": exact + zeroth, "attention_first": exact + zeroth + first_blocks}


def flops_counts(w, counts):
    """Algorithmic FLOPs of the attention call for exact-block counts per query
    block (`counts`: [b, h, nb] valid idx entries), e.g. a fixed block mask."""
    import numpy as np
    L, d, B, nb = w.seq_len, w.head_dim, w.block, w.nb
    c = np.asarray(counts, dtype=np.int64)
    exact = int(c.sum()) * 4 * B * B * d
    approx = int(((nb - c) * B * 4 * d).sum()) + c.size * B * 2 * d * d
    zeroth = int(((nb - c) * B * 4 * d).sum())
    stats = 2 * w.batch * w.heads * nb * 2 * B * d * d
    return {"exact": exact, "approx": approx, "attention": exact + approx, "stats": stats,
            "step": exact + approx + stats, "attention_zeroth": exact + zeroth}


def bytes_moved(w):
    """Algorithmic HBM bytes of the streaming kernels."""
    bh, L, d, nb = w.batch * w.heads, w.seq_len, w.head_dim, w.nb
    e = 2
    kv = bh * L * d * e * 2
    stats_out = bh * (2 * nb * d + d * d + nb) * 4
    return {"stats": 2 * kv + stats_out, "route": bh * L * d * e + bh * nb * (d + 1) * 4}


def _source_stamp(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        path = os.path.join(ROOT, "piecewise_block_sparse_amd", "csrc", f)
        if not os.path.exists(path):
            return None                   # matches no stamp
        h.update(open(path, "rb").read())
    return h.hexdigest()[:16]


# the sources each stamped counter line of a profile covers
_ATTN_SOURCES = ("attn_bf16.hip", "lds_stream.hpp", "common.hpp", "topk.hpp")
_STATS_SOURCES = ("stats.hip", "lds_stream.hpp", "common.hpp")


def profiled_counters(workload_name):
    """Counter figures from the committed rocprofv3 summary of a workload:
    `traffic` (HBM bytes per attention launch, FETCH_SIZE and WRITE_SIZE passes,
    copy-calibrated), `exact_phase` (the keep-or-drop call: MFMA GFLOP, busy
    fraction, co-execution, clock), `approx_phase` (APPROX call minus DROP call)
    and `statistics` (the three precompute kernels).  A line whose kernel source
    changed after the counters were taken is left out (its `source` stamp no
    longer matches), so stale counters are never reported."""
    import re
    path = os.path.join(ROOT, "profiles", f"kernels_{workload_name}.md")
    if not os.path.exists(path):
        return {}
    text = open(path).read()
    stamps = {"attn": _source_stamp(_ATTN_SOURCES), "stats": _source_stamp(_STATS_SOURCES)}
    out = {}
    for key, tag, which in (("traffic", "attn_bf16_kernel", "attn"), ("exact_phase", "exact_phase", "attn"),
                            ("approx_phase", "approx_phase", "attn"), ("statistics", "statistics", "stats")):
        m = re.search(rf"^{tag} ((?:\w+=[0-9.e+-]+ )+)source=([0-9a-f]+)$", text, re.M)
        if not m or m.group(2) != stamps[which]:
            continue
        vals = {}
        for kv in m.group(1).split():
            k, v = kv.split("=")
            vals[k] = float(v) if any(c in v for c in ".e") else int(v)
        out[key] = vals
    return out


def profiled_traffic(workload_name):
    """HBM bytes per launch of the attention kernel from the committed rocprofv3
    summary, or None when the kernel source changed after the counters were
    taken."""
    t = profiled_counters(workload_name).get("traffic")
    if t is None:
        return None
    return {"total": t["traffic_bytes_per_launch"], "read": t["read"], "write": t["write"],
            "profiled_avg_ms": t["avg_ns"] / 1e6}


def phase_counters(workload_name):
    """The profile's per-phase counter figures, with the rates they imply."""
    c = profiled_counters(workload_name)
    out = {}
    if "exact_phase" in c:
        e = c["exact_phase"]
        rate = e["mfma_gflop"] / (e["avg_ns"] * 1e-9) / 1e3          # TFLOP/s
        out["exact_phase"] = dict(e, profiled_tflops=rate, frac=rate / MFMA_BF16_PEAK_TFLOPS)
    if "approx_phase" in c:
        a = c["approx_phase"]
        t = a["avg_ns"] * 1e-9
        out["approx_phase"] = dict(a, operand_stream_gbs=a["operand_stream_bytes"] / t / 1e9 if t > 0 else None)
    if "statistics" in c:
        st = c["statistics"]
        gbs = st["algorithmic_bytes"] / (st["avg_ns"] * 1e-9) / 1e9
        out["statistics"] = dict(st, algorithmic_gbs=gbs, frac=gbs / HBM_PEAK_GBS)
    return out or None


def timed_phases(pisa, torch, Qd, Kd, Vd, w, k, steps, warmup, mode="approx"):
    """Run `steps` full steps back to back with nothing recorded between them
    (host clock around the loop, synchronized on both sides: the headline),
    then the same number again with one HIP event pair per step (latency
    percentiles) and again with an event between the calls (phase split; each
    event costs the GPU some microseconds, so these passes run apart from the
    headline).  Returns total wall ms and the per-phase event ms."""
    stream = torch.cuda.current_stream()
    ws = torch.empty(pisa.workspace_size(Kd, w.block), dtype=torch.uint8, device="cuda")

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        st = pisa.precompute(Kd, Vd, w.block, workspace=ws)
        if ev is not None:
            ev[1].record(stream)
        idx = pisa.route(Qd, st, k, w.lam, w.block)
        if ev is not None:
            ev[2].record(stream)
        out = pisa.attention(Qd, Kd, Vd, idx, st, w.block, mode=mode)
        if ev is not None:
            ev[3].record(stream)
        return st, idx, out

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        st, idx, out = step()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    # per-step latency: one event pair per step
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(steps)]
    for a, b in pairs:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    per_step = [a.elapsed_time(b) for a, b in pairs]
    # phase split: an event between the calls
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for i in range(steps):
        st, idx, out = step(evs[i])
    torch.cuda.synchronize()
    ph = {"precompute": 0.0, "route": 0.0, "attention": 0.0}
    for e in evs:
        ph["precompute"] += e[0].elapsed_time(e[1])
        ph["route"] += e[1].elapsed_time(e[2])
        ph["attention"] += e[2].elapsed_time(e[3])
    ph = {n: v / steps for n, v in ph.items()}
    ph["step_event_ms"] = percentiles(per_step)
    return wall_ms, ph, (st, idx, out)


def percentiles(xs):
    import numpy as np
    a = np.asarray(xs, dtype=np.float64)
    return {"p10": float(np.percentile(a, 10)), "p50": float(np.percentile(a, 50)),
            "p90": float(np.percentile(a, 90)), "n": int(a.size)}


def cold_steps(pisa, torch, Qd, Kd, Vd, w, reps=10):
    """Whole steps with the caches flushed first: a 512 MB scratch write (more
    than the 256 MB MALL and every L2) before each timed step."""
    stream = torch.cuda.current_stream()
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    times = []
    for r in range(reps + 1):
        scratch.fill_(r & 255)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        st = pisa.precompute(Kd, Vd, w.block)
        idx = pisa.route(Qd, st, w.k, w.lam, w.block)
        pisa.attention(Qd, Kd, Vd, idx, st, w.block, mode="approx")
        b.record(stream)
        b.synchronize()
        if r > 0:                                   # the first one warms the allocator
            times.append(a.elapsed_time(b))
    del scratch
    return percentiles(times)


def time_attention(pisa, torch, Qd, Kd, Vd, idx, st, w, mode, reps):
    stream = torch.cuda.current_stream()
    for _ in range(2):
        pisa.attention(Qd, Kd, Vd, idx, st, w.block, mode=mode)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        pisa.attention(Qd, Kd, Vd, idx, st, w.block, mode=mode)
    b.record(stream)
    b.synchronize()
    return a.elapsed_time(b) / reps


def time_route_attention(pisa, torch, Qd, Kd, Vd, st, w, reps):
    """The routing-and-attention call in its automatic form (in-kernel routing
    while the work fits one round of workgroups, else two launches), with the
    in-kernel form forced, and the two calls it replaces, each timed the same
    way: back-to-back calls between two HIP events, the forms alternated four
    times (best of each kept: the automatic form runs the same kernels as one of
    the other two, so only the noise between passes separates them).  Returns
    the three times in ms."""
    stream = torch.cuda.current_stream()

    def fused():
        pisa.route_attention(Qd, Kd, Vd, st, w.k, w.lam, w.block, mode="approx")

    def in_kernel():
        pisa.route_attention(Qd, Kd, Vd, st, w.k, w.lam, w.block, mode="approx", form="in_kernel")

    def split():
        idx = pisa.route(Qd, st, w.k, w.lam, w.block)
        pisa.attention(Qd, Kd, Vd, idx, st, w.block, mode="approx")

    best = {}
    for name, fn in (("fused", fused), ("in_kernel", in_kernel), ("split", split)) * 4:
        for _ in range(2):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        b.synchronize()
        best[name] = min(best.get(name, 1e30), a.elapsed_time(b) / reps)
    return best["fused"], best["in_kernel"], best["split"]


def fixed_mask(pisa, torch, steps, warmup):
    """The multimodal workload (24 heads, 512 text + 4096 image tokens, 64-token
    blocks) with the fixed text/image block mask as idx (-1 padded rows of 8 to
    72 exact blocks): whole steps (precompute + attention, no routing), the
    attention call in PISA and keep-or-drop modes, and the dense comparator."""
    import numpy as np
    from piecewise_block_sparse_amd import workloads as wl
    w = wl.WORKLOADS[5]
    log(f"{w.name}: fixed-mask steps")
    Q, K, V = wl.make_inputs(w)
    Qd, Kd, Vd = (torch.from_numpy(a).to("cuda", torch.bfloat16) for a in (Q, K, V))
    del Q, K, V
    idx_h = wl.idx_fixed_mask(w)
    counts = (idx_h >= 0).sum(-1)
    idx = torch.from_numpy(idx_h).to("cuda")
    stream = torch.cuda.current_stream()
    ws = torch.empty(pisa.workspace_size(Kd, w.block), dtype=torch.uint8, device="cuda")

    def step():
        st = pisa.precompute(Kd, Vd, w.block, workspace=ws)
        return st, pisa.attention(Qd, Kd, Vd, idx, st, w.block, mode="approx")

    for _ in range(warmup):
        st, _ = step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        st, _ = step()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    f = flops_counts(w, counts)
    reps = max(5, steps // 2)
    t_a = time_attention(pisa, torch, Qd, Kd, Vd, idx, st, w, "approx", reps)
    t_d = time_attention(pisa, torch, Qd, Kd, Vd, idx, st, w, "drop", reps)
    # the text rows' items (72 exact blocks) against the image rows' (about
    # 16): split items, the extra parts dispatched first (pisa_attention_split)
    split = {}
    for cap in (36, 24, 18, 12):
        wsz = pisa.attention_split_workspace_size(Qd, w.block, idx.shape[-1], cap)
        wsp = torch.empty(wsz, dtype=torch.uint8, device="cuda")
        row = {}
        for mode in ("approx", "drop"):
            for _ in range(2):
                pisa.attention(Qd, Kd, Vd, idx, st, w.block, mode=mode, split_blocks=cap, workspace=wsp)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                pisa.attention(Qd, Kd, Vd, idx, st, w.block, mode=mode, split_blocks=cap, workspace=wsp)
            b.record(stream)
            b.synchronize()
            row[mode + "_ms"] = a.elapsed_time(b) / reps
        row["workspace_mb"] = wsz / 1e6
        split[str(cap)] = row
        del wsp
    best = min(split, key=lambda c: split[c]["approx_ms"])
    nb = w.nb
    dense_idx = torch.arange(nb, dtype=torch.int32, device="cuda").expand(w.batch, w.heads, nb, nb).contiguous()
    t_dense = time_attention(pisa, torch, Qd, Kd, Vd, dense_idx, st, w, "drop", 3)
    fd = flops(w, nb)["exact"]
    res = {"wall_ms_per_step": wall, "step_tflops": f["step"] / wall / 1e9,
           "exact_blocks_per_row": {"min": int(counts.min()), "max": int(counts.max()),
                                    "mean": float(counts.mean())},
           "density": float(counts.sum()) / counts.size / nb,
           "attention_ms": {"approx": t_a, "drop": t_d},
           "tflops": {"attention": f["attention"] / t_a / 1e9, "exact_phase": f["exact"] / t_d / 1e9},
           "roofline_frac": {"attention": f["attention"] / t_a / 1e9 / MFMA_BF16_PEAK_TFLOPS,
                             "exact_phase": f["exact"] / t_d / 1e9 / MFMA_BF16_PEAK_TFLOPS},
           "split_items": {"by_max_blocks": split, "best_max_blocks": int(best),
                           "approx_ms": split[best]["approx_ms"], "drop_ms": split[best]["drop_ms"],
                           "tflops_attention": f["attention"] / split[best]["approx_ms"] / 1e9,
                           "tflops_exact_phase": f["exact"] / split[best]["drop_ms"] / 1e9,
                           "speedup_vs_one_workgroup_per_item": t_a / split[best]["approx_ms"]},
           "dense": {"ms": t_dense, "tflops": fd / t_dense / 1e9,
                     "speedup_of_pisa_attention": t_dense / t_a},
           "gflop": {n: v / 1e9 for n, v in f.items()}}
    del Qd, Kd, Vd, st, idx, dense_idx, ws
    torch.cuda.empty_cache()
    return res


def time_sdpa(torch, Qd, Kd, Vd, dense_flops, t_pisa):
    """torch's fused dense attention (flash or memory-efficient backend only;
    the math backend would materialise the L x L scores) on the same tensors."""
    from torch.nn.attention import sdpa_kernel, SDPBackend
    sdpa = torch.nn.functional.scaled_dot_product_attention
    try:
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION]):
            o = sdpa(Qd, Kd, Vd)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(torch.cuda.current_stream())
            for _ in range(3):
                o = sdpa(Qd, Kd, Vd)
            b.record(torch.cuda.current_stream())
            b.synchronize()
        del o
    except RuntimeError as ex:
        return {"unavailable": str(ex)[:200]}
    ms = a.elapsed_time(b) / 3
    return {"ms": ms, "tflops": dense_flops / ms / 1e9, "speedup_of_pisa_attention": ms / t_pisa}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(w, budget_s=20.0):
    """The fp64 oracle (as it stands) on whole heads of the same workload, until
    ~budget_s of oracle time, each of its three calls timed on its own."""
    import numpy as np
    import oracle
    from piecewise_block_sparse_amd import workloads as wl
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas = None
    done, fl = 0, 0.0
    calls = {"precompute": 0.0, "route": 0.0, "attention": 0.0}
    per_head = flops(wl.WORKLOADS[w.wid], w.k)
    for h in range(w.heads):
        Q, K, V = wl.make_inputs(w, heads=[h])
        t0 = time.perf_counter()
        st = oracle.precompute(K, V, w.block)
        t1 = time.perf_counter()
        idx = oracle.route(Q, st["centroid"], st["M"], w.k, w.lam, w.block, w.scale)
        t2 = time.perf_counter()
        oracle.attention(Q, K, V, idx, st["centroid"], st["vsum"], st["Hbar"], oracle.MODE_APPROX,
                         w.scale, w.block)
        t3 = time.perf_counter()
        calls["precompute"] += t1 - t0
        calls["route"] += t2 - t1
        calls["attention"] += t3 - t2
        done += 1
        fl += per_head["step"] / w.heads
        if sum(calls.values()) >= budget_s:
            break
    spent = sum(calls.values())
    return {"value": fl / spent / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} of {w.heads} heads of {w.name}, full precompute+route+attention "
                      f"each, {spent:.1f} s of fp64 numpy",
            "cpu_model": cpu_model(), "cores_available": cores, "blas_threads": blas,
            "seconds_per_call": {n: v / done for n, v in calls.items()},
            "seconds_per_call_unit": "s per head",
            "seconds_per_step_extrapolated": spent * w.heads / done}


def attainable_rates(pisa):
    """MFMA and HBM rates measured on this machine (libpisa_probe), at the
    attention kernel's occupancy: the bf16 MFMA stream alone with every operand
    in registers (N(0, 1)-like and all-zero operands: the clock the chip holds
    under MFMA work with and without operand toggling), the same MFMAs fed
    from LDS as the exact phase feeds them, the full per-chunk step of the
    exact phase (with and without toggling), and the HBM rate of a plain
    2 GiB streaming read."""
    import ctypes
    probe = pisa._lib.load_probe()
    out = {"unit": "TFLOP/s (MFMA rates), GB/s (hbm_read_gbs)",
           "data": "N(0,1)-like bf16 operands (zeros where named)",
           "probe": "pisa_probe_chunk_rate, pisa_probe_read_rate (include/pisa_probe.h)"}
    for name, mix, zeros in (("mfma_regs", 2, 0), ("mfma_regs_zeros", 2, 1), ("mfma_only", 0, 0),
                             ("chunk_mix", 1, 0), ("chunk_mix_zeros", 1, 1)):
        r = ctypes.c_double(0.0)
        rc = probe.pisa_probe_chunk_rate(mix, zeros, 2000, 5, ctypes.byref(r))
        if rc != 0:
            raise RuntimeError(f"pisa_probe_chunk_rate({mix}, {zeros}) failed with HIP error {rc}")
        out[name] = r.value
    # the streaming kernels' yardstick: a plain 2 GiB streaming read
    r = ctypes.c_double(0.0)
    rc = probe.pisa_probe_read_rate(2 << 30, 5, ctypes.byref(r))
    if rc != 0:
        raise RuntimeError(f"pisa_probe_read_rate failed with HIP error {rc}")
    out["hbm_read_gbs"] = r.value
    log(f"attainable MFMA rates: {out}")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=4, choices=[2, 3, 4],
                    help="main workload: 4 video-DiT-L (the headline), 3 video-DiT-S, 2 image-DiT "
                         "(the short-sequence case, for profiling)")
    ap.add_argument("--mode", choices=["approx", "drop"], default="approx",
                    help="attention mode of the timed step (drop: the exact phase alone, for counters)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true",
                    help="skip the dense comparators (all blocks exact; torch SDPA)")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the density sweep of the main workload")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-orders", action="store_true",
                    help="skip timing the zeroth-order and per-block first-order modes")
    ap.add_argument("--no-exact-split", action="store_true",
                    help="skip the keep-or-drop timing that splits exact / approximate phases")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache steps (e.g. under a counter profiler)")
    ap.add_argument("--no-probe", action="store_true",
                    help="skip measuring the attainable MFMA rate of the kernel's chunk mix")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (for HBM counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              f"(the path shards by heads with no exchange, so one GPU's share is what is measured).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import piecewise_block_sparse_amd as pisa
    from piecewise_block_sparse_amd import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    pisa._lib.load()

    if args.copy_calibration:
        x = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        y = torch.empty_like(x)
        y.copy_(x)
        torch.cuda.synchronize()
        del x, y

    def run(wid, steps, warmup, with_dense, split=True, orders=False, sweep=False, cold=True):
        w = wl.WORKLOADS[wid]
        log(f"{w.name}: generating inputs")
        Q, K, V = wl.make_inputs(w)
        Qd, Kd, Vd = (torch.from_numpy(a).to("cuda", torch.bfloat16) for a in (Q, K, V))
        del Q, K, V
        log(f"{w.name}: timing {steps} steps")
        wall_ms, ph, (st, idx, _) = timed_phases(pisa, torch, Qd, Kd, Vd, w, w.k, steps, warmup,
                                                 mode=args.mode)
        f, by = flops(w, w.k), bytes_moved(w)
        step_pct = ph.pop("step_event_ms")
        res = {"wall_ms_per_step": wall_ms / steps, "phases_ms": ph, "step_event_ms": step_pct}
        if cold:
            log(f"{w.name}: cold-cache steps")
            res["cold_step_ms"] = cold_steps(pisa, torch, Qd, Kd, Vd, w)
        res["tflops"] = {
            "step": f["step"] / (wall_ms / steps) / 1e9,
            # keep-or-drop steps (--mode drop) run the exact phase alone
            "attention": f["exact" if args.mode == "drop" else "attention"] / ph["attention"] / 1e9,
        }
        res["roofline_frac"] = {"attention": res["tflops"]["attention"] / MFMA_BF16_PEAK_TFLOPS}
        if split:
            t_drop = time_attention(pisa, torch, Qd, Kd, Vd, idx, st, w, "drop", max(5, steps // 2))
            res["exact_phase_ms"] = t_drop
            res["approx_phase_ms"] = ph["attention"] - t_drop
            res["tflops"]["exact_phase"] = f["exact"] / t_drop / 1e9
            res["roofline_frac"]["exact_phase"] = res["tflops"]["exact_phase"] / MFMA_BF16_PEAK_TFLOPS
            t_fused, t_ink, t_split = time_route_attention(pisa, torch, Qd, Kd, Vd, st, w,
                                                           max(5, steps // 2))
            res["route_attention_fused"] = {
                "ms": t_fused, "in_kernel_ms": t_ink, "route_plus_attention_ms": t_split,
                "step_ms_with_fused": ph["precompute"] + t_fused}
        res["gbs"] = {"precompute": by["stats"] / ph["precompute"] / 1e6,
                      "route": by["route"] / ph["route"] / 1e6}
        res["gflop"] = {n: v / 1e9 for n, v in f.items()}
        if with_dense:
            log(f"{w.name}: dense comparator")
            nb = w.nb
            dense_idx = torch.arange(nb, dtype=torch.int32, device="cuda").expand(
                w.batch, w.heads, nb, nb).contiguous()
            t_dense = time_attention(pisa, torch, Qd, Kd, Vd, dense_idx, st, w, "drop", 3)
            fd = flops(w, nb)["exact"]
            res["dense"] = {"ms": t_dense, "tflops": fd / t_dense / 1e9,
                            "speedup_of_pisa_attention": t_dense / ph["attention"]}
            del dense_idx
            res["sdpa"] = time_sdpa(torch, Qd, Kd, Vd, fd, ph["attention"])
        if sweep:
            log(f"{w.name}: density sweep")
            rows = []
            for k in (w.nb // 2, w.nb // 4, w.nb // 8, w.nb // 16):
                idx_k = pisa.route(Qd, st, k, w.lam, w.block)
                fk = flops(w, k)
                t_a = time_attention(pisa, torch, Qd, Kd, Vd, idx_k, st, w, "approx", 5)
                t_d = time_attention(pisa, torch, Qd, Kd, Vd, idx_k, st, w, "drop", 5)
                rows.append({"k": k, "density": k / w.nb,
                             "approx_ms": t_a, "approx_tflops": fk["attention"] / t_a / 1e9,
                             "drop_ms": t_d, "exact_tflops": fk["exact"] / t_d / 1e9})
                del idx_k
            res["density_sweep"] = rows
        if orders:
            # the other treatments of the unselected blocks, same inputs and idx
            log(f"{w.name}: zeroth-order and per-block first-order modes")
            st_ht = pisa.precompute(Kd, Vd, w.block, store_Ht=True)
            t0 = time_attention(pisa, torch, Qd, Kd, Vd, idx, st_ht, w, "zeroth", max(5, steps // 2))
            t1 = time_attention(pisa, torch, Qd, Kd, Vd, idx, st_ht, w, "first", 3)
            hbytes = w.batch * w.heads * w.nb * (w.nb - w.k) * w.head_dim ** 2 * 2
            res["orders"] = {
                "zeroth": {"ms": t0, "tflops": f["attention_zeroth"] / t0 / 1e9},
                "first_per_block": {"ms": t1, "tflops": f["attention_first"] / t1 / 1e9,
                                    "H_stream_gbs": hbytes / (t1 - t0) / 1e6},
            }
            res["gflop"]["attention_zeroth"] = f["attention_zeroth"] / 1e9
            res["gflop"]["attention_first"] = f["attention_first"] / 1e9
            del st_ht
            # the spectral reading of M_j (largest singular value) in the statistics
            for _ in range(2):
                st_sp = pisa.precompute(Kd, Vd, w.block, norm="spectral")
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(torch.cuda.current_stream())
            for _ in range(3):
                st_sp = pisa.precompute(Kd, Vd, w.block, norm="spectral")
            b.record(torch.cuda.current_stream())
            b.synchronize()
            idx_sp = pisa.route(Qd, st_sp, w.k, w.lam, w.block)
            same = (idx_sp.view(-1, w.k).unsqueeze(-1) == idx.view(-1, w.k).unsqueeze(-2)).any(-1)
            res["spectral_M"] = {"precompute_ms": a.elapsed_time(b) / 3,
                                 "routing_overlap_with_frobenius": float(same.float().mean())}
            del st_sp, idx_sp, same
        del Qd, Kd, Vd, st, idx
        torch.cuda.empty_cache()
        return w, res

    w, main_res = run(args.workload, args.steps, args.warmup, not args.no_dense,
                      not args.no_exact_split, not args.no_orders, not args.no_sweep, not args.no_cold)
    f = flops(w, w.k)
    ms = main_res["wall_ms_per_step"]
    t_attn = main_res["phases_ms"]["attention"]
    achieved = f["exact" if args.mode == "drop" else "attention"] / t_attn / 1e9
    traffic = profiled_traffic(w.name)
    bh = w.batch * w.heads
    min_bytes = 4 * bh * w.seq_len * w.head_dim * 2          # Q, K, V read once, O written once
    line = {
        "metric": "PISA attention latency (ms) & TFLOP/s at L=32K d=128 12.5% density; MFMA util",
        "value": f["step"] / ms / 1e9,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; smooth latent-grid field + N(0,1) noise)",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "seq_len": w.seq_len,
                   "head_dim": w.head_dim, "block": w.block, "k": w.k,
                   "density": w.k / w.nb, "lambda": w.lam, "mode": args.mode},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": traffic["total"] if traffic else None,
                     "traffic_detail": dict(traffic, algorithmic_min=min_bytes) if traffic else None,
                     "kernel": f"attn_bf16_kernel (d={w.head_dim}, block={w.block})",
                     # rocprofv3 counters of the same kernels (committed profile, source-stamped)
                     "phase_counters": phase_counters(w.name),
                     "avg_launch_ms": t_attn,
                     # the metric's MFMA utilisation: algorithmic bf16 rate over the peak
                     "mfma_util": {
                         "attention": achieved / MFMA_BF16_PEAK_TFLOPS,
                         "exact_phase": (main_res["tflops"]["exact_phase"] / MFMA_BF16_PEAK_TFLOPS
                                         if "exact_phase" in main_res["tflops"] else None)}},
        "phases": main_res,
    }
    if not args.no_probe:
        att = attainable_rates(pisa)
        if "exact_phase" in main_res["tflops"]:
            att["exact_phase_frac_of_chunk_mix"] = main_res["tflops"]["exact_phase"] / att["chunk_mix"]
        att["precompute_frac_of_read"] = main_res["gbs"]["precompute"] / att["hbm_read_gbs"]
        att["route_frac_of_read"] = main_res["gbs"]["route"] / att["hbm_read_gbs"]
        line["roofline"]["attainable"] = att
    if not args.no_secondary:
        other = 3 if args.workload == 4 else 4
        _, res2 = run(other, args.steps, max(3, args.warmup), False, cold=not args.no_cold)
        line["secondary"] = {wl.WORKLOADS[other].name: res2}
        # the short image workload (4K tokens): whole steps, the single-launch
        # routing call against route + attention, and the dense comparator
        if args.workload != 2:
            _, res3 = run(2, args.steps, max(3, args.warmup), not args.no_dense,
                          split=not args.no_exact_split, cold=False)
            line["secondary"][wl.WORKLOADS[2].name] = res3
        line["secondary"][wl.WORKLOADS[5].name] = fixed_mask(pisa, torch, args.steps, max(3, args.warmup))
    if not args.no_cpu_baseline:
        log("cpu baseline (fp64 oracle)")
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
