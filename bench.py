"""Benchmark of the delta-rule chunked forward (+ decode step) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

A step is one whole chunked forward (WY prep + state scan/output kernels)
over the long-context workload: bf16 q/k/v, B=1, H=32, L=65536,
d_k=d_v=128, C=128, fp32 beta/state, zero initial state, fp32 o, seeded
synthetic inputs resident in HBM before the timed region.  The same forward
with o stored in bf16 is reported under "bf16_out".  The decode step (B=256
sequences x H=32 heads, d=128, fp32 state of 512 MiB) runs 1000 successive
steps, each on its own seeded inputs staged in HBM beforehand, eagerly (HIP
events around every kernel) and as one captured HIP graph (the per-step
time), reported under "decode".  "cpu_baseline" is the fp64 oracle on the
whole long-context workload, its heads split over the host's cores.

Prints ONE JSON line.  value = tokens/s of the chunked forward (B*L tokens per
step; a token counts once across heads).  Model TFLOP/s follow the cost model
2 L d_k d_v + 2 L C d_k per head.  Rooflines use algorithmic bytes (each input
read once, each output written once) divided by the kernel's average duration
from HIP events recorded on the launch stream around every launch.
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

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s

CSRC = os.path.join(ROOT, "deltanet_delta_rule_chunk_amd", "csrc")
# Source files each kernel is built from (a change to any of them makes the
# committed counter measurement stale).
KERNEL_SOURCES = {
    "chunk_scan": ["dn_scan_mfma.hip", "dn_buffer.h", "dn_ktile.h", "dn_tfrag.h", "dn_mfma.h",
                   "dn_common.h"],
    "chunk_prep": ["dn_chunk_mfma.hip", "dn_features.h", "dn_ktile.h", "dn_tfrag.h", "dn_mfma.h",
                   "dn_common.h"],
    "decode": ["dn_decode.hip", "dn_features.h", "dn_common.h"],
    "features": ["dn_features.hip", "dn_features.h", "dn_common.h"],
}
# The gated instantiations, and the decode step that applies the feature
# maps in-kernel, come from the same sources.
KERNEL_SOURCES.update({"gated_" + k: v for k, v in list(KERNEL_SOURCES.items()) if k != "features"})
KERNEL_SOURCES["features_decode"] = KERNEL_SOURCES["decode"]
# The WY-prep kernel that applies the feature maps as it loads q and k.
KERNEL_SOURCES["features_chunk_prep"] = KERNEL_SOURCES["chunk_prep"]
KERNEL_SOURCES["kda_decode"] = KERNEL_SOURCES["decode"]
KERNEL_SOURCES["kda_chunk_prep"] = KERNEL_SOURCES["kda_chunk_scan"] = [
    "dn_kda.hip", "dn_kda.h", "dn_kda_mfma.hip", "dn_lds64.h", "dn_inv64.h", "dn_mfma.h",
    "dn_valu_common.h", "dn_common.h"]
for _k in ("bwd_prep", "bwd_scan", "bwd_qk"):
    KERNEL_SOURCES[_k] = ["dn_backward.hip", "dn_backward.h", "dn_backward_mfma.hip", "dn_lds64.h",
                          "dn_mfma.h", "dn_valu_common.h", "dn_common.h"]
# The backward's forward pass is the chunked forward's prep in its form that
# also writes X of each 64-token block, then the chunked forward's scan in
# its BWD form; one profiling slot brackets both.
KERNEL_SOURCES["bwd_fwd_prep"] = KERNEL_SOURCES["chunk_prep"]
KERNEL_SOURCES["bwd_fwd_scan"] = KERNEL_SOURCES["chunk_scan"]
SLOT_KERNELS = {"bwd_fwd_scan": ("bwd_fwd_prep", "bwd_fwd_scan")}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
MFMA_FILE = os.path.join(ROOT, "profiles", "mfma_counters.json")


def kernel_source_hash(kernel):
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE, each scaled by what the counter
    reads for a copy kernel of known size), or None when there is none or
    the kernel's sources changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)["kernels"][kernel]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha256") != kernel_source_hash(kernel):
        return None
    return rec["bytes_per_launch"]


def measured_mfma(kernel):
    """Executed bf16 MFMA flops per launch of `kernel` and its MFMA-busy share
    from the committed rocprofv3 counter summary
    (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512, SQ_VALU_MFMA_BUSY_CYCLES), or None
    when there is none or the kernel's sources changed since it was taken."""
    try:
        with open(MFMA_FILE) as fh:
            rec = json.load(fh)["kernels"][kernel]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha256") != kernel_source_hash(kernel):
        return None
    return rec


def hbm_rate(kernel, ms):
    """HBM rate of one launch of `kernel` taking `ms`: the counter-measured
    bytes per launch (workspace traffic included) over the time, or None
    when the committed counters are missing or stale.  A profiling slot that
    brackets several kernels (SLOT_KERNELS) sums their bytes."""
    parts = [measured_traffic(k) for k in SLOT_KERNELS.get(kernel, (kernel,))]
    b = None if any(p is None for p in parts) else sum(parts)
    if b is None:
        return None
    gbs = b / (ms * 1e-3) / 1e9
    return {"bytes": b, "gbs": gbs, "pct_hbm_peak": 100.0 * gbs / PEAK_HBM_GBS}


def chunk_bytes(w, in_bytes=2, out_bytes=4, s0=False):
    """Algorithmic bytes of one chunked forward: q, k, v, beta read once, o and
    S_final written once (S0 read once if given)."""
    tok_heads = w.B * w.H * w.L
    b = tok_heads * (2 * w.d_k + w.d_v) * in_bytes + tok_heads * 4 + tok_heads * w.d_v * out_bytes
    state = w.B * w.H * w.d_k * w.d_v * 4
    return b + state * (2 if s0 else 1)


def scan_kernel_bytes(w, in_bytes=2, out_bytes=4):
    """Algorithmic bytes of the scan kernel alone: q, k, v read once, o and
    S_final written once (beta is consumed by the prep kernel)."""
    tok_heads = w.B * w.H * w.L
    return (tok_heads * (2 * w.d_k + w.d_v) * in_bytes + tok_heads * w.d_v * out_bytes
            + w.B * w.H * w.d_k * w.d_v * 4)


def prep_bytes(w, in_bytes=2):
    """Algorithmic bytes of the WY-prep kernel: its share of the path's own
    inputs, k and beta, each read once.  (Its output, T, is an intermediate
    of the path: see ``t_workspace_bytes``.)"""
    return w.B * w.H * w.L * (w.d_k * in_bytes + 4)


def t_workspace_bytes(w):
    """Bytes of T fragments the WY-prep kernel writes and the scan reads back
    (C/32 (C/32 + 1) blocks of 2 KiB per chunk: the lower triangle at 16 x 32
    granularity, hi and lo planes)."""
    nc = -(-w.L // w.C)
    return w.B * w.H * nc * (w.C // 32) * (w.C // 32 + 1) * 2048


def feature_bytes(w, in_bytes=2):
    """Algorithmic bytes of the feature maps: raw q, k read and mapped q, k
    written once in the storage dtype, the beta logits read and beta written
    once (fp32).  The same figure serves the streaming feature kernel and the
    WY-prep kernel that applies the maps (which also writes T, counted
    apart)."""
    tok_heads = w.B * w.H * w.L
    return tok_heads * (4 * w.d_k * in_bytes + 8)


def model_flops(w):
    return w.B * w.H * (2 * w.L * w.d_k * w.d_v + 2 * w.L * w.C * w.d_k)


def decode_bytes(w, in_bytes=2, out_bytes=4):
    bh = w.B * w.H
    return 2 * bh * w.d_k * w.d_v * 4 + bh * ((2 * w.d_k + w.d_v) * in_bytes + 4 + w.d_v * out_bytes)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def cpu_baseline(w, x):
    """The fp64 oracle, as it stands, on the whole workload (every head, every
    token), its heads split over worker processes on the host's cores (at most
    16, the host share of one GPU); wall time from the start of the pool to
    the last result, process start-up and data transfer included."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from oracle import delta_rule_forward
    from oracle_pool import n_workers, oracle_heads

    nw = n_workers(w.B * w.H)
    t0 = time.perf_counter()
    o_ref, _ = oracle_heads(delta_rule_forward, (x["q"], x["k"], x["v"], x["beta"], x["S0"]))
    dt = time.perf_counter() - t0
    assert np.isfinite(o_ref).all()
    return {"value": w.B * w.L / dt, "unit": "tokens/s", "cores": nw, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"the whole workload: B={w.B}, H={w.H}, L={w.L}, d={w.d_k}; fp64 numpy "
                      f"token loop, heads split over {nw} worker processes, {dt:.1f} s wall"}


def stage_steps(make, steps, dev):
    """Inputs of decode steps 0 .. steps-1 from ``make(step)`` (a dict of host
    tensors), generated on host threads in blocks and stacked on the device
    as one ``[steps, ...]`` tensor per name."""
    from concurrent.futures import ThreadPoolExecutor

    import torch

    first = make(0)
    out = {k: torch.empty((steps,) + tuple(t.shape), dtype=t.dtype, device=dev)
           for k, t in first.items()}
    blk = 64
    with ThreadPoolExecutor(max_workers=16) as ex:
        for s0 in range(0, steps, blk):
            n = min(blk, steps - s0)
            for i, r in enumerate(ex.map(make, range(s0, s0 + n))):
                for k, t in r.items():
                    out[k][s0 + i].copy_(t, non_blocking=False)
    return out


def timed_steps(step, warmup, steps):
    """``warmup`` untimed calls of ``step()`` straight before ``steps`` timed
    ones, with nothing but a device synchronisation between the two: after
    an idle stretch the GPU's clocks take some milliseconds of load to
    settle, so a host-side pause (an allocation, a check that reads the
    result back) between warmup and timing would put that transient in the
    timed region.  Returns (ms per step from events around the timed calls,
    the library's per-kernel profile of them, wall seconds)."""
    import torch

    from deltanet_delta_rule_chunk_amd import binding

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    binding.profile_start()
    binding.profile_stop()  # creates the profiling events outside the timed region
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    binding.profile_start()
    t_wall = time.perf_counter()
    ev0.record()
    for _ in range(steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    prof = binding.profile_stop()
    return ev0.elapsed_time(ev1) / steps, prof, t_wall


def graph_ms_per_step(launch, steps, reset, check):
    """Captures ``launch(0) .. launch(steps-1)`` into one HIP graph and replays
    it three times, each from the same starting state (``reset()`` runs
    before every replay, outside the timed region).  Returns the mean time
    per step of the last two replays; ``check()`` compares every replay's
    result with the eager run's."""
    import torch

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            launch(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    for rep in range(3):
        reset()
        torch.cuda.synchronize()
        ev0.record()
        g.replay()
        ev1.record()
        torch.cuda.synchronize()
        times.append(ev0.elapsed_time(ev1) / steps)
        check()
    del g
    return sum(times[1:]) / 2


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip timing the two smaller chunked workloads")
    ap.add_argument("--no-gated", action="store_true",
                    help="skip the gated (Gated DeltaNet) forward and decode measurements")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the chunked backward (gradient) measurement")
    ap.add_argument("--no-kda", action="store_true",
                    help="skip the per-dimension-decay (KDA) forward and decode measurements")
    ap.add_argument("--no-features", action="store_true",
                    help="skip the forward and decode fed by raw projections (feature maps)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 5 device-to-device copies of MIB MiB (the known-size "
                         "reference for the HBM byte counters) and exit")
    a = ap.parse_args(argv)

    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(heads would shard with no communication; see the design notes).", file=sys.stderr)
        return 2

    import torch

    if a.copy_calibration:
        n = a.copy_calibration << 20
        src = torch.ones(n // 4, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 5}), flush=True)
        return 0

    from deltanet_delta_rule_chunk_amd import binding, inputs

    binding.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = inputs.WORKLOADS[3]
    print(f"[bench] generating {w.name}", file=sys.stderr, flush=True)
    x = inputs.make_chunk_inputs(w, seed=a.seed)
    g = {k: (None if t is None else t.to(dev)) for k, t in x.items()}
    o = torch.empty(w.B, w.H, w.L, w.d_v, device=dev, dtype=torch.float32)
    S_final = torch.empty(w.B, w.H, w.d_k, w.d_v, device=dev, dtype=torch.float32)
    ws = torch.empty(binding.workspace_bytes(w.B, w.H, w.L, w.d_k, w.d_v, w.C), dtype=torch.uint8,
                     device=dev)

    def step():
        binding.chunk_fwd(g["q"], g["k"], g["v"], g["beta"], None, w.C, o=o, S_final=S_final,
                          workspace=ws)

    print(f"[bench] {a.warmup} warmup + {a.steps} timed chunked-forward steps", file=sys.stderr,
          flush=True)
    ms_step, prof, t_wall = timed_steps(step, a.warmup, a.steps)
    assert torch.isfinite(o).all() and torch.isfinite(S_final).all()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    tokens_s = w.B * w.L / (ms_step * 1e-3)
    flops = model_flops(w)
    tflops = flops / (ms_step * 1e-3) / 1e12
    kern = {name: tot / n for name, (tot, n) in prof.items()}
    dom = max((k for k in kern if k.startswith("chunk")), key=lambda k: kern[k])
    dom_bytes = scan_kernel_bytes(w) if dom == "chunk_scan" else prep_bytes(w)
    achieved = dom_bytes / (kern[dom] * 1e-3) / 1e9
    path_gbs = chunk_bytes(w) / (ms_step * 1e-3) / 1e9

    result = {
        "metric": "delta-rule chunk fwd tokens/s + TFLOP/s (% bf16 MFMA peak); decode GB/s % HBM",
        "value": tokens_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded: q,v ~ N(0,1); k ~ N(0,1) L2-normalised; beta = sigmoid(N(0,1)))",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "L": w.L, "d_k": w.d_k, "d_v": w.d_v,
                   "C": w.C, "in_dtype": "bf16", "state_dtype": "f32", "out_dtype": "f32",
                   "global_batch": w.B, "seq_len": w.L, "parallelism": "single GPU"},
        "model_tflops": tflops,
        "pct_bf16_mfma_peak": 100.0 * tflops / PEAK_BF16_TFLOPS,
        "path_alg_gbs": path_gbs,
        "pct_hbm_peak_path": 100.0 * path_gbs / PEAK_HBM_GBS,
        "kernels_ms": kern,
        "prep_roofline": {"bound": "hbm", "kernel": "chunk_prep",
                          "achieved": prep_bytes(w) / (kern["chunk_prep"] * 1e-3) / 1e9,
                          "peak": PEAK_HBM_GBS, "unit": "GB/s",
                          "frac": prep_bytes(w) / (kern["chunk_prep"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
                          "traffic": measured_traffic("chunk_prep"),
                          "t_workspace_bytes_written": t_workspace_bytes(w)},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                     "traffic": measured_traffic(dom)},
        "wall_s_timed": t_wall,
    }
    # The matrix-core work the kernels really issue (split-precision operands,
    # the delta rule's three state products, per-slice diagonal blocks) is
    # well above the pages' cost model: executed flops from the counters,
    # rate from this run's kernel times.
    ex = {}
    for kname in ("chunk_prep", "chunk_scan"):
        rec = measured_mfma(kname)
        if rec is not None:
            tf = rec["bf16_flops"] / (kern[kname] * 1e-3) / 1e12
            ex[kname] = {"bf16_flops_per_launch": rec["bf16_flops"], "tflops": tf,
                         "pct_bf16_mfma_peak": 100.0 * tf / PEAK_BF16_TFLOPS,
                         "mfma_busy_pct_counters": rec["mfma_busy_pct"]}
    result["executed_mfma"] = ex or None

    # The same forward with o stored in bf16 (the other output mode the
    # boundary offers; fp32 o is the headline).
    print(f"[bench] timing {a.steps} chunked-forward steps, bf16 o", file=sys.stderr, flush=True)
    o16 = torch.empty(w.B, w.H, w.L, w.d_v, device=dev, dtype=torch.bfloat16)

    def step16():
        binding.chunk_fwd(g["q"], g["k"], g["v"], g["beta"], None, w.C, o=o16, S_final=S_final,
                          workspace=ws, out_dtype=torch.bfloat16)

    ms16, prof16, _ = timed_steps(step16, a.warmup, a.steps)
    assert torch.isfinite(o16).all()
    kern16 = {name: tot / n for name, (tot, n) in prof16.items()}
    b16 = scan_kernel_bytes(w, out_bytes=2)
    result["bf16_out"] = {
        "workload": w.name + "_bf16_out", "steps": a.steps, "ms_per_step": ms16,
        "tokens_per_s": w.B * w.L / (ms16 * 1e-3),
        "model_tflops": flops / (ms16 * 1e-3) / 1e12,
        "path_alg_gbs": chunk_bytes(w, out_bytes=2) / (ms16 * 1e-3) / 1e9,
        "kernels_ms": kern16,
        "roofline": {"bound": "hbm", "kernel": "chunk_scan",
                     "achieved": b16 / (kern16["chunk_scan"] * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s",
                     "frac": b16 / (kern16["chunk_scan"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
                     "traffic": None},
    }
    del o16

    if not a.no_decode:
        wd = inputs.WORKLOADS[4]
        nds = a.decode_steps
        print(f"[bench] decode {wd.name}: staging {nds} step inputs", file=sys.stderr, flush=True)
        S_init = inputs.make_decode_state(wd, seed=a.seed).to(dev)
        Sd = S_init.clone()
        D = stage_steps(lambda s: inputs.make_decode_step_inputs(wd, s, seed=a.seed), nds, dev)
        od = torch.empty(wd.B, wd.H, wd.d_v, device=dev, dtype=torch.float32)

        def dlaunch(s):
            binding.decode_step(D["q"][s], D["k"][s], D["v"][s], D["beta"][s], Sd, o=od)

        # Eager run over every step (HIP events around each kernel), then the
        # same steps from the same state as one captured graph.
        print(f"[bench] decode {wd.name}: {nds} steps eager, then as a HIP graph",
              file=sys.stderr, flush=True)
        for s in range(3):
            dlaunch(s)
        torch.cuda.synchronize()
        Sd.copy_(S_init)
        torch.cuda.synchronize()
        binding.profile_start()
        ev0.record()
        for s in range(nds):
            dlaunch(s)
        ev1.record()
        torch.cuda.synchronize()
        dprof = binding.profile_stop()
        assert torch.isfinite(od).all()
        ms_eager = ev0.elapsed_time(ev1) / nds
        k_ms = dprof["decode"][0] / dprof["decode"][1]
        S_eager, o_eager = Sd.clone(), od.clone()

        def dcheck():
            assert torch.equal(Sd, S_eager) and torch.equal(od, o_eager), \
                "graph replay differs from the eager decode run"

        ms_dec = graph_ms_per_step(dlaunch, nds, lambda: Sd.copy_(S_init), dcheck)
        del S_eager, o_eager
        db = decode_bytes(wd)
        result["decode"] = {
            "workload": wd.name, "steps": nds, "ms_per_step": ms_dec,
            "ms_per_step_eager": ms_eager,
            "kernel_ms": k_ms, "tokens_per_s": wd.B / (ms_dec * 1e-3),
            "alg_gbs": db / (ms_dec * 1e-3) / 1e9,
            "pct_hbm_peak": 100.0 * db / (ms_dec * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "roofline": {"bound": "hbm", "kernel": "decode", "achieved": db / (k_ms * 1e-3) / 1e9,
                         "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": db / (k_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                         "traffic": measured_traffic("decode")},
            "inputs": f"{nds} seeded step inputs, a fresh set per step, staged in HBM before "
                      "timing; state carried across all steps",
            "timing": "ms_per_step: the steps captured in one HIP graph and replayed (every "
                      "replay checked equal to the eager run); kernel_ms: HIP events around "
                      "each kernel of the eager run",
        }

    if not a.no_gated:
        # The gated form (per-token decay alpha) on the same workloads; a
        # secondary figure next to the plain path's headline number.
        print(f"[bench] gated forward {w.name}: {a.steps} steps", file=sys.stderr, flush=True)
        alpha = inputs.make_chunk_alpha(w, seed=a.seed).to(dev)
        gws = torch.empty(binding.workspace_bytes(w.B, w.H, w.L, w.d_k, w.d_v, w.C, gated=True),
                          dtype=torch.uint8, device=dev)

        def gstep():
            binding.chunk_fwd(g["q"], g["k"], g["v"], g["beta"], None, w.C, o=o, S_final=S_final,
                              workspace=gws, alpha=alpha)

        ms_g, gprof, _ = timed_steps(gstep, a.warmup, a.steps)
        assert torch.isfinite(o).all() and torch.isfinite(S_final).all()
        result["gated"] = {
            "workload": w.name + "_gated", "steps": a.steps, "ms_per_step": ms_g,
            "tokens_per_s": w.B * w.L / (ms_g * 1e-3),
            "kernels_ms": {name: tot / n for name, (tot, n) in gprof.items()},
            "alpha": "sigmoid(N(3, 1)) per token (seeded stream of its own)",
        }
        if not a.no_decode:
            nd = max(1, a.decode_steps // 4)
            print(f"[bench] gated decode {wd.name}: {nd} steps", file=sys.stderr, flush=True)
            GA = stage_steps(lambda s: {"alpha": inputs.make_decode_alpha(wd, s, seed=a.seed)},
                             nd, dev)["alpha"]
            Sd.copy_(S_init)
            binding.profile_start()
            ev0.record()
            for s in range(nd):
                binding.decode_step(D["q"][s], D["k"][s], D["v"][s], D["beta"][s], Sd, o=od,
                                    alpha=GA[s])
            ev1.record()
            torch.cuda.synchronize()
            gdprof = binding.profile_stop()
            assert torch.isfinite(od).all()
            ms_gd = ev0.elapsed_time(ev1) / nd
            gk = gdprof["decode"][0] / gdprof["decode"][1]
            gdb = decode_bytes(wd) + wd.B * wd.H * 4
            result["gated"]["decode"] = {
                "workload": wd.name + "_gated", "steps": nd,
                "inputs": "a fresh seeded set per step, staged in HBM before timing",
                "ms_per_step": ms_gd, "kernel_ms": gk,
                "tokens_per_s": wd.B / (ms_gd * 1e-3),
                "pct_hbm_peak": 100.0 * gdb / (gk * 1e-3) / 1e9 / PEAK_HBM_GBS,
            }

    if not a.no_backward:
        # The gradient of the same forward (recomputing it inside): dO ~ N(0, 1).
        print(f"[bench] backward {w.name}: {a.steps} steps", file=sys.stderr, flush=True)
        gen = torch.Generator(device=dev)
        gen.manual_seed(a.seed + 17)
        dO = torch.randn(w.B, w.H, w.L, w.d_v, device=dev, generator=gen)
        bws = torch.empty(binding.bwd_workspace_bytes(w.B, w.H, w.L, w.d_k, w.d_v, w.C),
                          dtype=torch.uint8, device=dev)

        grads = []

        def bstep():
            grads[:] = binding.chunk_bwd(g["q"], g["k"], g["v"], g["beta"], None, dO, None, w.C,
                                         workspace=bws)

        ms_b, bprof, _ = timed_steps(bstep, a.warmup, a.steps)
        assert all(torch.isfinite(t).all() for t in grads if t is not None)
        bms = {name: tot / n for name, (tot, n) in bprof.items()}
        result["backward"] = {
            "workload": w.name + "_backward", "steps": a.steps, "ms_per_step": ms_b,
            "tokens_per_s": w.B * w.L / (ms_b * 1e-3),
            "kernels_ms": bms,
            "kernels_hbm": {name: hbm_rate(name, t) for name, t in bms.items()},
            "path": "64-token chunks; the forward recomputed inside on the chunked forward's prep (also writing X of each 64-token block) and scan at 128-token chunks (slot bwd_fwd_scan: both kernels); every product on bf16 MFMA (split-precision operands), the triangular inverses' diagonal blocks fp32 vector ALU",
            "grads_in": "dO ~ N(0, 1) (torch generator seeded), no dS_final",
        }
        del bws, dO, grads

    if not a.no_kda:
        # Per-dimension decay (KDA): the chunked forward, and the decode step
        # with a d_k-vector gate per (b, h).
        print(f"[bench] kda forward {w.name}: {a.steps} steps", file=sys.stderr, flush=True)
        kalpha = inputs.make_chunk_kda_alpha(w, seed=a.seed).to(dev)
        kws = torch.empty(binding.kda_workspace_bytes(w.B, w.H, w.L, w.d_k, w.d_v, w.C),
                          dtype=torch.uint8, device=dev)

        def kstep():
            binding.kda_chunk_fwd(g["q"], g["k"], g["v"], kalpha, g["beta"], None, w.C, o=o,
                                  S_final=S_final, workspace=kws)

        ms_k, kprof, _ = timed_steps(kstep, a.warmup, a.steps)
        assert torch.isfinite(o).all() and torch.isfinite(S_final).all()
        kms = {name: tot / n for name, (tot, n) in kprof.items()}
        result["kda"] = {
            "workload": w.name + "_kda", "steps": a.steps, "ms_per_step": ms_k,
            "tokens_per_s": w.B * w.L / (ms_k * 1e-3),
            "kernels_ms": kms,
            "kernels_hbm": {name: hbm_rate("kda_" + name, t) for name, t in kms.items()},
            "path": "64-token chunks; bf16 MFMA with split-precision operands for the scan, the prep tiles below the 16-row block diagonal and the inverse's off-diagonal blocks; fp32 vector ALU for the diagonal tiles",
            "alpha": "sigmoid(N(3, 1)) per token and key dimension (seeded stream of its own)",
        }
        del kws, kalpha
        if not a.no_decode:
            nd = max(1, a.decode_steps // 4)
            print(f"[bench] kda decode {wd.name}: {nd} steps", file=sys.stderr, flush=True)
            KA = stage_steps(lambda s: {"alpha": inputs.make_decode_kda_alpha(wd, s, seed=a.seed)},
                             nd, dev)["alpha"]
            Sd.copy_(S_init)
            binding.profile_start()
            ev0.record()
            for s in range(nd):
                binding.kda_decode_step(D["q"][s], D["k"][s], D["v"][s], KA[s], D["beta"][s], Sd,
                                        o=od)
            ev1.record()
            torch.cuda.synchronize()
            kdprof = binding.profile_stop()
            assert torch.isfinite(od).all()
            ms_kd = ev0.elapsed_time(ev1) / nd
            kk = kdprof["decode"][0] / kdprof["decode"][1]
            kdb = decode_bytes(wd) + wd.B * wd.H * wd.d_k * 4
            result["kda"]["decode"] = {
                "workload": wd.name + "_kda", "steps": nd,
                "inputs": "a fresh seeded set per step, staged in HBM before timing",
                "ms_per_step": ms_kd, "kernel_ms": kk,
                "tokens_per_s": wd.B / (ms_kd * 1e-3),
                "roofline": {"bound": "hbm", "kernel": "kda_decode",
                             "achieved": kdb / (kk * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                             "unit": "GB/s", "frac": kdb / (kk * 1e-3) / 1e9 / PEAK_HBM_GBS,
                             "traffic": measured_traffic("kda_decode")},
            }

    if not a.no_features:
        # The layer's feature maps (silu + L2-normalise of q, k; sigmoid of the
        # beta logits) in front of the same forward, from raw projections.
        print(f"[bench] feature maps + forward {w.name}: {a.steps} steps", file=sys.stderr,
              flush=True)
        r = {k: (None if t is None else t.to(dev))
             for k, t in inputs.make_chunk_raw_inputs(w, seed=a.seed).items()}
        fws = torch.empty(binding.workspace_bytes(w.B, w.H, w.L, w.d_k, w.d_v, w.C, features=True),
                          dtype=torch.uint8, device=dev)

        def fstep():
            binding.chunk_fwd(r["q_raw"], r["k_raw"], r["v"], r["beta_logit"], None, w.C, o=o,
                              S_final=S_final, workspace=fws, features=True)

        ms_f, fprof, _ = timed_steps(fstep, a.warmup, a.steps)
        assert torch.isfinite(o).all() and torch.isfinite(S_final).all()
        fk = {name: tot / n for name, (tot, n) in fprof.items()}
        fb = feature_bytes(w)
        fpb = fb + t_workspace_bytes(w)
        result["features"] = {
            "workload": w.name + "_features", "steps": a.steps, "ms_per_step": ms_f,
            "tokens_per_s": w.B * w.L / (ms_f * 1e-3), "kernels_ms": fk,
            "path": "feature maps applied inside the WY-prep kernel (raw q, k, beta logits in; "
                    "mapped q, k, beta and T out), then the scan",
            "roofline": {"bound": "hbm", "kernel": "features_chunk_prep",
                         "achieved": fpb / (fk["chunk_prep"] * 1e-3) / 1e9,
                         "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": fpb / (fk["chunk_prep"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
                         "bytes": "feature maps' bytes + T written",
                         "traffic": measured_traffic("features_chunk_prep")},
            "inputs": "q_raw, k_raw, v ~ N(0,1) bf16; beta logits ~ N(0,1) fp32 (own seeded stream)",
        }
        # The streaming feature kernel alone (deltanet_feature_prep), which the
        # fp32 path runs in front of its forward.
        fo = [torch.empty_like(r["q_raw"]), torch.empty_like(r["k_raw"]),
              torch.empty_like(r["beta_logit"])]

        def mstep():
            lib = binding.load()
            st = lib.deltanet_feature_prep(r["q_raw"].data_ptr(), r["k_raw"].data_ptr(),
                                           r["beta_logit"].data_ptr(), fo[0].data_ptr(),
                                           fo[1].data_ptr(), fo[2].data_ptr(), w.B, w.H, w.L,
                                           w.d_k, 1, torch.cuda.current_stream().cuda_stream)
            assert st == 0, st

        ms_m, mprof, _ = timed_steps(mstep, a.warmup, a.steps)
        km = mprof["features"][0] / mprof["features"][1]
        result["features"]["feature_kernel"] = {
            "ms": km,
            "roofline": {"bound": "hbm", "kernel": "features", "achieved": fb / (km * 1e-3) / 1e9,
                         "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": fb / (km * 1e-3) / 1e9 / PEAK_HBM_GBS,
                         "traffic": measured_traffic("features")},
        }
        del r, fws, fo
        if not a.no_decode:
            nd = max(1, a.decode_steps // 4)
            print(f"[bench] decode with feature maps {wd.name}: {nd} steps", file=sys.stderr,
                  flush=True)
            FR = stage_steps(lambda s: inputs.make_decode_raw_step_inputs(wd, s, seed=a.seed),
                             nd, dev)
            Sd.copy_(S_init)
            binding.profile_start()
            ev0.record()
            for s in range(nd):
                binding.decode_step(FR["q_raw"][s], FR["k_raw"][s], FR["v"][s],
                                    FR["beta_logit"][s], Sd, o=od, features=True)
            ev1.record()
            torch.cuda.synchronize()
            fdprof = binding.profile_stop()
            assert torch.isfinite(od).all()
            ms_fd = ev0.elapsed_time(ev1) / nd
            fdk = fdprof["decode"][0] / fdprof["decode"][1]
            result["features"]["decode"] = {
                "workload": wd.name + "_features", "steps": nd,
                "inputs": "a fresh seeded set per step, staged in HBM before timing",
                "ms_per_step": ms_fd,
                "kernel_ms": fdk, "tokens_per_s": wd.B / (ms_fd * 1e-3),
                "pct_hbm_peak": 100.0 * decode_bytes(wd) / (fdk * 1e-3) / 1e9 / PEAK_HBM_GBS,
                "traffic": measured_traffic("features_decode"),
            }

    if not a.no_other_workloads:
        # The other chunked workloads (parity cases; timed here for reference).
        others = []
        for wo in (inputs.WORKLOADS[1], inputs.WORKLOADS[2]):
            print(f"[bench] {wo.name}: {a.steps} steps", file=sys.stderr, flush=True)
            xo = {k: (None if t is None else t.to(dev)) for k, t in inputs.make_chunk_inputs(wo, seed=a.seed).items()}
            oo = torch.empty(wo.B, wo.H, wo.L, wo.d_v, device=dev, dtype=torch.float32)
            So = torch.empty(wo.B, wo.H, wo.d_k, wo.d_v, device=dev, dtype=torch.float32)
            wso = torch.empty(binding.workspace_bytes(wo.B, wo.H, wo.L, wo.d_k, wo.d_v, wo.C),
                              dtype=torch.uint8, device=dev)

            def ostep():
                binding.chunk_fwd(xo["q"], xo["k"], xo["v"], xo["beta"], xo["S0"], wo.C, o=oo, S_final=So,
                                  workspace=wso)

            # Short steps: enough warmup calls for about 20 ms of load.
            mso, _, _ = timed_steps(ostep, max(a.warmup, 200), a.steps)
            assert torch.isfinite(oo).all()
            fo = model_flops(wo)
            others.append({"workload": wo.name, "ms_per_step": mso, "tokens_per_s": wo.B * wo.L / (mso * 1e-3),
                           "model_tflops": fo / (mso * 1e-3) / 1e12,
                           "path_alg_gbs": chunk_bytes(wo, s0=wo.s0_std is not None) / (mso * 1e-3) / 1e9})
        result["other_workloads"] = others

    if not a.no_cpu_baseline:
        print("[bench] cpu baseline (oracle sample)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, x)

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
