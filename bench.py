"""Throughput of the attention forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle-s S] [--no-cpu-baseline] [--extra]

One step = one attn_fwd launch over the causal workload B=4, H=16, N=4096,
d=128 in bf16 (inputs already resident in HBM; two buffer sets alternate so
the 256 MB Infinity Cache cannot hold a step's whole working set). Before
the W warmup steps, untimed launches run for S seconds (default 0.75) so
that the GPU clock settles at its sustained value under this load; exactly K
steps are then timed. Prints
ONE JSON line with TFLOP/s (FLOPs counted as 4*B*H*N_q*N_k*d, halved for the
causal mask), the kernel's roofline position, and the CPU oracle timed on a
bounded sample of the same workload.

Other modes (for profiling): --copy-calibration runs one plain 256 MiB
device copy, whose FETCH_SIZE / WRITE_SIZE counters calibrate the HBM-byte
counters of the attention kernel.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s + % of MI355X bf16 MFMA peak, B4 H16 N4096 d128 causal"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
WORKLOAD = dict(workload="sdpa_bf16_b4_h16_n4096_d128_causal", B=4, H=16, N=4096, d=128, mask="causal",
                dtype="bf16", scale="1/sqrt(128)")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_causal_b4h16n4096d128_hbm_traffic.json")
KERNEL_SOURCES = ["transformer_scaled_dot_amd/csrc/attn_fwd_bf16.hip", "transformer_scaled_dot_amd/csrc/attn_qb2_tile.inc",
                  "transformer_scaled_dot_amd/csrc/device_common.h", "transformer_scaled_dot_amd/csrc/attn_tiles.h",
                  "transformer_scaled_dot_amd/csrc/attn_sched.h"]


def strip_comments(src: str) -> str:
    """C/C++ source without its comments, whitespace runs folded to one space: what the
    compiler sees, so that editing a comment does not count as changing the kernel."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            h.update(strip_comments(f.read()).encode())
    return h.hexdigest()[:16]


def attn_flops(B, H, Nq, Nk, d, causal):
    f = 4.0 * B * H * Nq * Nk * d
    return f / 2 if causal else f


def hbm_traffic_per_launch():
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when it is missing or was taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE, encoding="utf-8") as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def settle_clock(fn, seconds):
    """Untimed launches, back to back, until ``seconds`` of wall time have
    passed (checked at a device synchronisation every 64 launches): the GPU
    clock ramps up for a few hundred milliseconds under a sustained matrix
    load, so without this the first timed launches run at a lower clock.
    Returns (launches issued, wall seconds spent)."""
    import torch

    t0 = time.perf_counter()
    n = 0
    while True:
        for _ in range(64):
            fn(n)
            n += 1
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return n, time.perf_counter() - t0


def time_launches(fn, nsteps, warmup, per_launch=False):
    """Warm up, then time exactly nsteps launches between two device
    synchronisations with HIP events on the launching (current) stream.
    Returns (mean ms per launch, wall seconds, per-launch ms or None): with
    per_launch, an event between consecutive launches gives each launch's
    time as well (the mean is still first event to last)."""
    import torch

    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(nsteps + 1 if per_launch else 2)]
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(nsteps):
        fn(i)
        if per_launch:
            ev[i + 1].record()
    ev[-1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    each = [ev[i].elapsed_time(ev[i + 1]) for i in range(nsteps)] if per_launch else None
    return ev[0].elapsed_time(ev[-1]) / nsteps, wall, each


def time_graph(fn, nsets, replays, outs):
    """The launches fn(0) .. fn(nsets - 1) captured once into a HIP graph (torch.cuda.CUDAGraph) and replayed
    ``replays`` times between two synchronisations, timed with HIP events: for launches shorter than the host's
    cost of one call the eager loop of time_launches measures the host, the replay the GPU. The outputs of the
    last replay must equal those of the same launches run eagerly afterwards. Returns ms per launch."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(nsets):
            fn(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(nsets):
            fn(i)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (replays * nsets)
    got = [o.clone() for o in outs]
    for i in range(nsets):
        fn(i)
    torch.cuda.synchronize()
    if not all(torch.equal(x, y) for x, y in zip(got, outs)):
        raise RuntimeError("bench.py: a graph replay's output differs from the eager launch")
    del g
    return ms


def bench_attention(dev, cfg_id, nsteps, warmup, mask, sets=2, out_dtype=None, settle_s=0.0, graph=False):
    import torch

    import synth
    import transformer_scaled_dot_amd as tsd

    q, k, v, vl = synth.attn_inputs(cfg_id)
    B, H, N, d = q.shape
    bufs = []
    for s in range(sets):
        bufs.append((q.torch(dev), k.torch(dev), v.torch(dev),
                     torch.empty((B, H, N, d), dtype=out_dtype or torch.bfloat16, device=dev)))
    vl_t = torch.from_numpy(vl).to(dev) if vl is not None else None
    del q, k, v

    def step(i):
        qq, kk, vv, oo = bufs[i % sets]
        tsd.attn_fwd(qq, kk, vv, mask=mask, valid_lens=vl_t, out=oo, out_dtype=oo.dtype)

    settled = settle_clock(step, settle_s) if settle_s > 0 else (0, 0.0)
    ms, wall, _ = time_launches(step, nsteps, warmup)
    # a second pass with an event between launches for the per-launch spread (the events could add a
    # little between launches, so the mean above comes from a pass without them)
    _, _, each = time_launches(step, nsteps, 0, per_launch=True)
    ms_graph = time_graph(step, sets, max(1, nsteps // sets), [b[3] for b in bufs]) if graph else None
    if mask == "padding":
        flops = attn_flops(B, H, N, N, d, False)
    else:
        flops = attn_flops(B, H, N, N, d, mask == "causal")
    return dict(ms=ms, wall=wall, flops=flops, shape=(B, H, N, d), valid_lens=vl, each=each, settled=settled,
                ms_graph=ms_graph)


def bench_mha(dev, nsteps, warmup, sets=4, settle_s=0.0):
    import torch

    import synth
    import transformer_scaled_dot_amd as tsd

    x, wqkv, wo = synth.mha_inputs(4)
    B, N, dm = x.shape
    h = synth.CONFIGS[4]["h"]
    need = tsd.mha_workspace_bytes(B, N, dm, h)
    bufs = [(x.torch(dev), wqkv.torch(dev), wo.torch(dev), torch.empty((B, N, dm), dtype=torch.bfloat16, device=dev),
             torch.empty(need, dtype=torch.uint8, device=dev)) for _ in range(sets)]

    def step(i):
        xx, ww, wwo, oo, ws = bufs[i % sets]
        tsd.mha_fwd(xx, ww, wwo, h, out=oo, workspace=ws)

    if settle_s > 0:
        settle_clock(step, settle_s)
    ms, wall, _ = time_launches(step, nsteps, warmup)
    dk = dm // h
    flops = 8.0 * B * N * dm * dm + 4.0 * B * h * N * N * dk
    return dict(ms=ms, wall=wall, flops=flops)


def bench_grouped_lse(dev, nsteps, warmup, sets=2, settle_s=0.0):
    """The causal 4K workload with 4 K/V heads for its 16 query heads, the causal-and-padding mask (every
    valid length = N, so the work is the causal work) and the per-row log-sum-exp written out."""
    import torch

    import synth
    import transformer_scaled_dot_amd as tsd

    B, H, Hkv, N, d = 4, 16, 4, 4096, 128
    bufs = []
    for s in range(sets):
        q = synth.normal_tensor(9100 + 3 * s, (B, H, N, d)).torch(dev)
        k = synth.normal_tensor(9101 + 3 * s, (B, Hkv, N, d)).torch(dev)
        v = synth.normal_tensor(9102 + 3 * s, (B, Hkv, N, d)).torch(dev)
        bufs.append((q, k, v, torch.empty_like(q), torch.empty((B, H, N), dtype=torch.float32, device=dev)))
    vl = torch.full((B,), N, dtype=torch.int32, device=dev)

    def step(i):
        q, k, v, o, lse = bufs[i % sets]
        tsd.attn_fwd(q, k, v, mask="causal_padding", valid_lens=vl, out=o, lse=lse)

    if settle_s > 0:
        settle_clock(step, settle_s)
    ms, _, _ = time_launches(step, nsteps, warmup)
    return dict(ms=ms, flops=attn_flops(B, H, N, N, d, True))


def bench_backward(dev, nsteps, warmup, sets=2, settle_s=0.0):
    """The backward pass at the causal 4K shape (B4 H16 N4096 d128): dQ, dK, dV from the forward's O and
    log-sum-exp and a synthetic output gradient. FLOPs: the five N x N x d products of the chain rule
    (S recomputed, dP, dV, dK, dQ), halved for causal, i.e. 2.5 times the forward's."""
    import torch

    import synth
    import transformer_scaled_dot_amd as tsd

    B, H, N, d = 4, 16, 4096, 128
    bufs = []
    for s in range(sets):
        q, k, v, g = (synth.normal_tensor(9200 + 4 * s + i, (B, H, N, d)).torch(dev) for i in range(4))
        o, lse = tsd.attn_fwd(q, k, v, mask="causal", return_lse=True)
        ws = torch.empty(tsd.load_library().attn_bwd_workspace_bytes(B, H, N), dtype=torch.uint8, device=dev)
        bufs.append((q, k, v, g, o, lse, ws))

    def step(i):
        q, k, v, g, o, lse, ws = bufs[i % sets]
        tsd.attn_bwd(q, k, v, o, g, lse, mask="causal", workspace=ws)

    if settle_s > 0:
        settle_clock(step, settle_s)
    ms, _, _ = time_launches(step, nsteps, warmup)
    return dict(ms=ms, flops=2.5 * attn_flops(B, H, N, N, d, True))


def bench_one(dev, which, nsteps, warmup, settle_s, graph=False):
    """One of the other workloads, timed like the benchmark line (settle, warmup, timed steps). graph: the
    padding workload's launches are timed a second time, replayed from a HIP graph (used by --extra; a
    profiled --only run keeps only the eager launches)."""
    if which == "padding":
        # an 11 us launch is close to the host's cost of one call through the binding (under a profiler, above
        # it): the same launches are also timed replayed from a HIP graph ("ms_graph")
        r2 = bench_attention(dev, 2, nsteps, warmup, "padding", sets=16, settle_s=settle_s, graph=graph)
        B2, H2, N2, d2 = r2["shape"]
        L = r2["valid_lens"].astype(np.float64)
        alg_flops = 4.0 * H2 * d2 * N2 * L.sum()
        hbm = 2.0 * B2 * H2 * N2 * d2 * 2 + 2.0 * H2 * d2 * 2 * L.sum()  # Q, O + valid K, V rows
        ms = r2["ms"]
        res = {"ms": round(ms, 5), "tflops_metric": round(r2["flops"] / ms / 1e9, 2),
               "tflops_valid_keys": round(alg_flops / ms / 1e9, 2), "hbm_gbs_algorithmic": round(hbm / ms / 1e6, 1),
               "hbm_frac": round(hbm / ms / 1e6 / PEAK_HBM_GBS, 4), "algorithmic_bytes": int(hbm)}
        if graph:
            res["ms_graph"] = round(r2["ms_graph"], 5)
        return res
    if which == "mha":
        r4 = bench_mha(dev, nsteps, warmup, settle_s=settle_s)
        return {"ms": round(r4["ms"], 5), "tflops": round(r4["flops"] / r4["ms"] / 1e9, 2)}
    if which == "causal32k":
        r5 = bench_attention(dev, 5, max(5, nsteps // 20), 5, "causal", sets=1, settle_s=settle_s)
        return {"ms": round(r5["ms"], 4), "tflops": round(r5["flops"] / r5["ms"] / 1e9, 2)}
    if which == "backward":
        rb = bench_backward(dev, max(20, nsteps // 5), 20, settle_s=settle_s)
        return {"ms": round(rb["ms"], 4), "tflops": round(rb["flops"] / rb["ms"] / 1e9, 2)}
    raise ValueError(which)


def cpu_baseline(target_s=15.0):
    """The CPU oracle on whole heads of the benchmark workload (same seeded
    inputs), as many heads as fit in about target_s seconds."""
    import oracle
    import synth

    q, k, v, _ = synth.attn_inputs(3)
    B, H, N, d = q.shape
    qf, kf, vf = q.f32, k.f32, v.f32

    def run(heads):
        sel = [(i // H, i % H) for i in heads]
        Q = np.stack([qf[b, h] for b, h in sel])[None].astype(np.float64)
        K = np.stack([kf[b, h] for b, h in sel])[None].astype(np.float64)
        V = np.stack([vf[b, h] for b, h in sel])[None].astype(np.float64)
        t0 = time.perf_counter()
        oracle.attention(Q, K, V, mask="causal")
        return time.perf_counter() - t0

    t1 = run([0])
    nheads = int(max(1, min(B * H - 1, round(target_s / max(t1, 1e-3)) - 1)))
    t2 = run(list(range(1, 1 + nheads)))
    total_heads, total_t = 1 + nheads, t1 + t2
    flops = total_heads * attn_flops(1, 1, N, N, d, True)
    threads = oracle.max_threads()
    return {"value": flops / total_t / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "%d of the %d (batch, head) slices of the workload, all %d causal rows each, float64; %.1f s"
                      % (total_heads, B * H, N, total_t)}


def copy_calibration(dev, nbytes=256 << 20):
    import torch

    src = torch.ones(nbytes // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=20)
    # the GPU clock ramps up for a few hundred ms under this load and the figure of interest is the sustained
    # rate: untimed launches run for this long before the warmup steps (reported as "clock_settle")
    ap.add_argument("--settle-s", type=float, default=0.75)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--extra", action="store_true",
                    help="also time the padding, multi-head and 32K workloads, the grouped-heads/log-sum-exp "
                         "variant and the backward pass")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--only", choices=["padding", "mha", "causal32k", "backward"],
                    help="time only one other workload (for its kernel trace and counters): the padding workload "
                         "B8 H8 N512 d64, the multi-head layer B4 N2048 d_model 512 h8, the causal B1 H32 N32768 "
                         "d128 workload, or the backward pass at the causal 4K shape")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the benchmark runs on one GPU only; --gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py: no GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    import transformer_scaled_dot_amd as tsd

    tsd.load_library()
    if args.copy_calibration:
        copy_calibration(dev)
        return
    if args.only:
        print(json.dumps({args.only: bench_one(dev, args.only, args.steps, args.warmup, args.settle_s)}), flush=True)
        return

    r = bench_attention(dev, 3, args.steps, args.warmup, "causal", settle_s=args.settle_s)
    tflops = r["flops"] / (r["ms"] * 1e-3) / 1e12
    B, H, N, d = r["shape"]
    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) Q, K, V (SplitMix64 + Box-Muller, rounded to bf16)",
        "config": dict(WORKLOAD, parallelism="none (1 GPU)"),
        "pct_of_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "roofline": {
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": hbm_traffic_per_launch(),
            "traffic_unit": "bytes per launch between L2 and memory (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled by a "
                            "256 MiB copy's counts)",
            "algorithmic_bytes_per_launch": 4 * B * H * N * d * 2,
            "kernel": "attn_fwd_qb2_kernel<causal, bf16 out>",
            "algorithmic_flops_per_launch": r["flops"],
            "avg_launch_ms": round(r["ms"], 5),
            "launch_ms_median": round(float(np.median(r["each"])), 5),
            "launch_ms_min": round(float(np.min(r["each"])), 5),
        },
        "wall_s_timed_region": round(r["wall"], 4),
        "clock_settle": {"seconds": round(r["settled"][1], 3), "launches": r["settled"][0],
                         "note": "untimed launches of the same step before the warmup steps, so that the timed "
                                 "steps run at the clock the GPU sustains under this load"},
    }
    # right after the timed launches: every SIMD issuing only bf16 MFMAs on pseudo-random operands. Its clock
    # and rate are the practical matrix ceiling of this chip (the power limit holds the clock well under the
    # 2.4 GHz the published peak assumes); the roofline's peak stays the published one.
    from transformer_scaled_dot_amd.probe import clock_probe

    probe = clock_probe(dev)
    out["sclk_mhz_after"] = round(probe["clock_mhz"], 0)
    out["mfma_only_probe"] = {"tflops": round(probe["tflops"], 1), "clock_mhz": round(probe["clock_mhz"], 0),
                               "operands": "pseudo-random bf16, uniform in [-2, 2)",
                               "value_over_probe": round(tflops / probe["tflops"], 4)}
    if args.extra:
        extra = {}
        extra["C2_padding_b8h8n512d64"] = bench_one(dev, "padding", args.steps, args.warmup, 0.2, graph=True)
        extra["C4_mha_b4n2048dm512h8"] = bench_one(dev, "mha", args.steps, args.warmup, 0.2)
        extra["C5_causal_b1h32n32768d128"] = bench_one(dev, "causal32k", args.steps, args.warmup, 0.3)
        rg = bench_grouped_lse(dev, args.steps, args.warmup, settle_s=0.3)
        extra["C3_gqa_h16_kv4_causal_padding_lse"] = {"ms": round(rg["ms"], 5),
                                                     "tflops": round(rg["flops"] / rg["ms"] / 1e9, 2)}
        # the fp32 accuracy path at its tiny shape [2,1,5,16]: launch-latency bound, reported in microseconds
        r1 = bench_attention(dev, 1, args.steps, 100, "none", out_dtype=torch.float32, sets=16, graph=True)
        extra["C1_f32_b2h1n5d16"] = {"us_per_launch": round(r1["ms"] * 1e3, 2),
                                     "us_median": round(float(np.median(r1["each"])) * 1e3, 2),
                                     "us_per_launch_graph": round(r1["ms_graph"] * 1e3, 2)}
        extra["C3_backward_causal_b4h16n4096d128"] = bench_one(dev, "backward", args.steps, args.warmup, 0.3)
        out["extra"] = extra
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
