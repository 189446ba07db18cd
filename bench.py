#!/usr/bin/env python3
"""Throughput of the RankMixer block forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c3]

A step is one rm_model_fwd over one batch of the ~1B-class dense workload
(B=1024, T=32 tokens, D=1536, hidden 6144, L=2 blocks, bf16): token mix +
residual + LayerNorm, the two grouped per-token FFN products, residual +
LayerNorm, for both blocks, with inputs and weights resident in HBM.  The
reported value is samples through one block per second (B * L / step time).

Prints ONE JSON line.  Besides the contract fields it carries
  roofline      the dominant kernel (by summed time over the profiled pass,
                which carries HIP events around every launch group), its
                algorithmic TFLOP/s from HIP events recorded around each of its
                launches during the timed region (the only events there, so
                the step time carries no other event overhead), against the
                bf16 dense MFMA peak; traffic from the committed rocprofv3
                counter summary if it was taken on the current kernel source,
                else null
  kernels       every launch group's average over a pass of PROFILE_STEPS
                steps between the warm-up and the timed steps
  cpu_baseline  the fp64 oracle on a bounded sample of the same workload,
                timed on this host's cores (rank 0, N=1 only)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "samples/sec RankMixer block fwd (bf16) + % of MI355X MFMA peak"
PROFILE_STEPS = 5  # untimed steps with events around every launch group


def log(msg: str) -> None:
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


CSRC = os.path.join(ROOT, "rankmixer_token_mixing_amd", "csrc")
# the sources that define each launch group's kernel
KERNEL_SOURCES = {
    "ffn1": ("kernels_gemm.hip", "frag.hpp", "common.hpp"),
    "ffn2": ("kernels_gemm.hip", "frag.hpp", "common.hpp"),
    "mix_ln1": ("kernels_rows.hip", "common.hpp"),
    "ln2": ("kernels_rows.hip", "common.hpp"),
    "ln2_mix_ln1": ("kernels_rows.hip", "common.hpp"),
    "tokenize_proj": ("kernels_tokproj.hip", "frag.hpp", "common.hpp"),
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "block_fwd_{config}_traffic.json")
PROJ_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "tokenize_project_traffic.json")


def source_sha(name: str) -> str:
    with open(os.path.join(CSRC, name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def committed_traffic(config: str, kernel: str, path: str = ""):
    """HBM bytes per launch of `kernel` from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary of this workload, or None when there is
    none or the kernel's sources changed since the counters were taken."""
    path = path or TRAFFIC_FILE.format(config=config)
    if not os.path.exists(path) or kernel not in KERNEL_SOURCES:
        return None
    with open(path) as f:
        tr = json.load(f)
    k = tr.get("kernels", {}).get(kernel)
    if not k:
        return None
    taken = k.get("source_sha", {})
    if any(taken.get(src) != source_sha(src) for src in KERNEL_SOURCES[kernel]):
        return None
    return k.get("hbm_bytes_per_launch")


def block0_protocol(bd, blocks, x0, B: int, flop_block, peak: float) -> dict:
    """One rm_block_fwd on block 0 of the workload: 10 warm-up calls, then 3
    groups of 30 timed calls (events on the launching stream), the median of
    the three group means."""
    import statistics
    import torch
    y = torch.empty_like(x0)
    for _ in range(10):
        bd.rm_block_fwd(x0, blocks[0], out=y)
    means = []
    for _ in range(3):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(30):
            bd.rm_block_fwd(x0, blocks[0], out=y)
        e1.record()
        e1.synchronize()
        means.append(e0.elapsed_time(e1) / 30)
    ms = statistics.median(means)
    rec = {"ms": round(ms, 4), "samples_per_s": round(B / (ms * 1e-3), 1),
           "group_means_ms": [round(m, 4) for m in means],
           "protocol": "rm_block_fwd on block 0: 10 warm-up calls, 3 groups of 30 timed calls, median of group means"}
    if flop_block:
        tf = flop_block / (ms * 1e-3) / 1e12
        rec["tflops"] = round(tf, 1)
        rec["frac_of_bf16_peak"] = round(tf / peak, 4)
    return rec


def measure_ceilings(bd, copy_mib: int = 100, pairs: int = 6) -> dict:
    """The chip's own ceilings, from the library's probes (tracked source):
    the bf16 MFMA loop on random operands (TFLOP/s over 10 launches of ~2 ms
    after 3 warm-up launches), and a copy of copy_mib MiB timed cold (each copy
    reads and writes buffers that the copies of the other `pairs` - 1 buffer
    pairs have pushed out of the 256 MB last-level cache) and warm (the same
    pair again and again); GB/s count bytes read + bytes written."""
    import statistics
    import torch
    lib = bd.load()
    frags = torch.randn(lib.rm_probe_mfma_frag_bytes() // 2, device="cuda").to(torch.bfloat16)
    out = torch.empty(lib.rm_probe_mfma_out_floats(), dtype=torch.float32, device="cuda")
    iters = 600
    for _ in range(3):
        bd.probe_mfma_bf16(frags, out, iters)
    ms = []
    for _ in range(10):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        bd.probe_mfma_bf16(frags, out, iters)
        e1.record()
        e1.synchronize()
        ms.append(e0.elapsed_time(e1))
    mfma = lib.rm_probe_mfma_flop(iters) / (statistics.median(ms) * 1e-3) / 1e12

    def timed_median(fn, reps=10, warm=3):
        for _ in range(warm):
            fn()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        return statistics.median(ts)

    # the same MFMA loop on constant operands (every fragment 1.0): the
    # multipliers' inputs never change, so this is the loop without the
    # data-dependent switching energy of random operands
    ones = torch.ones_like(frags)
    mfma_const = lib.rm_probe_mfma_flop(iters) / (timed_median(lambda: bd.probe_mfma_bf16(ones, out, iters)) * 1e-3) / 1e12
    del ones
    # the products' k-step (MFMAs fed by its LDS fragment reads) on random bf16
    slab = torch.randn(lib.rm_probe_kstep_slab_bytes() // 2, device="cuda").to(torch.bfloat16)
    kout = torch.empty(lib.rm_probe_kstep_out_floats(), dtype=torch.float32, device="cuda")
    kiters = 2000
    kstep = lib.rm_probe_kstep_flop(kiters) / (timed_median(lambda: bd.probe_kstep_bf16(slab, kout, kiters)) * 1e-3) / 1e12
    del slab, kout
    n = copy_mib << 20
    bufs = [(torch.empty(n, dtype=torch.uint8, device="cuda"), torch.empty(n, dtype=torch.uint8, device="cuda"))
            for _ in range(pairs)]
    for a, b in bufs:
        a.fill_(1)
        b.fill_(2)

    def timed_copy(a, b):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        bd.probe_copy(a, b, n)
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1)

    cold = [timed_copy(*bufs[i % pairs]) for i in range(2 * pairs)][pairs:]
    warm = [timed_copy(*bufs[0]) for _ in range(10)][2:]
    del bufs
    return {"mfma_bf16_random_tflops": round(mfma, 1),
            "mfma_bf16_constant_tflops": round(mfma_const, 1),
            "kstep_bf16_random_tflops": round(kstep, 1),
            "copy_cold_gbs": round(2 * n / (statistics.median(cold) * 1e-3) / 1e9, 1),
            "copy_warm_gbs": round(2 * n / (statistics.median(warm) * 1e-3) / 1e9, 1),
            "copy_bytes": 2 * n,
            "how": "librankmixer probes: rm_probe_mfma_bf16 (8 waves per CU of v_mfma_f32_32x32x16_bf16 on "
                   "random bf16 fragments, and on constant ones; median of 10 launches), rm_probe_kstep_bf16 (the "
                   "products' k-step: 8 MFMAs + 6 LDS fragment reads per wave, 8 waves per CU, random bf16 in LDS, "
                   "no DMA or barriers) and rm_probe_copy (median per copy, cold: "
                   f"round-robin over {pairs} buffer pairs)"}


def with_ceiling(roofline, ceil: dict):
    """The roofline object with the measured ceiling of its bound beside the
    data-sheet peak."""
    if roofline is None or not ceil:
        return roofline
    c = ceil["mfma_bf16_random_tflops"] if roofline["bound"] == "mfma" else ceil["copy_cold_gbs"]
    roofline["measured_ceiling"] = c
    roofline["frac_of_measured_ceiling"] = round(roofline["achieved"] / c, 4)
    return roofline


def bench_ceilings(args) -> int:
    import torch
    from rankmixer_token_mixing_amd import binding as bd
    from rankmixer_token_mixing_amd import perfmodel as pm
    c = measure_ceilings(bd)
    rec = {"metric": "MI355X ceilings measured by the library's probes", "value": c["mfma_bf16_random_tflops"],
           "unit": "TFLOP/s", "n_gpus": 1, "higher_is_better": True, "data": "synthetic (random bf16)",
           "dtype": "bf16", "config": {"workload": "MFMA loop and HBM copy probes"},
           "mfma_frac_of_spec": round(c["mfma_bf16_random_tflops"] / pm.PEAK_BF16_TFLOPS, 4),
           "mfma_constant_frac_of_spec": round(c["mfma_bf16_constant_tflops"] / pm.PEAK_BF16_TFLOPS, 4),
           "kstep_frac_of_spec": round(c["kstep_bf16_random_tflops"] / pm.PEAK_BF16_TFLOPS, 4),
           "copy_cold_frac_of_spec": round(c["copy_cold_gbs"] / pm.PEAK_HBM_GBS, 4),
           "copy_warm_frac_of_spec": round(c["copy_warm_gbs"] / pm.PEAK_HBM_GBS, 4), **c}
    print(json.dumps(rec), flush=True)
    return 0


def moe_active_rows(bd, blocks, x0, D: int) -> list:
    """Active (sample, token, expert) rows of each MoE block on this batch, for
    the flop count: block l's input comes from the library's own blocks, its S
    = LN1(TM(X) + X) from the library's token mix and torch's fp32 LayerNorm
    (bookkeeping only; a gate within rounding of zero may be counted on the
    other side), and the count from the library's router and compaction."""
    import torch
    x = x0
    counts = []
    for blk in blocks:
        y1 = bd.rm_token_mix(x).float() + x.float()
        s = torch.nn.functional.layer_norm(y1, (D,), blk["ln1_g"], blk["ln1_b"], eps=1e-5).to(x.dtype)
        _, offsets, _ = bd.rm_moe_route(s, blk["wr"], blk["br"])
        counts.append(int(offsets[-1].item()))
        x = bd.rm_block_fwd(x, blk)
    return counts


def cpu_baseline(inputs, L: int, n_rows: int) -> dict:
    import numpy as np
    from oracle import rankmixer_oracle as orc
    import synthetic_inputs as si
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    cfg = inputs["config"]
    rows = si.random_rows(cfg.B, n_rows, seed=99)
    t0 = time.perf_counter()
    orc.run_config(inputs, rows)
    dt = time.perf_counter() - t0
    return {
        "value": len(rows) * L / dt,
        "unit": "samples/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{len(rows)} of {cfg.B} samples through all {L} blocks (fp64 numpy, "
                  f"{dt:.1f} s); samples are independent, so the rate is per-sample exact",
    }


def bench_project(args) -> int:
    """The projection tokenizer alone: one rm_tokenize_project per step over
    the pad-split model's embedding batch (B=4096 x 5000 fp32 -> 16 segments
    of 320 -> [4096, 16, 320] bf16).  HBM-bound: the roofline is the
    compulsory bytes (embedding, weights, output) over the launch time."""
    import numpy as np
    import torch
    import synthetic_inputs as si
    from rankmixer_token_mixing_amd import binding as bd
    from rankmixer_token_mixing_amd import perfmodel as pm

    w = si.PROJ_WORKLOAD
    B, F, T, seg, D = w["B"], w["F"], w["T"], w["seg"], w["D"]
    t0 = time.perf_counter()
    inp = si.make_proj_inputs(B, F, T, seg, D, w["dtype"])
    log(f"generated projection-tokenizer inputs in {time.perf_counter() - t0:.1f}s")
    emb = bd.to_device(inp["emb"])
    p = {"w": bd.to_device(inp["w"]), "b": bd.to_device(inp["b"])}
    out = torch.empty((B, T, D), dtype=torch.bfloat16, device="cuda")

    def step():
        bd.rm_tokenize_project(emb, p, T, seg, out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # one launch per step on torch's current stream: a HIP event pair around
    # the timed launches on that stream gives the mean launch duration (a pair
    # around every launch would add its own overhead to a ~30 us kernel)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / args.steps
    nbytes = pm.project_bytes(B, F, T, seg, D, "bf16")
    ev_ms = e0.elapsed_time(e1)
    kernels = {"tokenize_proj": {"avg_ms": round(ev_ms / args.steps, 5), "launches": args.steps,
                                 "total_ms": round(ev_ms, 3)}}
    roofline = None
    if not args.no_profile:
        avg_s = kernels["tokenize_proj"]["avg_ms"] * 1e-3
        ach = nbytes / avg_s / 1e9
        roofline = {"bound": "hbm", "kernel": "tokenize_proj", "achieved": round(ach, 1),
                    "peak": pm.PEAK_HBM_GBS, "unit": "GB/s", "frac": round(ach / pm.PEAK_HBM_GBS, 4),
                    "bytes_per_launch": nbytes,
                    "traffic": committed_traffic("", "tokenize_proj", PROJ_TRAFFIC_FILE)}
        kernels["tokenize_proj"]["tflops"] = round(pm.project_flops(B, T, seg, D) / avg_s / 1e12, 1)
    rec = {
        "metric": "samples/sec projection tokenizer (bf16) + % of MI355X HBM roofline",
        "value": round(B / (ms_step * 1e-3), 1),
        "unit": "samples/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"projection tokenizer: B={B} embeddings of F={F} fp32 floats -> "
                               f"T={T} segments of {seg} -> D={D} each, bf16",
                   "B": B, "F": F, "T": T, "seg": seg, "D": D,
                   "step": "rm_tokenize_project over the batch"},
        "roofline": roofline,
        "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        from oracle import rankmixer_oracle as orc
        # the oracle does the whole batch in about a second: no sampling needed
        t0 = time.perf_counter()
        orc.tokenize_project(inp["emb"], inp["w"], inp["b"], T, seg, "bf16")
        dt = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": B / dt, "unit": "samples/s", "cores": 1, "kind": "oracle",
                               "sample": f"the whole batch of {B} samples (fp64 numpy einsum, one thread, {dt:.1f} s)"}
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)
    return 0


def bench_block_bwd(args) -> int:
    """The dense block backward alone: one rm_block_bwd per step on block 0 of
    the workload (default c3: B=1024, T=32, D=1536, hidden 6144, bf16), given
    the saved tensors of one rm_block_fwd_train and a seeded N(0, 1) upstream
    gradient.  Four grouped products of 2*B*D*Hd*T flops each (dH, dW2, dW1,
    dS); the roofline is the dominant one against the bf16 MFMA peak."""
    import numpy as np
    import torch
    import synthetic_inputs as si
    from rankmixer_token_mixing_amd import binding as bd
    from rankmixer_token_mixing_amd import perfmodel as pm

    cfg = si.CONFIGS[args.config]
    if cfg.E:
        print("block_bwd: dense workloads only", file=sys.stderr)
        return 2
    t0 = time.perf_counter()
    inputs = si.make_inputs(si.scaled(cfg, L=1))
    d_out_np = si.make_inputs(si.scaled(cfg, L=0), seed=100 + si.SEEDS[cfg.name])["x"]
    log(f"generated {cfg.name} inputs in {time.perf_counter() - t0:.1f}s: {cfg.description}")
    blk = bd.upload_blocks(inputs["blocks"][:1])[0]
    x = bd.to_device(inputs["x"])
    d_out = bd.to_device(d_out_np)
    B, T, D, Hd = cfg.B, cfg.T, cfg.D, cfg.hidden
    _, saved = bd.rm_block_fwd_train(x, blk)

    for _ in range(args.warmup):
        bd.rm_block_bwd(x, blk, saved, d_out)
    torch.cuda.synchronize()
    bd.profile_enable(not args.no_profile)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        bd.rm_block_bwd(x, blk, saved, d_out)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    prof = bd.profile_read() if not args.no_profile else {}
    bd.profile_enable(False)
    ms_step = elapsed * 1e3 / args.steps
    gemm = T * pm.gemm_flops(B, Hd, D)  # each of the four products
    kernels = {}
    for name, (tot_ms, n) in prof.items():
        avg = tot_ms / max(n, 1)
        e = {"avg_ms": round(avg, 5), "launches": n, "total_ms": round(tot_ms, 3)}
        if name.startswith("bwd_d"):
            e["tflops"] = round(gemm / (avg * 1e-3) / 1e12, 1)
        kernels[name] = e
    roofline = None
    gk = {k: v for k, v in kernels.items() if k.startswith("bwd_d")}
    if gk:
        dom = max(gk, key=lambda k: gk[k]["total_ms"])
        ach = gemm / (gk[dom]["avg_ms"] * 1e-3) / 1e12
        roofline = {"bound": "mfma", "kernel": dom, "achieved": round(ach, 1), "peak": pm.PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(ach / pm.PEAK_BF16_TFLOPS, 4), "flop_per_launch": gemm,
                    "traffic": None}
    bwd_tf = 4 * gemm / (ms_step * 1e-3) / 1e12
    rec = {
        "metric": "samples/sec RankMixer block backward (bf16) + % of MI355X MFMA peak",
        "value": round(B / (ms_step * 1e-3), 1),
        "unit": "samples/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": f"{cfg.description}: backward of block 0", "B": B, "T": T, "D": D, "hidden": Hd,
                   "step": "rm_block_bwd over the batch (dX and every parameter gradient)"},
        "roofline": roofline,
        "step_tflops": round(bwd_tf, 1),
        "step_frac_of_bf16_peak": round(bwd_tf / pm.PEAK_BF16_TFLOPS, 4),
        "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        from oracle import block_backward as obw
        n = min(B, 128)
        rows = si.random_rows(B, n, seed=99)
        t0 = time.perf_counter()
        obw.block_bwd(inputs["x"][rows], inputs["blocks"][0], d_out_np[rows])
        dt = time.perf_counter() - t0
        try:
            from threadpoolctl import threadpool_info
            threads = max([q.get("num_threads", 1) for q in threadpool_info() if q.get("user_api") == "blas"] or [1])
        except Exception:  # pragma: no cover
            threads = os.cpu_count() or 1
        rec["cpu_baseline"] = {"value": n / dt, "unit": "samples/s", "cores": int(threads), "kind": "oracle",
                               "sample": f"{n} of {B} samples (fp64 numpy forward + backward of block 0, {dt:.1f} s); "
                                         f"the work is linear in the samples, so the rate is per-sample exact"}
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)
    return 0


def bench_moe_train(args) -> int:
    """Training of the ReLU-routed MoE block with the dense-training /
    sparse-inference routers on block 0 of the MoE workload (c4: B=2048, T=16,
    D=768, 8 experts of 768 -> 1536 -> 768 per token, bf16), the inference
    router at about 25 % active gates and the training router at about 75 %.
    A step is rm_moe_block_fwd_train + rm_moe_block_bwd (lambda = 0.01) on one
    batch.  Every expert runs on every token in training, so the six expert
    products (W1, W2 forward; dH, dW2, dW1, dS backward) are 2*B*D*He*T*E
    flops each; the roofline is the dominant one against the bf16 MFMA peak."""
    import torch
    import synthetic_inputs as si
    from rankmixer_token_mixing_amd import binding as bd
    from rankmixer_token_mixing_amd import perfmodel as pm

    cfg = si.CONFIGS["c4"]
    t0 = time.perf_counter()
    inputs = si.make_inputs(si.scaled(cfg, L=1))
    blk_np = si.add_training_router(inputs["blocks"][0], cfg.dtype)
    d_out_np = si.make_inputs(si.scaled(cfg, L=0), seed=100 + si.SEEDS[cfg.name])["x"]
    log(f"generated {cfg.name} inputs in {time.perf_counter() - t0:.1f}s: {cfg.description}, training router added")
    blk = bd.upload_blocks([blk_np])[0]
    x = bd.to_device(inputs["x"])
    d_out = bd.to_device(d_out_np)
    B, T, D, E, He = cfg.B, cfg.T, cfg.D, cfg.E, cfg.He
    lam = 0.01

    def step():
        _, _, saved = bd.rm_moe_block_fwd_train(x, blk)
        bd.rm_moe_block_bwd(x, blk, saved, d_out, lam)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    bd.profile_enable(not args.no_profile)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    prof = bd.profile_read() if not args.no_profile else {}
    bd.profile_enable(False)
    ms_step = elapsed * 1e3 / args.steps
    gemm = T * E * pm.gemm_flops(B, He, D)  # each of the six expert products
    products = ("moe_ffn1", "moe_ffn2", "bwd_dH", "bwd_dW2", "bwd_dW1", "bwd_dS")
    kernels = {}
    for name, (tot_ms, n) in prof.items():
        avg = tot_ms / max(n, 1)
        e = {"avg_ms": round(avg, 5), "launches": n, "total_ms": round(tot_ms, 3)}
        if name in products:
            e["tflops"] = round(gemm / (avg * 1e-3) / 1e12, 1)
        kernels[name] = e
    roofline = None
    gk = {k: v for k, v in kernels.items() if k in products}
    if gk:
        dom = max(gk, key=lambda k: gk[k]["total_ms"])
        ach = gemm / (gk[dom]["avg_ms"] * 1e-3) / 1e12
        roofline = {"bound": "mfma", "kernel": dom, "achieved": round(ach, 1), "peak": pm.PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(ach / pm.PEAK_BF16_TFLOPS, 4), "flop_per_launch": gemm,
                    "traffic": None}
    step_tf = 6 * gemm / (ms_step * 1e-3) / 1e12
    rec = {
        "metric": "samples/sec RankMixer MoE block training step (bf16) + % of MI355X MFMA peak",
        "value": round(B / (ms_step * 1e-3), 1),
        "unit": "samples/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": f"{cfg.description}: training of block 0 with a dense training router",
                   "B": B, "T": T, "D": D, "E": E, "He": He, "lambda": lam,
                   "step": "rm_moe_block_fwd_train + rm_moe_block_bwd over the batch"},
        "roofline": roofline,
        "step_tflops": round(step_tf, 1),
        "step_frac_of_bf16_peak": round(step_tf / pm.PEAK_BF16_TFLOPS, 4),
        "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        from oracle import moe_training as omt
        n = min(B, 512)
        rows = si.random_rows(B, n, seed=99)
        t0 = time.perf_counter()
        omt.dtsi_bwd(inputs["x"][rows], blk_np, d_out_np[rows], lam)
        dt = time.perf_counter() - t0
        try:
            from threadpoolctl import threadpool_info
            threads = max([q.get("num_threads", 1) for q in threadpool_info() if q.get("user_api") == "blas"] or [1])
        except Exception:  # pragma: no cover
            threads = os.cpu_count() or 1
        rec["cpu_baseline"] = {"value": n / dt, "unit": "samples/s", "cores": int(threads), "kind": "oracle",
                               "sample": f"{n} of {B} samples (fp64 numpy training forward + backward of block 0, "
                                         f"{dt:.1f} s); the work is linear in the samples, so the rate is "
                                         f"per-sample exact"}
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)
    return 0


def bench_variants(args) -> int:
    """The block variants of the Taobao report on the 100M-class width (B=2048,
    T=16, D=768, bf16): the SwiGLU block D -> 4/3 D (hidden 1024) is the timed
    step; the GELU FFN block D -> 2D (hidden 1536, the same parameters and
    flops per token) and both without the Add & Norm after the mix are timed
    beside it the same way (one rm_block_fwd per step)."""
    import torch
    import synthetic_inputs as si
    from rankmixer_token_mixing_amd import binding as bd
    from rankmixer_token_mixing_amd import perfmodel as pm

    B, T, D = 2048, 16, 768
    Hs, Hd = 4 * D // 3, 2 * D
    x = bd.to_device(si.make_inputs(si.Config("variants", B=B, T=T, D=D, L=0, dtype="bf16"), seed=1)["x"])
    cases = {
        "swiglu_4_3": si.make_variant_block(T, D, Hs, "bf16", swiglu=True, seed=2),
        "gelu_2": si.make_variant_block(T, D, Hd, "bf16", seed=3),
        "swiglu_4_3_no_mix_norm": si.make_variant_block(T, D, Hs, "bf16", swiglu=True, no_mix_norm=True, seed=2),
        "gelu_2_no_mix_norm": si.make_variant_block(T, D, Hd, "bf16", no_mix_norm=True, seed=3),
    }
    flops = 6 * B * T * D * Hs  # = 4 * B * T * D * Hd for Hd = 2D: the same for every case
    res = {}
    main_prof = {}
    for name, host_blk in cases.items():
        blk = bd.upload_blocks([host_blk])[0]
        y = torch.empty_like(x)
        for _ in range(args.warmup):
            bd.rm_block_fwd(x, blk, out=y)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            bd.rm_block_fwd(x, blk, out=y)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        if name == "swiglu_4_3" and not args.no_profile:
            # per-launch HIP events in a separate pass (their own overhead stays
            # out of the timed steps)
            bd.profile_enable(True)
            for _ in range(args.steps):
                bd.rm_block_fwd(x, blk, out=y)
            torch.cuda.synchronize()
            main_prof = bd.profile_read()
            bd.profile_enable(False)
        ms = el * 1e3 / args.steps
        res[name] = {"ms": round(ms, 4), "samples_per_s": round(B / (ms * 1e-3), 1),
                     "tflops": round(flops / (ms * 1e-3) / 1e12, 1)}
        log(f"{name}: {ms:.4f} ms")
    kernels = {}
    for nm, (tot_ms, n) in main_prof.items():
        kernels[nm] = {"avg_ms": round(tot_ms / max(n, 1), 5), "launches": n, "total_ms": round(tot_ms, 3)}
    roofline = None
    if "ffn1" in kernels:
        f1 = T * pm.gemm_flops(B, 2 * Hs, D)
        ach = f1 / (kernels["ffn1"]["avg_ms"] * 1e-3) / 1e12
        roofline = {"bound": "mfma", "kernel": "ffn1 (gate | up product)", "achieved": round(ach, 1),
                    "peak": pm.PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(ach / pm.PEAK_BF16_TFLOPS, 4),
                    "flop_per_launch": f1, "traffic": None}
    main = res["swiglu_4_3"]
    rec = {
        "metric": "samples/sec RankMixer SwiGLU block fwd (bf16) + % of MI355X MFMA peak",
        "value": main["samples_per_s"],
        "unit": "samples/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"SwiGLU block D -> 4/3 D: B={B}, T={T}, D={D}, hidden {Hs}, bf16",
                   "B": B, "T": T, "D": D, "hidden": Hs, "step": "rm_block_fwd over the batch"},
        "roofline": roofline,
        "kernels": kernels,
        "variants": res,
    }
    if not args.no_cpu_baseline:
        from oracle import rankmixer_oracle as orc
        xh = si.make_inputs(si.Config("variants", B=B, T=T, D=D, L=0, dtype="bf16"), seed=1)["x"]
        rows = si.random_rows(B, 256, seed=99)
        t0 = time.perf_counter()
        orc.block_fwd(xh[rows], cases["swiglu_4_3"])
        dt = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": len(rows) / dt, "unit": "samples/s", "cores": os.cpu_count() or 1,
                               "kind": "oracle",
                               "sample": f"{len(rows)} of {B} samples through the SwiGLU block (fp64 numpy, {dt:.1f} s)"}
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)
    return 0


def bench_epilogue_overlap(args) -> int:
    """The two epilogue modes of the bf16 products (rm_set_epilogue_overlap)
    on the per-token FFN of block 0 of the ~1B-class workload (B=1024, T=32,
    D=1536, hidden 6144): rm_pffn_fwd with the epilogue after each tile (0,
    the default) and inside the next tile's main loop (1), alternated over
    several rounds so box drift hits both; per-launch HIP events give the W1
    product (bias + GELU) and the W2 product (bias) apart."""
    import torch
    import synthetic_inputs as si
    from rankmixer_token_mixing_amd import binding as bd
    from rankmixer_token_mixing_amd import perfmodel as pm

    cfg = si.CONFIGS["c3"]
    B, T, D = cfg.B, cfg.T, cfg.D
    Hd = cfg.hidden
    blk = bd.upload_blocks([si.make_inputs(si.scaled(cfg, L=1))["blocks"][0]])[0]
    p = {k: blk[k] for k in ("w1", "b1", "w2", "b2")}
    g = torch.Generator(device="cuda").manual_seed(5)
    s = torch.randn(B, T, D, device="cuda", generator=g).to(torch.bfloat16)  # LayerNorm-scaled operand
    out = torch.empty_like(s)
    flop = {"ffn1": T * pm.gemm_flops(B, Hd, D), "ffn2": T * pm.gemm_flops(B, D, Hd)}
    acc = {m: {"ffn1": [0.0, 0], "ffn2": [0.0, 0]} for m in (0, 1)}
    rounds = 4
    for r in range(rounds):
        for mode in (0, 1):
            bd.set_epilogue_overlap(bool(mode))
            for _ in range(args.warmup):
                bd.rm_pffn_fwd(s, p, out=out)
            torch.cuda.synchronize()
            bd.profile_enable(True)
            for _ in range(args.steps):
                bd.rm_pffn_fwd(s, p, out=out)
            torch.cuda.synchronize()
            prof = bd.profile_read()
            bd.profile_enable(False)
            for k in ("ffn1", "ffn2"):
                acc[mode][k][0] += prof[k][0]
                acc[mode][k][1] += prof[k][1]
        log(f"round {r + 1}/{rounds} done")
    bd.set_epilogue_overlap(False)
    res = {}
    for mode, name in ((0, "after_tile"), (1, "overlapped")):
        res[name] = {}
        for k in ("ffn1", "ffn2"):
            ms = acc[mode][k][0] / acc[mode][k][1]
            tf = flop[k] / (ms * 1e-3) / 1e12
            res[name][k] = {"avg_ms": round(ms, 5), "launches": acc[mode][k][1], "tflops": round(tf, 1),
                            "frac": round(tf / pm.PEAK_BF16_TFLOPS, 4)}
    base = res["after_tile"]["ffn1"]
    rec = {
        "metric": "W1 product TFLOP/s (bias + GELU epilogue), per-token FFN of block 0, bf16",
        "value": base["tflops"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(base["avg_ms"], 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"rm_pffn_fwd B={B}, T={T}, D={D}, hidden {Hd}, bf16, both epilogue modes",
                   "B": B, "T": T, "D": D, "hidden": Hd, "rounds": rounds},
        "modes": res,
        "overlapped_over_after_tile": {k: round(res["after_tile"][k]["avg_ms"] / res["overlapped"][k]["avg_ms"], 4)
                                       for k in ("ffn1", "ffn2")},
        "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)
    return 0


def bench_vendor_gemm(args) -> int:
    """The vendor library on the per-token FFN products of the ~1B-class
    workload's block (B=1024, T=32, D=1536, hidden 6144): torch.bmm (which
    calls hipBLASLt) on random bf16 operands of the W1 and W2 product shapes,
    both operands contiguous, no bias and no epilogue -- a reference point
    for the library's own fused products, not part of the method."""
    import torch
    from rankmixer_token_mixing_amd import perfmodel as pm

    B, T, D, Hd = 1024, 32, 1536, 6144
    g = torch.Generator(device="cuda").manual_seed(3)
    shapes = {"ffn1": (T, B, D, Hd), "ffn2": (T, B, Hd, D)}
    res = {}
    for name, (G, M, K, N) in shapes.items():
        a = torch.randn(G, M, K, device="cuda", generator=g).to(torch.bfloat16)
        w = torch.randn(G, K, N, device="cuda", generator=g).to(torch.bfloat16).contiguous()
        c = torch.empty(G, M, N, device="cuda", dtype=torch.bfloat16)
        for _ in range(args.warmup):
            torch.bmm(a, w, out=c)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            torch.bmm(a, w, out=c)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        fl = G * pm.gemm_flops(M, N, K)
        res[name] = {"avg_ms": round(ms, 5), "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
                     "frac": round(fl / (ms * 1e-3) / 1e12 / pm.PEAK_BF16_TFLOPS, 4)}
        log(f"{name}: {ms:.4f} ms")
        del a, w, c
    rec = {"metric": "vendor bf16 batched GEMM TFLOP/s on the W1 product shape (torch.bmm)",
           "value": res["ffn1"]["tflops"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": res["ffn1"]["avg_ms"], "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": f"torch.bmm [T,B,D]x[T,D,H] and [T,B,H]x[T,H,D], B={B}, T={T}, D={D}, "
                                  f"H={Hd}, bf16, no epilogue", "B": B, "T": T, "D": D, "hidden": Hd},
           "products": res, "cpu_baseline": None}
    print(json.dumps(rec), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="c3", help="workload (c3 is the benchmarked one)")
    ap.add_argument("--op", default="model",
                    choices=["model", "tokenize_project", "block_bwd", "block_variants", "moe_train", "ceilings",
                             "epilogue_overlap", "vendor_gemm"],
                    help="model: the block stack (default); tokenize_project: the projection "
                         "tokenizer alone on the pad-split model's embedding; block_bwd: the dense "
                         "block backward on block 0 of the workload; block_variants: the SwiGLU "
                         "(D -> 4/3 D) block beside the GELU FFN (D -> 2D) block of equal parameters and "
                         "flops, with and without the Add & Norm after the mix; moe_train: training "
                         "step of the MoE block with dense-training / sparse-inference routers; "
                         "ceilings: the MFMA-loop and HBM-copy probes alone; epilogue_overlap: the W1 "
                         "and W2 products of block 0 with the epilogue after each tile and inside the "
                         "next tile's main loop; vendor_gemm: torch.bmm (hipBLASLt) on the same two "
                         "product shapes, no epilogue")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the probes after the timed steps")
    ap.add_argument("--cpu-rows", type=int, default=1024, help="samples in the oracle leg")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-profile", action="store_true", help="skip the per-launch HIP events")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="before warmup, one device-to-device copy of this many MiB (a known-size "
                         "reference for rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}): "
              "this build has no multi-GPU path; the forward shards data-parallel over samples "
              "with no exchange, so the one-GPU number is the per-GPU rate.", file=sys.stderr)
        return 2

    import torch
    import synthetic_inputs as si
    from rankmixer_token_mixing_amd import binding as bd
    from rankmixer_token_mixing_amd import perfmodel as pm

    if not os.path.exists(bd.lib_path()):
        from rankmixer_token_mixing_amd.build import build
        build()
    bd.check_fresh()  # never time a library built from other sources than the tree's
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy probe: {n} bytes read, {n} bytes written")
        del src, dst

    if args.op == "tokenize_project":
        return bench_project(args)
    if args.op == "block_bwd":
        return bench_block_bwd(args)
    if args.op == "block_variants":
        return bench_variants(args)
    if args.op == "moe_train":
        return bench_moe_train(args)
    if args.op == "ceilings":
        return bench_ceilings(args)
    if args.op == "epilogue_overlap":
        return bench_epilogue_overlap(args)
    if args.op == "vendor_gemm":
        return bench_vendor_gemm(args)

    cfg = si.CONFIGS[args.config]
    t0 = time.perf_counter()
    inputs = si.make_inputs(cfg)
    log(f"generated {cfg.name} inputs in {time.perf_counter() - t0:.1f}s: {cfg.description}")
    blocks = bd.upload_blocks(inputs["blocks"])
    head = {"w": bd.to_device(inputs["head"]["w"]), "c": inputs["head"]["c"]} if "head" in inputs else None
    dtype = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    model = bd.Model(blocks, cfg.T, cfg.D, dtype, F=cfg.F, head=head)
    inp = bd.to_device(inputs["emb"] if cfg.F else inputs["x"])
    out = {}

    def step():
        bd.rm_model_fwd(model, inp, want_x=True, out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")
    # a short pass with events around every launch group: the per-kernel table
    # and the choice of the dominant kernel
    bd.profile_only(None)
    bd.profile_enable(not args.no_profile)
    for _ in range(PROFILE_STEPS):
        step()
    torch.cuda.synchronize()
    warm = bd.profile_read() if not args.no_profile else {}
    bd.profile_enable(False)
    dom = max(warm, key=lambda k: warm[k][0]) if warm else None

    # timed steps: events only around the dominant kernel's launches
    bd.profile_only(dom)
    bd.profile_enable(dom is not None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    live = bd.profile_read() if dom is not None else {}
    bd.profile_enable(False)
    bd.profile_only(None)
    log(f"timed {args.steps} steps in {elapsed * 1e3:.1f} ms")

    ms_step = elapsed * 1e3 / args.steps
    L = cfg.L
    hidden = cfg.hidden
    value = cfg.B * L / (elapsed / args.steps)

    # algorithmic work of each launch group (one launch group = one block's worth)
    x0 = bd.rm_tokenize_padsplit(inp, cfg.T, cfg.D, out_dtype=dtype) if cfg.F else inp
    active = None
    if cfg.E:
        # either expert product, averaged over the blocks: 2 * active rows * He * D
        active = moe_active_rows(bd, blocks, x0, cfg.D)
        gemm_flops = int(round(2 * (sum(active) / len(active)) * hidden * cfg.D))
        prod_names = ("moe_ffn1", "moe_ffn2")
    else:
        gemm_flops = cfg.T * pm.gemm_flops(cfg.B, hidden, cfg.D)  # either product of one block
        prod_names = ("ffn1", "ffn2")
    eb = pm.ELEM_BYTES[cfg.dtype]
    row_bytes = {  # compulsory HBM bytes per launch
        "mix_ln1": 2 * cfg.B * cfg.T * cfg.D * eb,
        "ln2": cfg.B * cfg.T * cfg.D * 3 * eb,  # Z and the residual S in, X' out
        "ln2_mix_ln1": cfg.B * cfg.T * cfg.D * 3 * eb,  # Z and S in, the next block's S out
        # the fp32 embedding in (each element once), the first block's S out
        "tokenize_mix_ln1": cfg.B * (4 * cfg.F + cfg.T * cfg.D * eb),
    }
    def table(prof):
        kern = {}
        for name, (tot_ms, n) in prof.items():
            avg = tot_ms / max(n, 1)
            e = {"avg_ms": round(avg, 5), "launches": n, "total_ms": round(tot_ms, 3)}
            if gemm_flops and name in prod_names:
                e["tflops"] = round(gemm_flops / (avg * 1e-3) / 1e12, 1)
            if name in row_bytes:
                e["gbs"] = round(row_bytes[name] / (avg * 1e-3) / 1e9, 1)
            kern[name] = e
        return kern

    kernels = table(warm)       # every launch group, over the warm-up steps
    live_k = table(live)        # the dominant one, over the timed steps

    roofline = None
    if dom in live_k:
        avg_s = live_k[dom]["avg_ms"] * 1e-3
        if gemm_flops and dom in prod_names:
            ach = gemm_flops / avg_s / 1e12
            roofline = {"bound": "mfma", "kernel": dom, "achieved": round(ach, 1),
                        "peak": pm.PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else pm.PEAK_FP32_MFMA_TFLOPS,
                        "unit": "TFLOP/s"}
            roofline["frac"] = round(ach / roofline["peak"], 4)
            roofline["flop_per_launch"] = gemm_flops
        elif dom in row_bytes:
            ach = row_bytes[dom] / avg_s / 1e9
            roofline = {"bound": "hbm", "kernel": dom, "achieved": round(ach, 1), "peak": pm.PEAK_HBM_GBS,
                        "unit": "GB/s", "frac": round(ach / pm.PEAK_HBM_GBS, 4)}
        if roofline is not None:
            roofline["launches_timed"] = live_k[dom]["launches"]
            roofline["traffic"] = committed_traffic(cfg.name, dom)

    if cfg.E:
        flops_l = [pm.moe_flops(a, cfg.B, cfg.T, cfg.D, cfg.E, hidden) for a in active]
        block_flops = flops_l[0]
        step_tflops = sum(flops_l) / (ms_step * 1e-3) / 1e12
    else:
        block_flops = pm.block_flops(cfg.B, cfg.T, cfg.D, hidden)
        step_tflops = block_flops * L / (ms_step * 1e-3) / 1e12
    block0 = block0_protocol(bd, blocks, x0, cfg.B, block_flops, pm.PEAK_BF16_TFLOPS)
    log(f"block 0 alone: {block0['ms']} ms")
    ceil = None if args.no_ceilings else measure_ceilings(bd)
    roofline = with_ceiling(roofline, ceil)
    if ceil:
        block0["frac_of_measured_mfma_ceiling"] = round(block0.get("tflops", 0) / ceil["mfma_bf16_random_tflops"], 4)

    rec = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "samples/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {
            "workload": cfg.description,
            "B": cfg.B, "T": cfg.T, "D": cfg.D, "hidden": hidden, "L": L,
            "step": "rm_model_fwd over the batch (all blocks)",
            "value_is": "B * L / step time (samples through one block per second)",
        },
        "roofline": roofline,
        "step_tflops": round(step_tflops, 1) if step_tflops else None,
        "step_frac_of_bf16_peak": round(step_tflops / pm.PEAK_BF16_TFLOPS, 4) if step_tflops else None,
        "kernels": kernels,
        "kernels_from": f"HIP events around every launch group over {PROFILE_STEPS} untimed steps after the "
                        "warm-up; the timed steps carry events around the dominant kernel only (its average is "
                        "the roofline's)",
        "block0_fwd": block0,
        "ceilings": ceil,
    }
    if active is not None:
        rec["moe_active_rows"] = {"per_block": active, "of": cfg.B * cfg.T * cfg.E,
                                  "note": "flops count active (sample, token, expert) rows only"}
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on a bounded sample ...")
        rec["cpu_baseline"] = cpu_baseline(inputs, L, args.cpu_rows)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
