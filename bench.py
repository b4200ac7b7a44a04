#!/usr/bin/env python3
"""Benchmark of the GLM-shape routed-expert int4 MoE layer on one MI355X.

Workload (one "step" = one pass of the whole block for one token): a GLM-5.2
MoE layer (hidden 6144, 256 routed experts with gate/up 2048x6144 and down
6144x2048 in packed int4 with a float scale per row, one shared expert of the
same shape, float32 sigmoid router 256x6144 plus correction bias, top-8,
routed scaling 2.5) applied to one token: router, top-8, int8 activation
quantization, 9 SwiGLU experts, weighted combine.  Weights and activations
are seeded synthetic data already resident in HBM.

Steps cycle over R independent layer replicas (different seeds) and 256
distinct tokens, so that consecutive steps never find a layer's weights in
the 256 MB last-level cache (a real decode visits every other layer in
between).

Timed regions (each bracketed by device synchronization):
  1. K steps replayed from HIP graphs of G consecutive steps (decode serving
     captures its step loop in graphs) -> "value";
  2. K steps launched directly on the stream -> "stream_us_per_token";
  3. K steps on the stream with HIP events handed to the second and third
     launches of every step (the library launches them with hipExtLaunchKernel,
     so each event pair holds that kernel's own start and end timestamps)
     -> "kernels_us" and "roofline" (the second launch, routed gate/up +
     shared-expert down, 107 MB of weights, is the dominant kernel).

Prints one JSON line.
"""
import argparse
import ctypes
import gc
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
INT8_PEAK_TOPS = 5000.0  # dense int8 MFMA
COPY_CAL_BYTES = 256 << 20
# rocprofv3 counter summary of the dominant kernel (HBM bytes per launch, and
# the hash of the kernel source it was taken on)
TRAFFIC_FILES = {k: os.path.join(ROOT, "profiles", f"{k}_glm_decode_traffic.md")
                 for k in ("decode_b_kernel",)}
# device code of the decode kernels (the counter summaries are valid while
# these files are unchanged)
KERNEL_SOURCES = [os.path.join(ROOT, "int4_expert_gemv_moe_amd", "csrc", f)
                  for f in ("decode.hip", "rowops.h", "moe_common.h", "quant.h", "topk.h",
                            "norm.h")]
D, I, E, K = 6144, 2048, 256, 8
EXPERT_GATEUP_BYTES = 2 * I * (D // 2) + 2 * I * 4          # 12,599,296
EXPERT_DOWN_BYTES = D * (I // 2) + D * 4                     # 6,316,032
EXPERT_BYTES = EXPERT_GATEUP_BYTES + EXPERT_DOWN_BYTES       # 18,915,328
ROUTER_BYTES = E * D * 4 + E * 4                             # 6,292,480
LAYER_TOKEN_BYTES = 9 * EXPERT_BYTES + ROUTER_BYTES + 2 * D * 4  # 176,579,584
# the three launches of one decode step (algorithmic weight bytes)
PHASE_A_BYTES = ROUTER_BYTES + EXPERT_GATEUP_BYTES           # router + shared gate/up
PHASE_B_BYTES = K * EXPERT_GATEUP_BYTES + EXPERT_DOWN_BYTES  # routed gate/up + shared down
PHASE_C_BYTES = K * EXPERT_DOWN_BYTES                        # routed down


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch of the kernel from the committed counter summary,
    or None when it is missing or was taken on other kernel sources."""
    path = TRAFFIC_FILES.get(kernel)
    if path is None or not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if line.startswith("- ") and ":" in line:
                k, v = line[2:].split(":", 1)
                vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return int(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ---- the CPU oracle timed on this host (the cpu_baseline leg) -------------------
#
# Every input is built and every expert generated before any GPU call; the
# worker processes are forked from that state (their inputs shared copy-on-
# write) before the GPU is initialised, and nothing forks or execs after it.

_CPU_WORK = {}  # inputs of the oracle jobs, inherited by the forked workers


def _cpu_job(job):
    """One oracle job: (config, lo, hi) over the prepared inputs; returns the
    seconds it took.  The oracle is single-threaded C."""
    import oracle
    from oracle.stack import stack_layer

    kind, lo, hi = job
    w = _CPU_WORK[kind]
    t0 = time.perf_counter()
    if kind == "decode":  # per-token decode, one call per token
        for s in range(lo, hi):
            oracle.layer_forward(w["layer"], w["x"][s:s + 1])
    elif kind in ("verify", "prefill"):  # the unique-expert union over the token range
        oracle.layer_forward_batch(w["layer"], w["x"][lo:hi])
    else:  # stack: the token range through the stack's layers
        x = w["x"][lo:hi].copy()
        for L in w["layers"]:
            x = stack_layer(L, x, w["gamma"])
    return time.perf_counter() - t0


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baselines(decode_tokens: int = 32, prefill_subset: int = 64, prefill_fanout: int = 512,
                  stack_layers: int = 4, seed: int = 0):
    """The oracle on bounded samples of every configuration, on 1 core and
    fanned out over N cores (N independent single-threaded processes over
    disjoint tokens).  Must run before the first GPU call."""
    import multiprocessing as mp

    import numpy as np

    import synth
    from oracle import layer_forward, rmsnorm, router_topk
    from oracle.layers import LazyLayer, bias_for

    try:
        n_cpu = len(os.sched_getaffinity(0))
    except AttributeError:
        n_cpu = os.cpu_count() or 1
    N = max(1, min(16, n_cpu))  # a process may use a 16-CPU share of the host
    t_prep = time.perf_counter()
    glm = synth.GLM
    gen = lambda L, ids: L.ensure(ids, workers=N)
    # decode tokens through one layer (the headline's replica 0 recipe)
    L2 = LazyLayer(seed, glm, 0, bias_for("uniform", seed, glm))
    x2 = synth.activations(7, decode_tokens, D)
    gen(L2, L2.ensure_for(x2))
    # the 64-token Zipf(1.1) verify
    wr = synth.router_w(0, glm)
    L3 = LazyLayer(0, glm, 0, np.zeros(E, np.float32), router_w=wr)
    x3, _, _ = synth.zipf_activations(0, glm, 64, wr)
    gen(L3, L3.ensure_for(x3))
    # the 2048-token bf16 prefill (uniform routing: every expert is used)
    L4 = LazyLayer(0, glm, 0, np.zeros(E, np.float32))
    x4 = synth.bf16_to_f32(synth.bf16_bits(synth.activations(5, 2048, D)))[:prefill_fanout]
    gen(L4, range(E))
    # the stack's first stack_layers layers, batch 1 and batch 4
    with open(os.path.join(ROOT, "tests", "golden", "stack_beta.json")) as f:
        beta = json.load(f)["beta"]
    L5 = [LazyLayer(0, glm, l, synth.zipf_bias(0, E, l, beta)) for l in range(stack_layers)]
    x5 = synth.activations(0, 4, D, item=74)
    gamma = np.ones(D, np.float32)
    # the experts each layer's tokens select (routing follows the residual
    # stream, so walk it once with the oracle's router only)
    xs = x5.copy()
    for L in L5:
        xn = rmsnorm(xs, gamma)
        idx, _, _, _ = router_topk(L.cfg, xn, L.router_w, L.router_b)
        gen(L, idx)
        xs = xs + layer_forward(L, xn)
    _CPU_WORK.update(decode={"layer": L2, "x": x2}, verify={"layer": L3, "x": x3},
                     prefill={"layer": L4, "x": x4},
                     stack={"layers": L5, "x": x5, "gamma": gamma})
    prep_s = time.perf_counter() - t_prep
    log(f"cpu baseline inputs ready in {prep_s:.1f}s ({N} workers)")

    def fanout(kind, n_tokens, per_proc=None):
        """Wall seconds of the job split over N processes (disjoint tokens)."""
        step = per_proc or (n_tokens + N - 1) // N
        jobs = [(kind, lo, min(n_tokens, lo + step)) for lo in range(0, n_tokens, step)]
        t0 = time.perf_counter()
        list(pool.map(_cpu_job, jobs))
        return time.perf_counter() - t0, len(jobs)

    ctx = mp.get_context("fork")
    res = {}
    with ctx.Pool(processes=N) as pool:
        one = lambda job: pool.apply(_cpu_job, (job,))  # 1 core: one worker, one job
        # per-token decode
        t1 = one(("decode", 0, decode_tokens))
        tn, nproc = fanout("decode", decode_tokens)
        res["decode"] = {"sample": f"{decode_tokens} GLM decode tokens, per-token path",
                            "us_per_token_1core": round(t1 / decode_tokens * 1e6, 1),
                            "us_per_token_ncore": round(tn / decode_tokens * 1e6, 1),
                            "tokens_per_s_ncore": round(decode_tokens / tn, 2), "procs": nproc}
        # the 64-token verify (the whole workload)
        t1 = one(("verify", 0, 64))
        tn, nproc = fanout("verify", 64)
        res["verify64"] = {"sample": "the whole 64-token Zipf verify, union path",
                              "us_per_step_1core": round(t1 * 1e6, 1),
                              "us_per_step_ncore": round(tn * 1e6, 1), "procs": nproc}
        # the prefill: 1 core on prefill_subset tokens, N cores on prefill_fanout,
        # both extrapolated
        t1 = one(("prefill", 0, prefill_subset))
        tn, nproc = fanout("prefill", prefill_fanout)
        res["prefill2048"] = {
            "sample": f"1 core: {prefill_subset} of the 2048 prefill tokens; N cores: {prefill_fanout} "
                      f"tokens; union path; per-step times extrapolated linearly to 2048 tokens",
            "us_per_step_1core_extrapolated": round(t1 * 2048 / prefill_subset * 1e6, 1),
            "us_per_step_ncore_extrapolated": round(tn * 2048 / prefill_fanout * 1e6, 1),
            "measured_s_1core": round(t1, 2), "measured_s_ncore": round(tn, 2), "procs": nproc}
        # the stack: batch 1 and batch 4 through stack_layers layers, extrapolated to 48
        t1b1 = one(("stack", 0, 1))
        t1b4 = one(("stack", 0, 4))
        tnb4, nproc = fanout("stack", 4, per_proc=1)
        sc = 48 / stack_layers
        res["stack48"] = {
            "sample": f"first {stack_layers} of the 48 stack layers (RMSNorm + block + residual), "
                      f"times extrapolated linearly to 48 layers",
            "batch1_us_per_token_1core": round(t1b1 * sc * 1e6, 1),
            "batch4_us_per_step_1core": round(t1b4 * sc * 1e6, 1),
            "batch4_us_per_step_ncore": round(tnb4 * sc * 1e6, 1), "procs_batch4": nproc}
    _CPU_WORK.clear()
    head = res["decode"]
    return {"value": head["us_per_token_1core"], "unit": "us/token", "cores": 1, "kind": "oracle",
            "sample": f"{decode_tokens} GLM-shape decode tokens through one layer, oracle per-token "
                      f"path, single-threaded C (per-config and {N}-process figures in 'configs')",
            "cpu_model": _cpu_model(), "nproc": os.cpu_count(), "cpus_available": n_cpu,
            "workers": N, "prep_s": round(prep_s, 1), "configs": res,
            "context": {
                "note": "the pages' numbers, other hardware and other scope; context only",
                "avx2_int8_matmul_GFLOPs": 119,
                "end_to_end_tok_per_s_12core_25GB": 0.3,
                "four_L40_expert_kernel_ms_per_token_all_layers": 289.7}}


def timed_cold(call, iters: int, flush_bytes: int = 1 << 30):
    """Per-iteration microseconds of call(): before each iteration, outside
    the events, a 1 GiB buffer is written, which evicts the 256 MB
    memory-side cache, so every weight byte comes from HBM."""
    import numpy as np
    import torch

    buf = torch.empty(flush_bytes // 4, dtype=torch.float32, device="cuda")
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(iters)]
    for i, (a, b) in enumerate(evs):
        buf.fill_(float(i))
        a.record()
        call()
        b.record()
    torch.cuda.synchronize()
    del buf
    return np.array([a.elapsed_time(b) * 1e3 for a, b in evs])


def spread(us):
    import numpy as np
    return {"p10": round(float(np.percentile(us, 10)), 1), "p50": round(float(np.median(us)), 1),
            "p90": round(float(np.percentile(us, 90)), 1), "iters": int(len(us))}


def bench_prefill(layer, iters: int = 5):
    """Prefill of 2048 tokens through one GLM-shape layer on the unique-expert
    union path (int8 MFMA grouped GEMMs): activations N(0,1) rounded to bf16
    and handed over as bf16 rows (the same bits as their float32 widening,
    which is timed beside them), router bias 0 (uniform routing)."""
    import numpy as np
    import torch

    import int4_expert_gemv_moe_amd as moe
    import synth

    S = 2048
    P = K + 1
    zl = moe.DeviceLayer(layer.cfg, layer.router_w,
                         torch.zeros(E, dtype=torch.float32, device="cuda"), layer.routed,
                         layer.shared)
    bits = synth.bf16_bits(synth.activations(5, S, D))
    x = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    x32 = torch.from_numpy(synth.bf16_to_f32(bits)).cuda()
    ws = moe.Workspace(zl.cfg, S, moe.WS_BATCH)
    out = moe.moe_layer_forward_batch(zl, x, ws)
    idx = torch.empty(S, K, dtype=torch.int32, device="cuda")
    moe.moe_layer_forward_batch(zl, x, ws, out=out, topk_idx=idx)
    out32 = moe.moe_layer_forward_batch(zl, x32, ws)
    torch.cuda.synchronize()
    if not torch.equal(out.view(torch.int32), out32.view(torch.int32)):
        raise RuntimeError("bf16 rows and their float32 widening gave different bits")
    used = int(np.unique(idx.cpu().numpy()).size) + 1  # + the shared expert
    cold = timed_cold(lambda: moe.moe_layer_forward_batch(zl, x, ws, out=out), 2 * iters)
    us = float(np.median(cold))
    cold32 = timed_cold(lambda: moe.moe_layer_forward_batch(zl, x32, ws, out=out32), 2 * iters)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        moe.moe_layer_forward_batch(zl, x, ws, out=out)
    e1.record()
    torch.cuda.synchronize()
    warm_us = e0.elapsed_time(e1) * 1e3 / iters
    ops = 2 * S * P * 3 * I * D  # int8 multiply-adds of the expert matmuls, x2
    nbytes = used * EXPERT_BYTES + ROUTER_BYTES + S * D * 2 + S * D * 4  # bf16 x, float32 out
    ideal_us = max(nbytes / (HBM_PEAK_GBPS * 1e3), ops / (INT8_PEAK_TOPS * 1e6))
    log(f"prefill 2048: {us:.1f} us cold ({warm_us:.1f} warm), {ops / us / 1e6:.1f} TOPS "
        f"({used} experts read); float32 rows {float(np.median(cold32)):.1f} us")
    return {"workload": "GLM-shape layer, 2048-token prefill (bf16 activation rows, uniform "
                        "routing), unique-expert union with int8 MFMA grouped GEMMs",
            "timing": "cold: a 1 GiB buffer written before each iteration (median reported)",
            "us": round(us, 1), "us_spread": spread(cold), "warm_us": round(warm_us, 1),
            "us_float32_rows": round(float(np.median(cold32)), 1),
            "tokens_per_s": round(S / us * 1e6, 1),
            "int8_TOPS": round(ops / us / 1e6, 1), "expert_int8_ops": ops,
            "experts_read": used, "hbm_bytes": nbytes,
            "roofline_us": round(ideal_us, 1), "frac_of_roofline": round(ideal_us / us, 4)}


def bench_verify(layer, iters: int = 20):
    """Batched verify of 64 tokens through one GLM-shape layer on the
    unique-expert union path, routing skewed so that expert popularity is
    Zipf(1.1): the token rows are solved so that the router gives
    log p_e + Gumbel noise (router bias 0)."""
    import numpy as np
    import torch

    import int4_expert_gemv_moe_amd as moe
    import synth

    S = 64
    wr = synth.router_w(0, synth.GLM)
    x_np, _, _ = synth.zipf_activations(0, synth.GLM, S, wr)
    zl = moe.DeviceLayer(layer.cfg, torch.from_numpy(wr).cuda(),
                         torch.zeros(E, dtype=torch.float32, device="cuda"), layer.routed,
                         layer.shared)
    x = torch.from_numpy(x_np).cuda()
    ws = moe.Workspace(zl.cfg, S, moe.WS_BATCH)
    idx = torch.empty(S, K, dtype=torch.int32, device="cuda")
    out = moe.moe_layer_forward_batch(zl, x, ws, topk_idx=idx)
    torch.cuda.synchronize()
    counts = np.bincount(idx.cpu().numpy().ravel(), minlength=E)
    used = int((counts > 0).sum()) + 1  # + the shared expert
    cold = timed_cold(lambda: moe.moe_layer_forward_batch(zl, x, ws, out=out), iters)
    us = float(np.median(cold))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        moe.moe_layer_forward_batch(zl, x, ws, out=out)
    e1.record()
    torch.cuda.synchronize()
    warm_us = e0.elapsed_time(e1) * 1e3 / iters
    nbytes = used * EXPERT_BYTES + ROUTER_BYTES + 2 * S * D * 4
    log(f"verify 64 (Zipf): {us:.1f} us cold ({warm_us:.1f} warm), union {used - 1} routed experts")
    return {"workload": "GLM-shape layer, 64-token batched verify, Zipf(1.1) expert popularity, "
                        "unique-expert union",
            "timing": "cold: a 1 GiB buffer written before each iteration (median reported)",
            "us": round(us, 1), "us_spread": spread(cold), "warm_us": round(warm_us, 1),
            "us_per_token": round(us / S, 2),
            "union_routed_experts": used - 1, "hottest_expert_tokens": int(counts.max()),
            "popularity_top8": [int(c) for c in np.sort(counts)[::-1][:8]],
            "experts_by_tokens": {"1": int((counts == 1).sum()), "2-3": int(((counts >= 2) & (counts <= 3)).sum()),
                                  "4-15": int(((counts >= 4) & (counts <= 15)).sum()),
                                  "16+": int((counts >= 16).sum())},
            "hbm_bytes": nbytes, "GBps": round(nbytes / us / 1e3, 1),
            "frac_of_hbm_peak": round(nbytes / us / 1e3 / HBM_PEAK_GBPS, 4)}


def bench_tiered(layer, slot_counts=(192, (128, 64), 64), warm: int = 64, timed: int = 192):
    """Decode through one GLM-shape layer whose routed experts live in pinned
    host memory and only n_slots HBM slab slots (section 05 LRU expert cache,
    section 13 slab reads), Zipf(1.1)-skewed routing, one token per call: the
    router runs on the device, the host maps the selected experts to slots and
    copies the missing 18.9 MB slabs in, then the block runs on the slot stack
    with the given routing.  Wall time per token after `warm` tokens."""
    import numpy as np
    import torch

    import int4_expert_gemv_moe_amd as moe
    import synth

    n = warm + timed
    wr = synth.router_w(0, synth.GLM)
    x_np, _, _ = synth.zipf_activations(1, synth.GLM, n, wr)
    zl = moe.DeviceLayer(layer.cfg, torch.from_numpy(wr).cuda(),
                         torch.zeros(E, dtype=torch.float32, device="cuda"), layer.routed,
                         layer.shared)
    x = torch.from_numpy(x_np).cuda()
    wsr = moe.Workspace(zl.cfg, 1, moe.WS_ROUTER)
    ws = moe.Workspace(zl.cfg, 1, moe.WS_FORWARD)
    out = torch.empty(1, D, dtype=torch.float32, device="cuda")
    res = {"workload": "GLM-shape layer decode, 1 token/call, Zipf(1.1) routing, routed experts in "
                       "pinned host memory with n_slots HBM slab slots (LRU), shared expert and "
                       "router resident",
           "tokens_timed": timed, "slab_bytes": EXPERT_BYTES}
    host = None
    for n_slots in slot_counts:
        # (lru, pinned): pinned slots kept by heat (section 13 swap rule)
        n_slots, n_pin = n_slots if isinstance(n_slots, tuple) else (n_slots, 0)
        tl = moe.TieredLayer.from_device_layer(zl, n_slots, host_slabs=host, n_pinned=n_pin)
        host = tl.host_slabs
        for t in range(warm):
            tl.forward(x[t:t + 1], wsr, ws, out=out)
        torch.cuda.synchronize()
        h0, m0 = tl.tier.stats()
        t0 = time.perf_counter()
        for t in range(warm, n):
            tl.forward(x[t:t + 1], wsr, ws, out=out)
        torch.cuda.synchronize()
        us = (time.perf_counter() - t0) * 1e6 / timed
        h1, m1 = tl.tier.stats()
        hits, misses = h1 - h0, m1 - m0
        key = (f"slots_{n_slots}_of_{E}" if not n_pin else
               f"slots_{n_slots}_lru_{n_pin}_pinned_of_{E}")
        res[key] = {"us_per_token": round(us, 1), "tokens_per_s": round(1e6 / us, 1),
                    "hit_rate": round(hits / max(1, hits + misses), 4),
                    "misses_per_token": round(misses / timed, 3),
                    "h2d_GB_per_token": round(misses * EXPERT_BYTES / timed / 1e9, 4),
                    "h2d_GBps": round(misses * EXPERT_BYTES / (us * timed) / 1e3, 1)}
        log(f"tiered {key}: {us:.1f} us/token, hit rate {res[key]['hit_rate']}")
        if n_slots >= 160 and not n_pin:
            # 64-token verify steps through the union path on the same slots
            S, nb = 64, 12
            xb_np, _, _ = synth.zipf_activations(2, synth.GLM, S * nb, wr)
            xb = torch.from_numpy(xb_np).cuda()
            wsrb = moe.Workspace(zl.cfg, S, moe.WS_ROUTER)
            wsb = moe.Workspace(zl.cfg, S, moe.WS_BATCH)
            outb = torch.empty(S, D, dtype=torch.float32, device="cuda")
            for b in range(4):
                tl.forward(xb[b * S:(b + 1) * S], wsrb, wsb, out=outb, union=True)
            torch.cuda.synchronize()
            h0, m0 = tl.tier.stats()
            t0 = time.perf_counter()
            for b in range(4, nb):
                tl.forward(xb[b * S:(b + 1) * S], wsrb, wsb, out=outb, union=True)
            torch.cuda.synchronize()
            us = (time.perf_counter() - t0) * 1e6 / (nb - 4)
            h1, m1 = tl.tier.stats()
            hits, misses = h1 - h0, m1 - m0
            res[key]["verify_64_union"] = {
                "us_per_step": round(us, 1), "us_per_token": round(us / S, 2),
                "hit_rate": round(hits / max(1, hits + misses), 4),
                "misses_per_step": round(misses / (nb - 4), 2),
                "h2d_GBps": round(misses * EXPERT_BYTES / (us * (nb - 4)) / 1e3, 1)}
            log(f"tiered {key} verify 64: {us:.1f} us/step")
        del tl
    del host
    torch.cuda.empty_cache()
    return res


def bench_topp(layers, x, steps: int = 512, ps=(0.7, 0.9, 1.0)):
    """Per-token decode with the adaptive expert top-p: the same layer
    replicas (cold in the MALL) and tokens as the headline decode, one token
    per call, plain stream launches between events.  Reports the experts
    kept per token and the weight bytes actually read."""
    import numpy as np
    import torch

    import int4_expert_gemv_moe_amd as moe

    T, R = x.shape[0], len(layers)
    res = {"workload": "GLM-shape MoE layer decode, 1 token/step, adaptive expert top-p "
                       "(keff of the top-8 per token), 8 cold layer replicas",
           "steps": steps}
    lib = moe.lib()
    stream = torch.cuda.current_stream()
    st = ctypes.c_void_p(stream.cuda_stream)
    out = torch.empty(1, D, dtype=torch.float32, device="cuda")
    xp = [ctypes.c_void_p(x[t].data_ptr()) for t in range(T)]
    op = ctypes.c_void_p(out.data_ptr())
    lstructs = [l.cstruct() for l in layers]
    lrefs = [ctypes.byref(s_) for s_ in lstructs]
    for p in ps:
        c = layers[0].cfg
        cfg = moe.config(c.D, c.I, c.E, c.K, c.n_shared, c.routed_scale, p)
        tl = [moe.DeviceLayer(cfg, l.router_w, l.router_b, l.routed, l.shared) for l in layers]
        ws = moe.Workspace(cfg, 1, moe.WS_FORWARD)
        keff = torch.empty(T, dtype=torch.int32, device="cuda")
        for t in range(T):  # kept experts per token (each token on its replica)
            moe.moe_layer_forward(tl[t % R], x[t:t + 1], ws, out=out, keff=keff[t:t + 1])
        torch.cuda.synchronize()
        mean_keff = float(keff.float().mean())
        cref = ctypes.byref(cfg)

        def run(n):
            rc = 0
            for i in range(n):
                rc |= lib.moe_layer_forward(cref, lrefs[i % R], xp[i % T], 1, op, 0, None, ws.ptr,
                                            ws.nbytes, st)
            if rc:
                raise moe.MoeError(f"moe_layer_forward failed ({rc})")

        run(64)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run(steps)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        nbytes = (mean_keff + 1) * EXPERT_BYTES + ROUTER_BYTES + 2 * D * 4
        res[f"topp_{p}"] = {"us_per_token": round(us, 3), "mean_keff": round(mean_keff, 3),
                            "bytes_per_token": int(nbytes),
                            "GBps": round(nbytes / us / 1e3, 1),
                            "frac_of_hbm_peak": round(nbytes / us / 1e3 / HBM_PEAK_GBPS, 4)}
        log(f"top-p {p}: {us:.2f} us/token, mean keff {mean_keff:.2f}")
    return res


EXPERT_I8_BYTES = 3 * I * D + (2 * I + D) * 4       # 37,789,696: int8 codes + row scales
EXPERT_I2_BYTES = 3 * I * D // 4 + (2 * I + D) * 4  # 9,478,144: packed int2 + row scales


def bench_fmt8(layer, steps: int = 512, n8: int = 8, n4: int = 16, n2: int = 32):
    """One GLM-shape SwiGLU expert on one token in the int8, int4 and packed
    int2 weight formats: each call reads one expert (cycling over 8 int8, 16
    int4 or 32 int2 experts, about 302 MB each, so the weights come from HBM
    rather than the MALL); plain stream launches between events."""
    import torch

    import int4_expert_gemv_moe_amd as moe
    import synth
    from synth.device_layers import build_device_experts_i2, build_device_experts_i8

    lib = moe.lib()
    cfg = layer.cfg
    stream = torch.cuda.current_stream()
    st = ctypes.c_void_p(stream.cuda_stream)
    e8 = build_device_experts_i8(0, synth.GLM, 0, n8)
    xq, sx = moe.moe_quant_act_i8(torch.from_numpy(synth.activations(7, 1, D)).cuda())
    y = torch.empty(1, D, dtype=torch.float32, device="cuda")
    ws8 = moe.Workspace(cfg, 1, moe.WS_SWIGLU8)
    ws4 = moe.Workspace(cfg, 1, moe.WS_SWIGLU)
    e2 = build_device_experts_i2(0, synth.GLM, 0, n2)
    s8, s4, s2 = e8.cstruct(), layer.routed.cstruct(), e2.cstruct()
    xqb, sxb = moe.moe_quant_act_b32(torch.from_numpy(synth.activations(7, 1, D)).cuda())
    cref = ctypes.byref(cfg)
    args = (ctypes.c_void_p(xq.data_ptr()), ctypes.c_void_p(sx.data_ptr()), 1)
    args_b = (ctypes.c_void_p(xqb.data_ptr()), ctypes.c_void_p(sxb.data_ptr()), 1)
    yp = ctypes.c_void_p(y.data_ptr())
    r8, r4, r2 = ctypes.byref(s8), ctypes.byref(s4), ctypes.byref(s2)
    nul4 = (None, None, None, None)

    def call(fn, a, eref, tail, ws):
        return lambda e: fn(cref, *a, eref, e, yp, *tail, ws.ptr, ws.nbytes, st)

    calls = {
        "int8": (call(lib.moe_expert_swiglu_i8, args, r8, nul4, ws8), n8, EXPERT_I8_BYTES),
        "int4": (call(lib.moe_expert_swiglu_i4, args, r4, nul4, ws4), n4, EXPERT_BYTES),
        "int2": (call(lib.moe_expert_swiglu_i2, args, r2, nul4, ws8), n2, EXPERT_I2_BYTES),
        "int4_block32_act": (call(lib.moe_expert_swiglu_i4_b32, args_b, r4, (None, None), ws8), n4,
                             EXPERT_BYTES),
    }
    res = {"workload": "one GLM-shape SwiGLU expert (6144 -> 2048 -> 6144), 1 token per call, "
                       "int8 / int4 / packed int2 weights and int4 with block-32 activation "
                       "scales, weights cycled over ~302 MB",
           "steps": steps}
    for name, (fn, n, nbytes) in calls.items():
        def run(k):
            rc = 0
            for i in range(k):
                rc |= fn(i % n)
            if rc:
                raise moe.MoeError(f"{name} expert call failed ({rc})")

        run(64)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run(steps)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        res[name] = {"us_per_call": round(us, 3), "weight_bytes": int(nbytes),
                     "GBps": round(nbytes / us / 1e3, 1),
                     "frac_of_hbm_peak": round(nbytes / us / 1e3 / HBM_PEAK_GBPS, 4)}
        log(f"expert {name}: {us:.2f} us/call ({nbytes / us / 1e3:.0f} GB/s)")
    return res


def bench_shared_i8(layers, x, steps: int = 512):
    """Per-token decode with the shared expert in the int8 format
    (moe_layer_forward_shared_i8): the headline decode's cold layer replicas
    and tokens, each replica with its own int8 shared expert; plain stream
    launches between events.  Weight bytes per token: the router, 8 int4
    routed experts and one int8 shared expert.  Then the union path with the
    int8 shared expert (moe_layer_forward_batch_shared_i8), timed cold: the
    64-token Zipf verify and the 2048-token prefill (uniform routing)."""
    import torch

    import int4_expert_gemv_moe_amd as moe
    import synth
    from synth.device_layers import build_device_experts_i8

    T, R = x.shape[0], len(layers)
    lib = moe.lib()
    stream = torch.cuda.current_stream()
    st = ctypes.c_void_p(stream.cuda_stream)
    sh8 = build_device_experts_i8(1, synth.GLM, 0, R)
    views = [moe.DeviceExpertsI8(sh8.gate_q[r:r + 1], sh8.gate_s[r:r + 1], sh8.up_q[r:r + 1],
                                 sh8.up_s[r:r + 1], sh8.down_q[r:r + 1], sh8.down_s[r:r + 1])
             for r in range(R)]
    s8 = [v.cstruct() for v in views]
    ls = [l.cstruct() for l in layers]
    cfg = layers[0].cfg
    ws = moe.Workspace(cfg, 1, moe.WS_SHARED8)
    out = torch.empty(1, D, dtype=torch.float32, device="cuda")
    xp = [ctypes.c_void_p(x[t].data_ptr()) for t in range(T)]
    op = ctypes.c_void_p(out.data_ptr())
    cref = ctypes.byref(cfg)

    def run(n):
        rc = 0
        for i in range(n):
            r = i % R
            rc |= lib.moe_layer_forward_shared_i8(cref, ctypes.byref(ls[r]), ctypes.byref(s8[r]),
                                                  xp[i % T], 1, op, 0, ws.ptr, ws.nbytes, st)
        if rc:
            raise moe.MoeError(f"moe_layer_forward_shared_i8 failed ({rc})")

    run(64)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    run(steps)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    nbytes = K * EXPERT_BYTES + EXPERT_I8_BYTES + ROUTER_BYTES + 2 * D * 4
    log(f"decode with int8 shared expert: {us:.2f} us/token")
    res = {"workload": "GLM-shape MoE layer decode, 1 token/step, shared expert in the int8 "
                       "format (moe_layer_forward_shared_i8: inside the per-token launches), "
                       "8 cold layer replicas",
           "steps": steps, "us_per_token": round(us, 3), "bytes_per_token": int(nbytes),
           "GBps": round(nbytes / us / 1e3, 1),
           "frac_of_hbm_peak": round(nbytes / us / 1e3 / HBM_PEAK_GBPS, 4)}
    # the 64-token Zipf verify through the union path with the int8 shared expert
    import numpy as np
    S = 64
    wr = synth.router_w(0, synth.GLM)
    x_np, _, _ = synth.zipf_activations(0, synth.GLM, S, wr)
    zl = moe.DeviceLayer(cfg, torch.from_numpy(wr).cuda(),
                         torch.zeros(E, dtype=torch.float32, device="cuda"), layers[0].routed,
                         layers[0].shared)
    xv = torch.from_numpy(x_np).cuda()
    wsb = moe.Workspace(cfg, S, moe.WS_BATCH)
    outb = torch.empty(S, D, dtype=torch.float32, device="cuda")
    call = lambda: moe.moe_layer_forward_shared_i8(zl, views[0], xv, wsb, out=outb,
                                                   fn_name="moe_layer_forward_batch_shared_i8")
    call()
    idx, _, _ = moe.moe_router_topk(cfg, xv, zl.router_w, zl.router_b,
                                    moe.Workspace(cfg, S, moe.WS_ROUTER))
    torch.cuda.synchronize()
    used = int(np.unique(idx.cpu().numpy()).size)
    cold = timed_cold(call, 20)
    vb = used * EXPERT_BYTES + EXPERT_I8_BYTES + ROUTER_BYTES + 2 * S * D * 4
    vus = float(np.median(cold))
    res["verify64_union"] = {"us": round(vus, 1), "us_spread": spread(cold),
                             "union_routed_experts": used, "hbm_bytes": vb,
                             "GBps": round(vb / vus / 1e3, 1),
                             "frac_of_hbm_peak": round(vb / vus / 1e3 / HBM_PEAK_GBPS, 4)}
    log(f"verify 64 with int8 shared expert: {vus:.1f} us cold")
    # the 2048-token prefill (uniform routing, float32 rows) with the int8 shared expert
    S = 2048
    xp_np = synth.bf16_to_f32(synth.bf16_bits(synth.activations(5, S, D)))
    zu = moe.DeviceLayer(cfg, layers[0].router_w, torch.zeros(E, dtype=torch.float32, device="cuda"),
                         layers[0].routed, layers[0].shared)
    xpf = torch.from_numpy(xp_np).cuda()
    wsp = moe.Workspace(cfg, S, moe.WS_BATCH)
    outp = torch.empty(S, D, dtype=torch.float32, device="cuda")
    callp = lambda: moe.moe_layer_forward_shared_i8(zu, views[0], xpf, wsp, out=outp,
                                                    fn_name="moe_layer_forward_batch_shared_i8")
    callp()
    idxp, _, _ = moe.moe_router_topk(cfg, xpf, zu.router_w, zu.router_b,
                                     moe.Workspace(cfg, S, moe.WS_ROUTER))
    torch.cuda.synchronize()
    usedp = int(np.unique(idxp.cpu().numpy()).size)
    coldp = timed_cold(callp, 10)
    pus = float(np.median(coldp))
    pb = usedp * EXPERT_BYTES + EXPERT_I8_BYTES + ROUTER_BYTES + 2 * S * D * 4
    res["prefill2048_union"] = {"us": round(pus, 1), "us_spread": spread(coldp),
                                "union_routed_experts": usedp, "hbm_bytes": pb,
                                "GBps": round(pb / pus / 1e3, 1)}
    log(f"prefill 2048 with int8 shared expert: {pus:.1f} us cold")
    return res


def bench_mla(contexts=(1024, 4096, 16384), steps: int = 200):
    """Section 09 absorbed MLA decode at the GLM shape (64 heads, latent 512,
    nope 192, rope 64, value 256; float32), one query per call over a cache of
    T rows.  Algorithmic bytes: kv_b once (64 * 448 * 512 floats) + the cache
    rows (T * 576 floats) + q and ctx."""
    import numpy as np
    import torch

    import int4_expert_gemv_moe_amd as moe

    H, kvl, nope, rope, vdim = 64, 512, 192, 64, 256
    cfg = moe.MlaConfig(H, kvl, nope, rope, vdim, float(1.0 / np.sqrt(nope + rope)))
    lib = moe.lib()
    stream = torch.cuda.current_stream()
    st = ctypes.c_void_p(stream.cuda_stream)
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    kv_b = torch.randn(H * (nope + vdim), kvl, device="cuda", generator=g) / kvl ** 0.5
    q = torch.randn(1, H, nope + rope, device="cuda", generator=g)
    ctx = torch.empty(1, H, vdim, device="cuda")
    res = {"workload": "GLM-shape MLA decode with weight absorption (64 heads, latent 512 + "
                       "rope 64, value 256, float32), 1 query per call", "steps": steps}
    for T in contexts:
        L = torch.randn(T, kvl, device="cuda", generator=g)
        R = torch.randn(T, rope, device="cuda", generator=g)
        ws = moe.MlaWorkspace(cfg, 1, T)
        args = (ctypes.byref(cfg), ctypes.c_void_p(q.data_ptr()), 1, ctypes.c_void_p(kv_b.data_ptr()),
                ctypes.c_void_p(L.data_ptr()), ctypes.c_void_p(R.data_ptr()), T,
                ctypes.c_void_p(ctx.data_ptr()), ws.ptr, ws.nbytes, st)

        def run(k):
            rc = 0
            for _ in range(k):
                rc |= lib.moe_mla_decode(*args)
            if rc:
                raise moe.MoeError(f"moe_mla_decode failed ({rc})")

        run(20)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run(steps)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        nbytes = (H * (nope + vdim) * kvl + T * (kvl + rope) + H * (nope + rope + vdim)) * 4
        res[f"T{T}"] = {"us_per_call": round(us, 3), "bytes": int(nbytes),
                        "GBps": round(nbytes / us / 1e3, 1),
                        "frac_of_hbm_peak": round(nbytes / us / 1e3 / HBM_PEAK_GBPS, 4)}
        log(f"mla T={T}: {us:.2f} us/call ({nbytes / us / 1e3:.0f} GB/s)")
        del L, R, ws
    return res


def bench_stack(steps: int = 64):
    """48 GLM-shape layers resident in HBM (per-layer Zipf-skewed routing,
    RMSNorm + residual, one MOE_F_PRENORM call per layer): decode steps of
    1 token (per-token path) and of 4 tokens (union path), each step one HIP
    graph replay."""
    import json as _json

    import torch

    import int4_expert_gemv_moe_amd as moe
    import synth
    from int4_expert_gemv_moe_amd.stack import Stack
    from synth.device_layers import build_device_layer

    with open(os.path.join(ROOT, "tests", "golden", "stack_beta.json")) as f:
        cal = _json.load(f)
    beta = cal["beta"]
    t0 = time.time()
    layers = [build_device_layer(0, synth.GLM, l, synth.zipf_bias(0, E, l, beta))
              for l in range(48)]
    torch.cuda.synchronize()
    log(f"built 48 layers in {time.time() - t0:.1f}s, "
        f"{torch.cuda.memory_allocated() / 2**30:.1f} GiB resident")
    stack = Stack(layers, torch.ones(D, dtype=torch.float32, device="cuda"))
    res = {"workload": "48 GLM-shape MoE layers resident in HBM, one call per layer: "
                       "x <- x + block(RMSNorm(x)) in place (RMSNorm eps 1e-5 inside the call), "
                       f"per-layer Zipf(1.1)-skewed routing (bias strength {beta})",
           "layers": 48, "bias_strength": beta, "target_zipf_exponent": cal["target_exponent"],
           "calibrated_zipf_exponent": cal["fitted_exponent"]}
    for S, union in ((1, False), (4, True)):
        x0 = torch.from_numpy(synth.activations(0, S, D, item=70 + S)).cuda()
        x = x0.clone()
        xn = torch.empty_like(x)
        ws = moe.Workspace(stack.cfg, S, moe.WS_BATCH if union else moe.WS_FORWARD)
        cap = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            x.copy_(x0)
            stack.forward(x, ws, xn=xn, union=union, stream=cap)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        step_us = e0.elapsed_time(e1) * 1e3 / steps
        key = "batch1" if S == 1 else "batch4_union"
        # the step's routing, layer by layer (an untimed pass from the same x0)
        idx = [torch.empty(S, K, dtype=torch.int32, device="cuda") for _ in range(48)]
        x.copy_(x0)
        stack.forward(x, ws, xn=xn, union=union, topk_idx=idx)
        torch.cuda.synchronize()
        uniq = [int(torch.unique(t).numel()) for t in idx]
        nbytes = sum((u + 1) * EXPERT_BYTES for u in uniq) + 48 * (ROUTER_BYTES + D * 4)
        gbps = nbytes / (step_us * 1e3)
        res[key] = {"us_per_step": round(step_us, 1), "us_per_token": round(step_us / S, 1),
                    "tokens_per_s": round(S / step_us * 1e6, 1),
                    "mean_union_routed_experts": round(sum(uniq) / 48, 2),
                    "bytes_per_step": nbytes, "hbm_GBps": round(gbps, 1),
                    "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}
        log(f"stack48 {key}: {step_us:.1f} us/step, {step_us / S:.1f} us/token, "
            f"union {sum(uniq) / 48:.1f}, {gbps:.0f} GB/s")
    del g, stack, layers
    return res


def hbm_read_probe(nbytes: int = 4 << 30, reps: int = 5):
    """Same-box reference for the HBM rates: the library's read-only stream
    (moe_stream_read, the decode kernels' load pattern) over 4 GiB, far
    beyond the 256 MB MALL; best of reps."""
    import torch

    import int4_expert_gemv_moe_amd as moe

    big = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    moe.moe_stream_read(big)
    torch.cuda.synchronize()
    best = None
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        moe.moe_stream_read(big)
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3
        best = us if best is None else min(best, us)
    del big
    torch.cuda.empty_cache()
    return {"GBps": round(nbytes / best / 1e3, 1), "kernel": "moe_stream_read over 4 GiB",
            "bytes": nbytes}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1024)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--replicas", type=int, default=8)
    ap.add_argument("--tokens", type=int, default=256)
    ap.add_argument("--cpu-tokens", type=int, default=32)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the verify, prefill and 48-layer stack measurements")
    ap.add_argument("--only", choices=["verify", "prefill", "stack", "tiered", "topp", "fmt8", "mla",
                                       "shared8"],
                    help="run only that secondary measurement and print its record (for profiling)")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the graph-replay pass (value then comes from the stream pass); "
                         "used for counter runs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy 8 times (the reference "
                         "kernel that scales rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(expert- or tensor-parallel sharding over RCCL is a design, not code).",
              file=sys.stderr)
        sys.exit(2)

    # the CPU oracle first: its worker processes are forked before any GPU call
    cpu = None
    if not args.no_cpu_baseline and not args.only and not args.copy_calibration:
        log("timing the CPU oracle ...")
        cpu = cpu_baselines(decode_tokens=args.cpu_tokens)
        log(f"oracle: {cpu['value']} us/token on 1 core; {json.dumps(cpu['configs'])}")

    import numpy as np
    import torch

    import int4_expert_gemv_moe_amd as moe
    import synth
    from synth.device_layers import build_device_layer

    torch.cuda.set_device(0)
    if args.copy_calibration:
        n = COPY_CAL_BYTES // 4
        src = torch.arange(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(8):
            dst.copy_(src)
        torch.cuda.synchronize()
        assert torch.equal(dst[-4:], src[-4:])
        log(f"copied {COPY_CAL_BYTES} bytes 8 times")
        return
    lib = moe.lib()
    if args.only:
        if args.only == "stack":
            rec = bench_stack()
        elif args.only == "mla":
            rec = bench_mla()
        elif args.only in ("topp", "shared8"):
            reps = [build_device_layer(r, synth.GLM, r, synth.router_b_uniform(r, synth.GLM, r))
                    for r in range(args.replicas)]
            fn = bench_topp if args.only == "topp" else bench_shared_i8
            rec = fn(reps, torch.from_numpy(synth.activations(7, args.tokens, D)).cuda())
        else:
            layer = build_device_layer(0, synth.GLM, 0, synth.router_b_uniform(0, synth.GLM, 0))
            rec = {"verify": bench_verify, "prefill": bench_prefill,
                   "tiered": bench_tiered, "fmt8": bench_fmt8}[args.only](layer)
        print(json.dumps(rec), flush=True)
        return
    t0 = time.time()
    layers = []
    for r in range(args.replicas):
        b = synth.router_b_uniform(r, synth.GLM, r)
        layers.append(build_device_layer(r, synth.GLM, r, b))
    torch.cuda.synchronize()
    log(f"built {args.replicas} layer replicas in {time.time() - t0:.1f}s")
    T = args.tokens
    x = torch.from_numpy(synth.activations(7, T, D)).cuda()
    out = torch.empty(T, D, dtype=torch.float32, device="cuda")
    cfg = layers[0].cfg
    ws = moe.Workspace(cfg, 1, moe.WS_FORWARD)
    stream = torch.cuda.current_stream()
    st = ctypes.c_void_p(stream.cuda_stream)
    lstructs = [l.cstruct() for l in layers]
    lrefs = [ctypes.byref(s) for s in lstructs]
    cref = ctypes.byref(cfg)
    xp = [ctypes.c_void_p(x[t].data_ptr()) for t in range(T)]
    op = [ctypes.c_void_p(out[t].data_ptr()) for t in range(T)]
    fn = lib.moe_layer_forward
    R = args.replicas

    def run(n, probes=None, stream_handle=st, start=0):
        rc = 0
        for i in range(start, start + n):
            pr = probes[i - start] if probes is not None else None
            rc |= fn(cref, lrefs[i % R], xp[i % T], 1, op[i % T], 0, pr, ws.ptr, ws.nbytes,
                     stream_handle)
        if rc:
            raise moe.MoeError(f"moe_layer_forward failed ({rc})")

    K = args.steps
    run(args.warmup)
    torch.cuda.synchronize()

    # 1. graph replay: G steps per graph, G the largest divisor of K up to 64
    G = max(g for g in range(1, min(64, K) + 1) if K % g == 0)
    if args.no_graph:
        G = 0
    graph_us = None
    graph_spread = None
    if G:
        try:
            n_graphs = max(1, min(K // G, (R * T) // G))
            graphs = []
            cap = torch.cuda.Stream()
            for j in range(n_graphs):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cap):
                    run(G, stream_handle=ctypes.c_void_p(cap.cuda_stream), start=j * G)
                graphs.append(g)
            for g in graphs:
                g.replay()
            torch.cuda.synchronize()
            t_start = time.perf_counter()
            for i in range(K // G):
                graphs[i % n_graphs].replay()
            torch.cuda.synchronize()
            graph_us = (time.perf_counter() - t_start) / K * 1e6
            # spread: 64 replays of graphs of 8 steps (independent of K), events
            # around each replay
            G8 = 8
            sg = []
            for j in range(8):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cap):
                    run(G8, stream_handle=ctypes.c_void_p(cap.cuda_stream), start=j * G8)
                sg.append(g)
            for g in sg:
                g.replay()
            torch.cuda.synchronize()
            reps = 64
            evr = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(reps)]
            for i, (a, b) in enumerate(evr):
                a.record(stream)
                sg[i % len(sg)].replay()
                b.record(stream)
            torch.cuda.synchronize()
            per = np.array([a.elapsed_time(b) for a, b in evr]) * 1e3 / G8
            graph_spread = {"replays": reps, "steps_per_replay": G8,
                            "p10": round(float(np.percentile(per, 10)), 3),
                            "p50": round(float(np.percentile(per, 50)), 3),
                            "p90": round(float(np.percentile(per, 90)), 3)}
            del sg
        except Exception as exc:  # a launch the graph capture does not take
            torch.cuda.synchronize()
            log(f"graph capture unavailable ({type(exc).__name__}: {exc}); timing stream launches")
            G = 0
            graph_us = None

    # 2. plain stream launches, events bracketing the timed region
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    ev0.record(stream)
    run(K)
    ev1.record(stream)
    torch.cuda.synchronize()
    stream_us = (time.perf_counter() - t_start) / K * 1e6
    region_us = ev0.elapsed_time(ev1) * 1e3 / K
    us_per_token = graph_us if graph_us is not None else stream_us

    # 3. instrumented pass: kernel timestamps of the gate/up and down kernels
    kernels_us = {}
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    for e4 in evs:
        for e in e4:
            e.record(stream)
    torch.cuda.synchronize()
    probes = []
    for e4 in evs:
        p = moe.Probe()
        p.ev_gateup[0], p.ev_gateup[1] = e4[0].cuda_event, e4[1].cuda_event
        p.ev_down[0], p.ev_down[1] = e4[2].cuda_event, e4[3].cuda_event
        probes.append(ctypes.byref(p))
        e4.append(p)  # keep the struct alive
    torch.cuda.synchronize()
    run(K, probes)
    torch.cuda.synchronize()
    gu = np.array([e4[0].elapsed_time(e4[1]) for e4 in evs]) * 1e3  # us
    dn = np.array([e4[2].elapsed_time(e4[3]) for e4 in evs]) * 1e3
    gu_avg, dn_avg = float(gu.mean()), float(dn.mean())
    kname, kbytes, k_us = "decode_b_kernel", PHASE_B_BYTES, gu_avg
    kernels_us["phase_b_routed_gateup_shared_down"] = round(gu_avg, 3)
    kernels_us["phase_c_routed_down_combine"] = round(dn_avg, 3)
    log(f"graph {graph_us} us/token (G={G}); stream {stream_us:.2f} "
        f"(events {region_us:.2f}); "
        f"phase B {gu_avg:.2f} us ({PHASE_B_BYTES / gu_avg / 1e3:.0f} GB/s); "
        f"phase C {dn_avg:.2f} us ({PHASE_C_BYTES / dn_avg / 1e3:.0f} GB/s)")
    achieved = kbytes / (k_us * 1e-6) / 1e9
    log(f"layer {LAYER_TOKEN_BYTES / us_per_token / 1e3:.0f} GB/s")

    probe = hbm_read_probe()
    log(f"read probe {probe['GBps']} GB/s")

    secondary = None
    if not args.no_secondary:
        secondary = {}
        try:
            secondary["topp_decode"] = bench_topp(layers, x)
        except Exception as exc:  # reported, the headline line is still printed
            secondary["topp_decode"] = {"error": f"{type(exc).__name__}: {exc}"}
        try:
            secondary["shared_int8_decode"] = bench_shared_i8(layers, x)
        except Exception as exc:
            secondary["shared_int8_decode"] = {"error": f"{type(exc).__name__}: {exc}"}
        for key, fn in (("verify_64_zipf", bench_verify), ("prefill_2048", bench_prefill),
                        ("tiered_decode", bench_tiered), ("expert_weight_formats", bench_fmt8)):
            try:
                secondary[key] = fn(layers[0])
            except Exception as exc:  # reported, the headline line is still printed
                secondary[key] = {"error": f"{type(exc).__name__}: {exc}"}
        del layers, lstructs, lrefs, ws
        gc.collect()
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        try:
            secondary["stack48_decode"] = bench_stack()
        except Exception as exc:
            secondary["stack48_decode"] = {"error": f"{type(exc).__name__}: {exc}"}
        try:
            secondary["mla_decode"] = bench_mla()
        except Exception as exc:
            secondary["mla_decode"] = {"error": f"{type(exc).__name__}: {exc}"}

    layer_gbps = LAYER_TOKEN_BYTES / (us_per_token * 1e-6) / 1e9
    rec = {
        "metric": "MoE layer decode us/token + achieved HBM GB/s (frac of peak); prefill TOPS",
        "value": round(us_per_token, 3),
        "unit": "us/token",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(us_per_token / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4xint8->int32, f32 epilogue",
        "data": "synthetic (seeded N(0,0.02) weights packed to int4, N(0,1) activations)",
        "config": {"workload": "GLM-shape MoE layer decode, 1 token/step (hidden 6144, 256 "
                               "experts top-8 + 1 shared, int4 experts 2048x6144)",
                   "global_batch": 1, "layer_replicas": R, "distinct_tokens": T},
        "tokens_per_s": round(1e6 / us_per_token, 1),
        "timing": (f"HIP graph replay, {G} steps per graph" if G else "stream launches"),
        "us_per_token_spread": graph_spread,
        "stream_us_per_token": round(stream_us, 3),
        "layer_bytes_per_token": LAYER_TOKEN_BYTES,
        "layer_GBps": round(layer_gbps, 1),
        "layer_frac_of_hbm_peak": round(layer_gbps / HBM_PEAK_GBPS, 4),
        "hbm_read_probe": probe,
        "layer_frac_of_read_probe": round(layer_gbps / probe["GBps"], 4),
        "kernels_us": kernels_us,
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": measured_traffic(kname),
                     "bytes_per_launch": kbytes},
        "cpu_baseline": cpu,
        "secondary": secondary,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
