"""Benchmark of the MoE layer forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config NAME] [--also NAME,...]

A step is one moe_forward call (router GEMM, top-k, dispatch, grouped-GEMM
experts + shared expert, combine) over one batch of seeded synthetic tokens
resident in HBM. The headline workload is the whole 256-expert DeepSeek-V3
layer at prefill shape (16384 tokens, bf16), where the grouped GEMM is bound
by the matrix cores; the same line carries a second measured block for the
decode shape (512 tokens), where it is bound by streaming the expert weights.
Prints one JSON line with tokens/s, the roofline of the dominant kernel
(measured with HIP events over the timed steps) and the CPU oracle timed on a
bounded sample of the headline workload.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/sec at 1 GPU; grouped-GEMM % MFMA peak / % HBM GB/s"
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0        # dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0
PEAK_F32_TFLOPS = 157.3          # fp32 MFMA/vector


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="full_prefill_bf16")
    ap.add_argument("--also", default="full_decode_bf16",
                    help="comma-separated workloads measured after the headline one and reported in the same "
                         "line under 'also' ('none' for none)")
    ap.add_argument("--out-dtype", default="bf16", choices=["bf16", "f32"])
    ap.add_argument("--cpu-sample", type=int, default=1024, help="tokens of the oracle's timed sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-packed", action="store_true",
                    help="bf16: run without the prepacked weight copy (the 256 x 256 tiles then read the "
                         "canonical weights through LDS)")
    ap.add_argument("--graph", action="store_true",
                    help="capture the timed steps in one HIP graph and replay it (no launch gaps)")
    ap.add_argument("--diag-steps", type=int, default=10,
                    help="untimed steps with events around every stage, for the per-stage breakdown")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the achievable-peak yardsticks (MFMA loop, device copy)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="instead of the layer, run a plain device copy of MIB MiB 5 times (the reference "
                         "kernel that scales the FETCH_SIZE / WRITE_SIZE counters to bytes)")
    return ap.parse_args()


# Kernel sources whose code a stored traffic measurement belongs to.
KERNEL_SOURCES = {"bf16": ["gemm.hip", "gemm_big.hip", "gemm_pf.hip", "gemm_cores.hip", "gemm_tile.h", "moe_internal.h", "moe_device.h"],
                  "f32": ["gemm.hip", "gemm_tile.h", "moe_internal.h", "moe_device.h"],
                  "fp8": ["gemm_fp8.hip", "gemm_tile.h", "moe_internal.h", "moe_device.h"],
                  "mxfp4": ["gemm_mx.hip", "gemm_tile.h", "moe_internal.h", "moe_device.h"]}


def _code_only(text):
    """The source with its comments removed and blank runs collapsed, so that
    the hash follows the code and not the comments (string and character
    literals are kept as they are)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            while i < n and text[i] != "\n":
                i += 1
        elif text.startswith("/*", i):
            k = text.find("*/", i + 2)
            i = n if k < 0 else k + 2
        else:
            out.append(c)
            i += 1
    return re.sub(r"\s+", " ", "".join(out)).strip()


def kernel_source_hash(dtype):
    """Hash of the code (comments excluded) of the sources a kernel is built from."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[dtype]:
        with open(os.path.join(ROOT, "mixture_experts_layer_10_amd", "csrc", f)) as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def stored_traffic(stage, workload, dtype):
    """HBM bytes per launch of `stage` from the committed counter summary
    (profiles/<stage>_<workload>_hbm_traffic.md), or None when there is none
    or the kernel's sources have changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{stage}_{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        text = fh.read()
    m = re.search(r"^traffic_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    hsh = re.search(r"^kernel_source_sha256:\s*([0-9a-f]+)", text, re.M)
    if not m or not hsh or hsh.group(1) != kernel_source_hash(dtype):
        return None
    return float(m.group(1))


def calibrate_copy(mib):
    """A plain copy kernel of known size: dst = src * 1 over `mib` MiB of
    float32, six times (the first untimed); each launch reads and writes
    exactly mib MiB."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.mul(src, 1.0, out=dst)                     # warm-up launch (not counted below)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(5):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / 5
    print(json.dumps({"copy_bytes_read_per_launch": n * 4, "copy_bytes_written_per_launch": n * 4,
                      "launches": 6, "copy_gbs_read_plus_write": 2 * n * 4 / dt / 1e9}), flush=True)


def achievable_peaks():
    """Yardsticks measured on this device, beside the spec peaks: the bf16
    matrix-core rate of a loop of independent MFMAs on every SIMD (no memory
    traffic) with the shader clock it ran at, the rate at which a plain
    coalesced read streams 4 GiB in from HBM, and the read + write rate of a
    device copy of 2 GiB (torch's copy kernel). Medians of 3 timed launches
    after one untimed one."""
    import torch
    from mixture_experts_layer_10_amd import mfma_loop, stream_read
    out = torch.zeros(3, dtype=torch.int64, device="cuda")
    mfma_loop(20000, out)
    rates, clocks = [], []
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        flops = mfma_loop(300000, out)
        e1.record()
        e1.synchronize()
        rates.append(flops / (e0.elapsed_time(e1) * 1e-3) / 1e12)
        ticks, rt = out[:2].tolist()
        clocks.append(ticks / rt * 100.0)
    buf = torch.ones(1 << 30, dtype=torch.float32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream_read(buf, sink)
    rd = []
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        nb = stream_read(buf, sink)
        e1.record()
        e1.synchronize()
        rd.append(nb / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del buf
    n = (2 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    gbs = []
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        e1.synchronize()
        gbs.append(2 * n * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del src, dst
    return {"mfma_loop_bf16_tflops": float(np.median(rates)), "mfma_loop_sclk_mhz": float(np.median(clocks)),
            "stream_read_gbs": float(np.median(rd)), "copy_gbs": float(np.median(gbs))}


def stage_bytes_flops(w, counts, stage):
    """Algorithmic HBM bytes and FLOPs of one launch of `stage`.

    GroupGEMM I/O model g*(m*k + n*k + m*n) elements and 2*g*m*k*n FLOPs
    (Perplexity, "Roofline > GroupGEMM"), with m_i the rows of expert i, only
    experts with rows counted, each term at its stored element size:
    weights wb bytes per element (fp8: 1, the 128x128 block scales
    negligible; mxfp4: half a byte plus one scale byte per 32), quantised
    activations ab (e4m3 plus a 4-byte scale per 128 or a 1-byte scale per
    32: 1 + 1/32 either way), expert output rows bf16 (fp32 for f32)."""
    H, I, Is, T = w["hidden"], w["inter"], w["shared_inter"], w["T"]
    wb = {"bf16": 2, "f32": 4, "fp8": 1, "mxfp4": 0.5 + 1 / 32}[w["dtype"]]
    ab = {"bf16": 2, "f32": 4, "fp8": 1 + 1 / 32, "mxfp4": 1 + 1 / 32}[w["dtype"]]
    ob = 4 if w["dtype"] == "f32" else 2
    R = int(counts.sum())
    active = int((counts > 0).sum())
    if stage == "gate_up":
        return (R * H + R * I) * ab + active * 2 * I * H * wb, 2.0 * R * H * 2 * I
    if stage == "down":
        return R * I * ab + active * H * I * wb + R * H * ob, 2.0 * R * I * H
    if stage == "shared_gate_up":
        return (T * H + T * Is) * ab + 2 * Is * H * wb, 2.0 * T * H * 2 * Is
    if stage == "shared_down":
        return T * Is * ab + H * Is * wb + T * H * 4, 2.0 * T * Is * H
    raise ValueError(stage)


def cpu_baseline(w, inp, sample, min_seconds=10.0):
    """The oracle as it stands, timed on the first `sample` tokens of the
    batch (a batch of its own: router GEMM, top-k, dispatch, one expert at a
    time, shared expert, combine), in passes repeated until at least
    `min_seconds` have elapsed. Its matmuls run in float32 (BLAS), the
    arithmetic type a CPU implementation of the bf16 layer would use; the
    weights are made resident in host memory as float32 beforehand (untimed,
    one expert at a time from the device)."""
    import platform
    import torch
    from oracle import moe_oracle as O

    def h(t):
        if t is None:
            return None
        if t.dtype == torch.float8_e4m3fn:
            return t.detach().cpu().view(torch.uint8).numpy()
        if t.dtype == torch.uint8:
            return t.detach().cpu().numpy()
        return t.detach().float().cpu().numpy()

    def experts(t):
        return None if t is None else [h(t[e]) for e in range(t.shape[0])]

    cfg = O.Config.from_workload(w)
    S = min(sample, w["T"])
    x = h(inp["x"][:S])
    args = dict(router_bias=h(inp["router_bias"]), score_bias=h(inp["score_bias"]),
                shared_w13=h(inp["shared_w13"]), shared_w2=h(inp["shared_w2"]))
    scales = {k: h(inp.get(k)) for k in ("w13_scale", "w2_scale", "shared_w13_scale", "shared_w2_scale")}
    wr, w13, w2 = h(inp["w_router"]), experts(inp["w13"]), experts(inp["w2"])
    passes = 0
    t0 = time.perf_counter()
    while True:
        O.forward(cfg, x, wr, w13, w2, scales=scales, work=np.float32, **args)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    cores = len(os.sched_getaffinity(0))
    # the BLAS libraries the oracle's matmuls loaded, and their thread pools
    # (queried after the passes, once the libraries are loaded)
    try:
        from threadpoolctl import threadpool_info
        blas = [{"api": d.get("internal_api"), "version": d.get("version"), "threads": d.get("num_threads")}
                for d in threadpool_info() if d.get("user_api") == "blas"]
    except Exception:
        blas = []
    blas_threads = max([b["threads"] or 1 for b in blas] or [0])
    cpu = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as fh:
            cpu = next(l.split(":", 1)[1].strip() for l in fh if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    del w13, w2
    return {"value": passes * S / dt, "unit": "tokens/s", "cores": blas_threads or cores, "kind": "oracle",
            "sample": f"first {S} of {w['T']} tokens of the {w['name']} workload as a batch of their own, whole "
                      f"layer (router GEMM, top-k, dispatch, every local expert, shared expert, combine), float32 "
                      f"BLAS matmuls, {passes} passes in {dt:.1f} s wall",
            "affinity_cores": cores, "cpu": cpu, "blas": blas}


def measure(name, a, peaks=None):
    """Time moe_forward on workload `name`: tokens/s over the timed steps, the
    dominant kernel's roofline from HIP events over those steps, the grouped
    GEMM's fractions and a per-stage breakdown from an untimed pass.
    Returns (result dict, inputs)."""
    import torch
    import mixture_experts_layer_10_amd as moe
    from synth import make_inputs, workload

    w = workload(name)
    T = w["T"]
    print(f"[bench] workload {name}: T={T} H={w['hidden']} E={w['n_experts']} "
          f"local=[{w['expert_begin']},{w['expert_end']}) dtype={w['dtype']}", file=sys.stderr, flush=True)
    inp = make_inputs(w, device="cuda")
    cfg = moe.config_from_workload(w, out_dtype=a.out_dtype)
    W = moe.make_weights(cfg, inp["w13"], inp["w2"], inp["shared_w13"], inp["shared_w2"], inp.get("w13_scale"),
                         inp.get("w2_scale"), inp.get("shared_w13_scale"), inp.get("shared_w2_scale"))
    packed = None
    if w["dtype"] == "bf16" and not a.no_packed:
        # the prepacked copy (once, untimed): the layer's 256 x 256 tiles
        # stream their weights from it
        packed = moe.moe_prepack_weights(cfg, W)
        W = moe.make_weights(cfg, inp["w13"], inp["w2"], inp["shared_w13"], inp["shared_w2"], packed=packed)
    ws = moe.workspace(cfg, T)
    y = torch.empty(T, w["hidden"], dtype=torch.bfloat16 if a.out_dtype == "bf16" else torch.float32,
                    device="cuda")
    ids = torch.empty(T, w["top_k"], dtype=torch.int32, device="cuda")

    def step():
        moe.moe_forward(cfg, inp["x"], inp["w_router"], inp["router_bias"], inp["score_bias"], W, y, ws,
                        topk_ids_out=ids)

    # The dominant kernel: the routed experts' gate/up grouped GEMM (the
    # largest share of the layer's bytes and FLOPs in every workload). In the
    # timed region only it is bracketed by HIP events (on the stream it runs
    # on); the per-stage breakdown comes from a separate untimed pass.
    dom = "gate_up"
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    moe.profile_select([dom])
    moe.profile_enable(0 if a.graph else a.steps + 16)
    graph = None
    if a.graph:
        # events recorded inside a graph cannot be timed: with --graph the
        # dominant kernel's time comes from the untimed per-stage pass
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(a.steps):
                step()
        torch.cuda.synchronize()
        graph.replay()                      # one untimed replay
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graph is not None:
        graph.replay()
    else:
        for _ in range(a.steps):
            step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    dom_ms, dom_n = moe.profile_query()[dom] if graph is None else (0.0, 0)
    ms = (t1 - t0) * 1e3 / a.steps
    value = T / (ms * 1e-3)

    moe.profile_select(None)
    moe.profile_enable(a.diag_steps * len(moe.STAGES) + 16)
    moe.profile_reset()
    for _ in range(a.diag_steps):
        step()
    torch.cuda.synchronize()
    prof = moe.profile_query()
    moe.profile_enable(0)

    # per-step times: a separate pass with an event between steps (kept out
    # of the timed region, which has no events between steps)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps + 1)]
    evs[0].record()
    for i in range(a.steps):
        step()
        evs[i + 1].record()
    evs[-1].synchronize()
    per_step = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(a.steps)])
    step_pct = {"median": float(np.median(per_step)), "p10": float(np.percentile(per_step, 10)),
                "p90": float(np.percentile(per_step, 90)), "source": "separate pass, an event between steps"}
    graphed = graph is not None
    del graph

    ids_h = ids.cpu().numpy().reshape(-1)
    loc = ids_h[(ids_h >= w["expert_begin"]) & (ids_h < w["expert_end"])] - w["expert_begin"]
    counts = np.bincount(loc, minlength=w["expert_end"] - w["expert_begin"])
    if w["capacity_factor"] > 0:
        import math
        cap = math.ceil(float(np.float32(w["capacity_factor"])) * T * w["top_k"] / w["n_experts"])
        counts = np.minimum(counts, cap)

    stage_ms = {k: (v[0] / v[1] if v[1] else 0.0) for k, v in prof.items()}
    byts, flops = stage_bytes_flops(w, counts, dom)
    if graphed:
        dom_ms, dom_n = prof[dom]
    t_dom = dom_ms / dom_n * 1e-3
    # e4m3 x E2M1 runs at the fp8 rate of the scaled MFMA
    peak_mfma = {"bf16": PEAK_BF16_TFLOPS, "fp8": PEAK_FP8_TFLOPS, "mxfp4": PEAK_FP8_TFLOPS,
                 "f32": PEAK_F32_TFLOPS}[w["dtype"]]
    ridge = peak_mfma * 1e12 / (PEAK_HBM_GBS * 1e9)
    if flops / byts < ridge:
        roof = {"bound": "hbm", "achieved": byts / t_dom / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": flops / t_dom / 1e12, "peak": peak_mfma, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = stored_traffic(dom, name, w["dtype"])
    family = {"fp8": "gemm_fp8_kernel", "mxfp4": "gemm_mx_kernel"}.get(
        w["dtype"], "gemm_kernel / gemm_pf_kernel" if packed is not None else "gemm_kernel / gemm_big_kernel")
    roof["kernel"] = f"{family} ({dom})"
    roof["kernel_ms"] = t_dom * 1e3
    roof["kernel_launches_timed"] = dom_n
    roof["kernel_time_source"] = "untimed per-stage pass" if graphed else "timed region"
    roof["algorithmic_bytes"] = byts
    roof["algorithmic_flops"] = flops

    # grouped GEMM as a whole (routed gate/up + down): both roofline fractions
    gb, gf = 0.0, 0.0
    for s in ("gate_up", "down"):
        b_, f_ = stage_bytes_flops(w, counts, s)
        gb += b_
        gf += f_
    gt = (stage_ms["gate_up"] + stage_ms["down"]) * 1e-3
    grouped = {"ms": gt * 1e3, "hbm_frac": gb / gt / 1e9 / PEAK_HBM_GBS,
               "mfma_frac": gf / gt / 1e12 / peak_mfma}
    if peaks:
        grouped["hbm_frac_of_stream_read"] = gb / gt / 1e9 / peaks["stream_read_gbs"]
        if w["dtype"] == "bf16":
            grouped["mfma_frac_of_loop"] = gf / gt / 1e12 / peaks["mfma_loop_bf16_tflops"]
        if roof["unit"] == "GB/s":
            roof["frac_of_stream_read"] = roof["achieved"] / peaks["stream_read_gbs"]
        elif w["dtype"] == "bf16":
            roof["frac_of_mfma_loop"] = roof["achieved"] / peaks["mfma_loop_bf16_tflops"]

    # expert load of this batch over all routed experts (device counts),
    # and how an 8-GPU expert-parallel placement would balance it
    load = torch.zeros(w["n_experts"], dtype=torch.int64, device="cuda")
    moe.moe_expert_load(cfg, ids, load)
    lc = load.cpu()
    per = w["n_experts"] // 8
    contig = lc.view(8, per).sum(1).double()
    expert_load = {"hottest": int(lc.max()), "coldest": int(lc.min()), "mean": float(lc.double().mean()),
                   "ep8_contiguous_imbalance": float(contig.max() / contig.mean()),
                   "ep8_replanned_imbalance": moe.moe_eplb_plan(lc, 8, 0)[3],
                   "ep8_replanned_8_redundant_imbalance": moe.moe_eplb_plan(lc, 8, 8)[3]}
    res = {
        "value": value, "unit": "tokens/s", "steps": a.steps, "warmup": a.warmup, "ms_per_step": ms,
        "dtype": w["dtype"],
        "config": {"workload": name, "tokens": T, "hidden": w["hidden"], "experts": w["n_experts"],
                   "local_experts": [w["expert_begin"], w["expert_end"]], "top_k": w["top_k"],
                   "inter": w["inter"], "shared_inter": w["shared_inter"], "out_dtype": a.out_dtype,
                   "packed_weights": packed is not None},
        "roofline": roof, "grouped_gemm": grouped, "stage_ms": stage_ms, "step_ms": step_pct,
        "rows": int(counts.sum()), "max_rows_per_expert": int(counts.max()), "expert_load": expert_load,
    }
    del W, ws, y, packed
    return res, (w, inp)


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU: --gpus {a.gpus} is not supported "
              "(the layer runs one GPU's share of experts; no collectives).", file=sys.stderr)
        sys.exit(2)
    if a.calibrate_copy:
        calibrate_copy(a.calibrate_copy)
        return
    import torch

    peaks = None if a.no_peaks else achievable_peaks()
    head, (w, inp) = measure(a.config, a, peaks)
    out = {"metric": METRIC, "value": head["value"], "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
           "warmup": a.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": head["dtype"], "data": "synthetic", "config": head["config"]}
    for key in ("roofline", "grouped_gemm", "stage_ms", "step_ms", "rows", "max_rows_per_expert", "expert_load"):
        out[key] = head[key]
    out["achievable"] = peaks
    if not a.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, inp, a.cpu_sample)
    del inp
    torch.cuda.empty_cache()
    also = [n for n in a.also.split(",") if n and n != "none" and n != a.config]
    if also:
        out["also"] = {}
        for n in also:
            res, (_, inp2) = measure(n, a, peaks)
            del inp2
            torch.cuda.empty_cache()
            out["also"][n] = res
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
