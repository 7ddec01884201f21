"""Throughput of the fused-linear generalized-JSD pass (forward + backward) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--num-chunks NC]

A step is one fljsd_forward_backward call over the 8192-row workload at the
Llama-3-8B lm_head shape (H = 4096, V = 128256, bf16, beta = 0.5, T = 2,
batchmean): both logits GEMMs, the three loss passes, grad_input and grad_W.
Inputs are seeded synthetic draws (workloads.py), resident in HBM before the
timed region; outputs and the workspace are preallocated. One JSON line on
stdout; progress goes to stderr.

Fields beyond the throughput:
  roofline      the kernel class with the most time: algorithmic flops (or
                bytes) per launch over its average launch time, from HIP
                events the library records around each launch during the
                timed steps, against MI355X's published peak.
  kernels       the same tally for every kernel class.
  jsd_*         the loss passes (statistics merge, pass 2, pass 3): algorithmic
                GB/s, the pages' three-pass byte count (7·V·s per row) over
                their time, the compulsory bytes (3·V·s) at 8 TB/s over their
                time, and HBM GB/s from the counter summary
                (profiles/traffic.json, current sources only).
  mfma_util_counter / mfma_counters
                matrix-core utilisation of the three products from rocprofv3
                counters (profiles/mfma.json, used only when it was taken with
                the current sources): busy fraction at the held clock, and
                counted matrix flops against the nominal peak.
  sweep         the 1024- and 8192-row workloads at 1, 8 and 32 chunks: ms,
                tokens/s, peak HBM of the pass and its roofline floor (each
                kernel class at the larger of its bytes at 8 TB/s and its
                flops at 2.5 PFLOP/s); small chunks are bound by weight and
                grad_W read-add-write traffic.
  cpu_baseline  the CPU oracle (numpy fp64) timed on the first rows of the
                same workload, in tokens/s, on all host threads.
  oracle_one_thread
                the oracle on one thread over the three small workloads.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fused-linear-JSD fwd+bwd tokens/s at H=4096,V=128256 bf16; MFMA util"
WORKLOAD = "large_batch"
# The pages' H100 80GB figure for this workload (B*T = 8192, num_chunks = 1,
# H = 4096, V = 128256, bf16): 60.62 ms per full pass, i.e. 135,137 tokens/s.
PAGES_TOKENS_PER_S = 8192 / 60.62e-3
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
GEMM_CLASSES = ("gemm_logits", "gemm_grad_input", "gemm_grad_weight")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CLOCK_FILE = os.path.join(ROOT, "profiles", "clock.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--num-chunks", type=int, default=0,
                   help="0: the library's policy for the free HBM (one chunk on 288 GB)")
    p.add_argument("--cpu-rows", type=int, default=2048,
                   help="rows of the workload the CPU oracle is timed on")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-sweep", action="store_true",
                   help="skip the 1024- and 8192-row workloads at 1, 8 and 32 chunks")
    p.add_argument("--no-oracle-1thread", action="store_true",
                   help="skip the one-thread oracle times of the three small workloads")
    p.add_argument("--flce", action="store_true",
                   help="also time the fused-linear cross-entropy at 1024..8192 rows")
    p.add_argument("--losses", action="store_true",
                   help="also time the one-pass TVD and log-probability JSD at 4096 x 32000 bf16")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run three plain 1 GiB device copies (the reference for scaling "
                        "the FETCH_SIZE / WRITE_SIZE counters) and exit")
    return p.parse_args()


def copy_calibration():
    """Three device-to-device copies of 1 GiB: under `rocprofv3 --pmc FETCH_SIZE`
    (or WRITE_SIZE) the counter per copy, against the 1 GiB it moves each way,
    gives the factor that turns the counter into bytes."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"copied {n} bytes three times")


def device_inputs(inp):
    import numpy as np
    import torch
    return [torch.from_numpy(inp[k].view(np.int16)).view(torch.bfloat16).cuda()
            for k in ("X_s", "W_s", "X_t", "W_t")]


def roofline_of(cls, k):
    """Achieved rate of one kernel class: algorithmic work per launch over the
    average launch time."""
    avg_s = k["ms"] / 1e3 / k["launches"]
    if cls in GEMM_CLASSES:
        per_launch = k["flops"] / k["launches"]
        return {"bound": "mfma", "achieved": per_launch / avg_s / 1e12, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "per_launch": per_launch, "avg_launch_ms": avg_s * 1e3}
    per_launch = k["bytes"] / k["launches"]
    return {"bound": "hbm", "achieved": per_launch / avg_s / 1e9, "peak": PEAK_HBM_GBPS,
            "unit": "GB/s", "per_launch": per_launch, "avg_launch_ms": avg_s * 1e3}


def _profile_entry(path, cls):
    """The entry for a kernel class in a counter summary under profiles/, if
    it was taken with the current kernel sources; else None."""
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get("kernels", {}).get(cls)
    if not entry:
        return None
    from lm_head_distillation_amd.build import source_digest
    if entry.get("source_digest") != source_digest():
        return None
    return entry


def traffic_for(cls):
    """Measured HBM bytes per launch for a kernel class (rocprofv3 FETCH_SIZE
    and WRITE_SIZE, copy-calibrated), or None."""
    entry = _profile_entry(TRAFFIC_FILE, cls)
    return entry.get("hbm_bytes_per_launch") if entry else None


def clock_for(cls):
    """Shader clock (MHz) a kernel class ran at (rocprofv3 GRBM_GUI_ACTIVE per
    dispatch over the traced durations), or None."""
    entry = _profile_entry(CLOCK_FILE, cls)
    return entry.get("clock_mhz") if entry else None


def pass_floor(kernels, steps):
    """Roofline floor of one pass from the library's per-class tallies: each
    kernel class is bound by the larger of its algorithmic bytes at the HBM
    peak and its flops at the bf16 matrix peak; the pass's floor is the sum
    (the kernels run one after another). Returns ms per step:
    (floor, all bytes at the HBM peak, all flops at the matrix peak)."""
    floor = hbm = mfma = 0.0
    for k in kernels.values():
        if not k["launches"]:
            continue
        t_hbm = k["bytes"] / (PEAK_HBM_GBPS * 1e9) * 1e3 / steps
        t_mfma = k["flops"] / (PEAK_BF16_TFLOPS * 1e12) * 1e3 / steps
        floor += max(t_hbm, t_mfma)
        hbm += t_hbm
        mfma += t_mfma
    return floor, hbm, mfma


MFMA_FILE = os.path.join(ROOT, "profiles", "mfma.json")


def mfma_counters():
    """Matrix-core utilisation of the three products from rocprofv3 counters
    (the committed summary, if it was taken with the current sources): the
    busy fraction of the matrix cores over the cycles the kernel ran
    (SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x SIMDs), at the clock the
    chip held) and the counted bf16 matrix flops (SQ_INSTS_VALU_MFMA_MOPS_BF16
    x 512) over the traced kernel time against the nominal 2.5 PFLOP/s."""
    out = {}
    for cls in GEMM_CLASSES:
        entry = _profile_entry(MFMA_FILE, cls)
        if entry:
            out[cls] = {k: entry[k] for k in ("mfma_busy_frac", "frac_nominal", "counted_flops_per_launch",
                                              "avg_ms", "launches_per_pass", "clock_mhz") if k in entry}
    if len(out) != len(GEMM_CLASSES):
        return {}
    # The three products together, weighted by their time in one pass.
    ms = sum(e["avg_ms"] * e["launches_per_pass"] for e in out.values())
    flops = sum(e["counted_flops_per_launch"] * e["launches_per_pass"] for e in out.values())
    busy = sum(e["mfma_busy_frac"] * e["avg_ms"] * e["launches_per_pass"] for e in out.values())
    out["gemms"] = {"mfma_busy_frac": round(busy / ms, 4),
                    "frac_nominal": round(flops / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    return out


def sweep(fljsd, steps, warmup, large_batch_dev):
    """ms per step, tokens/s, peak HBM and roofline floor of the two
    H=4096, V=128256 workloads (1024 and 8192 rows) per chunk count."""
    import torch

    import workloads
    out = []
    for key in ("llama3_head", "large_batch"):
        w = workloads.WORKLOADS[key]
        if key == "large_batch":
            X_s, W_s, X_t, W_t = large_batch_dev
        else:
            X_s, W_s, X_t, W_t = device_inputs(workloads.make_inputs(w))
        in_bytes = sum(t.numel() * t.element_size() for t in (X_s, W_s, X_t, W_t))
        for nc in (1, 8, 32):
            # Peak HBM of the pass: its inputs, outputs and workspace (buffers
            # other parts of this run still hold are left out).
            base = torch.cuda.memory_allocated()
            ws = torch.empty(fljsd.fljsd_workspace_size(w.BT, w.H_s, w.H_t, w.V, fljsd.BF16, nc),
                             dtype=torch.uint8, device="cuda")
            out_t = (torch.empty(1, dtype=torch.float32, device="cuda"), torch.empty_like(X_s),
                     torch.empty_like(W_s))
            torch.cuda.reset_peak_memory_stats()

            def step():
                fljsd.fljsd_forward_backward(X_s, W_s, X_t, W_t, w.beta, w.temperature,
                                             w.reduction, nc, workspace=ws, out=out_t)
            for _ in range(warmup):
                step()
            torch.cuda.synchronize()
            fljsd.fljsd_profile_enable(True)
            t0 = time.perf_counter()
            for _ in range(steps):
                step()
            torch.cuda.synchronize()
            ms = (time.perf_counter() - t0) / steps * 1e3
            kernels = fljsd.fljsd_profile_read()
            fljsd.fljsd_profile_enable(False)
            floor, hbm, mfma = pass_floor(kernels, steps)
            alg_bytes = sum(k["bytes"] for k in kernels.values()) / steps
            rec = {"workload": key, "BT": w.BT, "num_chunks": nc, "ms_per_step": round(ms, 3),
                   "tokens_per_s": round(w.BT / ms * 1e3, 1),
                   "peak_hbm_mb": round((torch.cuda.max_memory_allocated() - base + in_bytes) / 2**20, 1),
                   "workspace_mb": round(ws.numel() / 2**20, 1),
                   "alg_hbm_gb": round(alg_bytes / 1e9, 2),
                   "hbm_floor_ms": round(hbm, 3), "mfma_floor_ms": round(mfma, 3),
                   "floor_ms": round(floor, 3), "bound": "hbm" if hbm > mfma else "mfma",
                   "roofline_frac": round(floor / ms, 4),
                   "kernel_ms_per_step": {c: round(k["ms"] / steps, 3) for c, k in kernels.items()
                                          if k["launches"]}}
            log(f"  sweep {key:12s} nc={nc:2d}: {ms:8.2f} ms/step  {rec['tokens_per_s']:>10,.0f} tokens/s  "
                f"peak {rec['peak_hbm_mb']:.0f} MB  floor {floor:.2f} ms ({rec['bound']}, "
                f"{100 * floor / ms:.0f}%)  " +
                " ".join(f"{c}={v:.2f}" for c, v in rec["kernel_ms_per_step"].items()))
            out.append(rec)
            del ws, out_t
        del X_s, W_s, X_t, W_t
        torch.cuda.empty_cache()
    return out


# The pages' H100 figures for the fused-linear cross-entropy after the
# grad_weight change (Liger-Kernel PR #1429, Details, default provider, bf16,
# reduction mean, H = 4096, V = 128256): ms per full pass by rows. Context only.
PAGES_FLCE_MS = {1024: 5.86, 2048: 9.75, 4096: 20.18, 8192: 37.34}


def flce_sweep(fljsd, steps, warmup):
    """ms per fwd+bwd pass of the fused-linear cross-entropy at the pages' sizes."""
    import numpy as np
    import torch

    import workloads
    H, V = 4096, 128256
    W = workloads.draw(1101, (V, H), workloads.SIGMA_W, "bf16")
    W = torch.from_numpy(W.view(np.int16)).view(torch.bfloat16).cuda()
    out = []
    for BT in (1024, 2048, 4096, 8192):
        X = workloads.draw(1100 + BT, (BT, H), workloads.SIGMA_X, "bf16")
        X = torch.from_numpy(X.view(np.int16)).view(torch.bfloat16).cuda()
        labels = torch.from_numpy(np.random.default_rng(BT).integers(0, V, size=BT)).cuda()
        nc = fljsd.fljsd_flce_plan_num_chunks(BT, H, V, fljsd.BF16, fljsd.default_budget_bytes())
        ws = torch.empty(fljsd.fljsd_flce_workspace_size(BT, H, V, fljsd.BF16, nc),
                         dtype=torch.uint8, device="cuda")
        torch.cuda.reset_peak_memory_stats()

        def step():
            fljsd.fljsd_flce_forward_backward(X, W, labels, -100, 0.0, "mean", nc, workspace=ws)
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        fljsd.fljsd_profile_enable(True)
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) / steps * 1e3
        kernels = fljsd.fljsd_profile_read()
        fljsd.fljsd_profile_enable(False)
        floor, hbm, mfma = pass_floor(kernels, steps)
        rec = {"BT": BT, "num_chunks": nc, "ms_per_step": round(ms, 3),
               "tokens_per_s": round(BT / ms * 1e3, 1),
               "peak_hbm_mb": round(torch.cuda.max_memory_allocated() / 2**20, 1),
               "floor_ms": round(floor, 3), "bound": "hbm" if hbm > mfma else "mfma",
               "roofline_frac": round(floor / ms, 4),
               "kernel_ms_per_step": {c: round(k["ms"] / steps, 3) for c, k in kernels.items()
                                      if k["launches"]},
               "pages_h100_ms": PAGES_FLCE_MS[BT]}
        log(f"  flce BT={BT:5d} nc={nc}: {ms:7.2f} ms/step  {rec['tokens_per_s']:>10,.0f} tokens/s  "
            f"peak {rec['peak_hbm_mb']:.0f} MB  floor {floor:.2f} ms ({rec['bound']}, "
            f"{100 * floor / ms:.0f}%)  (pages, H100: {PAGES_FLCE_MS[BT]} ms)  " +
            " ".join(f"{c}={v:.2f}" for c, v in rec["kernel_ms_per_step"].items()))
        out.append(rec)
        del X, ws, labels
        torch.cuda.empty_cache()
    return out


# The pages' H100 NVL figure for the TVD forward op at (4096, 32000) bf16
# (Liger-Kernel PR #1374, Details: 0.2337 ms before and after the fix).
PAGES_TVD_MS = 0.2337


def losses_timing(fljsd, steps, warmup):
    """ms per call and HBM rate of the one-pass losses at the pages' TVD shape."""
    import numpy as np
    import torch

    import workloads
    R, V = 4096, 32000
    out = []

    def rows(seed, logspace):
        z = workloads.draw(seed, (R, V), 2.0, "f32")
        z = torch.from_numpy(z).cuda()
        t = torch.log_softmax(z, dim=-1) if logspace else torch.softmax(z, dim=-1)
        return t.to(torch.bfloat16).contiguous()
    for name in ("tvd", "jsd_logprob"):
        a, b = rows(1201, name != "tvd"), rows(1202, name != "tvd")
        grad = torch.empty_like(a)
        ws = torch.empty(fljsd.fljsd_generalized_jsd_workspace_size(R, V, fljsd.BF16),
                         dtype=torch.uint8, device="cuda")
        if name == "tvd":
            call = lambda: fljsd.fljsd_tvd(a, b, "batchmean", grad=grad, workspace=ws)
        else:
            call = lambda: fljsd.fljsd_jsd_logprob(a, b, 0.5, "batchmean", grad=grad, workspace=ws)
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            call()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) / steps * 1e3
        gbps = 3.0 * R * V * 2 / (ms * 1e-3) / 1e9     # two rows read, the gradient written
        rec = {"loss": name, "shape": [R, V], "dtype": "bf16", "ms_per_call": round(ms, 4),
               "hbm_gbps_algorithmic": round(gbps, 1), "frac": round(gbps / PEAK_HBM_GBPS, 4)}
        if name == "tvd":
            rec["pages_h100_ms"] = PAGES_TVD_MS
        log(f"  {name:12s} {R}x{V} bf16: {ms:.4f} ms  {gbps:,.0f} GB/s ({100 * gbps / PEAK_HBM_GBPS:.1f}% of HBM)"
            + (f"  (pages, H100 NVL forward: {PAGES_TVD_MS} ms)" if name == "tvd" else ""))
        out.append(rec)
        del a, b, grad, ws
    torch.cuda.empty_cache()
    return out


def cpu_baseline(inp, w, rows):
    import numpy as np
    import threadpoolctl

    import oracle
    import workloads
    log(f"cpu baseline: oracle on the first {rows} rows (fp64 widening excluded from the time)")
    X_s = workloads.to_f64(inp["X_s"][:rows], "bf16")
    X_t = workloads.to_f64(inp["X_t"][:rows], "bf16")
    W_s = workloads.to_f64(inp["W_s"], "bf16")
    W_t = workloads.to_f64(inp["W_t"], "bf16")
    blas = [i for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
    threads = max([i.get("num_threads", 1) for i in blas] or [1])
    blas_name = ", ".join(f"{i.get('internal_api', '?')} {i.get('version') or ''}".strip()
                          for i in blas) or "no BLAS reported"
    t0 = time.perf_counter()
    oracle.fused_linear_jsd(X_s, W_s, X_t, W_t, w.beta, w.temperature, w.reduction, block_rows=256)
    dt = time.perf_counter() - t0
    del W_s, W_t
    return {"value": rows / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": (f"first {rows} of {w.BT} rows, full H={w.H_s} and V={w.V} weights, "
                       f"fp64 numpy ({blas_name}) on {cpu_model()}, {dt:.1f} s"),
            "seconds": dt}


def oracle_one_thread():
    """The oracle on one host thread over the three small workloads in full
    (tiny fp32, multi-block tail, ties): seconds and tokens/s each."""
    import threadpoolctl

    import oracle
    import workloads
    out = []
    with threadpoolctl.threadpool_limits(limits=1):
        for key in ("tiny_f32", "multiblock_tail", "ties_padded"):
            w = workloads.WORKLOADS[key]
            inp = workloads.make_inputs(w)
            args = [workloads.to_f64(inp[k], w.dtype) for k in ("X_s", "W_s", "X_t", "W_t")]
            t0 = time.perf_counter()
            oracle.fused_linear_jsd(*args, w.beta, w.temperature, w.reduction)
            dt = time.perf_counter() - t0
            out.append({"workload": f"{key}: BT={w.BT} H={w.H_s} V={w.V} {w.dtype}",
                        "seconds": round(dt, 3), "tokens_per_s": round(w.BT / dt, 2), "cores": 1})
            log(f"cpu oracle, one thread: {key:16s} {dt:8.3f} s  {w.BT / dt:10.1f} tokens/s")
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the pass "
              "runs on a single MI355X (rows would shard across GPUs with one all-reduce of "
              "grad_W, which is not built).", file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        log("no GPU visible")
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration()
        return

    import workloads
    from lm_head_distillation_amd import fljsd

    fljsd.load_library()
    w = workloads.WORKLOADS[WORKLOAD]
    t0 = time.perf_counter()
    inp = workloads.make_inputs(w)
    log(f"inputs drawn in {time.perf_counter() - t0:.1f} s")
    X_s, W_s, X_t, W_t = device_inputs(inp)
    BT, H, V = w.BT, w.H_s, w.V
    nc = args.num_chunks or fljsd.fljsd_plan_num_chunks(BT, H, w.H_t, V, fljsd.BF16,
                                                         fljsd.default_budget_bytes())
    ws = torch.empty(fljsd.fljsd_workspace_size(BT, H, w.H_t, V, fljsd.BF16, nc),
                     dtype=torch.uint8, device="cuda")
    loss = torch.empty(1, dtype=torch.float32, device="cuda")
    gX = torch.empty_like(X_s)
    gW = torch.empty_like(W_s)
    out = (loss, gX, gW)

    def step():
        fljsd.fljsd_forward_backward(X_s, W_s, X_t, W_t, w.beta, w.temperature, w.reduction, nc,
                                     workspace=ws, out=out)

    torch.cuda.reset_peak_memory_stats()
    for i in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done; num_chunks={nc}, workspace {ws.numel() / 2**20:.0f} MiB")

    fljsd.fljsd_profile_enable(True)
    # Events between the steps (on the stream the library launches on) give
    # the spread of single steps; the throughput is the whole timed region.
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    marks[0].record()
    for i in range(args.steps):
        step()
        marks[i + 1].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    step_ms = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps))
    kernels = fljsd.fljsd_profile_read()
    fljsd.fljsd_profile_enable(False)
    ms_per_step = elapsed / args.steps * 1e3
    tokens_per_s = BT * args.steps / elapsed
    peak_mb = torch.cuda.max_memory_allocated() / 2**20
    log(f"timed {args.steps} steps: {ms_per_step:.2f} ms/step, {tokens_per_s:,.0f} tokens/s, "
        f"loss {float(loss):.6f}")

    per_class = {}
    for cls, k in kernels.items():
        if k["launches"]:
            r = roofline_of(cls, k)
            r["ms_per_step"] = k["ms"] / args.steps
            r["launches_per_step"] = k["launches"] / args.steps
            per_class[cls] = r
            log(f"  {cls:18s} {r['ms_per_step']:8.3f} ms/step  {r['achieved']:9.1f} {r['unit']}"
                f"  ({100 * r['achieved'] / r['peak']:.1f}% of peak)")
    dominant = max(per_class, key=lambda c: per_class[c]["ms_per_step"])
    d = per_class[dominant]
    traffic = traffic_for(dominant)
    roofline = {"bound": d["bound"], "achieved": round(d["achieved"], 2), "peak": d["peak"],
                "unit": d["unit"], "frac": round(d["achieved"] / d["peak"], 4), "traffic": traffic,
                "kernel": dominant, "avg_launch_ms": round(d["avg_launch_ms"], 4),
                "per_launch": d["per_launch"]}
    mentry = _profile_entry(MFMA_FILE, dominant)
    if mentry and d["bound"] == "mfma":
        # The published peak assumes 2.4 GHz. Beside it, from the committed
        # counter run (one box, one run): the clock the kernel held there and
        # its counted matrix flops over its own traced time against the peak
        # at that clock.
        roofline["clock_mhz"] = round(mentry["clock_mhz"])
        roofline["frac_at_clock"] = round(mentry["frac_nominal"] * 2400.0 / mentry["clock_mhz"], 4)
    gemm_ms = sum(kernels[c]["ms"] for c in GEMM_CLASSES)
    gemm_flops = sum(kernels[c]["flops"] for c in GEMM_CLASSES)
    jsd_cls = ("jsd_stats", "jsd_loss", "jsd_grad")
    jsd_ms = sum(kernels[c]["ms"] for c in jsd_cls)
    jsd_bytes = sum(kernels[c]["bytes"] for c in jsd_cls)
    result = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "step_ms": {"median": round(step_ms[len(step_ms) // 2], 3), "min": round(step_ms[0], 3),
                    "max": round(step_ms[-1], 3)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(tokens_per_s / PAGES_TOKENS_PER_S, 4),
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{WORKLOAD}: BT={BT} H={H} V={V} bf16 beta={w.beta} "
                               f"T={w.temperature} {w.reduction}",
                   "global_batch": BT, "num_chunks": nc, "parallelism": "single GPU"},
        "roofline": roofline,
        "mfma_util_gemms": round(gemm_flops / (gemm_ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "jsd_hbm_gbps_algorithmic": round(jsd_bytes / (jsd_ms / 1e3) / 1e9, 1),
        "peak_hbm_mb": round(peak_mb, 1),
        "kernels": {c: {"ms_per_step": round(r["ms_per_step"], 4), "achieved": round(r["achieved"], 2),
                        "unit": r["unit"], "frac": round(r["achieved"] / r["peak"], 4)}
                    for c, r in per_class.items()},
    }
    # The loss passes against the method's own byte counts: the three-pass
    # figure (7·V·s per row) and the compulsory one (3·V·s: each logit read
    # once, dX written once) at 8 TB/s; and, from the committed counter
    # summary, the HBM bytes the passes moved over their time.
    jsd_s = jsd_ms / args.steps / 1e3
    result["jsd_effective_gbps_7vs"] = round(7.0 * V * 2 * BT / jsd_s / 1e9, 1)
    result["jsd_compulsory_frac"] = round(3.0 * V * 2 * BT / (PEAK_HBM_GBPS * 1e9) / jsd_s, 4)
    jsd_traffic = [traffic_for(c) for c in jsd_cls]
    if all(t is not None for t in jsd_traffic):
        moved = sum(t * kernels[c]["launches"] / args.steps for t, c in zip(jsd_traffic, jsd_cls))
        result["jsd_hbm_gbps_counter"] = round(moved / jsd_s / 1e9, 1)
    mfma = mfma_counters()
    result["mfma_util_counter"] = mfma.get("gemms")
    if mfma:
        result["mfma_counters"] = mfma
    if not args.no_sweep:
        result["sweep"] = sweep(fljsd, max(3, args.steps // 4), 1, (X_s, W_s, X_t, W_t))
    if args.flce:
        result["flce"] = flce_sweep(fljsd, max(3, args.steps // 2), 1)
    if args.losses:
        result["losses"] = losses_timing(fljsd, 20, 3)
    if not args.no_cpu_baseline:
        if not args.no_oracle_1thread:
            result["oracle_one_thread"] = oracle_one_thread()
        del X_s, W_s, X_t, W_t, ws, gX, gW
        torch.cuda.empty_cache()
        cb = cpu_baseline(inp, w, args.cpu_rows)
        log(f"cpu baseline: {cb['value']:.1f} tokens/s on {cb['cores']} threads ({cb['seconds']:.1f} s)")
        cb.pop("seconds")
        cb["value"] = round(cb["value"], 2)
        result["cpu_baseline"] = cb
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
