"""Benchmark: chunked GRPO log-prob + loss forward/backward on one MI355X.

A step is one pass of the whole path over one synthetic batch: group advantages,
then grpo_loss_fwd_bwd (token index, target logits, per chunk the logits GEMM with
online log-sum-exp, the merge with the GRPO per-token terms, the recompute GEMM
writing probabilities and the dH GEMM; finally the fp64 loss sum).  Inputs are
resident in HBM before the timed region.  The default workload is the
Qwen3-8B-shaped long-context stream (D=4096, V=151936, 2 x 55000 tokens,
chunks of 8192 tokens).

Prints one JSON line: whole-step tokens/s, the roofline of the dominant kernel
(algorithmic flops over its event-timed launches inside the timed region) and the
fp64 oracle timed on the host cores on a bounded sample of the same workload.
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

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
METRIC = "GRPO logp+loss fwd+bwd tokens/s at 1 GPU; % of bf16 MFMA peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--chunk", type=int, default=0, help="override the workload's chunk tokens")
    ap.add_argument("--cpu-sample-tokens", type=int, default=4096)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variant", action="store_true",
                    help="skip timing the variant that keeps the chunk's logits (no recompute GEMM)")
    ap.add_argument("--no-entry-points", action="store_true",
                    help="skip timing grpo_logp_fwd / grpo_logp_bwd / grpo_ce_loss_fwd_bwd / grpo_advantages")
    ap.add_argument("--no-clocks", action="store_true",
                    help="do not sample the shader clock and socket power (sysfs reads in a helper thread)")
    ap.add_argument("--other-configs", default="1,2,4",
                    help="short runs of these other workloads, reported under other_configs ('' = none)")
    ap.add_argument("--other-steps", type=int, default=3)
    ap.add_argument("--other-warmup", type=int, default=1)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (for HBM counter scaling)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def copy_calibration():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}), flush=True)


# HBM-side bytes per launch of the GEMM kernels, from the rocprofv3 FETCH_SIZE / WRITE_SIZE
# passes summarized in this file, scaled by the same counters on a plain device copy.
# They describe the kernel sources whose hash the file records, and are reported only
# while the sources still hash the same.
COUNTERS_MD = os.path.join(ROOT, "profiles", "grpo_loss_qwen3-8b-110k_hbm_counters.md")
KERNEL_SOURCES = ["rl_fine_tuning_amd/csrc/grpo_kernels.hip", "rl_fine_tuning_amd/csrc/grpo_host.cpp",
                  "rl_fine_tuning_amd/csrc/grpo_plan.h"]


def measured_traffic(kernel, workload_is_profiled):
    """Scaled FETCH_SIZE + WRITE_SIZE bytes per launch of `kernel`, or None."""
    import hashlib
    import re
    if not workload_is_profiled or not os.path.exists(COUNTERS_MD):
        return None
    text = open(COUNTERS_MD).read()
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    m = re.search(r"sources_sha256 = ([0-9a-f]+)", text)
    if not m or m.group(1) != h.hexdigest():
        return None
    ff = float(re.search(r"fetch_factor = ([0-9.eE+-]+)", text).group(1))
    wf = float(re.search(r"write_factor = ([0-9.eE+-]+)", text).group(1))
    m = re.search(rf"^{kernel} fetch_kib = ([0-9.eE+-]+) write_kib = ([0-9.eE+-]+)", text, re.M)
    if not m:
        return None
    return (float(m.group(1)) * ff + float(m.group(2)) * wf) * 1024.0


def sysfs_dir(props):
    """The PCI device directory of the GPU in sysfs (its clock and power files), or None."""
    try:
        d = f"/sys/bus/pci/devices/{props.pci_domain_id:04x}:{props.pci_bus_id:02x}:{props.pci_device_id:02x}.0"
        return d if os.path.isdir(d) else None
    except Exception:
        return None


def _read(path):
    try:
        with open(path) as f:
            return f.read()
    except Exception:
        return None


def sclk_levels(dev):
    """(current MHz or None, max MHz or None) from the DPM table pp_dpm_sclk ('*' marks the
    current level)."""
    import re
    txt = _read(os.path.join(dev, "pp_dpm_sclk")) if dev else None
    if not txt:
        return None, None
    cur, top = None, None
    for line in txt.splitlines():
        m = re.search(r"(\d+)\s*Mhz", line, re.I)
        if not m:
            continue
        mhz = int(m.group(1))
        top = mhz if top is None else max(top, mhz)
        if "*" in line:
            cur = mhz
    return cur, top


def box_peak(props, dev):
    """CU count (device properties) and maximum shader clock (the DPM table) of the GPU, and
    the dense bf16 MFMA peak they imply (4096 flop per clock per CU)."""
    cus = int(props.multi_processor_count)
    _, mhz = sclk_levels(dev)
    if not mhz:
        return {"compute_units": cus, "max_sclk_mhz": None, "bf16_dense_tflops": None}
    return {"compute_units": cus, "max_sclk_mhz": mhz, "bf16_dense_tflops": cus * mhz * 1e6 * 4096 / 1e12,
            "source": "device properties, pp_dpm_sclk"}


class ClockSampler:
    """Samples the shader clock and the socket power from sysfs files of the GPU (read in this
    process by a helper thread: no child processes) while the timed steps run."""

    def __init__(self, dev, enabled=True, period=0.1):
        import glob
        import threading
        self.dev = dev
        self.enabled = enabled and dev is not None
        self.period = period
        self.sclk, self.power = [], []
        self.freq_file = self.power_file = None
        if self.enabled:
            for h in sorted(glob.glob(os.path.join(dev, "hwmon", "hwmon*"))):
                if self.freq_file is None and _read(os.path.join(h, "freq1_input")):
                    self.freq_file = os.path.join(h, "freq1_input")
                for name in ("power1_average", "power1_input"):
                    if self.power_file is None and _read(os.path.join(h, name)):
                        self.power_file = os.path.join(h, name)
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _sample(self):
        if self.freq_file:
            v = _read(self.freq_file)
            if v and v.strip().isdigit():
                self.sclk.append(int(v) / 1e6)  # Hz
        else:
            cur, _ = sclk_levels(self.dev)
            if cur:
                self.sclk.append(cur)
        if self.power_file:
            v = _read(self.power_file)
            if v and v.strip().isdigit():
                self.power.append(int(v) / 1e6)  # microwatts

    def _run(self):
        while not self._stop.wait(self.period):
            try:
                self._sample()
            except Exception:
                return

    def __enter__(self):
        if self.enabled:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self.enabled:
            self._thread.join(timeout=30)

    def summary(self):
        avg = lambda v: sum(v) / len(v) if v else None
        return {"sclk_mhz_avg": avg(self.sclk), "sclk_samples": len(self.sclk),
                "socket_power_w_avg": avg(self.power), "power_samples": len(self.power),
                "sources": {"sclk": self.freq_file or (os.path.join(self.dev, "pp_dpm_sclk") if self.dev else None),
                            "power": self.power_file}}


def cpu_baseline(case, n_tokens):
    """The fp64 oracle, as it stands, on the first n_tokens tokens of the workload."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count()
    n = min(n_tokens, case.T)
    H = oracle.widen(case.H[:n], case.dtype)
    W = oracle.widen(case.W, case.dtype)
    y = case.targets[:n]
    cu = np.array([0, n], dtype=np.int64)
    old = np.zeros(n)
    ref = np.zeros(n)
    adv = np.array([1.0])
    t0 = time.perf_counter()
    oracle.grpo_loss_and_grad(H, W, y, cu, np.ones(n, np.uint8), old, ref, adv)
    dt = time.perf_counter() - t0
    res = {"value": n / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
           "sample": f"first {n} tokens of the workload, full fwd+bwd (logp, loss, dH) in fp64 numpy; "
                     f"{dt:.1f} s"}
    # the same on one thread, on a smaller sample
    n1 = min(64, n)
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            oracle.grpo_loss_and_grad(H[:n1], W, y[:n1], np.array([0, n1], dtype=np.int64), np.ones(n1, np.uint8),
                                      old[:n1], ref[:n1], adv)
            dt1 = time.perf_counter() - t0
        res["value_1thread"] = n1 / dt1
        res["sample_1thread"] = f"first {n1} tokens, one BLAS thread; {dt1:.1f} s"
    except Exception as e:  # threadpoolctl missing: no one-thread figure
        res["value_1thread"] = None
        res["sample_1thread"] = f"not measured ({type(e).__name__})"
    return res


def prepare(cfg, chunk=0):
    """Synthetic inputs of workload `cfg` resident on the GPU, a workspace, and the step: group
    advantages, then grpo_loss_fwd_bwd (dH into a preallocated buffer)."""
    import numpy as np
    import torch

    from rl_fine_tuning_amd import grpo_advantages, grpo_logp_fwd, grpo_loss_fwd_bwd, grpo_workspace_bytes
    from synth import make_config

    t_gen = time.perf_counter()
    case = make_config(cfg)
    C = chunk or case.chunk
    T, D, V, S, G = case.T, case.D, case.V, case.S, case.G
    log(f"config {cfg}: T={T} D={D} V={V} S={S} chunk={C}; inputs drawn in {time.perf_counter() - t_gen:.1f} s")
    dev = torch.device("cuda:0")
    if case.dtype == "bf16":
        mat = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        mat = lambda x: torch.from_numpy(x).to(dev)
    H, W = mat(case.H), mat(case.W)
    targets = torch.from_numpy(case.targets).to(dev)
    rewards = torch.from_numpy(case.rewards).to(dev)
    # old / reference policy log-probs: the current policy's logp plus the workload's noise
    # (input preparation, outside the timed region)
    logp0 = grpo_logp_fwd(H, W, targets, C)
    old = (logp0.double() + torch.from_numpy(case.noise_old).to(dev)).float()
    ref = (logp0.double() + torch.from_numpy(case.noise_ref).to(dev)).float()
    del logp0
    ws_bytes = grpo_workspace_bytes(T, D, V, C, 0 if case.dtype == "bf16" else 1, num_seqs=S)
    # one buffer also serves the entry-point timings (the dW call may lay it out differently)
    ws_dw = grpo_workspace_bytes(T, D, V, C, 0, num_seqs=S, with_dW=True) if case.dtype == "bf16" else 0
    ws = torch.empty(max(ws_bytes, ws_dw), dtype=torch.uint8, device=dev)
    dH = torch.empty_like(H)
    adv = torch.empty(S, dtype=torch.float32, device=dev)
    cu = case.cu

    def step(timer=None, keep=False):
        grpo_advantages(rewards, G, out=adv)
        return grpo_loss_fwd_bwd(H, W, targets, cu, old, ref, adv, C, dH=dH, workspace=ws, timer=timer,
                                 want_logp=False, want_token_loss=False, keep_chunk_logits=keep)

    return dict(case=case, C=C, H=H, W=W, targets=targets, rewards=rewards, old=old, ref=ref, ws=ws,
                ws_bytes=ws_bytes, dH=dH, adv=adv, step=step)


def gemm_flops(T, D, V, C):
    """Algorithmic flops of each GEMM kind over one step (2 rows D V per chunk each)."""
    rows = [min(C, T - k * C) for k in range((T + C - 1) // C)]
    f = sum(2.0 * r * D * V for r in rows)
    return {"logits_lse": f, "probs": f, "dh_gemm": f}


def short_run(cfg, steps, warmup):
    """A short timing of the same step on another workload: tokens/s, MFMA fraction, per-GEMM
    TFLOP/s (HIP events around each launch), workspace and peak extra memory."""
    import torch

    from rl_fine_tuning_amd import Timer
    from synth import CONFIGS

    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    w = prepare(cfg)
    case, C, step = w["case"], w["C"], w["step"]
    T, D, V = case.T, case.D, case.V
    torch.cuda.synchronize()
    base_mem = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    for _ in range(warmup):
        step()
    timer = Timer(16384)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(timer)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    ms = 1e3 * el / steps
    gf = gemm_flops(T, D, V, C)
    gemms = {}
    for k, f in gf.items():
        t_ms, n, _ = timer.read(k)
        gemms[k] = {"tflops": f * steps / (t_ms * 1e-3) / 1e12 if t_ms else None, "launches_per_step": n / steps}
    timer.close()
    res = {"workload": CONFIGS[cfg]["workload"], "T": T, "D": D, "V": V, "chunk_tokens": C,
           "tokens_per_s": T * steps / el, "ms_per_step": ms, "steps": steps, "warmup": warmup,
           "mfma_frac_step": 6.0 * T * D * V / (ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12), "gemms": gemms,
           "workspace_bytes": w["ws_bytes"], "peak_extra_bytes": torch.cuda.max_memory_allocated() - base_mem}
    del w, step
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    log(f"config {cfg}: {res['tokens_per_s']:.0f} tokens/s ({res['mfma_frac_step']:.3f} of peak)")
    return res


def provenance(torch):
    """Where the numbers come from: hashes of the sources, the commit (when the tree is a git
    checkout), the ROCm and torch versions, the workloads' seeds.  Files only, no child
    processes."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES + ["include/grpo.h", "bench.py"]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    head = None
    try:
        ref = open(os.path.join(ROOT, ".git", "HEAD")).read().strip()
        if ref.startswith("ref: "):
            name = ref[5:]
            p = os.path.join(ROOT, ".git", name)
            if os.path.exists(p):
                head = open(p).read().strip()
            else:
                for line in open(os.path.join(ROOT, ".git", "packed-refs")):
                    if line.strip().endswith(" " + name):
                        head = line.split()[0]
        else:
            head = ref
    except Exception:
        head = None
    rocm = _read("/opt/rocm/.info/version")
    return {"sources_sha256": h.hexdigest(), "git_head": head, "rocm_version": rocm.strip() if rocm else None,
            "torch": torch.__version__, "torch_hip": getattr(torch.version, "hip", None),
            "seeds": {"rule": "synth.make_config(cfg) draws from PCG64(SeedSequence((1000 + cfg, stream, block)))",
                      "headline": 1000 + 3}}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this path runs on a single MI355X and has no multi-GPU mode "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import numpy as np
    import torch

    from rl_fine_tuning_amd import (Offload, Timer, grpo_advantages, grpo_ce_loss_fwd_bwd, grpo_logp_bwd,
                                    grpo_logp_bwd_offload, grpo_logp_fwd, grpo_logp_fwd_offload, grpo_loss_fwd_bwd,
                                    grpo_plan_info, grpo_workspace_bytes)
    from synth import CONFIGS, make_config

    cfg = args.config
    spec = CONFIGS[cfg]
    w = prepare(cfg, args.chunk)
    case, C, H, W, targets, rewards = w["case"], w["C"], w["H"], w["W"], w["targets"], w["rewards"]
    old, ref, ws, ws_bytes, dH, adv, step = w["old"], w["ref"], w["ws"], w["ws_bytes"], w["dH"], w["adv"], w["step"]
    T, D, V, S, G = case.T, case.D, case.V, case.S, case.G
    dev = H.device
    cu = case.cu

    torch.cuda.synchronize()
    base_mem = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")
    timer = Timer(16384)
    props = torch.cuda.get_device_properties(0)
    dev_dir = sysfs_dir(props)
    peak_box = box_peak(props, dev_dir)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    with ClockSampler(dev_dir, enabled=not args.no_clocks) as clocks:
        t0 = time.perf_counter()
        for i in range(args.steps):
            evs[i].record()
            out = step(timer)
        evs[args.steps].record()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    step_ms = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    log(f"timed {args.steps} steps in {elapsed:.3f} s")
    peak_extra = torch.cuda.max_memory_allocated() - base_mem
    loss = float(out["loss"].cpu()[0])

    ms_step = 1e3 * elapsed / args.steps
    tokens_per_s = T * args.steps / elapsed
    flops_step = 6.0 * T * D * V
    nchunks = (T + C - 1) // C
    rows = [min(C, T - k * C) for k in range(nchunks)]
    gemm_flops = globals()["gemm_flops"](T, D, V, C)
    kernels = {}
    for k in ("target_logit", "logits_lse", "merge", "probs", "dh_gemm", "dh_reduce", "token_index",
              "loss_finalize", "frag_copy", "transpose_w", "w_copy", "onehot_fix"):
        ms, n, dropped = timer.read(k)
        kernels[k] = {"ms_total": ms, "launches": n}
    dominant = max(gemm_flops, key=lambda k: kernels[k]["ms_total"])
    dk = kernels[dominant]
    achieved = gemm_flops[dominant] * args.steps / (dk["ms_total"] * 1e-3) / 1e12
    for k in gemm_flops:
        kk = kernels[k]
        kk["tflops"] = gemm_flops[k] * args.steps / (kk["ms_total"] * 1e-3) / 1e12 if kk["ms_total"] else None
    # the streaming kernels: algorithmic bytes per step (read + written) over their event time
    ntv, ks_d, ks_v = -(-V // 256), -(-D // 16), -(-V // 16)
    esz = 2 if case.dtype == "bf16" else 4
    stream_bytes = {
        # per token: the (max, sum-exp) partials of every vocabulary tile, zy / old / ref / advantage /
        # sequence weight read, lse / g / weighted loss written
        "merge": T * (8 * ntv + 44),
        "target_logit": T * (2 * D * esz + 8),             # the token's row of H and W[y]
        "frag_copy": sum(r * D * esz + -(-r // 256) * 256 * ks_d * 32 for r in rows),
        "w_copy": V * D * esz + ntv * 256 * ks_d * 32,
        "transpose_w": V * D * esz + -(-D // 256) * 256 * ks_v * 32,
    }
    bands = grpo_plan_info(T, D, V, C, 0 if case.dtype == "bf16" else 1, num_seqs=S)["w_transposed_bands"]
    if bands and kernels["transpose_w"]["launches"]:
        # W^T made band by band in every backward pass: each launch moves one band (V / bands rows)
        stream_bytes["transpose_w"] *= kernels["transpose_w"]["launches"] / args.steps / bands
    streaming = {}
    for k, b in stream_bytes.items():
        kk = kernels[k]
        if kk["launches"] and kk["ms_total"]:
            streaming[k] = {"bytes_per_step": b, "ms_per_step": kk["ms_total"] / args.steps,
                            "GB_per_s": b * args.steps / (kk["ms_total"] * 1e-3) / 1e9}
    result = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if case.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": spec["workload"], "T": T, "D": D, "V": V, "chunk_tokens": C,
                   "sequences": S, "group_size": G},
        "mfma_frac_step": flops_step / (ms_step * 1e-3) / (PEAK_BF16_TFLOPS * 1e12),
        "roofline": {"bound": "mfma", "kernel": dominant, "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": measured_traffic(dominant, cfg == 3 and C == 8192),
                     "traffic_unit": "bytes per launch (HBM-side: L2 fills from the fabric + writes)",
                     "avg_launch_ms": dk["ms_total"] / max(1, dk["launches"]),
                     "flops_per_launch_avg": gemm_flops[dominant] * args.steps / max(1, dk["launches"])},
        "kernels": kernels,
        "streaming_kernels": streaming,
        "step_ms": {"median": step_ms[len(step_ms) // 2], "min": step_ms[0], "max": step_ms[-1],
                    "source": "HIP events around each timed step"},
        "clocks": dict(clocks.summary(), box=peak_box,
                       note="read from sysfs every 0.1 s during the timed steps; the roofline peak stays the "
                            "published 2.5 PFLOP/s"),
        "workspace_bytes": ws_bytes,
        "peak_extra_bytes": peak_extra,
        "loss": loss,
    }
    timer.close()
    if not args.no_variant and case.dtype == "bf16":
        # The same step with keep_chunk_logits: the forward GEMM keeps the chunk's logits, so
        # the backward has no recompute GEMM (4 D V flop per token instead of 6 D V).
        for _ in range(args.warmup):
            step(keep=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step(keep=True)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        ms_v = 1e3 * el / args.steps
        result["variant_keep_chunk_logits"] = {
            "value": T * args.steps / el, "unit": "tokens/s", "ms_per_step": ms_v,
            "mfma_frac_step_4DV": 4.0 * T * D * V / (ms_v * 1e-3) / (PEAK_BF16_TFLOPS * 1e12),
            "note": "same outputs (logp/loss bitwise, dH within the fp16 rounding of the kept logits); "
                    "not the headline: the pages' backward recomputes the chunk's logits"}
        log(f"keep_chunk_logits variant: {result['variant_keep_chunk_logits']['value']:.0f} tokens/s")
    if not args.no_entry_points:
        # The other entry points on the same resident inputs, each timed like the step
        # (warm-up calls, then `steps` calls between two synchronizations).
        def timed(fn):
            for _ in range(args.warmup):
                fn()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(args.steps):
                fn()
            torch.cuda.synchronize()
            return 1e3 * (time.perf_counter() - t0) / args.steps
        lp_out = torch.empty(T, dtype=torch.float32, device=dev)
        lse = torch.empty(T, dtype=torch.float32, device=dev)
        ws_f = torch.empty(grpo_workspace_bytes(T, D, V, C, 0 if case.dtype == "bf16" else 1, with_backward=False),
                           dtype=torch.uint8, device=dev)
        ms_f = timed(lambda: grpo_logp_fwd(H, W, targets, C, out=lp_out, workspace=ws_f))
        _, lse = grpo_logp_fwd(H, W, targets, C, return_lse=True)
        grad = (old - ref) * 1e-3
        ms_b = timed(lambda: grpo_logp_bwd(H, W, targets, lse, grad, C, dH=dH, workspace=ws))
        ms_ce = timed(lambda: grpo_ce_loss_fwd_bwd(H, W, targets, C, dH=dH, workspace=ws, want_logp=False))
        ms_adv = timed(lambda: grpo_advantages(rewards, G, out=adv))
        ms_dw, dw_tf = None, None
        if case.dtype == "bf16":
            dW = torch.empty(V, D, dtype=torch.float32, device=dev)
            tmw = Timer(32768)  # two launches per vocabulary band per chunk for the dW GEMM
            def step_dw():
                grpo_advantages(rewards, G, out=adv)
                grpo_loss_fwd_bwd(H, W, targets, cu, old, ref, adv, C, dH=dH, dW=dW, workspace=ws,
                                  want_logp=False, want_token_loss=False, timer=tmw)
            step_dw()
            tmw.reset()
            ms_dw = timed(step_dw)
            ms_k, _, dropped = tmw.read("dw_gemm")
            calls = tmw.read("loss_finalize")[1]  # one per call
            assert dropped == 0, "timer capacity too small for the dW step"
            dw_tf = gemm_flops["dh_gemm"] * calls / (ms_k * 1e-3) / 1e12 if ms_k else None
            tmw.close()
            del dW
        # the split forward / backward with the hidden states offloaded to pinned host memory in
        # between (PCIe-inclusive: the forward's copy to the host and the backward's copies back)
        off = Offload()
        H_host = torch.empty((T, D), dtype=H.dtype, pin_memory=True)
        ws_h = torch.empty(grpo_workspace_bytes(T, D, V, C, 0 if case.dtype == "bf16" else 1, host_h=True),
                           dtype=torch.uint8, device=dev)
        ms_fo = timed(lambda: grpo_logp_fwd_offload(H, W, targets, C, off, H_host=H_host, out=lp_out, lse=lse,
                                                    workspace=ws_f))
        ms_bo = timed(lambda: grpo_logp_bwd_offload(H_host, W, targets, lse, grad, C, off, dH=dH, workspace=ws_h))
        off.close()
        del ws_h, H_host
        per = lambda ms, k: {"tokens_per_s": T / (ms * 1e-3), "ms": ms,
                             "mfma_frac": k * T * D * V / (ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12)}
        result["entry_points"] = {"grpo_logp_fwd": per(ms_f, 2.0), "grpo_logp_bwd": per(ms_b, 4.0),
                                  "grpo_ce_loss_fwd_bwd": per(ms_ce, 6.0),
                                  "grpo_loss_fwd_bwd_with_dW": dict(per(ms_dw, 8.0), dw_gemm_tflops=dw_tf)
                                  if ms_dw else None,
                                  "grpo_advantages": {"us": 1e3 * ms_adv, "sequences": S},
                                  "grpo_logp_fwd_offload": per(ms_fo, 2.0), "grpo_logp_bwd_offload": per(ms_bo, 4.0)}
        log(f"entry points: logp_fwd {ms_f:.1f} ms, logp_bwd {ms_b:.1f} ms, ce {ms_ce:.1f} ms, "
            f"advantages {1e3 * ms_adv:.1f} us, logp_fwd_offload {ms_fo:.1f} ms, logp_bwd_offload {ms_bo:.1f} ms")
    result["provenance"] = provenance(torch)
    others = [int(x) for x in args.other_configs.split(",") if x.strip() and int(x) != cfg]
    if others:
        result["other_configs"] = {str(c): short_run(c, args.other_steps, args.other_warmup) for c in others}
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on the host")
        result["cpu_baseline"] = cpu_baseline(case, args.cpu_sample_tokens)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
