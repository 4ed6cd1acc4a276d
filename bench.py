#!/usr/bin/env python3
"""Throughput of the strict-path selected-token logprob on one MI355X.

One step = one rlk_logprob_forward over the whole batch of the Qwen3-8B LM-head workload
(T=4096 rows, H=4096, V=151936, 4 vocab segments, one pass): LM-head MFMA tile kernel with the
fused max/sum-exp/target epilogue, the per-segment fold and the cross-segment merge. Inputs are
seeded synthetic bf16 of that shape (datagen) with targets drawn from the oracle's softmax
(tests/golden), resident in HBM before timing starts.

Prints ONE JSON line with the metric, a roofline object for the dominant kernel (its duration
measured live with HIP events recorded by the library around each LM-head launch) and the CPU
oracle timed on a bounded sample of the same rows.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
    python bench.py --copy-calibration-mib 1024   # a plain device copy, for PMC byte scaling
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "selected-token logprobs/sec at H=4096,V=151936; MFMA util; layout mismatch=0"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "lmhead_qwen3_8b_head_pmc.txt")
KERNEL_SRC = os.path.join(ROOT, "invariant_lm_head_deterministic_amd", "csrc", "rlk_kernels.hip")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t handles through the HIP runtime's C API (timing on the library's stream)."""

    def __init__(self, n: int):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            rc = self.hip.hipEventCreate(ctypes.byref(e))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed: {rc}")
            self.ev.append(e.value)

    def record(self, i: int, stream: int) -> None:
        rc = self.hip.hipEventRecord(ctypes.c_void_p(self.ev[i]), ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed: {rc}")

    def ms(self, a: int, b: int) -> float:
        self.hip.hipEventSynchronize(ctypes.c_void_p(self.ev[b]))
        out = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(out), ctypes.c_void_p(self.ev[a]),
                                          ctypes.c_void_p(self.ev[b]))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return out.value

    def close(self) -> None:
        for e in self.ev:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


def kernel_source_sha() -> str:
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()


def committed_traffic() -> tuple[float | None, str]:
    """HBM bytes per LM-head launch from the committed rocprofv3 PMC summary, or None when the
    summary is missing or was taken on a different kernel source."""
    if not os.path.exists(PROFILE_TRAFFIC):
        return None, "no PMC summary committed"
    kv = {}
    for line in open(PROFILE_TRAFFIC):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != kernel_source_sha():
        return None, "kernel changed since the PMC counters were taken"
    try:
        return float(kv["traffic_bytes_per_launch"]), "rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-scaled"
    except (KeyError, ValueError):
        return None, "PMC summary incomplete"


def copy_calibration(mib: int) -> None:
    import torch

    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "dispatches": 3}), flush=True)


def cpu_baseline(h, Wb, y, budget_s: float = 10.0, max_reps: int = 8) -> dict:
    """The float64 oracle as it stands, on a bounded sample of the workload's rows: all active
    rows when they fit the time budget (repeated until about ``budget_s`` of CPU work), else an
    evenly spaced subset sized from a 64-row probe."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info

        cores = max((i.get("num_threads", 1) for i in threadpool_info()
                     if i.get("user_api") == "blas"), default=os.cpu_count())
    except Exception:
        cores = os.cpu_count()
    t0 = time.perf_counter()
    W64 = oracle.bf16_bits_to_f64(Wb)
    decode_s = time.perf_counter() - t0
    active = np.nonzero(y >= 0)[0]
    probe = active[:64]
    t0 = time.perf_counter()
    oracle.logprob(h, W64, y, rows=probe)
    t_probe = time.perf_counter() - t0
    n = int(min(active.size, max(64, 64 * (3 * budget_s / max(t_probe, 1e-3)))))
    rows = active[np.linspace(0, active.size - 1, n).astype(np.int64)]
    total, reps = 0.0, 0
    while reps < max_reps and (reps == 0 or total < budget_s):
        t0 = time.perf_counter()
        res = oracle.logprob(h, W64, y, rows=rows)
        total += time.perf_counter() - t0
        reps += 1
    return {"value": n * reps / total, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{n} of {y.size} rows (evenly spaced), {reps} pass(es), float64, "
                      f"{total:.1f}s; bf16->f64 decode of W ({decode_s:.1f}s) excluded",
            "_rows": rows, "_logp": res["logp"]}


def time_layout(rlk, lp, hd, Wd, yd, gd, T, steps, warmup, layout_kw, flops_per_launch=None):
    """Time full forwards in one layout: step time, and the LM-head launches' summed duration
    from HIP events the library records around each launch. Returns host logp too."""
    import numpy as np
    import torch

    dev = hd.device
    layout, keep = rlk.make_layout(T, **layout_kw)
    n_launch = rlk.rlk_layout_check(lp.config, layout)
    ws_bytes = rlk.rlk_logprob_workspace_size(lp.config, layout)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    logp = torch.empty(T, dtype=torch.float32, device=dev)
    lse = torch.empty(T, dtype=torch.float32, device=dev)
    ent = torch.empty(T, dtype=torch.float32, device=dev) if lp.entropy else None
    sp = torch.cuda.current_stream(dev).cuda_stream

    def ptr(t):
        return None if t is None else t.data_ptr()

    def step(events=()):
        rlk.rlk_logprob_forward_timed(lp.handle, hd.data_ptr(), Wd.data_ptr(), yd.data_ptr(),
                                      layout, ptr(gd), logp.data_ptr(), lse.data_ptr(), ptr(ent),
                                      ws.data_ptr(), ws_bytes, sp, list(events))

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = HipEvents(2 + 2 * n_launch * steps)
    ev.record(0, sp)
    for i in range(steps):
        base = 2 + 2 * n_launch * i
        step(ev.ev[base:base + 2 * n_launch])
    ev.record(1, sp)
    torch.cuda.synchronize()
    total = ev.ms(0, 1)
    kern = sum(ev.ms(2 + 2 * j, 3 + 2 * j) for j in range(n_launch * steps))
    ev.close()
    del keep
    return {"ms_per_step": total / steps, "lmhead_ms_per_step": kern / steps,
            "lmhead_launches_per_step": n_launch, "_logp": logp.cpu().numpy().copy()}


def extras(rlk, datagen, np, torch, hd, Wd, yd, w, ref_logp) -> dict:
    """The other rows of the path, measured next to the headline: the rollout layout of the TP4
    workload (decode batches x 4 vocab shards; HBM-bound W stream) and the fused final RMSNorm +
    temperature + entropy head."""
    out = {}
    lp = rlk.Logprob(w.H, w.V, vocab_segments=w.segments, device=0)
    sizes = datagen.decode_layout(w.T)
    r = time_layout(rlk, lp, hd, Wd, yd, None, w.T, 3, 1,
                    dict(batch_sizes=sizes, vocab_shards=4))
    w_bytes = r["lmhead_launches_per_step"] * (w.V // 4) * w.H * 2
    out["tp4_decode_x4_shards"] = {
        "decode_batches": len(sizes), "lmhead_launches_per_step": r["lmhead_launches_per_step"],
        "ms_per_step": r["ms_per_step"], "tokens_per_s": w.T / (r["ms_per_step"] * 1e-3),
        "w_stream_GBps": w_bytes / (r["lmhead_ms_per_step"] * 1e-3) / 1e9,
        "hbm_frac": w_bytes / (r["lmhead_ms_per_step"] * 1e-3) / 8e12,
        "mismatch_count_vs_one_pass": int(np.count_nonzero(
            r["_logp"].view(np.uint32) != ref_logp.view(np.uint32)))}
    del lp
    wn = datagen.WORKLOADS["norm_head"]
    log("norm_head inputs")
    x = datagen.hidden_bits(wn)
    Wn = datagen.weight_bits(wn)
    g = datagen.gamma_bits(wn)
    yn = np.load(os.path.join(ROOT, "tests", "golden", "targets_norm_head.npy"))
    dev = hd.device
    xd = torch.from_numpy(x.view(np.int16)).to(dev)
    Wnd = torch.from_numpy(Wn.view(np.int16)).to(dev)
    gd = torch.from_numpy(g.view(np.int16)).to(dev)
    ynd = torch.from_numpy(yn.astype(np.int32)).to(dev)
    del x, Wn
    lpn = rlk.Logprob(wn.H, wn.V, vocab_segments=wn.segments, temperature=wn.tau, rmsnorm=True,
                      rms_eps=wn.rms_eps, entropy=True, device=0)
    r = time_layout(rlk, lpn, xd, Wnd, ynd, gd, wn.T, 5, 2, {})
    fl = 2.0 * wn.T * wn.H * wn.V
    out["norm_head_one_pass"] = {
        "T": wn.T, "H": wn.H, "V": wn.V, "tau": wn.tau, "ms_per_step": r["ms_per_step"],
        "tokens_per_s": wn.T / (r["ms_per_step"] * 1e-3),
        "lmhead_ms": r["lmhead_ms_per_step"],
        "lmhead_frac_of_bf16_peak": fl / (r["lmhead_ms_per_step"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
    del xd, Wnd, lpn
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen3_8b_head")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-layout-check", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0)
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the rollout-layout and norm_head measurements")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this path has no multi-GPU mode (asked for "
              f"--gpus {args.gpus}); see the sharding design, run with --gpus 1", file=sys.stderr)
        return 2
    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib)
        return 0

    import numpy as np
    import torch

    import datagen
    import invariant_lm_head_deterministic_amd as rlk

    rlk.require_library()
    w = datagen.WORKLOADS[args.workload]
    log(f"generating {args.workload} inputs T={w.T} H={w.H} V={w.V}")
    h = datagen.hidden_bits(w)
    Wb = datagen.weight_bits(w)
    y = np.load(os.path.join(ROOT, "tests", "golden", f"targets_{args.workload}.npy"))
    meta = json.load(open(os.path.join(ROOT, "tests", "golden", f"targets_{args.workload}.json")))
    if meta["sha256_hidden"] != datagen.sha256(h) or meta["sha256_W"] != datagen.sha256(Wb):
        raise RuntimeError("stored targets do not belong to the generated inputs")
    gamma = datagen.gamma_bits(w) if w.rmsnorm else None

    dev = torch.device("cuda", 0)
    hd = torch.from_numpy(h.view(np.int16)).to(dev)
    Wd = torch.from_numpy(Wb.view(np.int16)).to(dev)
    yd = torch.from_numpy(y.astype(np.int32)).to(dev)
    gd = None if gamma is None else torch.from_numpy(gamma.view(np.int16)).to(dev)
    lp = rlk.Logprob(w.H, w.V, vocab_segments=w.segments, temperature=w.tau, rmsnorm=w.rmsnorm,
                     rms_eps=w.rms_eps, entropy=w.rmsnorm, device=0)
    layout, keep = rlk.make_layout(w.T)
    ws_bytes = rlk.rlk_logprob_workspace_size(lp.config, layout)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    logp = torch.empty(w.T, dtype=torch.float32, device=dev)
    lse = torch.empty(w.T, dtype=torch.float32, device=dev)
    ent = torch.empty(w.T, dtype=torch.float32, device=dev) if lp.entropy else None
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream

    def ptr(t):
        return None if t is None else t.data_ptr()

    def step(events=()):
        rlk.rlk_logprob_forward_timed(lp.handle, hd.data_ptr(), Wd.data_ptr(), yd.data_ptr(),
                                      layout, ptr(gd), logp.data_ptr(), lse.data_ptr(), ptr(ent),
                                      ws.data_ptr(), ws_bytes, sp, list(events))

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ev = HipEvents(2 + 2 * args.steps)
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    ev.record(0, sp)
    for i in range(args.steps):
        step((ev.ev[2 + 2 * i], ev.ev[3 + 2 * i]))
    ev.record(1, sp)
    torch.cuda.synchronize()
    total_ms = ev.ms(0, 1)
    k_ms = [ev.ms(2 + 2 * i, 3 + 2 * i) for i in range(args.steps)]
    ev.close()
    ms_step = total_ms / args.steps
    kern_ms = float(np.mean(k_ms))
    active = int((y >= 0).sum())
    value = active / (ms_step * 1e-3)
    flops = 2.0 * w.T * w.H * w.V  # every row is computed, padded ones included
    achieved = flops / (kern_ms * 1e-3) / 1e12
    traffic, traffic_note = committed_traffic()
    out_logp = logp.cpu().numpy().copy()

    mismatch = None
    if not args.no_layout_check:
        log("layout check: rollout decode batches x 4 vocab shards")
        sizes = datagen.decode_layout(w.T)
        o = lp.forward(hd, Wd, yd, batch_sizes=sizes, vocab_shards=4,
                       gamma=gd)
        torch.cuda.synchronize()
        mismatch = int(np.count_nonzero(o["logp"].cpu().numpy().view(np.uint32)
                                        != out_logp.view(np.uint32)))

    result = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded bf16, oracle-sampled targets)",
        "config": {"workload": args.workload, "T": w.T, "H": w.H, "V": w.V,
                   "vocab_segments": w.segments, "layout": "one pass", "parallelism": "none"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic},
        "lmhead_kernel_ms": kern_ms,
        "mfma_util": achieved / PEAK_BF16_TFLOPS,
        "layout_mismatch_count": mismatch,
        "traffic_note": traffic_note,
    }
    if not args.no_extras:
        log("extras: rollout layout (decode batches x 4 shards), norm_head")
        result["extras"] = extras(rlk, datagen, np, torch, hd, Wd, yd, w, out_logp)
    if not args.no_cpu_baseline:
        log("cpu baseline (float64 oracle on a bounded sample)")
        cb = cpu_baseline(h, Wb, y)
        rows, ref = cb.pop("_rows"), cb.pop("_logp")
        result["cpu_baseline"] = cb
        result["oracle_max_abs_diff_on_sample"] = float(np.max(np.abs(
            out_logp[rows].astype(np.float64) - ref)))
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    del keep
    return 0


if __name__ == "__main__":
    sys.exit(main())
