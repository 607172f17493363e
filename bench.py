"""Benchmark of the fused 4-bit AdamW step (ZIP-SR / ZE-EDEN) on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama2b7]

One step = one adamw_step launch over the whole parameter list (every value: decode, AdamW,
weight update, requantize, pack), inputs resident in HBM.  The default workload is the
Llama-style 2.7B list (291 tensors, BF16 grads, ZIP-SR, LM-head m stochastically rounded in
the last 10% of a 200-step schedule).  The K timed steps take t = 200/K, 2*200/K, ..., 200, so
the stochastic-rounding phase has its share of the job.  Prints one JSON line.

roofline: algorithmic bytes per launch (12.125 B per quantized value with BF16 grads: FP32
weight read+write 8, grad 2, m and v codes read+write 2, four FP32 block scales per 128 values
0.125; 26 B per FP32-state value) over the mean launch time from HIP events on the launch
stream.  traffic: HBM bytes per launch from rocprofv3 FETCH_SIZE/WRITE_SIZE counters stored in
profiles/counters_<workload>.json, used only if the kernel source is unchanged since.
cpu_baseline: the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "optimizer-step G params/s and achieved HBM GB/s (% of peak), 2.7B list"
PEAK_HBM_GBS = 8000.0
KERNEL_SRC = os.path.join(ROOT, "bit_adamw_step_amd", "csrc", "adamw4_kernels.hip")


def kernel_hash() -> str:
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def algorithmic_bytes(w) -> tuple[int, int, int]:
    """(bytes per launch, quantized values, FP32-state values)."""
    gb = 2 if w.grad_dtype == "bf16" else 4
    q = f = 0
    for s in w.specs:
        if s.numel >= 4096 and not (s.flags & 1):
            q += s.numel
        else:
            f += s.numel
    nblk = sum((s.numel + 127) // 128 for s in w.specs if s.numel >= 4096 and not (s.flags & 1))
    qbytes = q * (8 + gb + 2) + nblk * 16     # w r/w, grad, codes r/w, 4 scale words per block
    fbytes = f * (8 + gb + 16)                # w r/w, grad, FP32 m and v r/w
    return qbytes + fbytes, q, f


def setup(w, device):
    import torch
    import workloads as W
    import bit_adamw_step_amd as A
    params, grads = [], []
    for i, s in enumerate(w.specs):
        params.append(W.make_param(s, i, device))
        grads.append(W.make_grad(w, s, i, 1, device))
    pl = A.ParamList(params, grads, [s.flags for s in w.specs])
    v0 = None
    if w.v0_kind != "zeros":
        v0 = [W.make_v0(w, s, i, device) for i, s in enumerate(w.specs)]
    pl.init(w.mode_at(1), None, v0)
    del v0
    torch.cuda.synchronize()
    return pl


def timed_schedule(w, K: int) -> list[int]:
    return [max(1, round((k + 1) * w.steps / K)) for k in range(K)]


def run_gpu(w, steps: int, warmup: int, device):
    import torch
    import bit_adamw_step_amd as A
    pl = setup(w, device)
    stream = torch.cuda.current_stream()
    prev = w.mode_at(1)

    def hp(t):
        nonlocal prev
        m = w.mode_at(t)
        h = A.hparams(step=t, mode=m, prev_mode=prev, sr_head=w.sr_head_at(t), seed=0)
        prev = m
        return h

    for t in range(1, warmup + 1):
        pl.step(hp(t), stream)
    torch.cuda.synchronize()
    ts = timed_schedule(w, steps)
    hps = [hp(t) for t in ts]
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in ts]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for (a, b), h in zip(ev, hps):
        a.record(stream)
        pl.step(h, stream)
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [a.elapsed_time(b) for a, b in ev]   # ms per launch
    return pl, ts, per, wall


def cpu_baseline(w, pl, budget_s: float = 15.0):
    """The oracle (unchanged) on a bounded sample of the workload: the first blocks of every
    quantized tensor, in rounds, until about budget_s of CPU time; plus every FP32-state tensor
    once.  Returns the oracle's throughput on that sample."""
    import numpy as np
    import torch
    import oracle as orc
    import bit_adamw_step_amd as A
    orc.build()
    specs = w.specs
    quant = [i for i, s in enumerate(specs) if A.is_quantized(s.numel, s.flags)]
    fp = [i for i, s in enumerate(specs) if not A.is_quantized(s.numel, s.flags)]
    per_tensor = 128 * 512                        # 65,536 values (512 blocks) per sampled tensor
    t_total = 0.0
    n_total = 0
    hp = orc.HParams(step=w.steps, mode=w.mode_at(w.steps), sr_head=w.sr_head_at(w.steps), seed=0)

    def host(i, e0, cnt):
        s = specs[i]
        n = s.numel
        buf = pl.states[i]
        off = A.state_layout(n, s.flags)
        w_ = pl.params[i][e0:e0 + cnt].cpu().numpy().copy()
        g = pl.grads[i][e0:e0 + cnt]
        g = g.view(torch.int16).cpu().numpy().view(np.uint16).copy() if g.dtype == torch.bfloat16 \
            else g.cpu().numpy().copy()
        if A.is_quantized(n, s.flags):
            b0, nb = e0 // 128, (cnt + 127) // 128
            c0, c1 = e0 // 2, (e0 + cnt + 1) // 2
            sb = lambda o, a, z: buf[o + a:o + z].cpu().numpy().copy()
            st = orc.State(True, sb(off[0], c0, c1), sb(off[1], c0, c1),
                           sb(off[2], 4 * b0, 4 * (b0 + nb)).view(np.float32),
                           sb(off[3], 4 * b0, 4 * (b0 + nb)).view(np.float32))
        else:
            st = orc.State(False, m=buf[off[0]:off[0] + 4 * n].cpu().numpy().view(np.float32).copy(),
                           v=buf[off[1]:off[1] + 4 * n].cpu().numpy().view(np.float32).copy())
        return w_, g, st

    for i in fp:
        w_, g, st = host(i, 0, specs[i].numel)
        t0 = time.perf_counter()
        orc.step_tensor(w_, g, st, hp, pos=i)
        t_total += time.perf_counter() - t0
        n_total += specs[i].numel
    rnd = 0
    while t_total < budget_s and rnd < 64:
        for i in quant:
            n = specs[i].numel
            e0 = min(rnd * per_tensor, ((n - 1) // 128) * 128)
            cnt = min(per_tensor, n - e0)
            w_, g, st = host(i, e0, cnt)
            t0 = time.perf_counter()
            orc.step_tensor(w_, g, st, hp, pos=i, head=bool(specs[i].flags & 2), e0=e0, n=n)
            t_total += time.perf_counter() - t0
            n_total += cnt
            if t_total >= budget_s:
                break
        rnd += 1
    cores = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or os.cpu_count()
    return {"value": round(n_total / t_total / 1e9, 6), "unit": "Gparams/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{n_total} values ({len(fp)} FP32-state tensors whole, leading 512-block "
                      f"slices of the quantized tensors), one oracle step at t={w.steps}, "
                      f"{t_total:.1f} s of oracle time"}


def traffic_from_profile(wname: str, bytes_alg: int):
    path = os.path.join(ROOT, "profiles", f"counters_{wname}.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("kernel_sha") != kernel_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama2b7")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 4 GiB device copy (counter calibration under rocprofv3)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the 4-bit AdamW step needs no communication and every "
              "box here has a single MI355X; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as W
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    device = torch.device("cuda:0")
    w = W.WORKLOADS[args.workload]
    print(f"# setup {w.name}: {len(w.specs)} tensors, {w.numel} values", file=sys.stderr, flush=True)
    pl, ts, per, wall = run_gpu(w, args.steps, args.warmup, device)
    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.float32, device=device)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    bytes_alg, q, f = algorithmic_bytes(w)
    ms = sum(per) / len(per)
    ms_wall = wall * 1000 / len(per)
    gparams = w.numel * len(per) / wall / 1e9
    achieved = bytes_alg / (ms / 1000) / 1e9
    sr = [p for t, p in zip(ts, per) if w.sr_head_at(t)]
    rtn = [p for t, p in zip(ts, per) if not w.sr_head_at(t)]
    out = {
        "metric": METRIC,
        "value": round(gparams, 3),
        "unit": "Gparams/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_wall, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name, "values": w.numel, "tensors": len(w.specs),
            "quantized_values": q, "fp32_state_values": f, "grad_dtype": w.grad_dtype,
            "v_mode": w.mode_schedule, "timed_t": [ts[0], ts[-1]],
            "ms_launch_rtn_phase": round(sum(rtn) / len(rtn), 4) if rtn else None,
            "ms_launch_sr_head_phase": round(sum(sr) / len(sr), 4) if sr else None,
            "algorithmic_bytes_per_launch": bytes_alg,
            "achieved_hbm_GBs": round(achieved, 1),
            "pct_of_peak_hbm": round(100 * achieved / PEAK_HBM_GBS, 2),
        },
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic_from_profile(w.name, bytes_alg)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, pl, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
