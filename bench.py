"""Benchmark of the fused 4-bit AdamW step (ZIP-SR / ZE-EDEN) on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama2b7] [--v-mode RULE]
                [--bf16-copy] [--shard-of N] [--optimizer] [--no-cpu-baseline] [--no-ceiling]

One step = one adamw4_step call over the whole parameter list (every value: decode, AdamW,
weight update, requantize, pack), inputs resident in HBM.  The K timed steps run back to back
between two synchronisations (value, ms_per_step); the same K steps then run again with HIP
events around each launch on the launch stream (per-launch median, percentiles, the roofline's
achieved rate).  The default workload is the
Llama-style 2.7B list (291 tensors, BF16 grads, ZIP-SR, LM-head m stochastically rounded in
the last 10% of a 200-step schedule).  The K timed steps take t = 200/K, 2*200/K, ..., 200, so
the stochastic-rounding phase has its share of the job.  Prints one JSON line.

roofline: algorithmic bytes per launch (12.125 B per quantized value with BF16 grads: FP32
weight read+write 8, grad 2, m and v codes read+write 2, four FP32 block scales per 128 values
0.125; 26 B per FP32-state value) over the mean launch time from HIP events recorded on the
launch stream.  traffic: HBM bytes per launch from rocprofv3 FETCH_SIZE/WRITE_SIZE counters,
scaled by the counters' reading on a copy of known size, stored in
profiles/counters_<workload>.json and used only while the kernel source is unchanged.
ceiling: a streaming kernel (libadamw4_ceiling.so) that moves the same bytes per value in the
same access pattern with trivial arithmetic, at its best of two grid sizes: what a plain
streaming kernel reaches with this byte mix on the GPU at hand (the step can come close to it
or pass it; it is a reference point, not a bound).
cpu_baseline: the CPU oracle (test infrastructure, timed here only) stepping the same list,
tensor by tensor from host copies of the GPU's current state, until a time budget is spent.
--v-mode runs every step with one v rule; --bf16-copy adds the fused BF16 weight copy (2 B per
value more); --shard-of N times rank 0's share of an N-way 128-aligned split of every tensor;
--optimizer adds an "optimizer" object: the torch front end's opt.step() on the list as a BF16
model (GPU and host time).

python bench.py --hbm-study [FILTER] runs the measurement program hbm_mix_probe (built by the
package's build step): the step's byte mix over 2.7B values under many access patterns, one CSV
line per pattern (see its source for the names).

python bench.py --summarize-profiles TRACE_DIR FETCH_DIR WRITE_DIR [REQUEST_DIR] [--workload W]
reads rocprofv3 CSV output (kernel trace + stats, FETCH_SIZE pass, WRITE_SIZE pass and, if given,
a pass of read-request counts by size, each from a run with --copy-calibration), prints a text
summary and writes profiles/counters_<W>.json.  With the request counts the read bytes are
counted directly (128-, 64- and 32-byte requests times their sizes) and the copy-calibrated
FETCH_SIZE is kept beside them as a cross-check.
"""
from __future__ import annotations

import argparse
import csv
import ctypes
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
CEILING_LIB = os.path.join(ROOT, "bit_adamw_step_amd", "libadamw4_ceiling.so")
PROBE_EXE = os.path.join(ROOT, "bit_adamw_step_amd", "hbm_mix_probe")
STEP_KERNEL = "adamw4::step_kernel"
CALIB_BYTES = 4 << 30          # the --copy-calibration copy: 4 GiB read + 4 GiB written


def kernel_hash() -> str:
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def shard_len(n: int, shard_of: int) -> int:
    """Length of rank 0's piece when a tensor of n values is split into shard_of pieces at
    128-value block boundaries."""
    if shard_of <= 1:
        return n
    return min(n, -(-n // (shard_of * 128)) * 128)


def algorithmic_bytes(w, shard_of: int = 1, bf16_copy: bool = False) -> tuple[int, int, int]:
    """(bytes per launch, quantized values, FP32-state values) of the launch's entries: the
    whole tensors, or rank 0's pieces with shard_of > 1; a BF16 weight copy adds 2 B/value."""
    gb = 2 if w.grad_dtype == "bf16" else 4
    q = f = total = 0
    for s in w.specs:
        n = shard_len(s.numel, shard_of)
        nblk = (n + 127) // 128
        if bf16_copy:
            total += 2 * n
        if s.numel >= 4096 and not (s.flags & 1):
            q += n
            if s.flags & 4:   # FP32 m: w r/w, grad, m r/w, v codes r/w, 2 v-scale words per block
                total += n * (8 + gb + 8 + 1) + nblk * 8
            else:             # w r/w, grad, m and v codes r/w, 4 scale words per block
                total += n * (8 + gb + 2) + nblk * 16
        else:
            f += n
            total += n * (8 + gb + 16)   # w r/w, grad, FP32 m and v r/w
    return total, q, f


def pct(xs, p):
    s = sorted(xs)
    k = (len(s) - 1) * p / 100.0
    lo = int(k)
    hi = min(lo + 1, len(s) - 1)
    return s[lo] + (s[hi] - s[lo]) * (k - lo)


def setup(w, device, shard_of: int = 1, bf16_copy: bool = False):
    """The workload's parameter list with its state; with shard_of > 1, rank 0's piece of every
    tensor (quantized pieces flagged as shards, keyed by the tensor's index)."""
    import torch
    import workloads as W
    import bit_adamw_step_amd as A
    params, grads, flags = [], [], []
    for i, s in enumerate(w.specs):
        L = shard_len(s.numel, shard_of)
        p = W.make_param(s, i, device)
        g = W.make_grad(w, s, i, 1, device)
        params.append(p if L == s.numel else p[:L].clone())
        grads.append(g if L == s.numel else g[:L].clone())
        del p, g
        f = s.flags
        if shard_of > 1 and A.is_quantized(s.numel, s.flags):
            f |= A.T_SHARD
        flags.append(f)
    copies = [torch.zeros(p.numel(), dtype=torch.bfloat16, device=device) for p in params] \
        if bf16_copy else None
    keys = list(range(len(params))) if shard_of > 1 else None
    pl = A.ParamList(params, grads, flags, bf16_copies=copies, keys=keys)
    v0 = None
    if w.v0_kind != "zeros":
        v0 = [W.make_v0(w, s, i, device)[:shard_len(s.numel, shard_of)].clone()
              for i, s in enumerate(w.specs)]
    pl.init(w.mode_at(1), None, v0)
    del v0
    torch.cuda.synchronize()
    return pl


def timed_schedule(w, K: int) -> list[int]:
    return [max(1, round((k + 1) * w.steps / K)) for k in range(K)]


V_MODES = {"zip": 0, "eden": 1, "rtn": 2, "ssr": 3, "prtn": 4, "baseline": 5}


def run_gpu(w, steps: int, warmup: int, device, v_mode: str | None = None, shard_of: int = 1,
            bf16_copy: bool = False):
    import torch
    import bit_adamw_step_amd as A
    mode_at = (lambda t: V_MODES[v_mode]) if v_mode else w.mode_at
    pl = setup(w, device, shard_of, bf16_copy)
    stream = torch.cuda.current_stream()
    prev = mode_at(1)

    def hp(t):
        nonlocal prev
        m = mode_at(t)
        h = A.hparams(step=t, mode=m, prev_mode=prev, sr_head=w.sr_head_at(t), seed=0)
        prev = m
        return h

    for t in range(1, warmup + 1):
        pl.step(hp(t), stream)
    torch.cuda.synchronize()
    ts = timed_schedule(w, steps)
    hps = [hp(t) for t in ts]
    # the timed job: K steps back to back, nothing else on the stream (timing events recorded
    # between launches cost the GPU tens of microseconds each, which small lists would feel)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for h in hps:
        pl.step(h, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the same K steps again with HIP events around each launch: per-launch times
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in ts]
    for (a, b), h in zip(ev, hps):
        a.record(stream)
        pl.step(h, stream)
        b.record(stream)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in ev]   # ms per launch
    return pl, ts, per, wall


def run_optimizer(w, steps: int, warmup: int, device) -> dict:
    """The torch front end end to end on the workload as a BF16 model: BF16 parameters and
    grads, FP32 masters in the optimizer state, norm and LM-head tensors in their own groups
    (one library call for all three).  Times opt.step() on the GPU (events) and on the host."""
    import torch
    import workloads as W
    from bit_adamw_step_amd.optim import AdamW4bit
    params, groups = [], {"plain": [], "norm": [], "head": []}
    for i, s in enumerate(w.specs):
        p = W.make_param(s, i, device).to(torch.bfloat16)
        p.grad = W.make_grad(w, s, i, 1, device).to(torch.bfloat16)
        params.append(p)
        groups["norm" if s.flags & 1 else "head" if s.flags & 2 else "plain"].append(p)
    opt = AdamW4bit([{"params": groups["plain"]}, {"params": groups["norm"], "norm": True},
                     {"params": groups["head"], "head": True}], lr=1e-3, weight_decay=0.1,
                    mode="zip-sr", total_steps=w.steps, seed=0)
    for _ in range(warmup):
        opt.step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    host = []
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        h0 = time.perf_counter()
        opt.step()
        host.append(time.perf_counter() - h0)
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu = [a.elapsed_time(b) for a, b in ev]
    n = sum(p.numel() for p in params)
    return {"values": n, "gpu_ms_median": round(pct(gpu, 50), 4),
            "host_ms_median": round(1000 * pct(host, 50), 4),
            "wall_ms_per_step": round(1000 * wall / steps, 4),
            "bytes_per_value": 14.125,
            "note": "BF16 params and grads, FP32 masters; 14.125 B/value (master r/w 8, BF16 copy 2, "
                    "grad 2, codes 2, scales 0.125)"}


def ceiling(q: int, device, reps: int = 5) -> dict | None:
    """Time the same-byte-mix streaming kernel over q quantized values in flat buffers, at 2
    and 4 workgroups per CU (256-block chunks); report the faster."""
    import torch
    if not os.path.exists(CEILING_LIB) or q < 128:
        return None
    L = ctypes.CDLL(CEILING_LIB)
    P = ctypes.c_void_p
    L.adamw4_ceiling_mix.argtypes = [P, P, P, P, P, P, ctypes.c_int64, ctypes.c_int32,
                                     ctypes.c_int32, P]
    L.adamw4_ceiling_mix.restype = ctypes.c_int
    nb = q // 128
    n = nb * 128
    wv = torch.zeros(n, dtype=torch.float32, device=device)
    g = torch.zeros(n, dtype=torch.bfloat16, device=device)
    mc = torch.zeros(n // 8, dtype=torch.int32, device=device)
    vc = torch.zeros(n // 8, dtype=torch.int32, device=device)
    sm = torch.ones(nb, dtype=torch.float32, device=device)
    sv = torch.ones(nb, dtype=torch.float32, device=device)
    stream = torch.cuda.current_stream()
    cus = torch.cuda.get_device_properties(device).multi_processor_count
    best = None
    for grid, chunk in ((2 * cus, 256), (4 * cus, 256)):
        args = [wv.data_ptr(), g.data_ptr(), mc.data_ptr(), vc.data_ptr(), sm.data_ptr(),
                sv.data_ptr(), nb, grid, chunk, ctypes.c_void_p(stream.cuda_stream)]
        for _ in range(2):
            if L.adamw4_ceiling_mix(*args) != 0:
                raise RuntimeError("ceiling kernel launch failed")
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for a, b in ev:
            a.record(stream)
            L.adamw4_ceiling_mix(*args)
            b.record(stream)
        torch.cuda.synchronize()
        ms = sum(a.elapsed_time(b) for a, b in ev) / reps
        if best is None or ms < best[0]:
            best = (ms, grid, chunk)
    ms, grid, chunk = best
    byts = n * 12 + nb * 16
    del wv, g, mc, vc, sm, sv
    torch.cuda.empty_cache()
    return {"kernel": "same-byte-mix streaming (12.125 B/value, step access pattern, "
                      "non-temporal weights, grads and codes)",
            "values": n, "ms": round(ms, 4), "GBs": round(byts / (ms / 1000) / 1e9, 1),
            "grid": grid, "chunk_blocks": chunk}


def cpu_baseline(w, pl, budget_s: float = 30.0):
    """The oracle, unchanged, stepping the workload's tensors in list order from host copies of
    the GPU's current state (copies not timed) until about budget_s of oracle time, at the last
    step of the schedule.  Also times the oracle on one thread over the first 4M values."""
    import numpy as np
    import torch
    import oracle as orc
    import bit_adamw_step_amd as A
    orc.build()
    L = orc.lib()
    threads = L.orc_threads()
    specs = w.specs
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

    def run(i, e0, cnt):
        w_, g, st = host(i, e0, cnt)
        t0 = time.perf_counter()
        orc.step_tensor(w_, g, st, hp, pos=i, head=bool(specs[i].flags & 2), e0=e0, n=specs[i].numel)
        return time.perf_counter() - t0

    t_total, n_total, done = 0.0, 0, 0
    for i, s in enumerate(specs):
        if t_total >= budget_s:
            break
        t_total += run(i, 0, s.numel)
        n_total += s.numel
        done += 1
    # one thread, for scale
    q0 = next(i for i, s in enumerate(specs) if A.is_quantized(s.numel, s.flags))
    cnt1 = min(specs[q0].numel, 1 << 22)
    L.orc_set_threads(1)
    try:
        t1 = run(q0, 0, cnt1)
    finally:
        L.orc_set_threads(threads)
    whole = done == len(specs)
    what = ("the whole list" if whole else f"the first {done} of {len(specs)} tensors")
    return {"value": round(n_total / t_total / 1e9, 6), "unit": "Gparams/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{what} ({n_total} values), one oracle step at t={w.steps} from the GPU's "
                      f"state, {t_total:.1f} s of oracle time on {threads} threads",
            "value_1thread": round(cnt1 / t1 / 1e9, 6)}


def traffic_from_profile(wname: str):
    """(HBM bytes per launch, how they were counted) from the stored counters, or (None, None)
    when there are none for the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"counters_{wname}.json")
    if not os.path.exists(path):
        return None, None
    d = json.load(open(path))
    if d.get("kernel_sha") != kernel_hash():
        return None, None
    return d.get("hbm_bytes_per_launch"), d.get("traffic_method")


# ---------------------------------------------------------------------------------------------
# rocprofv3 summaries
# ---------------------------------------------------------------------------------------------

def _csv(d: str, name: str) -> list[dict]:
    for root, _, files in os.walk(d):
        for f in files:
            if f.endswith(name):
                return list(csv.DictReader(open(os.path.join(root, f))))
    raise FileNotFoundError(f"no *{name} under {d}")


def _is_copy(name: str) -> bool:
    return "copyBuffer" in name or "copy" in name.lower() and "adamw4" not in name


def _per_dispatch(d: str, counters) -> dict:
    """{dispatch id: (kernel name, {counter: value summed over instances})}"""
    per = {}
    for r in _csv(d, "counter_collection.csv"):
        if r["Counter_Name"] not in counters:
            continue
        nm, vals = per.setdefault(int(r["Dispatch_Id"]), (r["Kernel_Name"], {}))
        vals[r["Counter_Name"]] = vals.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return per


REQ_COUNTERS = ("TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum",
                "TCC_EA0_RDREQ_128B_sum")


def summarize_profiles(trace_dir: str, fetch_dir: str, write_dir: str, wname: str,
                       req_dir: str | None = None) -> None:
    import workloads as W
    w = W.WORKLOADS[wname]
    bytes_alg, q, f = algorithmic_bytes(w)
    stats = _csv(trace_dir, "kernel_stats.csv")
    trace = _csv(trace_dir, "kernel_trace.csv")
    step = [r for r in trace if STEP_KERNEL in r["Kernel_Name"]]
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6 for r in step]
    print(f"## rocprofv3 kernel trace ({wname}: {w.numel} values, {len(w.specs)} tensors)\n")
    print("| kernel | calls | avg ms | min ms | max ms | share % |")
    print("|---|---|---|---|---|---|")
    for r in stats[:8]:
        nm = r["Name"]
        nm = nm if len(nm) < 60 else nm[:57] + "..."
        print(f"| {nm} | {r['Calls']} | {float(r['AverageNs']) / 1e6:.4f} | "
              f"{float(r['MinNs']) / 1e6:.4f} | {float(r['MaxNs']) / 1e6:.4f} | {r['Percentage']} |")
    if step:
        r0 = step[0]
        avg = sum(durs) / len(durs)
        print(f"\nstep_kernel: {len(durs)} dispatches, mean {avg:.4f} ms, "
              f"{int(r0['Grid_Size_X']) // int(r0['Workgroup_Size_X'])} workgroups of "
              f"{r0['Workgroup_Size_X']} threads, VGPR {r0['VGPR_Count']}, "
              f"SGPR {r0['SGPR_Count']}, LDS {r0['LDS_Block_Size']} B, scratch {r0['Scratch_Size']} B")
        print(f"algorithmic bytes per launch {bytes_alg} -> {bytes_alg / (avg / 1000) / 1e9:.1f} GB/s "
              f"({100 * bytes_alg / (avg / 1000) / 1e9 / PEAK_HBM_GBS:.2f}% of {PEAK_HBM_GBS:.0f})")
    out = {"workload": wname, "kernel_sha": kernel_hash(), "algorithmic_bytes_per_launch": bytes_alg}
    for label, d, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        rows = [r for r in _csv(d, "counter_collection.csv") if r["Counter_Name"] == counter]
        per = {}
        for r in rows:
            per.setdefault(int(r["Dispatch_Id"]), [r["Kernel_Name"], 0.0])[1] += float(r["Counter_Value"])
        stepv = [v for nm, v in per.values() if STEP_KERNEL in nm]
        copyv = [v for nm, v in per.values() if _is_copy(nm)]
        if not stepv or not copyv:
            print(f"\n{counter}: step or calibration copy dispatches missing")
            return
        cal_kib = max(copyv)                     # the 4 GiB copy is the largest copy dispatch
        factor = (CALIB_BYTES / 1024) / cal_kib  # true KiB per counted KiB
        kib = sum(stepv) / len(stepv)
        out[f"{label}_kib_per_dispatch_raw"] = kib
        out[f"{label}_calibration_copy_kib_raw"] = cal_kib
        out[f"{label}_calibration_factor"] = factor
        out[f"{label}_bytes_per_launch"] = kib * 1024 * factor
        print(f"\n{counter}: step_kernel {len(stepv)} dispatches, mean {kib:.1f} KiB raw; "
              f"calibration copy of {CALIB_BYTES} B {'read' if label == 'fetch' else 'written'} "
              f"counted {cal_kib:.1f} KiB -> factor {factor:.4f}; "
              f"step {kib * 1024 * factor / 1e9:.3f} GB per launch")
    out["hbm_bytes_per_launch"] = out["fetch_bytes_per_launch"] + out["write_bytes_per_launch"]
    out["traffic_method"] = ("FETCH_SIZE x copy calibration + WRITE_SIZE x copy calibration "
                             "(rocprofv3, per step dispatch)")
    if req_dir:
        per = _per_dispatch(req_dir, REQ_COUNTERS)
        stepr = [v for nm, v in per.values() if STEP_KERNEL in nm]
        copyr = [v for nm, v in per.values() if _is_copy(nm)]
        def rbytes(v):
            return (128 * v["TCC_EA0_RDREQ_128B_sum"] + 64 * v["TCC_EA0_RDREQ_64B_sum"] +
                    32 * v["TCC_EA0_RDREQ_32B_sum"])
        mean = lambda xs: sum(xs) / len(xs)
        rb = mean([rbytes(v) for v in stepr])
        unsized = mean([v["TCC_EA0_RDREQ_sum"] - v["TCC_EA0_RDREQ_32B_sum"] - v["TCC_EA0_RDREQ_64B_sum"]
                        - v["TCC_EA0_RDREQ_128B_sum"] for v in stepr])
        cal = max(rbytes(v) for v in copyr) if copyr else None
        out["read_bytes_per_launch_from_requests"] = rb
        out["read_requests_unsized_per_launch"] = unsized
        out["calibration_copy_read_bytes_from_requests"] = cal
        out["fetch_vs_requests"] = out["fetch_bytes_per_launch"] / rb
        out["hbm_bytes_per_launch"] = rb + out["write_bytes_per_launch"]
        out["traffic_method"] = ("read: TCC_EA0_RDREQ_128B*128 + RDREQ_64B*64 + RDREQ_32B*32; "
                                 "write: WRITE_SIZE (64- and 32-byte write requests); the "
                                 "copy-calibrated FETCH_SIZE agrees within "
                                 f"{abs(out['fetch_vs_requests'] - 1) * 100:.2f}%")
        print(f"\nread requests by size: step {len(stepr)} dispatches, {rb / 1e9:.3f} GB per launch "
              f"({unsized:.0f} requests of no listed size); calibration copy "
              f"{(cal or 0) / 1e9:.3f} GB of {CALIB_BYTES / 1e9:.3f} GB read; copy-calibrated "
              f"FETCH_SIZE / request bytes = {out['fetch_vs_requests']:.5f}")
    print(f"\nHBM traffic per launch {out['hbm_bytes_per_launch'] / 1e9:.3f} GB vs algorithmic "
          f"{bytes_alg / 1e9:.3f} GB (ratio {out['hbm_bytes_per_launch'] / bytes_alg:.4f}); "
          f"{out['traffic_method']}")
    path = os.path.join(ROOT, "profiles", f"counters_{wname}.json")
    os.makedirs(os.path.dirname(path), exist_ok=True)
    json.dump(out, open(path, "w"), indent=1)
    print(f"wrote {os.path.relpath(path, ROOT)}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama2b7")
    ap.add_argument("--v-mode", choices=sorted(V_MODES), default=None,
                    help="v encoder for every step (default: the workload's own schedule)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=30.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 4 GiB device copy (counter calibration under rocprofv3)")
    ap.add_argument("--bf16-copy", action="store_true",
                    help="the step also writes a BF16 copy of the updated weights")
    ap.add_argument("--shard-of", type=int, default=1, metavar="N",
                    help="time rank 0's share of an N-way 128-aligned split of every tensor")
    ap.add_argument("--optimizer", action="store_true",
                    help="also time the torch front end end to end on the workload as a BF16 model")
    ap.add_argument("--summarize-profiles", nargs="+", metavar="DIR",
                    help="TRACE FETCH WRITE [REQUESTS] rocprofv3 output directories")
    ap.add_argument("--hbm-study", nargs="?", const="", default=None, metavar="FILTER",
                    help="run the byte-mix bandwidth probe (all patterns, or those matching FILTER)")
    ap.add_argument("--hbm-reps", type=int, default=5)
    args = ap.parse_args()
    if args.hbm_study is not None:
        import subprocess
        if not os.path.exists(PROBE_EXE):
            sys.exit(f"{PROBE_EXE} is not built (run the package's build step)")
        cmd = [PROBE_EXE] + ([args.hbm_study, str(args.hbm_reps)] if args.hbm_study else [])
        sys.exit(subprocess.run(cmd).returncode)
    if args.summarize_profiles:
        dirs = args.summarize_profiles
        if len(dirs) not in (3, 4):
            ap.error("--summarize-profiles takes TRACE FETCH WRITE [REQUESTS]")
        summarize_profiles(dirs[0], dirs[1], dirs[2], args.workload, dirs[3] if len(dirs) == 4 else None)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the 4-bit AdamW step needs no communication, a sharded "
              "run is N copies of rank 0's share (see --shard-of); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as W
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    device = torch.device("cuda:0")
    w = W.WORKLOADS[args.workload]
    print(f"# setup {w.name}: {len(w.specs)} tensors, {w.numel} values", file=sys.stderr, flush=True)
    pl, ts, per, wall = run_gpu(w, args.steps, args.warmup, device, args.v_mode, args.shard_of,
                                args.bf16_copy)
    print(f"# timed {len(per)} steps: mean {sum(per) / len(per):.4f} ms", file=sys.stderr, flush=True)
    if args.copy_calibration:
        a = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device=device)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b
        torch.cuda.empty_cache()
    bytes_alg, q, f = algorithmic_bytes(w, args.shard_of, args.bf16_copy)
    traffic, traffic_method = (traffic_from_profile(w.name) if args.shard_of == 1 and
                               not args.bf16_copy and not args.v_mode else (None, None))
    values = q + f
    ms = sum(per) / len(per)
    ms_wall = wall * 1000 / len(per)
    gparams = values * len(per) / wall / 1e9
    achieved = bytes_alg / (ms / 1000) / 1e9
    sr = [p for t, p in zip(ts, per) if w.sr_head_at(t)]
    rtn = [p for t, p in zip(ts, per) if not w.sr_head_at(t)]
    ceil = None if args.no_ceiling else ceiling(q, device)
    if ceil:
        ceil["step_frac_of_ceiling"] = round(achieved / ceil["GBs"], 4)
        print(f"# ceiling {ceil['GBs']} GB/s", file=sys.stderr, flush=True)
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
            "workload": w.name, "values": values, "tensors": len(w.specs),
            "shard_of": args.shard_of, "bf16_copy": args.bf16_copy,
            "quantized_values": q, "fp32_state_values": f, "grad_dtype": w.grad_dtype,
            "v_mode": args.v_mode or w.mode_schedule, "timed_t": [ts[0], ts[-1]],
            "ms_launch_median": round(pct(per, 50), 4), "ms_launch_p10": round(pct(per, 10), 4),
            "ms_launch_p90": round(pct(per, 90), 4),
            "ms_launch_rtn_phase": round(sum(rtn) / len(rtn), 4) if rtn else None,
            "ms_launch_sr_head_phase": round(sum(sr) / len(sr), 4) if sr else None,
            "algorithmic_bytes_per_launch": bytes_alg,
            "achieved_hbm_GBs": round(achieved, 1),
            "pct_of_peak_hbm": round(100 * achieved / PEAK_HBM_GBS, 2),
        },
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic, "traffic_method": traffic_method},
        "ceiling": ceil,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline and args.shard_of == 1:
        out["cpu_baseline"] = cpu_baseline(w, pl, args.cpu_budget)
    if args.optimizer:
        del pl
        torch.cuda.empty_cache()
        out["optimizer"] = run_optimizer(w, args.steps, args.warmup, device)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
