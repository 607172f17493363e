"""Helpers for the GPU parity tests: move states between the HIP library's buffers and the
oracle's arrays, replay one step on the oracle, and compare to the acceptance bar:
  - packed codes and block scales bit-exact, except a code may differ where the element made a
    stochastic choice with |u - p| < 1e-6 (the oracle records u and p);
  - weights and FP32 moments within 1e-6 relative of the oracle (the kernel follows the same
    FP32 operation order, so they are expected to be bit-exact; the test reports both).
"""
from __future__ import annotations

import sys

import numpy as np

import bit_adamw_step_amd as A
import oracle as orc

f32 = np.float32
FLIP_TOL = 1e-6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_np(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.detach().cpu().numpy()


def oracle_state(buf: np.ndarray, n: int, flags: int, b0: int = 0, nb: int | None = None) -> orc.State:
    """Oracle State for blocks [b0, b0+nb) of a tensor from its HIP-layout state bytes."""
    off = A.state_layout(n, flags)
    if A.is_quantized(n, flags):
        nbt = (n + 127) // 128
        nb = nbt - b0 if nb is None else nb
        c0, c1 = 64 * b0, min((n + 1) // 2, 64 * (b0 + nb))
        sc = lambda o: buf[o + 4 * b0: o + 4 * (b0 + nb)].view(f32).copy()
        if flags & A.T_FP32_M:
            e0, e1 = 128 * b0, min(n, 128 * (b0 + nb))
            return orc.State(True, None, buf[off[1] + c0: off[1] + c1].copy(), None, sc(off[3]),
                             m=buf[off[0] + 4 * e0: off[0] + 4 * e1].view(f32).copy())
        return orc.State(True, buf[off[0] + c0: off[0] + c1].copy(), buf[off[1] + c0: off[1] + c1].copy(),
                         sc(off[2]), sc(off[3]))
    return orc.State(False, m=buf[off[0]: off[0] + 4 * n].view(f32).copy(),
                     v=buf[off[1]: off[1] + 4 * n].view(f32).copy())


def unpack(codes: np.ndarray, n: int) -> np.ndarray:
    out = np.empty(2 * codes.size, np.uint8)
    out[0::2] = codes & 15
    out[1::2] = codes >> 4
    return out[:n]


class Mismatch(AssertionError):
    pass


def compare_state(name: str, n: int, gpu: orc.State, ref: orc.State, dbg: np.ndarray | None,
                  report: dict) -> None:
    """Codes and scales: bit-exact except permitted stochastic flips; FP32 moments: <= 1e-6 rel."""
    if not ref.quantized:
        for k in ("m", "v"):
            a, b = getattr(gpu, k), getattr(ref, k)
            exact = np.array_equal(a.view(np.uint32), b.view(np.uint32))
            report[f"{name}.{k}_bitexact"] = exact
            if not exact:
                bad = np.abs(a.astype(np.float64) - b) > 1e-6 * np.abs(b.astype(np.float64)) + 1e-30
                if bad.any():
                    raise Mismatch(f"{name}: FP32 {k} differs at {np.nonzero(bad)[0][:8]}")
        return
    cnt = n
    packed = (("vcodes", 0, 1),) if ref.fp32_m else (("mcodes", 2, 3), ("vcodes", 0, 1))
    if ref.fp32_m:
        exact = np.array_equal(gpu.m.view(np.uint32), ref.m.view(np.uint32))
        report[f"{name}.m_bitexact"] = exact
        if not exact:
            bad = np.abs(gpu.m.astype(np.float64) - ref.m) > 1e-6 * np.abs(ref.m.astype(np.float64)) + 1e-30
            if bad.any():
                raise Mismatch(f"{name}: FP32 m differs at {np.nonzero(bad)[0][:8]}")
    for k, col_u, col_p in packed:
        a, b = unpack(getattr(gpu, k), cnt), unpack(getattr(ref, k), cnt)
        diff = np.nonzero(a != b)[0]
        report[f"{name}.{k}_flips"] = int(diff.size)
        if diff.size:
            if dbg is None:
                raise Mismatch(f"{name}: {k} differ at {diff[:8]} (no u/p record)")
            u, p = dbg[diff, col_u], dbg[diff, col_p]
            ok = (p >= 0) & (np.abs(u.astype(np.float64) - p) < FLIP_TOL) & \
                 (np.abs(a[diff].astype(int) - b[diff].astype(int)) == 1)
            if not ok.all():
                j = diff[~ok][:8]
                raise Mismatch(f"{name}: {k} differ beyond permitted flips at {j}: gpu {a[j]} "
                               f"oracle {b[j]} u {dbg[j, col_u]} p {dbg[j, col_p]}")
        if cnt % 2 == 1:
            assert getattr(gpu, k)[-1] >> 4 == 0, f"{name}: {k} padding nibble not zero"
    for k in (("vscale",) if ref.fp32_m else ("mscale", "vscale")):
        a, b = getattr(gpu, k), getattr(ref, k)
        if not np.array_equal(a.view(np.uint32), b.view(np.uint32)):
            j = np.nonzero(a.view(np.uint32) != b.view(np.uint32))[0][:8]
            raise Mismatch(f"{name}: {k} differ at blocks {j}: gpu {a[j]} oracle {b[j]}")


def compare_weights(name: str, w_gpu: np.ndarray, w_ref: np.ndarray, report: dict) -> None:
    exact = np.array_equal(w_gpu.view(np.uint32), w_ref.view(np.uint32))
    report[f"{name}.w_bitexact"] = exact
    if not exact:
        rel = np.abs(w_gpu.astype(np.float64) - w_ref) / np.maximum(np.abs(w_ref.astype(np.float64)), 1e-30)
        bad = np.abs(w_gpu.astype(np.float64) - w_ref) > 1e-6 * np.abs(w_ref.astype(np.float64)) + 1e-12
        report[f"{name}.w_max_rel"] = float(rel.max())
        if bad.any():
            j = np.nonzero(bad)[0][:8]
            raise Mismatch(f"{name}: weights differ at {j}: gpu {w_gpu[j]} oracle {w_ref[j]}")


def compare_bf16_copy(name: str, copy: np.ndarray, w_ref: np.ndarray, w_gpu: np.ndarray) -> None:
    """The BF16 copy is the oracle's round-to-nearest-even of the oracle's weights: bit-exact
    where the weights are (one BF16 step allowed where the weights differ within tolerance)."""
    exp = orc.bf16_rne(w_ref)
    same_w = w_gpu.view(np.uint32) == w_ref.view(np.uint32)
    bad = (copy != exp) & (same_w | (np.abs(copy.astype(np.int32) - exp.astype(np.int32)) > 1))
    if bad.any():
        j = np.nonzero(bad)[0][:8]
        raise Mismatch(f"{name}: BF16 copy differs at {j}: gpu {copy[j]} oracle {exp[j]}")


class GpuList:
    """A parameter list on the GPU with its states, plus host snapshots for replay."""

    def __init__(self, sizes, flags, grad_dtypes, device="cuda", seed=0, copies=None):
        import torch
        self.n = list(sizes)
        self.flags = list(flags)
        self.params, self.grads = [], []
        g = torch.Generator(device="cpu")
        g.manual_seed(seed)
        for n, gd in zip(self.n, grad_dtypes):
            self.params.append((torch.randn(n, generator=g) * 0.02).to(device))
            self.grads.append(torch.zeros(n, dtype=torch.bfloat16 if gd == "bf16" else torch.float32,
                                          device=device))
        # optional BF16 copies of the updated weights (copies[i] True: tensor i gets one)
        self.copies = [torch.zeros(n, dtype=torch.bfloat16, device=device) if c else None
                       for n, c in zip(self.n, copies or [False] * len(self.n))]
        self.pl = A.ParamList(self.params, self.grads, self.flags,
                              bf16_copies=self.copies if copies else None)

    def set_grads(self, t, seed=0, scale=1e-3, zero_frac=0.0):
        import torch
        g = torch.Generator(device="cpu")
        g.manual_seed(seed * 10007 + t)
        for gr in self.grads:
            x = torch.randn(gr.numel(), generator=g) * scale
            if zero_frac:
                x[torch.rand(gr.numel(), generator=g) < zero_frac] = 0
            gr.copy_(x.to(gr.dtype))

    def snapshot(self):
        import torch
        torch.cuda.synchronize()
        return ([to_np(p).copy() for p in self.params], [to_np(g).copy() for g in self.grads],
                [to_np(s).copy() for s in self.pl.states])

    def replay_and_compare(self, before, hp_kwargs, report, tag=""):
        """Oracle step from `before`; compare with the current GPU tensors."""
        ws, gs, ss = before
        w_now, _, s_now = self.snapshot()
        ohp = orc.HParams(**hp_kwargs)
        for i, n in enumerate(self.n):
            f = self.flags[i]
            st = oracle_state(ss[i], n, f)
            w = ws[i].copy()
            dbg = orc.step_tensor(w, gs[i], st, ohp, pos=i, head=bool(f & A.T_HEAD), dbg=True)
            name = f"{tag}t{i}(n={n},f={f})"
            compare_weights(name, w_now[i], w, report)
            if self.copies[i] is not None:
                compare_bf16_copy(name, to_np(self.copies[i]), w, w_now[i])
            compare_state(name, n, oracle_state(s_now[i], n, f), st, dbg, report)
