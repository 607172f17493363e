"""Seeded synthetic workloads for the 4-bit AdamW step: parameter-list shapes and input
generators (weights, gradients, initial moments).  Holds no optimizer arithmetic; both the
HIP-path tests/benchmark and the oracle-side checks draw their inputs from here.

Lists (no public dataset or checkpoint is involved; these stand in for the pages' GPT- and
Llama-style models of 130M-2.7B parameters, zhichai.net summary and kongchang.com
"Experimental Results"):
  flat1m  one FP32 tensor of 1,048,576 values, FP32 grads N(0, 1e-3)
  gpt130m GPT d=768 x12, 4d MLP, vocab 50304, untied head, LayerNorm w/b in FP32 states;
          BF16 grads N(0,1e-3) with a fixed seeded 1% of each matrix's rows scaled by 1e-4
  gpt834m same family d=1536 x24; v0 = 10^U(-20,-4), m0 = 0 (ZE-EDEN)
  llama2b7 Llama d=2560 x32, SwiGLU 6912, vocab 32000, untied head, RMSNorm states FP32;
          BF16 grads N(0, 1e-3)
  stress  one 2^30-value FP32 tensor + 2000 tensors of U{64..4095} values (FP32 states);
          FP32 grads 1e-3 * Student-t(3) with 30% exact zeros
  study834m the 834M GPT shapes with FP32 first moments on the quantized tensors and the
          zero-inclusive v rules in turn (ZIP-SR, state RTN, state SR, preconditioner RTN), the
          configuration of the pages' controlled study (learnaivisually.com explainer)
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

T_NORM, T_HEAD, T_FP32_M = 1, 2, 4


@dataclass(frozen=True)
class PSpec:
    name: str
    shape: tuple
    flags: int = 0
    init: str = "normal"     # normal: N(0, 0.02); ones; zeros

    @property
    def numel(self) -> int:
        n = 1
        for s in self.shape:
            n *= s
        return n


def gpt_list(d: int, layers: int, vocab: int) -> list[PSpec]:
    L = [PSpec("wte", (vocab, d))]
    for i in range(layers):
        L += [PSpec(f"h{i}.ln1.w", (d,), T_NORM, "ones"), PSpec(f"h{i}.ln1.b", (d,), T_NORM, "zeros"),
              PSpec(f"h{i}.qkv", (3 * d, d)), PSpec(f"h{i}.o", (d, d)),
              PSpec(f"h{i}.ln2.w", (d,), T_NORM, "ones"), PSpec(f"h{i}.ln2.b", (d,), T_NORM, "zeros"),
              PSpec(f"h{i}.fc", (4 * d, d)), PSpec(f"h{i}.proj", (d, 4 * d))]
    L += [PSpec("lnf.w", (d,), T_NORM, "ones"), PSpec("lnf.b", (d,), T_NORM, "zeros"),
          PSpec("lm_head", (vocab, d), T_HEAD)]
    return L


def llama_list(d: int, layers: int, hidden: int, vocab: int) -> list[PSpec]:
    L = [PSpec("emb", (vocab, d))]
    for i in range(layers):
        L += [PSpec(f"l{i}.attn_norm", (d,), T_NORM, "ones"),
              PSpec(f"l{i}.q", (d, d)), PSpec(f"l{i}.k", (d, d)), PSpec(f"l{i}.v", (d, d)),
              PSpec(f"l{i}.o", (d, d)), PSpec(f"l{i}.mlp_norm", (d,), T_NORM, "ones"),
              PSpec(f"l{i}.gate", (hidden, d)), PSpec(f"l{i}.up", (hidden, d)),
              PSpec(f"l{i}.down", (d, hidden))]
    L += [PSpec("norm", (d,), T_NORM, "ones"), PSpec("lm_head", (vocab, d), T_HEAD)]
    return L


def with_fp32_m(specs) -> list[PSpec]:
    """The same list with the first moment kept in FP32 on every non-norm tensor."""
    return [s if s.flags & T_NORM else PSpec(s.name, s.shape, s.flags | T_FP32_M, s.init)
            for s in specs]


def stress_list(seed: int = 5) -> list[PSpec]:
    rng = np.random.default_rng(seed)
    sizes = rng.integers(64, 4096, 2000)
    return [PSpec("big", (1 << 30,))] + [PSpec(f"tiny{i}", (int(n),)) for i, n in enumerate(sizes)]


@dataclass(frozen=True)
class Workload:
    name: str
    specs: tuple
    grad_dtype: str          # "f32" | "bf16"
    mode_schedule: str       # "zip" | "eden" | "alternate" | "study" | "baseline"
    steps: int
    data_seed: int
    grad_kind: str = "normal"   # normal | rowscaled | student_t
    v0_kind: str = "zeros"      # zeros | loguniform

    @property
    def numel(self) -> int:
        return sum(s.numel for s in self.specs)

    def mode_at(self, t: int) -> int:
        """v encoder at step t (0 ZIP-SR, 1 ZE-EDEN, 5 the baseline); 'alternate' = ZIP-SR at
        odd t."""
        if self.mode_schedule == "zip":
            return 0
        if self.mode_schedule == "eden":
            return 1
        if self.mode_schedule == "study":   # ZIP-SR, state RTN, state SR, preconditioner RTN
            return (0, 2, 3, 4)[t % 4]
        if self.mode_schedule == "baseline":   # zero-free codebook, nearest level, no rescale
            return 5
        return 0 if t % 2 == 1 else 1

    def sr_head_at(self, t: int) -> int:
        """LM-head m stochastic rounding over the last 10% of the steps (t > 0.9 T)."""
        return int(10 * t > 9 * self.steps)


WORKLOADS = {
    "flat1m": Workload("flat1m", (PSpec("w", (1 << 20,)),), "f32", "zip", 10, 1001),
    "gpt130m": Workload("gpt130m", tuple(gpt_list(768, 12, 50304)), "bf16", "zip", 100, 1002,
                        grad_kind="rowscaled"),
    "gpt834m": Workload("gpt834m", tuple(gpt_list(1536, 24, 50304)), "bf16", "eden", 50, 1003,
                        v0_kind="loguniform"),
    "llama2b7": Workload("llama2b7", tuple(llama_list(2560, 32, 6912, 32000)), "bf16", "zip", 200,
                         1004),
    "stress": Workload("stress", tuple(stress_list()), "f32", "alternate", 20, 1005,
                       grad_kind="student_t"),
    "study834m": Workload("study834m", tuple(with_fp32_m(gpt_list(1536, 24, 50304))), "bf16", "study",
                          40, 1006),
    "baseline130m": Workload("baseline130m", tuple(gpt_list(768, 12, 50304)), "bf16", "baseline",
                             100, 1007, v0_kind="loguniform"),
}


def quantized_numel(w: Workload) -> int:
    return sum(s.numel for s in w.specs if s.numel >= 4096 and not (s.flags & T_NORM))


# ---------------------------------------------------------------------------------------------
# generators (torch; the same calls serve CPU and GPU tensors)
# ---------------------------------------------------------------------------------------------

def _gen(device, seed: int):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed & 0x7FFFFFFFFFFFFFFF)
    return g


def make_param(spec: PSpec, index: int, device, seed: int = 7):
    """FP32 weights: N(0, 0.02) for matrices, 1 for norm weights, 0 for norm biases."""
    import torch
    if spec.init == "ones":
        return torch.ones(spec.numel, dtype=torch.float32, device=device)
    if spec.init == "zeros":
        return torch.zeros(spec.numel, dtype=torch.float32, device=device)
    g = _gen(device, seed * 1_000_003 + index)
    return torch.randn(spec.numel, generator=g, dtype=torch.float32, device=device).mul_(0.02)


def make_grad(w: Workload, spec: PSpec, index: int, t: int, device, out=None):
    """Gradient of tensor `index` at step t, seeded by (data_seed, t, index)."""
    import torch
    g = _gen(device, (w.data_seed * 100_003 + t) * 65_537 + index)
    n = spec.numel
    if w.grad_kind == "student_t":
        z = torch.randn(n, generator=g, dtype=torch.float32, device=device)
        chi = torch.zeros_like(z)
        for _ in range(3):
            chi.add_(torch.randn(n, generator=g, dtype=torch.float32, device=device).square_())
        x = z.div_(chi.div_(3.0).sqrt_()).mul_(1e-3)
        del chi
        zero = torch.rand(n, generator=g, dtype=torch.float32, device=device) < 0.3
        x.masked_fill_(zero, 0.0)
    else:
        x = torch.randn(n, generator=g, dtype=torch.float32, device=device).mul_(1e-3)
        if w.grad_kind == "rowscaled" and len(spec.shape) == 2:
            rows = spec.shape[0]
            rg = _gen("cpu", w.data_seed * 7919 + index)
            pick = torch.randperm(rows, generator=rg)[: max(1, rows // 100)]
            x.view(spec.shape)[pick.to(device)] *= 1e-4
    dt = torch.bfloat16 if w.grad_dtype == "bf16" else torch.float32
    if out is not None:
        out.copy_(x)
        return out
    return x.to(dt)


def make_v0(w: Workload, spec: PSpec, index: int, device):
    """Initial second moment: zeros, or 10^U(-20,-4) per value."""
    import torch
    if w.v0_kind != "loguniform":
        return None
    g = _gen(device, w.data_seed * 31 + index)
    e = torch.rand(spec.numel, generator=g, dtype=torch.float32, device=device).mul_(-16.0).add_(-4.0)
    return torch.pow(10.0, e)
