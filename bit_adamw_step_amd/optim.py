"""``torch.optim.Optimizer`` front end of the fused 4-bit AdamW step.

The step itself is one library call (``adamw4_step``) per set of groups sharing their
hyperparameters; this module only keeps the per-parameter state buffers, builds the tensor
lists and carries the step counter, the v encoder and the LM-head switch between calls.

Methods (daiwk.github.io "ZIP-SR / ZE-EDEN: 4-bit AdamW state quantization", "Core equation"
and "Paper method and evidence"; learnaivisually.com "ZIP-SR 4-bit AdamW", ZE-EDEN / LM-head
paragraph): m in NF4, v by ZIP-SR or ZE-EDEN, one FP32 scale per 128 values, FP32 states for
normalization layers and tensors under 4096 elements, and stochastic rounding of the LM head's
m over the last tenth of training.

Parameters may be FP32 (updated in place; they are the master weights) or BF16.  A BF16
parameter gets an FP32 master copy in the optimizer state; the step reads the BF16 gradient,
updates the master and writes the rounded weight back into the parameter in the same pass.
"""
from __future__ import annotations

import torch

import bit_adamw_step_amd as A

MODES = {"zip-sr": A.ZIP_SR, "ze-eden": A.ZE_EDEN, "state-rtn": A.V_RTN, "state-sr": A.V_SSR,
         "precond-rtn": A.V_PRTN, "baseline": A.V_ZE_RTN}


def mode_id(mode) -> int:
    """adamw4_mode of a mode name (or id)."""
    if isinstance(mode, int) and mode in MODES.values():
        return mode
    if mode in MODES:
        return MODES[mode]
    raise ValueError(f"unknown v encoder {mode!r}; one of {sorted(MODES)}")


def sr_head_at(t: int, total_steps: int | None) -> int:
    """LM-head m stochastic rounding over the last 10% of training: t > 0.9 T."""
    return int(total_steps is not None and 10 * t > 9 * total_steps)


class AdamW4bit(torch.optim.Optimizer):
    """AdamW with 4-bit optimizer states on MI355X.

    Group options: lr, betas, eps, weight_decay, mode (a name of ``MODES``), norm (FP32 states:
    normalization layers), head (the LM head), fp32_m (keep m in FP32, the controlled study's
    setting).  Optimizer options: seed (RNG key), total_steps (for the LM-head switch; None:
    never).  Each parameter's RNG key is its position over all groups, so groups stepped in
    separate calls never share random streams.
    """

    def __init__(self, params, lr: float = 1e-3, betas=(0.9, 0.999), eps: float = 1e-8,
                 weight_decay: float = 0.1, mode="zip-sr", norm: bool = False,
                 head: bool = False, fp32_m: bool = False, seed: int = 0,
                 total_steps: int | None = None):
        defaults = dict(lr=lr, betas=tuple(betas), eps=eps, weight_decay=weight_decay,
                        mode=mode, norm=norm, head=head, fp32_m=fp32_m)
        super().__init__(params, defaults)
        for g in self.param_groups:
            mode_id(g["mode"])
            for p in g["params"]:
                self._check_param(p)
        self.seed = int(seed)
        self.total_steps = total_steps
        self._arrays: dict = {}   # pointer signature -> tensor array of the last few calls

    @staticmethod
    def _check_param(p: torch.Tensor) -> None:
        if not p.is_cuda:
            raise ValueError("AdamW4bit needs CUDA (HIP) parameters: the step runs only in the "
                             "library's GPU kernels")
        if p.dtype not in (torch.float32, torch.bfloat16) or not p.is_contiguous():
            raise ValueError("parameters must be contiguous float32 or bfloat16")

    @staticmethod
    def _flags(group: dict) -> int:
        f = A.T_KEYED
        if group["norm"]:
            f |= A.T_NORM
        if group["head"]:
            f |= A.T_HEAD
        if group["fp32_m"]:
            f |= A.T_FP32_M
        return f

    def _keys(self) -> dict[int, int]:
        keys, k = {}, 0
        for g in self.param_groups:
            for p in g["params"]:
                keys[id(p)] = k
                k += 1
        return keys

    def _init_param_state(self, p: torch.Tensor, flags: int, mode: int) -> dict:
        st = self.state[p]
        st["step"] = 0
        st["v_mode"] = mode
        st["packed"] = torch.empty(A.state_bytes(p.numel(), flags), dtype=torch.uint8,
                                   device=p.device)
        if p.dtype == torch.bfloat16:
            st["master"] = p.detach().float().contiguous()
        return st

    @torch.no_grad()
    def step(self, closure=None):
        """One optimizer step.  Groups that share their hyperparameters, step count and v
        encoder (e.g. weights, norms and the LM head of one model) go to the library in one
        call, i.e. one kernel launch; each tensor keeps its own flags and RNG key."""
        loss = None
        if closure is not None:
            with torch.enable_grad():
                loss = closure()
        keys = self._keys()
        stream = torch.cuda.current_stream()
        batches: dict[tuple, list] = {}
        for group in self.param_groups:
            mode = mode_id(group["mode"])
            flags = self._flags(group)
            ps = [p for p in group["params"] if p.grad is not None]
            if not ps:
                continue
            fresh = [p for p in ps if len(self.state[p]) == 0]
            for p in fresh:
                self._init_param_state(p, flags, mode)
            if fresh:
                A.init_state(self._array([(p, flags) for p in fresh], keys), mode, stream=stream)
            t = self.state[ps[0]]["step"] + 1
            prev = self.state[ps[0]]["v_mode"]
            for p in ps:
                st = self.state[p]
                if st["step"] + 1 != t or st["v_mode"] != prev:
                    raise RuntimeError("parameters of one group must share their step count and "
                                       "v encoder (add new parameters as a new group)")
            b1, b2 = group["betas"]
            hkey = (t, float(group["lr"]), float(b1), float(b2), float(group["eps"]),
                    float(group["weight_decay"]), mode, prev)
            batches.setdefault(hkey, []).extend((p, flags) for p in ps)
        for (t, lr, b1, b2, eps, wd, mode, prev), items in batches.items():
            hp = A.hparams(step=t, lr=lr, beta1=b1, beta2=b2, eps=eps, weight_decay=wd, mode=mode,
                           prev_mode=prev, sr_head=sr_head_at(t, self.total_steps), seed=self.seed)
            A.step(self._cached_array(items, keys), hp, stream)
            for p, _ in items:
                st = self.state[p]
                st["step"] = t
                st["v_mode"] = mode
        return loss

    def _cached_array(self, items, keys: dict):
        """The tensor array of a batch, rebuilt only when a pointer, flag or key changed (grads
        are usually reallocated at the same addresses every step)."""
        sig = []
        for p, flags in items:
            st = self.state[p]
            m = st.get("master")
            sig.append((p.data_ptr(), p.grad.data_ptr(), p.grad.dtype, p.numel(),
                        st["packed"].data_ptr(), 0 if m is None else m.data_ptr(), flags,
                        keys[id(p)]))
        sig = tuple(sig)
        arr = self._arrays.get(sig)
        if arr is None:
            arr = self._array(items, keys)
            if len(self._arrays) >= 8:
                self._arrays.pop(next(iter(self._arrays)))
            self._arrays[sig] = arr
        return arr

    def _array(self, items, keys: dict):
        """adamw4_tensor array for (param, flags) pairs (the tensors it points into are held by
        the parameters, their gradients and the optimizer state)."""
        specs = []
        for p, flags in items:
            g = p.grad
            if g.numel() != p.numel() or not g.is_contiguous():
                raise ValueError("gradients must be contiguous with the parameter's numel")
            if g.dtype not in (torch.float32, torch.bfloat16):
                raise ValueError("gradients must be float32 or bfloat16")
            st = self.state[p]
            master = st.get("master")
            w, copy = (master, p) if master is not None else (p, None)
            gd = A.GRAD_BF16 if g.dtype == torch.bfloat16 else A.GRAD_F32
            packed = st["packed"]
            specs.append((w.data_ptr(), g.data_ptr(), p.numel(), flags, gd, packed.data_ptr(),
                          packed.numel(), copy.data_ptr() if copy is not None else None, 0,
                          keys[id(p)], 0))
        return A.tensor_array(specs)

    def decoded_moments(self, p: torch.Tensor):
        """FP32 (m, v) of one parameter's state (checkpoint inspection and tests)."""
        st = self.state[p]
        group = next(g for g in self.param_groups if any(q is p for q in g["params"]))
        flags = self._flags(group)
        packed = st["packed"]
        m = torch.empty(p.numel(), dtype=torch.float32, device=p.device)
        v = torch.empty_like(m)
        t = A.Tensor(0, 0, p.numel(), flags, 0, packed.data_ptr(), packed.numel())
        A.decode_state(t, st["v_mode"], m.data_ptr(), v.data_ptr())
        return m.view_as(p), v.view_as(p)

    def state_dict(self):
        sd = super().state_dict()
        sd["adamw4"] = {"seed": self.seed, "total_steps": self.total_steps}
        return sd

    def load_state_dict(self, state_dict):
        """Load a state_dict of this optimizer.  The packed states and FP32 masters keep their
        dtypes (torch's default load would cast them to the parameters' dtype)."""
        sd = dict(state_dict)
        extra = sd.pop("adamw4", None)
        raw, plain = {}, {}
        for k, v in sd["state"].items():
            v = dict(v)
            raw[k] = {name: v.pop(name) for name in ("packed", "master") if name in v}
            plain[k] = v
        sd["state"] = plain
        super().load_state_dict(sd)
        params = [p for g in self.param_groups for p in g["params"]]
        groups = {id(p): g for g in self.param_groups for p in g["params"]}
        for k, tensors in raw.items():
            p = params[k]
            st = self.state[p]
            for name, t in tensors.items():
                dt = torch.uint8 if name == "packed" else torch.float32
                st[name] = t.to(device=p.device, dtype=dt).contiguous().clone()
            need = A.state_bytes(p.numel(), self._flags(groups[id(p)]))
            if st["packed"].numel() != need:
                raise ValueError(f"packed state of parameter {k} has {st['packed'].numel()} "
                                 f"bytes, expected {need}")
            if p.dtype == torch.bfloat16 and "master" not in st:
                raise ValueError(f"BF16 parameter {k} has no FP32 master in the state_dict")
        if extra:
            self.seed = int(extra["seed"])
            self.total_steps = extra["total_steps"]
        self._arrays.clear()
