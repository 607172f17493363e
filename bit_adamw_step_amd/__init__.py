"""Fused 4-bit AdamW optimizer step (ZIP-SR / ZE-EDEN) for MI355X (gfx950).

A thin ctypes binding over ``libadamw4.so`` whose C ABI is ``include/adamw4.h``; names and
arguments mirror that header.  This module only marshals arguments: every step of the
optimizer runs in the library's HIP kernels.  PyTorch supplies device memory and the stream.
There is no CPU fallback: if the library is missing or the device call fails, calls raise.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libadamw4.so")

ZIP_SR, ZE_EDEN, V_RTN, V_SSR, V_PRTN, V_ZE_RTN = 0, 1, 2, 3, 4, 5   # adamw4_mode
T_NORM, T_HEAD, T_FP32_M, T_SHARD, T_KEYED = 1, 2, 4, 8, 16
GRAD_F32, GRAD_BF16 = 0, 1
CB_NF4, CB_V0, CB_V1 = 0, 1, 2
BLOCK = 128
MIN_QUANT = 4096
STATUS = {0: "OK", -1: "EINVAL", -2: "EALIGN", -3: "ESIZE", -4: "EHIP", -5: "ENOMEM"}


class Adamw4Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({status_string(status)})")


class Tensor(ctypes.Structure):
    """adamw4_tensor"""
    _fields_ = [("param", ctypes.c_void_p), ("grad", ctypes.c_void_p), ("numel", ctypes.c_int64),
                ("flags", ctypes.c_uint32), ("grad_dtype", ctypes.c_uint32),
                ("state", ctypes.c_void_p), ("state_size", ctypes.c_size_t),
                ("param_bf16", ctypes.c_void_p), ("offset", ctypes.c_int64),
                ("key", ctypes.c_uint32), ("reserved", ctypes.c_uint32)]


class HParams(ctypes.Structure):
    """adamw4_hparams"""
    _fields_ = [("step", ctypes.c_int64), ("lr", ctypes.c_float), ("beta1", ctypes.c_float),
                ("beta2", ctypes.c_float), ("eps", ctypes.c_float),
                ("weight_decay", ctypes.c_float), ("mode", ctypes.c_int32),
                ("prev_mode", ctypes.c_int32), ("sr_head", ctypes.c_int32),
                ("seed", ctypes.c_uint64)]


def hparams(step: int, lr: float = 1e-3, beta1: float = 0.9, beta2: float = 0.999,
            eps: float = 1e-8, weight_decay: float = 0.1, mode: int = ZIP_SR,
            prev_mode: int = -1, sr_head: int = 0, seed: int = 0) -> HParams:
    return HParams(step, lr, beta1, beta2, eps, weight_decay, mode, prev_mode, sr_head, seed)


_lib = None


def lib():
    """Load libadamw4.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library {LIB_PATH} is not built; run "
                               "`python -m bit_adamw_step_amd.build` (or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        L.adamw4_state_bytes.argtypes = [ctypes.c_int64, ctypes.c_uint32]
        L.adamw4_state_bytes.restype = ctypes.c_size_t
        L.adamw4_state_layout.argtypes = [ctypes.c_int64, ctypes.c_uint32, P]
        L.adamw4_state_layout.restype = ctypes.c_int32
        L.adamw4_codebook.argtypes = [ctypes.c_int32, P]
        L.adamw4_codebook.restype = ctypes.c_int32
        L.adamw4_init_state.argtypes = [P, ctypes.c_int32, ctypes.c_int32, P, P, P]
        L.adamw4_init_state.restype = ctypes.c_int32
        L.adamw4_step.argtypes = [P, ctypes.c_int32, P, P]
        L.adamw4_step.restype = ctypes.c_int32
        L.adamw4_step_noalloc.argtypes = [P, ctypes.c_int32, P, P]
        L.adamw4_step_noalloc.restype = ctypes.c_int32
        L.adamw4_decode_state.argtypes = [P, ctypes.c_int32, P, P, P]
        L.adamw4_decode_state.restype = ctypes.c_int32
        L.adamw4_status_string.argtypes = [ctypes.c_int32]
        L.adamw4_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().adamw4_status_string(status).decode()


def _check(status: int, what: str) -> None:
    if status != 0:
        raise Adamw4Error(status, what)


def state_bytes(numel: int, flags: int = 0) -> int:
    return int(lib().adamw4_state_bytes(numel, flags))


def state_layout(numel: int, flags: int = 0) -> tuple[int, int, int, int]:
    off = (ctypes.c_size_t * 4)()
    _check(lib().adamw4_state_layout(numel, flags, ctypes.addressof(off)), "adamw4_state_layout")
    return tuple(int(x) for x in off)


def is_quantized(numel: int, flags: int = 0) -> bool:
    return (numel >= MIN_QUANT or bool(flags & T_SHARD)) and not (flags & T_NORM)


def codebook(which: int) -> list[float]:
    out = (ctypes.c_float * 16)()
    _check(lib().adamw4_codebook(which, ctypes.addressof(out)), "adamw4_codebook")
    return list(out)


def tensor_array(specs) -> ctypes.Array:
    """ctypes array of adamw4_tensor from (param, grad, numel, flags, grad_dtype, state, size
    [, param_bf16, offset, key]) tuples."""
    arr = (Tensor * len(specs))()
    for i, s in enumerate(specs):
        arr[i] = Tensor(*s)
    return arr


def _stream_handle(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if hasattr(stream, "cuda_stream"):
        return stream.cuda_stream
    return int(stream)


def step(ts: ctypes.Array, hp: HParams, stream=None) -> None:
    """adamw4_step over a prepared tensor array."""
    _check(lib().adamw4_step(ctypes.addressof(ts) if len(ts) else None, len(ts), ctypes.byref(hp),
                             _stream_handle(stream)), "adamw4_step")


def step_noalloc(ts: ctypes.Array, hp: HParams, stream=None) -> None:
    """adamw4_step_noalloc: the same step with its tables in the library's fixed device array
    (allocates nothing; calls on one GPU must not overlap)."""
    _check(lib().adamw4_step_noalloc(ctypes.addressof(ts) if len(ts) else None, len(ts),
                                     ctypes.byref(hp), _stream_handle(stream)),
           "adamw4_step_noalloc")


def init_state(ts: ctypes.Array, mode: int, m0=None, v0=None, stream=None) -> None:
    """adamw4_init_state; m0/v0: None or per-tensor sequences of device pointers (0 = zeros)."""
    n = len(ts)
    pm = (ctypes.c_void_p * n)(*[p or None for p in m0]) if m0 is not None else None
    pv = (ctypes.c_void_p * n)(*[p or None for p in v0]) if v0 is not None else None
    _check(lib().adamw4_init_state(ctypes.addressof(ts) if n else None, n, mode,
                                   ctypes.addressof(pm) if pm is not None else None,
                                   ctypes.addressof(pv) if pv is not None else None,
                                   _stream_handle(stream)), "adamw4_init_state")


def decode_state(t: Tensor, mode: int, m_out: int | None, v_out: int | None, stream=None) -> None:
    _check(lib().adamw4_decode_state(ctypes.byref(t), mode, m_out, v_out, _stream_handle(stream)),
           "adamw4_decode_state")


# ---------------------------------------------------------------------------------------------
# torch-side convenience: a parameter list with its persistent 4-bit state
# ---------------------------------------------------------------------------------------------

@dataclass
class ParamList:
    """Parameters, gradients and optimizer states of one step call (torch device tensors).

    params: FP32 CUDA tensors; grads: FP32 or BF16 CUDA tensors of the same numel;
    flags: per-tensor T_* flags.  States are allocated here with the library's sizes.
    Optional per-tensor lists (None entries allowed): bf16_copies, BF16 tensors that receive
    the updated weights; offsets, a shard's start within its whole tensor; keys, RNG keys
    (sets T_KEYED).
    """
    params: list
    grads: list
    flags: list
    states: list = field(default_factory=list)
    bf16_copies: list | None = None
    offsets: list | None = None
    keys: list | None = None
    _arr: ctypes.Array | None = None

    def __post_init__(self):
        import torch
        if not self.states:
            for p, f in zip(self.params, self.flags):
                nb = state_bytes(p.numel(), f)
                self.states.append(torch.empty(nb, dtype=torch.uint8, device=p.device))
        self.refresh()

    def refresh(self):
        """Rebuild the tensor array (after grads or states were replaced)."""
        import torch
        specs = []
        n = len(self.params)
        copies = self.bf16_copies or [None] * n
        offsets = self.offsets or [0] * n
        keys = self.keys or [None] * n
        for p, g, f, s, c, off, k in zip(self.params, self.grads, self.flags, self.states,
                                         copies, offsets, keys):
            if p.dtype != torch.float32 or not p.is_contiguous():
                raise TypeError("params must be contiguous float32")
            if g.numel() != p.numel() or not g.is_contiguous():
                raise TypeError("grad must be contiguous with the param's numel")
            if c is not None and (c.dtype != torch.bfloat16 or c.numel() != p.numel()
                                  or not c.is_contiguous()):
                raise TypeError("a BF16 copy must be contiguous bfloat16 with the param's numel")
            gd = {torch.float32: GRAD_F32, torch.bfloat16: GRAD_BF16}[g.dtype]
            f = f | (T_KEYED if k is not None else 0)
            specs.append((p.data_ptr(), g.data_ptr(), p.numel(), f, gd, s.data_ptr(), s.numel(),
                          c.data_ptr() if c is not None else None, off, k or 0, 0))
        self._arr = tensor_array(specs)

    @property
    def array(self) -> ctypes.Array:
        return self._arr

    def init(self, mode: int = ZIP_SR, m0=None, v0=None, stream=None):
        ptr = lambda xs: None if xs is None else [0 if x is None else x.data_ptr() for x in xs]
        init_state(self._arr, mode, ptr(m0), ptr(v0), stream)

    def step(self, hp: HParams, stream=None):
        step(self._arr, hp, stream)
