"""CPU oracle of the fused 4-bit AdamW step (ZIP-SR / ZE-EDEN): a thin numpy/ctypes binding
over ``adamw4_oracle.c``.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the benchmark's
CPU-baseline leg import this module.  The HIP library and its Python binding never import it,
and the two implementations share no code.

Every function cites the page passage it follows; see the C file's header for the tags
([daiwk-CE] = daiwk.github.io "ZIP-SR / ZE-EDEN: 4-bit AdamW state quantization", section
"Core equation"; [lav-ST] = learnaivisually.com "ZIP-SR 4-bit AdamW", storage paragraph; ...).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "adamw4_oracle.c")
LIB = os.path.join(HERE, "liboracle_adamw4.so")
# The pin suite's mutation test points this at deliberately broken copies of the oracle.
_LIB_OVERRIDE = os.environ.get("ADAMW4_ORACLE_LIB")

BLOCK = 128          # values per FP32 block scale ([lav-ST])
MIN_QUANT = 4096     # tensors below this stay FP32 ([daiwk-LR])
# v encoders: the two methods, the controlled study's three other rules, and the baseline
# (round to nearest on the zero-free codebook, absmax scale, no rescale)
ZIP_SR, ZE_EDEN, V_RTN, V_SSR, V_PRTN, V_ZE_RTN = 0, 1, 2, 3, 4, 5
MODES = (ZIP_SR, ZE_EDEN, V_RTN, V_SSR, V_PRTN, V_ZE_RTN)
CB_NF4, CB_V0, CB_V1 = 0, 1, 2
(RULE_M_RTN, RULE_M_SR, RULE_V_ZIP, RULE_V_EDEN, RULE_V_RTN, RULE_V_SSR, RULE_V_PRTN,
 RULE_V_ZE_RTN) = 0, 1, 2, 3, 4, 5, 6, 7


def v_codebook_of(mode: int) -> int:
    """Codebook a v encoded under `mode` decodes with: V1 for ZE-EDEN and the baseline."""
    return CB_V1 if mode in (ZE_EDEN, V_ZE_RTN) else CB_V0


def build(force: bool = False) -> str:
    """Compile the oracle with gcc: IEEE FP32, no contraction, no fast-math, OpenMP over blocks."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB)
    return LIB


class _HP(ctypes.Structure):
    _fields_ = [("step", ctypes.c_int64), ("lr", ctypes.c_float), ("beta1", ctypes.c_float),
                ("beta2", ctypes.c_float), ("eps", ctypes.c_float),
                ("weight_decay", ctypes.c_float), ("mode", ctypes.c_int32),
                ("prev_mode", ctypes.c_int32), ("sr_head", ctypes.c_int32),
                ("seed", ctypes.c_uint64)]


@dataclass
class HParams:
    step: int
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.1
    mode: int = ZIP_SR
    prev_mode: int = -1
    sr_head: int = 0
    seed: int = 0

    def c(self) -> _HP:
        return _HP(self.step, self.lr, self.beta1, self.beta2, self.eps, self.weight_decay,
                   self.mode, self.prev_mode, self.sr_head, self.seed)


_lib = None


def lib():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            L = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            build()
            L = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        L.orc_codebook.argtypes = [ctypes.c_int, P]
        L.orc_philox4x32_10.argtypes = [P, P, P]
        L.orc_uniform.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_uint32, ctypes.c_int,
                                  ctypes.c_int64]
        L.orc_uniform.restype = ctypes.c_float
        L.orc_step_scalars.argtypes = [P, P]
        L.orc_zip_p.argtypes = [ctypes.c_float] * 5
        L.orc_zip_p.restype = ctypes.c_float
        L.orc_zip_p64.argtypes = [ctypes.c_double] * 5
        L.orc_zip_p64.restype = ctypes.c_double
        L.orc_step_fp32.argtypes = [P, P, ctypes.c_int, ctypes.c_int64, P, P, P]
        L.orc_step_quant.argtypes = [P, P, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                     ctypes.c_int64, P, P, P, P, ctypes.c_int, ctypes.c_uint32,
                                     P, P]
        L.orc_step_quant.restype = ctypes.c_int
        L.orc_step_fp32m.argtypes = [P, P, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                     ctypes.c_int64, P, P, P, ctypes.c_uint32, P, P]
        L.orc_step_fp32m.restype = ctypes.c_int
        L.orc_encode_init.argtypes = [P, P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                      ctypes.c_int, P, P, P, P]
        L.orc_encode_init.restype = ctypes.c_int
        L.orc_decode.argtypes = [P, P, P, P, ctypes.c_int64, ctypes.c_int, P, P]
        L.orc_threads.restype = ctypes.c_int
        L.orc_set_threads.argtypes = [ctypes.c_int]
        L.orc_encode_block.argtypes = [P, ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                       ctypes.c_float, ctypes.c_uint64, ctypes.c_int64,
                                       ctypes.c_uint32, ctypes.c_int64, P, P, P]
        L.orc_bf16_rne.argtypes = [P, ctypes.c_int64, P]
        _lib = L
    return _lib


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be contiguous"
    return a.ctypes.data


# ---------------------------------------------------------------------------------------------
# constants and primitives
# ---------------------------------------------------------------------------------------------

def codebook(which: int) -> np.ndarray:
    """16 FP32 words of NF4 (m), V0 = k/15 (ZIP-SR v) or V1 = (k+1)/16 (ZE-EDEN v)."""
    out = np.zeros(16, np.float32)
    lib().orc_codebook(which, _p(out))
    return out


def bf16_rne(x: np.ndarray) -> np.ndarray:
    """BF16 bit patterns (uint16) of FP32 values, round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.size, np.uint16)
    lib().orc_bf16_rne(_p(x), x.size, _p(out))
    return out.reshape(x.shape)


def philox4x32_10(ctr, key) -> np.ndarray:
    """Philox4x32-10 (Salmon et al., SC'11) on one counter block."""
    c = np.asarray(ctr, np.uint32).copy()
    k = np.asarray(key, np.uint32).copy()
    out = np.zeros(4, np.uint32)
    lib().orc_philox4x32_10(_p(c), _p(k), _p(out))
    return out


def uniform(seed: int, t: int, pos: int, stream: int, i: int) -> float:
    return float(lib().orc_uniform(seed, t, pos, stream, i))


def step_scalars(hp: HParams) -> dict:
    """step_size = lr/(1-b1^t), rs2 = 1/sqrt(1-b2^t), decay = 1 - lr*wd, 1-b1, 1-b2 (FP32)."""
    out = np.zeros(5, np.float32)
    h = hp.c()
    lib().orc_step_scalars(ctypes.byref(h), _p(out))
    return dict(zip(["step_size", "rs2", "decay", "omb1", "omb2"], out.tolist()))


def zip_p(y: float, alpha: float, beta: float, c: float, eps: float) -> float:
    """ZIP-SR probability of the lower level, FP32, block-normalised form ([daiwk-CE])."""
    return float(lib().orc_zip_p(y, alpha, beta, c, eps))


def zip_p64(v: float, a: float, b: float, bc2: float, eps: float) -> float:
    """The printed ratio [h(v)-h(b)]/[h(a)-h(b)], h(x) = 1/(sqrt(x/bc2)+eps), in binary64."""
    return float(lib().orc_zip_p64(v, a, b, bc2, eps))


def encode_block(x: np.ndarray, rule: int, *, nvalid: int | None = None, rs2: float = 1.0,
                 eps: float = 1e-8, seed: int = 0, t: int = 1, pos: int = 0, i0: int = 0):
    """Quantize one 128-slot block (zero-padded).  Returns (codes[128], scale, dbg[128,4])
    with dbg columns (u_v, p_v, u_m, p_m); p = -1 where no random choice was made."""
    xb = np.zeros(BLOCK, np.float32)
    x = np.asarray(x, np.float32)
    xb[: x.size] = x
    nv = x.size if nvalid is None else nvalid
    codes = np.zeros(BLOCK, np.uint8)
    scale = np.zeros(1, np.float32)
    dbg = np.full((BLOCK, 4), -1.0, np.float32)
    lib().orc_encode_block(_p(xb), nv, rule, rs2, eps, seed, t, pos, i0, _p(codes), _p(scale),
                           _p(dbg))
    return codes, float(scale[0]), dbg


# ---------------------------------------------------------------------------------------------
# per-tensor state and step
# ---------------------------------------------------------------------------------------------

def is_quantized(numel: int, norm: bool) -> bool:
    """Quantize iff numel >= 4096 and the tensor is not a normalization layer ([lav-ST], [daiwk-LR])."""
    return numel >= MIN_QUANT and not norm


@dataclass
class State:
    """Oracle-side optimizer state of one tensor: packed codes + block scales, or FP32 m/v.
    A quantized state with mcodes None keeps m in FP32 (m) and only v packed (fp32_m)."""
    quantized: bool
    mcodes: np.ndarray | None = None
    vcodes: np.ndarray | None = None
    mscale: np.ndarray | None = None
    vscale: np.ndarray | None = None
    m: np.ndarray | None = None
    v: np.ndarray | None = None

    @property
    def fp32_m(self) -> bool:
        return self.quantized and self.mcodes is None

    def copy(self) -> "State":
        c = lambda a: None if a is None else a.copy()
        return State(self.quantized, c(self.mcodes), c(self.vcodes), c(self.mscale),
                     c(self.vscale), c(self.m), c(self.v))


def init_state(n: int, norm: bool, mode: int, m0=None, v0=None, fp32_m: bool = False) -> State:
    """Zero state, or deterministic RTN encoding of given FP32 moments (ZE-EDEN adds its rescale).
    fp32_m: a quantized tensor keeps m in FP32 (only v is encoded)."""
    if not is_quantized(n, norm):
        m = np.zeros(n, np.float32) if m0 is None else np.asarray(m0, np.float32).copy()
        v = np.zeros(n, np.float32) if v0 is None else np.asarray(v0, np.float32).copy()
        return State(False, m=m, v=v)
    nb = (n + BLOCK - 1) // BLOCK
    if fp32_m:
        full = init_state(n, norm, mode, None, v0)
        m = np.zeros(n, np.float32) if m0 is None else np.asarray(m0, np.float32).copy()
        return State(True, None, full.vcodes, None, full.vscale, m=m)
    st = State(True, np.zeros((n + 1) // 2, np.uint8), np.zeros((n + 1) // 2, np.uint8),
               np.zeros(nb, np.float32), np.zeros(nb, np.float32))
    if m0 is not None or v0 is not None:
        m0a = None if m0 is None else np.ascontiguousarray(m0, np.float32)
        v0a = None if v0 is None else np.ascontiguousarray(v0, np.float32)
        rc = lib().orc_encode_init(_p(m0a), _p(v0a), n, 0, n, mode, _p(st.mcodes),
                                   _p(st.vcodes), _p(st.mscale), _p(st.vscale))
        assert rc == 0
    else:
        st.mcodes[:] = 0x77  # NF4 code 7 is exact zero; scale 0 decodes to 0 either way
    return st


def decode(st: State, n: int, mode: int):
    """FP32 m, v of a state: m = NF4[code]*s_m, v = V[code]*s_v ([daiwk-PM] decode step)."""
    if not st.quantized:
        return st.m.copy(), st.v.copy()
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    if st.fp32_m:
        dummy_c = np.zeros_like(st.vcodes)
        dummy_s = np.zeros_like(st.vscale)
        lib().orc_decode(_p(dummy_c), _p(st.vcodes), _p(dummy_s), _p(st.vscale), n, mode,
                         _p(m), _p(v))
        return st.m.copy(), v
    lib().orc_decode(_p(st.mcodes), _p(st.vcodes), _p(st.mscale), _p(st.vscale), n, mode,
                     _p(m), _p(v))
    return m, v


def grad_arg(g: np.ndarray):
    """(array, is_bf16): FP32 grads as float32, BF16 grads as their uint16 bit patterns."""
    if g.dtype == np.float32:
        return np.ascontiguousarray(g), 0
    if g.dtype == np.uint16:
        return np.ascontiguousarray(g), 1
    raise TypeError("grads must be float32 or bf16 bit patterns (uint16)")


def step_tensor(w: np.ndarray, g: np.ndarray, st: State, hp: HParams, *, pos: int,
                head: bool = False, e0: int = 0, n: int | None = None, dbg: bool = False):
    """One oracle step of one tensor, in place on w and st.  For a quantized tensor the arrays
    may cover only elements [e0, e0 + w.size) of an n-element tensor (e0 a multiple of 128),
    with codes/scales sliced to match.  Returns the (cnt, 4) debug array when dbg is set."""
    ga, bf16 = grad_arg(g)
    cnt = w.size
    if not st.quantized:
        lib().orc_step_fp32(_p(w), _p(ga), bf16, cnt, _p(st.m), _p(st.v), ctypes.byref(hp.c()))
        return None
    n = cnt if n is None else n
    d = np.full((cnt, 4), -1.0, np.float32) if dbg else None
    h = hp.c()
    if st.fp32_m:
        rc = lib().orc_step_fp32m(_p(w), _p(ga), bf16, n, e0, cnt, _p(st.m), _p(st.vcodes),
                                  _p(st.vscale), pos, ctypes.byref(h), _p(d))
        if rc != 0:
            raise ValueError("bad element range or mode for the oracle step")
        return d
    rc = lib().orc_step_quant(_p(w), _p(ga), bf16, n, e0, cnt, _p(st.mcodes), _p(st.vcodes),
                              _p(st.mscale), _p(st.vscale), int(head), pos, ctypes.byref(h),
                              _p(d))
    if rc != 0:
        raise ValueError("bad element range for the oracle step")
    return d


def step_list(ws, gs, states, flags_head, hp: HParams, dbg: bool = False):
    """Multi-tensor step: tensor k of the list uses RNG position k ([daiwk-PM]: per-tensor loop)."""
    out = []
    for k, (w, g, st, head) in enumerate(zip(ws, gs, states, flags_head)):
        out.append(step_tensor(w, g, st, hp, pos=k, head=head, dbg=dbg))
    return out

