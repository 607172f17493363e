"""C-ABI checks that need no GPU: the library builds and loads, exports every function that
include/adamw4.h declares, sizes states as documented, carries the oracle's codebook words, and
rejects bad arguments on the host before any device work."""
import ctypes
import os
import re
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "adamw4.h")


@pytest.fixture(scope="module")
def A():
    import bit_adamw_step_amd as A
    if not os.path.exists(A.LIB_PATH):
        from bit_adamw_step_amd import build
        build.build()
    A.lib()
    return A


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(adamw4_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_function(A):
    names = declared_functions()
    assert {"adamw4_step", "adamw4_init_state", "adamw4_state_bytes", "adamw4_decode_state",
            "adamw4_status_string", "adamw4_state_layout", "adamw4_codebook"} <= set(names)
    L = ctypes.CDLL(A.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", A.LIB_PATH], capture_output=True,
                         text=True).stdout
    for n in names:
        assert re.search(r"\bT " + n + r"\b", out), n


def test_struct_layouts_match_header(A, tmp_path):
    """The binding's ctypes structures have the header's sizes and field offsets (checked with
    a host C program compiled against include/adamw4.h)."""
    import ctypes
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    fields = {"adamw4_tensor": [f for f, _ in A.Tensor._fields_],
              "adamw4_hparams": [f for f, _ in A.HParams._fields_]}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "adamw4.h"', "int main(void) {"]
    for st, fs in fields.items():
        lines.append(f'printf("{st} %zu\\n", sizeof({st}));')
        for f in fs:
            lines.append(f'printf("{st}.{f} %zu\\n", offsetof({st}, {f}));')
    lines += ["return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(root, "include"), "-o", str(exe), str(src)],
                   check=True)
    got = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True, text=True,
                                                        check=True).stdout.splitlines())
    for st, cls in (("adamw4_tensor", A.Tensor), ("adamw4_hparams", A.HParams)):
        assert int(got[st]) == ctypes.sizeof(cls), st
        for f in fields[st]:
            assert int(got[f"{st}.{f}"]) == getattr(cls, f).offset, (st, f)


def test_state_bytes_fp32_m(A):
    """FP32-m tensors: FP32 m, then v codes, then v scales, 16-byte aligned; no m scales."""
    for n in (4096, 4097, 12345, 1 << 20):
        off = A.state_layout(n, A.T_FP32_M)
        m32 = (4 * n + 15) // 16 * 16
        codes = ((n + 1) // 2 + 15) // 16 * 16
        scales = ((n + 127) // 128 * 4 + 15) // 16 * 16
        assert off[0] == 0 and off[1] == m32 and off[2] >= 2**63 and off[3] == m32 + codes
        assert A.state_bytes(n, A.T_FP32_M) == m32 + codes + scales
    # tensors that keep both moments in FP32 are unaffected by the flag
    assert A.state_bytes(100, A.T_FP32_M) == A.state_bytes(100, 0)
    assert A.state_bytes(5000, A.T_FP32_M | A.T_NORM) == A.state_bytes(5000, A.T_NORM)


def test_state_bytes_shard(A):
    """A shard of a quantized tensor is quantized whatever its own length (its blocks are the
    whole tensor's); SHARD has no other effect on the layout."""
    al = lambda x: (x + 15) // 16 * 16
    for n in (128, 300, 4095, 4096, 10000):
        assert A.state_bytes(n, A.T_SHARD) == 2 * al((n + 1) // 2) + 2 * al(4 * ((n + 127) // 128))
        assert A.is_quantized(n, A.T_SHARD)
    assert A.state_bytes(5000, A.T_SHARD) == A.state_bytes(5000, 0)
    assert A.state_bytes(300, A.T_SHARD | A.T_FP32_M) == al(4 * 300) + al(150) + al(12)
    assert A.state_bytes(300, A.T_SHARD | A.T_KEYED) == A.state_bytes(300, A.T_SHARD)


def test_state_bytes_formula(A):
    """Quantized: two code sections of ceil(n/2) bytes and two scale sections of ceil(n/128)
    FP32, 16-byte aligned; FP32 tensors: 2 x 4n bytes."""
    al = lambda x: (x + 15) // 16 * 16
    for n in [4096, 4097, 5000, 1 << 20, 2701 * 4096 + 3]:
        assert A.state_bytes(n, 0) == 2 * al((n + 1) // 2) + 2 * al(4 * ((n + 127) // 128))
        assert A.state_bytes(n, A.T_NORM) == 2 * al(4 * n)
    for n in [1, 64, 4095]:
        assert A.state_bytes(n, 0) == 2 * al(4 * n)
    assert A.state_bytes(0, 0) == 0 and A.state_bytes(-5, 0) == 0
    assert A.state_bytes((1 << 38) + 1, 0) == 0 and A.state_bytes(1 << 38, A.T_NORM) > 0


def test_state_bytes_pages_accounting(A):
    """Persistent moment bytes of the A100 table (daiwk.github.io "Local reproduction"):
    33 x 4096 quantized + 7 x 256 fallback elements -> 157,952 bytes (no padding at these sizes)."""
    total = sum(A.state_bytes(4096, 0) for _ in range(33)) + sum(A.state_bytes(256, 0) for _ in range(7))
    assert total == 157952


def test_codebooks_equal_oracle(A, orc):
    for which in range(3):
        lib_words = np.array(A.codebook(which), np.float32)
        assert np.array_equal(lib_words.view(np.uint32), orc.codebook(which).view(np.uint32)), which


VALIDATION_SCRIPT = r"""
import ctypes, sys
sys.path.insert(0, %(root)r)
import bit_adamw_step_amd as A
L = A.lib()
EINVAL, EALIGN, ESIZE, EHIP = -1, -2, -3, -4
FAKE = 0x7F0000000000          # never dereferenced: every case below fails validation first
def T(**kw):
    d = dict(param=FAKE, grad=FAKE + 4096, numel=8192, flags=0, grad_dtype=0, state=FAKE + 65536,
             state_size=A.state_bytes(8192, 0), param_bf16=None, offset=0, key=0, reserved=0)
    d.update(kw)
    return A.Tensor(d["param"], d["grad"], d["numel"], d["flags"], d["grad_dtype"], d["state"],
                    d["state_size"], d["param_bf16"], d["offset"], d["key"], d["reserved"])
def step(ts, hp, n=None):
    arr = (A.Tensor * len(ts))(*ts)
    return L.adamw4_step(ctypes.addressof(arr) if ts else None, len(ts) if n is None else n, ctypes.byref(hp), None)
def step_na(ts, hp):
    arr = (A.Tensor * len(ts))(*ts)
    return L.adamw4_step_noalloc(ctypes.addressof(arr), len(ts), ctypes.byref(hp), None)
good = A.hparams(step=1)
cases = [
  ("null hp", L.adamw4_step(None, 0, None, None), EINVAL),
  ("negative n", step([T()], good, n=-1), EINVAL),
  ("null list", L.adamw4_step(None, 3, ctypes.byref(good), None), EINVAL),
  ("step 0", step([T()], A.hparams(step=0)), EINVAL),
  ("beta1 1", step([T()], A.hparams(step=1, beta1=1.0)), EINVAL),
  ("beta2 -0.1", step([T()], A.hparams(step=1, beta2=-0.1)), EINVAL),
  ("eps 0", step([T()], A.hparams(step=1, eps=0.0)), EINVAL),
  ("eps subnormal", step([T()], A.hparams(step=1, eps=1e-39)), EINVAL),
  ("eps above 2^64", step([T()], A.hparams(step=1, eps=2.0**64 * 1.0000001)), EINVAL),
  ("lr nan", step([T()], A.hparams(step=1, lr=float("nan"))), EINVAL),
  ("wd inf", step([T()], A.hparams(step=1, weight_decay=float("inf"))), EINVAL),
  ("mode 6", step([T()], A.hparams(step=1, mode=6)), EINVAL),
  ("mode -1", step([T()], A.hparams(step=1, mode=-1)), EINVAL),
  ("prev_mode 7", step([T()], A.hparams(step=1, prev_mode=7)), EINVAL),
  ("sr_head 2", step([T()], A.hparams(step=1, sr_head=2)), EINVAL),
  ("step > 2^32-1", step([T()], A.hparams(step=1 << 32)), EINVAL),
  ("numel 0", step([T(numel=0)], good), EINVAL),
  ("numel too big", step([T(numel=(1 << 38) + 1)], good), ESIZE),
  ("bad flag", step([T(flags=32)], good), EINVAL),
  ("shard of a norm tensor", step([T(flags=A.T_SHARD | A.T_NORM)], good), EINVAL),
  ("offset not a block multiple", step([T(offset=64)], good), EINVAL),
  ("negative offset", step([T(offset=-128)], good), EINVAL),
  ("offset past the limit", step([T(offset=(1 << 38) - 4096)], good), EINVAL),
  ("reserved set", step([T(reserved=1)], good), EINVAL),
  ("misaligned bf16 copy", step([T(param_bf16=FAKE + 8192 + 2)], good), EALIGN),
  ("bad dtype", step([T(grad_dtype=2)], good), EINVAL),
  ("null param", step([T(param=0)], good), EINVAL),
  ("null grad", step([T(grad=0)], good), EINVAL),
  ("null state", step([T(state=0)], good), EINVAL),
  ("misaligned param", step([T(param=FAKE + 4)], good), EALIGN),
  ("misaligned grad", step([T(grad=FAKE + 2)], good), EALIGN),
  ("misaligned state", step([T(state=FAKE + 8)], good), EALIGN),
  ("state too small", step([T(state_size=A.state_bytes(8192, 0) - 1)], good), ESIZE),
  ("fallback state too small", step([T(numel=100, state_size=799)], good), ESIZE),
  ("second tensor bad", step([T(), T(numel=-1)], good), EINVAL),
  ("more tensors than a list holds", step([T()] * 65537, good), ESIZE),
  ("init bad mode", L.adamw4_init_state(None, 0, 7, None, None, None), EINVAL),
  ("decode null", L.adamw4_decode_state(None, 0, None, None, None), EINVAL),
  ("decode bad mode", L.adamw4_decode_state(ctypes.byref(T()), 6, None, None, None), EINVAL),
  ("layout null", L.adamw4_state_layout(100, 0, None), EINVAL),
  ("codebook 3", L.adamw4_codebook(3, None), EINVAL),
  ("empty list is a no-op", L.adamw4_step(None, 0, ctypes.byref(good), None), 0),
  ("noalloc: empty list is a no-op", L.adamw4_step_noalloc(None, 0, ctypes.byref(good), None), 0),
  ("noalloc: more tensors than its array holds", step_na([T()] * 4097, good), ESIZE),
  ("noalloc: bad hparams", step_na([T()], A.hparams(step=0)), EINVAL),
  ("noalloc: misaligned grad", step_na([T(grad=FAKE + 2)], good), EALIGN),
]
bad = [(n, got, exp) for n, got, exp in cases if got != exp]
print("RESULTS", len(cases), bad)
sys.exit(1 if bad else 0)
"""


def test_argument_validation_without_device(A):
    """Invalid arguments return the documented status before any device work.  Runs in a child
    process that sees no GPU, so even a broken check could not launch a kernel."""
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1",
               CUDA_VISIBLE_DEVICES="-1")
    r = subprocess.run([sys.executable, "-c", VALIDATION_SCRIPT % {"root": ROOT}], env=env,
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr


def test_status_strings(A):
    for s in [0, -1, -2, -3, -4, -5, -99]:
        assert isinstance(A.status_string(s), str) and A.status_string(s)


def test_missing_library_fails_loudly(tmp_path):
    """The binding has no CPU fallback: without the built library every call raises."""
    code = ("import sys; sys.path.insert(0, %r)\n"
            "import bit_adamw_step_amd as A\n"
            "A.LIB_PATH = %r\n"
            "try:\n    A.state_bytes(4096)\nexcept RuntimeError as e:\n    print('RAISED', e)\n"
            % (ROOT, str(tmp_path / "missing.so")))
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True).stdout
    assert "RAISED" in out
