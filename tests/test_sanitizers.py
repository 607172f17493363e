"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only, no GPU):

- the chunk plan (bit_adamw_step_amd/csrc/chunk_plan.h) driven over the workload lists and
  random lists, built with g++ -fsanitize=address,undefined;
- the CPU oracle (oracle/adamw4_oracle.c) built the same way with gcc and put through its pin
  suite;
- the library's host runtime (argument checks, state layout, per-step scalars) built with the
  sanitizers on its host side only, running the argument-validation cases with no device.

Any report aborts the process (-fno-sanitize-recover=all, halt_on_error), so a finding fails
the test."""
import glob
import os
import random
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "bit_adamw_step_amd", "csrc")
sys.path.insert(0, ROOT)
sys.path.insert(0, HERE)

SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _gcc_asan_runtime():
    gcc = shutil.which("gcc")
    if gcc is None:
        return None
    p = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_chunk_plan_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    from test_chunk_plan import DRIVER, units_of, check
    src = tmp_path / "driver.cpp"
    src.write_text(DRIVER)
    exe = tmp_path / "driver_san"
    subprocess.run([gxx, "-std=c++17", *SAN, "-I", CSRC, "-o", str(exe), str(src)], check=True)
    import json
    import workloads as W
    env = dict(os.environ, **SAN_ENV)

    def run(G, units):
        inp = f"{G} {len(units)} " + " ".join(str(u) for u in units)
        r = subprocess.run([str(exe)], input=inp, capture_output=True, text=True, env=env)
        assert r.returncode == 0, r.stderr[-3000:]
        return json.loads(r.stdout)

    for wname in ["llama2b7", "gpt834m", "gpt130m", "stress", "flat1m"]:
        for G in (1280, 768):
            check(run(G, units_of(W.WORKLOADS[wname].specs)), G)
    rng = random.Random(7)
    for _ in range(60):
        G = rng.choice([2, 7, 64, 320, 1280])
        units = [rng.choice([rng.randint(1, 40), rng.randint(1, 3000), rng.randint(1000, 80000)])
                 for _ in range(rng.randint(1, 40))]
        check(run(G, units), G)


def test_oracle_pins_under_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    asan = _gcc_asan_runtime()
    if gcc is None or asan is None:
        pytest.skip("gcc with its AddressSanitizer runtime not available")
    lib = tmp_path / "liboracle_san.so"
    subprocess.run([gcc, "-std=c11", *SAN, "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
                    "-shared", "-o", str(lib), os.path.join(ROOT, "oracle", "adamw4_oracle.c"), "-lm"],
                   check=True)
    pre = os.environ.get("LD_PRELOAD", "")
    env = dict(os.environ, ADAMW4_ORACLE_LIB=str(lib), **SAN_ENV,
               LD_PRELOAD=(asan + (" " + pre if pre else "")))
    # the rocRAND known-answer test builds and runs a hipcc helper, which is not sanitized code
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_oracle_pins.py"), "-k", "not rocrand"],
                       env=env, capture_output=True, text=True, cwd=ROOT)
    assert r.returncode == 0, (r.stdout[-3000:] + r.stderr[-3000:])
    assert " passed" in r.stdout


def test_host_runtime_under_sanitizers(tmp_path):
    """The library's host side (adamw4_api.cpp and the host half of the kernels' file) with
    ASan/UBSan, device code unchanged; the argument-validation cases of test_abi run against it
    in a process that sees no GPU."""
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not os.path.exists(hipcc) or not rt:
        pytest.skip("hipcc or clang's AddressSanitizer runtime not available")
    from bit_adamw_step_amd import build as B
    from test_abi import VALIDATION_SCRIPT
    lib = tmp_path / "libadamw4_san.so"
    host_san = []
    for f in ("-fsanitize=address,undefined", "-fno-sanitize-recover=all"):
        host_san += ["-Xarch_host", f]
    cmd = [hipcc] + B.flags() + host_san + ["-Xarch_host", "-fno-omit-frame-pointer", "-shared",
                                            "-o", str(lib)] + B.SOURCES
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    script = ("import bit_adamw_step_amd as _A\n_A.LIB_PATH = %r\n" % str(lib)) + \
        VALIDATION_SCRIPT % {"root": ROOT}
    pre = os.environ.get("LD_PRELOAD", "")
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1",
               CUDA_VISIBLE_DEVICES="-1", LD_PRELOAD=(rt[-1] + (" " + pre if pre else "")), **SAN_ENV)
    # the script imports the package first, so the LIB_PATH override must come after sys.path
    script = script.replace("import ctypes, sys\nsys.path.insert(0, %r)\n" % ROOT, "")
    script = ("import ctypes, sys\nsys.path.insert(0, %r)\n" % ROOT) + script
    r = subprocess.run([sys.executable, "-c", script], env=env, capture_output=True, text=True)
    assert r.returncode == 0, (r.stdout[-3000:] + r.stderr[-3000:])
    assert "RESULTS" in r.stdout
