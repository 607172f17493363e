"""GPU parity: the HIP library (through its C ABI) against the CPU oracle, element by element.

Every case replays single steps: the GPU's inputs are snapshotted, one oracle step runs on the
snapshot, and the GPU's outputs are compared (codes and scales bit-exact except stochastic
flips with |u - p| < 1e-6; weights and FP32 moments within 1e-6 relative, reported when not
bit-exact).  Sizes span several 128-blocks, ragged tails, the 4096-element fallback boundary,
odd lengths, norm and LM-head tensors, FP32 and BF16 grads, both modes and mode changes.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

f32 = np.float32


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_adamw_step_amd as A
    A.lib()
    import oracle
    oracle.build()
    return A, oracle


def test_codebooks_match_oracle(env):
    A, orc = env
    for which in range(3):
        a = np.array(A.codebook(which), f32)
        assert np.array_equal(a.view(np.uint32), orc.codebook(which).view(np.uint32)), which


def test_state_layout_and_bytes(env):
    A, orc = env
    for n, f in [(4096, 0), (4097, 0), (4095, 0), (1, 0), (10000, A.T_NORM), (1 << 20, A.T_HEAD)]:
        off = A.state_layout(n, f)
        if A.is_quantized(n, f):
            c, nb = (n + 1) // 2, (n + 127) // 128
            assert off[0] == 0 and off[1] >= c and off[2] >= off[1] + c and off[3] >= off[2] + 4 * nb
            assert A.state_bytes(n, f) >= off[3] + 4 * nb
        else:
            assert off[1] >= 4 * n and A.state_bytes(n, f) >= off[1] + 4 * n
        assert all(o % 16 == 0 for o in off if o < 2**63)


@pytest.mark.parametrize("mode", [0, 1, 2, 3, 4, 5])
def test_init_matches_oracle(env, mode):
    """Deterministic encoding of given initial moments (and of zeros) matches the oracle: v to
    the nearest level of the zero-inclusive codebook, or of the zero-excluding one for ZE-EDEN
    (plus its rescale) and the baseline."""
    import torch
    from gpu_harness import GpuList, oracle_state, compare_state, say
    A, orc = env
    sizes = [4096, 4097, 128 * 37 + 5, 9000, 100, 6000, 128 * 33 + 9]
    flags = [0, 0, A.T_HEAD, 0, 0, A.T_NORM, A.T_FP32_M]
    gl = GpuList(sizes, flags, ["f32"] * len(sizes))
    rng = np.random.default_rng(mode)
    m0, v0 = [], []
    for i, n in enumerate(sizes):
        m = rng.normal(0, 1e-3, n).astype(f32)
        v = (10 ** rng.uniform(-20, -4, n)).astype(f32)
        if i == 3:
            m[:300] = 0
            v[:300] = 0       # all-zero blocks
        m0.append(m)
        v0.append(v)
    dm0 = [torch.from_numpy(x).cuda() for x in m0]
    dv0 = [torch.from_numpy(x).cuda() for x in v0]
    say(f"init mode={mode} sizes={sizes}")
    gl.pl.init(mode, dm0, [None if i == 1 else x for i, x in enumerate(dv0)])
    _, _, ss = gl.snapshot()
    rep = {}
    for i, n in enumerate(sizes):
        ref = orc.init_state(n, bool(flags[i] & A.T_NORM), mode, m0[i], None if i == 1 else v0[i],
                             fp32_m=bool(flags[i] & A.T_FP32_M))
        compare_state(f"init{i}", n, oracle_state(ss[i], n, flags[i]), ref, None, rep)


@pytest.mark.parametrize("mode", [0, 1, 3, 5])
def test_decode_matches_oracle(env, mode):
    import torch
    from gpu_harness import GpuList, to_np, say
    A, orc = env
    sizes = [4096 * 2 + 77, 300, 4096 + 129]
    fl = [0, 0, A.T_FP32_M]
    gl = GpuList(sizes, fl, ["f32"] * 3)
    rng = np.random.default_rng(3)
    m0 = [rng.normal(0, 1, n).astype(f32) for n in sizes]
    v0 = [rng.random(n).astype(f32) for n in sizes]
    gl.pl.init(mode, [torch.from_numpy(x).cuda() for x in m0], [torch.from_numpy(x).cuda() for x in v0])
    for i, n in enumerate(sizes):
        mo = torch.empty(n, device="cuda")
        vo = torch.empty(n, device="cuda")
        say(f"decode tensor {i} n={n} mode={mode}")
        A.decode_state(gl.pl.array[i], mode, mo.data_ptr(), vo.data_ptr())
        ref = orc.init_state(n, False, mode, m0[i], v0[i], fp32_m=bool(fl[i] & A.T_FP32_M))
        rm, rv = orc.decode(ref, n, mode)
        assert np.array_equal(to_np(mo), rm) and np.array_equal(to_np(vo), rv)


def _run_steps(env, sizes, flags, gdt, schedule, seed=0, report=None, zero_frac=0.0,
               hp_extra=None, grad_scale=1e-3):
    """Run the schedule [(t, mode, prev_mode, sr_head), ...] with single-step replay each step."""
    from gpu_harness import GpuList, say
    A, orc = env
    gl = GpuList(sizes, flags, gdt, seed=seed)
    gl.pl.init(schedule[0][1])
    report = {} if report is None else report
    for (t, mode, prev, srh) in schedule:
        gl.set_grads(t, seed=seed, zero_frac=zero_frac, scale=grad_scale)
        kw = dict(step=t, mode=mode, prev_mode=prev, sr_head=srh, seed=1234 + seed)
        kw.update(hp_extra or {})
        before = gl.snapshot()
        say(f"step t={t} mode={mode} prev={prev} sr_head={srh} sizes={sizes}")
        gl.pl.step(A.hparams(**kw))
        gl.replay_and_compare(before, kw, report, tag=f"t{t}:")
    return report


def test_flat1m_every_step(env):
    """1,048,576-value FP32 tensor (8192 blocks), FP32 grads, 10 ZIP-SR steps, all replayed."""
    rep = _run_steps(env, [1 << 20], [0], ["f32"], [(t, 0, -1, 0) for t in range(1, 11)])
    print(rep)


def test_mixed_list_modes(env):
    """Ragged list: fallback boundary 4095/4096/4097, odd lengths, partial blocks, norm and head
    tensors, BF16 and FP32 grads; ZIP-SR, then ZE-EDEN (decoding ZIP-SR's codebook), ZE-EDEN,
    back to ZIP-SR; head SR switched on mid-way."""
    A = env[0]
    sizes = [4095, 4096, 4097, 128 * 50 + 3, 64, 1, 7000, 128 * 200, 33333]
    flags = [0, 0, 0, 0, 0, 0, A.T_NORM, A.T_HEAD, 0]
    gdt = ["f32", "bf16", "f32", "bf16", "f32", "bf16", "bf16", "bf16", "f32"]
    sched = [(1, 0, -1, 0), (2, 0, -1, 1), (3, 1, 0, 1), (4, 1, -1, 0), (5, 0, 1, 1), (6, 0, -1, 1)]
    rep = _run_steps(env, sizes, flags, gdt, sched, seed=1)
    print({k: v for k, v in rep.items() if "flips" in k and v})


def test_tail_positions_in_the_lane_map(env):
    """A lane holds slots 4r..4r+3 (half A) and 64+4r..64+4r+3 (half B) of its block, so a
    partial last block can end inside a lane's half A, exactly at the half boundary, inside half
    B, or one slot short of full.  Tails at each of those positions (1, 3, 4, 5, 63, 64, 65, 67,
    68, 124, 127 values), each with 8 full blocks before it, through every v rule, the LM-head
    switch and FP32 m, with FP32 and BF16 grads; the init encoder and decode on the same list."""
    A, orc = env
    rems = [1, 3, 4, 5, 63, 64, 65, 67, 68, 124, 127]
    sizes = [128 * 40 + r for r in rems]
    flags = [0, A.T_HEAD, A.T_FP32_M, 0, A.T_HEAD, 0, A.T_FP32_M, 0, A.T_HEAD, 0, A.T_FP32_M]
    gdt = ["bf16" if i % 2 else "f32" for i in range(len(sizes))]
    sched = [(1, A.ZIP_SR, -1, 0), (2, A.ZE_EDEN, A.ZIP_SR, 1), (3, A.V_SSR, A.ZE_EDEN, 1),
             (4, A.V_RTN, A.V_SSR, 0), (5, A.V_PRTN, A.V_RTN, 1), (6, A.V_ZE_RTN, A.V_PRTN, 0),
             (7, A.ZIP_SR, A.V_ZE_RTN, 1)]
    rep = _run_steps(env, sizes, flags, gdt, sched, seed=21)
    assert all(v for k, v in rep.items() if k.endswith("w_bitexact"))
    # the deterministic init encoder from given moments, then decode, at the same tails
    import torch
    from gpu_harness import GpuList, oracle_state, compare_state, to_np, say
    rng = np.random.default_rng(22)
    for mode in (A.ZIP_SR, A.ZE_EDEN, A.V_ZE_RTN):
        gl = GpuList(sizes, flags, ["f32"] * len(sizes))
        m0 = [rng.normal(0, 1e-3, n).astype(f32) for n in sizes]
        v0 = [(10 ** rng.uniform(-12, -4, n)).astype(f32) for n in sizes]
        say(f"init+decode mode={mode} sizes={sizes}")
        gl.pl.init(mode, [torch.from_numpy(x).cuda() for x in m0],
                   [torch.from_numpy(x).cuda() for x in v0])
        _, _, ss = gl.snapshot()
        crep = {}
        for i, n in enumerate(sizes):
            ref = orc.init_state(n, False, mode, m0[i], v0[i], fp32_m=bool(flags[i] & A.T_FP32_M))
            compare_state(f"init{i}", n, oracle_state(ss[i], n, flags[i]), ref, None, crep)
            mo = torch.empty(n, device="cuda")
            vo = torch.empty(n, device="cuda")
            A.decode_state(gl.pl.array[i], mode, mo.data_ptr(), vo.data_ptr())
            rm, rv = orc.decode(ref, n, mode)
            assert np.array_equal(to_np(mo), rm) and np.array_equal(to_np(vo), rv), (mode, n)


def test_balanced_last_rounds(env):
    """Lists with more chunks than the launch has workgroups: the plan deals chunks round-robin
    and re-cuts the last partial round and the round before it into two pieces per workgroup
    (the whole list in the first case here, its second half in the second, across tensor
    boundaries, ragged tails and FP32-state tensors).  Every value of every tensor is compared
    with the oracle, so a unit stepped twice or not at all fails."""
    A = env[0]
    sizes = [65536] * 40 + [65536 + 77, 3000, 4096 * 3 + 5, 200000 + 33]
    flags = [0] * 40 + [A.T_HEAD, 0, A.T_FP32_M, 0]
    gdt = ["bf16"] * 20 + ["f32"] * 20 + ["bf16", "f32", "bf16", "f32"]
    _run_steps(env, sizes, flags, gdt, [(1, A.ZIP_SR, -1, 1), (2, A.ZE_EDEN, A.ZIP_SR, 0)],
               seed=31)
    sizes = [1 << 20] * 6 + [300000 + 17, 5000, 2000, 128 * 700 + 1]
    flags = [0, A.T_FP32_M, 0, 0, A.T_HEAD, 0, 0, A.T_NORM, 0, 0]
    gdt = ["bf16", "f32"] * 5
    _run_steps(env, sizes, flags, gdt, [(1, A.ZIP_SR, -1, 0), (2, A.V_SSR, A.ZIP_SR, 1)], seed=32)


def test_study_modes(env):
    """The controlled study's other v rules (state-space RTN, state-space SR, preconditioner-
    space RTN) on the ragged mixed list, alone and switching with ZIP-SR and ZE-EDEN (decoding
    the previous step's codebook), LM-head SR on and off, FP32 and BF16 grads."""
    A = env[0]
    sizes = [4095, 4096, 4097, 128 * 50 + 3, 7000, 128 * 200, 33333]
    flags = [0, 0, 0, 0, A.T_NORM, A.T_HEAD, 0]
    gdt = ["f32", "bf16", "f32", "bf16", "bf16", "bf16", "f32"]
    R, S, P = A.V_RTN, A.V_SSR, A.V_PRTN
    sched = [(1, R, -1, 0), (2, R, -1, 1), (3, S, R, 1), (4, S, -1, 0), (5, P, S, 0), (6, P, -1, 1),
             (7, A.ZE_EDEN, P, 0), (8, S, A.ZE_EDEN, 1), (9, A.ZIP_SR, S, 0), (10, R, A.ZIP_SR, 0)]
    rep = _run_steps(env, sizes, flags, gdt, sched, seed=8)
    print({k: v for k, v in rep.items() if "flips" in k and v})


def test_baseline_mode(env):
    """The baseline v rule (zero-excluding codebook, round to nearest, absmax scale) on the
    ragged mixed list, alone, after and before ZE-EDEN (same codebook) and ZIP-SR (the other
    one), LM-head SR on and off, zero-gradient blocks, FP32 and BF16 grads."""
    A = env[0]
    sizes = [4095, 4096, 4097, 128 * 50 + 3, 7000, 128 * 200, 33333, 300]
    flags = [0, 0, 0, 0, A.T_NORM, A.T_HEAD, 0, A.T_FP32_M]
    gdt = ["f32", "bf16", "f32", "bf16", "bf16", "bf16", "f32", "f32"]
    B, E, Z = A.V_ZE_RTN, A.ZE_EDEN, A.ZIP_SR
    sched = [(1, B, -1, 0), (2, B, -1, 1), (3, E, B, 1), (4, B, E, 0), (5, Z, B, 0), (6, B, Z, 1),
             (7, B, -1, 0)]
    rep = _run_steps(env, sizes, flags, gdt, sched, seed=11)
    print({k: v for k, v in rep.items() if "flips" in k and v})
    _run_steps(env, sizes, flags, gdt, [(1, B, -1, 1), (2, B, -1, 0)], seed=12, zero_frac=0.3)


def test_fp32_m_tensors(env):
    """Quantized tensors that keep m in FP32 (the controlled study's configuration) next to
    ordinary ones, ragged lengths, head and norm flags, BF16 and FP32 grads, every v mode."""
    A = env[0]
    F = A.T_FP32_M
    sizes = [4096, 4097, 128 * 50 + 3, 5000, 128 * 200, 33333, 300]
    flags = [F, F, F, F | A.T_NORM, F | A.T_HEAD, 0, F]
    gdt = ["f32", "bf16", "bf16", "f32", "bf16", "f32", "bf16"]
    sched = [(1, A.ZIP_SR, -1, 0), (2, A.V_SSR, A.ZIP_SR, 1), (3, A.V_RTN, A.V_SSR, 0),
             (4, A.V_PRTN, A.V_RTN, 1), (5, A.ZE_EDEN, A.V_PRTN, 0), (6, A.ZIP_SR, A.ZE_EDEN, 1),
             (7, A.V_ZE_RTN, A.ZIP_SR, 0), (8, A.V_ZE_RTN, -1, 1)]
    rep = _run_steps(env, sizes, flags, gdt, sched, seed=10)
    assert all(v for k, v in rep.items() if k.endswith("m_bitexact"))


def test_edge_cases(env):
    """Zero gradients (all-zero blocks), 30% exact zeros, beta2 = 0.95 as on the worked example,
    a late step (bias corrections ~1), tiny gradients (denormal-range v), and gradients so small
    that the m block scales fall below 2^-119."""
    A = env[0]
    sizes = [4096, 128 * 9 + 1, 200]
    flags = [0, A.T_HEAD, 0]
    _run_steps(env, sizes, flags, ["f32"] * 3, [(1, 0, -1, 1), (2, 1, 0, 1)], seed=2, grad_scale=0.0)
    _run_steps(env, sizes, flags, ["f32"] * 3, [(1, 0, -1, 0), (2, 0, -1, 1)], seed=3, zero_frac=0.3)
    _run_steps(env, sizes, flags, ["bf16"] * 3, [(1, 0, -1, 0), (2, 1, 0, 0)], seed=4,
               hp_extra=dict(beta2=0.95, eps=1e-8))
    _run_steps(env, sizes, flags, ["f32"] * 3, [(1000000, 0, -1, 1), (1000001, 1, 0, 1)], seed=5)
    _run_steps(env, sizes, flags, ["f32"] * 3, [(1, 0, -1, 0), (2, 1, 0, 1), (3, 0, 1, 0)], seed=6,
               grad_scale=1e-19)
    # block scales below 2^-119 but not zero (m' ~ 1e-38, v' underflows): the encoders' small-
    # scale branch, in both modes and with LM-head stochastic rounding
    _run_steps(env, sizes, flags, ["f32"] * 3, [(1, 0, -1, 1), (2, 1, 0, 1), (3, 0, 1, 0)], seed=7,
               grad_scale=1e-37)


def test_large_scales_and_eps(env):
    """Block scales above 2^100, where the reciprocal of the scale takes the exact division
    branch: |g| ~ 1e17 gives v' ~ 1e31 (2^103); with beta2 = 0, v' = g^2 reaches 2^127, so 1/s is
    subnormal; and an eps of 2^60, near the top of its range (2^64).  Every step replayed."""
    A = env[0]
    sizes = [4096, 128 * 9 + 1, 200]
    flags = [0, A.T_HEAD, 0]
    _run_steps(env, sizes, flags, ["f32"] * 3, [(1, 0, -1, 1), (2, 1, 0, 1), (3, 0, 1, 0)],
               seed=21, grad_scale=1e17)
    _run_steps(env, sizes, flags, ["f32"] * 3, [(1, 0, -1, 0), (2, 1, 0, 1), (3, 0, 1, 1)],
               seed=22, grad_scale=3e18, hp_extra=dict(beta2=0.0))
    _run_steps(env, sizes, flags, ["bf16"] * 3, [(1, 0, -1, 1), (2, 1, 0, 0), (3, 5, 1, 0)],
               seed=23, hp_extra=dict(eps=2.0 ** 60))


def test_extreme_hyperparameters(env):
    """Hyperparameters at the edges of their ranges, every step replayed:
    - the last step numbers the RNG counter holds (t = 2^32 - 2, 2^32 - 1, where both bias
      corrections round to 1) with the largest seed;
    - beta1 = 0 (m' = g), beta2 = 0.5, no weight decay;
    - lr = 0: the weights keep their bits while the moments move;
    - lr = 2e-3 at t = 1..3, where the update is as large as the N(0, 0.02) weights, so about
      half of them cancel towards zero or change sign (the weight bar at its hardest);
    - beta2 = 1 - 2^-24, the largest below 1, where bias correction divides by 1 - beta2^t ~ t 2^-24."""
    A = env[0]
    sizes = [4096, 128 * 9 + 1, 200, 128 * 64]
    flags = [0, A.T_HEAD, 0, 0]
    gdt = ["f32", "bf16", "f32", "bf16"]
    top = (1 << 32) - 1
    rep = {}
    _run_steps(env, sizes, flags, gdt, [(top - 1, 0, -1, 1), (top, 1, 0, 1)], seed=31,
               hp_extra=dict(seed=(1 << 64) - 1), report=rep)
    _run_steps(env, sizes, flags, gdt, [(1, 0, -1, 1), (2, 0, -1, 0), (3, 1, 0, 1)], seed=32,
               hp_extra=dict(beta1=0.0, beta2=0.5, weight_decay=0.0), report=rep)
    _run_steps(env, sizes, flags, gdt, [(1, 0, -1, 1), (2, 1, 0, 0)], seed=33,
               hp_extra=dict(lr=0.0), report=rep)
    _run_steps(env, sizes, flags, gdt, [(1, 0, -1, 0), (2, 0, -1, 1), (3, 1, 0, 0)], seed=34,
               hp_extra=dict(lr=2e-3), report=rep)
    _run_steps(env, sizes, flags, gdt, [(1, 0, -1, 1), (2, 1, 0, 0), (3, 0, 1, 1)], seed=35,
               hp_extra=dict(beta2=float(np.float32(1.0 - 2.0 ** -24))), report=rep)
    exact = [v for k, v in rep.items() if k.endswith("w_bitexact")]
    print(f"weights bit-exact in {sum(exact)} of {len(exact)} tensor-steps")


def test_run_twice_bit_identical(env):
    """Same inputs, same step: identical bits (no race in the block reductions)."""
    import torch
    from gpu_harness import GpuList, say
    A, orc = env
    sizes = [128 * 301 + 7, 5000]
    gl = GpuList(sizes, [A.T_HEAD, 0], ["bf16", "f32"], seed=9)
    gl.pl.init(0)
    gl.set_grads(1, seed=9)
    hp = A.hparams(step=1, sr_head=1, seed=5)
    gl.pl.step(hp)
    gl.set_grads(2, seed=9)
    p0 = [p.clone() for p in gl.params]
    s0 = [s.clone() for s in gl.pl.states]
    outs = []
    for rep in range(2):
        for p, q in zip(gl.params, p0):
            p.copy_(q)
        for s, q in zip(gl.pl.states, s0):
            s.copy_(q)
        say(f"repeat {rep}")
        gl.pl.step(A.hparams(step=2, sr_head=1, seed=5))
        torch.cuda.synchronize()
        outs.append([x.clone() for x in gl.params + gl.pl.states])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_random_lists(env):
    """Twelve seeded random lists (lengths from 1 to 3e5 around the 128-block and 4096-value
    boundaries, random NORM / HEAD / FP32_M flags and grad dtypes) stepped under random v-rule
    schedules with the LM-head switch on and off: every step replayed on the oracle."""
    A = env[0]
    rng = np.random.default_rng(2024)
    for case in range(12):
        k = int(rng.integers(1, 9))
        sizes = []
        for _ in range(k):
            kind = rng.integers(0, 4)
            if kind == 0:
                sizes.append(int(rng.integers(1, 4096)))
            elif kind == 1:
                sizes.append(4096 + int(rng.integers(-2, 3)) * int(rng.integers(0, 200)))
            elif kind == 2:
                sizes.append(128 * int(rng.integers(32, 400)) + int(rng.integers(0, 128)))
            else:
                sizes.append(int(rng.integers(4096, 300000)))
        sizes = [max(1, n) for n in sizes]
        flags = []
        for _ in sizes:
            f = 0
            r = rng.random()
            if r < 0.15:
                f |= A.T_NORM
            elif r < 0.3:
                f |= A.T_FP32_M
            if rng.random() < 0.2:
                f |= A.T_HEAD
            flags.append(f)
        gdt = [("bf16" if rng.random() < 0.6 else "f32") for _ in sizes]
        modes = [int(m) for m in rng.integers(0, 6, 3)]
        sched = []
        prev = -1
        for t, m in enumerate(modes, start=1):
            sched.append((t, m, prev if t > 1 else -1, int(rng.random() < 0.5)))
            prev = m
        _run_steps(env, sizes, flags, gdt, sched, seed=100 + case,
                   zero_frac=0.2 if case % 3 == 0 else 0.0)
