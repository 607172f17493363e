"""The step's host runtime on the GPU: buffers that move between steps, calls that never wait for
the device, and results that do not depend on how the work is cut into chunks and workgroups.
Every step goes through the C ABI (adamw4_step)."""
import os
import time

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import bit_adamw_step_amd as A
    import oracle as orc
    orc.build()
    return A, orc


SIZES = [128 * 40 + 3, 300, 4096, 128 * 333, 5000]
DTYPES = ["bf16", "f32", "bf16", "f32", "bf16"]


def _flags(A):
    return [A.T_HEAD, 0, A.T_NORM, 0, A.T_FP32_M]


def test_fresh_buffers_every_step(env):
    """Fourteen steps, each with gradients (and on even steps the weights too) in newly
    allocated buffers, half of them on a second stream: every step is replayed on the oracle
    from a snapshot of its inputs.  The list outgrows the descriptor tables' slots many times
    over, so slots are refilled while earlier steps may still read them."""
    import torch
    from gpu_harness import GpuList, say
    A, orc = env
    gl = GpuList(SIZES, _flags(A), DTYPES, seed=31)
    gl.pl.init(A.ZIP_SR)
    side = torch.cuda.Stream()
    report = {}
    for t in range(1, 15):
        gl.grads = [torch.empty_like(g) for g in gl.grads]
        if t % 2 == 0:
            gl.params = [p.clone() for p in gl.params]
        gl.pl.params, gl.pl.grads = gl.params, gl.grads
        gl.pl.refresh()
        gl.set_grads(t, seed=31)
        mode_at = lambda k: A.ZE_EDEN if k % 3 == 0 else A.ZIP_SR
        kw = dict(step=t, mode=mode_at(t), prev_mode=mode_at(t - 1) if t > 1 else -1,
                  sr_head=t % 2, seed=77)
        before = gl.snapshot()
        say(f"fresh buffers: step {t} mode {kw['mode']} stream {'side' if t % 2 else 'current'}")
        if t % 2:
            side.wait_stream(torch.cuda.current_stream())
            gl.pl.step(A.hparams(**kw), side)
            torch.cuda.current_stream().wait_stream(side)
        else:
            gl.pl.step(A.hparams(**kw))
        gl.replay_and_compare(before, kw, report, tag=f"t{t}:")
    print({k: v for k, v in report.items() if k.endswith("_flips") and v})


def _run(A, torch, gl, steps, stream=None):
    for t in steps:
        gl.set_grads(t, seed=41)
        gl.pl.step(A.hparams(step=t, sr_head=1, seed=3), stream)
    torch.cuda.synchronize()
    return [x.clone() for x in gl.params + gl.pl.states]


def test_step_calls_do_not_wait_for_the_device(env):
    """While a bounded sleep kernel keeps another stream busy for about a quarter of a second,
    twelve steps are enqueued on a second stream.  Each step's gradients are first copied on the
    device into one of four gradient-buffer sets, in rotation.  The first four calls see new
    buffer addresses and refill a descriptor slot asynchronously; the rest find their table
    resident.  Host time for all twelve calls stays far below the sleep, and the sleep is still
    running afterwards, so no call waited for the whole device.  The results equal the same
    twelve steps run with fixed buffers."""
    import torch
    from gpu_harness import GpuList, say
    A, orc = env
    flags = _flags(A)
    ref = GpuList(SIZES, flags, DTYPES, seed=41)
    for st in ref.pl.states:        # alignment padding between state sections is never written
        st.zero_()
    ref.pl.init(A.ZIP_SR)
    expect = _run(A, torch, ref, range(1, 13))

    gl = GpuList(SIZES, flags, DTYPES, seed=41)
    for st in gl.pl.states:
        st.zero_()
    gl.pl.init(A.ZIP_SR)
    grad_vals = []
    for t in range(1, 13):
        gl.set_grads(t, seed=41)
        grad_vals.append([g.clone() for g in gl.grads])
    # four buffer sets for the timed steps and four to warm the shape plan and the descriptor
    # slots (their results are discarded); all allocated outside the timed region
    sets = [[torch.zeros_like(g) for g in gl.grads] for _ in range(8)]
    work = torch.cuda.Stream()
    busy = torch.cuda.Stream()
    saved = ([p.clone() for p in gl.params], [s.clone() for s in gl.pl.states])
    for k in range(4):
        gl.pl.grads = sets[4 + k]
        gl.pl.refresh()
        gl.pl.step(A.hparams(step=1, seed=3), work)
    torch.cuda.synchronize()
    for p, q in zip(gl.params, saved[0]):
        p.copy_(q)
    for s, q in zip(gl.pl.states, saved[1]):
        s.copy_(q)
    arrays = []
    for k in range(4):
        gl.pl.grads = sets[k]
        gl.pl.refresh()
        arrays.append(gl.pl.array)
    torch.cuda.synchronize()
    done = torch.cuda.Event()
    with torch.cuda.stream(busy):
        torch.cuda._sleep(int(5e8))          # one spinning workgroup, about 0.25 s
        done.record(busy)
    say("sleep kernel enqueued; stepping")
    host = 0.0
    with torch.cuda.stream(work):
        for k in range(12):
            for g, v in zip(sets[k % 4], grad_vals[k]):
                g.copy_(v)
            t0 = time.perf_counter()
            A.step(arrays[k % 4], A.hparams(step=k + 1, sr_head=1, seed=3), work)
            host += time.perf_counter() - t0
    still_busy = not done.query()
    torch.cuda.synchronize()
    say(f"12 step calls took {1000 * host:.2f} ms of host time; sleep still running: {still_busy}")
    assert still_busy, "the sleep kernel finished before the step calls returned"
    assert host < 0.05
    got = [x.clone() for x in gl.params + gl.pl.states]
    for a, b in zip(got, expect):
        assert torch.equal(a, b)


@pytest.mark.parametrize("grid,chunk", [(37, 16), (1000, 1024), (256, 64)])
def test_launch_shape_does_not_change_bits(env, grid, chunk):
    """The same three steps (ZIP-SR with the LM head's stochastic rounding, ZE-EDEN, ZIP-SR)
    with the step launch forced to another workgroup count and chunk size: every weight, code,
    scale and FP32 moment is bit-identical to the default launch (the random numbers are keyed
    by element, never by workgroup)."""
    import torch
    from gpu_harness import GpuList, say
    A, orc = env
    sizes = [128 * 3000 + 77, 4096, 300, 1 << 20, 128 * 17]
    flags = [A.T_HEAD, 0, 0, A.T_FP32_M, 0]
    dts = ["bf16", "f32", "bf16", "bf16", "f32"]
    sched = [(1, 0, -1, 1), (2, 1, 0, 0), (3, 0, 1, 1)]

    def run():
        gl = GpuList(sizes, flags, dts, seed=5)
        for st in gl.pl.states:     # alignment padding between state sections is never written
            st.zero_()
        gl.pl.init(A.ZIP_SR)
        for t, mode, prev, srh in sched:
            gl.set_grads(t, seed=5)
            gl.pl.step(A.hparams(step=t, mode=mode, prev_mode=prev, sr_head=srh, seed=9))
        torch.cuda.synchronize()
        return [x.clone() for x in gl.params + gl.pl.states]

    base = run()
    os.environ["ADAMW4_GRID_OVERRIDE"] = str(grid)
    os.environ["ADAMW4_CHUNK_OVERRIDE"] = str(chunk)
    try:
        say(f"forced launch: {grid} workgroups, chunks of {chunk} blocks")
        other = run()
    finally:
        del os.environ["ADAMW4_GRID_OVERRIDE"]
        del os.environ["ADAMW4_CHUNK_OVERRIDE"]
    for a, b in zip(base, other):
        assert torch.equal(a, b)


def test_the_longest_list(env):
    """adamw4_step at its tensor limit, 65536 entries (ADAMW4_MAX_TENSORS): FP32-state tensors,
    quantized shards shorter than a block and of a few blocks, a quantized tensor of several
    chunks and an LM head, BF16 grads; every tensor a view into shared buffers, each starting
    16-byte aligned, with sentinel padding between the weight views.  One ZIP-SR step with the
    LM head's stochastic rounding: 600-odd sampled tensors replayed on the oracle, and every
    padding word still holds its sentinel."""
    import torch
    from gpu_harness import oracle_state, compare_state, compare_weights, to_np, say
    A, orc = env
    n_max = 65536
    rng = np.random.default_rng(90)
    sizes = [int(x) for x in rng.integers(1, 300, n_max)]
    flags = [A.T_SHARD if k % 3 == 0 else 0 for k in range(n_max)]
    sizes[7], flags[7] = 128 * 400 + 5, 0
    sizes[n_max - 2], flags[n_max - 2] = 128 * 90, A.T_HEAD
    pad8 = [(n + 7) // 8 * 8 for n in sizes]        # 16-byte starts for FP32 and BF16 views
    offs = np.concatenate([[0], np.cumsum(pad8)]).astype(np.int64)
    sb = [A.state_bytes(n, f) for n, f in zip(sizes, flags)]
    soffs = np.concatenate([[0], np.cumsum(sb)]).astype(np.int64)
    sentinel = 1234.5
    total = int(offs[-1])
    pad_np = np.ones(total, bool)
    for k, n in enumerate(sizes):
        pad_np[offs[k]: offs[k] + n] = False
    pad = torch.from_numpy(pad_np).cuda()
    g = torch.Generator(device="cpu")
    g.manual_seed(90)
    wbuf = (torch.randn(total, generator=g) * 0.02).cuda()
    wbuf[pad] = sentinel
    gbuf = (torch.randn(total, generator=g) * 1e-3).to(torch.bfloat16).cuda()
    sbuf = torch.zeros(int(soffs[-1]), dtype=torch.uint8, device="cuda")
    params = [wbuf.narrow(0, int(offs[k]), n) for k, n in enumerate(sizes)]
    grads = [gbuf.narrow(0, int(offs[k]), n) for k, n in enumerate(sizes)]
    states = [sbuf.narrow(0, int(soffs[k]), sb[k]) for k in range(n_max)]
    pl = A.ParamList(params, grads, flags, states=states)
    say(f"init of {n_max} tensors")
    pl.init(A.ZIP_SR)
    torch.cuda.synchronize()
    sample = sorted(set(range(0, n_max, 109)) | {7, n_max - 2, n_max - 1})
    w0 = {i: to_np(params[i]).copy() for i in sample}
    g0 = {i: to_np(grads[i]).copy() for i in sample}
    s0 = {i: oracle_state(to_np(states[i]), sizes[i], flags[i]) for i in sample}
    kw = dict(step=9, mode=A.ZIP_SR, sr_head=1, seed=12)
    say(f"step of {n_max} tensors")
    pl.step(A.hparams(**kw))
    torch.cuda.synchronize()
    assert torch.all(wbuf[pad] == sentinel), "a weight outside its view was written"
    rep = {}
    for i in sample:
        n, f = sizes[i], flags[i]
        w = w0[i]
        dbg = orc.step_tensor(w, g0[i], s0[i], orc.HParams(**kw), pos=i, head=bool(f & A.T_HEAD),
                              dbg=True)
        compare_weights(f"{i}", to_np(params[i]), w, rep)
        compare_state(f"{i}", n, oracle_state(to_np(states[i]), n, f), s0[i], dbg, rep)
    exact = [v for k, v in rep.items() if k.endswith("w_bitexact")]
    say(f"{len(sample)} sampled tensors match; weights bit-exact in {sum(exact)} of {len(exact)}")
