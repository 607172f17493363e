"""Parity at the benchmark workloads' full sizes, in the launch configuration bench.py times:
the whole parameter list is stepped on the GPU, and at selected steps sampled 128-value blocks
of every quantized tensor (first, last and random blocks, 64 per tensor) plus every FP32-state
tensor are replayed on the oracle from a snapshot taken just before the step.

Lists (workloads module): GPT 130M-shape (ZIP-SR, BF16 row-scaled grads), GPT 834M-shape
(ZE-EDEN, v pre-seeded 10^U(-20,-4) through the init encoder), Llama 2.7B-shape (ZIP-SR,
LM-head stochastic rounding switched on at t = 181 of 200), the stress list (one 2^30-value
tensor + 2000 FP32-state tensors, Student-t grads with 30% zeros, ZIP-SR / ZE-EDEN alternating),
and the 834M shapes with FP32 first moments under the four zero-inclusive v rules in turn.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

BLOCKS_PER_TENSOR = 64


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


def _setup(w, A):
    import torch
    import workloads as W
    dev = torch.device("cuda:0")
    params = [W.make_param(s, i, dev) for i, s in enumerate(w.specs)]
    grads = [W.make_grad(w, s, i, 1, dev) for i, s in enumerate(w.specs)]
    pl = A.ParamList(params, grads, [s.flags for s in w.specs])
    v0 = None
    if w.v0_kind != "zeros":
        v0 = [W.make_v0(w, s, i, dev) for i, s in enumerate(w.specs)]
    pl.init(w.mode_at(1), None, v0)
    torch.cuda.synchronize()
    return pl, v0


def _samples(w, A, rng):
    out = []
    for i, s in enumerate(w.specs):
        n = s.numel
        if not A.is_quantized(n, s.flags):
            out.append((i, 0, n))                       # whole FP32-state tensor
            continue
        nb = (n + 127) // 128
        picks = {0, nb - 1} | set(rng.integers(0, nb, BLOCKS_PER_TENSOR - 2).tolist())
        for b in sorted(picks):
            e0 = 128 * b
            out.append((i, e0, min(128, n - e0)))
    return out


def _grab(pl, A, w, i, e0, cnt):
    """Host copies of (w, g, state section slices) for elements [e0, e0+cnt) of tensor i."""
    import torch
    from gpu_harness import to_np
    import oracle as orc
    s = w.specs[i]
    n = s.numel
    wv = to_np(pl.params[i][e0:e0 + cnt]).copy()
    gv = to_np(pl.grads[i][e0:e0 + cnt]).copy()
    buf = pl.states[i]
    off = A.state_layout(n, s.flags)
    if A.is_quantized(n, s.flags):
        b0, nb = e0 // 128, (cnt + 127) // 128
        c0, c1 = e0 // 2, (e0 + cnt + 1) // 2
        sl = lambda o, a, z: to_np(buf[o + a:o + z]).copy()
        if s.flags & A.T_FP32_M:
            st = orc.State(True, None, sl(off[1], c0, c1), None,
                           sl(off[3], 4 * b0, 4 * (b0 + nb)).view(np.float32),
                           m=sl(off[0], 4 * e0, 4 * (e0 + cnt)).view(np.float32))
        else:
            st = orc.State(True, sl(off[0], c0, c1), sl(off[1], c0, c1),
                           sl(off[2], 4 * b0, 4 * (b0 + nb)).view(np.float32),
                           sl(off[3], 4 * b0, 4 * (b0 + nb)).view(np.float32))
    else:
        st = orc.State(False, m=to_np(buf[off[0]:off[0] + 4 * n]).view(np.float32).copy(),
                       v=to_np(buf[off[1]:off[1] + 4 * n]).view(np.float32).copy())
    return wv, gv, st


def _run(env, wname, replay_ts):
    import torch
    import workloads as W
    from gpu_harness import compare_state, compare_weights, say
    A, orc = env
    w = W.WORKLOADS[wname]
    say(f"fullsize {wname}: {len(w.specs)} tensors, {w.numel} values")
    pl, v0 = _setup(w, A)
    rng = np.random.default_rng(17)
    samples = _samples(w, A, rng)
    report = {}
    if v0 is not None:   # the init encoder on the sampled blocks
        for (i, e0, cnt) in samples:
            s = w.specs[i]
            if not A.is_quantized(s.numel, s.flags):
                continue
            _, _, st = _grab(pl, A, w, i, e0, cnt)
            ref = orc.State(True, np.zeros_like(st.mcodes), np.zeros_like(st.vcodes),
                            np.zeros_like(st.mscale), np.zeros_like(st.vscale))
            v0h = v0[i][e0:e0 + cnt].cpu().numpy()
            orc.lib().orc_encode_init(None, v0h.ctypes.data, s.numel, e0, cnt, w.mode_at(1),
                                      ref.mcodes.ctypes.data, ref.vcodes.ctypes.data,
                                      ref.mscale.ctypes.data, ref.vscale.ctypes.data)
            compare_state(f"init:{i}@{e0}", cnt, st, ref, None, report)
    del v0
    prev = w.mode_at(1)
    last = max(replay_ts)
    for t in range(1, last + 1):
        mode = w.mode_at(t)
        kw = dict(step=t, mode=mode, prev_mode=prev, sr_head=w.sr_head_at(t), seed=0)
        prev = mode
        if t in replay_ts:
            before = [(i, e0, cnt) + _grab(pl, A, w, i, e0, cnt) for (i, e0, cnt) in samples]
            say(f"  replay t={t} mode={mode} sr_head={kw['sr_head']} ({len(samples)} samples)")
        pl.step(A.hparams(**kw))
        if t not in replay_ts:
            continue
        torch.cuda.synchronize()
        for (i, e0, cnt, wv, gv, st) in before:
            s = w.specs[i]
            dbg = orc.step_tensor(wv, gv, st, orc.HParams(**kw), pos=i, head=bool(s.flags & 2),
                                  e0=e0, n=s.numel, dbg=True)
            w_now, _, st_now = _grab(pl, A, w, i, e0, cnt)
            name = f"{wname}:t{t}:{i}@{e0}"
            compare_weights(name, w_now, wv, report)
            compare_state(name, cnt, st_now, st, dbg, report)
    flips = sum(v for k, v in report.items() if k.endswith("_flips"))
    exact = all(v for k, v in report.items() if k.endswith("_bitexact"))
    say(f"  {wname}: permitted stochastic flips {flips}, weights/FP32 states bit-exact {exact}")


@pytest.mark.timeout(900)
def test_llama2b7_full(env):
    _run(env, "llama2b7", {1, 2, 180, 181, 200})


@pytest.mark.timeout(900)
def test_gpt130m_full(env):
    _run(env, "gpt130m", {1, 2, 50, 100})


@pytest.mark.timeout(900)
def test_gpt834m_full(env):
    _run(env, "gpt834m", {1, 2, 25, 50})


@pytest.mark.timeout(900)
def test_stress_full(env):
    _run(env, "stress", {1, 2, 3, 20})


@pytest.mark.timeout(900)
def test_study834m_full(env):
    """834M GPT shapes with FP32 first moments, v by ZIP-SR / state RTN / state SR /
    preconditioner RTN in turn (the controlled study's configuration)."""
    _run(env, "study834m", {1, 2, 3, 4, 5, 40})


@pytest.mark.timeout(900)
def test_baseline130m_full(env):
    """130M GPT shapes under the baseline v rule (zero-free codebook, round to nearest, absmax
    scale), from log-uniform initial second moments, across the LM-head SR switch."""
    _run(env, "baseline130m", {1, 2, 90, 91, 100})


@pytest.mark.timeout(900)
def test_llama2b7_rank0_share_equals_whole(env):
    """Rank 0's share of an 8-way split of the 2.7B list (the shape `bench.py --shard-of 8`
    times: the first 128-aligned eighth of every tensor, quantized pieces flagged as shards,
    keyed by tensor index) stepped in one call, against the whole list stepped in another: the
    share's weights, codes and scales equal the whole tensors' leading slices bit for bit over
    ZIP-SR steps with and without LM-head stochastic rounding (compared on the device)."""
    import torch
    import bench
    import workloads as W
    from gpu_harness import say
    A, orc = env
    w = W.WORKLOADS["llama2b7"]
    say(f"rank-0 share vs whole: {len(w.specs)} tensors, {w.numel} values")
    whole, _ = _setup(w, A)
    lens = [bench.shard_len(s.numel, 8) for s in w.specs]
    flags = [s.flags | (A.T_SHARD if A.is_quantized(s.numel, s.flags) else 0) for s in w.specs]
    share = A.ParamList([whole.params[i][:L].clone() for i, L in enumerate(lens)],
                        [whole.grads[i][:L].clone() for i, L in enumerate(lens)], flags,
                        keys=list(range(len(lens))))
    share.init(A.ZIP_SR)
    dev = torch.device("cuda:0")
    for t in (1, 2, 3):
        if t > 1:
            for i, s in enumerate(w.specs):
                W.make_grad(w, s, i, t, dev, out=whole.grads[i])
                share.grads[i].copy_(whole.grads[i][:lens[i]])
        hp = A.hparams(step=t, mode=A.ZIP_SR, sr_head=int(t == 3), seed=0)
        say(f"  step t={t} sr_head={int(t == 3)}")
        whole.step(hp)
        share.step(hp)
        torch.cuda.synchronize()
        for i, (s, L) in enumerate(zip(w.specs, lens)):
            assert torch.equal(share.params[i].view(torch.int32),
                               whole.params[i][:L].view(torch.int32)), (t, i, "weights")
            ow, osh = A.state_layout(s.numel, s.flags), A.state_layout(L, flags[i])
            if A.is_quantized(s.numel, s.flags):
                nb = (L + 127) // 128
                secs = [(0, (L + 1) // 2), (1, (L + 1) // 2), (2, 4 * nb), (3, 4 * nb)]
            else:
                secs = [(0, 4 * L), (1, 4 * L)]
            for k, length in secs:
                a = share.states[i][osh[k]:osh[k] + length]
                b = whole.states[i][ow[k]:ow[k] + length]
                assert torch.equal(a, b), (t, i, "state section", k)


class _Spec:
    def __init__(self, numel, flags):
        self.numel, self.flags = numel, flags


class _List:
    def __init__(self, specs):
        self.specs = specs


@pytest.mark.timeout(900)
def test_tensor_past_2_31_elements(env):
    """One LM-head tensor of 2^31 + 717 values (element offsets, RNG counters and block indices
    past 32-bit signed range; a ragged last block of 77 values) beside a small tensor, three
    steps (ZIP-SR with the LM head's stochastic rounding, ZE-EDEN, ZIP-SR again), each replayed
    on the oracle over sampled blocks: the first, those around element 2^31, the last full one,
    the partial last one and 40 random ones."""
    import torch
    from gpu_harness import compare_state, compare_weights, say
    A, orc = env
    n_big = (1 << 31) + 128 * 5 + 77
    lst = _List([_Spec(n_big, A.T_HEAD), _Spec(5000, 0)])
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(31)
    params = [torch.randn(s.numel, generator=gen, device=dev).mul_(0.02) for s in lst.specs]
    grads = [torch.empty(s.numel, dtype=torch.bfloat16, device=dev) for s in lst.specs]
    pl = A.ParamList(params, grads, [s.flags for s in lst.specs])
    for st in pl.states:
        st.zero_()
    pl.init(A.ZIP_SR)
    nb = (n_big + 127) // 128
    rng = np.random.default_rng(31)
    picks = {0, (1 << 24) - 2, (1 << 24) - 1, 1 << 24, (1 << 24) + 1, nb - 2, nb - 1}
    picks |= set(rng.integers(0, nb, 40).tolist())
    samples = [(0, 128 * b, min(128, n_big - 128 * b)) for b in sorted(picks)] + [(1, 0, 5000)]
    report = {}
    prev = A.ZIP_SR
    for t, mode, srh in [(1, A.ZIP_SR, 1), (2, A.ZE_EDEN, 0), (3, A.ZIP_SR, 1)]:
        for g in grads:
            g.copy_(torch.randn(g.numel(), generator=gen, device=dev).mul_(1e-3))
        kw = dict(step=t, mode=mode, prev_mode=prev, sr_head=srh, seed=5)
        prev = mode
        torch.cuda.synchronize()
        before = [(i, e0, cnt) + _grab(pl, A, lst, i, e0, cnt) for (i, e0, cnt) in samples]
        say(f"tensor of {n_big} values: step t={t} mode={mode} ({len(samples)} samples)")
        pl.step(A.hparams(**kw))
        torch.cuda.synchronize()
        for (i, e0, cnt, wv, gv, st) in before:
            s = lst.specs[i]
            dbg = orc.step_tensor(wv, gv, st, orc.HParams(**kw), pos=i, head=bool(s.flags & A.T_HEAD),
                                  e0=e0, n=s.numel, dbg=True)
            w_now, _, st_now = _grab(pl, A, lst, i, e0, cnt)
            name = f"big:t{t}:{i}@{e0}"
            compare_weights(name, w_now, wv, report)
            compare_state(name, cnt, st_now, st, dbg, report)
    flips = sum(v for k, v in report.items() if k.endswith("_flips"))
    exact = all(v for k, v in report.items() if k.endswith("_bitexact"))
    say(f"  permitted stochastic flips {flips}, weights/FP32 states bit-exact {exact}")
    del pl, params, grads
    torch.cuda.empty_cache()
