"""GPU parity of the step's optional outputs and entry forms, through the C ABI:
  - the fused BF16 copy of the updated weights (round to nearest even, the oracle's bf16_rne);
  - shards: a tensor split at 128-value block boundaries into entries with offsets and a common
    RNG key gives exactly the bits of the whole-tensor step (each block, its scales and its RNG
    counters stay the same), so a sharded caller needs no exchange inside the step;
  - RNG keys: with keys given, the list order does not change any result.
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


def test_bf16_copy_every_layout(env):
    """BF16 copies next to tensors without one: full blocks, a ragged tail, the fallback
    boundary, norm and head tensors, FP32-m, BF16 and FP32 grads; ZIP-SR with head SR, ZE-EDEN,
    state-space SR; each step replayed on the oracle (weights, state and copy)."""
    from gpu_harness import GpuList, say
    A, orc = env
    sizes = [4096, 4097, 128 * 50 + 3, 300, 7000, 128 * 200, 33333, 5000]
    flags = [0, 0, 0, 0, A.T_NORM, A.T_HEAD, A.T_FP32_M, 0]
    gdt = ["f32", "bf16", "bf16", "f32", "bf16", "bf16", "f32", "bf16"]
    copies = [True, True, True, True, True, True, True, False]
    gl = GpuList(sizes, flags, gdt, seed=21, copies=copies)
    gl.pl.init(A.ZIP_SR)
    rep = {}
    for t, mode, prev, srh in [(1, A.ZIP_SR, -1, 1), (2, A.ZE_EDEN, A.ZIP_SR, 0),
                               (3, A.V_SSR, A.ZE_EDEN, 1)]:
        gl.set_grads(t, seed=21)
        kw = dict(step=t, mode=mode, prev_mode=prev, sr_head=srh, seed=77)
        before = gl.snapshot()
        say(f"bf16 copy: step t={t} mode={mode}")
        gl.pl.step(A.hparams(**kw))
        gl.replay_and_compare(before, kw, rep, tag=f"t{t}:")
    assert all(v for k, v in rep.items() if k.endswith("w_bitexact"))


def test_bf16_copy_rounding_edges(env):
    """With lr = 0 and wd = 0 the step leaves every non-zero weight bit-identical (a zero may
    change sign), so the copy is the rounding of crafted weights: every BF16 exponent and
    mantissa, exact ties with even and odd kept halves and their neighbours, subnormals, signed
    zeros and the overflow edge.  Weights and copy are compared with the oracle's step."""
    import torch
    from gpu_harness import oracle_state, to_np, say
    A, orc = env
    hi = np.arange(0, 0x7F80, dtype=np.uint32)
    low = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF], np.uint32)
    bits = (hi[:, None] << 16 | low[None, :]).ravel()
    bits = np.concatenate([bits, bits | 0x80000000,
                           np.array([0x7F7FFFFF, 0x7F7F8000, 0xFF7F8000, 0x00000001], np.uint32)])
    w0 = bits.view(f32)
    n = w0.size
    nonzero = (bits & 0x7FFFFFFF) != 0
    for flags in (0, A.T_NORM):                       # quantized and FP32-state paths
        p = torch.from_numpy(w0.copy()).cuda()
        gh = (np.random.default_rng(5).normal(0, 1e-3, n)).astype(f32)
        g = torch.from_numpy(gh).cuda()
        c = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
        pl = A.ParamList([p], [g], [flags], bf16_copies=[c])
        pl.init(A.ZIP_SR)
        torch.cuda.synchronize()
        st = oracle_state(to_np(pl.states[0]).copy(), n, flags)
        say(f"bf16 rounding edges: n={n} flags={flags}")
        kw = dict(step=1, lr=0.0, weight_decay=0.0)
        pl.step(A.hparams(**kw))
        torch.cuda.synchronize()
        w_ref = w0.copy()
        orc.step_tensor(w_ref, gh, st, orc.HParams(**kw), pos=0, head=False)
        assert np.array_equal(w_ref.view(np.uint32)[nonzero], bits[nonzero])
        w_gpu = to_np(p)
        bad = np.nonzero(w_gpu.view(np.uint32) != w_ref.view(np.uint32))[0]
        assert bad.size == 0, (flags, "weights", bits[bad[:8]], w_gpu.view(np.uint32)[bad[:8]])
        got = to_np(c)
        exp = orc.bf16_rne(w_ref)
        bad = np.nonzero(got != exp)[0]
        assert bad.size == 0, (flags, "copy", bits[bad[:8]], got[bad[:8]], exp[bad[:8]])


def _split_list(A, sizes, flags, cuts):
    """Entries for the sharded list: tensor i split at the offsets in cuts[i]."""
    out = []
    for i, (n, f) in enumerate(zip(sizes, flags)):
        edges = [0] + list(cuts[i]) + [n]
        for a, b in zip(edges[:-1], edges[1:]):
            sf = f
            if A.is_quantized(n, f):
                sf |= A.T_SHARD
            out.append((i, a, b, sf))
    return out


def _assert_state_slice(A, whole, n, f, shard, a, b, sf, name):
    """A shard's state equals the matching slice of the whole tensor's state."""
    from gpu_harness import to_np
    W, S = to_np(whole), to_np(shard)
    ow, os_ = A.state_layout(n, f), A.state_layout(b - a, sf)
    if A.is_quantized(n, f):
        nb = (b - a + 127) // 128
        secs = [(1, (b - a + 1) // 2, a // 2), (3, 4 * nb, 4 * (a // 128))]
        if f & A.T_FP32_M:
            secs.append((0, 4 * (b - a), 4 * a))
        else:
            secs += [(0, (b - a + 1) // 2, a // 2), (2, 4 * nb, 4 * (a // 128))]
        for k, length, start in secs:
            lhs = S[os_[k]: os_[k] + length]
            rhs = W[ow[k] + start: ow[k] + start + length]
            assert np.array_equal(lhs, rhs), f"{name}: state section {k} differs"
    else:
        for k in (0, 1):
            lhs = S[os_[k]: os_[k] + 4 * (b - a)]
            rhs = W[ow[k] + 4 * a: ow[k] + 4 * b]
            assert np.array_equal(lhs, rhs), f"{name}: FP32 state {k} differs"


def test_shards_equal_whole_tensor(env):
    """The whole list in one call vs the same tensors as shards (offsets multiples of 128,
    lengths multiples of 128 but the last, a common key per tensor, shards shorter than 4096
    included) in one call: weights, BF16 copies and states bit-identical over ZIP-SR with head
    SR, state-space SR and ZE-EDEN steps.  The whole list's first step is also replayed on the
    oracle."""
    import torch
    from gpu_harness import GpuList, to_np, say
    A, orc = env
    sizes = [128 * 50 + 37, 9000, 128 * 300, 6000, 128 * 40]
    flags = [0, A.T_HEAD, A.T_FP32_M, A.T_NORM, 0]
    cuts = [[1280, 128 * 30], [4096], [128 * 7, 128 * 100, 128 * 299], [128 * 3], [128 * 39]]
    gdt = ["bf16", "bf16", "f32", "bf16", "f32"]
    gl = GpuList(sizes, flags, gdt, seed=31, copies=[True] * len(sizes))
    gl.pl.init(A.ZIP_SR)
    ents = _split_list(A, sizes, flags, cuts)
    params = [gl.params[i][a:b].clone() for (i, a, b, _) in ents]
    grads = [gl.grads[i][a:b].clone() for (i, a, b, _) in ents]
    copies = [torch.zeros(b - a, dtype=torch.bfloat16, device="cuda") for (i, a, b, _) in ents]
    sh = A.ParamList(params, grads, [sf for (_, _, _, sf) in ents], bf16_copies=copies,
                     offsets=[a for (_, a, _, _) in ents], keys=[i for (i, _, _, _) in ents])
    sh.init(A.ZIP_SR)
    for t, mode, prev, srh in [(1, A.ZIP_SR, -1, 1), (2, A.V_SSR, A.ZIP_SR, 1),
                               (3, A.ZE_EDEN, A.V_SSR, 0), (4, A.ZIP_SR, A.ZE_EDEN, 1)]:
        gl.set_grads(t, seed=31)
        for k, (i, a, b, _) in enumerate(ents):
            grads[k].copy_(gl.grads[i][a:b])
        kw = dict(step=t, mode=mode, prev_mode=prev, sr_head=srh, seed=99)
        before = gl.snapshot() if t == 1 else None
        say(f"shards: step t={t} mode={mode} entries={len(ents)}")
        gl.pl.step(A.hparams(**kw))
        sh.step(A.hparams(**kw))
        torch.cuda.synchronize()
        if before is not None:
            gl.replay_and_compare(before, kw, {}, tag="whole:")
        for k, (i, a, b, sf) in enumerate(ents):
            name = f"t{t} tensor {i} [{a}, {b})"
            assert np.array_equal(to_np(params[k]).view(np.uint32),
                                  to_np(gl.params[i][a:b]).view(np.uint32)), f"{name}: weights"
            assert np.array_equal(to_np(copies[k]), to_np(gl.copies[i][a:b])), f"{name}: BF16 copy"
            _assert_state_slice(A, gl.pl.states[i], sizes[i], flags[i], sh.states[k], a, b, sf, name)


def test_keys_make_list_order_irrelevant(env):
    """The same tensors keyed 0..n-1, stepped in the given order and reversed: identical bits
    (stochastic rounding of v and of the head's m included)."""
    import torch
    from gpu_harness import GpuList, oracle_state, to_np, say
    A, orc = env
    sizes = [4096 * 3, 128 * 77 + 5, 5000, 9000]
    flags = [0, 0, 0, A.T_HEAD]
    gl = GpuList(sizes, flags, ["bf16"] * 4, seed=41)
    order = list(range(len(sizes)))[::-1]
    rp = [gl.params[i].clone() for i in order]
    rg = [gl.grads[i] for i in order]
    rev = A.ParamList(rp, rg, [flags[i] for i in order], keys=order)
    fwd = A.ParamList(gl.params, gl.grads, flags, keys=list(range(len(sizes))))
    fwd.init(A.ZIP_SR)
    rev.init(A.ZIP_SR)
    for t in (1, 2, 3):
        gl.set_grads(t, seed=41)
        hp = A.hparams(step=t, mode=A.ZIP_SR, sr_head=1, seed=5)
        say(f"keys: step t={t}")
        fwd.step(hp)
        rev.step(hp)
        torch.cuda.synchronize()
        for k, i in enumerate(order):
            assert np.array_equal(to_np(rp[k]).view(np.uint32), to_np(gl.params[i]).view(np.uint32))
            # compare the state's sections (padding between them is never written)
            sa = oracle_state(to_np(rev.states[k]), sizes[i], flags[i])
            sb = oracle_state(to_np(fwd.states[i]), sizes[i], flags[i])
            for name in ("mcodes", "vcodes", "mscale", "vscale"):
                assert np.array_equal(getattr(sa, name), getattr(sb, name)), (t, i, name)


@pytest.mark.parametrize("mode", [0, 1, 2, 3, 4, 5])
def test_extra_kernel_equals_plain(env, mode):
    """Lists with BF16 copies run the step kernel's second instantiation: for every v rule it
    gives the plain kernel's weights and state bit for bit, and the copies are the weights'
    rounding (oracle's bf16_rne)."""
    import torch
    from gpu_harness import GpuList, oracle_state, to_np, say
    A, orc = env
    sizes = [4096 * 5 + 128 * 3, 128 * 77 + 5, 6000, 9000, 300]
    flags = [0, 0, A.T_NORM, A.T_HEAD, 0]
    gdt = ["bf16", "f32", "bf16", "bf16", "f32"]
    plain = GpuList(sizes, flags, gdt, seed=51)
    extra = GpuList(sizes, flags, gdt, seed=51, copies=[True] * len(sizes))
    plain.pl.init(mode)
    extra.pl.init(mode)
    for t in (1, 2, 3):
        plain.set_grads(t, seed=51)
        extra.set_grads(t, seed=51)
        hp = A.hparams(step=t, mode=mode, sr_head=int(t == 3), seed=8)
        say(f"extra vs plain: mode={mode} t={t}")
        plain.pl.step(hp)
        extra.pl.step(hp)
        torch.cuda.synchronize()
        for i, n in enumerate(sizes):
            wp, we = to_np(plain.params[i]), to_np(extra.params[i])
            assert np.array_equal(wp.view(np.uint32), we.view(np.uint32)), (mode, t, i)
            assert np.array_equal(to_np(extra.copies[i]), orc.bf16_rne(we)), (mode, t, i)
            sp = oracle_state(to_np(plain.pl.states[i]), n, flags[i])
            se = oracle_state(to_np(extra.pl.states[i]), n, flags[i])
            for k in ("mcodes", "vcodes", "mscale", "vscale", "m", "v"):
                a, b = getattr(sp, k), getattr(se, k)
                assert (a is None and b is None) or np.array_equal(a, b), (mode, t, i, k)
