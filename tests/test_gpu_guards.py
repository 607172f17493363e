"""Out-of-bounds guard: every parameter, gradient and state buffer lives inside a larger device
allocation whose surrounding bytes hold a random pattern; after steps in both modes (ragged
lengths, FP32-state tensors, LM-head stochastic rounding, BF16 weight copies, init and decode)
the pattern must be intact and the results must still match the oracle."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

GUARD = 4096   # bytes of canary on each side


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


class Guarded:
    """A device byte buffer with `nbytes` usable bytes (16-B aligned) between two canaries."""

    def __init__(self, nbytes, rng):
        import torch
        self.n = nbytes
        self.total = GUARD + ((nbytes + 15) // 16) * 16 + GUARD
        host = rng.integers(0, 256, self.total, dtype=np.uint8)
        self.pattern = host.copy()
        self.buf = torch.from_numpy(host).cuda()

    def view(self, dtype, count):
        return self.buf[GUARD:GUARD + self.n].view(dtype)[:count]

    def intact(self):
        import torch
        torch.cuda.synchronize()
        h = self.buf.cpu().numpy()
        lo = np.array_equal(h[:GUARD], self.pattern[:GUARD])
        hi = np.array_equal(h[GUARD + self.n:], self.pattern[GUARD + self.n:])
        return lo and hi


def test_no_writes_outside_buffers(env):
    import torch
    from gpu_harness import oracle_state, compare_state, compare_weights, compare_bf16_copy, say, to_np
    A, orc = env
    rng = np.random.default_rng(21)
    sizes = [4095, 4096, 4097, 128 * 50 + 3, 64, 1, 7000, 128 * 40, 33333, 129]
    flags = [0, 0, 0, 0, 0, 0, A.T_NORM, A.T_HEAD, A.T_HEAD, 0]
    gdt = ["f32", "bf16", "bf16", "f32", "bf16", "f32", "bf16", "f32", "bf16", "f32"]
    guards, params, grads, states, specs, copies = [], [], [], [], [], []
    for n, f, gd in zip(sizes, flags, gdt):
        gc = Guarded(2 * n, rng)
        guards.append(gc)
        copies.append(gc.view(torch.bfloat16, n))
        gp = Guarded(4 * n, rng)
        gg = Guarded((2 if gd == "bf16" else 4) * n, rng)
        sb = A.state_bytes(n, f)
        gs = Guarded(sb, rng)
        p = gp.view(torch.float32, n)
        p.copy_(torch.from_numpy(rng.normal(0, 0.02, n).astype(np.float32)))
        g = gg.view(torch.bfloat16 if gd == "bf16" else torch.float32, n)
        guards += [gp, gg, gs]
        params.append(p)
        grads.append(g)
        states.append(gs.view(torch.uint8, sb))
    pl = A.ParamList(params, grads, flags, states=states, bf16_copies=copies)
    m0 = [torch.from_numpy(rng.normal(0, 1e-4, n).astype(np.float32)).cuda() for n in sizes]
    pl.init(A.ZIP_SR, m0, None)
    ostates = [orc.init_state(n, bool(f & A.T_NORM), orc.ZIP_SR, m0[i].cpu().numpy(), None)
               for i, (n, f) in enumerate(zip(sizes, flags))]
    ws = [to_np(p).copy() for p in params]
    sched = [(1, 0, -1, 0), (2, 1, 0, 1), (3, 0, 1, 1), (4, 0, -1, 0)]
    for t, mode, prev, srh in sched:
        for g in grads:
            g.copy_(torch.from_numpy(rng.normal(0, 1e-3, g.numel()).astype(np.float32)).to(g.dtype))
        kw = dict(step=t, mode=mode, prev_mode=prev, sr_head=srh, seed=3)
        gh = [to_np(g).copy() for g in grads]
        say(f"guarded step t={t} mode={mode}")
        pl.step(A.hparams(**kw))
        assert all(gd.intact() for gd in guards), f"canary overwritten at step {t}"
        rep = {}
        for i, n in enumerate(sizes):
            dbg = orc.step_tensor(ws[i], gh[i], ostates[i], orc.HParams(**kw), pos=i,
                                  head=bool(flags[i] & A.T_HEAD), dbg=True)
            compare_weights(f"t{t}:{i}", to_np(params[i]), ws[i], rep)
            compare_bf16_copy(f"t{t}:{i}", to_np(copies[i]), ws[i], to_np(params[i]))
            compare_state(f"t{t}:{i}", n, oracle_state(to_np(states[i]), n, flags[i]), ostates[i], dbg, rep)
            ws[i] = to_np(params[i]).copy()          # continue from the GPU's values
            ostates[i] = oracle_state(to_np(states[i]), n, flags[i])
    # decode into guarded outputs
    for i, n in enumerate(sizes):
        gm, gv = Guarded(4 * n, rng), Guarded(4 * n, rng)
        A.decode_state(pl.array[i], 0, gm.view(torch.float32, n).data_ptr(), gv.view(torch.float32, n).data_ptr())
        assert gm.intact() and gv.intact()


@pytest.mark.parametrize("entry", ["adamw4_step", "adamw4_step_noalloc"])
def test_shards_stay_inside_their_buffers(env, entry):
    """Shard entries (offsets into their whole tensors, RNG keys, short shards kept quantized,
    shards shorter than one block, which are all tail, an FP32-m shard, ragged last blocks)
    between canaries, stepped through either entry point: after four steps the canaries are
    intact and every step matches the oracle's step of the same element range."""
    import torch
    from gpu_harness import oracle_state, compare_state, compare_weights, compare_bf16_copy, say, to_np
    A, orc = env
    rng = np.random.default_rng(22)
    f32 = np.float32
    ents = [(300, A.T_SHARD, 1280), (128 * 5 + 7, A.T_SHARD | A.T_HEAD, 128 * 33),
            (4095, A.T_SHARD, 0), (1000, A.T_SHARD | A.T_FP32_M, 256), (129, A.T_SHARD, 128 * 7),
            (100, A.T_SHARD, 128 * 11), (1, A.T_SHARD | A.T_HEAD, 128 * 2)]
    keys = [11, 12, 13, 14, 15, 16, 17]
    guards, params, grads, states, copies = [], [], [], [], []
    for n, f, off in ents:
        gp, gg, gc = Guarded(4 * n, rng), Guarded(2 * n, rng), Guarded(2 * n, rng)
        sb = A.state_bytes(n, f)
        gs = Guarded(sb, rng)
        p = gp.view(torch.float32, n)
        p.copy_(torch.from_numpy(rng.normal(0, 0.02, n).astype(f32)))
        guards += [gp, gg, gs, gc]
        params.append(p)
        grads.append(gg.view(torch.bfloat16, n))
        states.append(gs.view(torch.uint8, sb))
        copies.append(gc.view(torch.bfloat16, n))
    pl = A.ParamList(params, grads, [f for _, f, _ in ents], states=states, bf16_copies=copies,
                     offsets=[o for _, _, o in ents], keys=keys)
    pl.init(A.ZIP_SR)
    assert all(gd.intact() for gd in guards), "canary overwritten by init"
    ws = [to_np(p).copy() for p in params]
    ostates = []
    for n, f, _ in ents:
        nb = (n + 127) // 128
        z8, zs = np.zeros((n + 1) // 2, np.uint8), np.zeros(nb, f32)
        if f & A.T_FP32_M:
            ostates.append(orc.State(True, None, z8.copy(), None, zs.copy(), m=np.zeros(n, f32)))
        else:
            ostates.append(orc.State(True, z8.copy(), z8.copy(), zs.copy(), zs.copy()))
    for t, mode, prev, srh in [(1, 0, -1, 1), (2, 3, 0, 1), (3, 1, 3, 0), (4, 0, 1, 1)]:
        for g in grads:
            g.copy_(torch.from_numpy(rng.normal(0, 1e-3, g.numel()).astype(f32)).to(g.dtype))
        kw = dict(step=t, mode=mode, prev_mode=prev, sr_head=srh, seed=4)
        gh = [to_np(g).copy() for g in grads]
        say(f"guarded shard step t={t} mode={mode} through {entry}")
        if entry == "adamw4_step":
            pl.step(A.hparams(**kw))
        else:
            A.step_noalloc(pl.array, A.hparams(**kw))
        assert all(gd.intact() for gd in guards), f"canary overwritten at step {t}"
        rep = {}
        for i, (n, f, off) in enumerate(ents):
            dbg = orc.step_tensor(ws[i], gh[i], ostates[i], orc.HParams(**kw), pos=keys[i],
                                  head=bool(f & A.T_HEAD), e0=off, n=off + n, dbg=True)
            compare_weights(f"t{t}:{i}", to_np(params[i]), ws[i], rep)
            compare_bf16_copy(f"t{t}:{i}", to_np(copies[i]), ws[i], to_np(params[i]))
            compare_state(f"t{t}:{i}", n, oracle_state(to_np(states[i]), n, f), ostates[i], dbg, rep)
            ws[i] = to_np(params[i]).copy()
            ostates[i] = oracle_state(to_np(states[i]), n, f)
