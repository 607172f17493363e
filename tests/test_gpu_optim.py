"""The torch Optimizer front end (bit_adamw_step_amd.optim.AdamW4bit) on the GPU:
  - every step equals the oracle's step of each parameter (single-step replay from the GPU's
    own state), across groups (norm, LM head with its late stochastic rounding, FP32 m), a
    v-encoder switch and FP32 and BF16 parameters;
  - BF16 parameters hold the round-to-nearest-even of their FP32 masters after every step;
  - a checkpoint taken mid-run (state_dict through torch.save / torch.load(weights_only=True))
    and loaded into a fresh model and optimizer continues bit-identically to the run that was
    never interrupted.
"""
import io

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
    from bit_adamw_step_amd import optim
    return A, oracle, optim


SHAPES = [("emb", (300, 64), {}), ("w1", (64, 129), {}), ("small", (40, 50), {}),
          ("norm", (64,), {"norm": True}), ("head", (300, 64), {"head": True}),
          ("w2", (80, 70), {"fp32_m": True})]


def _model(dtype, seed):
    import torch
    g = torch.Generator().manual_seed(seed)
    return [(torch.randn(*s, generator=g) * 0.02).to(dtype).cuda() for _, s, _ in SHAPES]


def _groups(params, mode):
    plain = [p for p, (_, _, o) in zip(params, SHAPES) if not o]
    gs = [{"params": plain, "mode": mode}]
    for p, (_, _, o) in zip(params, SHAPES):
        if o:
            gs.append(dict(params=[p], mode=mode, **o))
    return gs


def _set_grads(params, t, seed):
    import torch
    g = torch.Generator().manual_seed(seed * 1000 + t)
    for p in params:
        p.grad = (torch.randn(p.shape, generator=g) * 1e-3).to(p.dtype).cuda()


def _snap(opt, params):
    """Host copies of (FP32 weights, grads, packed state) per parameter."""
    from gpu_harness import to_np
    out = []
    for p in params:
        st = opt.state[p]
        # a BF16 parameter's master starts as the widened parameter
        w = st["master"] if "master" in st else p.float()
        out.append((to_np(w).copy().ravel(), to_np(p.grad).copy().ravel(),
                    to_np(st["packed"]).copy() if "packed" in st else None))
    return out


def _replay(A, orc, optim, opt, params, before, t, report):
    """Oracle step of every parameter from `before`; compare with the GPU's new state."""
    import torch
    from gpu_harness import oracle_state, compare_state, compare_weights, compare_bf16_copy, to_np
    torch.cuda.synchronize()
    key = 0
    for group in opt.param_groups:
        flags = optim.AdamW4bit._flags(group)
        for p in group["params"]:
            i = next(j for j, q in enumerate(params) if q is p)
            w, g, packed = before[i]
            st = opt.state[p]
            n = p.numel()
            b1, b2 = group["betas"]
            hp = orc.HParams(step=t, lr=group["lr"], beta1=b1, beta2=b2, eps=group["eps"],
                             weight_decay=group["weight_decay"], mode=optim.mode_id(group["mode"]),
                             prev_mode=report.get(("prev", key), -1),
                             sr_head=optim.sr_head_at(t, opt.total_steps), seed=opt.seed)
            ost = oracle_state(packed, n, flags) if packed is not None else \
                orc.init_state(n, bool(group["norm"]), hp.mode, fp32_m=bool(group["fp32_m"]))
            wr = w.copy()
            dbg = orc.step_tensor(wr, g, ost, hp, pos=key, head=bool(group["head"]), dbg=True)
            name = f"t{t} param {i}"
            wn = to_np(st["master"] if "master" in st else p).ravel()
            compare_weights(name, wn, wr, report)
            compare_state(name, n, oracle_state(to_np(st["packed"]), n, flags), ost, dbg, report)
            if p.dtype == torch.bfloat16:
                compare_bf16_copy(name, to_np(p).ravel(), wr, wn)
            report[("prev", key)] = hp.mode
            key += 1


def _run(A, orc, optim, dtype, schedule, seed, total_steps=None):
    import torch
    params = _model(dtype, seed)
    opt = optim.AdamW4bit(_groups(params, schedule[0]), lr=2e-3, weight_decay=0.05, seed=11,
                          total_steps=total_steps)
    report = {}
    for t, mode in enumerate(schedule, start=1):
        for g in opt.param_groups:
            g["mode"] = mode
        _set_grads(params, t, seed)
        before = _snap(opt, params)
        opt.step()
        _replay(A, orc, optim, opt, params, before, t, report)
    return params, opt, report


def test_optimizer_steps_match_oracle_fp32(env):
    """FP32 parameters through every v rule (mode switches included) and the LM-head switch."""
    import torch
    A, orc, optim = env
    sched = ["zip-sr", "zip-sr", "ze-eden", "ze-eden", "state-sr", "zip-sr", "baseline",
             "precond-rtn", "zip-sr", "zip-sr"]
    _, _, rep = _run(A, orc, optim, torch.float32, sched, seed=3, total_steps=10)
    assert all(v for k, v in rep.items() if isinstance(k, str) and k.endswith("w_bitexact"))


def test_optimizer_steps_match_oracle_bf16(env):
    """BF16 parameters: FP32 masters in the state, BF16 grads, rounded copy written back."""
    import torch
    A, orc, optim = env
    _, _, rep = _run(A, orc, optim, torch.bfloat16, ["zip-sr"] * 4 + ["ze-eden"] * 2, seed=4,
                     total_steps=5)
    assert all(v for k, v in rep.items() if isinstance(k, str) and k.endswith("w_bitexact"))


@pytest.mark.parametrize("dtype_name", ["bfloat16", "float32"])
def test_checkpoint_resume_bit_identical(env, dtype_name):
    """Save after 3 of 7 steps, restore into a fresh model and optimizer, finish: parameters,
    masters and packed states equal those of the uninterrupted run, bit for bit."""
    import torch
    from gpu_harness import to_np
    A, orc, optim = env
    dtype = getattr(torch, dtype_name)
    sched = ["zip-sr"] * 4 + ["ze-eden"] * 3

    def make():
        params = _model(dtype, 7)
        return params, optim.AdamW4bit(_groups(params, "zip-sr"), lr=2e-3, seed=5, total_steps=7)

    pa, oa = make()
    for t, mode in enumerate(sched, start=1):
        for g in oa.param_groups:
            g["mode"] = mode
        _set_grads(pa, t, 7)
        oa.step()

    pb, ob = make()
    for t, mode in enumerate(sched[:3], start=1):
        for g in ob.param_groups:
            g["mode"] = mode
        _set_grads(pb, t, 7)
        ob.step()
    buf = io.BytesIO()
    torch.save({"model": [p.detach().cpu() for p in pb], "optim": ob.state_dict()}, buf)
    del pb, ob
    buf.seek(0)
    ck = torch.load(buf, weights_only=True)
    pc = [t.cuda().contiguous() for t in ck["model"]]
    oc = optim.AdamW4bit(_groups(pc, "zip-sr"), lr=1.0, seed=0)   # hyperparameters come back
    oc.load_state_dict(ck["optim"])
    assert oc.seed == 5 and oc.total_steps == 7 and oc.param_groups[0]["lr"] == 2e-3
    for t, mode in enumerate(sched[3:], start=4):
        for g in oc.param_groups:
            g["mode"] = mode
        _set_grads(pc, t, 7)
        oc.step()
    torch.cuda.synchronize()
    for i, (a, c) in enumerate(zip(pa, pc)):
        assert torch.equal(a.view(torch.int16) if dtype == torch.bfloat16 else a.view(torch.int32),
                           c.view(torch.int16) if dtype == torch.bfloat16 else c.view(torch.int32)), i
        sa, sc = oa.state[a], oc.state[c]
        assert sa["step"] == sc["step"] == 7 and sa["v_mode"] == sc["v_mode"]
        if dtype == torch.bfloat16:
            assert torch.equal(sa["master"].view(torch.int32), sc["master"].view(torch.int32)), i
        from gpu_harness import oracle_state
        flags = optim.AdamW4bit._flags(next(g for g in oa.param_groups
                                            if any(q is a for q in g["params"])))
        xa = oracle_state(to_np(sa["packed"]), a.numel(), flags)
        xc = oracle_state(to_np(sc["packed"]), c.numel(), flags)
        for k in ("mcodes", "vcodes", "mscale", "vscale", "m", "v"):
            va, vc = getattr(xa, k), getattr(xc, k)
            assert (va is None and vc is None) or np.array_equal(va, vc), (i, k)


def test_decoded_moments(env):
    """decoded_moments returns the oracle's decode of the packed state."""
    import torch
    from gpu_harness import oracle_state, to_np
    A, orc, optim = env
    params, opt, _ = _run(A, orc, optim, torch.float32, ["ze-eden", "ze-eden"], seed=9)
    for group in opt.param_groups:
        flags = optim.AdamW4bit._flags(group)
        for p in group["params"]:
            m, v = opt.decoded_moments(p)
            st = oracle_state(to_np(opt.state[p]["packed"]), p.numel(), flags)
            rm, rv = orc.decode(st, p.numel(), orc.ZE_EDEN)
            assert np.array_equal(to_np(m).ravel(), rm) and np.array_equal(to_np(v).ravel(), rv)
