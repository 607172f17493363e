"""adamw4_step_noalloc, the entry point for callers that cannot allocate device memory, against
adamw4_step on identical copies of a list: every weight, BF16 copy, code, scale and FP32 moment
must be bit-identical.  Two lists in a row, the second smaller than the first (the fixed device
array keeps the first call's tables), two steps each, through the C ABI.  Also the same call
recorded into a HIP graph and replayed: after every replay the list equals an identical copy
stepped by eager calls, with the program's own eager work and synchronizations between replays
(a replay repeats the captured call exactly, hyperparameters and step number included)."""
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import bit_adamw_step_amd as A
    return A


def _make(A, sizes, flags, dts, copies, seed):
    from gpu_harness import GpuList
    gl = GpuList(sizes, flags, dts, seed=seed, copies=copies)
    for st in gl.pl.states:        # alignment padding between state sections is never written
        st.zero_()
    gl.pl.init(A.ZIP_SR)
    return gl


def test_noalloc_equals_step(env):
    import torch
    from gpu_harness import say
    A = env
    lists = [
        # ragged quantized tensors, the 4096 boundary, FP32-state tensors, an FP32-m tensor,
        # a LM head, BF16 and FP32 gradients, one BF16 weight copy
        ([128 * 3000 + 77, 4096, 300, 1 << 20, 128 * 17, 5000],
         [A.T_HEAD, 0, 0, A.T_FP32_M, A.T_NORM, 0],
         ["bf16", "f32", "bf16", "bf16", "f32", "bf16"],
         [False, True, False, False, False, False]),
        # smaller: fewer tensors, fewer chunks, one tail
        ([4096 + 5, 200, 128 * 40], [0, A.T_NORM, A.T_HEAD], ["f32", "bf16", "bf16"],
         [False, False, False]),
    ]
    for k, (sizes, flags, dts, copies) in enumerate(lists):
        x = _make(A, sizes, flags, dts, copies, seed=60 + k)
        y = _make(A, sizes, flags, dts, copies, seed=60 + k)
        for t, mode, prev, srh in [(1, A.ZIP_SR, -1, 1), (2, A.ZE_EDEN, A.ZIP_SR, 0)]:
            x.set_grads(t, seed=60 + k)
            y.set_grads(t, seed=60 + k)
            hp = A.hparams(step=t, mode=mode, prev_mode=prev, sr_head=srh, seed=8)
            say(f"list {k} ({len(sizes)} tensors) step {t}: adamw4_step vs adamw4_step_noalloc")
            A.step(x.pl.array, hp)
            A.step_noalloc(y.pl.array, hp)
            torch.cuda.synchronize()
            outs_x = x.params + x.pl.states + [c for c in x.copies if c is not None]
            outs_y = y.params + y.pl.states + [c for c in y.copies if c is not None]
            for i, (a, b) in enumerate(zip(outs_x, outs_y)):
                assert torch.equal(a, b), f"list {k} step {t}: output {i} differs"


@pytest.mark.timeout(900)
def test_noalloc_equals_step_fullsize(env):
    """The Llama-style 2.7B list (291 tensors, 2.7e9 values; its chunk table at 64-block chunks
    would overflow the fixed array, so the allocation-free call takes 128-block chunks) stepped
    by both entry points from identical copies: weights and every state byte equal, compared on
    the device, over a round-to-nearest step and an LM-head stochastic-rounding step."""
    import torch
    import workloads as W
    from gpu_harness import say
    A = env
    w = W.WORKLOADS["llama2b7"]
    dev = torch.device("cuda:0")
    lists = []
    for copy in range(2):
        params = [W.make_param(s, i, dev) for i, s in enumerate(w.specs)]
        grads = [W.make_grad(w, s, i, 1, dev) for i, s in enumerate(w.specs)]
        pl = A.ParamList(params, grads, [s.flags for s in w.specs])
        for st in pl.states:
            st.zero_()
        pl.init(A.ZIP_SR)
        lists.append(pl)
    x, y = lists
    for t, srh in [(1, 0), (2, 1)]:
        if t > 1:
            for i, s in enumerate(w.specs):
                W.make_grad(w, s, i, t, dev, out=x.grads[i])
                y.grads[i].copy_(x.grads[i])
        hp = A.hparams(step=t, mode=A.ZIP_SR, sr_head=srh, seed=0)
        say(f"2.7B list step {t}: adamw4_step vs adamw4_step_noalloc")
        A.step(x.array, hp)
        A.step_noalloc(y.array, hp)
        torch.cuda.synchronize()
        for i in range(len(w.specs)):
            assert torch.equal(x.params[i].view(torch.int32), y.params[i].view(torch.int32)), (t, i)
            assert torch.equal(x.states[i], y.states[i]), (t, i)
    del lists, x, y
    torch.cuda.empty_cache()


def _outputs(gl):
    return gl.params + gl.pl.states + [c for c in gl.copies if c is not None]


def test_noalloc_graph_replays_equal_eager(env):
    import torch
    from gpu_harness import say
    A = env
    # ragged quantized tensors (a tail launch), an FP32-state tensor, an LM head, BF16 and FP32
    # grads, one BF16 weight copy (the kernel instance with extras)
    sizes = [128 * 700 + 33, 4096, 1000, 128 * 64, 5000]
    flags = [A.T_HEAD, 0, A.T_NORM, 0, 0]
    dts = ["bf16", "f32", "bf16", "bf16", "f32"]
    copies = [False, False, False, True, False]
    x = _make(A, sizes, flags, dts, copies, seed=90)     # stepped by the graph
    y = _make(A, sizes, flags, dts, copies, seed=90)     # stepped eagerly
    z = _make(A, [128 * 50, 700], [0, 0], ["bf16", "f32"], [False, False], seed=91)
    for gl in (x, y, z):
        gl.set_grads(1, seed=90)
    hp = A.hparams(step=7, mode=A.ZIP_SR, sr_head=1, seed=4)
    say("warm-up: one eager allocation-free step on both copies")
    A.step_noalloc(x.pl.array, hp)
    A.step_noalloc(y.pl.array, hp)
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(_outputs(x), _outputs(y))):
        assert torch.equal(a, b), f"warm-up: output {i} differs"

    say("capture one adamw4_step_noalloc call into a graph")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        A.step_noalloc(x.pl.array, hp)
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(_outputs(x), _outputs(y))):
        assert torch.equal(a, b), f"capture changed output {i}"   # capture runs nothing

    hz = A.hparams(step=3, mode=A.ZE_EDEN, prev_mode=A.ZIP_SR, seed=4)
    for r in range(4):
        say(f"replay {r}: graph on one copy, eager call on the other")
        g.replay()
        torch.cuda.synchronize()
        A.step_noalloc(y.pl.array, hp)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(_outputs(x), _outputs(y))):
            assert torch.equal(a, b), f"replay {r}: output {i} differs"
        A.step(z.pl.array, hz)             # other work of the program between replays
        torch.cuda.synchronize()
    del g


def test_noalloc_at_the_tensor_limit(env):
    """The longest list the allocation-free call takes (4096 entries, ADAMW4_NOALLOC_MAX_TENSORS:
    a hundred-odd upload launches, the plan kernel's search over every entry): FP32-state
    tensors, quantized shards shorter than a block (all tail) and of a few blocks, a quantized
    tensor of several chunks and an LM head, BF16 and FP32 grads.  Bit-identical to adamw4_step
    over two steps."""
    import numpy as np
    import torch
    from gpu_harness import say
    A = env
    n_max = 4096
    rng = np.random.default_rng(70)
    sizes = [int(x) for x in rng.integers(1, 1500, n_max)]
    flags = [A.T_SHARD if k % 3 == 0 else 0 for k in range(n_max)]
    sizes[5], flags[5] = 128 * 300 + 9, 0
    sizes[4000], flags[4000] = 128 * 1000, A.T_HEAD
    dts = ["bf16" if k % 2 else "f32" for k in range(n_max)]
    x = _make(A, sizes, flags, dts, None, seed=70)
    y = _make(A, sizes, flags, dts, None, seed=70)
    for t, mode, prev, srh in [(1, A.ZIP_SR, -1, 1), (2, A.ZE_EDEN, A.ZIP_SR, 0)]:
        x.set_grads(t, seed=70)
        y.set_grads(t, seed=70)
        hp = A.hparams(step=t, mode=mode, prev_mode=prev, sr_head=srh, seed=3)
        say(f"{n_max} tensors, step {t}: adamw4_step vs adamw4_step_noalloc")
        A.step(x.pl.array, hp)
        A.step_noalloc(y.pl.array, hp)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(_outputs(x), _outputs(y))):
            assert torch.equal(a, b), f"step {t}: output {i} differs"
