"""Pins of the CPU oracle to facts fixed by the pages and by mathematics (no GPU needed).

Each test names the passage or the identity it checks.  Page tags: [lav-*] learnaivisually.com
explainer "ZIP-SR 4-bit AdamW", [daiwk-*] daiwk.github.io notes "ZIP-SR / ZE-EDEN: 4-bit AdamW
state quantization" ("Core equation", "Local reproduction"), [kc-*] kongchang.com explainer.
"""
import json
import os
import shutil
import subprocess
import sys

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
HELPERS = os.path.join(os.path.dirname(__file__), "helpers")

f32 = np.float32


def h64(v, bc2, eps):
    """Preconditioner multiplier h(v) = 1/(sqrt(v/bc2) + eps) ([daiwk-CE]), binary64."""
    return 1.0 / (np.sqrt(np.asarray(v, np.float64) / bc2) + eps)


# ---------------------------------------------------------------------------------------------
# P-12  NF4 and the v codebooks
# ---------------------------------------------------------------------------------------------

def test_nf4_matches_scipy_quantile_construction(orc):
    """NF4 ([lav-ZE], [kc-TC]) = QLoRA normal-quantile construction; scipy's norm.ppf is an
    independent quantile routine (the oracle uses bisection on erfc)."""
    from scipy.stats import norm
    d = 1 - 0.5 * (1 / 30 + 1 / 32)
    pos = norm.ppf(np.linspace(d, 0.5, 9)[:-1])
    neg = -norm.ppf(np.linspace(d, 0.5, 8)[:-1])
    ref = (np.sort(np.concatenate([pos, neg, [0.0]])) / norm.ppf(d)).astype(f32)
    nf4 = orc.codebook(orc.CB_NF4)
    assert np.array_equal(nf4, ref)
    assert nf4[0] == -1 and nf4[15] == 1 and nf4[7] == 0
    assert np.all(np.diff(nf4) > 0)
    assert (nf4 > 0).sum() == 8 and (nf4 < 0).sum() == 7


def test_v_codebooks(orc):
    """ZIP-SR keeps zero in the v codebook, ZE-EDEN's lowest level is positive ([kc-TC], [lav-ST])."""
    from fractions import Fraction
    v0 = orc.codebook(orc.CB_V0)
    v1 = orc.codebook(orc.CB_V1)
    for k in range(16):
        # V0[k] is k/15 correctly rounded: the nearest float to the exact fraction
        x = Fraction(k, 15)
        cand = float(v0[k])
        assert abs(Fraction(cand) - x) <= abs(Fraction(float(np.nextafter(f32(cand), f32(2)))) - x)
        assert abs(Fraction(cand) - x) <= abs(Fraction(float(np.nextafter(f32(cand), f32(-2)))) - x)
        assert v1[k] == (k + 1) / 16
    assert v0[0] == 0 and v0[15] == 1 and v1.min() > 0 and v1[15] == 1
    assert np.all(np.diff(v0) > 0) and np.all(np.diff(v1) > 0)


# ---------------------------------------------------------------------------------------------
# P-13  Philox4x32-10 against rocRAND's implementation
# ---------------------------------------------------------------------------------------------

def test_philox_matches_rocrand(orc, tmp_path):
    """The oracle's Philox4x32-10 equals rocRAND's philox4x32_10 engine (independent code)."""
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available to build the rocRAND known-answer helper")
    exe = tmp_path / "kat"
    subprocess.run([hipcc, "-O1", "-o", str(exe), os.path.join(HELPERS, "rocrand_philox_kat.cpp")],
                   check=True, cwd=str(tmp_path), capture_output=True)
    rng = np.random.default_rng(5)
    cases = [[0, 0, 0, 0, 0, 0], [1, 2, 3, 4, 5, 6],
             [0xFFFFFFFF, 0x3FFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF]]
    for _ in range(200):
        c = rng.integers(0, 2**32, 6, dtype=np.uint64).tolist()
        c[1] &= 0x3FFFFFFF
        cases.append(c)
    inp = "\n".join(" ".join("%x" % x for x in c) for c in cases) + "\n"
    out = subprocess.run([str(exe)], input=inp, capture_output=True, text=True, check=True).stdout
    for c, line in zip(cases, out.strip().splitlines()):
        ref = [int(x, 16) for x in line.split()]
        got = orc.philox4x32_10(c[:4], c[4:]).tolist()
        assert got == ref, (c, got, ref)


def test_uniform_counter_layout(orc):
    """u for element i = word (i & 3) of the block with counter (i>>2, stream<<31, pos, t)."""
    for (seed, t, pos, stream, i) in [(0, 1, 0, 0, 0), (123456789012, 7, 5, 1, 2**33 + 6),
                                      (2**63 + 5, 200, 290, 0, 1023)]:
        j = i >> 2
        ctr = [j & 0xFFFFFFFF, ((j >> 32) | (stream << 31)) & 0xFFFFFFFF, pos, t]
        key = [seed & 0xFFFFFFFF, seed >> 32]
        w = orc.philox4x32_10(ctr, key)[i & 3]
        assert orc.uniform(seed, t, pos, stream, i) == f32(int(w) >> 8) * f32(2.0**-24)


# ---------------------------------------------------------------------------------------------
# P-1 / P-2 / P-3  AdamW recurrence, update order
# ---------------------------------------------------------------------------------------------

def _torch_adamw_traj(w0, grads, hp):
    import torch
    p = torch.nn.Parameter(torch.tensor(w0.copy()))
    x32 = lambda x: float(f32(x))  # the step takes its hyperparameters as FP32 values
    opt = torch.optim.AdamW([p], lr=x32(hp.lr), betas=(x32(hp.beta1), x32(hp.beta2)),
                            eps=x32(hp.eps), weight_decay=x32(hp.weight_decay), foreach=False,
                            fused=False)
    for g in grads:
        p.grad = torch.tensor(g)
        opt.step()
    st = opt.state[p]
    return p.detach().numpy().copy(), st["exp_avg"].numpy().copy(), st["exp_avg_sq"].numpy().copy()


def test_fp32_path_equals_torch_adamw(orc):
    """Quantization off (FP32 states) the step is textbook AdamW with decoupled weight decay and
    bias correction ([kc-WHY], [daiwk-CE]); torch.optim.AdamW is an independent implementation
    whose op order differs (lerp for m, division by sqrt(bc2)), so agreement is to a few ulp of
    the operands of each final subtraction."""
    rng = np.random.default_rng(0)
    n = 5000
    w0 = rng.normal(0, 0.02, n).astype(f32)
    grads = [rng.normal(0, 1e-3, n).astype(f32) for _ in range(10)]
    w = w0.copy()
    st = orc.init_state(n, True, orc.ZIP_SR)
    for t, g in enumerate(grads, 1):
        orc.step_tensor(w, g, st, orc.HParams(step=t), pos=0)
    hp = orc.HParams(step=1)
    tw, tm, tv = _torch_adamw_traj(w0, grads, hp)
    # m and v are sums of opposite-sign or tiny terms; rounding error scales with the operands,
    # bounded here by the largest moment magnitude (a few ulp of it per step)
    np.testing.assert_allclose(st.m, tm, rtol=2e-6, atol=2e-6 * np.abs(tm).max())
    np.testing.assert_allclose(st.v, tv, rtol=2e-6, atol=2e-6 * np.abs(tv).max())
    # ten updates of size <= ~lr each: bound by operand magnitude
    tol = 2e-6 * (np.abs(tw) + 10 * hp.lr)
    assert np.all(np.abs(w - tw) <= tol)


def test_fp32_path_near_binary64_textbook(orc):
    """One FP32 step vs the same recurrence in binary64: error within a few FP32 roundings."""
    rng = np.random.default_rng(1)
    n = 20000
    w = rng.normal(0, 0.02, n).astype(f32)
    g = rng.normal(0, 1e-3, n).astype(f32)
    m = rng.normal(0, 1e-4, n).astype(f32)
    v = (rng.random(n) * 1e-6).astype(f32)
    for t in (1, 2, 50, 1000):
        hp = orc.HParams(step=t)
        st = orc.State(False, m=m.copy(), v=v.copy())
        w1 = w.copy()
        orc.step_tensor(w1, g, st, hp, pos=0)
        b1, b2 = float(f32(hp.beta1)), float(f32(hp.beta2))
        m64 = b1 * m.astype(np.float64) + (1 - b1) * g
        v64 = b2 * v.astype(np.float64) + (1 - b2) * g.astype(np.float64) ** 2
        den64 = np.sqrt(v64 / (1 - b2**t)) + float(f32(hp.eps))
        step = float(f32(hp.lr)) / (1 - b1**t)
        upd = step * m64 / den64
        w64 = w.astype(np.float64) * (1 - float(f32(hp.lr)) * float(f32(hp.weight_decay))) - upd
        u = 2.0**-24
        # a rounded sum of two rounded products: error <= 2u (|b1 m| + |(1-b1) g|)
        dm = 2 * u * (b1 * np.abs(m) + (1 - b1) * np.abs(g))
        assert np.all(np.abs(st.m - m64) <= dm)
        np.testing.assert_allclose(st.v, v64, rtol=4 * u, atol=0)
        # w: a few roundings of each operand, plus the moment error carried through the update
        assert np.all(np.abs(w1 - w64) <= 8 * u * (np.abs(w) + np.abs(upd)) + 1.01 * step * dm / den64)


def _quant_tensor(orc, n, rng, head=False, mode=0):
    w = rng.normal(0, 0.02, n).astype(f32)
    st = orc.init_state(n, False, mode)
    return w, st


@pytest.mark.parametrize("mode", [0, 1, 2, 3, 4, 5])
def test_step1_weights_equal_fp32_adamw(orc, mode):
    """From m0 = v0 = 0 the quantized state decodes to 0, and weights are updated from the
    unquantized working moments before requantization ([daiwk-CE], [daiwk-PM]), so step-1
    weights equal the FP32 path bit for bit in both modes."""
    rng = np.random.default_rng(2)
    n = 8192 + 77
    w, st = _quant_tensor(orc, n, rng, mode=mode)
    g = rng.normal(0, 1e-3, n).astype(f32)
    w_fp = w.copy()
    st_fp = orc.init_state(n, True, mode)
    hp = orc.HParams(step=1, mode=mode)
    orc.step_tensor(w, g, st, hp, pos=0)
    orc.step_tensor(w_fp, g, st_fp, hp, pos=0)
    assert np.array_equal(w.view(np.uint32), w_fp.view(np.uint32))


@pytest.mark.parametrize("mode,prev", [(0, -1), (1, -1), (1, 0), (0, 1), (2, -1), (3, -1),
                                       (4, -1), (3, 1), (1, 4), (2, 0), (5, -1), (5, 1),
                                       (1, 5), (0, 5), (5, 2)])
def test_every_step_uses_decoded_state(orc, mode, prev):
    """Each step's weights = FP32 AdamW applied to decode(state) (decode -> update -> weights,
    [daiwk-PM] flowchart); the codebook for decoding is the one that encoded the state."""
    rng = np.random.default_rng(3)
    n = 4096 * 3 + 5
    w, st = _quant_tensor(orc, n, rng, mode=prev if prev >= 0 else mode)
    enc_mode = prev if prev >= 0 else mode
    for t in range(1, 5):
        g = rng.normal(0, 1e-3, n).astype(f32)
        hp = orc.HParams(step=t, mode=enc_mode)
        orc.step_tensor(w, g, st, hp, pos=1)
    g = rng.normal(0, 1e-3, n).astype(f32)
    m_dec, v_dec = orc.decode(st, n, enc_mode)
    w_ref = w.copy()
    fp = orc.State(False, m=m_dec, v=v_dec)
    hp = orc.HParams(step=5, mode=mode, prev_mode=prev)
    orc.step_tensor(w_ref, g, fp, hp, pos=1)
    orc.step_tensor(w, g, st, hp, pos=1)
    assert np.array_equal(w.view(np.uint32), w_ref.view(np.uint32))


# ---------------------------------------------------------------------------------------------
# P-4 / P-5  worked example and closed form for the zero cell
# ---------------------------------------------------------------------------------------------

def test_worked_example(orc):
    """[lav] worked example: eps = 1e-8, beta2 = 0.95, bias correction ignored, v = 1e-12 between
    levels 0 and 4e-12.  The page prints ~0.5% for ZIP-SR's probability of storing zero, 75% for
    state-space SR, next-step multipliers ~1.0M / 0.51M / 100M and expectations ~75M vs ~1.0M."""
    G = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    eps, b2, v, a, b = G["eps"], G["beta2"], G["v_true"], G["level_a"], G["level_b"]
    tol = G["rel_tol_about"]
    V0 = orc.codebook(orc.CB_V0)
    # a block whose scale puts the first positive level at 4e-12 (s = 15 * 4e-12)
    s = f32(b) / V0[1]
    c = float(np.sqrt(f32(s)))           # c = sqrt(s) * rs2 with rs2 = 1 (bc2 = 1)
    y = float(f32(v) * (f32(1) / f32(s)))
    p_zip = orc.zip_p(y, 0.0, float(V0[1]), c, eps)
    assert abs(p_zip - G["zip_sr_prob_zero"]) <= 0.05 * G["zip_sr_prob_zero"] * 2  # page: "about 0.5%"
    # exact value of the printed closed form eps(1 - sqrt(v/b))/(sqrt(v) + eps) = 0.0049505
    assert abs(p_zip - eps * (1 - np.sqrt(v / b)) / (np.sqrt(v) + eps)) < 1e-6
    p_state = (b - v) / (b - a)
    assert p_state == pytest.approx(G["state_sr_prob_zero"])
    # next-step multipliers with a zero gradient: v_next = beta2 * stored
    mult = lambda stored: 1.0 / (np.sqrt(b2 * stored) + eps)
    assert mult(v) == pytest.approx(G["next_multiplier_if_exact"], rel=tol)
    assert mult(b) == pytest.approx(G["next_multiplier_if_b"], rel=tol)
    assert mult(0.0) == pytest.approx(G["next_multiplier_if_zero"], rel=1e-12)
    e_state = p_state * mult(0.0) + (1 - p_state) * mult(b)
    e_zip = p_zip * mult(0.0) + (1 - p_zip) * mult(b)
    assert e_state == pytest.approx(G["state_sr_expected_next_multiplier"], rel=tol)
    assert e_state / mult(v) == pytest.approx(G["state_sr_overshoot_factor"], rel=tol)
    assert e_zip == pytest.approx(G["zip_sr_expected_next_multiplier"], rel=tol)


def test_worked_example_monte_carlo(orc):
    """The same block through the full ZIP-SR block encoder: the fraction of elements stored as
    zero is ~0.495% (binomial, 5 sigma) and the mean stored h matches h(v) at storage time."""
    V0 = orc.codebook(orc.CB_V0)
    s = f32(4e-12) / V0[1]
    x = np.full(128, 1e-12, f32)
    x[0] = s
    zeros = 0
    total = 0
    hsum = 0.0
    for seed in range(400):
        codes, scale, dbg = orc.encode_block(x, orc.RULE_V_ZIP, rs2=1.0, eps=1e-8, seed=seed, t=3)
        assert scale == s
        dec = V0[codes[1:]].astype(np.float64) * scale
        zeros += int((codes[1:] == 0).sum())
        total += 127
        hsum += h64(dec, 1.0, 1e-8).sum()
    p = 1e-8 * (1 - np.sqrt(1e-12 / 4e-12)) / (1e-6 + 1e-8)
    sigma = np.sqrt(total * p * (1 - p))
    assert abs(zeros - total * p) < 5 * sigma
    assert abs(hsum / total - h64(1e-12, 1.0, 1e-8)) < 5 * np.sqrt(p) * 1e8 / np.sqrt(total)


def test_state_sr_worked_example(orc):
    """The state-space SR rule of the controlled study on the worked example's block ([lav-RO],
    worked example): zero is stored with probability (b - v)/b = 75%; the block encoder's p
    matches it and the stored-zero frequency over seeds is 75% within 5 sigma; the mean stored v
    is v (the rule is unbiased in state space)."""
    G = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    V0 = orc.codebook(orc.CB_V0)
    s = f32(G["level_b"]) / V0[1]
    x = np.full(128, G["v_true"], f32)
    x[0] = s
    zeros = total = 0
    vsum = 0.0
    for seed in range(200):
        codes, scale, dbg = orc.encode_block(x, orc.RULE_V_SSR, seed=seed, t=5)
        assert scale == s and codes[0] == 15
        p = dbg[1:, 1]
        assert np.all(np.abs(p - G["state_sr_prob_zero"]) < 1e-6)
        zeros += int((codes[1:] == 0).sum())
        total += 127
        vsum += (V0[codes[1:]].astype(np.float64) * float(scale)).sum()
    p0 = G["state_sr_prob_zero"]
    assert abs(zeros - total * p0) < 5 * np.sqrt(total * p0 * (1 - p0))
    b = float(V0[1]) * float(s)
    assert abs(vsum / total - G["v_true"]) < 5 * b * np.sqrt(p0 * (1 - p0) / total)


def test_state_sr_unbiased_in_state_space(orc):
    """State-space SR on random blocks: over seeds the mean decoded v equals v for every element
    (5 sigma of the binomial spread of its own cell), the mirror image of ZIP-SR's exact mean h."""
    rng = np.random.default_rng(41)
    V0 = orc.codebook(orc.CB_V0).astype(np.float64)
    x = (10 ** rng.uniform(-9, -6, 128)).astype(f32)
    n = 600
    acc = np.zeros(128)
    for seed in range(n):
        codes, scale, _ = orc.encode_block(x, orc.RULE_V_SSR, seed=seed, t=2, pos=3)
        acc += V0[codes] * scale
    mean = acc / n
    s = float(x.max())
    y = x.astype(np.float64) / s
    k = np.clip(np.searchsorted(V0, y, side="right") - 1, 0, 14)
    width = (V0[k + 1] - V0[k]) * s
    assert np.all(np.abs(mean - x) <= 5 * width * 0.5 / np.sqrt(n) + 1e-6 * s)


def test_prtn_is_nearest_in_preconditioner_space(orc):
    """Preconditioner-space RTN picks the level whose h = 1/(sqrt(level/bc2) + eps) is nearest to
    h(v) among all 16 levels (brute force in binary64 over random blocks, scales and bias
    corrections); it can differ only where the binary64 distances tie to 1e-6 of h(a) - h(b).
    On the worked example it stores b, never zero."""
    rng = np.random.default_rng(42)
    V0 = orc.codebook(orc.CB_V0).astype(np.float64)
    checked = 0
    for _ in range(60):
        s = float(f32(10 ** rng.uniform(-14, -2)))
        bc2 = float(rng.choice([1e-3, 0.2, 1.0]))
        rs2 = float(f32(1 / np.sqrt(bc2)))
        eps = 1e-8
        x = (rng.uniform(0, 1, 128) ** 3 * s).astype(f32)
        x[0] = f32(s)
        codes, scale, dbg = orc.encode_block(x, orc.RULE_V_PRTN, rs2=rs2, eps=eps)
        h = lambda v: 1.0 / (np.sqrt(v) * rs2 + eps)
        lv = V0 * float(scale)
        for j in range(128):
            hv = h(float(x[j]))
            dist = np.abs(h(lv) - hv)
            best = int(np.argmin(dist))
            if codes[j] != best:
                k = min(int(codes[j]), best)
                span = h(lv[k]) - h(lv[k + 1])
                assert abs(dist[codes[j]] - dist[best]) <= 1e-6 * span, (j, codes[j], best)
            checked += 1
    assert checked == 60 * 128
    G = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    sb = f32(G["level_b"]) / f32(orc.codebook(orc.CB_V0)[1])
    xw = np.full(128, G["v_true"], f32)
    xw[0] = sb
    codes, _, dbg = orc.encode_block(xw, orc.RULE_V_PRTN, rs2=1.0, eps=G["eps"])
    assert np.all(codes[1:] == 1) and np.all(dbg[1:, 0] == 0.5)


@pytest.mark.parametrize("mode", [0, 2, 3, 4, 5])
def test_fp32_m_variant(orc, mode):
    """The controlled study's configuration ([lav-RO]: FP32 first moments, zero-inclusive v):
    over several steps m equals the FP32 AdamW recurrence bit for bit, v's codes and scales equal
    those of the fully quantized path from the same v state (the v side never reads m), and the
    weights equal FP32 AdamW applied to (m, decode(v))."""
    rng = np.random.default_rng(50 + mode)
    n = 4096 * 2 + 300
    w = rng.normal(0, 0.02, n).astype(f32)
    st = orc.init_state(n, False, mode, fp32_m=True)
    fp = orc.init_state(n, True, mode)            # FP32 reference for m
    wq = w.copy()
    q = orc.init_state(n, False, mode)            # fully quantized path, for v
    for t in range(1, 6):
        g = rng.normal(0, 1e-3, n).astype(f32)
        hp = orc.HParams(step=t, mode=mode, seed=9)
        m_dec, v_dec = orc.decode(st, n, mode)
        w_ref = w.copy()
        orc.step_tensor(w_ref, g, orc.State(False, m=m_dec, v=v_dec), hp, pos=2)
        q.vcodes[:], q.vscale[:] = st.vcodes, st.vscale
        orc.step_tensor(wq, g, q, hp, pos=2)
        orc.step_tensor(w, g, st, hp, pos=2)
        w_fp = w_ref.copy()
        orc.step_tensor(w_fp, g, fp, hp, pos=2)
        assert np.array_equal(st.m.view(np.uint32), fp.m.view(np.uint32))
        assert np.array_equal(st.vcodes, q.vcodes) and np.array_equal(st.vscale, q.vscale)
        assert np.array_equal(w.view(np.uint32), w_ref.view(np.uint32))
        fp.m[:] = st.m
        fp.v[:] = orc.decode(st, n, mode)[1]


def test_closed_form_zero_cell(orc):
    """For a = 0: p = eps (1 - sqrt(v/b)) / (sqrt(v/bc2) + eps) (the worked example's formula with
    bias correction restored per [daiwk-CE])."""
    rng = np.random.default_rng(4)
    V0 = orc.codebook(orc.CB_V0)
    for _ in range(3000):
        s = f32(10 ** rng.uniform(-30, 0))
        bc2 = float(rng.choice([1e-3, 0.05, 0.5, 1.0]))
        rs2 = f32(1 / np.sqrt(bc2))
        eps = 1e-8
        y = f32(rng.uniform(0, float(V0[1])))
        if y == 0:
            continue
        c = float(f32(np.sqrt(s)) * rs2)
        p = orc.zip_p(float(y), 0.0, float(V0[1]), c, eps)
        v = float(y) * float(s)
        b = float(V0[1]) * float(s)
        ref = eps * (1 - np.sqrt(v / b)) / (np.sqrt(v * float(rs2) ** 2) + eps)
        assert abs(p - ref) < 1e-6, (s, bc2, y, p, ref)


# ---------------------------------------------------------------------------------------------
# P-6 / P-10  ZIP-SR probability: printed formula, storage identity, endpoints, monotonicity
# ---------------------------------------------------------------------------------------------

def test_zip_p_equals_printed_formula(orc):
    """FP32 p (factored, normalised) vs the printed [h(v)-h(b)]/[h(a)-h(b)] in binary64, over all
    16-level cells, scales 1e-30..1 and bc2 in {1e-3, 0.5, 1}: |dp| <= 1e-6."""
    rng = np.random.default_rng(6)
    V0 = orc.codebook(orc.CB_V0)
    worst = 0.0
    for s in [1e-30, 1e-20, 1e-12, 1e-8, 1e-4, 1.0]:
        for bc2 in [1e-3, 0.5, 1.0]:
            rs2 = f32(1 / np.sqrt(bc2))
            c = float(f32(np.sqrt(f32(s))) * rs2)
            for k in range(15):
                lo, hi = float(V0[k]), float(V0[k + 1])
                for y in rng.uniform(lo, hi, 40).astype(f32):
                    if not (lo < y < hi):
                        continue
                    p = orc.zip_p(float(y), lo, hi, c, 1e-8)
                    sv = float(f32(s))
                    p64 = orc.zip_p64(float(y) * sv, lo * sv, hi * sv, 1.0 / float(rs2) ** 2, 1e-8)
                    worst = max(worst, abs(p - p64))
                    assert 0.0 <= p <= 1.0
    assert worst <= 1e-6, worst


def test_zip_storage_identity(orc):
    """ZIP-SR makes the expected multiplier exact at storage: p h(a) + (1-p) h(b) = h(v) ([lav-RO])."""
    rng = np.random.default_rng(7)
    V0 = orc.codebook(orc.CB_V0)
    for _ in range(2000):
        s = float(f32(10 ** rng.uniform(-16, -2)))
        bc2 = float(rng.choice([1e-2, 0.5, 1.0]))
        rs2 = f32(1 / np.sqrt(bc2))
        k = int(rng.integers(0, 15))
        y = f32(rng.uniform(float(V0[k]), float(V0[k + 1])))
        if not (V0[k] < y < V0[k + 1]):
            continue
        p = orc.zip_p(float(y), float(V0[k]), float(V0[k + 1]), float(f32(np.sqrt(f32(s))) * rs2), 1e-8)
        bc2r = 1.0 / float(rs2) ** 2
        ha, hb, hv = (h64(float(V0[k]) * s, bc2r, 1e-8), h64(float(V0[k + 1]) * s, bc2r, 1e-8),
                      h64(float(y) * s, bc2r, 1e-8))
        assert abs(p * ha + (1 - p) * hb - hv) <= 1e-6 * abs(ha - hb) + 1e-12 * hv


def test_zip_endpoints_and_monotone(orc):
    """p = 1 at the lower level, p -> 0 at the upper, p decreasing in between."""
    V0 = orc.codebook(orc.CB_V0)
    for k in range(15):
        lo, hi = float(V0[k]), float(V0[k + 1])
        c = 3e-5
        assert orc.zip_p(lo, lo, hi, c, 1e-8) == 1.0 if lo > 0 else True
        assert orc.zip_p(hi, lo, hi, c, 1e-8) == 0.0
        ys = np.linspace(lo, hi, 2001).astype(f32)
        ps = np.array([orc.zip_p(float(y), lo, hi, c, 1e-8) for y in ys])
        assert np.all(np.diff(ps) <= 1e-7)


def test_zip_zero_value_and_zero_block(orc):
    """v' = 0 is stored as the zero level; an all-zero block has scale 0 and zero codes (m: the
    NF4 zero, index 7)."""
    x = np.zeros(128, f32)
    x[5] = 1e-6
    codes, s, _ = orc.encode_block(x, orc.RULE_V_ZIP, rs2=1.0)
    assert s == f32(1e-6) and codes[5] == 15 and np.all(np.delete(codes, 5) == 0)
    for rule, zc in [(orc.RULE_M_RTN, 7), (orc.RULE_M_SR, 7), (orc.RULE_V_ZIP, 0),
                     (orc.RULE_V_EDEN, 0), (orc.RULE_V_RTN, 0), (orc.RULE_V_ZE_RTN, 0)]:
        codes, s, _ = orc.encode_block(np.zeros(128, f32), rule)
        assert s == 0.0 and np.all(codes == zc)


def test_zip_mc_preconditioner_unbiased(orc):
    """Monte-Carlo over seeds: the mean stored h equals h(v') ([lav-RO]: ZIP-SR makes the
    expected multiplier exact at storage).  Checked per element and pooled against the
    binomial variance p(1-p)(h(a)-h(b))^2 of each element, p from the oracle's own record."""
    V0 = orc.codebook(orc.CB_V0)
    rng = np.random.default_rng(8)
    for s, bc2 in [(3e-14, 1.0), (1e-15, 0.01), (2e-13, 0.5)]:
        s = f32(s)
        rs2 = f32(1 / np.sqrt(bc2))
        bc2r = 1.0 / float(rs2) ** 2
        x = (rng.random(128) * float(s)).astype(f32)
        x[0] = s
        nseed = 300
        hsum = np.zeros(128)
        var = np.zeros(128)
        for seed in range(nseed):
            codes, scale, dbg = orc.encode_block(x, orc.RULE_V_ZIP, rs2=float(rs2), eps=1e-8,
                                                 seed=seed, t=9)
            dec = V0[codes].astype(np.float64) * scale
            hsum += h64(dec, bc2r, 1e-8)
            p = np.where(dbg[:, 1] >= 0, dbg[:, 1], 0.0).astype(np.float64)
            y = (x * (f32(1) / s)).astype(np.float64)
            k = np.clip(np.floor(y * 15 + 1e-7).astype(int), 0, 14)
            ha = h64(V0[k].astype(np.float64) * float(s), bc2r, 1e-8)
            hb = h64(V0[k + 1].astype(np.float64) * float(s), bc2r, 1e-8)
            var += p * (1 - p) * (ha - hb) ** 2
        hv = h64(x.astype(np.float64), bc2r, 1e-8)
        mean = hsum / nseed
        sd = np.sqrt(var) / nseed
        assert np.all(np.abs(mean - hv) <= 5 * sd + 2e-6 * hv)
        z = (hsum.sum() - nseed * hv.sum()) / np.sqrt(var.sum())
        assert abs(z) < 5, z


def test_zip_state_space_biased_near_zero(orc):
    """Near zero, ZIP-SR rounds toward the positive level almost always, so the mean stored v
    exceeds the true v: it does not keep the state unbiased, state-space SR does ([lav-RO])."""
    V0 = orc.codebook(orc.CB_V0)
    rng = np.random.default_rng(18)
    s = f32(1.5e-10)
    x = (rng.uniform(0.05, 0.9, 128) * float(V0[1]) * float(s)).astype(f32)
    x[0] = s
    vs = []
    for seed in range(100):
        codes, scale, _ = orc.encode_block(x, orc.RULE_V_ZIP, rs2=1.0, eps=1e-8, seed=seed, t=9)
        vs.append(V0[codes[1:]].astype(np.float64) * scale)
    assert np.mean(vs) > 1.2 * x[1:].astype(np.float64).mean()


# ---------------------------------------------------------------------------------------------
# P-7  state-space SR for the LM-head m
# ---------------------------------------------------------------------------------------------

def test_m_sr_unbiased(orc):
    """Stochastic rounding between adjacent NF4 levels keeps the mean stored value exact
    ([lav-RO] on state-space SR; [lav-ZE] applies it to the LM head's m)."""
    nf4 = orc.codebook(orc.CB_NF4)
    rng = np.random.default_rng(9)
    x = rng.normal(0, 1e-3, 128).astype(f32)
    x[0] = f32(4e-3)
    acc = []
    for seed in range(600):
        codes, scale, dbg = orc.encode_block(x, orc.RULE_M_SR, seed=seed, t=190, pos=3)
        acc.append(nf4[codes].astype(np.float64) * scale)
    acc = np.array(acc)
    se = acc.std(0) / np.sqrt(acc.shape[0])
    ok = np.abs(acc.mean(0) - x) <= 5 * se + 2e-7 * np.abs(x) + 1e-12
    assert ok.sum() >= 127, np.nonzero(~ok)


def test_m_rtn_uses_no_randomness(orc):
    rng = np.random.default_rng(10)
    x = rng.normal(0, 1e-3, 128).astype(f32)
    c1, s1, d = orc.encode_block(x, orc.RULE_M_RTN, seed=1)
    c2, s2, _ = orc.encode_block(x, orc.RULE_M_RTN, seed=2)
    assert np.array_equal(c1, c2) and s1 == s2 and np.all(d[:, 3] == -1)


# ---------------------------------------------------------------------------------------------
# P-8  ZE-EDEN
# ---------------------------------------------------------------------------------------------

def test_eden_no_zero_and_scale_closed_form(orc):
    """ZE-EDEN uses a zero-free codebook ([kc-TC]) and rescales the block scale by
    gamma = |x|^2 / max(<x, Q(x)>, 1e-12 s^2) ([daiwk-CE]); recomputed in binary64 from the codes."""
    V1 = orc.codebook(orc.CB_V1)
    rng = np.random.default_rng(11)
    for trial in range(300):
        x = (10 ** rng.uniform(-20, -4, 128)).astype(f32)
        if trial % 3 == 0:
            x[rng.random(128) < 0.3] = 0
        codes, s2, _ = orc.encode_block(x, orc.RULE_V_EDEN)
        s = x.max()
        dec = V1[codes].astype(np.float64) * s2
        assert np.all(dec > 0)
        q = V1[codes].astype(np.float64) * float(s)          # Q(x) with the absmax scale
        xd = x.astype(np.float64)
        gamma = (xd @ xd) / max(xd @ q, 1e-12 * float(s) ** 2)
        # FP32 error budget: y = x*fl(1/s) (2u), y^2 or y*V1 (1u), 7 levels of pairwise sums of
        # positive terms (7u), so <= 12u per sum, then the division and the product (2u): 24u
        assert abs(s2 - gamma * float(s)) <= 24 * 2**-24 * gamma * float(s)
        assert xd @ q >= float(s) ** 2 * (1 - 1e-6)             # the max element maps to level 1


# ---------------------------------------------------------------------------------------------
# P-8b  the baseline: zero-free codebook, round to nearest, absmax scale, no rescale
# ---------------------------------------------------------------------------------------------

def test_baseline_is_eden_without_rescale(orc):
    """The baseline keeps the positive floor ([lav-ZE]: TorchAO's; [lav-ST]: its codebook's lowest
    level is positive), so no value of a non-zero block decodes to zero; it takes the
    same nearest V1 codes as ZE-EDEN ([kc-TC]: ZE-EDEN = zero removal + block rescale) and
    stores the plain absmax, which ZE-EDEN multiplies by gamma."""
    V1 = orc.codebook(orc.CB_V1)
    rng = np.random.default_rng(41)
    rescaled = 0
    for trial in range(200):
        x = (10 ** rng.uniform(-20, -4, 128)).astype(f32)
        if trial % 3 == 0:
            x[rng.random(128) < 0.4] = 0
        c_b, s_b, _ = orc.encode_block(x, orc.RULE_V_ZE_RTN)
        c_e, s_e, _ = orc.encode_block(x, orc.RULE_V_EDEN)
        assert np.array_equal(c_b, c_e)
        assert s_b == x.max()
        dec = V1[c_b] * s_b
        assert np.all(dec >= s_b / 16) and np.all(dec > 0)
        rescaled += int(s_e != s_b)
    assert rescaled > 150           # ZE-EDEN's gamma moves the scale; the baseline never does


def test_baseline_step_brute_force(orc):
    """A 3-element tensor (one block) stepped under the baseline, over every incoming v code:
    incoming v decodes with V1, and the new v codes are the nearest V1 level to v'/max v'
    (binary64 brute force), scale max v'."""
    V1 = orc.codebook(orc.CB_V1).astype(np.float64)
    n = 3
    hp = orc.HParams(step=6, mode=orc.V_ZE_RTN)
    for cv in range(16):
        for g1 in [0.0, 1e-3, -4e-4, 3e-5]:
            st = orc.State(True, np.array([0x77, 7], np.uint8),
                           np.array([cv | (3 << 4), 15], np.uint8),
                           np.array([1e-3], f32), np.array([1e-6], f32))
            w = np.array([0.01, -0.02, 0.03], f32)
            g = np.array([g1, -g1, 2e-3], f32)
            _, v_in = orc.decode(st, n, orc.V_ZE_RTN)
            assert v_in[0] == f32(V1[cv]) * f32(1e-6) and v_in[1] == f32(V1[3]) * f32(1e-6)
            orc.step_tensor(w, g, st, hp, pos=0, n=n)
            b2 = float(f32(hp.beta2))
            v64 = b2 * v_in.astype(np.float64) + (1 - b2) * g.astype(np.float64) ** 2
            assert abs(st.vscale[0] - v64.max()) <= 4 * 2**-24 * v64.max()
            for j in range(n):
                dd = np.abs(v64[j] / v64.max() - V1)
                cands = np.nonzero(dd <= dd.min() + 1e-6)[0]
                code = (st.vcodes[j >> 1] >> (4 * (j & 1))) & 15
                assert code in cands, (cv, g1, j, code, cands)
            assert st.vcodes[1] >> 4 == 0


# ---------------------------------------------------------------------------------------------
# P-9 / P-15  round-to-nearest vs brute force; tiny tensors enumerated
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("rule,cb", [(0, 0), (3, 2), (4, 1), (7, 2)])
def test_rtn_is_nearest_level(orc, rule, cb):
    """RTN = argmin over 16 levels |y - C[k]| (binary64); disagreement only where y sits within
    an ulp of a midpoint (the FP32 midpoint decides)."""
    C = orc.codebook(cb).astype(np.float64)
    rng = np.random.default_rng(12 + rule)
    for _ in range(40):
        x = rng.normal(0, 1, 128).astype(f32) if rule == 0 else rng.random(128).astype(f32) ** 3
        codes, scale, _ = orc.encode_block(x, rule)
        s = np.abs(x).max()  # codes are chosen on x / absmax (ZE-EDEN stores gamma * absmax)
        if rule != orc.RULE_V_EDEN:
            assert scale == s
        y = (x * (f32(1) / f32(s))).astype(np.float64)
        d = np.abs(y[:, None] - C[None, :])
        best = d.argmin(1)
        bad = np.nonzero(best != codes)[0]
        for j in bad:
            k0, k1 = sorted((int(best[j]), int(codes[j])))
            assert k1 - k0 == 1
            mid = 0.5 * (C[k0] + C[k1])
            assert abs(y[j] - mid) <= 2 * np.spacing(f32(mid))


def test_rtn_midpoint_ties_go_low(orc):
    """A value exactly on a midpoint keeps the lower code."""
    C = orc.codebook(orc.CB_NF4)
    x = np.zeros(128, f32)
    x[0] = 1.0
    for k in range(15):
        x[1 + k] = f32(0.5) * (C[k] + C[k + 1])
    codes, s, _ = orc.encode_block(x, orc.RULE_M_RTN)
    assert s == 1.0
    assert codes[1:16].tolist() == list(range(15))


def test_tiny_tensors_brute_force(orc):
    """Every (m code, v code) pair of a 2-element tensor whose block scales are fixed by a third
    element, times a grid of grads: decode, AdamW and re-encode recomputed independently here
    (binary64 AdamW, brute-force nearest NF4 level for m)."""
    nf4 = orc.codebook(orc.CB_NF4)
    V0 = orc.codebook(orc.CB_V0)
    n = 3
    hp = orc.HParams(step=4, mode=orc.ZIP_SR)
    sc = orc.step_scalars(hp)
    grads = [0.0, 1e-3, -2e-3, 5e-5]
    for cm in range(16):
        for cv in range(16):
            for g1 in grads:
                st = orc.State(True, np.array([cm | (cv << 4), 15 | (0 << 4)], np.uint8),
                               np.array([cv | (cm << 4), 15], np.uint8),
                               np.array([1e-3], f32), np.array([1e-6], f32))
                w = np.array([0.01, -0.02, 0.03], f32)
                g = np.array([g1, -g1, 2e-3], f32)
                w0 = w.copy()
                m_in, v_in = orc.decode(st, n, orc.ZIP_SR)
                assert m_in[0] == nf4[cm] * f32(1e-3) and v_in[1] == V0[cm] * f32(1e-6)
                orc.step_tensor(w, g, st, hp, pos=0, n=n)
                b1, b2 = float(f32(hp.beta1)), float(f32(hp.beta2))
                m64 = b1 * m_in.astype(np.float64) + (1 - b1) * g.astype(np.float64)
                v64 = b2 * v_in.astype(np.float64) + (1 - b2) * g.astype(np.float64) ** 2
                upd = float(f32(sc["step_size"])) * m64 / (np.sqrt(v64) * sc["rs2"] + 1e-8)
                w64 = w0.astype(np.float64) * sc["decay"] - upd
                assert np.all(np.abs(w - w64) <= 8 * 2**-24 * (np.abs(w0) + np.abs(upd)))
                # m codes: nearest NF4 level to m'/s_m (brute force), s_m = max |m'|
                m_new, _ = orc.decode(st, n, orc.ZIP_SR)
                sm = np.abs(m64).max()
                for j in range(n):
                    y = m64[j] / sm
                    dd = np.abs(y - nf4.astype(np.float64))
                    cands = np.nonzero(dd <= dd.min() + 1e-6)[0]
                    code = (st.mcodes[j >> 1] >> (4 * (j & 1))) & 15
                    assert code in cands, (cm, cv, g1, j, code, cands)
                # v scale = max v'; odd tail nibble of the last byte stays 0
                assert abs(st.vscale[0] - v64.max()) <= 4 * 2**-24 * v64.max()
                assert st.mcodes[1] >> 4 == 0 and st.vcodes[1] >> 4 == 0


# ---------------------------------------------------------------------------------------------
# P-16  BF16 copy of the updated weights
# ---------------------------------------------------------------------------------------------

def test_bf16_copy_matches_torch_rounding(orc):
    """Round to nearest even into BF16 equals torch's CPU conversion (an independent library
    routine) on every exponent, exact ties with even and odd kept halves, the values next to
    ties, subnormals, signed zeros and the overflow edge; plus 2^20 random bit patterns."""
    import torch
    rng = np.random.default_rng(61)
    hi = np.arange(0, 0x7F80, dtype=np.uint32)            # every finite non-negative BF16 word
    low = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF], np.uint32)
    bits = (hi[:, None] << 16 | low[None, :]).ravel()
    bits = np.concatenate([bits, bits | 0x80000000,
                           rng.integers(0, 0x7F800000, 1 << 20, dtype=np.uint32),
                           np.array([0x7F7FFFFF, 0x7F7F7FFF, 0x7F7F8000, 0xFF7F8000], np.uint32)])
    x = bits.view(f32)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = orc.bf16_rne(x)
    assert np.array_equal(got, ref)
    # spot values: 1 + 2^-8 is a tie with an even kept half (stays 1.0), 1 + 3 * 2^-8 a tie with
    # an odd one (goes up); the largest float rounds to +inf
    spot = np.array([1 + 2**-8, 1 + 3 * 2**-8, 3.4028235e38], f32)
    assert orc.bf16_rne(spot).tolist() == [0x3F80, 0x3F82, 0x7F80]


# ---------------------------------------------------------------------------------------------
# P-11  storage accounting
# ---------------------------------------------------------------------------------------------

def test_state_bytes_match_pages(orc):
    """1.0625 B/param for 4-bit m and v with one FP32 scale per 128 values each, 8 B/param
    FP32, 7.53x ([lav-ST]); the A100 table's 1,095,680 vs 157,952 bytes ([daiwk-LR])."""
    G = json.load(open(os.path.join(GOLDEN, "a100_state_bytes.json")))
    sizes = [4096] * 33 + [256] * 7   # 135,168 quantized + 1,792 fallback elements
    fp32 = 0
    quant = 0
    for n in sizes:
        st = orc.init_state(n, False, orc.ZIP_SR)
        fp32 += 8 * n
        if st.quantized:
            quant += st.mcodes.nbytes + st.vcodes.nbytes + st.mscale.nbytes + st.vscale.nbytes
        else:
            quant += st.m.nbytes + st.v.nbytes
    assert fp32 == G["fp32_adamw_moment_bytes"]
    assert quant == G["zip_sr_moment_bytes"] == G["ze_eden_moment_bytes"]
    assert round(100 * (1 - quant / fp32), 1) == G["state_savings_percent_about"]
    assert (2 * 0.5 + 2 * 4 / 128) == G["bytes_per_param_4bit"]
    assert round(G["bytes_per_param_fp32"] / G["bytes_per_param_4bit"], 2) == G["reduction_about"]


def test_fallback_boundary(orc):
    """Tensors below the pages' 4096-element boundary keep FP32 moments, 4096 and above are
    quantized, and a normalization layer keeps FP32 moments at any size ([daiwk-LR] results
    table and the line after it, [lav-ST])."""
    G = json.load(open(os.path.join(GOLDEN, "a100_state_bytes.json")))
    edge = G["fallback_below_elements"]
    for n in (1, 255, edge - 1):
        st = orc.init_state(n, False, orc.ZIP_SR)
        assert not st.quantized and st.m.nbytes + st.v.nbytes == G["bytes_per_param_fp32"] * n, n
    for n in (edge, edge + 1, 5 * edge):
        st = orc.init_state(n, False, orc.ZIP_SR)
        assert st.quantized, n
        nbytes = st.mcodes.nbytes + st.vcodes.nbytes + st.mscale.nbytes + st.vscale.nbytes
        assert nbytes == 2 * ((n + 1) // 2) + 2 * 4 * ((n + 127) // 128), n
    st = orc.init_state(5 * edge, True, orc.ZIP_SR)
    assert not st.quantized


# ---------------------------------------------------------------------------------------------
# P-14  determinism: thread count, sub-range replay
# ---------------------------------------------------------------------------------------------

def _run_threads(nthreads):
    code = r"""
import sys, numpy as np
sys.path.insert(0, %r)
import oracle
rng = np.random.default_rng(13)
n = 128 * 300 + 17
w = rng.normal(0, 0.02, n).astype(np.float32)
st = oracle.init_state(n, False, oracle.ZIP_SR)
for t in range(1, 4):
    g = rng.normal(0, 1e-3, n).astype(np.float32)
    oracle.step_tensor(w, g, st, oracle.HParams(step=t, seed=77, sr_head=1), pos=2, head=True)
sys.stdout.buffer.write(w.tobytes() + st.mcodes.tobytes() + st.vcodes.tobytes() +
                        st.mscale.tobytes() + st.vscale.tobytes())
""" % os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, OMP_NUM_THREADS=str(nthreads))
    return subprocess.run([sys.executable, "-c", code], env=env, capture_output=True,
                          check=True).stdout


def test_thread_count_invariance(orc):
    assert _run_threads(1) == _run_threads(8)


def test_subrange_replay_matches_full(orc):
    """Blocks are independent and the RNG is counter-based, so stepping a sub-range of blocks
    (the parity protocol's sampled replay) reproduces the full-tensor step on that range."""
    rng = np.random.default_rng(14)
    n = 128 * 40 + 33
    w = rng.normal(0, 0.02, n).astype(f32)
    st = orc.init_state(n, False, orc.ZIP_SR)
    for t in range(1, 3):
        orc.step_tensor(w, rng.normal(0, 1e-3, n).astype(f32), st, orc.HParams(step=t), pos=4)
    g = rng.normal(0, 1e-3, n).astype(f32)
    hp = orc.HParams(step=3, seed=5)
    w_full, st_full = w.copy(), st.copy()
    orc.step_tensor(w_full, g, st_full, hp, pos=4)
    for b0, nb in [(0, 1), (7, 5), (39, 2), (40, 1)]:
        e0, e1 = 128 * b0, min(n, 128 * (b0 + nb))
        sub = orc.State(True, st.mcodes[e0 // 2:(e1 + 1) // 2].copy(),
                        st.vcodes[e0 // 2:(e1 + 1) // 2].copy(),
                        st.mscale[b0:b0 + nb].copy(), st.vscale[b0:b0 + nb].copy())
        ws = w[e0:e1].copy()
        orc.step_tensor(ws, g[e0:e1].copy(), sub, hp, pos=4, e0=e0, n=n)
        assert np.array_equal(ws, w_full[e0:e1])
        assert np.array_equal(sub.mcodes, st_full.mcodes[e0 // 2:(e1 + 1) // 2])
        assert np.array_equal(sub.vcodes, st_full.vcodes[e0 // 2:(e1 + 1) // 2])
        assert np.array_equal(sub.vscale, st_full.vscale[b0:b0 + nb])


def test_bf16_grads_widen_exactly(orc):
    """BF16 grads are widened exactly (bits << 16): same result as passing the FP32 value."""
    rng = np.random.default_rng(15)
    n = 4096 + 128
    g32 = rng.normal(0, 1e-3, n).astype(f32)
    gbf = (g32.view(np.uint32) >> 16).astype(np.uint16)
    gw = (gbf.astype(np.uint32) << 16).view(f32)
    w = rng.normal(0, 0.02, n).astype(f32)
    sa, sb = orc.init_state(n, False, 0), orc.init_state(n, False, 0)
    wa, wb = w.copy(), w.copy()
    orc.step_tensor(wa, gbf, sa, orc.HParams(step=1), pos=0)
    orc.step_tensor(wb, gw, sb, orc.HParams(step=1), pos=0)
    assert np.array_equal(wa, wb) and np.array_equal(sa.vcodes, sb.vcodes)


# ---------------------------------------------------------------------------------------------
# P-16  the initial-state encoder (no page defines one; the reading is a deterministic nearest
# level with the pages' block format, plus ZE-EDEN's rescale): each block recomputed here by
# brute force over the 16 levels and the rescale's closed form in binary64
# ---------------------------------------------------------------------------------------------

def _unpack(codes, n):
    return np.stack([codes & 15, codes >> 4], 1).reshape(-1)[:n]


def _init_inputs(seed, n):
    """m0 ~ N(0, 1e-3) with 10% exact zeros and one all-zero block; v0 log-uniform in
    [1e-20, 1e-4] (the pre-seeded v of the 834M list) with its own all-zero block; the last block
    is partial."""
    rng = np.random.default_rng(seed)
    m0 = rng.normal(0, 1e-3, n).astype(f32)
    m0[rng.random(n) < 0.1] = 0
    m0[128:256] = 0
    v0 = (10 ** rng.uniform(-20, -4, n)).astype(f32)
    v0[256:384] = 0
    v0[rng.random(n) < 0.05] = 0
    return m0, v0


def _nearest_low(y, C):
    """Index of the nearest level, a tie going to the lower one (argmin keeps the first)."""
    return np.abs(y.astype(np.float64)[:, None] - C.astype(np.float64)[None, :]).argmin(1)


def _check_near(codes, y, C, what):
    """codes equal the binary64 nearest level, except where y lies within two FP32 ulps of a
    midpoint (the encoder's own FP32 midpoint then decides), which must be rare."""
    best = _nearest_low(y, C)
    bad = np.nonzero(best != codes)[0]
    for j in bad:
        k0, k1 = sorted((int(best[j]), int(codes[j])))
        assert k1 - k0 == 1, (what, j)
        mid = 0.5 * (float(C[k0]) + float(C[k1]))
        assert abs(float(y[j]) - mid) <= 2 * np.spacing(f32(mid)), (what, j, y[j], mid)
    assert bad.size <= 2, (what, bad.size)


@pytest.mark.parametrize("mode", [0, 1, 2, 3, 4, 5])
def test_init_encoder_brute_force(orc, mode):
    """Initial states from given moments: per 128-value block (zero-padded), the m scale is
    max|m0| ([lav-ST]: one FP32 scale per 128 values) and each m code the nearest NF4 level of
    m0/scale; the v scale is max v0 and each v code the nearest level of the mode's codebook
    (zero-free V1 for ZE-EDEN and the baseline, V0 otherwise); ZE-EDEN then multiplies the v
    scale by gamma = |y|^2 / max(<y, V1[c]>, 1e-12) ([daiwk-CE]).  All-zero blocks store code 7
    (NF4's zero) / code 0 with scale 0."""
    n = 128 * 40 + 45
    m0, v0 = _init_inputs(70 + mode, n)
    st = orc.init_state(n, False, mode, m0, v0)
    NF4 = orc.codebook(orc.CB_NF4)
    V = orc.codebook(orc.CB_V1 if mode in (orc.ZE_EDEN, orc.V_ZE_RTN) else orc.CB_V0)
    mc, vc = _unpack(st.mcodes, n), _unpack(st.vcodes, n)
    for b in range((n + 127) // 128):
        lo, hi = 128 * b, min(n, 128 * b + 128)
        xm, xv = m0[lo:hi], v0[lo:hi]
        sm, sv = np.abs(xm).max(), xv.max()
        assert st.mscale[b] == sm
        if sm == 0:
            assert np.all(mc[lo:hi] == 7)
        else:
            _check_near(mc[lo:hi], xm * (f32(1) / sm), NF4, ("m", b))
        if sv == 0:
            assert np.all(vc[lo:hi] == 0) and st.vscale[b] == 0
            continue
        y = xv * (f32(1) / sv)
        _check_near(vc[lo:hi], y, V, ("v", b))
        if mode == orc.ZE_EDEN:
            yd = y.astype(np.float64)
            q = V[vc[lo:hi]].astype(np.float64)
            gamma = (yd @ yd) / max(yd @ q, 1e-12)
            assert abs(st.vscale[b] - gamma * float(sv)) <= 24 * 2**-24 * gamma * float(sv), b
            assert yd @ q >= 1 - 1e-6       # the block's maximum maps to the top level
        else:
            assert st.vscale[b] == sv
        if mode in (orc.ZE_EDEN, orc.V_ZE_RTN):
            assert np.all(V[vc[lo:hi]] * st.vscale[b] > 0)   # no decoded zero
    # the pad nibble of the odd last byte is zero
    assert st.mcodes[-1] >> 4 == 0 and st.vcodes[-1] >> 4 == 0


def test_init_encoder_uses_no_randomness(orc):
    """No step t exists before the first step, so the initial encoding is deterministic: it is
    the same whatever the mode's RNG would draw, and a tie between two levels goes low."""
    NF4 = orc.codebook(orc.CB_NF4)
    V0 = orc.codebook(orc.CB_V0)
    n = 4096
    m0 = np.zeros(n, f32)
    v0 = np.zeros(n, f32)
    m0[0], v0[0] = 1.0, 1.0
    for k in range(15):   # exact FP32 midpoints of adjacent levels
        m0[1 + k] = f32(0.5) * (NF4[k] + NF4[k + 1])
        v0[1 + k] = f32(0.5) * (V0[k] + V0[k + 1])
    a = orc.init_state(n, False, orc.ZIP_SR, m0, v0)
    b = orc.init_state(n, False, orc.V_SSR, m0, v0)
    assert np.array_equal(a.mcodes, b.mcodes) and np.array_equal(a.vcodes, b.vcodes)
    assert _unpack(a.mcodes, n)[1:16].tolist() == list(range(15))
    assert _unpack(a.vcodes, n)[1:16].tolist() == list(range(15))


@pytest.mark.parametrize("mode", [0, 1, 5])
def test_init_encoder_fp32_m(orc, mode):
    """A tensor with FP32 first moments ([lav-RO]) stores m0 bit for bit and encodes v exactly as
    the fully quantized tensor does."""
    n = 128 * 40 + 9
    m0, v0 = _init_inputs(90 + mode, n)
    st = orc.init_state(n, False, mode, m0, v0, fp32_m=True)
    full = orc.init_state(n, False, mode, m0, v0)
    assert st.fp32_m and np.array_equal(st.m.view(np.uint32), m0.view(np.uint32))
    assert np.array_equal(st.vcodes, full.vcodes) and np.array_equal(st.vscale, full.vscale)
    m_dec, _ = orc.decode(st, n, mode)
    assert np.array_equal(m_dec.view(np.uint32), m0.view(np.uint32))
