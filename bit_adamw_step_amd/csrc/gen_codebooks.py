"""Print the 16-word FP32 codebooks compiled into the HIP library (as hex-float literals).

NF4 (QLoRA's normal-quantile 4-bit type, named for m on the kongchang.com explainer's
"Two Complementary Technical Approaches" section): 8 positive levels are normal quantiles of
8 evenly spaced probabilities from delta = 1 - (1/30 + 1/32)/2 towards 1/2, 7 negative levels
the mirrored quantiles of 7 such probabilities, plus 0, all divided by the largest.
V0 = k/15 (zero kept, ZIP-SR) and V1 = (k+1)/16 (positive floor, ZE-EDEN).

Run: python gen_codebooks.py  -> paste into adamw4_kernels.hip.
"""
import numpy as np
from scipy.stats import norm


def nf4():
    d = 1.0 - 0.5 * (1.0 / 30.0 + 1.0 / 32.0)
    pos = norm.ppf(np.linspace(d, 0.5, 9)[:-1])
    neg = -norm.ppf(np.linspace(d, 0.5, 8)[:-1])
    return (np.sort(np.concatenate([pos, neg, [0.0]])) / norm.ppf(d)).astype(np.float32)


def v0():
    return np.array([np.float32(k / 15.0) for k in range(16)], np.float32)


def v1():
    return np.array([(k + 1) / 16.0 for k in range(16)], np.float32)


def fmt(name, arr):
    words = ", ".join(float(x).hex() + "f" if x != 0 else "0.0f" for x in arr)
    return f"{name} = {{{words}}};"


if __name__ == "__main__":
    for n, a in (("NF4", nf4()), ("V0", v0()), ("V1", v1())):
        print(fmt(n, a))
