"""Host-side logic of the torch Optimizer front end (no GPU needed): encoder names, the
LM-head switch over the last tenth of training, and argument checks that refuse CPU tensors
(there is no CPU path)."""
import pytest
import torch

from bit_adamw_step_amd import optim


def test_mode_names():
    assert [optim.mode_id(k) for k in ("zip-sr", "ze-eden", "state-rtn", "state-sr",
                                       "precond-rtn", "baseline")] == [0, 1, 2, 3, 4, 5]
    assert optim.mode_id(1) == 1
    with pytest.raises(ValueError):
        optim.mode_id("adamw")
    with pytest.raises(ValueError):
        optim.mode_id(9)


def test_lm_head_switch_last_tenth():
    """learnaivisually.com ZE-EDEN / LM-head paragraph: stochastic rounding over the final 10%:
    on for 10 t > 9 T, i.e. t = 181..200 of 200; never without a planned length."""
    on = [t for t in range(1, 201) if optim.sr_head_at(t, 200)]
    assert on == list(range(181, 201))
    assert optim.sr_head_at(10 ** 6, None) == 0
    assert [t for t in range(1, 11) if optim.sr_head_at(t, 10)] == [10]


def test_refuses_cpu_and_bad_dtypes():
    with pytest.raises(ValueError, match="CUDA"):
        optim.AdamW4bit([torch.zeros(8)])
    with pytest.raises(ValueError, match="unknown v encoder"):
        optim.AdamW4bit([{"params": [], "mode": "nope"}])
