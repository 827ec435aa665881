"""Pins for the oracle's gated activations.

Source: "kimi-k3-in-c" README §9 (k3_situ_glu: SiTU-GLU with betas 4 and 25,
the sigmoid on the raw gate, the bound b1*b2 = 100)."""
import json
import math
import os

import numpy as np
import torch

import oracle
from conftest import GOLDEN

CFG = json.load(open(os.path.join(GOLDEN, "layer_config.json")))
B1, B2 = CFG["situ_b1"], CFG["situ_b2"]


def silu_glu(g, u):
    """Library reference: torch's SiLU (g * sigmoid(g)) times u, in fp64."""
    return float(torch.nn.functional.silu(torch.tensor(g, dtype=torch.float64)) * u)


def test_zero_gate_or_up_gives_zero():
    for v in (-1000.0, -3.0, -0.1, 0.0, 0.1, 3.0, 1000.0):
        assert oracle.act(0.0, v, oracle.ACT_SITU, B1, B2) == 0.0
        assert oracle.act(v, 0.0, oracle.ACT_SITU, B1, B2) == 0.0


def test_bound_and_saturation():
    vals = np.concatenate([np.geomspace(0.1, 1000.0, 41), -np.geomspace(0.1, 1000.0, 41)])
    worst = 0.0
    for g in vals:
        for u in vals:
            worst = max(worst, abs(oracle.act(g, u, oracle.ACT_SITU, B1, B2)))
    assert worst <= B1 * B2 == CFG["situ_bound"]
    # saturated gate and up reach the analytic cap exactly
    assert oracle.act(200.0, 1000.0, oracle.ACT_SITU, B1, B2) == CFG["situ_bound"]
    # the sigmoid reads the raw gate: a very negative gate switches the unit off.
    # (A capped sigmoid would see -4 here and give about -1.8.)
    assert abs(oracle.act(-200.0, 1000.0, oracle.ACT_SITU, B1, B2)) < 1e-80


def test_raw_gate_sigmoid_distinguishes_capping():
    # at g = 40 the cap makes b1*tanh(g/b1) ~ 4 while sigmoid(40) = 1 to 1e-17;
    # a capped sigmoid would give sigmoid(4) = 0.982
    r = oracle.act(40.0, 1000.0, oracle.ACT_SITU, B1, B2) / (B1 * B2)
    assert abs(r - 1.0) < 1e-8


def test_odd_in_up():
    for g in (-7.0, -0.3, 0.2, 5.0, 60.0):
        for u in (0.01, 0.7, 9.0, 300.0):
            a = oracle.act(g, u, oracle.ACT_SITU, B1, B2)
            assert oracle.act(g, -u, oracle.ACT_SITU, B1, B2) == -a


def test_large_betas_reduce_to_silu_glu():
    # b*tanh(v/b) -> v as b grows, so SiTU-GLU tends to SiLU(g)*u
    for g in (-6.0, -1.0, -0.2, 0.0, 0.4, 2.0, 7.5):
        for u in (-3.0, 0.5, 2.0):
            got = oracle.act(g, u, oracle.ACT_SITU, 1e7, 1e7)
            ref = silu_glu(g, u)
            assert abs(got - ref) <= 1e-9 * max(1.0, abs(ref))


def test_swiglu_kind_is_silu_glu():
    for g in (-30.0, -6.0, -1.0, 0.0, 0.4, 2.0, 7.5, 30.0):
        for u in (-3.0, 0.5, 200.0):
            got = oracle.act(g, u, oracle.ACT_SWIGLU)
            ref = silu_glu(g, u)
            assert abs(got - ref) <= 1e-14 * max(1.0, abs(ref))


def test_swiglu_closed_forms():
    # sigmoid(ln 3) = 3/4 and sigmoid(-ln 3) = 1/4 exactly, so
    # g * sigmoid(g) * u is known in closed form there; g = 0 or u = 0 give 0;
    # a large gate passes g * u, a very negative one gives 0
    l3 = math.log(3.0)
    for u in (-2.0, 0.5, 3.0):
        assert abs(oracle.act(l3, u, oracle.ACT_SWIGLU) - 0.75 * l3 * u) <= 1e-15 * abs(u) * 2
        assert abs(oracle.act(-l3, u, oracle.ACT_SWIGLU) - (-0.25 * l3 * u)) <= 1e-15 * abs(u) * 2
        assert oracle.act(0.0, u, oracle.ACT_SWIGLU) == 0.0
        assert abs(oracle.act(60.0, u, oracle.ACT_SWIGLU) - 60.0 * u) <= 1e-12 * abs(60.0 * u)
        assert abs(oracle.act(-60.0, u, oracle.ACT_SWIGLU)) <= 60.0 * abs(u) * math.exp(-60.0)  # sigmoid(-60) < e^-60
    assert oracle.act(1.3, 0.0, oracle.ACT_SWIGLU) == 0.0


def test_raw_gate_sigmoid_worked_value():
    # g = 8, u = 25: 4 tanh(2) = 3.856110, sigmoid(8) = 0.999665,
    # 25 tanh(1) = 19.039854, so the unit gives 73.3952 (73.39 to two
    # places, truncated). Feeding the sigmoid the capped gate instead
    # (sigmoid(3.856110) = 0.979332) would give 71.8991: the README's
    # warning that the sigmoid takes the uncapped gate (§9, k3_situ_glu).
    v = oracle.act(8.0, 25.0, oracle.ACT_SITU, B1, B2)
    assert abs(v - 73.3952) < 1e-4
    assert abs(v - 71.8991) > 1.4
    # and the sign follows the up half
    assert abs(oracle.act(8.0, -25.0, oracle.ACT_SITU, B1, B2) + 73.3952) < 1e-4
