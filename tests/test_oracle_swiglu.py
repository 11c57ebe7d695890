"""Pins for the oracle's SwiGLU and float64 -> bf16 rounding (the harness
activation between the two forward GEMMs; not on the pages).

round_bf16 is checked against torch's float32 -> bfloat16 conversion on
float32-representable values (a library routine taking another route), on
hand-worked ties and on the subnormal / overflow ends.  swiglu is checked on
closed forms of silu.
"""
import math

import numpy as np
import torch

from workloads import f32_to_bf16_bits, rng_for


def _torch_bf16_bits(x32):
    return torch.from_numpy(np.asarray(x32, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_round_bf16_matches_torch_on_float32_values(orc):
    rng = rng_for(0, salt=91)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(3.0),
        (rng.standard_normal(5000) * 1e-39).astype(np.float32),   # float32 subnormals
        (rng.standard_normal(5000) * 1e30).astype(np.float32),
    ])
    assert np.array_equal(orc.round_bf16(x.astype(np.float64)), _torch_bf16_bits(x))


def test_round_bf16_hand_ties():
    import oracle as orc
    ulp = 2.0 ** -7
    cases = {
        1.0 + ulp / 2: 0x3F80,            # tie, even neighbour 1.0
        1.0 + 3 * ulp / 2: 0x3F82,        # tie between 1+ulp (odd) and 1+2ulp (even)
        1.0 + ulp / 2 + 2.0 ** -40: 0x3F81,  # just above the tie (not float32-representable)
        -(1.0 + ulp / 2 - 2.0 ** -40): 0xBF80,
        2.0 ** -133: 0x0001,              # smallest bf16 subnormal
        2.0 ** -134: 0x0000,              # tie with zero, rounds to even (0)
        3 * 2.0 ** -134: 0x0002,          # tie between 1 and 2 quanta -> 2
        3.3895313892515355e38: 0x7F7F,    # largest finite bf16
        2.0 ** 128: 0x7F80,
        0.0: 0x0000,
    }
    for v, bits in cases.items():
        assert int(orc.round_bf16(np.array([v]))[0]) == bits, (v, hex(bits))
    assert int(orc.round_bf16(np.array([-0.0]))[0]) == 0x8000


def test_swiglu_closed_forms(orc):
    g = np.array([0.0, math.log(3.0), -math.log(3.0), 30.0, -30.0, 2.5])
    u = np.array([5.0, 1.0, 1.0, 1.0, 1.0, -2.0])
    h = orc.swiglu(np.concatenate([g, u])[None, :])[0]
    assert h[0] == 0.0
    assert math.isclose(h[1], 0.75 * math.log(3.0), rel_tol=1e-15)   # sigmoid(ln 3) = 3/4
    assert math.isclose(h[2], -0.25 * math.log(3.0), rel_tol=1e-15)  # sigmoid(-ln 3) = 1/4
    assert math.isclose(h[3], 30.0, rel_tol=1e-12)
    assert abs(h[4]) < 1e-11
    # very negative gates: g e^g, no overflow to g / inf
    t = orc.swiglu(np.array([[-50.0, -800.0, 1.0, 1.0]]))[0]
    assert math.isclose(t[0], -50.0 * math.exp(-50.0) / (1 + math.exp(-50.0)), rel_tol=1e-14)
    assert t[1] == 0.0 and math.copysign(1.0, t[1]) == -1.0
    # silu(x) - silu(-x) = x
    assert math.isclose(h[5] / -2.0 - orc.swiglu(np.array([[-2.5, 1.0]]))[0, 0], 2.5, rel_tol=1e-15)


def test_swiglu_bf16_splits_gate_and_up(orc):
    rng = rng_for(1, salt=92)
    gu32 = rng.standard_normal((6, 64)).astype(np.float32)
    gu = f32_to_bf16_bits(gu32)
    f = (gu.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    g, u = f[:, :32], f[:, 32:]
    ref = orc.round_bf16(g * u / (1.0 + np.exp(-g)))
    assert np.array_equal(orc.swiglu_bf16(gu), ref)
