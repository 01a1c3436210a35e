"""The CPU oracle against its pins (no GPU)."""
import numpy as np
import pytest

import pins
import pins_landing
import pins_stage


@pytest.mark.parametrize("pin", pins.ALL_PINS + pins_landing.ALL_PINS + pins_stage.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_layout_matches_workload_table(orc):
    """Per-rank packed sizes and byte counts of the five workloads (values
    computed by hand from the shapes: S = sum ceil(T_p/N) * K_p)."""
    from workloads.configs import CONFIGS
    want_S = {"worked_example": 24, "llama70b_layer": 13_369_600,
              "qwen3_moe_layer": 9_736_256, "padding_stress": 41_196_789,
              "wan22_dit_block": 5_493_920}
    for name, cfg in CONFIGS.items():
        assert orc.layout(cfg.shapes, cfg.N)["S"] == want_S[name], name
    # Llama by hand: q,o: 128*8192; k,v: 16*8192; gate,up: 448*8192;
    # down: 128*28672; norms: 128 each.
    assert 2 * 128 * 8192 + 2 * 16 * 8192 + 2 * 448 * 8192 + 128 * 28672 + 2 * 128 == 13_369_600


def test_rejects_invalid(orc):
    with pytest.raises(ValueError):
        orc.layout([(4, 0)], 2)
    with pytest.raises(ValueError):
        orc.layout([(-1, 3)], 2)
    with pytest.raises(ValueError):
        orc.layout([(4, 3)], 0)
    with pytest.raises(ValueError):
        orc.reduce_scatter([(4, 3)], 2, 1, [[np.zeros(12, np.uint16)]], out_stride=5)


def test_empty_and_zero_row_params(orc):
    # An empty group, and a group with a zero-row parameter, are valid.
    assert orc.layout([], 4)["S"] == 0
    shapes = [(0, 5), (3, 2)]
    lay = orc.layout(shapes, 2)
    assert list(lay["s"]) == [0, 4] and lay["S"] == 4
    g = [[np.zeros(0, np.uint16), np.arange(6, dtype=np.uint16) + 0x3F80] for _ in range(2)]
    out = orc.reduce_scatter(shapes, 2, 2, g)
    assert out.shape == (2, 4)
