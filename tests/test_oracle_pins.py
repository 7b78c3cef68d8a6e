"""The CPU oracle against its pins (closed forms, special cases, exact brute force,
invariants, library conversions). No GPU needed."""
import json
import os

import numpy as np
import pytest

import pins

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_page_example_shapes(orc):
    """The page's own example (the "Qwen3.5-2B decode configuration") fixes only shapes."""
    with open(os.path.join(HERE, "golden", "page_example_shapes.json")) as f:
        gold = json.load(f)
    B, H, T, Dk, Dv = (gold["inputs"][k] for k in ("B", "H", "T", "Dk", "Dv"))
    rng = np.random.default_rng(0)
    c = pins.f64_case(rng, B, H, H, T, Dk, Dv, B, idx=[0], zero_state=True)
    out, pool = pins.call_f64(orc, c)
    assert list(out.shape) == gold["out_shape"]
    assert list(pool.shape) == gold["state_out_shape"]
