"""The CPU oracle against its pins, and the pins against planted mistakes.

Both accumulation precisions are pinned: fp32 (the default, the contract's
fp32 accumulation) and fp64 (nearly exact)."""
import os

import pytest

import oracle_pins
from oracle import build as oracle_build
from oracle.oracle import load

PLANTS = ["DROP_PEER", "SKIP_LAST_K", "SLICE_FLOOR", "ROUND_TRUNC", "AG_LOCAL_ONLY",
          "B_TRANSPOSED", "WS_ALL_ROWS", "ACC32_IN_DOUBLE", "K_DESCENDING", "PEERS_FIRST"]


@pytest.fixture(scope="module")
def orc():
    return load()


@pytest.mark.parametrize("acc", ["fp32", "fp64"])
@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin, acc):
    pin(load(acc=acc))


def test_default_precision_is_fp32():
    assert load().acc == "fp32"


@pytest.mark.parametrize("plant", PLANTS)
def test_pins_catch_planted_mistake(plant, tmp_path):
    lib = oracle_build.build(str(tmp_path / f"liboracle_{plant}.so"),
                             defines=(f"ORACLE_PLANT_{plant}",))
    caught = []
    for acc in ("fp32", "fp64"):
        bad = load(lib, acc=acc)
        for pin in oracle_pins.ALL_PINS:
            try:
                pin(bad)
            except AssertionError:
                caught.append(f"{pin.__name__}[{acc}]")
    assert caught, f"no pin catches the planted mistake {plant}"
    if plant in ("ACC32_IN_DOUBLE", "K_DESCENDING", "PEERS_FIRST"):
        # mistakes that only change roundings must be caught on the fp32 oracle
        assert any(c.endswith("[fp32]") for c in caught), (plant, caught)


def test_oracle_thread_count_independent(orc):
    """Rows are split whole over threads: one thread and many give the same bits."""
    import subprocess
    import sys
    code = (
        "import numpy as np, sys; sys.path.insert(0, %r);"
        "from oracle.oracle import load; o = load();"
        "rng = np.random.default_rng(0);"
        "A = rng.integers(0, 0x3f00, (64, 256)).astype(np.uint16);"
        "B = rng.integers(0, 0x3f00, (256, 96)).astype(np.uint16);"
        "P = rng.integers(0, 0x3f00, (3, 64, 96)).astype(np.uint16);"
        "sys.stdout.write(o.gemm_ar(A, B, P, 4).tobytes().hex())"
    ) % os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    outs = []
    for n in ("1", "7"):
        env = dict(os.environ, OMP_NUM_THREADS=n)
        outs.append(subprocess.run([sys.executable, "-c", code], env=env, check=True,
                                   capture_output=True, text=True).stdout)
    assert outs[0] == outs[1] and len(outs[0]) > 0
