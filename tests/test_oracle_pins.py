"""The CPU oracle against its pins (no GPU)."""
import pytest

import oracle
from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oracle.default())


def test_bad_arguments_rejected():
    import numpy as np
    x = np.zeros((2, 3), np.float32)
    w = np.ones(3, np.float32)
    with pytest.raises(ValueError):
        oracle.fwd(7, oracle.F32, x, w)                      # unknown kind
    with pytest.raises(ValueError):
        oracle.fwd(oracle.RMSNORM, oracle.F32, x, w, B=w)    # RMSNorm has no bias
    with pytest.raises(ValueError):
        oracle.fwd(oracle.LAYERNORM, oracle.F32, x, w, eps=-1.0)
    with pytest.raises(ValueError):
        oracle.fwd(oracle.LAYERNORM, oracle.F32, x, w, rows=(1, 3))
    with pytest.raises(TypeError):
        oracle.fwd(oracle.LAYERNORM, oracle.BF16, x, w)      # fp32 bits given as bf16
