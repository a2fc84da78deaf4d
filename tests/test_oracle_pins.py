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


def test_attention_bad_arguments_rejected():
    import numpy as np
    q = np.zeros((1, 4, 4, 8), np.uint16)
    k = np.zeros((1, 4, 3, 8), np.uint16)
    w = np.zeros(8, np.uint16)
    with pytest.raises(ValueError):
        oracle.norm_attention(oracle.RMSNORM, q, k, k, w, None, w, None)   # 4 % 3 heads
    k = np.zeros((1, 4, 2, 8), np.uint16)
    with pytest.raises(ValueError):
        oracle.norm_attention(oracle.RMSNORM, q, k, k, w, w, w, w)         # RMSNorm, no beta
    with pytest.raises(ValueError):
        oracle.norm_attention(oracle.NO_NORM, q, k, k, w, None, None, None)  # no norm, a gamma
    with pytest.raises(ValueError):
        oracle.norm_attention(oracle.LAYERNORM, q, k, k, None, None, None, None)
    with pytest.raises(ValueError):
        oracle.norm_attention(oracle.NO_NORM, q, k, k, h=4)                # head out of range
    with pytest.raises(ValueError):
        oracle.norm_attention(oracle.NO_NORM, q, k, k, rows=(2, 5))        # rows past S
