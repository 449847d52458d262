"""The fp64 oracle against its pins (CPU only)."""
import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(orc, pin):
    pin(orc)


def test_oracle_rejects_bad_arguments(orc):
    import numpy as np
    x = np.zeros((1, 4, 4))
    with pytest.raises(ValueError):
        orc.headwise_fwd(x, np.zeros((1, 4, 3, 2)))      # D % H != 0
    with pytest.raises(ValueError):
        orc.headwise_fwd(x, np.zeros((1, 4, 4, 2)), cu_seqlens=[0, 3, 2, 4])
    with pytest.raises(ValueError):
        orc.headwise_fwd(x, np.zeros((1, 4, 4, 2)), cu_seqlens=[0, 2, 5])
    with pytest.raises(ValueError):
        orc.rope(x, rot=3, head_dim=2)                     # rot not a multiple of head_dim
    with pytest.raises(ValueError):
        orc.rope(x, rot=4, head_dim=3)                     # odd head_dim
    with pytest.raises(ValueError):
        orc.rope(x, rot=6, head_dim=2)                     # rot > D
