"""The CPU oracle against facts fixed by the pages, by mathematics and by libraries."""
import pytest

import oracle_pins

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(orc, pin):
    pin(orc)


def test_oracle_rejects_bad_arguments(orc):
    import numpy as np
    x = np.zeros((1, 1, 4, 4), dtype=np.float32)
    y = np.zeros((1, 1, 4, 4), dtype=np.float64)
    f = orc.lib.gtms_oracle_f64
    assert f(x.ctypes.data, y.ctypes.data, None, 1, 1, 4, 1.0, 0) == 1   # no lengths
    assert f(None, None, None, 1, 1, 4, 1.0, 7) == 2                     # unknown type
    assert f(None, None, None, -1, 1, 4, 1.0, 0) == 1                    # negative dim
    assert f(None, None, None, 0, 1, 4, 1.0, 0) == 0                     # empty: no-op
    assert f(None, None, None, 1 << 40, 1 << 20, 1 << 20, 1.0, 0) == 1   # overflow
