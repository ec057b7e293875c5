"""The decode at its argument limits (T = 64 tokens, n_householder = 4), with
and without per-token scatter, against the fp64 oracle: the token loop's
staging passes (8 tokens each) run to the last one, and every slot is
checked (written ones to tolerance, untouched ones bitwise)."""
import pytest

import synth
from gpu_util import require_gpu
from test_gpu_kernels import _check_decode, _gpu_decode, _oracle_decode

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("scatter", [True, False], ids=["scatter", "write_back"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_at_limits(scatter, dtype):
    B = 4
    x = synth.decode_inputs(1900 + scatter, pool_size=B * (64 + 1) + 6, batch=B, T=64, n_hh=4, hq=2,
                            hv=4, dk=64, dv=64, dtype=dtype, skip_rows=1, write_slots=not scatter,
                            scatter=scatter)
    out_g, pool_g = _gpu_decode(x)
    out_r, pool_r = _oracle_decode(x)
    _check_decode(x, out_g, pool_g, out_r, pool_r, dtype)


def test_decode_at_limits_d128():
    """T = 64 with two sub-steps at the largest head size (128 x 128)."""
    x = synth.decode_inputs(1910, pool_size=20, batch=6, T=64, n_hh=2, hq=2, hv=4, dk=128, dv=128,
                            dtype="bf16", skip_rows=2, write_slots=True)
    out_g, pool_g = _gpu_decode(x)
    out_r, pool_r = _oracle_decode(x)
    _check_decode(x, out_g, pool_g, out_r, pool_r, "bf16")
