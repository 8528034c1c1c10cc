"""The machine probes (libspin_probe) run and give figures of the right size:
they are measurements, not part of the hot path, so there is nothing to
compare bit for bit; the checks bound them by what the chip can do."""

import pytest
import torch

from rotation_bit_quantization_amd import machine

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    machine.load()


@pytest.mark.parametrize("kind,peak", [(0, 5033.0), (1, 2517.0), (2, 10066.0)])
def test_mfma_rate_is_below_the_peak_and_the_clock_is_plausible(kind, peak):
    r = machine.mfma_rate(kind, waves_per_cu=8, iters=2000)
    # the published dense peaks at 2.4 GHz bound the rate; a busy chip stays above half of them
    assert 0.3 * peak < r["tops"] < 1.02 * peak, r
    assert 1.0 < r["clock_ghz"] < 2.5, r


def test_read_bandwidth_is_below_hbm_peak():
    r = machine.read_bandwidth(nbytes=1 << 30)
    assert 1.0 < r["tbps"] < 8.2, r


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_lds_rate_is_below_the_lds_width(mode):
    """One CU's LDS moves at most 128 bytes per cycle per direction on this
    family (a wider port would still bound it by 256); a working probe moves
    more than 16."""
    r = machine.lds_rate(mode, iters=1024)
    assert 16.0 < r["bytes_per_clk_per_cu"] < 260.0, r
    assert 1.0 < r["clock_ghz"] < 2.5, r
