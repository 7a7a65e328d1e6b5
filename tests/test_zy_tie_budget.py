"""Near-tie budget over every GPU comparison of the session (collected after
the other GPU tests): draws whose GPU result differs from the oracle's are
allowed only where the oracle's own margin is below 1e-6, and such near-ties
must stay below 0.01% of the draws compared.  Also logs the largest deviations
of the GPU's normalisers (lse of p^d and p^t), acceptance log-ratio and
log p^d output from the oracle's."""
import pytest

from parity_util import STATS, log

pytestmark = pytest.mark.gpu


def test_near_tie_budget():
    if STATS["draws"] == 0:
        pytest.skip("no GPU comparison ran in this session")
    log(f"session: {STATS['draws']} draws compared, {STATS['ties']} near-ties; "
        f"max |lse_d gpu - oracle| {STATS['max_lse_d_err']:.3e}, "
        f"max |lse_t gpu - oracle| {STATS['max_lse_t_err']:.3e}, "
        f"max |rho gpu - oracle| {STATS['max_rho_err']:.3e}, "
        f"max |log p^d gpu - oracle| {STATS['max_logpd_err']:.3e} over {STATS['logpd_values']} values")
    assert STATS["ties"] < 1e-4 * STATS["draws"], \
        f"{STATS['ties']} near-ties in {STATS['draws']} draws exceed 0.01%"
