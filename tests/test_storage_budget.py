"""Error budget of the 24-bit storage of the filter rows (CPU, oracle only).

The GPU pipeline keeps each interaction's filter rows phi in HBM as fp32
values rounded to their upper three bytes (sign, exponent and 15 mantissa
bits, the magnitude rounded half up): a relative error of at most 2^-16 per
value.  Here the oracle is run with exactly that rounding applied to phi and
compared with the exact oracle: the format must use at most a quarter of the
parity tolerances (energy 1e-5 relative, forces 1e-4 relative per
component), leaving the rest to the arithmetic of the GPU path.
"""
import numpy as np
import pytest

import synth
from oracle import schnet_oracle as O
from helpers import energy_errors, force_errors


def fp24(x):
    """Round float values to the 24-bit format: fp32 bit pattern + 0x80, low byte cleared."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = ((u + np.uint64(0x80)) & np.uint64(0xFFFFFF00)).astype(np.uint32)
    return u.view(np.float32).astype(np.float64)


def test_fp24_rounding_bound():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(100000) * 10.0 ** rng.uniform(-6, 6, 100000)).astype(np.float32)
    r = fp24(x)
    rel = np.abs(r - x.astype(np.float64)) / np.abs(x.astype(np.float64))
    assert rel.max() <= 2.0 ** -16 * (1 + 1e-12)
    # the rounding is not biased: the mean relative error over many values is tiny
    assert abs(np.mean((r - x) / np.abs(x))) < 1e-6
    # values exact in 15 mantissa bits survive unchanged
    y = fp24(x).astype(np.float32)
    assert np.array_equal(fp24(y), y.astype(np.float64))


@pytest.mark.parametrize("name", ["tiny_chain", "single_protein"])
def test_filter_row_storage_error_budget(name):
    cfg = synth.make_config(name)
    h = cfg["hyper"]
    csr = O.neighbors_bruteforce(cfg["pos"], cfg["replica_ptr"], h["cutoff"], cfg["box"])
    args = (cfg["params"], h, cfg["types"], cfg["pos"], cfg["replica_ptr"], csr, cfg["box"])
    E0, F0, inter = O.energy_forces(*args, return_intermediates=True)
    E1, F1 = O.energy_forces(*args, phi_store=fp24)
    rp = np.asarray(cfg["replica_ptr"], np.int64)
    eabs = np.array([np.abs(inter["eps"][rp[b]:rp[b + 1]]).sum() for b in range(len(rp) - 1)])
    e_err = energy_errors(E1, E0, eabs).max()
    f_err = force_errors(F1, F0, cfg["replica_ptr"]).max()
    print(f"{name}: energy {e_err:.2e}, forces {f_err:.2e}")
    assert e_err < 2.5e-6
    assert f_err < 2.5e-5
