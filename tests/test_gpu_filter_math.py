"""The filter network with one fp16 product per fp32 product (sn_model.filter_math = 1).

That mode rounds both operands of each matrix product of the filter network to fp16 (after the same
power-of-two scaling as the split path) and accumulates in fp32: the reduced-precision tensor-core
arithmetic of the FlashSchNet summary page ("How", the TF32/MFU bullet).  Its filter rows are checked
against the oracle's filter within the error bound that this arithmetic implies; its energies and
forces are reported against the oracle and against the fp32-accurate mode (drift), and bounded
loosely.
"""
import sys

import numpy as np
import pytest

import oracle as O
import synth
from helpers import energy_errors, force_errors, oracle_full

pytestmark = pytest.mark.gpu

U16 = 2.0 ** -11          # unit roundoff of fp16
U32 = 2.0 ** -24          # unit roundoff of fp32


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def sn():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import schnet_cfconv_force_amd as sn
    sn.lib()
    return sn


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def fp16_product_bound(e, blk):
    """Bound on |phi_fp16 - phi| for the two rounded products, from the arithmetic.

    Layer 1, a = e A1 + b1: each operand is rounded to fp16 (relative error <= u), so each term has
    relative error <= 2u + u^2; values of e below fp16's normal range (2^-14) are rounded to an
    absolute 2^-25; the fp32 accumulation of K terms adds K u32 relative to sum |e||A1|.  ssp is
    1-Lipschitz, so |dz| <= |da| plus its own fp32 evaluation error.  Layer 2, phi = z A2 + b2: the
    same per-term bound on z's rounding, plus the propagated |dz| |A2|.
    """
    A1 = np.abs(np.asarray(blk["A1"], np.float64))
    A2 = np.asarray(blk["A2"], np.float64)
    K, F = A1.shape
    ea = np.abs(e)
    da = (2 * U16 + U16 ** 2 + K * U32) * (ea @ A1) + 2.0 ** -25 * A1.sum(axis=0)[None, :]
    a = e @ np.asarray(blk["A1"], np.float64) + np.asarray(blk["b1"], np.float64)
    z = O.ssp(a)
    dz = da + 2.0 ** -21 * (np.abs(z) + 1.0)
    absA2 = np.abs(A2)
    return (2 * U16 + U16 ** 2 + F * U32) * (np.abs(z) @ absA2) + (1 + U16) ** 2 * (dz @ absA2)


@pytest.mark.parametrize("name", ["tiny_chain", "single_protein", "dense_box"])
def test_filter_rows_within_the_fp16_product_bound(sn, name):
    say(f"[filter, fp16 products] {name}")
    cfg = synth.make_config(name)
    h = cfg["hyper"]
    model = sn.Model(cfg["params"], h, filter_math=1)
    system = sn.System(cfg["replica_ptr"], cfg["types"], cfg["box"])
    ws = sn.workspace(model, system, 64)
    rng = np.random.default_rng(6)
    d = np.concatenate([np.linspace(0.05, h["cutoff"] * 1.1, 997), rng.uniform(0, h["cutoff"], 1003)])
    d = d.astype(np.float32)
    e, _ = O.gaussian_rbf(d, h["n_rbf"], h["rbf_lo"], h["rbf_hi"], h["rbf_gamma"])
    worst, seen = 0.0, 0.0
    for t in range(h["n_interactions"]):
        phi = sn.filter_forward(model, t, dev(d), ws).cpu().numpy().astype(np.float64)
        blk = {k: np.asarray(v, np.float64) for k, v in cfg["params"]["interactions"][t].items()}
        ref = O.ssp(e @ blk["A1"] + blk["b1"]) @ blk["A2"] + blk["b2"]
        bound = fp16_product_bound(e, blk) + 2.0 ** -22 * np.abs(ref)
        err = np.abs(phi - ref)
        ratio = err / bound
        worst = max(worst, float(ratio.max()))
        seen = max(seen, float((err / np.maximum(np.abs(ref), np.sqrt((ref ** 2).mean()))).max()))
        assert np.all(err <= bound), f"t={t}: error/bound up to {ratio.max():.3f}"
    say(f"   largest error / bound {worst:.3f}; largest relative error {seen:.2e}")
    # the mode is really reduced precision (a bound this loose would also pass fp32 results)
    assert seen > 1e-6


def test_energy_forces_fp16_filter_math_against_oracle_and_fp32_mode(sn):
    """One evaluation of four 269-bead replicas in both modes.  The fp16 products give errors of
    the TF32 class; bounds: energy 2e-3, forces 2e-2 (relative, as the parity tests measure them),
    several times what the mode shows, and the fp32-accurate mode on the same inputs still meets
    1e-5 / 1e-4."""
    cfg = synth.make_config("batched_replicas")
    rp = cfg["replica_ptr"]
    n = int(rp[4])
    cfg = dict(cfg, pos=cfg["pos"][:n], types=cfg["types"][:n], replica_ptr=rp[:5])
    E_ref, F_ref, eps_abs, _ = oracle_full(cfg)
    out = {}
    for math in (0, 1):
        model = sn.Model(cfg["params"], cfg["hyper"], filter_math=math)
        system = sn.System(cfg["replica_ptr"], cfg["types"], cfg["box"])
        pos = dev(cfg["pos"])
        cap = n * 200
        ws = sn.workspace(model, system, cap)
        row_ptr, col, rev, E = sn.build_csr_neighbors(system, pos, cfg["hyper"]["cutoff"], cap, ws)
        en, f = sn.energy_forces(model, system, pos, row_ptr, col, rev, E, ws)
        assert sn.read_status(ws) == sn.SN_OK
        out[math] = (en.cpu().numpy().astype(np.float64), f.cpu().numpy().astype(np.float64))
    for math, (en, f) in out.items():
        ee = energy_errors(en, E_ref, eps_abs).max()
        fe = force_errors(f, F_ref, cfg["replica_ptr"]).max()
        say(f"   filter_math={math}: energy max rel err {ee:.2e}  force max rel err {fe:.2e}")
        if math == 0:
            assert ee <= 1e-5 and fe <= 1e-4
        else:
            assert np.all(np.isfinite(en)) and np.all(np.isfinite(f))
            assert ee <= 2e-3 and fe <= 2e-2
    f0, f1 = out[0][1], out[1][1]
    say(f"   RMS force change {np.sqrt(((f1 - f0) ** 2).mean() / (f0 ** 2).mean()):.2e}")
