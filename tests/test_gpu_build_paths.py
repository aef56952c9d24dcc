"""GPU: both neighbour-build paths against the oracle.

Replicas of at most 512 atoms are built from all-pairs row bit masks (one
block per replica slice, two launches, pair arrays included on the MD path;
a system of one replica of at most 128 atoms in one launch); larger ones by
the cell list.  The library picks the path from the largest replica, so
systems just below and just above each size run both paths on the same kind
of input: the CSR must be bit-identical to the oracle's either way, and a few
Verlet steps must follow the oracle's trajectory.
"""
import sys

import numpy as np
import pytest

import oracle as O
import synth
from helpers import E_TOL, F_TOL, md_evaluation_errors

pytestmark = pytest.mark.gpu

TILE_MAX = 512   # the largest replica the mask path builds
TILE_ONE_MAX = 128   # the largest single replica the mask path builds in one launch


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


def _system(sizes, side, seed, min_d=2.5):
    pos = np.concatenate([synth.box_rsa(n, side, min_d, synth.seed64(seed, b)) for b, n in enumerate(sizes)])
    rp = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    return pos.astype(np.float32), rp


def _model(F=32, K=8, I=1, T=3, rc=7.0, seed=11):
    return synth.init_params(T, I, F, K, seed), {"n_types": T, "n_interactions": I, "n_features": F, "n_rbf": K,
                                                  "cutoff": rc, **synth.rbf_hyper(K, 0.0, rc)}


def test_cell_list_rows_longer_and_shorter_than_the_kept_length(sn):
    """The cell-list fill pass sorts the rows its count pass kept (up to 256 entries) and tests the
    candidates again for longer ones: a dense replica (rows of ~300-450) and a sparse one (rows of
    ~40) in one build, CSR bit-identical to the oracle's."""
    say("[build paths] cell list, rows above and below the kept length")
    pos = np.concatenate([synth.box_rsa(1500, 24.0, 1.0, synth.seed64(77, 0)),
                          synth.box_rsa(700, 40.0, 1.0, synth.seed64(77, 1)) + 100.0]).astype(np.float32)
    rp = np.array([0, 1500, 2200], np.int32)
    params, hyper = _model(rc=6.5)
    model = sn.Model(params, hyper)
    system = sn.System(rp, np.zeros(len(pos), np.int32), None)
    cap = 600 * len(pos)
    ws = sn.workspace(model, system, cap)
    row_ptr, col, rev, E = sn.build_csr_neighbors(system, dev(pos), 9.5, cap, ws)
    ref = O.neighbors_bruteforce(pos, rp, 9.5, None)
    lens = np.diff(ref[0])
    say(f"   E={E}, row lengths {lens.min()}..{lens.max()}, {int((lens > 256).sum())} rows above 256")
    assert lens.max() > 256 and lens.min() < 256
    assert E == len(ref[1])
    assert np.array_equal(row_ptr.cpu().numpy(), ref[0])
    assert np.array_equal(col.cpu().numpy()[:E], ref[1])
    assert np.array_equal(rev.cpu().numpy()[:E], ref[2])


@pytest.mark.parametrize("sizes,periodic", [
    ([TILE_MAX, TILE_MAX], False),         # mask path at its largest replica
    ([TILE_MAX, TILE_MAX + 1], False),     # one atom more: the cell list
    ([300, 0, 1, 2, 211], False),          # empty and tiny replicas on the mask path
    ([400], True),                         # periodic, mask path
    ([TILE_MAX + 88], True),               # periodic, cell list
    ([64], False),                         # one replica, one launch: one mask word per row
    ([65], False),                         # ... two words
    ([TILE_ONE_MAX], False),               # ... at its largest
    ([TILE_ONE_MAX + 1], False),           # one atom more: two launches
    ([100], True),                         # periodic, one launch
])
def test_csr_bit_exact_on_both_paths(sn, sizes, periodic):
    say(f"[build paths] sizes={sizes} periodic={periodic}")
    side = 26.0
    pos, rp = _system(sizes, side, 7 + len(sizes) + int(periodic))
    box = np.array([side] * 3, np.float32) if periodic else None
    params, hyper = _model(rc=6.5)
    model = sn.Model(params, hyper)
    system = sn.System(rp, np.zeros(len(pos), np.int32), box)
    cap = max(64, 200 * len(pos))
    ws = sn.workspace(model, system, cap)
    for r_list in (6.5, 8.0):
        row_ptr, col, rev, E = sn.build_csr_neighbors(system, dev(pos), r_list, cap, ws)
        ref = O.neighbors_bruteforce(pos, rp, r_list, box)
        say(f"   r_list={r_list}: E={E}")
        assert E == len(ref[1]) and E > 0
        assert np.array_equal(row_ptr.cpu().numpy(), ref[0])
        assert np.array_equal(col.cpu().numpy()[:E], ref[1])
        assert np.array_equal(rev.cpu().numpy()[:E], ref[2])


def test_one_launch_build_edge_cases(sn):
    """One-replica systems on the one-launch mask build: a lone atom (no edges), pairs at the
    strict fp32 cutoff (just below, at and just above r_list), and a periodic wrap."""
    rc = np.float32(10.0)
    below = np.nextafter(rc, np.float32(0))
    above = np.nextafter(rc, np.float32(20))
    cases = [
        (np.array([[1.0, 2.0, 3.0]], np.float32), None, 10.0),
        (np.array([[0, 0, 0], [below, 0, 0], [0, rc, 0], [0, 0, above]], np.float32), None, 10.0),
        (np.array([[0.5, 10, 10], [19.5, 10, 10], [10, 10, 10]], np.float32), np.array([20.0] * 3, np.float32),
         6.0),
    ]
    params, hyper = _model(rc=6.0)
    for pos, box, r_list in cases:
        say(f"[build paths] one launch, {len(pos)} atoms, periodic={box is not None}")
        rp = np.array([0, len(pos)], np.int32)
        model = sn.Model(params, hyper)
        system = sn.System(rp, np.zeros(len(pos), np.int32), box)
        ws = sn.workspace(model, system, 64)
        row_ptr, col, rev, E = sn.build_csr_neighbors(system, dev(pos), r_list, 64, ws)
        ref = O.neighbors_bruteforce(pos, rp, r_list, box)
        assert E == len(ref[1])
        assert np.array_equal(row_ptr.cpu().numpy(), ref[0])
        assert np.array_equal(col.cpu().numpy()[:E], ref[1])
        assert np.array_equal(rev.cpu().numpy()[:E], ref[2])


@pytest.mark.parametrize("sizes", [[200, 200], [120], [60]])
def test_capacity_error_on_the_mask_path(sn, sizes):
    pos, rp = _system(sizes, 20.0, 3)
    params, hyper = _model()
    model = sn.Model(params, hyper)
    system = sn.System(rp, np.zeros(len(pos), np.int32))
    ws = sn.workspace(model, system, 50_000)
    ref = O.neighbors_bruteforce(pos, rp, 7.0)
    st, ne = sn.build_csr_status(system, dev(pos), 7.0, 100, ws)
    assert st == sn.SN_ERR_CAPACITY and ne == len(ref[1])
    st, ne = sn.build_csr_status(system, dev(pos), 7.0, 50_000, ws)
    assert st == sn.SN_OK and ne == len(ref[1])


@pytest.mark.parametrize("sizes", [[250, 250], [TILE_MAX + 100], [120], [60]])
def test_verlet_on_both_paths_matches_oracle(sn, sizes):
    """Three steps: the mask path (two launches, or one for a single replica of at most 128 atoms)
    also writes the pair arrays; the cell path runs the pair setup."""
    import torch
    say(f"[build paths] verlet sizes={sizes}")
    pos, rp = _system(sizes, 24.0 if len(sizes) > 1 else 28.0, 21)
    params, hyper = _model(F=32, K=8, I=2, rc=7.0)
    types = np.random.default_rng(5).integers(0, 3, len(pos)).astype(np.int32)
    inv_mass = np.full(len(pos), 1.0 / 110.0, np.float32)
    vel = synth.maxwell_boltzmann(len(pos), rp, 110.0, 300.0, 9).astype(np.float32)
    model = sn.Model(params, hyper)
    system = sn.System(rp, types)
    cap = 200 * len(pos)
    ws = sn.workspace(model, system, cap)
    p, v, im = dev(pos), dev(vel), dev(inv_mass)
    row_ptr, col, rev, E = sn.build_csr_neighbors(system, p, 7.0, cap, ws)
    _, forces = sn.energy_forces(model, system, p, row_ptr, col, rev, E, ws)
    n = 3
    B = len(sizes)
    epot = torch.zeros((n, B), dtype=torch.float64, device="cuda")
    sn.verlet_step(model, system, p, v, forces, im, 2.0, synth.FORCE_TO_ACCEL, n, 7.0, cap, ws, epot)
    torch.cuda.synchronize()
    r_ref, v_ref, f_ref, ep_ref, _ = O.verlet(params, hyper, types, pos, vel, inv_mass, rp, 2.0,
                                              synth.FORCE_TO_ACCEL, n, 7.0)
    dr = np.abs(p.cpu().numpy() - r_ref).max()
    dv = np.abs(v.cpu().numpy() - v_ref).max() / np.abs(v_ref).max()
    say(f"   max |dr| {dr:.2e} A, max rel dv {dv:.2e}")
    assert dr < 5e-5 and dv < 5e-5
    # the final state's energy and forces against the oracle at the GPU's positions
    e_err, f_err = md_evaluation_errors(params, hyper, types, rp, None, p.cpu().numpy(), forces.cpu().numpy(),
                                        epot.cpu().numpy()[-1])
    say(f"   final state: energy err {e_err.max():.2e}, force err {f_err.max():.2e}")
    assert e_err.max() <= E_TOL and f_err.max() <= F_TOL


@pytest.mark.parametrize("n", [400, TILE_MAX + 88])
def test_periodic_verlet_on_both_paths_matches_oracle(sn, n):
    """Three steps in a periodic box on the mask path (400 particles) and the cell list (600), with
    the particles shifted so that nearly all of them lie outside [0, L): the library never wraps
    positions, the predicate takes the minimum image and the cell binning wraps.  Against the
    oracle's trajectory, and the final state at the contract tolerances."""
    import torch
    say(f"[build paths] periodic verlet n={n}")
    side = 26.0
    pos, rp = _system([n], side, 31 + n)
    pos = (pos + np.array([-0.3, 0.2, 25.9], np.float32)).astype(np.float32)   # mostly outside the box
    box = np.array([side] * 3, np.float32)
    params, hyper = _model(F=32, K=8, I=2, rc=7.0)
    types = np.random.default_rng(n).integers(0, 3, len(pos)).astype(np.int32)
    inv_mass = np.full(len(pos), 1.0 / 110.0, np.float32)
    vel = synth.maxwell_boltzmann(len(pos), rp, 110.0, 300.0, 13).astype(np.float32)
    model = sn.Model(params, hyper)
    system = sn.System(rp, types, box)
    cap = 200 * len(pos)
    ws = sn.workspace(model, system, cap)
    p, v, im = dev(pos), dev(vel), dev(inv_mass)
    row_ptr, col, rev, E = sn.build_csr_neighbors(system, p, 7.0, cap, ws)
    _, forces = sn.energy_forces(model, system, p, row_ptr, col, rev, E, ws)
    steps = 3
    epot = torch.zeros((steps, 1), dtype=torch.float64, device="cuda")
    sn.verlet_step(model, system, p, v, forces, im, 2.0, synth.FORCE_TO_ACCEL, steps, 7.0, cap, ws, epot)
    torch.cuda.synchronize()
    r_ref, v_ref, f_ref, ep_ref, _ = O.verlet(params, hyper, types, pos, vel, inv_mass, rp, 2.0,
                                              synth.FORCE_TO_ACCEL, steps, 7.0, box)
    dr = np.abs(p.cpu().numpy() - r_ref).max()
    dv = np.abs(v.cpu().numpy() - v_ref).max() / np.abs(v_ref).max()
    outside = int(((r_ref < 0) | (r_ref >= side)).any(axis=1).sum())
    say(f"   {outside} particles outside [0, L); max |dr| {dr:.2e} A, max rel dv {dv:.2e}")
    assert outside > 0
    assert dr < 5e-5 and dv < 5e-5
    e_err, f_err = md_evaluation_errors(params, hyper, types, rp, box, p.cpu().numpy(), forces.cpu().numpy(),
                                        epot.cpu().numpy()[-1])
    say(f"   final state: energy err {e_err.max():.2e}, force err {f_err.max():.2e}")
    assert e_err.max() <= E_TOL and f_err.max() <= F_TOL


@pytest.mark.parametrize("F,I,log_ekin", [(32, 1, False), (64, 1, True), (64, 2, False), (128, 2, True)])
def test_verlet_model_shapes_match_oracle(sn, F, I, log_ekin):
    """MD on the tile path for other feature widths and interaction counts: with one interaction
    the last chain reads the embedding rows kept across steps; logging the kinetic energy splits
    the opening kick from the force assembly."""
    import torch
    say(f"[md shapes] F={F} I={I} ekin={log_ekin}")
    pos, rp = _system([150, 170], 22.0, 40 + F + I)
    params, hyper = _model(F=F, K=12, I=I, T=4, rc=7.0, seed=F + I)
    types = np.random.default_rng(F).integers(0, 4, len(pos)).astype(np.int32)
    inv_mass = np.full(len(pos), 1.0 / 110.0, np.float32)
    vel = synth.maxwell_boltzmann(len(pos), rp, 110.0, 300.0, 3).astype(np.float32)
    model = sn.Model(params, hyper)
    system = sn.System(rp, types)
    cap = 200 * len(pos)
    ws = sn.workspace(model, system, cap)
    p, v, im = dev(pos), dev(vel), dev(inv_mass)
    row_ptr, col, rev, E = sn.build_csr_neighbors(system, p, 7.0, cap, ws)
    _, forces = sn.energy_forces(model, system, p, row_ptr, col, rev, E, ws)
    n, B = 4, len(rp) - 1
    epot = torch.zeros((n, B), dtype=torch.float64, device="cuda")
    ekin = torch.zeros((n, B), dtype=torch.float64, device="cuda") if log_ekin else None
    sn.verlet_step(model, system, p, v, forces, im, 2.0, synth.FORCE_TO_ACCEL, n, 7.0, cap, ws, epot, ekin)
    torch.cuda.synchronize()
    r_ref, v_ref, f_ref, ep_ref, ek_ref = O.verlet(params, hyper, types, pos, vel, inv_mass, rp, 2.0,
                                                   synth.FORCE_TO_ACCEL, n, 7.0)
    assert np.abs(p.cpu().numpy() - r_ref).max() < 5e-5
    assert np.abs(v.cpu().numpy() - v_ref).max() < 5e-5 * np.abs(v_ref).max()
    e_err, f_err = md_evaluation_errors(params, hyper, types, rp, None, p.cpu().numpy(), forces.cpu().numpy(),
                                        epot.cpu().numpy()[-1])
    say(f"   final state: energy err {e_err.max():.2e}, force err {f_err.max():.2e}")
    assert e_err.max() <= E_TOL and f_err.max() <= F_TOL
    if log_ekin:
        ek = O.kinetic_energy(v.cpu().numpy(), inv_mass, rp, synth.FORCE_TO_ACCEL)
        assert np.abs(ekin.cpu().numpy()[-1] - ek).max() <= 2e-7 * np.abs(ek).max()   # the library takes c as fp32


def test_verlet_empty_system_counts_steps(sn):
    """No atoms: the steps still complete and every energy is zero."""
    import torch
    params, hyper = _model()
    model = sn.Model(params, hyper)
    system = sn.System(np.array([0, 0], np.int32), np.zeros(0, np.int32))
    ws = sn.workspace(model, system, 64)
    z = torch.zeros((0, 3), dtype=torch.float32, device="cuda")
    epot = torch.full((3, 1), 7.0, dtype=torch.float64, device="cuda")
    rp, _, _, ne = sn.verlet_step(model, system, z, z.clone(), z.clone(), torch.zeros(0, device="cuda"), 2.0,
                                  synth.FORCE_TO_ACCEL, 3, 7.0, 64, ws, epot)
    torch.cuda.synchronize()
    assert ne == 0 and np.all(epot.cpu().numpy() == 0.0)
