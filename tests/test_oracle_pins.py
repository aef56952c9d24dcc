"""Pins of the CPU oracle to facts outside itself (CPU only).

Each test ties a part of the oracle to something it does not compute itself:
a library routine (scipy's k-d tree), closed forms and special values, a
50-digit scalar evaluation of tiny systems written index by index,
finite differences, symmetries of the energy, and Verlet special cases.
"""
import json
import os

import mpmath as mp
import numpy as np
import pytest
from scipy.spatial import cKDTree

import oracle as O
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _tiny_model(F=4, K=3, I=2, T=3, rc=5.0, seed=11):
    hyper = {"n_types": T, "n_interactions": I, "n_features": F, "n_rbf": K, "cutoff": rc,
             **synth.rbf_hyper(K, 0.0, rc)}
    params = synth.init_params(T, I, F, K, seed)
    return params, hyper


def _ef(params, hyper, types, pos, rp, box=None, r_list=None):
    csr = O.neighbors_bruteforce(pos, rp, hyper["cutoff"] if r_list is None else r_list, box)
    return O.energy_forces(params, hyper, types, pos, rp, csr, box)


# ---------------------------------------------------------------- neighbours

@pytest.mark.parametrize("name", ["tiny_chain", "single_protein", "dense_box"])
def test_neighbors_match_kdtree(name):
    """The fp32 brute-force sets agree with scipy's k-d tree (fp64) away from ties."""
    c = synth.make_config(name)
    rc = c["hyper"]["cutoff"]
    pos = c["pos"].astype(np.float64)
    row_ptr, col, rev = O.neighbors_bruteforce(c["pos"], c["replica_ptr"], rc, c["box"])
    rows = np.repeat(np.arange(len(pos)), np.diff(row_ptr))
    got = set(zip(rows.tolist(), col.tolist()))
    if c["box"] is not None:
        L = float(c["box"][0])
        tree = cKDTree(np.mod(pos, L), boxsize=L)
    else:
        tree = cKDTree(pos)
    pairs = tree.query_pairs(rc + 1e-3, output_type="ndarray")
    want = set()
    amb = set()
    for i, j in pairs:
        d = pos[j] - pos[i]
        if c["box"] is not None:
            d -= L * np.rint(d / L)
        r = np.sqrt((d * d).sum())
        if abs(r - rc) < 1e-4:
            amb |= {(i, j), (j, i)}
        elif r < rc:
            want |= {(int(i), int(j)), (int(j), int(i))}
    assert (got - amb) == want
    # CSR structure: sorted rows, reverse edges
    for i in range(len(pos)):
        seg = col[row_ptr[i]:row_ptr[i + 1]]
        assert np.all(np.diff(seg) > 0)
    assert np.array_equal(rev[rev], np.arange(len(col)))
    assert np.array_equal(col[rev], rows)


def test_neighbors_cutoff_is_strict_in_fp32():
    rc = np.float32(10.0)
    below = np.nextafter(rc, np.float32(0))
    above = np.nextafter(rc, np.float32(20))
    pos = np.array([[0, 0, 0], [below, 0, 0], [0, rc, 0], [0, 0, above]], np.float32)
    rp = np.array([0, 4], np.int32)
    row_ptr, col, _ = O.neighbors_bruteforce(pos, rp, rc)
    row0 = col[row_ptr[0]:row_ptr[1]].tolist()
    assert row0 == [1]                     # 10 - ulp in, exactly 10 out, 10 + ulp out


def test_neighbors_periodic_wrap_and_degenerate_rows():
    box = np.array([20.0, 20.0, 20.0], np.float32)
    pos = np.array([[0.5, 10, 10], [19.5, 10, 10], [10, 10, 10], [5, 5, 5]], np.float32)
    # replica 0: atoms 0..2 ; replica 1: the single atom 3 (an empty row)
    rp = np.array([0, 3, 4], np.int32)
    row_ptr, col, rev = O.neighbors_bruteforce(pos, rp, 6.0, box)
    assert row_ptr.tolist() == [0, 1, 2, 2, 2]
    assert col.tolist() == [1, 0]          # 0 and 1 are 1 Å apart through the boundary
    assert rev.tolist() == [1, 0]


def test_dense_box_degree_matches_density():
    c = synth.make_config("dense_box")
    row_ptr, _, _ = O.neighbors_bruteforce(c["pos"], c["replica_ptr"], 6.0, c["box"])
    mean_deg = row_ptr[-1] / (len(row_ptr) - 1)
    ideal = 0.1 * 4.0 / 3.0 * np.pi * 6.0 ** 3          # 90.48 for an ideal gas
    assert abs(mean_deg - ideal) / ideal < 0.02


# ------------------------------------------------------- radial functions

def test_radial_special_values():
    rc = 7.0
    fc, dfc = O.cosine_envelope(np.array([0.0, rc / 2, rc, rc + 1.0]), rc)
    assert np.allclose(fc, [1.0, 0.5, 0.0, 0.0], atol=1e-15)
    assert np.allclose(dfc, [0.0, -np.pi / (2 * rc), 0.0, 0.0], atol=1e-15)
    K, lo, hi, gamma = 5, 0.0, 4.0, 0.7
    mu = O.gaussian_centres(K, lo, hi)
    assert np.allclose(mu, [0, 1, 2, 3, 4])
    e, de = O.gaussian_rbf(mu, K, lo, hi, gamma)
    assert np.allclose(np.diag(e), 1.0) and np.allclose(np.diag(de), 0.0)
    assert np.isclose(e[0, 1], np.exp(-0.7))
    assert O.ssp(0.0) == 0.0 and O.sigmoid(0.0) == 0.5
    assert np.isclose(O.ssp(50.0), 50.0 - np.log(2.0)) and np.isclose(O.ssp(-50.0), -np.log(2.0))
    x = np.linspace(-6, 6, 13)
    h = 1e-6
    assert np.allclose((O.ssp(x + h) - O.ssp(x - h)) / (2 * h), O.sigmoid(x), atol=1e-9)
    assert np.allclose(O.sigmoid(x), 1.0 / (1.0 + np.exp(-x)), atol=1e-15)


def test_rbf_derivative_matches_difference():
    d = np.linspace(0.3, 9.7, 41)
    e_p, _ = O.gaussian_rbf(d + 1e-6, 6, 0.0, 10.0, 0.5)
    e_m, _ = O.gaussian_rbf(d - 1e-6, 6, 0.0, 10.0, 0.5)
    _, de = O.gaussian_rbf(d, 6, 0.0, 10.0, 0.5)
    assert np.allclose((e_p - e_m) / 2e-6, de, atol=1e-8)
    fp, _ = O.cosine_envelope(d + 1e-6, 10.0)
    fm, _ = O.cosine_envelope(d - 1e-6, 10.0)
    _, dfc = O.cosine_envelope(d, 10.0)
    assert np.allclose((fp - fm) / 2e-6, dfc, atol=1e-8)


# --------------------------------------- 50-digit scalar evaluation, index by index

def _mp_energy(params, hyper, types, pos):
    """Energy of one small open system, every sum written out by index, 50 digits."""
    mp.mp.dps = 50
    F, K = hyper["n_features"], hyper["n_rbf"]
    rc = mp.mpf(float(hyper["cutoff"]))
    lo, hi, gam = (mp.mpf(float(hyper[k])) for k in ("rbf_lo", "rbf_hi", "rbf_gamma"))
    n = len(pos)
    M = lambda a: [[mp.mpf(float(v)) for v in row] for row in np.atleast_2d(a)]
    V = lambda a: [mp.mpf(float(v)) for v in np.ravel(a)]
    sspm = lambda x: mp.log(mp.exp(x) / 2 + mp.mpf(1) / 2)
    r = [[mp.mpf(float(v)) for v in p] for p in pos]
    emb = M(params["emb"])
    h = [[emb[types[i]][f] for f in range(F)] for i in range(n)]
    for blk in params["interactions"]:
        Win, A1, b1, A2, b2 = M(blk["W_in"]), M(blk["A1"]), V(blk["b1"]), M(blk["A2"]), V(blk["b2"])
        Wo1, bo1, Wo2, bo2 = M(blk["Wo1"]), V(blk["bo1"]), M(blk["Wo2"]), V(blk["bo2"])
        x = [[sum(h[i][g] * Win[g][f] for g in range(F)) for f in range(F)] for i in range(n)]
        y = [[mp.mpf(0)] * F for _ in range(n)]
        for i in range(n):
            for j in range(n):
                if i == j:
                    continue
                d = mp.sqrt(sum((r[j][c] - r[i][c]) ** 2 for c in range(3)))
                if d >= rc:
                    continue
                fc = (mp.cos(mp.pi * d / rc) + 1) / 2
                rbf = [mp.exp(-gam * (d - (lo + k * (hi - lo) / (K - 1))) ** 2) for k in range(K)]
                a = [sum(rbf[k] * A1[k][f] for k in range(K)) + b1[f] for f in range(F)]
                phi = [sum(sspm(a[g]) * A2[g][f] for g in range(F)) + b2[f] for f in range(F)]
                for f in range(F):
                    y[i][f] += fc * phi[f] * x[j][f]
        for i in range(n):
            o = [sum(y[i][g] * Wo1[g][f] for g in range(F)) + bo1[f] for f in range(F)]
            v = [sum(sspm(o[g]) * Wo2[g][f] for g in range(F)) + bo2[f] for f in range(F)]
            h[i] = [h[i][f] + v[f] for f in range(F)]
    R1, c1, R2, c2 = M(params["R1"]), V(params["c1"]), V(params["R2"]), mp.mpf(float(params["c2"]))
    H = len(c1)
    E = mp.mpf(0)
    for i in range(n):
        q = [sum(h[i][g] * R1[g][m] for g in range(F)) + c1[m] for m in range(H)]
        E += sum(sspm(q[m]) * R2[m] for m in range(H)) + c2
    return E


@pytest.mark.parametrize("npart", [2, 3])
def test_energy_matches_50_digit_scalar_evaluation(npart):
    params, hyper = _tiny_model(F=4, K=3, I=2, T=3, rc=5.0, seed=npart)
    pos = np.array([[0.0, 0.0, 0.0], [3.1, 0.4, -0.2], [1.2, 2.6, 0.9]], np.float32)[:npart]
    types = np.array([0, 2, 1], np.int32)[:npart]
    rp = np.array([0, npart], np.int32)
    E, _ = _ef(params, hyper, types, pos, rp)
    Emp = _mp_energy(params, hyper, types, pos)
    assert abs(E[0] - float(Emp)) <= 1e-12 * max(1.0, abs(float(Emp)))


# ------------------------------------------------------------ forces

def _fd_forces(params, hyper, types, pos, rp, box=None, h=1e-5):
    csr = O.neighbors_bruteforce(pos.astype(np.float32), rp, hyper["cutoff"] + 0.5, box)
    f = np.zeros_like(pos)
    for a in range(len(pos)):
        for c in range(3):
            pp, pm = pos.copy(), pos.copy()
            pp[a, c] += h
            pm[a, c] -= h
            ep = O.energy_only(params, hyper, types, pp, rp, csr, box).sum()
            em = O.energy_only(params, hyper, types, pm, rp, csr, box).sum()
            f[a, c] = -(ep - em) / (2 * h)
    return f, csr


def test_forces_match_central_differences_open():
    c = synth.make_config("tiny_chain")
    pos = c["pos"].astype(np.float64)
    fd, csr = _fd_forces(c["params"], c["hyper"], c["types"], pos, c["replica_ptr"])
    _, f = O.energy_forces(c["params"], c["hyper"], c["types"], pos, c["replica_ptr"], csr)
    assert np.max(np.abs(f - fd)) <= 1e-6 * np.max(np.abs(f))


def test_forces_match_central_differences_periodic():
    params, hyper = _tiny_model(F=8, K=6, I=2, T=2, rc=4.0, seed=5)
    rng = np.random.default_rng(3)
    box = np.array([9.0, 9.0, 9.0], np.float32)
    pos = synth.box_rsa(12, 9.0, 1.5, synth.seed64(77))
    types = rng.integers(0, 2, 12).astype(np.int32)
    rp = np.array([0, 12], np.int32)
    fd, csr = _fd_forces(params, hyper, types, pos, rp, box)
    assert len(csr[1]) > 12
    _, f = O.energy_forces(params, hyper, types, pos, rp, csr, box)
    assert np.max(np.abs(f - fd)) <= 1e-6 * np.max(np.abs(f))


def _periodic_cell(n=10, L=9.0, seed=31):
    """n particles in a cubic periodic cell of side L (min distance 1.5 A), 2 types."""
    params, hyper = _tiny_model(F=8, K=6, I=2, T=2, rc=4.0, seed=13)
    pos = synth.box_rsa(n, L, 1.5, synth.seed64(seed))
    types = np.random.default_rng(seed).integers(0, 2, n).astype(np.int32)
    return params, hyper, pos, types, np.array([L, L, L], np.float32)


def test_periodic_energy_and_forces_equal_explicit_replication():
    """The periodic branch (minimum image) against an open-boundary system built by hand.

    In an I-interaction model the energy of atom i depends on the atoms within I rc of it,
    and the force on i on the atom energies within I rc of i, whose own inputs reach
    another I rc: with a shell of 2 L >= 2 I rc (L = 9, rc = 4, I = 2) around the central
    cell, the 5 x 5 x 5 replication gives the central atoms their full periodic environment.
    Their atom energies and forces must then equal the periodic system's; the sum of the
    central atom energies is the periodic energy.  Removing the minimum image from the
    oracle's pair geometry breaks this (the cross-boundary pairs would fall beyond rc).
    """
    params, hyper, pos, types, box = _periodic_cell()
    L = float(box[0])
    n = len(pos)
    rp1 = np.array([0, n], np.int32)
    csr_p = O.neighbors_bruteforce(pos.astype(np.float32), rp1, hyper["cutoff"], box)
    Ep, Fp, inter_p = O.energy_forces(params, hyper, types, pos, rp1, csr_p, box, return_intermediates=True)
    shifts = np.array([(a, b, c) for a in range(-2, 3) for b in range(-2, 3) for c in range(-2, 3)], np.float64)
    centre = int(np.flatnonzero((shifts == 0).all(axis=1))[0])
    big = (pos[None, :, :] + L * shifts[:, None, :]).reshape(-1, 3)
    big_types = np.tile(types, len(shifts))
    rpb = np.array([0, len(big)], np.int32)
    csr_o = O.neighbors_bruteforce(big.astype(np.float32), rpb, hyper["cutoff"])
    # every image pair the periodic list holds appears in the open one (no ties at rc)
    assert len(csr_p[1]) > 2 * n
    _, Fo, inter_o = O.energy_forces(params, hyper, big_types, big, rpb, csr_o, return_intermediates=True)
    sl = slice(centre * n, (centre + 1) * n)
    eps_o, eps_p = inter_o["eps"][sl], inter_p["eps"]
    assert np.max(np.abs(eps_o - eps_p)) <= 1e-12 * np.max(np.abs(eps_p))
    assert abs(eps_o.sum() - Ep[0]) <= 1e-12 * np.abs(eps_p).sum()
    assert np.max(np.abs(Fo[sl] - Fp)) <= 1e-12 * np.max(np.abs(Fp))
    assert np.max(np.abs(Fp)) > 1e-3                      # the cell does interact


def test_periodic_lattice_translation_invariance():
    """Shifting every atom by one vector and wrapping into [0, L) leaves the periodic energy and
    forces unchanged (the wrap moves atoms across the boundary, so pairs change images)."""
    params, hyper, pos, types, box = _periodic_cell(seed=47)
    L = float(box[0])
    rp1 = np.array([0, len(pos)], np.int32)
    E0, F0 = _ef(params, hyper, types, pos, rp1, box)
    rng = np.random.default_rng(8)
    for _ in range(3):
        moved = np.mod(pos + rng.uniform(0.0, L, 3), L)
        assert np.any(np.abs(moved - pos - (moved - pos).mean(axis=0)) > 1.0)   # some atoms wrapped
        E1, F1 = _ef(params, hyper, types, moved, rp1, box)
        assert abs(E1[0] - E0[0]) <= 1e-12 * abs(E0[0])
        assert np.max(np.abs(F1 - F0)) <= 1e-11 * np.max(np.abs(F0))


def test_net_force_and_torque_vanish():
    c = synth.make_config("batched_replicas", n_replicas=3)
    pos = c["pos"].astype(np.float64)
    _, f = _ef(c["params"], c["hyper"], c["types"], pos, c["replica_ptr"])
    for b in range(3):
        s, e = c["replica_ptr"][b], c["replica_ptr"][b + 1]
        scale = np.abs(f[s:e]).max()
        assert np.abs(f[s:e].sum(axis=0)).max() < 1e-11 * scale * (e - s)
        torque = np.cross(pos[s:e], f[s:e]).sum(axis=0)
        assert np.abs(torque).max() < 1e-10 * scale * (e - s) * np.abs(pos[s:e]).max()


# ------------------------------------------------------------ invariances

def _rand_rot(seed):
    q, r = np.linalg.qr(np.random.default_rng(seed).standard_normal((3, 3)))
    q = q * np.sign(np.diag(r))
    if np.linalg.det(q) < 0:
        q[:, 0] = -q[:, 0]
    return q


def test_translation_rotation_permutation_invariance():
    c = synth.make_config("single_protein")
    pos = c["pos"].astype(np.float64)
    args = (c["params"], c["hyper"])
    rp = c["replica_ptr"]
    r_list = c["hyper"]["cutoff"] + 0.5      # same edge set for every transformed copy
    E0, F0 = _ef(*args, c["types"], pos, rp, r_list=r_list)
    E1, F1 = _ef(*args, c["types"], pos + np.array([3.7, -1.2, 8.9]), rp, r_list=r_list)
    assert abs(E1[0] - E0[0]) < 1e-10 * abs(E0[0]) and np.allclose(F1, F0, atol=1e-9)
    R = _rand_rot(4)
    E2, F2 = _ef(*args, c["types"], pos @ R.T, rp, r_list=r_list)
    assert abs(E2[0] - E0[0]) < 1e-10 * abs(E0[0]) and np.allclose(F2, F0 @ R.T, atol=1e-9)
    perm = np.random.default_rng(9).permutation(len(pos))
    E3, F3 = _ef(*args, c["types"][perm], pos[perm], rp, r_list=r_list)
    assert abs(E3[0] - E0[0]) < 1e-10 * abs(E0[0]) and np.allclose(F3, F0[perm], atol=1e-9)


def test_replicas_are_independent():
    c = synth.make_config("batched_replicas", n_replicas=3)
    E, F = _ef(c["params"], c["hyper"], c["types"], c["pos"], c["replica_ptr"])
    rp = c["replica_ptr"]
    for b in range(3):
        s, e = rp[b], rp[b + 1]
        Eb, Fb = _ef(c["params"], c["hyper"], c["types"][s:e], c["pos"][s:e], np.array([0, e - s]))
        assert abs(Eb[0] - E[b]) < 1e-11 * abs(E[b]) and np.allclose(Fb, F[s:e], atol=1e-11)


def test_smooth_decay_at_cutoff():
    """For two beads, E(d) - E(far) = O((rc - d)^2) and the pair force = O(rc - d)."""
    params, hyper = _tiny_model(F=8, K=5, I=2, T=1, rc=6.0, seed=21)
    rp = np.array([0, 2], np.int32)
    types = np.zeros(2, np.int32)

    def ef(d):
        pos = np.array([[0, 0, 0], [d, 0, 0]], np.float64)
        csr = (np.array([0, 1, 2]), np.array([1, 0]), np.array([1, 0])) if d < 6.0 else \
              (np.array([0, 0, 0]), np.zeros(0, int), np.zeros(0, int))
        E, F = O.energy_forces(params, hyper, types, pos, rp, csr)
        return E[0], F[1, 0]
    e_far, _ = ef(7.0)
    ratios, fr = [], []
    for delta in (1e-2, 1e-3, 1e-4):
        e, f = ef(6.0 - delta)
        ratios.append((e - e_far) / delta ** 2)
        fr.append(f / delta)
    assert abs(ratios[1] / ratios[2] - 1) < 0.01 and abs(ratios[0] / ratios[1] - 1) < 0.1
    assert abs(fr[1] / fr[2] - 1) < 0.01
    assert abs(ratios[2]) > 1e-6          # the pair does interact


def test_cfconv_is_self_adjoint_for_pair_symmetric_filters():
    """With W_e = W_rev(e) the CSR segment reduce equals its own transpose."""
    c = synth.make_config("single_protein")
    row_ptr, col, rev = O.neighbors_bruteforce(c["pos"], c["replica_ptr"], 12.0)
    rng = np.random.default_rng(0)
    W = rng.standard_normal((len(col), 16))
    W = 0.5 * (W + W[rev])
    x = rng.standard_normal((len(row_ptr) - 1, 16))
    g = rng.standard_normal((len(row_ptr) - 1, 16))
    lhs = (g * O.cfconv(W, x, row_ptr, col)).sum()
    rhs = (O.cfconv(W, g, row_ptr, col) * x).sum()
    assert abs(lhs - rhs) < 1e-10 * abs(lhs)
    Wa = W + rng.standard_normal(W.shape) * 0.1        # asymmetric filters break it
    assert abs((g * O.cfconv(Wa, x, row_ptr, col)).sum() - (O.cfconv(Wa, g, row_ptr, col) * x).sum()) > 1e-6


# ------------------------------------------------------------ quantisation

def test_quantization_hand_example():
    gold = json.load(open(os.path.join(GOLDEN, "quantize_hand.json")))
    w = np.array(gold["w"], np.float32)
    q, s = O.quantize_per_out_channel(w)
    assert q.tolist() == gold["q"]
    want_s = [np.float32(v / 32767.0) for v in gold["scale_numerator"]]
    assert s.tolist() == [float(v) for v in want_s]


def test_quantization_error_bound():
    w = synth.init_params(4, 1, 128, 50, 3)["interactions"][0]["A2"]
    q, s = O.quantize_per_out_channel(w)
    wd = O.dequantize(q, s)
    # half a quantisation step, plus the float32 rounding of q * s
    bound = 0.5 * s[None, :].astype(np.float64) + np.abs(wd) * 2.0 ** -24
    assert np.all(np.abs(w.astype(np.float64) - wd) <= bound)
    assert np.all(np.abs(q).max(axis=0) == 32767)


# ------------------------------------------------------------ Verlet

def _md_system(B=2):
    c = synth.make_config("batched_replicas", n_replicas=B)
    return c


def test_verlet_free_flight_with_zero_weights():
    c = _md_system(2)
    zero = {k: np.zeros_like(v) for k, v in c["params"].items() if k != "interactions"}
    zero["interactions"] = [{k: np.zeros_like(v) for k, v in b.items()} for b in c["params"]["interactions"]]
    pos0 = c["pos"].astype(np.float64)
    vel = c["vel"].astype(np.float64)
    r, v, f, ep, ek = O.verlet(zero, c["hyper"], c["types"], pos0, vel, c["inv_mass"], c["replica_ptr"],
                               2.0, synth.FORCE_TO_ACCEL, 3, 12.0)
    assert np.all(f == 0.0)
    assert np.allclose(r, pos0 + 3 * 2.0 * vel, rtol=0, atol=1e-12)
    assert np.array_equal(v, vel)


def test_verlet_first_step_hand_formula_and_reversibility():
    c = _md_system(1)
    args = (c["params"], c["hyper"], c["types"])
    pos0, vel0 = c["pos"].astype(np.float64), c["vel"].astype(np.float64)
    im, rp, cst = c["inv_mass"], c["replica_ptr"], synth.FORCE_TO_ACCEL
    _, f0 = _ef(*args, pos0, rp)
    r1, v1, f1, _, _ = O.verlet(*args, pos0, vel0, im, rp, 2.0, cst, 1, 12.0)
    vh = vel0 + 0.5 * 2.0 * cst * f0 * im[:, None]
    assert np.allclose(r1, pos0 + 2.0 * vh, atol=1e-12)
    assert np.allclose(v1, vh + 0.5 * 2.0 * cst * f1 * im[:, None], atol=1e-15)
    r5, v5, _, _, _ = O.verlet(*args, pos0, vel0, im, rp, 2.0, cst, 5, 12.0)
    rb, vb, _, _, _ = O.verlet(*args, r5, -v5, im, rp, 2.0, cst, 5, 12.0)
    assert np.allclose(rb, pos0, atol=1e-9) and np.allclose(-vb, vel0, atol=1e-12)


def test_verlet_energy_error_scales_as_dt_squared():
    c = _md_system(1)
    args = (c["params"], c["hyper"], c["types"])
    pos0, vel0 = c["pos"].astype(np.float64), c["vel"].astype(np.float64) * 4.0
    im, rp, cst = c["inv_mass"], c["replica_ptr"], synth.FORCE_TO_ACCEL
    errs = []
    for dt, n in ((4.0, 10), (2.0, 20)):
        _, _, _, ep, ek = O.verlet(*args, pos0, vel0, im, rp, dt, cst, n, 12.0)
        tot = ep[:, 0] + ek[:, 0]
        E0 = _ef(*args, pos0, rp)[0][0] + O.kinetic_energy(vel0, im, rp, cst)[0]
        errs.append(np.abs(tot - E0).max())
    assert 2.5 < errs[0] / errs[1] < 6.0
