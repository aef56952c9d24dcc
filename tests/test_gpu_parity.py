"""GPU parity: libsn.so against the CPU oracle on the same seeded inputs.

Neighbour lists must be bit-identical; energies agree to 1e-5 and forces to
1e-4 relative (with the floors documented in helpers.py); the int16 filter
path is compared with the oracle run on the dequantised weights.
"""
import sys

import numpy as np
import pytest

import oracle as O
import synth
from helpers import E_TOL, F_TOL, energy_errors, force_errors, oracle_full, oracle_replica

pytestmark = pytest.mark.gpu


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


class Loaded:
    def __init__(self, sn, cfg, fmt=0, capacity=None):
        self.cfg = cfg
        self.model = sn.Model(cfg["params"], cfg["hyper"], filter_format=fmt)
        self.system = sn.System(cfg["replica_ptr"], cfg["types"], cfg["box"])
        self.pos = dev(cfg["pos"])
        n = len(cfg["pos"])
        self.capacity = capacity if capacity is not None else max(64, n * 200)
        self.ws = sn.workspace(self.model, self.system, self.capacity)

    def csr(self, sn, r_list=None):
        r = self.cfg["hyper"]["cutoff"] if r_list is None else r_list
        return sn.build_csr_neighbors(self.system, self.pos, r, self.capacity, self.ws)

    def eval(self, sn, csr=None):
        row_ptr, col, rev, E = csr or self.csr(sn)
        en, f = sn.energy_forces(self.model, self.system, self.pos, row_ptr, col, rev, E, self.ws)
        import torch
        torch.cuda.synchronize()
        assert sn.read_status(self.ws) == sn.SN_OK
        return en.cpu().numpy().astype(np.float64), f.cpu().numpy().astype(np.float64)


# ------------------------------------------------------------------ filter network

@pytest.mark.parametrize("name", ["tiny_chain", "single_protein", "dense_box"])
@pytest.mark.parametrize("fmt", [0, 1])
def test_filter_forward_matches_oracle(sn, name, fmt):
    say(f"[filter] {name} fmt={fmt}")
    cfg = synth.make_config(name)
    h = cfg["hyper"]
    model = sn.Model(cfg["params"], h, filter_format=fmt)
    rng = np.random.default_rng(5)
    d = np.concatenate([np.linspace(0.05, h["cutoff"] * 1.1, 997), rng.uniform(0, h["cutoff"], 1003)])
    d = d.astype(np.float32)       # 2000 values: several tiles plus a ragged one
    params = O.dequantized_params(cfg["params"]) if fmt == 1 else cfg["params"]
    for t in range(h["n_interactions"]):
        phi = sn.filter_forward(model, t, dev(d)).cpu().numpy().astype(np.float64)
        blk = {k: np.asarray(v, np.float64) for k, v in params["interactions"][t].items()}
        e, _ = O.gaussian_rbf(d, h["n_rbf"], h["rbf_lo"], h["rbf_hi"], h["rbf_gamma"])
        ref = O.ssp(e @ blk["A1"] + blk["b1"]) @ blk["A2"] + blk["b2"]
        scale = np.maximum(np.abs(ref), np.sqrt((ref ** 2).mean()))
        err = np.abs(phi - ref) / scale
        say(f"   t={t} max rel err {err.max():.2e}")
        assert err.max() < 1e-5


# ------------------------------------------------------------------ neighbour list

def _oracle_csr(cfg, r_list=None):
    r = cfg["hyper"]["cutoff"] if r_list is None else r_list
    return O.neighbors_bruteforce(cfg["pos"], cfg["replica_ptr"], r, cfg["box"])


@pytest.mark.parametrize("name", list(synth.CONFIG_NAMES))
def test_neighbors_bit_exact(sn, name):
    say(f"[neighbours] {name}")
    cfg = synth.make_config(name)
    L = Loaded(sn, cfg)
    row_ptr, col, rev, E = L.csr(sn)
    ref = _oracle_csr(cfg)
    assert E == len(ref[1])
    assert np.array_equal(row_ptr.cpu().numpy(), ref[0])
    assert np.array_equal(col.cpu().numpy(), ref[1])
    assert np.array_equal(rev.cpu().numpy(), ref[2])
    # a second build gives the same bits (atomic binning order must not leak)
    row_ptr2, col2, rev2, E2 = L.csr(sn)
    assert E2 == E and np.array_equal(col2.cpu().numpy(), ref[1])
    say(f"   E={E}")


def test_neighbors_list_radius_larger_than_cutoff(sn):
    cfg = synth.make_config("single_protein")
    L = Loaded(sn, cfg)
    row_ptr, col, rev, E = L.csr(sn, r_list=13.5)
    ref = _oracle_csr(cfg, 13.5)
    assert np.array_equal(col.cpu().numpy(), ref[1]) and np.array_equal(rev.cpu().numpy(), ref[2])


def test_neighbors_edge_cases(sn):
    import torch
    rc = np.float32(10.0)
    below = np.nextafter(rc, np.float32(0))
    above = np.nextafter(rc, np.float32(20))
    # replica 0: strict cutoff in fp32; replica 1: empty; replica 2: one atom;
    # replica 3: atoms at large coordinates on cell boundaries
    pos = np.array([[0, 0, 0], [below, 0, 0], [0, rc, 0], [0, 0, above],
                    [5, 5, 5],
                    [1000.0, 1000.0, 1000.0], [1000.0 + 2 * 10.02, 1000.0, 1000.0], [1010.0, 1009.99, 1000.0],
                    [1000.0, 1009.999, 1000.0]], np.float32)
    rp = np.array([0, 4, 4, 5, 9], np.int32)
    cfg = {"pos": pos, "replica_ptr": rp, "types": np.zeros(len(pos), np.int32), "box": None,
           "params": synth.init_params(1, 1, 32, 4, 0),
           "hyper": {"n_types": 1, "n_interactions": 1, "n_features": 32, "n_rbf": 4, "cutoff": 10.0,
                     **synth.rbf_hyper(4, 0.0, 10.0)}}
    L = Loaded(sn, cfg)
    row_ptr, col, rev, E = L.csr(sn)
    ref = _oracle_csr(cfg)
    assert np.array_equal(row_ptr.cpu().numpy(), ref[0])
    assert np.array_equal(col.cpu().numpy(), ref[1]) and np.array_equal(rev.cpu().numpy(), ref[2])
    assert ref[1][ref[0][0]:ref[0][1]].tolist() == [1]
    # periodic wrap across the boundary
    box = np.array([20.0, 20.0, 20.0], np.float32)
    pos2 = np.array([[0.5, 10, 10], [19.5, 10, 10], [10, 10, 10], [5, 5, 5]], np.float32)
    cfg2 = dict(cfg, pos=pos2, replica_ptr=np.array([0, 3, 4], np.int32), types=np.zeros(4, np.int32),
                box=box, hyper=dict(cfg["hyper"], cutoff=6.0))
    L2 = Loaded(sn, cfg2)
    row_ptr, col, rev, E = L2.csr(sn)
    assert row_ptr.cpu().numpy().tolist() == [0, 1, 2, 2, 2]
    assert col.cpu().numpy().tolist() == [1, 0] and rev.cpu().numpy().tolist() == [1, 0]
    torch.cuda.synchronize()


def test_neighbors_error_paths(sn):
    cfg = synth.make_config("single_protein")
    L = Loaded(sn, cfg)
    ref = _oracle_csr(cfg)
    st, ne = sn.build_csr_status(L.system, L.pos, 12.0, 100, L.ws)
    assert st == sn.SN_ERR_CAPACITY and ne == len(ref[1])
    # box shorter than three cells of r_list
    bad = sn.System(cfg["replica_ptr"], cfg["types"], box=[30.0, 30.0, 30.0])
    st, _ = sn.build_csr_status(bad, L.pos, 12.0, L.capacity, L.ws)
    assert st == sn.SN_ERR_BOX
    # a non-finite position
    p = cfg["pos"].copy()
    p[7, 1] = np.nan
    st, _ = sn.build_csr_status(L.system, dev(p), 12.0, L.capacity, L.ws)
    assert st == sn.SN_ERR_NONFINITE
    # the workspace still works afterwards
    st, ne = sn.build_csr_status(L.system, L.pos, 12.0, L.capacity, L.ws)
    assert st == sn.SN_OK and ne == len(ref[1])


# ------------------------------------------------------------------ energy and forces

def _compare(E, F, E_ref, F_ref, eps_abs, rp, label):
    e_err = energy_errors(E, E_ref, eps_abs)
    f_err = force_errors(F, F_ref, rp)
    say(f"   {label}: energy max rel err {e_err.max():.2e}  force max rel err {f_err.max():.2e}")
    assert e_err.max() <= E_TOL
    assert f_err.max() <= F_TOL


@pytest.mark.parametrize("name", ["tiny_chain", "single_protein", "dense_box"])
def test_energy_forces_match_oracle(sn, name):
    say(f"[energy/forces] {name}")
    cfg = synth.make_config(name)
    L = Loaded(sn, cfg)
    E, F = L.eval(sn)
    E_ref, F_ref, eps_abs, _ = oracle_full(cfg)
    _compare(E, F, E_ref, F_ref, eps_abs, cfg["replica_ptr"], name)


@pytest.mark.parametrize("name,sample", [("batched_replicas", [0, 31, 63]), ("larger_cg", [0, 15])])
def test_energy_forces_full_size_sampled_replicas(sn, name, sample):
    """Full workload on the GPU (the benchmark's launch configuration); the
    oracle recomputes sampled replicas on their own."""
    say(f"[energy/forces full size] {name} replicas {sample}")
    cfg = synth.make_config(name)
    L = Loaded(sn, cfg)
    E, F = L.eval(sn)
    rp = cfg["replica_ptr"]
    for b in sample:
        E_ref, F_ref, eps_abs = oracle_replica(cfg, b)
        s, e = rp[b], rp[b + 1]
        _compare(E[b:b + 1], F[s:e], np.array([E_ref]), F_ref, np.array([eps_abs]),
                 np.array([0, e - s]), f"replica {b}")


def test_energy_forces_are_deterministic(sn):
    cfg = synth.make_config("batched_replicas", n_replicas=16)
    L = Loaded(sn, cfg)
    csr = L.csr(sn)
    E1, F1 = L.eval(sn, csr)
    E2, F2 = L.eval(sn, csr)
    assert np.array_equal(E1, E2) and np.array_equal(F1, F2)


def test_int16_filter_weights_match_dequantised_oracle(sn):
    say("[int16] batched_replicas x4")
    cfg = synth.make_config("batched_replicas", n_replicas=4)
    Lq = Loaded(sn, cfg, fmt=1)
    Eq, Fq = Lq.eval(sn)
    deq = O.dequantized_params(cfg["params"])
    E_ref, F_ref, eps_abs, _ = oracle_full(cfg, params=deq)
    _compare(Eq, Fq, E_ref, F_ref, eps_abs, cfg["replica_ptr"], "int16 vs dequantised oracle")
    # drift of the 16-bit weights from the fp32 weights (reported, not bounded by the pages)
    E32, F32_, _, _ = oracle_full(cfg)
    say(f"   int16 drift: rel dE {np.abs(E_ref - E32).max() / np.abs(E32).max():.2e}, "
        f"rms dF / rms F {np.sqrt(((F_ref - F32_) ** 2).mean() / (F32_ ** 2).mean()):.2e}")


def test_nonfinite_force_is_flagged(sn):
    cfg = synth.make_config("tiny_chain")
    L = Loaded(sn, cfg)
    p = cfg["pos"].copy()
    p[5] = p[4]                    # a coincident pair: zero distance on an edge
    L.pos = dev(p)
    row_ptr, col, rev, E = L.csr(sn)
    sn.energy_forces(L.model, L.system, L.pos, row_ptr, col, rev, E, L.ws)
    assert sn.read_status(L.ws) == sn.SN_ERR_NONFINITE
    assert sn.read_status(L.ws) == sn.SN_OK      # reading clears it


# ------------------------------------------------------------------ velocity Verlet

@pytest.mark.parametrize("n_steps", [1, 10])
def test_verlet_matches_oracle(sn, n_steps):
    import torch
    say(f"[verlet] {n_steps} steps")
    cfg = synth.make_config("batched_replicas", n_replicas=2)
    L = Loaded(sn, cfg)
    vel = dev(cfg["vel"])
    inv_mass = dev(cfg["inv_mass"])
    row_ptr, col, rev, E = L.csr(sn)
    _, forces = sn.energy_forces(L.model, L.system, L.pos, row_ptr, col, rev, E, L.ws)
    B = 2
    epot = torch.zeros((n_steps, B), dtype=torch.float32, device="cuda")
    ekin = torch.zeros((n_steps, B), dtype=torch.float32, device="cuda")
    sn.verlet_step(L.model, L.system, L.pos, vel, forces, inv_mass, 2.0, synth.FORCE_TO_ACCEL, n_steps, 12.0,
                   L.capacity, L.ws, epot, ekin)
    torch.cuda.synchronize()
    r, v, f, ep, ek = O.verlet(cfg["params"], cfg["hyper"], cfg["types"], cfg["pos"], cfg["vel"],
                               cfg["inv_mass"], cfg["replica_ptr"], 2.0, synth.FORCE_TO_ACCEL, n_steps, 12.0)
    dr = np.abs(L.pos.cpu().numpy() - r).max()
    dv = np.abs(vel.cpu().numpy() - v).max() / np.abs(v).max()
    say(f"   max |dr| {dr:.2e} A, max rel dv {dv:.2e}")
    assert dr < 1e-4
    assert dv < 1e-4
    f_err = force_errors(forces.cpu().numpy(), f, cfg["replica_ptr"])
    assert f_err.max() < 1e-3
    ep_g, ek_g = epot.cpu().numpy(), ekin.cpu().numpy()
    assert np.abs(ep_g - ep).max() <= 1e-5 * np.abs(ep).max() * 10
    assert np.abs(ek_g - ek).max() <= 1e-4 * np.abs(ek).max()
