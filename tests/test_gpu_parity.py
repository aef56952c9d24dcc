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
    system = sn.System(cfg["replica_ptr"], cfg["types"], cfg["box"])
    ws = sn.workspace(model, system, 64)
    rng = np.random.default_rng(5)
    d = np.concatenate([np.linspace(0.05, h["cutoff"] * 1.1, 997), rng.uniform(0, h["cutoff"], 1003)])
    d = d.astype(np.float32)       # 2000 values: several tiles plus a ragged one
    params = O.dequantized_params(cfg["params"]) if fmt == 1 else cfg["params"]
    for t in range(h["n_interactions"]):
        phi = sn.filter_forward(model, t, dev(d), ws).cpu().numpy().astype(np.float64)
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


@pytest.mark.parametrize("name", ["batched_replicas", "larger_cg"])
def test_energy_forces_full_size_every_replica(sn, name):
    """Full workload on the GPU, in the benchmark's launch configuration; the oracle recomputes
    every replica on its own (replicas are independent, so this is the whole workload's answer)."""
    cfg = synth.make_config(name)
    rp = cfg["replica_ptr"]
    B = len(rp) - 1
    say(f"[energy/forces full size] {name}: all {B} replicas")
    L = Loaded(sn, cfg)
    E, F = L.eval(sn)
    e_worst = f_worst = 0.0
    for b in range(B):
        E_ref, F_ref, eps_abs = oracle_replica(cfg, b)
        s, e = rp[b], rp[b + 1]
        e_err = energy_errors(E[b:b + 1], np.array([E_ref]), np.array([eps_abs])).max()
        f_err = force_errors(F[s:e], F_ref, np.array([0, e - s])).max()
        e_worst, f_worst = max(e_worst, e_err), max(f_worst, f_err)
        assert e_err <= E_TOL, (b, e_err)
        assert f_err <= F_TOL, (b, f_err)
    say(f"   worst over {B} replicas: energy {e_worst:.2e}, force {f_worst:.2e}")


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


# ------------------------------------------------------------------ more shapes and edge cases

def _random_system(n_rep, n_per, box_side, seed, min_d=3.0):
    """n_rep replicas of n_per particles placed by the seeded box generator (open boundaries)."""
    pos = np.concatenate([synth.box_rsa(n_per, box_side, min_d, synth.seed64(seed, b)) for b in range(n_rep)])
    rp = np.arange(0, n_rep * n_per + 1, n_per, dtype=np.int32)
    return pos.astype(np.float32), rp


@pytest.mark.parametrize("F,K,I,T", [(64, 64, 1, 3), (32, 2, 2, 2), (64, 33, 2, 4), (128, 7, 1, 2)])
def test_energy_forces_other_model_shapes(sn, F, K, I, T):
    """Every supported feature width and edge values of the basis size, against the oracle."""
    say(f"[shapes] F={F} K={K} I={I} T={T}")
    pos, rp = _random_system(3, 90, 18.0, 1000 + F + K)
    rc = 7.0
    cfg = {"pos": pos, "replica_ptr": rp, "box": None,
           "types": np.random.default_rng(F * K).integers(0, T, len(pos)).astype(np.int32),
           "params": synth.init_params(T, I, F, K, [F, K, I]),
           "hyper": {"n_types": T, "n_interactions": I, "n_features": F, "n_rbf": K, "cutoff": rc,
                     **synth.rbf_hyper(K, 0.0, rc)}}
    L = Loaded(sn, cfg)
    E, Fo = L.eval(sn)
    E_ref, F_ref, eps_abs, csr = oracle_full(cfg)
    assert len(csr[1]) > 100
    _compare(E, Fo, E_ref, F_ref, eps_abs, rp, f"F={F} K={K}")


@pytest.mark.parametrize("I", [8, 9, 16])
def test_energy_forces_interaction_counts(sn, I):
    """Small systems run every interaction's filter in one launch up to 8 interactions (each
    writing its own slice of the per-pair force scalar, summed by the force assembly) and one
    launch per interaction beyond; 16 is the largest count the library takes.  Against the
    oracle either way."""
    say(f"[interaction counts] I={I}")
    pos, rp = _random_system(3, 90, 18.0, 3000 + I)
    rc, F, K, T = 7.0, 32, 8, 3
    cfg = {"pos": pos, "replica_ptr": rp, "box": None,
           "types": np.random.default_rng(I).integers(0, T, len(pos)).astype(np.int32),
           "params": synth.init_params(T, I, F, K, [F, K, I, 7]),
           "hyper": {"n_types": T, "n_interactions": I, "n_features": F, "n_rbf": K, "cutoff": rc,
                     **synth.rbf_hyper(K, 0.0, rc)}}
    L = Loaded(sn, cfg)
    E, Fo = L.eval(sn)
    E_ref, F_ref, eps_abs, csr = oracle_full(cfg)
    assert len(csr[1]) > 100
    _compare(E, Fo, E_ref, F_ref, eps_abs, rp, f"I={I}")


@pytest.mark.parametrize("F,K,I,T,n_rep", [(32, 16, 2, 4, 56), (64, 33, 2, 4, 100), (64, 16, 1, 3, 60),
                                           (128, 50, 2, 5, 150), (32, 16, 2, 4, 190)])
def test_energy_forces_atomwise_block_sizes(sn, F, K, I, T, n_rep):
    """Systems of 5,040 to 17,100 atoms, so that the atom-wise layers run with every number of
    16-atom tiles per block (one to five, chosen from the tile count and 256 compute units), each
    with a ragged last block, for every feature width; every replica against the oracle."""
    say(f"[atom-wise block sizes] F={F} K={K} I={I} T={T} replicas={n_rep}")
    pos, rp = _random_system(n_rep, 90, 18.0, 2000 + F + n_rep)
    rc = 7.0
    cfg = {"pos": pos, "replica_ptr": rp, "box": None,
           "types": np.random.default_rng(F + n_rep).integers(0, T, len(pos)).astype(np.int32),
           "params": synth.init_params(T, I, F, K, [F, K, I, n_rep]),
           "hyper": {"n_types": T, "n_interactions": I, "n_features": F, "n_rbf": K, "cutoff": rc,
                     **synth.rbf_hyper(K, 0.0, rc)}}
    L = Loaded(sn, cfg)
    E, Fo = L.eval(sn)
    E_ref, F_ref, eps_abs, csr = oracle_full(cfg)
    assert len(csr[1]) > 8 * len(pos)
    _compare(E, Fo, E_ref, F_ref, eps_abs, rp, f"F={F} replicas={n_rep}")


def test_energy_forces_with_saturated_first_layer(sn):
    """Half of the first layer's features pushed to a ~ -60, where the sigmoid and softplus are
    below 1e-26 (the backward filter caps its exponent there, below a = -44): energies and forces
    still match the oracle."""
    say("[saturated first layer] tiny_chain, b1 - 60 on even features")
    base = synth.make_config("tiny_chain")
    F = base["hyper"]["n_features"]
    shift = np.where(np.arange(F) % 2 == 0, -60.0, 0.0)
    blocks = [dict(blk, b1=(blk["b1"] + shift).astype(np.float32)) for blk in base["params"]["interactions"]]
    cfg = dict(base, params=dict(base["params"], interactions=blocks))
    L = Loaded(sn, cfg)
    E, Fo = L.eval(sn)
    E_ref, F_ref, eps_abs, _ = oracle_full(cfg)
    assert np.all(np.isfinite(E)) and np.all(np.isfinite(Fo))
    _compare(E, Fo, E_ref, F_ref, eps_abs, cfg["replica_ptr"], "saturated first layer")


def test_graph_without_edges_and_single_atom_replicas(sn):
    """No pair within the cutoff: forces are exactly zero and the energy is the readout of the
    atom-wise layers alone; replicas of one atom and of zero atoms are allowed."""
    params = synth.init_params(3, 2, 32, 8, 5)
    hyper = {"n_types": 3, "n_interactions": 2, "n_features": 32, "n_rbf": 8, "cutoff": 5.0,
             **synth.rbf_hyper(8, 0.0, 5.0)}
    pos = np.array([[0, 0, 0], [10, 0, 0], [0, 10, 0], [3, 3, 3], [50, 50, 50]], np.float32)
    rp = np.array([0, 3, 3, 4, 5], np.int32)
    cfg = {"pos": pos, "replica_ptr": rp, "types": np.array([0, 1, 2, 1, 0], np.int32), "box": None,
           "params": params, "hyper": hyper}
    L = Loaded(sn, cfg)
    row_ptr, col, rev, E = L.csr(sn)
    assert E == 0
    en, f = L.eval(sn, (row_ptr, col, rev, E))
    assert np.all(f == 0.0)
    E_ref, _, eps_abs, _ = oracle_full(cfg)
    assert en[1] == 0.0                       # the empty replica
    assert np.all(energy_errors(en, E_ref, np.maximum(eps_abs, 1e-30)) <= E_TOL)


def test_list_radius_beyond_cutoff_changes_nothing(sn):
    """Pairs between the cutoff and the list radius carry a zero envelope."""
    cfg = synth.make_config("batched_replicas", n_replicas=4)
    L = Loaded(sn, cfg)
    E1, F1 = L.eval(sn, L.csr(sn))
    E2, F2 = L.eval(sn, L.csr(sn, r_list=13.5))
    assert np.abs(E1 - E2).max() <= 1e-6 * np.abs(E1).max()
    assert np.abs(F1 - F2).max() <= 1e-5 * np.abs(F1).max()


def test_verlet_is_deterministic_and_reports_capacity(sn):
    import torch
    cfg = synth.make_config("batched_replicas", n_replicas=4)
    runs = []
    for _ in range(2):
        L = Loaded(sn, cfg)
        vel, inv_mass = dev(cfg["vel"]), dev(cfg["inv_mass"])
        row_ptr, col, rev, E = L.csr(sn)
        _, forces = sn.energy_forces(L.model, L.system, L.pos, row_ptr, col, rev, E, L.ws)
        elog = torch.zeros(10, dtype=torch.int32, device="cuda")
        rp, _, _, ne = sn.verlet_step(L.model, L.system, L.pos, vel, forces, inv_mass, 2.0, synth.FORCE_TO_ACCEL,
                                      10, 12.0, L.capacity, L.ws, edge_log=elog)
        torch.cuda.synchronize()
        # the per-step edge log ends with the edge count of the returned list
        el = elog.cpu().numpy()
        assert el[-1] == ne == int(rp[-1].item()) and np.all(el > 0)
        runs.append((L.pos.cpu().numpy(), vel.cpu().numpy(), forces.cpu().numpy()))
    for a, b in zip(runs[0], runs[1]):
        assert np.array_equal(a, b)
    # a capacity that the first rebuild already exceeds
    L = Loaded(sn, cfg, capacity=1000)
    vel, inv_mass = dev(cfg["vel"]), dev(cfg["inv_mass"])
    forces = torch.zeros_like(L.pos)
    with pytest.raises(sn.SnError) as exc:
        sn.verlet_step(L.model, L.system, L.pos, vel, forces, inv_mass, 2.0, synth.FORCE_TO_ACCEL, 3, 12.0,
                       L.capacity, L.ws)
    assert exc.value.status == sn.SN_ERR_CAPACITY and exc.value.steps_done == 0
    assert exc.value.n_edges > 1000
