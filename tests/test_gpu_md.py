"""GPU: velocity-Verlet MD through sn_verlet_step against the oracle.

Each MD state is checked in two ways.  The energy/force evaluation of the
state must meet the contract tolerances against the oracle evaluated at the
GPU's own positions (helpers.md_evaluation_errors); the trajectory itself is
compared with the oracle's fp64 trajectory, from which the GPU's fp32
positions part by rounding, within bounds derived from that rounding.  The
neighbour skin (a list kept across steps at r_list = cutoff + skin) and the
graph replay of a rebuild interval are checked against the per-step rebuild.
"""
import sys

import numpy as np
import pytest

import oracle as O
import synth
from helpers import E_TOL, F_TOL, md_evaluation_errors

pytestmark = pytest.mark.gpu

DT = 2.0
# One 2 fs step moves a bead ~0.005 A; fp32 positions of 10-50 A carry a rounding of
# 0.5-2 ulp (1e-6-4e-6 A) per step, so one step agrees with the oracle's fp64 step to 1e-5 A.
ONE_STEP_DR = 1e-5
# Over ten steps the rounding of each step accumulates, and the force differences it causes
# feed back into the velocities: the observed divergence is 3.5e-6 A (64 x 269 workload) to
# 9e-6 A (a 600-bead box, positions up to 30 A); the bound is twice the larger.
TEN_STEP_DR = 2e-5


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


class MD:
    """A seeded system on the device with F(r0) evaluated, ready for sn_verlet_step."""

    def __init__(self, sn, cfg, fmt=0, capacity=None):
        self.sn, self.cfg = sn, cfg
        self.params = cfg["params"]
        self.hyper = cfg["hyper"]
        self.model = sn.Model(cfg["params"], cfg["hyper"], filter_format=fmt)
        self.system = sn.System(cfg["replica_ptr"], cfg["types"], cfg["box"])
        n = len(cfg["pos"])
        self.capacity = capacity if capacity is not None else max(64, 220 * n)
        self.ws = sn.workspace(self.model, self.system, self.capacity)
        self.reset()

    def reset(self):
        sn, cfg = self.sn, self.cfg
        self.pos = dev(cfg["pos"])
        self.vel = dev(cfg["vel"])
        self.inv_mass = dev(cfg["inv_mass"])
        row_ptr, col, rev, E = sn.build_csr_neighbors(self.system, self.pos, self.hyper["cutoff"], self.capacity,
                                                      self.ws)
        _, self.forces = sn.energy_forces(self.model, self.system, self.pos, row_ptr, col, rev, E, self.ws)

    def run(self, n, r_list=None, rebuild_every=1, graph=False, log_ekin=True):
        """n steps in one call.  Logging the kinetic energy runs each step's opening kick in its own
        launch (after the log); without it the force assembly applies it."""
        import torch
        B = self.system.n_replicas
        epot = torch.zeros((n, B), dtype=torch.float64, device="cuda")
        ekin = torch.zeros((n, B), dtype=torch.float64, device="cuda") if log_ekin else None
        elog = torch.zeros(n, dtype=torch.int32, device="cuda")
        r = self.hyper["cutoff"] if r_list is None else r_list
        csr = self.sn.verlet_step(self.model, self.system, self.pos, self.vel, self.forces, self.inv_mass, DT,
                                  synth.FORCE_TO_ACCEL, n, r, self.capacity, self.ws, epot, ekin, edge_log=elog,
                                  rebuild_every=rebuild_every, graph=graph)
        torch.cuda.synchronize()
        return {"pos": self.pos.cpu().numpy(), "vel": self.vel.cpu().numpy(), "forces": self.forces.cpu().numpy(),
                "epot": epot.cpu().numpy(), "ekin": None if ekin is None else ekin.cpu().numpy(),
                "edges": elog.cpu().numpy(),
                "csr": (csr[0].cpu().numpy(), csr[1].cpu().numpy())}

    def check_state(self, st, label, epot_row=-1):
        c = self.cfg
        e_err, f_err = md_evaluation_errors(self.params, self.hyper, c["types"], c["replica_ptr"], c["box"],
                                            st["pos"], st["forces"], st["epot"][epot_row])
        say(f"   {label}: energy err {e_err.max():.2e}, force err {f_err.max():.2e}")
        assert e_err.max() <= E_TOL
        assert f_err.max() <= F_TOL
        if st["ekin"] is not None:
            ek = O.kinetic_energy(st["vel"], c["inv_mass"], c["replica_ptr"], synth.FORCE_TO_ACCEL)
            assert np.abs(st["ekin"][epot_row] - ek).max() <= 2e-7 * np.abs(ek).max()   # the library takes c as fp32

    def oracle_steps(self, pos, vel, n):
        c = self.cfg
        return O.verlet(self.params, self.hyper, c["types"], pos, vel, c["inv_mass"], c["replica_ptr"], DT,
                        synth.FORCE_TO_ACCEL, n, self.hyper["cutoff"], c["box"])


def _batched(B):
    return synth.make_config("batched_replicas", n_replicas=B)


def _cell_path_cfg():
    """One 600-bead replica (above the 512-atom limit of the mask build: the cell list runs)."""
    pos = synth.box_rsa(600, 30.0, 2.5, synth.seed64(71)).astype(np.float32)
    rp = np.array([0, 600], np.int32)
    params = synth.init_params(3, 2, 64, 12, 17)
    hyper = {"n_types": 3, "n_interactions": 2, "n_features": 64, "n_rbf": 12, "cutoff": 7.0,
             **synth.rbf_hyper(12, 0.0, 7.0)}
    return {"pos": pos, "replica_ptr": rp, "box": None, "params": params, "hyper": hyper,
            "types": np.random.default_rng(3).integers(0, 3, 600).astype(np.int32),
            "vel": synth.maxwell_boltzmann(600, rp, 110.0, 300.0, 5).astype(np.float32),
            "inv_mass": np.full(600, 1.0 / 110.0, np.float32)}


def _same(a, b):
    for k in ("pos", "vel", "forces", "epot", "ekin", "edges"):
        if a[k] is None or b[k] is None:
            assert a[k] is None and b[k] is None, k
        else:
            assert np.array_equal(a[k], b[k]), k


# ------------------------------------------------------------------ contract tolerance

def test_one_step_meets_the_contract_tolerances(sn):
    say("[md] one step, 4 x 269 beads")
    md = MD(sn, _batched(4))
    st = md.run(1)
    md.check_state(st, "step 1")
    r_ref, v_ref, _, _, _ = md.oracle_steps(md.cfg["pos"], md.cfg["vel"], 1)
    dr = np.abs(st["pos"] - r_ref).max()
    dv = np.abs(st["vel"] - v_ref).max() / np.abs(v_ref).max()
    say(f"   |dr| {dr:.2e} A, rel |dv| {dv:.2e}")
    assert dr <= ONE_STEP_DR
    assert dv <= 1e-5


def test_ten_steps_track_the_oracle_step_by_step(sn):
    """Ten one-step calls and one ten-step call give the same bits; every state meets the contract
    against the oracle at its positions; each step matches the oracle's step taken from the GPU's
    previous state; the whole trajectory stays within the accumulated rounding of the oracle's."""
    say("[md] ten steps, 2 x 269 beads")
    md = MD(sn, _batched(2))
    states = [md.run(1) for _ in range(10)]
    md.reset()
    whole = md.run(10)
    for k in ("pos", "vel", "forces"):
        assert np.array_equal(whole[k], states[-1][k]), k
    assert np.array_equal(whole["epot"], np.concatenate([s["epot"] for s in states]))
    # without the kinetic log the force assembly applies each next opening kick itself
    md.reset()
    fused = md.run(10, log_ekin=False)
    for k in ("pos", "vel", "forces", "epot"):
        assert np.array_equal(fused[k], whole[k]), k
    prev_pos, prev_vel = md.cfg["pos"], md.cfg["vel"]
    worst = 0.0
    for k, st in enumerate(states):
        md.check_state(st, f"step {k + 1}")
        r1, v1, _, _, _ = md.oracle_steps(prev_pos, prev_vel, 1)
        worst = max(worst, np.abs(st["pos"] - r1).max())
        prev_pos, prev_vel = st["pos"], st["vel"]
    say(f"   worst one-step |dr| {worst:.2e} A")
    assert worst <= ONE_STEP_DR
    r_ref, _, _, _, _ = md.oracle_steps(md.cfg["pos"], md.cfg["vel"], 10)
    dr = np.abs(whole["pos"] - r_ref).max()
    say(f"   ten-step |dr| against the oracle's trajectory {dr:.2e} A")
    assert dr <= TEN_STEP_DR


# ------------------------------------------------------------------ graph replay

@pytest.mark.parametrize("path", ["mask", "cell"])
@pytest.mark.parametrize("log_ekin", [False, True])
def test_graph_replay_is_bit_identical(sn, path, log_ekin):
    """12 steps recorded as a 10-step graph replayed once plus two ordinary steps, against 12
    ordinary steps: the same bits in positions, velocities, forces and every log."""
    say(f"[md graph] {path} path, kinetic log {log_ekin}")
    cfg = _batched(4) if path == "mask" else _cell_path_cfg()
    md = MD(sn, cfg)
    plain = md.run(12, log_ekin=log_ekin)
    md.reset()
    replayed = md.run(12, graph=True, log_ekin=log_ekin)
    _same(plain, replayed)
    md.check_state(replayed, "graph, step 12")


# ------------------------------------------------------------------ neighbour skin

@pytest.mark.parametrize("path", ["mask", "cell", "periodic"])
@pytest.mark.parametrize("rebuild_every", [0, 4])
def test_skin_matches_the_oracle(sn, path, rebuild_every):
    """A list built at cutoff + 1 A and kept across steps (rebuilt every 4 steps, or only on
    displacement): states meet the contract at their positions and the trajectory matches both the
    oracle's (rebuilt every step at the cutoff) and the per-step rebuild's; with the graph the same
    bits again.  "periodic": the cell-list system in a periodic 30 A box (the kept pairs' geometry
    is refreshed with the minimum image)."""
    say(f"[md skin] {path} path, rebuild_every={rebuild_every}")
    if path == "mask":
        cfg = _batched(4)
    else:
        cfg = _cell_path_cfg()
        if path == "periodic":
            cfg["box"] = np.array([30.0, 30.0, 30.0], np.float32)
    rc = cfg["hyper"]["cutoff"]
    md = MD(sn, cfg)
    every = md.run(10, log_ekin=False)
    md.reset()
    kept = md.run(10, r_list=rc + 1.0, rebuild_every=rebuild_every, log_ekin=False)
    md.check_state(kept, "skin, step 10")
    edges = kept["edges"]
    say(f"   edge counts per step {edges.tolist()}")
    # the list changes only at rebuilds: never for rebuild_every = 0 (no atom moves 0.5 A in 20 fs),
    # at steps 4 and 8 otherwise
    for k in range(1, 10):
        if rebuild_every == 0 or k % rebuild_every != 0:
            assert edges[k] == edges[0 if rebuild_every == 0 else k - 1], k
    assert edges[0] > every["edges"][0]          # the skin adds pairs
    dr_every = np.abs(kept["pos"] - every["pos"]).max()
    r_ref, _, _, _, _ = md.oracle_steps(cfg["pos"], cfg["vel"], 10)
    dr_ref = np.abs(kept["pos"] - r_ref).max()
    say(f"   |dr| against the per-step rebuild {dr_every:.2e} A, against the oracle {dr_ref:.2e} A")
    assert dr_every <= TEN_STEP_DR and dr_ref <= TEN_STEP_DR
    md.reset()
    replayed = md.run(10, r_list=rc + 1.0, rebuild_every=rebuild_every, graph=True, log_ekin=False)
    _same(kept, replayed)
    # the returned list (built at cutoff + skin from positions within skin/2 of the final ones)
    # holds every pair within the cutoff at the final positions
    row_ptr, col = kept["csr"]
    ref = O.neighbors_bruteforce(kept["pos"], cfg["replica_ptr"], rc, cfg["box"])
    got = set(zip(np.repeat(np.arange(len(row_ptr) - 1), np.diff(row_ptr)).tolist(), col.tolist()))
    want = set(zip(np.repeat(np.arange(len(ref[0]) - 1), np.diff(ref[0])).tolist(), ref[1].tolist()))
    assert want <= got


def test_zero_skin_rebuilds_every_step_with_the_same_bits(sn):
    """r_list = cutoff and no schedule: any motion exceeds half of a zero skin, so every step
    rebuilds, and the device-driven steps reproduce the host-driven ones bit for bit."""
    say("[md skin] zero skin")
    cfg = _batched(2)
    md = MD(sn, cfg)
    for log_ekin in (False, True):
        md.reset()
        plain = md.run(6, log_ekin=log_ekin)
        md.reset()
        _same(plain, md.run(6, r_list=cfg["hyper"]["cutoff"], rebuild_every=0, log_ekin=log_ekin))


def test_small_skin_rebuilds_on_displacement(sn):
    """A skin of 0.02 A is crossed within a few steps: the displacement check must trigger the
    rebuilds (the list changes without a schedule) and the states still meet the contract."""
    say("[md skin] displacement-triggered rebuilds")
    cfg = _batched(2)
    md = MD(sn, cfg)
    st = md.run(12, r_list=cfg["hyper"]["cutoff"] + 0.02, rebuild_every=0)
    say(f"   edge counts per step {st['edges'].tolist()}")
    assert len(set(st["edges"].tolist())) > 1
    md.check_state(st, "small skin, step 12")
    r_ref, _, _, _, _ = md.oracle_steps(cfg["pos"], cfg["vel"], 12)
    assert np.abs(st["pos"] - r_ref).max() <= TEN_STEP_DR


# ------------------------------------------------------------------ energy conservation

def test_md_100_steps_energy_drift_fp32_and_int16_weights(sn):
    """100 NVE steps of 2 fs on 8 x 269 beads with fp32 and with int16 filter weights.  The total
    energy (fp64 logs) is conserved to the integrator's accuracy; the drift of the int16 run from the
    fp32 run (relative energy, RMS force, total-energy trace) is reported."""
    say("[md drift] 100 steps, 8 x 269 beads")
    cfg = _batched(8)
    out = {}
    for fmt in (0, 1):
        md = MD(sn, cfg, fmt=fmt)
        st = md.run(100)
        tot = st["epot"] + st["ekin"]
        drift = np.abs(tot - tot[0]).max(axis=0)
        rel = drift / st["ekin"].mean(axis=0)
        say(f"   fmt={fmt}: max |E_tot(t) - E_tot(0)| {drift.max():.3e} kcal/mol "
            f"({rel.max():.2e} of the mean kinetic energy)")
        assert np.all(np.isfinite(tot))
        # bound near the observed size (about 3e-6 of the kinetic energy)
        assert rel.max() < 2e-5
        out[fmt] = (st, tot)
    d_tot = np.abs(out[1][1] - out[0][1]).max()
    say(f"   int16 - fp32: max |E_tot difference| over 100 steps {d_tot:.3e} kcal/mol")
