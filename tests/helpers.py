"""Shared helpers of the test-suite: tolerances and oracle/library plumbing."""
import numpy as np

import oracle as O
import synth

# fp32 path against the fp64 oracle (tolerances of the spec contract):
#   energy  |dE_b|  <= 1e-5 * max(|E_b|, sum_i |eps_i|)
#   forces  |dF_ic| <= 1e-4 * max(|F_ic|, RMS of F over the replica)
E_TOL = 1e-5
F_TOL = 1e-4


def energy_errors(E_gpu, E_ref, eps_abs_sum):
    scale = np.maximum(np.abs(E_ref), eps_abs_sum)
    return np.abs(np.asarray(E_gpu, np.float64) - E_ref) / scale


def force_errors(F_gpu, F_ref, replica_ptr):
    F_gpu = np.asarray(F_gpu, np.float64)
    err = np.zeros_like(F_ref)
    for b in range(len(replica_ptr) - 1):
        s, e = replica_ptr[b], replica_ptr[b + 1]
        if e == s:
            continue
        rms = np.sqrt((F_ref[s:e] ** 2).mean())
        scale = np.maximum(np.abs(F_ref[s:e]), rms)
        err[s:e] = np.abs(F_gpu[s:e] - F_ref[s:e]) / scale
    return err


def oracle_replica(cfg, b, params=None):
    """Oracle energy, forces and sum|eps| of replica b of a workload, alone."""
    rp = cfg["replica_ptr"]
    s, e = int(rp[b]), int(rp[b + 1])
    pos = cfg["pos"][s:e]
    types = cfg["types"][s:e]
    sub_rp = np.array([0, e - s], np.int32)
    box = cfg["box"]
    csr = O.neighbors_bruteforce(pos, sub_rp, cfg["hyper"]["cutoff"], box)
    E, F, inter = O.energy_forces(params or cfg["params"], cfg["hyper"], types, pos, sub_rp, csr, box,
                                  return_intermediates=True)
    return E[0], F, np.abs(inter["eps"]).sum()


def oracle_full(cfg, params=None):
    csr = O.neighbors_bruteforce(cfg["pos"], cfg["replica_ptr"], cfg["hyper"]["cutoff"], cfg["box"])
    E, F, inter = O.energy_forces(params or cfg["params"], cfg["hyper"], cfg["types"], cfg["pos"],
                                  cfg["replica_ptr"], csr, cfg["box"], return_intermediates=True)
    rp = cfg["replica_ptr"]
    eps_abs = np.array([np.abs(inter["eps"][rp[b]:rp[b + 1]]).sum() for b in range(len(rp) - 1)])
    return E, F, eps_abs, csr


def md_evaluation_errors(cfg_params, hyper, types, replica_ptr, box, pos_gpu, forces_gpu, epot_gpu):
    """Energy and force errors of an MD state against the oracle evaluated at the GPU's own positions.

    The GPU carries positions in fp32 and the oracle's trajectory in fp64, so their trajectories part
    by rounding; evaluating the oracle at the GPU's positions separates the energy/force evaluation,
    which must meet the contract tolerances, from that divergence.  Returns the per-replica energy
    errors and the per-component force errors (both relative, as energy_errors / force_errors)."""
    pos = np.asarray(pos_gpu, np.float32)
    csr = O.neighbors_bruteforce(pos, replica_ptr, hyper["cutoff"], box)
    E, F, inter = O.energy_forces(cfg_params, hyper, types, pos.astype(np.float64), replica_ptr, csr, box,
                                  return_intermediates=True)
    rp = replica_ptr
    eps_abs = np.array([np.abs(inter["eps"][rp[b]:rp[b + 1]]).sum() for b in range(len(rp) - 1)])
    return energy_errors(epot_gpu, E, eps_abs), force_errors(forces_gpu, F, rp)
