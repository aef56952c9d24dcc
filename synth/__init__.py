"""Seeded synthetic inputs for the SchNet CFConv energy/force path.

This module only builds inputs: coarse-grained bead chains, a periodic
particle box, bead types, random-init model weights and Maxwell-Boltzmann
velocities.  It holds none of the potential's arithmetic and is shared by
the tests, the benchmark and the CPU oracle's callers alike.

The measured systems of the FlashSchNet pages (a 269-bead CG model of the
1ENH protein, and the 15,668-atom 1HCI benchmark of the GROMACS/DeePMD
page) are not available here; the configurations below are seeded stand-ins
with the same sizes, densities and neighbour statistics.
"""
from __future__ import annotations

import ctypes
import functools
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "_chaingen.so")
_SRC = os.path.join(_HERE, "chaingen.c")


def build(force: bool = False) -> str:
    """Compile the C coordinate generator with gcc (in-tree)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _SO)
    return _SO


@functools.lru_cache(maxsize=1)
def _lib():
    lib = ctypes.CDLL(build())
    dp = ctypes.POINTER(ctypes.c_double)
    lib.synth_grow_chain.argtypes = [ctypes.c_int, ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                     ctypes.c_uint64, ctypes.c_int, ctypes.c_int, ctypes.c_int64, dp]
    lib.synth_grow_chain.restype = ctypes.c_int
    lib.synth_compact_chain.argtypes = [ctypes.c_int, ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                        ctypes.c_int64, ctypes.c_uint64, dp, dp]
    lib.synth_compact_chain.restype = ctypes.c_int64
    lib.synth_box_rsa.argtypes = [ctypes.c_int, ctypes.c_double, ctypes.c_double, ctypes.c_uint64,
                                  ctypes.c_int64, dp]
    lib.synth_box_rsa.restype = ctypes.c_int
    return lib


def _dptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


BOND = 3.8        # Å, CG bond length
EXCL = 4.0        # Å, hard core between non-bonded beads (|i-j| >= 2)
KB_KCAL = 0.0019872041   # kcal/mol/K
FORCE_TO_ACCEL = 4.184e-4  # (kcal/mol/Å)/Da -> Å/fs^2


def seed64(*entropy) -> int:
    """64-bit seed for the C generator, derived through numpy's SeedSequence."""
    return int(np.random.SeedSequence(list(entropy)).generate_state(1, np.uint64)[0])


def grow_chain(n: int, seed: int, r_conf: float = 0.0) -> np.ndarray:
    pos = np.zeros((n, 3), np.float64)
    rc = _lib().synth_grow_chain(n, BOND, EXCL, float(r_conf), seed, 200, 4, 200_000_000, _dptr(pos))
    if rc != 0:
        raise RuntimeError(f"chain growth failed (n={n}, r_conf={r_conf})")
    return pos


def compact_chain(pos: np.ndarray, rg_target: float, max_moves: int, seed: int):
    pos = np.ascontiguousarray(pos, np.float64).copy()
    rg = ctypes.c_double(0.0)
    moves = _lib().synth_compact_chain(pos.shape[0], BOND, EXCL, float(rg_target), int(max_moves), seed,
                                       _dptr(pos), ctypes.byref(rg))
    return pos, float(rg.value), int(moves)


def box_rsa(n: int, L: float, dmin: float, seed: int) -> np.ndarray:
    pos = np.zeros((n, 3), np.float64)
    rc = _lib().synth_box_rsa(n, float(L), float(dmin), seed, 1_000_000_000, _dptr(pos))
    if rc != 0:
        raise RuntimeError("random sequential addition ran out of trials")
    return pos


def morton_order(pos: np.ndarray, L: float, cell: float) -> np.ndarray:
    """Permutation that numbers particles of a periodic box along a Morton (Z-order) curve of
    cells of edge >= `cell`, ties in their existing order: the spatial numbering MD engines keep
    their atoms in, so that neighbours have nearby indices.  Random sequential addition numbers
    the particles in the random order they were placed."""
    m = max(1, int(np.floor(L / cell)))
    c = np.clip(np.floor(np.mod(pos, L) * (m / L)).astype(np.int64), 0, m - 1)
    code = np.zeros(len(pos), np.int64)
    for bit in range(int(np.ceil(np.log2(m))) + 1):
        for axis in range(3):
            code |= ((c[:, axis] >> bit) & 1) << (3 * bit + axis)
    return np.argsort(code, kind="stable")


def radius_of_gyration(pos: np.ndarray) -> float:
    c = pos - pos.mean(axis=0)
    return float(np.sqrt((c * c).sum(axis=1).mean()))


# ---------------------------------------------------------------------------
# model weights
# ---------------------------------------------------------------------------

INTERACTION_KEYS = ("W_in", "A1", "b1", "A2", "b2", "Wo1", "bo1", "Wo2", "bo2")


def init_params(n_types: int, n_interactions: int, n_features: int, n_rbf: int, seed) -> dict:
    """Random-init weights: every matrix and bias ~ N(0, 1/fan_in), embeddings ~ N(0, 1).

    Row-vector convention: a layer maps x[in] to x @ W[in, out] + b[out].
    Draw order is fixed (embedding, then each interaction in INTERACTION_KEYS
    order, then the readout) so that a seed fixes every value.  All arrays are
    float32.
    """
    rng = np.random.default_rng(seed)
    T, I, F, K = n_types, n_interactions, n_features, n_rbf
    H = F // 2

    def nrm(shape, fan_in):
        return (rng.standard_normal(shape) / np.sqrt(fan_in)).astype(np.float32)

    p = {"emb": rng.standard_normal((T, F)).astype(np.float32), "interactions": []}
    for _ in range(I):
        blk = {}
        blk["W_in"] = nrm((F, F), F)
        blk["A1"] = nrm((K, F), K)
        blk["b1"] = nrm((F,), K)
        blk["A2"] = nrm((F, F), F)
        blk["b2"] = nrm((F,), F)
        blk["Wo1"] = nrm((F, F), F)
        blk["bo1"] = nrm((F,), F)
        blk["Wo2"] = nrm((F, F), F)
        blk["bo2"] = nrm((F,), F)
        p["interactions"].append(blk)
    p["R1"] = nrm((F, H), F)
    p["c1"] = nrm((H,), F)
    p["R2"] = nrm((H,), H)
    p["c2"] = nrm((), H).reshape(())
    return p


def rbf_hyper(n_rbf: int, lo: float, hi: float) -> dict:
    """Gaussian centres linspace(lo, hi, K) with width gamma = 1 / (2 dmu^2)."""
    dmu = (hi - lo) / (n_rbf - 1)
    return {"rbf_lo": float(np.float32(lo)), "rbf_hi": float(np.float32(hi)),
            "rbf_gamma": float(np.float32(1.0 / (2.0 * dmu * dmu)))}


def maxwell_boltzmann(n_atoms: int, replica_ptr: np.ndarray, mass: float, temperature: float, seed) -> np.ndarray:
    """Velocities (Å/fs) at `temperature` K for beads of `mass` Da, per-replica COM motion removed."""
    rng = np.random.default_rng(seed)
    sigma = np.sqrt(FORCE_TO_ACCEL * KB_KCAL * temperature / mass)
    v = rng.standard_normal((n_atoms, 3)) * sigma
    for b in range(len(replica_ptr) - 1):
        s, e = replica_ptr[b], replica_ptr[b + 1]
        if e > s:
            v[s:e] -= v[s:e].mean(axis=0)
    return v.astype(np.float32)


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------

CONFIG_NAMES = ("tiny_chain", "single_protein", "batched_replicas", "larger_cg", "dense_box")
# the periodic box with its particles in the order random sequential addition placed them
EXTRA_CONFIG_NAMES = ("dense_box_random_order",)


def _compact_protein_chain(n: int, seed: int, r_conf: float, rg_target: float, moves: int):
    p = grow_chain(n, seed, r_conf)
    p, rg, _ = compact_chain(p, rg_target, moves, seed ^ 0x5DEECE66D)
    p -= p.mean(axis=0)
    return p, rg


def _parallel(fn, seeds):
    """Run independent chain builds on a few threads (the C calls release the GIL)."""
    from concurrent.futures import ThreadPoolExecutor
    workers = max(1, min(16, os.cpu_count() or 1, len(seeds)))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(fn, seeds))


@functools.lru_cache(maxsize=16)
def _chain_set(kind: str, count: int):
    """Positions and achieved Rg for the chains of a workload (cached per process)."""
    out = []
    if kind == "tiny":
        p = grow_chain(32, seed64(0), 0.0)
        out.append((p - p.mean(axis=0), radius_of_gyration(p)))
    elif kind == "protein1":
        out.append(_compact_protein_chain(269, seed64(1), 20.0, 12.0, 600_000))
    elif kind == "protein64":
        seeds = [int(ss.generate_state(1, np.uint64)[0]) for ss in np.random.SeedSequence(2).spawn(count)]
        out = _parallel(lambda s: _compact_protein_chain(269, s, 20.0, 12.0, 600_000), seeds)
    elif kind == "cg1000":
        seeds = [int(ss.generate_state(1, np.uint64)[0]) for ss in np.random.SeedSequence(3).spawn(count)]
        out = _parallel(lambda s: _compact_protein_chain(1000, s, 32.0, 20.0, 1_500_000), seeds)
    else:
        raise KeyError(kind)
    return tuple(out)


def make_config(name: str, n_replicas: int | None = None) -> dict:
    """Build one of the five seeded workloads.

    `n_replicas` keeps only the first replicas of a batched workload; each
    kept replica is identical to the same replica of the full workload.

    Returns a dict with float32 positions [N,3], int32 types [N], int32
    replica_ptr [B+1], box (float32[3] or None), the model hyper-parameters
    and the named float32 weights (see init_params).
    """
    box = None
    extra = {}
    if name == "tiny_chain":
        chains = _chain_set("tiny", 1)
        T, I, F, K, rc, lo, hi = 8, 2, 32, 16, 10.0, 0.0, 10.0
        types = np.random.default_rng([0, 1]).integers(0, T, 32)
        params = init_params(T, I, F, K, [0, 2])
        per_chain_types = [types]
    elif name in ("single_protein", "batched_replicas"):
        T, I, F, K, rc, lo, hi = 20, 3, 128, 50, 12.0, 0.0, 12.0
        types = np.random.default_rng([1, 1]).integers(0, T, 269)
        params = init_params(T, I, F, K, [1, 2])
        if name == "single_protein":
            chains = _chain_set("protein1", 1)
        else:
            B = 64 if n_replicas is None else n_replicas
            chains = _chain_set("protein64", 64)[:B] if B <= 64 else _chain_set("protein64", B)
            extra = {"mass": 110.0, "dt_fs": 2.0, "n_md_steps": 100, "temperature": 300.0}
        per_chain_types = [types] * len(chains)
    elif name == "larger_cg":
        T, I, F, K, rc, lo, hi = 20, 5, 128, 50, 12.0, 0.0, 12.0
        B = 16 if n_replicas is None else n_replicas
        chains = _chain_set("cg1000", 16)[:B] if B <= 16 else _chain_set("cg1000", B)
        trng = np.random.default_rng([3, 1])
        per_chain_types = [trng.integers(0, T, 1000) for _ in range(16)][:len(chains)]
        params = init_params(T, I, F, K, [3, 2])
    elif name in ("dense_box", "dense_box_random_order"):
        T, I, F, K, rc, lo, hi = 4, 3, 128, 32, 6.0, 0.0, 6.0
        n = 15668
        L = (n / 0.1) ** (1.0 / 3.0)
        p = box_rsa(n, L, 1.0, seed64(4))
        if name == "dense_box":
            p = p[morton_order(p, L, rc)]
        chains = ((p, float("nan")),)
        per_chain_types = [np.random.default_rng([4, 1]).integers(0, T, n)]
        params = init_params(T, I, F, K, [4, 2])
        box = np.full(3, L, np.float32)
    else:
        raise KeyError(name)

    pos = np.concatenate([c[0] for c in chains]).astype(np.float32)
    types = np.concatenate(per_chain_types).astype(np.int32)
    counts = [len(c[0]) for c in chains]
    replica_ptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    hyper = {"n_types": T, "n_interactions": I, "n_features": F, "n_rbf": K,
             "cutoff": float(np.float32(rc)), **rbf_hyper(K, lo, hi)}
    cfg = {"name": name, "pos": pos, "types": types, "replica_ptr": replica_ptr, "box": box,
           "hyper": hyper, "params": params, "rg": [c[1] for c in chains], **extra}
    if "mass" in extra:
        cfg["vel"] = maxwell_boltzmann(len(pos), replica_ptr, extra["mass"], extra["temperature"], 2)
        cfg["inv_mass"] = np.full(len(pos), 1.0 / extra["mass"], np.float32)
    return cfg
