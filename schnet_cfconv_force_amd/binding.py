"""ctypes binding of libsn.so (include/sn.h).

Argument marshalling only: every stage of the energy/force path runs in the
HIP library.  PyTorch supplies device memory and the current stream.  If the
compiled library is missing, loading fails loudly; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsn.so")

SN_OK = 0
SN_ERR_INVALID = -1
SN_ERR_CAPACITY = -2
SN_ERR_BOX = -3
SN_ERR_HIP = -4
SN_ERR_NONFINITE = -5
SN_ERR_WORKSPACE = -6
SN_ERR_ROW = -7
SN_MAX_ROW = 2048
SN_MD_GRAPH = 1

EXPORTED = (
    "sn_param_count", "sn_param_offsets", "sn_quantize_filter_weights", "sn_workspace_bytes",
    "sn_status_string", "sn_version", "sn_build_csr_neighbors", "sn_energy_forces", "sn_verlet_step",
    "sn_filter_forward", "sn_read_status", "sn_profile_enable", "sn_profile_classes", "sn_profile_name",
    "sn_profile_collect", "sn_energy_forces_static",
)
SN_STATIC_SCRATCH_BYTES = 64 << 20


class SnSystem(ctypes.Structure):
    _fields_ = [("n_atoms", ctypes.c_int32), ("n_replicas", ctypes.c_int32),
                ("replica_ptr", ctypes.c_void_p), ("types", ctypes.c_void_p),
                ("periodic", ctypes.c_int32), ("box", ctypes.c_float * 3)]


class SnModel(ctypes.Structure):
    _fields_ = [("n_types", ctypes.c_int32), ("n_interactions", ctypes.c_int32),
                ("n_features", ctypes.c_int32), ("n_rbf", ctypes.c_int32),
                ("cutoff", ctypes.c_float), ("rbf_lo", ctypes.c_float), ("rbf_hi", ctypes.c_float),
                ("rbf_gamma", ctypes.c_float), ("filter_format", ctypes.c_int32),
                ("params", ctypes.c_void_p), ("qweights", ctypes.c_void_p), ("qscales", ctypes.c_void_p),
                ("filter_math", ctypes.c_int32)]


class SnError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


_LIB = None


def lib() -> ctypes.CDLL:
    """Load libsn.so (raises if it has not been built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m schnet_cfconv_force_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    P64 = ctypes.POINTER(ctypes.c_int64)
    PS, PM = ctypes.POINTER(SnSystem), ctypes.POINTER(SnModel)
    sig = {
        "sn_param_count": (i64, [i32, i32, i32, i32]),
        "sn_param_offsets": (i32, [i32, i32, i32, i32, P64, i32]),
        "sn_quantize_filter_weights": (i32, [i32, i32, i32, i32, vp, vp, vp]),
        "sn_workspace_bytes": (sz, [PM, PS, i64]),
        "sn_status_string": (ctypes.c_char_p, [i32]),
        "sn_version": (i32, []),
        "sn_build_csr_neighbors": (i32, [PS, vp, f32, vp, vp, vp, i64, P64, vp, sz, vp]),
        "sn_energy_forces": (i32, [PM, PS, vp, vp, vp, vp, i64, vp, vp, vp, sz, vp]),
        "sn_energy_forces_static": (i32, [PM, PS, vp, vp, vp, vp, i64, vp, vp, vp, vp]),
        "sn_verlet_step": (i32, [PM, PS, vp, vp, vp, vp, f32, f32, i32, i32, f32, vp, vp, vp, i64, P64, vp, vp, vp,
                                 ctypes.POINTER(ctypes.c_int32), ctypes.c_uint32, vp, sz, vp]),
        "sn_filter_forward": (i32, [PM, i32, vp, i64, vp, vp, sz, vp]),
        "sn_read_status": (i32, [vp, vp]),
        "sn_profile_enable": (None, [i32]),
        "sn_profile_classes": (i32, []),
        "sn_profile_name": (ctypes.c_char_p, [i32]),
        "sn_profile_collect": (i32, [ctypes.POINTER(ctypes.c_double), P64]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = L
    return L


def status_string(st: int) -> str:
    return lib().sn_status_string(st).decode()


def _check(st: int, what: str):
    if st != SN_OK:
        raise SnError(st, what)


# ------------------------------------------------------------------ host helpers

def param_offsets(n_types: int, n_interactions: int, n_features: int, n_rbf: int) -> np.ndarray:
    n = 9 * n_interactions + 6
    buf = (ctypes.c_int64 * n)()
    got = lib().sn_param_offsets(n_types, n_interactions, n_features, n_rbf, buf, n)
    if got != n:
        raise SnError(SN_ERR_INVALID, "sn_param_offsets")
    return np.frombuffer(buf, dtype=np.int64).copy()


def pack_params(params: dict, hyper: dict) -> np.ndarray:
    """Place named float32 weights into the packed layout the library reports."""
    T, I, F, K = (hyper[k] for k in ("n_types", "n_interactions", "n_features", "n_rbf"))
    off = param_offsets(T, I, F, K)
    out = np.zeros(off[-1], np.float32)
    keys = ("W_in", "A1", "b1", "A2", "b2", "Wo1", "bo1", "Wo2", "bo2")
    arrays = [params["emb"]]
    for blk in params["interactions"]:
        arrays += [blk[k] for k in keys]
    arrays += [params["R1"], params["c1"], params["R2"], np.reshape(params["c2"], (1,))]
    for k, a in enumerate(arrays):
        a = np.asarray(a, np.float32).ravel()
        if off[k] + a.size != off[k + 1]:
            raise ValueError(f"parameter {k} has {a.size} values, layout expects {off[k + 1] - off[k]}")
        out[off[k]:off[k + 1]] = a
    return out


def quantize_filter_weights(packed: np.ndarray, hyper: dict):
    """Host int16 per-output-channel quantisation of every A1, A2 (sn_quantize_filter_weights)."""
    T, I, F, K = (hyper[k] for k in ("n_types", "n_interactions", "n_features", "n_rbf"))
    packed = np.ascontiguousarray(packed, np.float32)
    q = np.zeros(I * (K * F + F * F), np.int16)
    s = np.zeros(I * 2 * F, np.float32)
    _check(lib().sn_quantize_filter_weights(T, I, F, K, packed.ctypes.data, q.ctypes.data, s.ctypes.data),
           "sn_quantize_filter_weights")
    return q, s


# ------------------------------------------------------------------ device objects

def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> int:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


class Model:
    """Device copy of the packed weights plus the hyper-parameters (sn_model)."""

    def __init__(self, params: dict, hyper: dict, filter_format: int = 0, filter_math: int = 0, device="cuda"):
        torch = _torch()
        self.hyper = dict(hyper)
        self.filter_format = int(filter_format)
        self.filter_math = int(filter_math)
        packed = pack_params(params, hyper)
        self.params = torch.from_numpy(packed).to(device)
        self.qweights = self.qscales = None
        if self.filter_format == 1:
            q, s = quantize_filter_weights(packed, hyper)
            self.qweights = torch.from_numpy(q).to(device)
            self.qscales = torch.from_numpy(s).to(device)
        h = self.hyper
        self.c = SnModel(h["n_types"], h["n_interactions"], h["n_features"], h["n_rbf"], h["cutoff"],
                         h["rbf_lo"], h["rbf_hi"], h["rbf_gamma"], self.filter_format, _ptr(self.params),
                         _ptr(self.qweights), _ptr(self.qscales), self.filter_math)


class System:
    """Device copy of replica_ptr and types plus the box (sn_system)."""

    def __init__(self, replica_ptr, types, box=None, device="cuda"):
        torch = _torch()
        self.replica_ptr = torch.as_tensor(np.asarray(replica_ptr, np.int32)).to(device)
        self.types = torch.as_tensor(np.asarray(types, np.int32)).to(device)
        self.n_atoms = int(self.types.numel())
        self.n_replicas = int(self.replica_ptr.numel()) - 1
        self.box = None if box is None else [float(v) for v in box]
        b = (ctypes.c_float * 3)(*(self.box or [0.0, 0.0, 0.0]))
        self.c = SnSystem(self.n_atoms, self.n_replicas, _ptr(self.replica_ptr), _ptr(self.types),
                          1 if box is not None else 0, b)


def workspace_bytes(model: Optional[Model], system: System, max_edges: int) -> int:
    mp = ctypes.byref(model.c) if model is not None else None
    return int(lib().sn_workspace_bytes(mp, ctypes.byref(system.c), int(max_edges)))


def workspace(model: Optional[Model], system: System, max_edges: int, device="cuda"):
    torch = _torch()
    n = workspace_bytes(model, system, max_edges)
    ws = torch.empty(n + 256, dtype=torch.uint8, device=device)
    pad = (-ws.data_ptr()) % 256
    return ws[pad:pad + n]


def build_csr_neighbors(system: System, pos, r_list: float, capacity: int, ws, stream=None):
    """sn_build_csr_neighbors -> (row_ptr, col_idx, rev_idx, n_edges); raises SnError on failure."""
    torch = _torch()
    dev = pos.device
    row_ptr = torch.empty(system.n_atoms + 1, dtype=torch.int32, device=dev)
    col = torch.empty(max(capacity, 1), dtype=torch.int32, device=dev)
    rev = torch.empty(max(capacity, 1), dtype=torch.int32, device=dev)
    ne = ctypes.c_int64(0)
    st = lib().sn_build_csr_neighbors(ctypes.byref(system.c), pos.data_ptr(), float(r_list), row_ptr.data_ptr(),
                                      col.data_ptr(), rev.data_ptr(), int(capacity), ctypes.byref(ne),
                                      ws.data_ptr(), ws.numel(), _stream(stream))
    if st != SN_OK:
        err = SnError(st, "sn_build_csr_neighbors")
        err.n_edges = ne.value
        raise err
    E = ne.value
    return row_ptr, col[:E], rev[:E], E


def build_csr_status(system: System, pos, r_list: float, capacity: int, ws, stream=None):
    """Like build_csr_neighbors but returns (status, n_edges) instead of raising."""
    torch = _torch()
    dev = pos.device
    row_ptr = torch.empty(system.n_atoms + 1, dtype=torch.int32, device=dev)
    col = torch.empty(max(capacity, 1), dtype=torch.int32, device=dev)
    rev = torch.empty(max(capacity, 1), dtype=torch.int32, device=dev)
    ne = ctypes.c_int64(0)
    st = lib().sn_build_csr_neighbors(ctypes.byref(system.c), pos.data_ptr(), float(r_list), row_ptr.data_ptr(),
                                      col.data_ptr(), rev.data_ptr(), int(capacity), ctypes.byref(ne),
                                      ws.data_ptr(), ws.numel(), _stream(stream))
    return st, ne.value


def energy_forces(model: Model, system: System, pos, row_ptr, col, rev, n_edges: int, ws, energy=None,
                  forces=None, stream=None):
    """sn_energy_forces -> (energy[B], forces[N,3]) device tensors."""
    torch = _torch()
    dev = pos.device
    if energy is None:
        energy = torch.empty(system.n_replicas, dtype=torch.float32, device=dev)
    if forces is None:
        forces = torch.empty((system.n_atoms, 3), dtype=torch.float32, device=dev)
    st = lib().sn_energy_forces(ctypes.byref(model.c), ctypes.byref(system.c), pos.data_ptr(), row_ptr.data_ptr(),
                                col.data_ptr(), rev.data_ptr(), int(n_edges), energy.data_ptr(), forces.data_ptr(),
                                ws.data_ptr(), ws.numel(), _stream(stream))
    _check(st, "sn_energy_forces")
    return energy, forces


def energy_forces_static(model: Model, system: System, pos, row_ptr, col, rev, n_edges: int, energy=None,
                         forces=None, status=None, stream=None):
    """sn_energy_forces_static (no workspace, nothing allocated by the library) -> (energy[B], forces[N,3]).
    status (optional int32 device tensor [1]) receives the call's device status in stream order."""
    torch = _torch()
    dev = pos.device
    if energy is None:
        energy = torch.empty(system.n_replicas, dtype=torch.float32, device=dev)
    if forces is None:
        forces = torch.empty((system.n_atoms, 3), dtype=torch.float32, device=dev)
    if status is not None and (status.dtype != torch.int32 or status.numel() < 1 or status.device != dev):
        raise ValueError("status must be an int32 tensor on the device with at least one value")
    st = lib().sn_energy_forces_static(ctypes.byref(model.c), ctypes.byref(system.c), pos.data_ptr(),
                                       row_ptr.data_ptr(), col.data_ptr(), rev.data_ptr(), int(n_edges),
                                       energy.data_ptr(), forces.data_ptr(), _ptr(status), _stream(stream))
    _check(st, "sn_energy_forces_static")
    return energy, forces


def verlet_step(model: Model, system: System, pos, vel, forces, inv_mass, dt: float, force_to_accel: float,
                n_steps: int, r_list: float, capacity: int, ws, epot_log=None, ekin_log=None, csr=None,
                stream=None, edge_log=None, rebuild_every: int = 1, graph: bool = False):
    """sn_verlet_step; pos, vel, forces are updated in place.  Returns (row_ptr, col, rev, n_edges).
    epot_log, ekin_log (optional float64 device tensors [n_steps, B]) receive each step's replica energies,
    edge_log (optional int32 device tensor [n_steps]) each step's edge count.
    rebuild_every != 1 keeps a list built at r_list = cutoff + skin across steps (rebuilt on schedule
    and when an atom drifts beyond skin/2); graph=True replays one rebuild interval as a HIP graph."""
    torch = _torch()
    dev = pos.device
    if csr is None:
        row_ptr = torch.empty(system.n_atoms + 1, dtype=torch.int32, device=dev)
        col = torch.empty(max(capacity, 1), dtype=torch.int32, device=dev)
        rev = torch.empty(max(capacity, 1), dtype=torch.int32, device=dev)
    else:
        row_ptr, col, rev = csr
    # the logs are written by the device: wrong types or sizes would be written out of bounds
    for name, t, dt_ in (("epot_log", epot_log, torch.float64), ("ekin_log", ekin_log, torch.float64),
                         ("edge_log", edge_log, torch.int32)):
        need = n_steps * (system.n_replicas if name != "edge_log" else 1)
        if t is not None and (t.dtype != dt_ or t.numel() < need or not t.is_contiguous() or t.device != dev):
            raise ValueError(f"{name} must be a contiguous {dt_} tensor on {dev} with at least {need} values")
    ne = ctypes.c_int64(0)
    done = ctypes.c_int32(0)
    st = lib().sn_verlet_step(ctypes.byref(model.c), ctypes.byref(system.c), pos.data_ptr(), vel.data_ptr(),
                              forces.data_ptr(), inv_mass.data_ptr(), float(dt), float(force_to_accel),
                              int(n_steps), int(rebuild_every), float(r_list), row_ptr.data_ptr(), col.data_ptr(),
                              rev.data_ptr(), int(capacity), ctypes.byref(ne), _ptr(epot_log), _ptr(ekin_log),
                              _ptr(edge_log), ctypes.byref(done), SN_MD_GRAPH if graph else 0, ws.data_ptr(),
                              ws.numel(), _stream(stream))
    if st != SN_OK:
        err = SnError(st, "sn_verlet_step")
        err.steps_done = done.value
        err.n_edges = ne.value
        raise err
    return row_ptr, col[:ne.value], rev[:ne.value], ne.value


def filter_forward(model: Model, interaction: int, d, ws, phi=None, stream=None):
    """sn_filter_forward: phi[n, F] = ssp(rbf(d) A1 + b1) A2 + b2 (no envelope); ws: a workspace."""
    torch = _torch()
    n = d.numel()
    if phi is None:
        phi = torch.empty((n, model.hyper["n_features"]), dtype=torch.float32, device=d.device)
    _check(lib().sn_filter_forward(ctypes.byref(model.c), int(interaction), d.data_ptr(), n, phi.data_ptr(),
                                   ws.data_ptr(), ws.numel(), _stream(stream)), "sn_filter_forward")
    return phi


def read_status(ws, stream=None) -> int:
    return int(lib().sn_read_status(ws.data_ptr(), _stream(stream)))


# ------------------------------------------------------------------ timing

def profile_enable(on: bool = True):
    lib().sn_profile_enable(1 if on else 0)


def profile_collect() -> dict:
    """Per kernel class: (total ms, launches) of the launches since the last collect."""
    n = lib().sn_profile_classes()
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    _check(lib().sn_profile_collect(ms, cnt), "sn_profile_collect")
    return {lib().sn_profile_name(k).decode(): (ms[k], cnt[k]) for k in range(n) if cnt[k] > 0}
