"""GPU: sn_energy_forces_static, the entry point that allocates nothing (its scratch is a static
device array of SN_STATIC_SCRATCH_BYTES per GPU), against sn_energy_forces on the same inputs:
two calls in a row, the second on a smaller system, must give the same bits as the workspace
entry point (and so meet the oracle's tolerances, which the other tests establish for it); a
system whose scratch would exceed the array is refused before any GPU work."""
import sys

import numpy as np
import pytest

import oracle as O
import synth
from helpers import E_TOL, F_TOL, energy_errors, force_errors, oracle_full

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


def _prepare(sn, cfg):
    import torch
    model = sn.Model(cfg["params"], cfg["hyper"])
    system = sn.System(cfg["replica_ptr"], cfg["types"], cfg["box"])
    pos = torch.from_numpy(np.ascontiguousarray(cfg["pos"])).cuda()
    cap = max(64, 200 * len(cfg["pos"]))
    ws = sn.workspace(model, system, cap)
    csr = sn.build_csr_neighbors(system, pos, cfg["hyper"]["cutoff"], cap, ws)
    return model, system, pos, ws, csr


def test_static_scratch_entry_point_matches_the_workspace_one(sn):
    import torch
    status = torch.full((1,), 99, dtype=torch.int32, device="cuda")
    # first call: 4 x 269 beads (about 52 MiB of scratch); second: the 32-bead chain
    for name, B in (("batched_replicas", 4), ("tiny_chain", None)):
        cfg = synth.make_config(name, n_replicas=B) if B else synth.make_config(name)
        model, system, pos, ws, (row_ptr, col, rev, E) = _prepare(sn, cfg)
        need = sn.workspace_bytes(model, system, E)
        say(f"[no-alloc] {name}: E={E}, scratch {need / 2**20:.1f} MiB of {sn.SN_STATIC_SCRATCH_BYTES / 2**20:.0f}")
        assert need <= sn.SN_STATIC_SCRATCH_BYTES
        e_ws, f_ws = sn.energy_forces(model, system, pos, row_ptr, col, rev, E, ws)
        e_st, f_st = sn.energy_forces_static(model, system, pos, row_ptr, col, rev, E, status=status)
        torch.cuda.synchronize()
        assert int(status.item()) == sn.SN_OK
        assert np.array_equal(e_st.cpu().numpy(), e_ws.cpu().numpy())
        assert np.array_equal(f_st.cpu().numpy(), f_ws.cpu().numpy())
        E_ref, F_ref, eps_abs, _ = oracle_full(cfg)
        assert energy_errors(e_st.cpu().numpy(), E_ref, eps_abs).max() <= E_TOL
        assert force_errors(f_st.cpu().numpy(), F_ref, cfg["replica_ptr"]).max() <= F_TOL


def test_static_scratch_reports_device_errors_and_refuses_oversize_systems(sn):
    import torch
    cfg = synth.make_config("tiny_chain")
    p = cfg["pos"].copy()
    p[5] = p[4]                        # a coincident pair: a non-finite force
    cfg = dict(cfg, pos=p)
    model, system, pos, ws, (row_ptr, col, rev, E) = _prepare(sn, cfg)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    sn.energy_forces_static(model, system, pos, row_ptr, col, rev, E, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == sn.SN_ERR_NONFINITE
    # 8 x 269 beads need more scratch than the static array holds
    big = synth.make_config("batched_replicas", n_replicas=8)
    model, system, pos, ws, (row_ptr, col, rev, E) = _prepare(sn, big)
    assert sn.workspace_bytes(model, system, E) > sn.SN_STATIC_SCRATCH_BYTES
    with pytest.raises(sn.SnError) as exc:
        sn.energy_forces_static(model, system, pos, row_ptr, col, rev, E)
    assert exc.value.status == sn.SN_ERR_WORKSPACE
