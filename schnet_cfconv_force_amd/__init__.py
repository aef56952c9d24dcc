"""MI355X SchNet continuous-filter-convolution energy/force library.

The compute lives in libsn.so (hand-written HIP for gfx950, C ABI in
include/sn.h); this package is its ctypes binding.  Build the library with
`python -m schnet_cfconv_force_amd.build`.
"""
from .binding import (  # noqa: F401
    EXPORTED, LIB_PATH, Model, SN_ERR_BOX, SN_ERR_CAPACITY, SN_ERR_HIP, SN_ERR_INVALID, SN_ERR_NONFINITE,
    SN_ERR_ROW, SN_ERR_WORKSPACE, SN_MAX_ROW, SN_MD_GRAPH, SN_OK, SN_STATIC_SCRATCH_BYTES, SnError, System, build_csr_neighbors, build_csr_status,
    energy_forces, energy_forces_static, filter_forward, lib, pack_params, param_offsets, profile_collect, profile_enable,
    quantize_filter_weights, read_status, status_string, verlet_step, workspace, workspace_bytes,
)
