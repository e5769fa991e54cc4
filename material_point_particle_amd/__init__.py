"""MI355X (gfx950) particle-to-grid transfer of the material point method.

The compute path is libmpm.so (hand-written HIP kernels behind a C ABI, see
include/mpm.h); this package holds the HIP sources (csrc/), the build step
(build.py), the ctypes binding (_lib.py) and a small device-memory driver
(transfer.py).  PyTorch is used for device memory and streams only.
"""
from ._lib import (  # noqa: F401
    EXPORTS, LIB_PATH, MpmError, grid_desc, lib, mpm_bin_particles, mpm_bin_resident, mpm_check_bounds, mpm_g2p,
    mpm_g2p_update_deformation_stress, mpm_g2p2g, mpm_g2p_records, mpm_gather_records, mpm_grid_clear, mpm_grid_clear_tiles, mpm_grid_update,
    mpm_grid_update_tiles, mpm_isplit_workspace_bytes, mpm_neohookean_affine, mpm_p2g, mpm_p2g_cic_split,
    mpm_p2g_isplit, mpm_p2g_isplit_noalloc, mpm_pbmpm_g2p_integrate, mpm_pbmpm_g2p_project, mpm_pbmpm_g2p_project_records,
    mpm_pbmpm_grid_update, mpm_pbmpm_integrate,
    mpm_pbmpm_project_elastic, mpm_strerror, mpm_update_deformation, mpm_update_deformation_stress, mpm_version,
    mpm_workspace_bytes, mpm_workspace_layout, particles, ranges,
)

__version__ = "0.1.0"
