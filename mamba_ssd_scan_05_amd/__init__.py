"""libssd: the Mamba-2 SSD selective scan for AMD MI355X (gfx950).

The compute lives in libssd.so (HIP kernels behind a C ABI, include/ssd.h);
``mamba_ssd_scan_05_amd.ssd`` is its ctypes binding for torch tensors.
``inputs`` draws the seeded synthetic workloads, ``staging`` moves them to
the device.
"""
from .ssd import (SSD_ALGO_AUTO, SSD_ALGO_CHUNKED, SSD_ALGO_FUSED, SSD_ALGO_ROWS,  # noqa: F401
                  SsdError, ssd_last_error, ssd_scan_fwd, ssd_scan_fwd_gated, ssd_scan_fwd_rows, ssd_selective_scan_fwd,
                  ssd_scan_plan,
                  ssd_status_string, ssd_step, ssd_version,
                  ssd_release_scratch, ssd_scan_bwd, ssd_scan_bwd_gated)
