"""MI355X-native forward selective scan (HIP kernels for gfx950 behind a C ABI).

The compute path is the shared library ``libssmscan.so`` built from ``csrc/``;
``scan.py`` is the thin ctypes binding (argument marshalling only).  The
binding is imported lazily so that ``selective_state_space_42_amd.inputs`` can
be used without loading the HIP library.
"""

__all__ = ["ssm_scan_fwd", "ssm_scan_fwd_ex", "ssm_scan_fwd_noalloc", "ssm_scan_step", "ssm_scan_bwd",
           "ssm_scan_workspace_bytes", "ssm_scan_bwd_workspace_bytes", "ssm_ssd_fwd", "ssm_ssd_workspace_bytes", "ssm_mimo_fwd", "ssm_mimo_step",
           "ssm_mimo_workspace_bytes", "ssm_scan_status_string", "ssm_scan_abi_version",
           "ssm_calibrate_stream", "ssm_calibrate_device_math"]


def __getattr__(name):
    if name in __all__:
        from . import scan
        return getattr(scan, name)
    raise AttributeError(name)
