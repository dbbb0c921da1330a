"""libm3scan: the Mamba-3 sequence mixer (exponential-trapezoidal recurrence,
data-dependent rotations, MIMO) as hand-written HIP for MI355X (gfx950),
behind a C ABI.  This package holds the HIP sources (csrc/), their build
(build.py), the ctypes binding (binding.py) and the seeded input generator
(synth.py)."""
from .binding import (M3_BF16, M3_F32, PHASE_MODES, DecodeCall, M3Error, Premix, ScanBwdCall,
                      ScanCall, ScanGrads, State, load_library, m3_scan_bwd,
                      m3_scan_bwd_supported,
                      m3_abi_version,
                      m3_decode_step, m3_decode_supported, m3_scan_fwd, m3_scan_fwd_noalloc,
                      m3_scan_supported, m3_scan_workspace_bytes, m3_status_string, zero_state)

__all__ = ["M3_BF16", "M3_F32", "PHASE_MODES", "DecodeCall", "M3Error", "Premix", "ScanBwdCall",
           "ScanCall", "ScanGrads", "State", "m3_scan_bwd", "m3_scan_bwd_supported", "load_library", "m3_abi_version",
           "m3_decode_step", "m3_decode_supported", "m3_scan_fwd", "m3_scan_fwd_noalloc",
           "m3_scan_supported",
           "m3_scan_workspace_bytes", "m3_status_string", "zero_state"]
