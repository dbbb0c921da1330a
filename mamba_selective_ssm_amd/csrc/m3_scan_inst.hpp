// Helper for the instantiation units: one table entry per compiled variant.
#pragma once

#include "m3_scan_kernel.hpp"

#define M3_SCAN_VARIANT(IO, IOCODE, N, R, Q, PS, NWM, NWP, OCC)                              \
    {IOCODE, N, R, Q, PS, NWM + NWP, OCC,                                                    \
     ::m3::ScanCfg<IO, N, PS, R, Q, NWM, NWP, OCC>::lds_bytes,                               \
     &::m3::launch_scan<::m3::ScanCfg<IO, N, PS, R, Q, NWM, NWP, OCC>>,                      \
     &::m3::scan_workspace_bytes<::m3::ScanCfg<IO, N, PS, R, Q, NWM, NWP, OCC>>, 0}

// The same with one chunk buffer (prepared operands held in registers).
#define M3_SCAN_VARIANT_SB(IO, IOCODE, N, R, Q, PS, NWM, NWP, OCC)                           \
    {IOCODE, N, R, Q, PS, NWM + NWP, OCC,                                                    \
     ::m3::ScanCfg<IO, N, PS, R, Q, NWM, NWP, OCC, 1>::lds_bytes,                            \
     &::m3::launch_scan<::m3::ScanCfg<IO, N, PS, R, Q, NWM, NWP, OCC, 1>>,                   \
     &::m3::scan_workspace_bytes<::m3::ScanCfg<IO, N, PS, R, Q, NWM, NWP, OCC, 1>>, 0}

// A variant for calls with the pre-mixer only (preferred for them).
#define M3_SCAN_VARIANT_PM(IO, IOCODE, N, R, Q, PS, NWM, NWP, OCC)                           \
    {IOCODE, N, R, Q, PS, NWM + NWP, OCC,                                                    \
     ::m3::ScanCfg<IO, N, PS, R, Q, NWM, NWP, OCC>::lds_bytes,                               \
     &::m3::launch_scan<::m3::ScanCfg<IO, N, PS, R, Q, NWM, NWP, OCC>>,                      \
     &::m3::scan_workspace_bytes<::m3::ScanCfg<IO, N, PS, R, Q, NWM, NWP, OCC>>, 1}
