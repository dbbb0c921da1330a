// Helper for the instantiation units: one table entry per compiled variant.
#pragma once

#include "m3_scan_kernel.hpp"

#define M3_SCAN_VARIANT(IO, IOCODE, N, R, Q, PS, NW)                                   \
    {IOCODE, N, R, Q, PS, NW, ::m3::ScanCfg<IO, N, PS, R, Q, NW>::lds_bytes,            \
     &::m3::launch_scan<::m3::ScanCfg<IO, N, PS, R, Q, NW>>,                          \
     &::m3::scan_workspace_bytes<::m3::ScanCfg<IO, N, PS, R, Q, NW>>}
