// Per-wave phase timeline, compiled in only with M3_TIMELINE=1 (a separate,
// instrumented build of the library, read by mamba_selective_ssm_amd/timeline.py).
// Lane 0 of every wave writes, into its own kTlSlots-entry row of a device
// buffer: s_memrealtime, s_memtime and a header word (pass, role, wave,
// segment or unit) at entry, then one 64-bit entry per phase boundary (the
// event code in the top byte, s_memtime below it), and s_memtime and
// s_memrealtime again in the row's last two entries at exit.  In the product
// build every stamp compiles to nothing.
#pragma once

#include <stddef.h>

#ifndef M3_TIMELINE
#define M3_TIMELINE 0
#endif

namespace m3 {

constexpr int kTlSlots = 256;

enum TlEvent {
    // chunked prefill (scan_kernel)
    kTlFirstIssue = 1, kTlFirstArrived = 2, kTlProloguePrep = 3, kTlPrologueBarrier = 4, kTlSetup = 5,
    kTlPrepStart = 10, kTlAngleScan = 11, kTlDecayScan = 12, kTlXRows = 13, kTlWaitTotals = 14,
    kTlRotate = 15, kTlBarrier = 16, kTlAngleIn = 17, kTlAngleScanned = 18,
    kTlFold = 20, kTlStage0 = 21, kTlPhaseC = 22, kTlPhaseD = 23, kTlStage = 24,
    kTlExit = 30,
    // gradient of the chunked form (bc_grad_kernel), per unit
    kTlUnit = 40, kTlStaged = 41, kTlScores = 42, kTlGradX = 43, kTlGradB = 44, kTlGradC = 45,
    kTlAngleSuffix = 46, kTlGradTheta = 47, kTlGradDecay = 48, kTlGradBStored = 49, kTlGradCProducts = 50
};

// Header bit of a gradient kernel's row (the prefill's rows leave it clear).
constexpr unsigned long long kTlBackward = 1ull << 61;

// One wave's timeline row (instrumented builds; otherwise empty).
struct TlRow {
    unsigned long long* w = nullptr;
    int n = 0;
    __device__ __forceinline__ void open(unsigned long long* buf, size_t row, int lane, unsigned long long hdr)
    {
        if constexpr (M3_TIMELINE) {
            if (buf == nullptr) return;
            w = buf + row * kTlSlots;
            const unsigned long long rt = __builtin_amdgcn_s_memrealtime();
            const unsigned long long t0 = __builtin_amdgcn_s_memtime();
            if (lane == 0) {
                w[0] = rt;
                w[1] = t0;
                w[2] = hdr;
            }
            n = 3;
        }
    }
    __device__ __forceinline__ void stamp(int code, int lane)
    {
        if constexpr (M3_TIMELINE) {
            if (w != nullptr && n < kTlSlots - 2) {
                const unsigned long long t = __builtin_amdgcn_s_memtime();
                if (lane == 0) w[n] = ((unsigned long long)code << 56) | (t & ((1ull << 56) - 1));
                ++n;
            }
        }
    }
    __device__ __forceinline__ void close(int lane)
    {
        if constexpr (M3_TIMELINE) {
            if (w != nullptr) {
                const unsigned long long t = __builtin_amdgcn_s_memtime();
                const unsigned long long rt = __builtin_amdgcn_s_memrealtime();
                if (lane == 0) {
                    w[kTlSlots - 2] = t;
                    w[kTlSlots - 1] = rt;
                    if (n < kTlSlots - 2) w[n] = (unsigned long long)kTlExit << 56;
                }
            }
        }
    }
};

}  // namespace m3
