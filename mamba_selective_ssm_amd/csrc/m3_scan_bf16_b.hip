// bf16 variants for the measured workload shapes: full 64-column headdim
// slices and other chunk lengths.
#include "m3_scan_inst.hpp"

namespace m3 {

const ScanVariant* scan_variants_bf16b(int* count)
{
    // Order matters: among variants with the same (N, R, chunk) and the widest
    // headdim slice, the first listed is the one the library picks.
    static const ScanVariant table[] = {
    M3_SCAN_VARIANT(bf16, 1, 64, 1, 64, 64, 4, 4, 2),
    // with the pre-mixer the two-per-unit variant spills: one workgroup per
    // compute unit with 8 prep waves (54.3 -> 47.6 us on the single-layer
    // prefill with the pre-mixer)
    M3_SCAN_VARIANT_PM(bf16, 1, 64, 1, 64, 64, 4, 8, 1),
    // dstate 128 at one workgroup per compute unit: 4 matrix-core waves and 8
    // operand-prep waves (prep is the critical path; 13% faster on the MIMO
    // prefill and 7% on the long prefill than 4 + 4)
    M3_SCAN_VARIANT(bf16, 1, 128, 1, 64, 64, 4, 8, 1),
    M3_SCAN_VARIANT(bf16, 1, 128, 1, 32, 64, 4, 4, 2),
    M3_SCAN_VARIANT(bf16, 1, 128, 4, 16, 64, 4, 8, 1),
    M3_SCAN_VARIANT(bf16, 1, 128, 4, 8, 64, 4, 4, 1),
    // 128-row chunks at dstate 128 (the long-context chunk sweep's 128 and
    // the MIMO prefill at chunk 32), with one chunk buffer: two do not fit
    // in LDS
    M3_SCAN_VARIANT_SB(bf16, 1, 128, 1, 128, 64, 4, 8, 1),
    M3_SCAN_VARIANT_SB(bf16, 1, 128, 4, 32, 64, 4, 8, 1),
    M3_SCAN_VARIANT(bf16, 1, 64, 1, 32, 16, 4, 4, 1),
    M3_SCAN_VARIANT(bf16, 1, 64, 1, 128, 16, 4, 4, 1),
    };
    *count = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}

}  // namespace m3
