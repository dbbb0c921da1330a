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
    M3_SCAN_VARIANT(bf16, 1, 128, 1, 64, 64, 4, 4, 1),
    M3_SCAN_VARIANT(bf16, 1, 128, 1, 32, 64, 4, 4, 2),
    M3_SCAN_VARIANT(bf16, 1, 128, 4, 16, 64, 4, 4, 1),
    M3_SCAN_VARIANT(bf16, 1, 128, 4, 8, 64, 4, 4, 1),
    M3_SCAN_VARIANT(bf16, 1, 64, 1, 32, 16, 4, 4, 1),
    M3_SCAN_VARIANT(bf16, 1, 64, 1, 128, 16, 4, 4, 1),
    };
    *count = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}

}  // namespace m3
