// bf16 I/O, bf16 matrix-core operands, fp32 accumulation: the generic set
// (64 operand rows per chunk, 16-column headdim slices).
#include "m3_scan_inst.hpp"

namespace m3 {

#define V(N, R, Q) M3_SCAN_VARIANT(bf16, 1, N, R, Q, 16, 4, 4, 1)
const ScanVariant* scan_variants_bf16a(int* count)
{
    static const ScanVariant table[] = {
    V(16, 1, 64),  V(32, 1, 64),  V(64, 1, 64),  V(128, 1, 64),
    V(16, 2, 32),  V(32, 2, 32),  V(64, 2, 32),  V(128, 2, 32),
    V(16, 4, 16),  V(32, 4, 16),  V(64, 4, 16),  V(128, 4, 16),
    };
    *count = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}
#undef V

}  // namespace m3
