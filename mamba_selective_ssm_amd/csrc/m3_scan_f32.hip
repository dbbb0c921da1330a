// fp32 I/O and fp32 matrix-core operands (the 1e-4 correctness path):
// 32 operand rows per chunk (Q = 32 / R) and 16-column headdim slices.
#include "m3_scan_inst.hpp"

namespace m3 {

#define V(N, R, Q) M3_SCAN_VARIANT(float, 0, N, R, Q, 16, 4, 4, 1)
const ScanVariant* scan_variants_f32(int* count)
{
    static const ScanVariant table[] = {
    V(16, 1, 32),  V(32, 1, 32),  V(64, 1, 32),  V(128, 1, 32),
    V(16, 2, 16),  V(32, 2, 16),  V(64, 2, 16),  V(128, 2, 16),
    V(16, 4, 8),   V(32, 4, 8),   V(64, 4, 8),   V(128, 4, 8),
    };
    *count = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}
#undef V

}  // namespace m3
