// Chunked scan gradient, bf16 operands, dstate 128.
#include "m3_bwd_chunk.hpp"

namespace m3 {
namespace bc {
hipError_t launch_bf16_n128(const BcParams& p, hipStream_t s) { return launch_pr<bf16, 128>(p, s); }
}  // namespace bc
}  // namespace m3
