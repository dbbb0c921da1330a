// Chunked scan gradient, bf16 operands, dstate 32 and 64.
#include "m3_bwd_chunk.hpp"

namespace m3 {
namespace bc {
hipError_t launch_bf16_n32(const BcParams& p, hipStream_t s) { return launch_pr<bf16, 32>(p, s); }
hipError_t launch_bf16_n64(const BcParams& p, hipStream_t s) { return launch_pr<bf16, 64>(p, s); }
}  // namespace bc
}  // namespace m3
