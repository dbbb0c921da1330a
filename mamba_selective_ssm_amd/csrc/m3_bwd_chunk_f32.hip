// Chunked scan gradient, float32 operands (dstate 32 and 64: the larger
// states' operand tiles exceed the LDS of one compute unit), and the
// dispatch of the chunked gradient.
#include "m3_bwd_chunk.hpp"

namespace m3 {
namespace bc {
hipError_t launch_f32_n32(const BcParams& p, hipStream_t s) { return launch_pr<float, 32>(p, s); }
hipError_t launch_f32_n64(const BcParams& p, hipStream_t s) { return launch_pr<float, 64>(p, s); }

static_assert(Lay<Cfg<float, 64, 64, 1>, true>::bytes <= 160 * 1024, "LDS");
static_assert(Lay<Cfg<bf16, 128, 64, 1>, true>::bytes <= 160 * 1024, "LDS");
}  // namespace bc

bool bwd_chunked_supported(int64_t N, int64_t P, int64_t R, int io_dtype)
{
    if (R != 1 && R != 2 && R != 4) return false;
    if (P != 32 && P != 64) return false;
    if (io_dtype == 1) return N == 32 || N == 64 || N == 128;
    if (io_dtype == 0) return N == 32 || N == 64;
    return false;
}

int bwd_chunk_tokens(int64_t R) { return (int)(64 / R); }

hipError_t launch_bwd_chunked(const BcParams& p, int io_dtype, hipStream_t stream)
{
    if (io_dtype == 0) return p.N == 32 ? bc::launch_f32_n32(p, stream) : bc::launch_f32_n64(p, stream);
    switch (p.N) {
    case 32: return bc::launch_bf16_n32(p, stream);
    case 64: return bc::launch_bf16_n64(p, stream);
    default: return bc::launch_bf16_n128(p, stream);
    }
}

}  // namespace m3
