// Accumulated rotation angle of a scan, per (sequence, head, pair):
//   Phi_out = Phi_in + sum over the call's tokens of dt_t theta_t[i]
// (Mamba-3 summary on b-lab.team, section 2, Proposition 3: the product of
// the step rotations R(dt_s theta_s) is the rotation by their running sum),
// with dt and theta as the recurrence uses them: the phase transform (zero,
// reverse, shuffled increments) and the pre-mixer's softplus on dt.
//
// Two launches, both deterministic: per (row, head, block of 64 tokens) one
// thread per pair sums its block in float64; then one thread per (row, head,
// pair) adds the blocks in order to Phi_in and reduces into [-pi, pi).
#include "m3_device.hpp"
#include "m3_internal.hpp"

namespace m3 {

namespace {

__device__ __forceinline__ float softplus_p(float z) { return z > 20.f ? z : log1pf(expf(z)); }

__global__ __launch_bounds__(64) void phase_block_kernel(const PhaseParams p)
{
    const int64_t bh = blockIdx.x;            // row * H + head
    const int64_t blk = blockIdx.y;
    int64_t b, h;
    split_bh(bh, p.H, b, h);
    const int NPR = p.NPR;
    // this row's tokens: a dense batch row, or a packed sequence
    int64_t L = p.L, base = b * p.L;
    if (p.opt.cu != nullptr) {
        int64_t lo = p.opt.cu[b], hi = p.opt.cu[b + 1];
        lo = lo < 0 ? 0 : (lo > p.L ? p.L : lo);
        hi = hi < lo ? lo : (hi > p.L ? p.L : hi);
        base = lo;
        L = hi - lo < p.opt.max_len ? hi - lo : p.opt.max_len;
    }
    const int64_t t0 = blk * kPhaseBlock;
    const int64_t t1 = t0 + kPhaseBlock < L ? t0 + kPhaseBlock : L;
    const float dtb = (p.opt.premix && p.opt.dtb != nullptr) ? p.opt.dtb[h] : 0.f;
    for (int i = threadIdx.x; i < NPR; i += 64) {
        int src = i;
        if (p.opt.phase == 3) {
            src = p.opt.perm[i];
            src = src < 0 ? 0 : (src >= NPR ? NPR - 1 : src);
        }
        const float sign = p.opt.phase == 2 ? -1.f : 1.f;
        double s = 0.0;
        if (p.opt.phase != 1) {
            for (int64_t t = t0; t < t1; ++t) {
                const int64_t k = (base + t) * p.H + h;
                const float d = p.opt.premix ? softplus_p(p.dt[k] + dtb) : p.dt[k];
                s += (double)d * (double)(sign * p.theta[k * NPR + src]);
            }
        }
        p.part[(bh * p.nblk + blk) * NPR + i] = s;
    }
}

__global__ __launch_bounds__(256) void phase_total_kernel(const PhaseParams p)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t n = p.rows * p.H * p.NPR;
    if (idx >= n) return;
    const int64_t bh = idx / p.NPR;
    const int i = (int)(idx % p.NPR);
    double s = p.opt.phase_in != nullptr ? (double)p.opt.phase_in[idx] : 0.0;
    for (int64_t blk = 0; blk < p.nblk; ++blk) s += p.part[(bh * p.nblk + blk) * p.NPR + i];
    const double twopi = 6.283185307179586;
    double w = s - twopi * floor((s + 3.141592653589793) / twopi);
    if (w >= 3.141592653589793) w -= twopi;   // rounding at the upper edge
    p.opt.phase_out[idx] = (float)w;
}

}  // namespace

hipError_t launch_phase_accumulate(const PhaseParams& p, hipStream_t stream)
{
    const int64_t nbh = p.rows * p.H;
    if (nbh == 0) return hipSuccess;
    if (p.nblk > 0) {
        hipLaunchKernelGGL(phase_block_kernel, dim3((unsigned)nbh, (unsigned)p.nblk), dim3(64), 0, stream, p);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t n = nbh * p.NPR;
    hipLaunchKernelGGL(phase_total_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace m3
