// Options of the scan gradient: head groups, phase interventions and the
// pre-mixer, as maps around the plain gradient.
//
// Before the gradient kernels the inputs are materialised as the recurrence
// uses them: B and C repeated for every head of their group and pre-mixed,
// theta after the phase map, dt and lam through softplus and sigmoid.  After
// them the gradients with respect to those are carried back by the chain rule:
//   groups     dB_g = sum over the heads h of group g of dB'_h (C alike)
//   phase      zero: dtheta = 0; reverse: dtheta = -dtheta'; shuffle: pair j
//              collects dtheta' of every pair i with perm[i] = j
//   pre-mixer  B' = xh w + b_h with xh = v r, r = (mean_n v^2 + eps)^(-1/2) per
//              (token, group, rank) row v.  With G = sum_h dB'_h and g = G w:
//              dv = r (g - xh mean_n(g xh)); dw = sum over rows of G xh;
//              db_h = sum over (batch, token) of dB'_h;
//              ddt_raw = ddt' sigmoid(dt_raw + dt_bias_h), ddt_bias = sum over
//              (batch, token) of ddt_raw; dlam_raw = dlam' s (1 - s) with
//              s = sigmoid(lam_raw).
// The pre-mixer follows the Towards AI explainer of Mamba-3, section II
// (RMSNorm with gains and channel biases on B and C); the phase maps follow
// "Understanding Mamba-3 Through Oscillatory Dynamics", section 5.3.
//
// Every kernel here is bound by HBM bytes and runs once per call.  Sums over
// tokens are column sums in two fixed-order stages (partials per block of
// rows, then the partials in block order): the result is deterministic.
#include "m3scan.h"

#include "m3_device.hpp"
#include "m3_internal.hpp"

namespace m3 {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / 64;   // one wave per row of dstate values
constexpr int kMaxNK = 4;                      // dstate <= 256: 4 values per lane
constexpr int kMaxPairs = 128;

__device__ __forceinline__ float wave_sum(float v)
{
    // butterfly: every lane ends with the same value (each step adds a
    // commutative pair)
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

__device__ __forceinline__ float softplus_acc(float z)
{
    return fmaxf(z, 0.f) + log1pf(expf(-fabsf(z)));
}

__device__ __forceinline__ float sigmoid_acc(float z)
{
    const float e = expf(-fabsf(z));
    return z >= 0.f ? 1.f / (1.f + e) : e / (1.f + e);
}

struct RowIdx {
    int64_t bt, g;
    int r;
};

__device__ __forceinline__ RowIdx row_index(const BwdOptParams& p, int64_t row)
{
    RowIdx i;
    i.r = (int)(row % p.R);
    i.g = (row / p.R) % p.G;
    i.bt = row / ((int64_t)p.R * p.G);
    return i;
}

// The row's dstate values (zero past N) and its RMS scale r (1 without the
// pre-mixer).
template <typename IO>
__device__ __forceinline__ float load_row(const IO* src, int N, int lane, float eps, bool norm,
                                          float (&v)[kMaxNK])
{
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < kMaxNK; ++k) {
        const int n = lane + 64 * k;
        v[k] = n < N ? to_f32(src[n]) : 0.f;
        ss += v[k] * v[k];
    }
    if (!norm) return 1.f;
    return rsqrtf(wave_sum(ss) / (float)N + eps);
}

// B' and C' for every head: one wave per (token, group, rank) row; blockIdx.y
// picks B (0) or C (1).
template <typename IO>
__global__ void __launch_bounds__(kThreads) bo_prep_bc_kernel(BwdOptParams p)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (row >= p.BtL * p.G * p.R) return;
    const bool isC = blockIdx.y != 0;
    const IO* src = static_cast<const IO*>(isC ? p.C : p.B) + row * p.N;
    IO* dst = static_cast<IO*>(isC ? p.Ce : p.Be);
    const float* w = isC ? p.opt.Cw : p.opt.Bw;
    const float* bias = isC ? p.opt.Cb : p.opt.Bb;
    const RowIdx ri = row_index(p, row);
    float v[kMaxNK];
    const float sc = load_row(src, p.N, lane, p.opt.eps, p.opt.premix != 0, v);
    const int64_t hpg = p.H / p.G;
    for (int64_t j = 0; j < hpg; ++j) {
        const int64_t h = ri.g * hpg + j;
        IO* out = dst + ((ri.bt * p.H + h) * p.R + ri.r) * p.N;
        const float* bh = bias ? bias + (h * p.R + ri.r) * p.N : nullptr;
#pragma unroll
        for (int k = 0; k < kMaxNK; ++k) {
            const int n = lane + 64 * k;
            if (n >= p.N) continue;
            float o = v[k];
            if (p.opt.premix) o = v[k] * sc * (w ? w[n] : 1.f) + (bh ? bh[n] : 0.f);
            out[n] = from_f32<IO>(o);
        }
    }
}

// dt = softplus(dt_raw + dt_bias_h), lam = sigmoid(lam_raw).
__global__ void __launch_bounds__(kThreads) bo_prep_scalar_kernel(BwdOptParams p)
{
    const int64_t tok = p.BtL * p.H;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < tok;
         i += (int64_t)gridDim.x * kThreads) {
        const int64_t h = i % p.H;
        p.dte[i] = softplus_acc(p.dt[i] + (p.opt.dtb ? p.opt.dtb[h] : 0.f));
        p.lame[i] = sigmoid_acc(p.lam[i]);
    }
}

__device__ __forceinline__ int clamp_pair(int s, int npr) { return s < 0 ? 0 : (s >= npr ? npr - 1 : s); }

// theta after the phase map (zero mode: theta is not read).
__global__ void __launch_bounds__(kThreads) bo_prep_theta_kernel(BwdOptParams p)
{
    const int npr = p.N / 2;
    const int64_t total = p.BtL * p.H * npr;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * kThreads) {
        const int j = (int)(i % npr);
        float t = 0.f;
        if (p.opt.phase == M3_PHASE_REVERSE) t = -p.theta[i];
        else if (p.opt.phase == M3_PHASE_SHUFFLE) t = p.theta[i - j + clamp_pair(p.opt.perm[j], npr)];
        p.thetae[i] = t;
    }
}

// Group sums of dB', dC' and, with the pre-mixer, the RMSNorm backward and the
// gain terms G xh of every row.  One wave per (token, group, rank) row.
template <typename IO>
__global__ void __launch_bounds__(kThreads) bo_post_bc_kernel(BwdOptParams p)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (row >= p.BtL * p.G * p.R) return;
    const bool isC = blockIdx.y != 0;
    const float* dsrc = isC ? p.dCe : p.dBe;
    float* dout = (isC ? p.dC : p.dB) + row * p.N;
    float* q = isC ? p.qC : p.qB;
    const float* w = isC ? p.opt.Cw : p.opt.Bw;
    const RowIdx ri = row_index(p, row);
    const int64_t hpg = p.H / p.G;
    float G[kMaxNK];
#pragma unroll
    for (int k = 0; k < kMaxNK; ++k) G[k] = 0.f;
    for (int64_t j = 0; j < hpg; ++j) {
        const float* d = dsrc + ((ri.bt * p.H + ri.g * hpg + j) * p.R + ri.r) * p.N;
#pragma unroll
        for (int k = 0; k < kMaxNK; ++k) {
            const int n = lane + 64 * k;
            if (n < p.N) G[k] += d[n];
        }
    }
    if (!p.opt.premix) {
#pragma unroll
        for (int k = 0; k < kMaxNK; ++k) {
            const int n = lane + 64 * k;
            if (n < p.N) dout[n] = G[k];
        }
        return;
    }
    float v[kMaxNK];
    const float sc = load_row(static_cast<const IO*>(isC ? p.C : p.B) + row * p.N, p.N, lane,
                              p.opt.eps, true, v);
    float gx = 0.f;
#pragma unroll
    for (int k = 0; k < kMaxNK; ++k) {
        const int n = lane + 64 * k;
        if (n < p.N) gx += G[k] * (w ? w[n] : 1.f) * (v[k] * sc);
    }
    gx = wave_sum(gx) / (float)p.N;
#pragma unroll
    for (int k = 0; k < kMaxNK; ++k) {
        const int n = lane + 64 * k;
        if (n >= p.N) continue;
        const float xh = v[k] * sc;
        dout[n] = sc * (G[k] * (w ? w[n] : 1.f) - xh * gx);
        if (q) q[row * p.N + n] = G[k] * xh;
    }
}

// ddt and dlam through softplus and sigmoid, in place.
__global__ void __launch_bounds__(kThreads) bo_post_scalar_kernel(BwdOptParams p)
{
    const int64_t tok = p.BtL * p.H;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < tok;
         i += (int64_t)gridDim.x * kThreads) {
        const int64_t h = i % p.H;
        p.ddt[i] *= sigmoid_acc(p.dt[i] + (p.opt.dtb ? p.opt.dtb[h] : 0.f));
        const float s = sigmoid_acc(p.lam[i]);
        p.dlam[i] *= s * (1.f - s);
    }
}

// dtheta from the gradient of the mapped theta.  Shuffle: each block first
// lists, per pair j, the pairs i with perm[i] = j in increasing order (a chain
// first[j] -> next[i] -> ...); every i is on exactly one chain.
__global__ void __launch_bounds__(kThreads) bo_post_theta_kernel(BwdOptParams p)
{
    __shared__ int first[kMaxPairs], next[kMaxPairs];
    const int npr = p.N / 2;
    const bool shuffle = p.opt.phase == M3_PHASE_SHUFFLE;
    if (shuffle) {
        for (int j = threadIdx.x; j < npr; j += kThreads) {
            int prev = -1;
            first[j] = -1;
            for (int i = 0; i < npr; ++i) {
                if (clamp_pair(p.opt.perm[i], npr) != j) continue;
                if (prev < 0) first[j] = i;
                else next[prev] = i;
                prev = i;
            }
            if (prev >= 0) next[prev] = -1;
        }
        __syncthreads();
    }
    const int64_t total = p.BtL * p.H * npr;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * kThreads) {
        float o = 0.f;
        if (p.opt.phase == M3_PHASE_REVERSE) {
            o = -p.dthetae[i];
        } else if (shuffle) {
            const int j = (int)(i % npr);
            const float* d = p.dthetae + (i - j);
            for (int c = first[j]; c >= 0; c = next[c]) o += d[c];
        }
        p.dtheta[i] = o;
    }
}

// Column sums of a [rows][cols] float32 array, stage 1: block (x, y) sums
// rows y*rpc .. y*rpc + rpc - 1 of 256 columns into part[y][cols].
__global__ void __launch_bounds__(kThreads) bo_colsum_partial_kernel(const float* src, int64_t rows,
                                                                      int64_t cols, int64_t rpc,
                                                                      float* part)
{
    const int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (c >= cols) return;
    const int64_t r0 = (int64_t)blockIdx.y * rpc;
    const int64_t r1 = r0 + rpc < rows ? r0 + rpc : rows;
    float acc = 0.f;
    for (int64_t r = r0; r < r1; ++r) acc += src[r * cols + c];
    part[(int64_t)blockIdx.y * cols + c] = acc;
}

// Stage 2: the partials of each column in block order.
__global__ void __launch_bounds__(kThreads) bo_colsum_final_kernel(const float* part, int nchunk,
                                                                    int64_t cols, float* dst)
{
    const int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (c >= cols) return;
    float acc = 0.f;
    for (int k = 0; k < nchunk; ++k) acc += part[(int64_t)k * cols + c];
    dst[c] = acc;
}

// Row blocks of a column sum: at least 32 rows each, at most 1024 blocks, and
// at most 4 Mi partial values.
void colsum_plan(int64_t rows, int64_t cols, int64_t* rpc, int* nchunk)
{
    int64_t nc = (rows + 31) / 32;
    if (nc > 1024) nc = 1024;
    const int64_t cap = ((int64_t)1 << 22) / (cols > 0 ? cols : 1);
    if (nc > cap) nc = cap;
    if (nc < 1) nc = 1;
    int64_t r = (rows + nc - 1) / nc;
    if (r < 1) r = 1;
    *rpc = r;
    *nchunk = (int)((rows + r - 1) / r);
    if (*nchunk < 1) *nchunk = 1;
}

hipError_t colsum(const float* src, int64_t rows, int64_t cols, float* part, float* dst,
                  hipStream_t s)
{
    if (cols <= 0) return hipSuccess;
    int64_t rpc;
    int nchunk;
    colsum_plan(rows, cols, &rpc, &nchunk);
    const unsigned gx = (unsigned)((cols + kThreads - 1) / kThreads);
    hipLaunchKernelGGL(bo_colsum_partial_kernel, dim3(gx, nchunk), dim3(kThreads), 0, s, src, rows,
                       cols, rpc, part);
    hipLaunchKernelGGL(bo_colsum_final_kernel, dim3(gx), dim3(kThreads), 0, s, part, nchunk, cols,
                       dst);
    return hipGetLastError();
}

unsigned stride_grid(int64_t n)
{
    const int64_t b = (n + kThreads - 1) / kThreads;
    return (unsigned)(b < ((int64_t)1 << 20) ? b : ((int64_t)1 << 20));
}

template <typename IO>
hipError_t pre_impl(const BwdOptParams& p, hipStream_t s)
{
    const int64_t rows = p.BtL * p.G * p.R, tok = p.BtL * p.H;
    if (p.Be != nullptr && rows > 0)
        hipLaunchKernelGGL(bo_prep_bc_kernel<IO>, dim3((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock), 2),
                           dim3(kThreads), 0, s, p);
    if (p.dte != nullptr && tok > 0)
        hipLaunchKernelGGL(bo_prep_scalar_kernel, dim3(stride_grid(tok)), dim3(kThreads), 0, s, p);
    if (p.thetae != nullptr && tok > 0)
        hipLaunchKernelGGL(bo_prep_theta_kernel, dim3(stride_grid(tok * (p.N / 2))), dim3(kThreads), 0,
                           s, p);
    return hipGetLastError();
}

template <typename IO>
hipError_t post_impl(const BwdOptParams& p, hipStream_t s)
{
    const int64_t rows = p.BtL * p.G * p.R, tok = p.BtL * p.H;
    if (p.opt.premix && tok > 0)
        hipLaunchKernelGGL(bo_post_scalar_kernel, dim3(stride_grid(tok)), dim3(kThreads), 0, s, p);
    if (p.dBe != nullptr && rows > 0)
        hipLaunchKernelGGL(bo_post_bc_kernel<IO>, dim3((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock), 2),
                           dim3(kThreads), 0, s, p);
    if (p.dthetae != nullptr && p.dtheta != nullptr && tok > 0)
        hipLaunchKernelGGL(bo_post_theta_kernel, dim3(stride_grid(tok * (p.N / 2))), dim3(kThreads), 0,
                           s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !p.opt.premix) return e;
    const int64_t hrn = p.H * p.R * p.N;
    if (p.ddtb && (e = colsum(p.ddt, p.BtL, p.H, p.part, p.ddtb, s)) != hipSuccess) return e;
    if (p.dBw && (e = colsum(p.qB, rows, p.N, p.part, p.dBw, s)) != hipSuccess) return e;
    if (p.dCw && (e = colsum(p.qC, rows, p.N, p.part, p.dCw, s)) != hipSuccess) return e;
    if (p.dBb && (e = colsum(p.dBe, p.BtL, hrn, p.part, p.dBb, s)) != hipSuccess) return e;
    if (p.dCb && (e = colsum(p.dCe, p.BtL, hrn, p.part, p.dCb, s)) != hipSuccess) return e;
    return hipSuccess;
}

}  // namespace

size_t bwd_options_partial_floats(int64_t BtL, int64_t H, int64_t G, int N, int R)
{
    size_t most = 0;
    const int64_t shapes[3][2] = {{BtL, H}, {BtL * G * R, N}, {BtL, H * R * N}};
    for (const auto& sh : shapes) {
        int64_t rpc;
        int nchunk;
        colsum_plan(sh[0], sh[1], &rpc, &nchunk);
        const size_t n = (size_t)nchunk * (size_t)(sh[1] > 0 ? sh[1] : 0);
        if (n > most) most = n;
    }
    return most;
}

hipError_t launch_bwd_options_pre(const BwdOptParams& p, int io_dtype, hipStream_t stream)
{
    return io_dtype == M3_F32 ? pre_impl<float>(p, stream) : pre_impl<bf16>(p, stream);
}

hipError_t launch_bwd_options_post(const BwdOptParams& p, int io_dtype, hipStream_t stream)
{
    return io_dtype == M3_F32 ? post_impl<float>(p, stream) : post_impl<bf16>(p, stream);
}

}  // namespace m3
