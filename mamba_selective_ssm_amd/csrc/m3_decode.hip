// One autoregressive step of the Mamba-3 mixer on a resident fp32 state.
//
//   h_t = alpha_t R_t h_{t-1} + beta_t R_t U_{t-1} + gamma_t U_t,  U = B X,
//   y_t = C_t^T h_t
// (Mamba-3 summary on b-lab.team, section 1 recurrence; section 2 block
// rotations R(dt theta_i) on adjacent state rows; section 3 MIMO: B_t is
// N x R, X_t is R x P, y_t has one P-vector per rank.)  The previous
// endpoint U_{t-1} = B_prev X_prev comes from the state record, which the step
// then overwrites with (h_t, B_t, X_t).
//
// The update is memory-bound: per (b, h) it streams the N x P fp32 state in
// and out once (2*4*N*P bytes) against about (4R + 10) N P flops.  One
// workgroup of 256 threads per (b, h); each thread owns rotation-pair rows
// (2i, 2i+1) x 4 consecutive columns, read and written as float4 so that a
// wave moves whole 256-byte rows.  All state loads of a thread are issued
// before any arithmetic.  The rank-R readout is reduced across the threads
// that share a column group through LDS.
#include "m3_device.hpp"
#include "m3_internal.hpp"

namespace m3 {

namespace {

constexpr int kDecThreads = 256;
constexpr int kDecBatch = 4;   // pair-row items per thread held in flight

template <typename IO, int R>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(const DecodeParams p)
{
    extern __shared__ __attribute__((aligned(16))) float dsm[];
    const int N = p.N, P = p.P, NPR = N / 2, P4 = P / 4;
    float* sBp = dsm;                 // [R][N]
    float* sB = sBp + R * N;          // [R][N]
    float* sC = sB + R * N;           // [R][N]
    float* sXp = sC + R * N;          // [R][P]
    float* sX = sXp + R * P;          // [R][P]
    float* sCS = sX + R * P;          // [NPR][2]
    float* sY = sCS + 2 * NPR;        // [kDecThreads][R][4] partial readouts

    const int tid = threadIdx.x;
    const int64_t bh = blockIdx.x;
    const int64_t h = bh % p.H;
    const IO* x = reinterpret_cast<const IO*>(p.x) + bh * R * P;
    const IO* Bt = reinterpret_cast<const IO*>(p.B) + bh * R * N;
    const IO* Ct = reinterpret_cast<const IO*>(p.C) + bh * R * N;
    IO* Bp = reinterpret_cast<IO*>(p.Bp) + bh * R * N;
    IO* xp = reinterpret_cast<IO*>(p.xp) + bh * R * P;
    float* hs = p.h + bh * (int64_t)N * P;

    // State loads first (the bulk of the traffic): the first round of a
    // thread's rows is in flight while the small operands go to LDS.
    const int items = NPR * P4;
    float4 hv[kDecBatch][2];
    const int nrounds = (items + kDecThreads * kDecBatch - 1) / (kDecThreads * kDecBatch);
    const int cg = tid % P4;   // fixed per thread: kDecThreads is a multiple of P4
    auto load_round = [&](int rd) {
        const int base = rd * kDecThreads * kDecBatch;
#pragma unroll
        for (int k = 0; k < kDecBatch; ++k) {
            const int it = base + k * kDecThreads + tid;
            if (it < items) {
                const int i = it / P4;
                const float4* src = reinterpret_cast<const float4*>(hs + (int64_t)(2 * i) * P) + cg;
                hv[k][0] = src[0];
                hv[k][1] = src[P4];
            }
        }
    };
    if (nrounds > 0) load_round(0);

    for (int idx = tid; idx < R * N; idx += kDecThreads) {
        sBp[idx] = to_f32(Bp[idx]);
        sB[idx] = to_f32(Bt[idx]);
        sC[idx] = to_f32(Ct[idx]);
    }
    for (int idx = tid; idx < R * P; idx += kDecThreads) {
        sXp[idx] = to_f32(xp[idx]);
        sX[idx] = to_f32(x[idx]);
    }
    const float d = p.dt[bh], lm = p.lam[bh];
    for (int i = tid; i < NPR; i += kDecThreads) {
        float sn, cs;
        sincosf(d * p.theta[bh * NPR + i], &sn, &cs);
        sCS[2 * i] = cs;
        sCS[2 * i + 1] = sn;
    }
    __syncthreads();

    // The record's (B, X) has been read into LDS by every thread: overwrite it.
    for (int idx = tid; idx < R * N; idx += kDecThreads) Bp[idx] = Bt[idx];
    for (int idx = tid; idx < R * P; idx += kDecThreads) xp[idx] = x[idx];

    const float alpha = expf(d * p.A[h]);
    const float beta = (1.f - lm) * d * alpha;
    const float gamma = lm * d;

    float yp[R][4];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int q = 0; q < 4; ++q) yp[r][q] = 0.f;

    for (int rd = 0; rd < nrounds; ++rd) {
        const int base = rd * kDecThreads * kDecBatch;
        if (rd > 0) load_round(rd);
#pragma unroll
        for (int k = 0; k < kDecBatch; ++k) {
            const int it = base + k * kDecThreads + tid;
            if (it < items) {
                const int i = it / P4;
                const float cs = sCS[2 * i], sn = sCS[2 * i + 1];
                float h0[4] = {hv[k][0].x, hv[k][0].y, hv[k][0].z, hv[k][0].w};
                float h1[4] = {hv[k][1].x, hv[k][1].y, hv[k][1].z, hv[k][1].w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int col = 4 * cg + q;
                    float up0 = 0.f, up1 = 0.f, u0 = 0.f, u1 = 0.f;
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const float xpv = sXp[r * P + col], xv = sX[r * P + col];
                        up0 += sBp[r * N + 2 * i] * xpv;
                        up1 += sBp[r * N + 2 * i + 1] * xpv;
                        u0 += sB[r * N + 2 * i] * xv;
                        u1 += sB[r * N + 2 * i + 1] * xv;
                    }
                    // alpha R h + beta R U_prev = R (alpha h + beta U_prev)
                    const float a0 = alpha * h0[q] + beta * up0;
                    const float a1 = alpha * h1[q] + beta * up1;
                    const float n0 = cs * a0 - sn * a1 + gamma * u0;
                    const float n1 = sn * a0 + cs * a1 + gamma * u1;
                    h0[q] = n0;
                    h1[q] = n1;
#pragma unroll
                    for (int r = 0; r < R; ++r)
                        yp[r][q] += sC[r * N + 2 * i] * n0 + sC[r * N + 2 * i + 1] * n1;
                }
                float4* dst = reinterpret_cast<float4*>(hs + (int64_t)(2 * i) * P) + cg;
                dst[0] = make_float4(h0[0], h0[1], h0[2], h0[3]);
                dst[P4] = make_float4(h1[0], h1[1], h1[2], h1[3]);
            }
        }
    }

#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int q = 0; q < 4; ++q) sY[(tid * R + r) * 4 + q] = yp[r][q];
    __syncthreads();
    IO* y = reinterpret_cast<IO*>(p.y) + bh * R * P;
    for (int o = tid; o < R * P; o += kDecThreads) {
        const int r = o / P, col = o % P, c4 = col / 4, q = col % 4;
        float s = 0.f;
        for (int t = c4; t < kDecThreads; t += P4) s += sY[(t * R + r) * 4 + q];
        y[o] = from_f32<IO>(s);
    }
}

template <typename IO, int R>
hipError_t launch_decode_t(const DecodeParams& p, hipStream_t stream)
{
    const size_t lds = sizeof(float) * (3 * R * p.N + 2 * R * p.P + p.N + kDecThreads * R * 4);
    // The largest supported shape (N = 1024, P = 256, R = 4) needs 76 KiB;
    // raise the limit once.
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&decode_kernel<IO, R>),
        hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024);
    if (attr != hipSuccess) return attr;
    (void)hipGetLastError();
    hipLaunchKernelGGL((decode_kernel<IO, R>), dim3((unsigned)p.nbh), dim3(kDecThreads), lds,
                       stream, p);
    return hipGetLastError();
}

}  // namespace

bool decode_supported(int64_t N, int64_t P, int64_t R, int io_dtype)
{
    if (io_dtype != 0 && io_dtype != 1) return false;
    if (R != 1 && R != 2 && R != 4) return false;
    if (N < 2 || N > 1024 || (N % 2) != 0) return false;
    if (P < 4 || P > 256 || (P % 4) != 0 || (64 % (P / 4)) != 0) return false;
    return true;
}

hipError_t launch_decode(const DecodeParams& p, int io_dtype, hipStream_t stream)
{
    if (io_dtype == 0) {
        switch (p.R) {
        case 1: return launch_decode_t<float, 1>(p, stream);
        case 2: return launch_decode_t<float, 2>(p, stream);
        default: return launch_decode_t<float, 4>(p, stream);
        }
    }
    switch (p.R) {
    case 1: return launch_decode_t<bf16, 1>(p, stream);
    case 2: return launch_decode_t<bf16, 2>(p, stream);
    default: return launch_decode_t<bf16, 4>(p, stream);
    }
}

}  // namespace m3
