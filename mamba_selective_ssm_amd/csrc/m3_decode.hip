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
// The update streams the N x P fp32 state in and out once (8 N P bytes per
// (b, h)) against about (3R + 5) N P flops: memory-bound.  One wavefront per
// (b, h), no workgroup barriers:
//   * lane l owns columns 4*(l % P4) .. +3 (P4 = P/4) of the rotation pairs
//     i = l / P4 + RG * k (RG = 64 / P4 row groups), so one load instruction
//     moves 2*RG consecutive state rows -- contiguous, 16 bytes per lane;
//   * pairs are streamed in batches of PB with the next batch's loads in
//     flight while the current one is updated and stored;
//   * B_prev, B and C go to the wave's own LDS slice as [n][r] rows (read as
//     broadcasts by the lanes of a row group); X_prev, X stay in registers;
//   * the rank-R readout of each column is reduced across the row groups
//     with lane shuffles.
// Options: per-token decay A_t, B/C shared by head groups, phase
// interventions (zero / reverse / shuffled increments; the rotation removed
// from writing or readout, with the accumulated angle carried in and out:
// "Understanding Mamba-3 Through Oscillatory Dynamics", section 5.3 and
// appendix D.4) and the pre-mixer
// (softplus / sigmoid of the raw dt / lam, RMSNorm with gains and biases on
// B and C, applied to the wave's LDS copy; the record keeps the normalised B).
#include "m3_device.hpp"
#include "m3_internal.hpp"

namespace m3 {

namespace {

constexpr int kDecWaves = 4;   // wavefronts (one (b, h) each) per workgroup, at most
constexpr int kPB = 1;         // rotation pairs per batch and lane
// The pre-mixer on row pieces (dstate 32, 64 or 128): each row's sum of
// squares within an aligned lane group of N/8 lanes.
__device__ constexpr bool decode_row_premix(bool pm, int N)
{
    return pm && (N == 32 || N == 64 || N == 128);
}

template <int R> struct RVec;
template <> struct RVec<1> {
    float v[1];
    __device__ __forceinline__ void load(const float* p) { v[0] = p[0]; }
};
template <> struct RVec<2> {
    float v[2];
    __device__ __forceinline__ void load(const float* p) {
        const float2 a = *reinterpret_cast<const float2*>(p);
        v[0] = a.x; v[1] = a.y;
    }
};
template <> struct RVec<4> {
    float v[4];
    __device__ __forceinline__ void load(const float* p) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(p);
        v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
    }
};

// 8 consecutive io elements copied (16 or 32 bytes).
__device__ __forceinline__ void copy8(bf16* d, const bf16* s) {
    *reinterpret_cast<uint4*>(d) = *reinterpret_cast<const uint4*>(s);
}
__device__ __forceinline__ void copy8(float* d, const float* s) {
    reinterpret_cast<uint4*>(d)[0] = reinterpret_cast<const uint4*>(s)[0];
    reinterpret_cast<uint4*>(d)[1] = reinterpret_cast<const uint4*>(s)[1];
}

// 8 consecutive io elements as floats, streamed (read once).
__device__ __forceinline__ void gload8_nt(float (&d)[8], const bf16* p) {
    const bf16x8 v = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(p));
#pragma unroll
    for (int e = 0; e < 8; ++e) d[e] = (float)v[e];
}
__device__ __forceinline__ void gload8_nt(float (&d)[8], const float* p) {
    const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4));
#pragma unroll
    for (int e = 0; e < 4; ++e) { d[e] = a[e]; d[4 + e] = b[e]; }
}

// 4 consecutive io elements as floats.
__device__ __forceinline__ void load4(float (&d)[4], const bf16* p) {
    const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) d[e] = (float)v[e];
}
__device__ __forceinline__ void load4(float (&d)[4], const float* p) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) d[e] = v[e];
}

__device__ __forceinline__ float softplus_d(float z) { return z > 20.f ? z : log1pf(expf(z)); }
__device__ __forceinline__ float sigmoid_d(float z) { return 1.f / (1.f + expf(-z)); }

template <typename IO, int R, bool PM>
__global__ __launch_bounds__(64 * kDecWaves) void decode_kernel(const DecodeParams p)
{
    extern __shared__ __attribute__((aligned(16))) float dsm[];
    const int N = p.N, P = p.P, NPR = N / 2;
    const int P4 = P / 4, RG = 64 / P4;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t bh = (int64_t)blockIdx.x * (blockDim.x >> 6) + wv;
    if (bh >= p.nbh) return;   // whole wavefront
    int64_t bb, h;
    split_bh(bh, p.H, bb, h);   // (batch x heads <= 2^30, checked on the host)
    const int64_t G = p.opt.groups;
    const int64_t bg = bb * G + (int)h / ((int)p.H / (int)G);   // B/C row of this head's group

    float* sBp = dsm + (int64_t)wv * (3 * R * N + 2 * N);   // this wave's slice: [N][R]
    float* sB = sBp + R * N;                            // [N][R]
    float* sC = sB + R * N;                             // [N][R]
    float* sCS = sC + R * N;                            // [NPR][2] cos, sin of dt theta
    float* sCW = sCS + N;                               // [NPR][2] cos, sin of the accumulated angle
    // rotation removed from writing / readout (wave-uniform)
    const bool no_write = p.opt.phase == 4 || p.opt.phase == 6;
    const bool no_read = p.opt.phase == 5 || p.opt.phase == 6;

    const IO* x = reinterpret_cast<const IO*>(p.x) + bh * R * P;
    const IO* Bt = reinterpret_cast<const IO*>(p.B) + bg * R * N;
    const IO* Ct = reinterpret_cast<const IO*>(p.C) + bg * R * N;
    IO* Bp = reinterpret_cast<IO*>(p.Bp) + bh * R * N;
    IO* xp = reinterpret_cast<IO*>(p.xp) + bh * R * P;
    float* hs = p.h + bh * (int64_t)N * P;

    const int cg = lane % P4, rg = lane / P4;
    const int npl = (NPR - rg + RG - 1) / RG;   // pairs of this lane
    const int nbat = (NPR / RG + (NPR % RG ? 1 : 0) + kPB - 1) / kPB;   // wave-uniform

    // State batches: rows 2i and 2i+1 of pair i = rg + RG*(kPB*bt + k).
    f32x4 ha[kPB][2], hb[kPB][2];
    auto load_batch = [&](f32x4 (&hv)[kPB][2], int bt) {
#pragma unroll
        for (int k = 0; k < kPB; ++k) {
            int j = kPB * bt + k;
            if (j >= npl) j = npl - 1;   // clamped duplicate (never stored)
            const int i = j >= 0 ? rg + RG * j : 0;
            const f32x4* src = reinterpret_cast<const f32x4*>(hs + (int64_t)(2 * i) * P) + cg;
            hv[k][0] = src[0];
            hv[k][1] = src[P4];
        }
    };
    if (npl > 0) load_batch(ha, 0);

    // Pre-mixer, dstate 32, 64 or 128 (row pieces): each lane loads 8
    // consecutive entries of one rank row of B and C below, so the N/8 lanes
    // of an aligned lane group hold a whole row; the gains and biases of the
    // lane's 8 entries are loaded now, in flight with the state.
    const bool rowpm = decode_row_premix(PM, N);   // wave-uniform
    f32x4 fw[4][2];   // B gain, C gain, B bias, C bias at the lane's entries
    if constexpr (PM) {
        if (rowpm && 8 * lane < R * N) {
            const int r = 8 * lane / N, n = 8 * lane % N;
            const int64_t bo = (h * R + r) * (int64_t)N + n;
            const float* src[4] = {p.opt.Bw != nullptr ? p.opt.Bw + n : nullptr,
                                   p.opt.Cw != nullptr ? p.opt.Cw + n : nullptr,
                                   p.opt.Bb != nullptr ? p.opt.Bb + bo : nullptr,
                                   p.opt.Cb != nullptr ? p.opt.Cb + bo : nullptr};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const float dflt = m < 2 ? 1.f : 0.f;
                if (src[m] != nullptr) {
                    fw[m][0] = *reinterpret_cast<const f32x4*>(src[m]);
                    fw[m][1] = *reinterpret_cast<const f32x4*>(src[m] + 4);
                } else {
                    fw[m][0] = f32x4{dflt, dflt, dflt, dflt};
                    fw[m][1] = fw[m][0];
                }
            }
        }
    }

    // Pre-mixer gains and biases of this lane's first GPF entries n = lane +
    // 64 k (other dstates), loaded now so that they are in flight with the
    // state (entries past 64 GPF, for N > 128, are read where they are used).
    constexpr int GPF = 2;
    float gwb[GPF], gwc[GPF], gbb[GPF][R], gbc[GPF][R];
    if constexpr (PM) {
#pragma unroll
        for (int k = 0; k < GPF && !rowpm; ++k) {
            const int n = lane + 64 * k;
            const bool ok = n < N;
            gwb[k] = (ok && p.opt.Bw != nullptr) ? p.opt.Bw[n] : 1.f;
            gwc[k] = (ok && p.opt.Cw != nullptr) ? p.opt.Cw[n] : 1.f;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int64_t bi = (h * R + r) * (int64_t)N + n;
                gbb[k][r] = (ok && p.opt.Bb != nullptr) ? p.opt.Bb[bi] : 0.f;
                gbc[k][r] = (ok && p.opt.Cb != nullptr) ? p.opt.Cb[bi] : 0.f;
            }
        }
    }

    // Small operands: B_prev, B, C transposed into the wave's LDS slice, the
    // pair rotations, this lane's columns of X_prev and X.
    // 8 consecutive elements (one rank row) per lane and load when N % 8 == 0.
    const int n8 = (N % 8 == 0) ? R * N : 0;
    for (int idx = 8 * lane; idx < n8; idx += 512) {
        const int r = idx / N, n = idx % N;
        float vbp[8], vb[8], vc[8];
        gload8(vbp, Bp + idx);
        gload8_nt(vb, Bt + idx);
        gload8_nt(vc, Ct + idx);
        if constexpr (PM) {
            if (rowpm) {
                // each row scaled by 1/rms over its N entries (the lane
                // group's sum of squares), times the gain, plus the bias
                float sb = 0.f, sc = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    sb += vb[e] * vb[e];
                    sc += vc[e] * vc[e];
                }
                if (N == 128) {
                    sb = lane_group_sum<16>(sb);
                    sc = lane_group_sum<16>(sc);
                } else if (N == 64) {
                    sb = lane_group_sum<8>(sb);
                    sc = lane_group_sum<8>(sc);
                } else {
                    sb = lane_group_sum<4>(sb);
                    sc = lane_group_sum<4>(sc);
                }
                const float kb = rsqrtf(sb / (float)N + p.opt.eps);
                const float kc = rsqrtf(sc / (float)N + p.opt.eps);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    vb[e] = vb[e] * kb * fw[0][e / 4][e % 4] + fw[2][e / 4][e % 4];
                    vc[e] = vc[e] * kc * fw[1][e / 4][e % 4] + fw[3][e / 4][e % 4];
                }
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            sBp[(n + e) * R + r] = vbp[e];
            sB[(n + e) * R + r] = vb[e];
            sC[(n + e) * R + r] = vc[e];
        }
        if constexpr (PM) {
            // the record's B: this step's pre-mixed row piece (the piece's
            // old value, read above, is in LDS by now)
            if (rowpm) {
                gstore4(Bp + idx, f32x4{vb[0], vb[1], vb[2], vb[3]});
                gstore4(Bp + idx + 4, f32x4{vb[4], vb[5], vb[6], vb[7]});
            }
        }
    }
    for (int idx = n8 + lane; idx < R * N; idx += 64) {
        const int r = idx / N, n = idx % N;
        sBp[n * R + r] = to_f32(Bp[idx]);
        sB[n * R + r] = to_f32(Bt[idx]);
        sC[n * R + r] = to_f32(Ct[idx]);
    }
    float d = p.dt[bh], lm = p.lam[bh];
    if constexpr (PM) {
        d = softplus_d(d + (p.opt.dtb != nullptr ? p.opt.dtb[h] : 0.f));
        lm = sigmoid_d(lm);
    }
    for (int i = lane; i < NPR; i += 64) {
        float th = 0.f;                                        // zero: theta not read
        if (p.opt.phase == 0 || p.opt.phase >= 4) th = p.theta[bh * NPR + i];
        else if (p.opt.phase == 2) th = -p.theta[bh * NPR + i];
        else if (p.opt.phase == 3) {
            int src = p.opt.perm[i];
            src = src < 0 ? 0 : (src >= NPR ? NPR - 1 : src);
            th = p.theta[bh * NPR + src];
        }
        const float phi = d * th;
        float sn, cs;
        sincosf(phi, &sn, &cs);
        *reinterpret_cast<float2*>(sCS + 2 * i) = make_float2(cs, sn);
        // accumulated angle after this step (read before it is overwritten
        // when phase_out is phase_in: same lane, same element)
        const float Phi = (p.opt.phase_in != nullptr ? p.opt.phase_in[bh * NPR + i] : 0.f) + phi;
        if (no_write || no_read) {
            float sw, cw;
            sincosf(Phi, &sw, &cw);
            *reinterpret_cast<float2*>(sCW + 2 * i) = make_float2(cw, sw);
        }
        if (p.opt.phase_out != nullptr) {
            const float twopi = 6.28318530717958648f, pi = 3.14159265358979324f;
            float w = Phi - twopi * floorf((Phi + pi) / twopi);
            if (w >= pi) w -= twopi;
            p.opt.phase_out[bh * NPR + i] = w;
        }
    }
    float xv[R][4], xpv[R][4];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        load4(xv[r], x + r * P + 4 * cg);
        load4(xpv[r], xp + r * P + 4 * cg);
    }
    const float alpha = expf(d * p.A[p.opt.a_tok ? bh : h]);
    const float beta = (1.f - lm) * d * alpha;
    const float gamma = lm * d;
    // The record's (B, X) are in LDS / registers: overwrite it with this
    // step's (every element is rewritten by an instruction of this wave that
    // follows the one that read it).
    if constexpr (PM) {
        if (!rowpm) {
            // Pre-mixer on the LDS copies of B and C (other dstates): each
            // (matrix, rank) row is scaled by 1/rms over its N entries, times the
            // gain, plus the bias.
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // Row sums of squares: the 2R rows' wavefront sums (DPP scans) are
            // independent chains.
            float sc[2][R];
    #pragma unroll
            for (int m = 0; m < 2; ++m)
    #pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float* row = m == 0 ? sB : sC;
                    float ss = 0.f;
                    for (int n = lane; n < N; n += 64) ss += row[n * R + r] * row[n * R + r];
                    ss = wave_read_lane(wave_inclusive_sum(ss), 63);
                    sc[m][r] = rsqrtf(ss / (float)N + p.opt.eps);
                }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            auto premix_entry = [&](int n, float wb, float wc, const float (&bb)[R], const float (&bcv)[R]) {
    #pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float vb = sB[n * R + r] * sc[0][r] * wb + bb[r];
                    const float vc = sC[n * R + r] * sc[1][r] * wc + bcv[r];
                    sB[n * R + r] = vb;
                    sC[n * R + r] = vc;
                    Bp[r * N + n] = from_f32<IO>(vb);
                }
            };
    #pragma unroll
            for (int k = 0; k < GPF; ++k)
                if (lane + 64 * k < N) premix_entry(lane + 64 * k, gwb[k], gwc[k], gbb[k], gbc[k]);
            for (int n = lane + 64 * GPF; n < N; n += 64) {
                float bb[R], bcv[R];
    #pragma unroll
                for (int r = 0; r < R; ++r) {
                    const int64_t bi = (h * R + r) * (int64_t)N + n;
                    bb[r] = p.opt.Bb != nullptr ? p.opt.Bb[bi] : 0.f;
                    bcv[r] = p.opt.Cb != nullptr ? p.opt.Cb[bi] : 0.f;
                }
                premix_entry(n, p.opt.Bw != nullptr ? p.opt.Bw[n] : 1.f, p.opt.Cw != nullptr ? p.opt.Cw[n] : 1.f,
                             bb, bcv);
            }
        }
    } else {
        for (int idx = 8 * lane; idx < n8; idx += 512) copy8(Bp + idx, Bt + idx);
        for (int idx = n8 + lane; idx < R * N; idx += 64) Bp[idx] = Bt[idx];
    }
    if (rg == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r) gstore4(xp + r * P + 4 * cg, f32x4{xv[r][0], xv[r][1], xv[r][2], xv[r][3]});
    }
    // The LDS slice is written and read by this wavefront only.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (no_read) {
        // readout through R(Phi) C: rotate the wave's copy of C per pair
        for (int i = lane; i < NPR; i += 64) {
            const float2 cw = *reinterpret_cast<const float2*>(sCW + 2 * i);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float c0 = sC[(2 * i) * R + r], c1 = sC[(2 * i + 1) * R + r];
                sC[(2 * i) * R + r] = cw.x * c0 - cw.y * c1;
                sC[(2 * i + 1) * R + r] = cw.y * c0 + cw.x * c1;
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    float yacc[R][4];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int q = 0; q < 4; ++q) yacc[r][q] = 0.f;

    auto update_batch = [&](f32x4 (&hv)[kPB][2], int bt) {
#pragma unroll
        for (int k = 0; k < kPB; ++k) {
            const int j = kPB * bt + k;
            if (j < npl) {
                const int i = rg + RG * j;
                const float2 csn = *reinterpret_cast<const float2*>(sCS + 2 * i);
                RVec<R> bp0, bp1, b0, b1, c0, c1;
                bp0.load(sBp + (2 * i) * R); bp1.load(sBp + (2 * i + 1) * R);
                b0.load(sB + (2 * i) * R);   b1.load(sB + (2 * i + 1) * R);
                c0.load(sC + (2 * i) * R);   c1.load(sC + (2 * i + 1) * R);
                f32x4 n0v, n1v;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float up0 = 0.f, up1 = 0.f, u0 = 0.f, u1 = 0.f;
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        up0 += bp0.v[r] * xpv[r][q];
                        up1 += bp1.v[r] * xpv[r][q];
                        u0 += b0.v[r] * xv[r][q];
                        u1 += b1.v[r] * xv[r][q];
                    }
                    float n0, n1;
                    if (!no_write) {
                        // alpha R h + beta R U_prev = R (alpha h + beta U_prev)
                        const float a0 = alpha * hv[k][0][q] + beta * up0;
                        const float a1 = alpha * hv[k][1][q] + beta * up1;
                        n0 = csn.x * a0 - csn.y * a1 + gamma * u0;
                        n1 = csn.y * a0 + csn.x * a1 + gamma * u1;
                    } else {
                        // alpha R(dt theta) h + R(Phi) (beta U_prev + gamma U)
                        const float2 cw = *reinterpret_cast<const float2*>(sCW + 2 * i);
                        const float a0 = alpha * hv[k][0][q], a1 = alpha * hv[k][1][q];
                        const float w0 = beta * up0 + gamma * u0, w1 = beta * up1 + gamma * u1;
                        n0 = csn.x * a0 - csn.y * a1 + cw.x * w0 - cw.y * w1;
                        n1 = csn.y * a0 + csn.x * a1 + cw.y * w0 + cw.x * w1;
                    }
                    n0v[q] = n0;
                    n1v[q] = n1;
#pragma unroll
                    for (int r = 0; r < R; ++r) yacc[r][q] += c0.v[r] * n0 + c1.v[r] * n1;
                }
                f32x4* dst = reinterpret_cast<f32x4*>(hs + (int64_t)(2 * i) * P) + cg;
                dst[0] = n0v;
                dst[P4] = n1v;
            }
        }
    };

    // Batches alternate between two register sets; the next one's loads are
    // in flight while the current one is updated.
    for (int bt = 0; bt < nbat; bt += 2) {
        if (bt + 1 < nbat) load_batch(hb, bt + 1);
        update_batch(ha, bt);
        if (bt + 1 < nbat) {
            if (bt + 2 < nbat) load_batch(ha, bt + 2);
            update_batch(hb, bt + 1);
        }
    }

    // Readout: sum the row groups' partial products of each column.
#pragma unroll
    for (int off = P4; off < 64; off <<= 1)
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int q = 0; q < 4; ++q) yacc[r][q] += __shfl_xor(yacc[r][q], off, 64);
    if (rg == 0) {
        IO* y = reinterpret_cast<IO*>(p.y) + bh * R * P;
#pragma unroll
        for (int r = 0; r < R; ++r)
            gstore4(y + r * P + 4 * cg, f32x4{yacc[r][0], yacc[r][1], yacc[r][2], yacc[r][3]});
    }
}

// LDS slice of one wavefront: B_prev, B, C as [N][R] and the pair rotations
// (of this step's angle and of the accumulated angle).
size_t decode_wave_lds(int N, int R) { return sizeof(float) * (size_t)(3 * R * N + 2 * N); }

template <typename IO, int R, bool PM>
hipError_t launch_decode_t(const DecodeParams& p, hipStream_t stream)
{
    // Up to kDecWaves wavefronts per workgroup, as many as fit in LDS (the
    // largest supported shape, N = 1024 and R = 4, takes 56 KiB per wave).
    const size_t per_wave = decode_wave_lds(p.N, R);
    int waves = (int)((160 * 1024) / per_wave);
    if (waves > kDecWaves) waves = kDecWaves;
    auto* const kern = &decode_kernel<IO, R, PM>;
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (attr != hipSuccess) return attr;
    (void)hipGetLastError();
    const int64_t blocks = (p.nbh + waves - 1) / waves;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(64 * waves), per_wave * waves, stream, p);
    return hipGetLastError();
}

template <typename IO, int R>
hipError_t launch_decode_r(const DecodeParams& p, hipStream_t stream)
{
    return p.opt.premix ? launch_decode_t<IO, R, true>(p, stream) : launch_decode_t<IO, R, false>(p, stream);
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
        case 1: return launch_decode_r<float, 1>(p, stream);
        case 2: return launch_decode_r<float, 2>(p, stream);
        default: return launch_decode_r<float, 4>(p, stream);
        }
    }
    switch (p.R) {
    case 1: return launch_decode_r<bf16, 1>(p, stream);
    case 2: return launch_decode_r<bf16, 2>(p, stream);
    default: return launch_decode_r<bf16, 4>(p, stream);
    }
}

}  // namespace m3
