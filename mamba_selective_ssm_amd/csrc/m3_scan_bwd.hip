// Gradient of the Mamba-3 scan: a reverse-time recurrence over the adjoint
// state, with the forward states recomputed from checkpoints.
//
// Forward (Mamba-3 summary on b-lab.team, section 1 recurrence, section 2
// block rotations R(phi_i), phi = dt theta_i, on adjacent rows, section 3
// MIMO), per (b, h) and step t:
//   a_t = alpha_t h_{t-1} + beta_t U_{t-1},  h_t = R_t a_t + gamma_t U_t,
//   U_t = B_t X_t,  y_t = C_t^T h_t.
// Adjoint, t = L-1 .. 0 (g_t = dLoss/dh_t, da_t = dLoss/da_t):
//   g_t  = C_t dy_t + alpha_{t+1} da_{t+1}        (dh_out enters as da_L)
//   da_t = R_t^T g_t
//   dU_t = gamma_t g_t + beta_{t+1} da_{t+1}
//   dX_t = B_t^T dU_t,  dB_t = dU_t X_t^T,  dC_t = h_t dy_t^T
//   dalpha_t = <da_t, h_{t-1}>,  dbeta_t = <da_t, U_{t-1}>,  dgamma_t = <g_t, U_t>
//   dphi_t,i = sum_p (g1 r0 - g0 r1) over pair i, r = R_t a_t = h_t - gamma_t U_t
// and through alpha = e^{dt A}, beta = (1-lam) dt alpha, gamma = lam dt,
// phi_i = dt theta_i to dt, A, lam, theta.  The initial record gets
// dh_in = alpha_0 da_0 and dU_prev = beta_0 da_0.
//
// One workgroup per (b, h, part of PP = 16 KP rotation pairs); wave w owns
// headdim columns 16w .. 16w+15 of the part's rows (lane: 4 columns x the rows
// of pairs rg + 16k), so each wave reduces dX over its own rows, and the column
// sums (dB, dC, dphi and the scalar gradients) of the waves meet in LDS once
// per step (one barrier).  dX and the scalar sums of the parts are added in a
// second kernel in a fixed order (deterministic), which also maps the scalar
// sums to dt, lam and A.
// States: a checkpoint every T1 = K*TB steps in HBM (pass A); per superblock
// the K sub-block start states go to a scratch area (pass B1); per sub-block
// the TB step states are recomputed into the wave's LDS slots (pass B2) and
// the adjoint steps run backward over them.  Each lane only reads back what
// it wrote (checkpoints, scratch and LDS slots), so those need no barriers.
// The inputs of a superblock's steps (and of the step before it) are staged
// in LDS by the whole workgroup with one batch of 16-byte loads, so the
// sequential steps read them at LDS latency instead of waiting on memory.
#include "m3_device.hpp"
#include "m3_internal.hpp"

namespace m3 {
namespace {

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;

__device__ __forceinline__ float2 ld2(const bf16* p) {
    const bf16x2 v = *reinterpret_cast<const bf16x2*>(p);
    return make_float2((float)v[0], (float)v[1]);
}
__device__ __forceinline__ float2 ld2(const float* p) { return *reinterpret_cast<const float2*>(p); }
__device__ __forceinline__ void ld4(float (&d)[4], const bf16* p) {
    const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) d[e] = (float)v[e];
}
__device__ __forceinline__ void ld4(float (&d)[4], const float* p) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) d[e] = v[e];
}

// Cross-lane sums on the DPP paths (no LDS round trip): over the 4 lanes of
// a quad (one row group's columns), over the lanes of a 16-lane row with the
// same lane % 4, and over the whole wave (inclusive scan, then lane 63).
__device__ __forceinline__ float quad_sum(float v)
{
    v += dpp_moved<0xB1, 0xf>(v);   // quad_perm [1,0,3,2]
    v += dpp_moved<0x4E, 0xf>(v);   // quad_perm [2,3,0,1]
    return v;
}
__device__ __forceinline__ float row_class_sum(float v)
{
    v += dpp_moved<0x124, 0xf>(v);  // row_ror:4
    v += dpp_moved<0x128, 0xf>(v);  // row_ror:8
    return v;
}
__device__ __forceinline__ float wave_sum(float v) { return wave_read_lane(wave_inclusive_sum(v), 63); }

template <int R, int KP> struct StepIn {
    float B[KP][R][2];    // rows 2i, 2i+1 of this lane's pairs
    float X[R][4];        // this lane's 4 columns
};

template <typename IO, int R, int KP, int TB>
__global__ __launch_bounds__(256) void bwd_kernel(const BwdParams p)
{
    extern __shared__ __attribute__((aligned(16))) float bsm[];
    constexpr int E = 8 * KP;                     // state elements per lane
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int NW = blockDim.x >> 6, NT = blockDim.x, tid = threadIdx.x;
    const int N = p.N, NPR = N / 2, P = p.P;
    const int64_t L = p.L, H = p.H;
    constexpr int PP = 16 * KP;                   // pairs of one part
    const int part = blockIdx.x % p.parts;
    const int bh = blockIdx.x / p.parts;
    int64_t b, h;
    split_bh(bh, H, b, h);
    const int p_lo = part * PP;                   // first pair of this part
    const int NPRp = NPR - p_lo < PP ? NPR - p_lo : PP;
    const int cg = lane & 3, rg = lane >> 2;
    const int col0 = 16 * wv + 4 * cg;
    const int V = 4 * R * PP + PP + 4;            // per-wave partial sums of one step
    float* slots = bsm + (size_t)wv * TB * E * 64;               // this wave's step states
    float* red = bsm + (size_t)NW * TB * E * 64;                 // [2][NW][V]
    // Staged step inputs, per step: the part's rows of B, C [R][2 PP] and X,
    // dy [R][P] (io), then float32 [dt, lam, alpha, beta, gamma, -, -, -],
    // theta, cos phi, sin phi [PP each]; a step's block is SB bytes.
    constexpr int ESZ = (int)sizeof(IO);
    const int oC = ESZ * R * 2 * PP, oX = 2 * oC, oDY = oX + ESZ * R * P;
    const int oSC = oDY + ESZ * R * P;
    const int SB = (oSC + 4 * (8 + 3 * PP) + 15) / 16 * 16;
    unsigned char* stg = reinterpret_cast<unsigned char*>(red + 2 * (size_t)NW * V);
    int64_t stg_t0 = 0;                                          // step held in block 0

    const IO* Xg = reinterpret_cast<const IO*>(p.x);
    const IO* Bg = reinterpret_cast<const IO*>(p.B);
    const IO* Cg = reinterpret_cast<const IO*>(p.C);
    const IO* dYg = reinterpret_cast<const IO*>(p.dy);
    const IO* Bpr = reinterpret_cast<const IO*>(p.Bp_in);
    const IO* Xpr = reinterpret_cast<const IO*>(p.xp_in);
    const float A = p.a_tok ? 0.f : p.A[h];
    auto tok = [&](int64_t t) -> int64_t { return (b * L + t) * H + h; };
    auto lp_of = [&](int k) { return rg + 16 * k; };             // pair within the part
    auto pair_of = [&](int k) { return p_lo + rg + 16 * k; };    // pair of the state
    auto pvalid = [&](int k) { return rg + 16 * k < NPRp; };

    // Stage steps t0 .. t0+cnt-1 (t0 may be -1: the state record's previous
    // token, or zeros) into LDS; every thread of the workgroup takes part.
    auto stage = [&](int64_t t0, int cnt) {
        __syncthreads();                                         // previous block's readers done
        stg_t0 = t0;
        const int q_io = (2 * oC + 2 * ESZ * R * P) / 16;          // 16-byte pieces per step
        const int rowb = ESZ * 2 * PP;                           // staged bytes of one B/C row
        for (int idx = tid; idx < cnt * q_io; idx += NT) {
            const int sidx = idx / q_io, piece = idx % q_io;
            const int64_t t = t0 + sidx;
            const int off = piece * 16;                          // byte offset in the step block
            const unsigned char* src = nullptr;
            if (off < oX) {                                      // the part's rows of B or C
                const int m = off / oC, o = off % oC, r = o / rowb, ob = o % rowb;
                const int64_t go = (int64_t)ESZ * (r * N + 2 * p_lo) + ob;
                if (ob < ESZ * 2 * NPRp) {
                    if (t >= 0) src = reinterpret_cast<const unsigned char*>(m == 0 ? Bg : Cg) + tok(t) * (int64_t)(ESZ * R * N) + go;
                    else if (m == 0 && Bpr != nullptr) src = reinterpret_cast<const unsigned char*>(Bpr) + (int64_t)bh * (ESZ * R * N) + go;
                }
            } else {                                             // X or dy
                const int m = (off - oX) / (ESZ * R * P), o = (off - oX) % (ESZ * R * P);
                if (t >= 0) src = reinterpret_cast<const unsigned char*>(m == 0 ? Xg : dYg) + tok(t) * (int64_t)(ESZ * R * P) + o;
                else if (m == 0 && Xpr != nullptr) src = reinterpret_cast<const unsigned char*>(Xpr) + (int64_t)bh * (ESZ * R * P) + o;
            }
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (src != nullptr) v = *reinterpret_cast<const uint4*>(src);
            *reinterpret_cast<uint4*>(stg + (size_t)sidx * SB + off) = v;
        }
        // per-step scalars and per-pair rotations, computed once per stage
        for (int idx = tid; idx < cnt * (PP + 1); idx += NT) {
            const int sidx = idx / (PP + 1), j = idx % (PP + 1);
            const int64_t t = t0 + sidx;
            float* f = reinterpret_cast<float*>(stg + (size_t)sidx * SB + oSC);
            const float d = t >= 0 ? p.dt[tok(t)] : 0.f;
            if (j == PP) {
                const float lm = t >= 0 ? p.lam[tok(t)] : 0.f;
                const float al = expf(d * (p.a_tok && t >= 0 ? p.A[tok(t)] : A));
                f[0] = d;
                f[1] = lm;
                f[2] = al;
                f[3] = (1.f - lm) * d * al;
                f[4] = lm * d;
            } else {
                const float th = (t >= 0 && j < NPRp) ? p.theta[tok(t) * NPR + p_lo + j] : 0.f;
                float sn, cs;
                sincosf(d * th, &sn, &cs);
                f[8 + j] = th;
                f[8 + PP + j] = cs;
                f[8 + 2 * PP + j] = sn;
            }
        }
        __syncthreads();
    };
    auto blk = [&](int64_t t) { return stg + (size_t)(t - stg_t0) * SB; };
    auto io_at = [&](const unsigned char* base, int o) -> const IO* {
        return reinterpret_cast<const IO*>(base + o);
    };
    // Inputs of a staged step t (t = -1 allowed when staged).
    auto load_in = [&](int64_t t, StepIn<R, KP>& s) {
        const unsigned char* bb = blk(t);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            ld4(s.X[r], io_at(bb, oX) + r * P + col0);
#pragma unroll
            for (int k = 0; k < KP; ++k) {
                const float2 v = ld2(io_at(bb, 0) + r * 2 * PP + 2 * lp_of(k));
                s.B[k][r][0] = v.x;                              // zero-padded past the part's pairs
                s.B[k][r][1] = v.y;
            }
        }
    };
    auto outer = [&](const StepIn<R, KP>& s, float (&U)[E]) {
#pragma unroll
        for (int k = 0; k < KP; ++k)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float u = 0.f;
#pragma unroll
                    for (int r = 0; r < R; ++r) u += s.B[k][r][j] * s.X[r][q];
                    U[(k * 2 + j) * 4 + q] = u;
                }
    };
    struct Sc { float d, lm, al, be, ga, cs[KP], sn[KP], th[KP]; };
    auto scalars = [&](int64_t t, Sc& c) {
        const float* f = reinterpret_cast<const float*>(blk(t) + oSC);
        const f32x4 s4 = *reinterpret_cast<const f32x4*>(f);
        c.d = s4[0];
        c.lm = s4[1];
        c.al = s4[2];
        c.be = s4[3];
        c.ga = f[4];
#pragma unroll
        for (int k = 0; k < KP; ++k) {
            const int i = lp_of(k);
            c.th[k] = f[8 + i];                                  // zero past the part's pairs
            c.cs[k] = f[8 + PP + i];
            c.sn[k] = f[8 + 2 * PP + i];
        }
    };
    // One forward step on this lane's elements: hs <- R(alpha hs + beta Uprev) + gamma U.
    auto fwd_step = [&](int64_t t, float (&hs)[E], float (&Uprev)[E]) {
        Sc c;
        scalars(t, c);
        StepIn<R, KP> s;
        load_in(t, s);
        float U[E];
        outer(s, U);
#pragma unroll
        for (int k = 0; k < KP; ++k)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int e0 = (k * 2) * 4 + q, e1 = (k * 2 + 1) * 4 + q;
                const float a0 = c.al * hs[e0] + c.be * Uprev[e0];
                const float a1 = c.al * hs[e1] + c.be * Uprev[e1];
                hs[e0] = c.cs[k] * a0 - c.sn[k] * a1 + c.ga * U[e0];
                hs[e1] = c.sn[k] * a0 + c.cs[k] * a1 + c.ga * U[e1];
            }
#pragma unroll
        for (int e = 0; e < E; ++e) Uprev[e] = U[e];
    };
    // Lane-ordered state storage (16-byte pieces, consecutive lanes adjacent).
    auto st_state = [&](float* base, const float (&hs)[E]) {
#pragma unroll
        for (int e4 = 0; e4 < E / 4; ++e4)
            *reinterpret_cast<f32x4*>(base + ((size_t)e4 * 64 + lane) * 4) =
                f32x4{hs[4 * e4], hs[4 * e4 + 1], hs[4 * e4 + 2], hs[4 * e4 + 3]};
    };
    auto ld_state = [&](const float* base, float (&hs)[E]) {
#pragma unroll
        for (int e4 = 0; e4 < E / 4; ++e4) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(base + ((size_t)e4 * 64 + lane) * 4);
#pragma unroll
            for (int q = 0; q < 4; ++q) hs[4 * e4 + q] = v[q];
        }
    };
    const size_t unit_sz = (size_t)NW * E * 64;                 // = N * P floats (padded pairs)
    const int64_t T1 = (int64_t)p.K * TB;
    const int64_t nsup = (L + T1 - 1) / T1;
    float* ck = p.ckpt + (size_t)blockIdx.x * (size_t)(nsup > 0 ? nsup : 1) * unit_sz + (size_t)wv * E * 64;
    float* sc = p.scr + (size_t)blockIdx.x * p.K * unit_sz + (size_t)wv * E * 64;
    // ck/sc point at this wave's part of entry 0; entry j adds j * unit_sz.

    // ---- pass A: checkpoints every T1 steps ------------------------------
    float hs[E], Up[E];
#pragma unroll
    for (int k = 0; k < KP; ++k)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = 2 * (pvalid(k) ? pair_of(k) : 0) + j;
                hs[(k * 2 + j) * 4 + q] =
                    (p.h_in != nullptr && pvalid(k)) ? p.h_in[((int64_t)bh * N + n) * P + col0 + q] : 0.f;
            }
    if (nsup > 0) st_state(ck, hs);
    for (int64_t sup = 0; sup < nsup; ++sup) {
        const int64_t s0 = sup * T1, s1 = s0 + T1 < L ? s0 + T1 : L;
        stage(s0 - 1, (int)(s1 - s0 + 1));
        {
            StepIn<R, KP> s;
            load_in(s0 - 1, s);
            outer(s, Up);
        }
        for (int64_t t = s0; t < s1; ++t) fwd_step(t, hs, Up);
        if (s1 < L) st_state(ck + (size_t)(sup + 1) * unit_sz, hs);
    }

    // ---- pass B: adjoint, superblocks and sub-blocks from the end --------
    // A virtual step L with alpha = 1, no rotation and beta = 0 carries dh_out.
    float dan[E];
#pragma unroll
    for (int k = 0; k < KP; ++k)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = 2 * (pvalid(k) ? pair_of(k) : 0) + j;
                dan[(k * 2 + j) * 4 + q] = (p.dh_out != nullptr && pvalid(k))
                    ? p.dh_out[((int64_t)bh * N + n) * P + col0 + q] : 0.f;
            }
    float a_nx = 1.f, b_nx = 0.f;
    int par = 0;

    for (int64_t sup = nsup - 1; sup >= 0; --sup) {
        const int64_t s0 = sup * T1, s1 = s0 + T1 < L ? s0 + T1 : L;
        const int nsub = (int)((s1 - s0 + TB - 1) / TB);
        stage(s0 - 1, (int)(s1 - s0 + 1));
        // B1: sub-block start states of this superblock
        ld_state(ck + (size_t)sup * unit_sz, hs);
        {
            StepIn<R, KP> s;
            load_in(s0 - 1, s);
            outer(s, Up);
        }
        for (int sb = 0; sb < nsub; ++sb) {
            st_state(sc + (size_t)sb * unit_sz, hs);
            const int64_t tA = s0 + (int64_t)sb * TB, tB = tA + TB < s1 ? tA + TB : s1;
            for (int64_t t = tA; t < tB; ++t) fwd_step(t, hs, Up);
        }
        for (int sb = nsub - 1; sb >= 0; --sb) {
            const int64_t tA = s0 + (int64_t)sb * TB, tB = tA + TB < s1 ? tA + TB : s1;
            // B2: the sub-block's step states into this wave's LDS slots
            float hb[E];
            ld_state(sc + (size_t)sb * unit_sz, hs);
            {
                StepIn<R, KP> s;
                load_in(tA - 1, s);
                outer(s, Up);
            }
#pragma unroll
            for (int e = 0; e < E; ++e) hb[e] = hs[e];
            for (int64_t t = tA; t < tB; ++t) {
                fwd_step(t, hs, Up);
                st_state(slots + (size_t)(t - tA) * E * 64, hs);
            }
            // adjoint steps tB-1 .. tA
            for (int64_t t = tB - 1; t >= tA; --t) {
                Sc c;
                scalars(t, c);
                StepIn<R, KP> cur, prv;
                load_in(t, cur);
                load_in(t - 1, prv);
                float Cv[KP][R][2], dyv[R][4];
                {
                    const unsigned char* bb = blk(t);
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        ld4(dyv[r], io_at(bb, oDY) + r * P + col0);
#pragma unroll
                        for (int k = 0; k < KP; ++k) {
                            const float2 v = ld2(io_at(bb, oC) + r * 2 * PP + 2 * lp_of(k));
                            Cv[k][r][0] = v.x;
                            Cv[k][r][1] = v.y;
                        }
                    }
                }
                float ht[E], hp[E], Ut[E], Upv[E];
                ld_state(slots + (size_t)(t - tA) * E * 64, ht);
                if (t > tA) ld_state(slots + (size_t)(t - tA - 1) * E * 64, hp);
                else {
#pragma unroll
                    for (int e = 0; e < E; ++e) hp[e] = hb[e];
                }
                outer(cur, Ut);
                outer(prv, Upv);
                float g[E], da[E], dU[E];
#pragma unroll
                for (int k = 0; k < KP; ++k)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int e = (k * 2 + j) * 4 + q;
                            float v = a_nx * dan[e];
#pragma unroll
                            for (int r = 0; r < R; ++r) v += Cv[k][r][j] * dyv[r][q];
                            g[e] = v;
                        }
                float s_a = 0.f, s_b = 0.f, s_g = 0.f, s_th = 0.f;
                float dph[KP];
#pragma unroll
                for (int k = 0; k < KP; ++k) {
                    float acc = 0.f;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int e0 = (k * 2) * 4 + q, e1 = (k * 2 + 1) * 4 + q;
                        da[e0] = c.cs[k] * g[e0] + c.sn[k] * g[e1];     // R^T g
                        da[e1] = -c.sn[k] * g[e0] + c.cs[k] * g[e1];
                        const float r0 = ht[e0] - c.ga * Ut[e0], r1 = ht[e1] - c.ga * Ut[e1];
                        acc += g[e1] * r0 - g[e0] * r1;
                    }
                    dph[k] = acc;
                    s_th += c.th[k] * acc;
                }
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    dU[e] = c.ga * g[e] + b_nx * dan[e];
                    s_a += da[e] * hp[e];
                    s_b += da[e] * Upv[e];
                    s_g += g[e] * Ut[e];
                }
                float dBp[KP][R][2], dCp[KP][R][2], dXp[R][4];
#pragma unroll
                for (int k = 0; k < KP; ++k)
#pragma unroll
                    for (int r = 0; r < R; ++r)
#pragma unroll
                        for (int j = 0; j < 2; ++j) {
                            float sb_ = 0.f, sc_ = 0.f;
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                const int e = (k * 2 + j) * 4 + q;
                                sb_ += dU[e] * cur.X[r][q];
                                sc_ += ht[e] * dyv[r][q];
                            }
                            dBp[k][r][j] = sb_;
                            dCp[k][r][j] = sc_;
                        }
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        float v = 0.f;
#pragma unroll
                        for (int k = 0; k < KP; ++k)
#pragma unroll
                            for (int j = 0; j < 2; ++j) v += cur.B[k][r][j] * dU[(k * 2 + j) * 4 + q];
                        dXp[r][q] = v;
                    }
                // column sums within the wave: over the 4 lanes of a row group
#pragma unroll
                for (int k = 0; k < KP; ++k) {
                    dph[k] = quad_sum(dph[k]);
#pragma unroll
                    for (int r = 0; r < R; ++r)
#pragma unroll
                        for (int j = 0; j < 2; ++j) {
                            dBp[k][r][j] = quad_sum(dBp[k][r][j]);
                            dCp[k][r][j] = quad_sum(dCp[k][r][j]);
                        }
                }
                // row sums within the wave: over the 16 row groups (4 per
                // 16-lane row on DPP, then across the 4 rows)
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        float v = row_class_sum(dXp[r][q]);
                        v += __shfl_xor(v, 16, 64);
                        v += __shfl_xor(v, 32, 64);
                        dXp[r][q] = v;
                    }
                s_a = wave_sum(s_a);
                s_b = wave_sum(s_b);
                s_g = wave_sum(s_g);
                s_th = wave_sum(s_th);
                const int64_t tk = tok(t);
                if (rg == 0) {                                   // this part's share of dX
#pragma unroll
                    for (int r = 0; r < R; ++r)
                        *reinterpret_cast<f32x4*>(p.dx_part + ((size_t)part * p.ntok + tk) * R * P + r * P + col0) =
                            f32x4{dXp[r][0], dXp[r][1], dXp[r][2], dXp[r][3]};
                }
                float* rb = red + ((size_t)par * NW + wv) * V;
                if (cg == 0) {
#pragma unroll
                    for (int k = 0; k < KP; ++k) {
                        const int i = lp_of(k);
#pragma unroll
                        for (int r = 0; r < R; ++r) {
                            *reinterpret_cast<float2*>(rb + r * 2 * PP + 2 * i) =
                                make_float2(dBp[k][r][0], dBp[k][r][1]);
                            *reinterpret_cast<float2*>(rb + 2 * R * PP + r * 2 * PP + 2 * i) =
                                make_float2(dCp[k][r][0], dCp[k][r][1]);
                        }
                        rb[4 * R * PP + i] = dph[k];
                    }
                }
                if (lane == 0)
                    *reinterpret_cast<f32x4*>(rb + 4 * R * PP + PP) = f32x4{s_a, s_b, s_g, s_th};
                __syncthreads();
                // sums over the waves (column slices); buffers alternate by step
                const float* r0b = red + (size_t)par * NW * V;
                for (int v = tid; v < 4 * R * PP + PP + 4; v += NT) {
                    float sum = 0.f;
                    for (int w = 0; w < NW; ++w) sum += r0b[(size_t)w * V + v];
                    if (v < 4 * R * PP) {
                        const int m = v / (2 * R * PP), o = v % (2 * R * PP), r = o / (2 * PP), ro = o % (2 * PP);
                        if (ro < 2 * NPRp) (m == 0 ? p.dB : p.dC)[tk * R * N + r * N + 2 * p_lo + ro] = sum;
                    } else if (v < 4 * R * PP + PP) {
                        const int i = v - 4 * R * PP;
                        if (i < NPRp) p.dtheta[tk * NPR + p_lo + i] = c.d * sum;
                    } else {                                     // this part's scalar sums
                        p.scal[((size_t)part * p.ntok + tk) * 4 + (v - 4 * R * PP - PP)] = sum;
                    }
                }
                par ^= 1;
#pragma unroll
                for (int e = 0; e < E; ++e) dan[e] = da[e];
                a_nx = c.al;
                b_nx = c.be;
            }
        }
    }

    // ---- the state record's gradients -------------------------------------
    if (p.dh_in != nullptr) {
#pragma unroll
        for (int k = 0; k < KP; ++k)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                if (pvalid(k)) {
                    const int n = 2 * pair_of(k) + j;
                    const int e = (k * 2 + j) * 4;
                    *reinterpret_cast<f32x4*>(p.dh_in + ((int64_t)bh * N + n) * P + col0) =
                        f32x4{a_nx * dan[e], a_nx * dan[e + 1], a_nx * dan[e + 2], a_nx * dan[e + 3]};
                }
        stage(-1, 1);
        StepIn<R, KP> s;
        load_in(-1, s);
        float dXp[R][4], dBp[KP][R][2];
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float v = 0.f;
#pragma unroll
                for (int k = 0; k < KP; ++k)
#pragma unroll
                    for (int j = 0; j < 2; ++j) v += s.B[k][r][j] * b_nx * dan[(k * 2 + j) * 4 + q];
                dXp[r][q] = v;
            }
#pragma unroll
            for (int k = 0; k < KP; ++k)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    float v = 0.f;
#pragma unroll
                    for (int q = 0; q < 4; ++q) v += b_nx * dan[(k * 2 + j) * 4 + q] * s.X[r][q];
                    dBp[k][r][j] = v;
                }
        }
#pragma unroll
        for (int off = 4; off < 64; off <<= 1)
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int q = 0; q < 4; ++q) dXp[r][q] += __shfl_xor(dXp[r][q], off, 64);
#pragma unroll
        for (int off = 1; off < 4; off <<= 1)
#pragma unroll
            for (int k = 0; k < KP; ++k)
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int j = 0; j < 2; ++j) dBp[k][r][j] += __shfl_xor(dBp[k][r][j], off, 64);
        if (rg == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r)
                *reinterpret_cast<f32x4*>(p.dxprev_part + ((size_t)part * p.nbh + bh) * R * P + r * P + col0) =
                    f32x4{dXp[r][0], dXp[r][1], dXp[r][2], dXp[r][3]};
        }
        float* rb = red + ((size_t)par * NW + wv) * V;
        if (cg == 0) {
#pragma unroll
            for (int k = 0; k < KP; ++k)
#pragma unroll
                for (int r = 0; r < R; ++r)
                    *reinterpret_cast<float2*>(rb + r * 2 * PP + 2 * lp_of(k)) =
                        make_float2(dBp[k][r][0], dBp[k][r][1]);
        }
        __syncthreads();
        const float* r0b = red + (size_t)par * NW * V;
        for (int v = tid; v < 2 * R * PP; v += NT) {
            float sum = 0.f;
            for (int w = 0; w < NW; ++w) sum += r0b[(size_t)w * V + v];
            const int r = v / (2 * PP), ro = v % (2 * PP);
            if (ro < 2 * NPRp) p.dBp[(int64_t)bh * R * N + r * N + 2 * p_lo + ro] = sum;
        }
    }
}

// Per (b, h): dX and the scalar sums of the pair parts added in part order,
// the scalar sums mapped through alpha = e^{dt A}, beta = (1-lam) dt alpha,
// gamma = lam dt (and phi = dt theta) to dt and lam, and this unit's share of
// dA; the record's dx_prev likewise.
template <int R>
__global__ __launch_bounds__(256) void bwd_finalize_kernel(const BwdParams p)
{
    const int bh = blockIdx.x, tid = threadIdx.x;
    const int64_t H = p.H, L = p.L;
    int64_t b, h;
    split_bh(bh, H, b, h);
    const int P = p.P, S = p.parts;
    const int64_t RP4 = (int64_t)R * P / 4;
    for (int64_t idx = tid; idx < L * RP4; idx += 256) {
        const int64_t t = idx / RP4, q = idx % RP4;
        const int64_t tk = (b * L + t) * H + h;
        f32x4 sum = {0.f, 0.f, 0.f, 0.f};
        for (int k = 0; k < S; ++k)
            sum += *reinterpret_cast<const f32x4*>(p.dx_part + ((size_t)k * p.ntok + tk) * R * P + 4 * q);
        *reinterpret_cast<f32x4*>(p.dx + tk * R * P + 4 * q) = sum;
    }
    float dA_acc = 0.f;
    for (int64_t t = tid; t < L; t += 256) {
        const int64_t tk = (b * L + t) * H + h;
        f32x4 sc = {0.f, 0.f, 0.f, 0.f};      // dalpha, dbeta, dgamma, sum_i theta_i dphi_i
        for (int k = 0; k < S; ++k) sc += *reinterpret_cast<const f32x4*>(p.scal + ((size_t)k * p.ntok + tk) * 4);
        const float A = p.A[p.a_tok ? tk : h];
        const float d = p.dt[tk], lm = p.lam[tk], al = expf(d * A);
        p.ddt[tk] = sc[0] * al * A + sc[1] * (1.f - lm) * al * (1.f + d * A) + sc[2] * lm + sc[3];
        p.dlam[tk] = -d * al * sc[1] + d * sc[2];
        const float dAk = sc[0] * al * d + sc[1] * (1.f - lm) * d * d * al;
        if (p.a_tok) p.dAt[tk] = dAk;                 // a per-token rate: its own gradient
        dA_acc += dAk;
    }
    if (p.dxp != nullptr) {
        for (int64_t q = tid; q < RP4; q += 256) {
            f32x4 sum = {0.f, 0.f, 0.f, 0.f};
            for (int k = 0; k < S; ++k)
                sum += *reinterpret_cast<const f32x4*>(p.dxprev_part + ((size_t)k * p.nbh + bh) * R * P + 4 * q);
            *reinterpret_cast<f32x4*>(p.dxp + (int64_t)bh * R * P + 4 * q) = sum;
        }
    }
    // this unit's dA share: a fixed-order tree over the workgroup
    __shared__ float red[256];
    red[tid] = dA_acc;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (tid < w) red[tid] += red[tid + w];
        __syncthreads();
    }
    if (tid == 0) p.dA_part[bh] = red[0];
}

// dA[h] = sum over the batch rows of the units' shares (fixed order).
__global__ void bwd_dA_kernel(const float* part, float* dA, int64_t batch, int64_t H)
{
    const int64_t h = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (h >= H) return;
    float s = 0.f;
    for (int64_t b = 0; b < batch; ++b) s += part[b * H + h];
    dA[h] = s;
}

// LDS of one workgroup: step states, the per-step partial sums and the
// staged inputs of T1 + 1 steps (16 pairs per part: KP = 1).
constexpr int kBwdPP = 16;
constexpr size_t kBwdLds = 80 * 1024;     // two workgroups per compute unit
size_t bwd_fixed_lds(int64_t N, int64_t P, int64_t R)
{
    (void)N;
    const int TB = bwd_sub_steps(N);
    const int64_t NW = P / 16;
    return sizeof(float) * ((size_t)NW * TB * 8 * 64 + 2 * (size_t)NW * (4 * R * kBwdPP + kBwdPP + 4));
}
size_t bwd_step_bytes(int64_t N, int64_t P, int64_t R, int io)
{
    (void)N;
    const int64_t e = io == 0 ? 4 : 2;
    return (size_t)((4 * e * R * kBwdPP + 2 * e * R * P + 4 * (8 + 3 * kBwdPP) + 15) / 16 * 16);
}

template <typename IO, int R, int KP, int TB>
hipError_t launch_bwd_t(const BwdParams& p, float* dA, hipStream_t stream)
{
    const int NW = p.P / 16;
    const size_t lds = bwd_fixed_lds(p.N, p.P, R) +
                       (size_t)(p.K * TB + 1) * bwd_step_bytes(p.N, p.P, R, sizeof(IO) == 4 ? 0 : 1);
    auto* kern = &bwd_kernel<IO, R, KP, TB>;
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (attr != hipSuccess) return attr;
    (void)hipGetLastError();
    hipLaunchKernelGGL(kern, dim3((unsigned)(p.nbh * p.parts)), dim3(64 * NW), lds, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_finalize_kernel<R>, dim3((unsigned)p.nbh), dim3(256), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (p.a_tok) return hipSuccess;               // dA was written per token
    const int64_t batch = p.nbh / p.H;
    hipLaunchKernelGGL(bwd_dA_kernel, dim3((unsigned)((p.H + 63) / 64)), dim3(64), 0, stream,
                       (const float*)p.dA_part, dA, batch, p.H);
    return hipGetLastError();
}

template <typename IO, int R>
hipError_t launch_bwd_r(const BwdParams& p, float* dA, hipStream_t stream)
{
    return launch_bwd_t<IO, R, 1, 4>(p, dA, stream);
}

}  // namespace

int bwd_sub_steps(int64_t N) { (void)N; return 4; }

int bwd_pair_parts(int64_t N) { return (int)((N / 2 + kBwdPP - 1) / kBwdPP); }

int bwd_blocks_per_checkpoint(int64_t N, int64_t P, int64_t R, int io_dtype)
{
    const size_t avail = kBwdLds - bwd_fixed_lds(N, P, R);
    const int64_t steps = (int64_t)(avail / bwd_step_bytes(N, P, R, io_dtype)) - 1;
    const int64_t K = steps / bwd_sub_steps(N);
    return (int)(K > 8 ? 8 : K);
}

bool bwd_supported(int64_t N, int64_t P, int64_t R, int io_dtype)
{
    if (io_dtype != 0 && io_dtype != 1) return false;
    if (R != 1 && R != 2 && R != 4) return false;
    if (N < 8 || N > 128 || (N % 8) != 0) return false;
    if (P != 16 && P != 32 && P != 64) return false;
    return bwd_blocks_per_checkpoint(N, P, R, io_dtype) >= 1;
}

hipError_t launch_bwd(const BwdParams& p, int io_dtype, float* dA, hipStream_t stream)
{
    if (io_dtype == 0) {
        switch (p.R) {
        case 1: return launch_bwd_r<float, 1>(p, dA, stream);
        case 2: return launch_bwd_r<float, 2>(p, dA, stream);
        default: return launch_bwd_r<float, 4>(p, dA, stream);
        }
    }
    switch (p.R) {
    case 1: return launch_bwd_r<bf16, 1>(p, dA, stream);
    case 2: return launch_bwd_r<bf16, 2>(p, dA, stream);
    default: return launch_bwd_r<bf16, 4>(p, dA, stream);
    }
}

}  // namespace m3
