// Gradient of the Mamba-3 scan in chunked (SSD) form on gfx950.
//
// Forward, per (b, h), in the augmented state g_t = h_t + bhat_{t+1} U_t,
// bhat_t = (1 - lam_t) dt_t, U_t = B_t X_t (the exact rewrite the prefill
// kernel evaluates; Mamba-3 summary on b-lab.team, sections 1-3):
//   g_t = alpha_t R_t g_{t-1} + w_t U_t,   w_t = gamma_t + bhat_{t+1},
//   y_t = C_t^T (alpha_t R_t g_{t-1} + gamma_t U_t).
// For a chunk of Q tokens with chunk-local prefix sums Lam_j = sum_{k<=j} dt_k A
// and Phi_j = sum_{k<=j} dt_k theta_k (per pair), and rotated rows
// Bbar_j = R(Phi_j)^T B_j, Cbar_j = R(Phi_j)^T C_j (data-dependent RoPE):
//   y_j   = e^{Lam_j} Cbar_j^T G_in + sum_{k<=j} M_jk (Cbar_j^T Bbar_k) X_k,
//   M_jk  = e^{Lam_j - Lam_k} w_k (k < j),  gamma_j (k = j),
//   G_out = R(Phi_tot) (e^{Lam_tot} G_in + sum_k d_k Bbar_k X_k),
//   d_k   = e^{Lam_tot - Lam_k} w_k.
// Reverse mode of that form (dGbar = R(Phi_tot)^T dG_out, S = Cbar Bbar^T,
// dS = (dY X^T) o M, P = (dY X^T) o S o M):
//   dG_in  = e^{Lam_tot} dGbar + sum_j e^{Lam_j} Cbar_j dY_j
//   dX     = (S o M)^T dY + diag(d) Bbar dGbar^T
//   dBbar  = dS^T Cbar + diag(d) X dGbar^T
//   dCbar  = dS Bbar + diag(e^{Lam}) dY G_in^T
//   dLam_j = sum_{k<j} P_jk - sum_{i>j} P_ij + e^{Lam_j} <Cbar_j, dY_j G_in^T>
//            - d_j dd_j,  dd_j = <Bbar_j, X_j dGbar^T>
//            (+ <Gbar_out, dGbar> = e^{Lam_tot} <G_in, dGbar> + sum_k d_k dd_k
//            at the last token)
//   dPhi_j = per pair and summed over ranks, dBbar_0 Bbar_1 - dBbar_1 Bbar_0
//            + dCbar_0 Cbar_1 - dCbar_1 Cbar_0
//            (+ sum_p Gbar_out,0 dGbar_1 - Gbar_out,1 dGbar_0 at the last token,
//            split the same way into the G_in term and the per-token terms)
//   dB = R(Phi) dBbar, dC = R(Phi) dCbar; suffix sums over the chunk turn dLam
//   and dPhi into the gradients of dt A and dt theta; then dt, lam, theta and A
//   follow from gamma = lam dt and w_k = gamma_k + (1 - lam_{k+1}) dt_{k+1}.
//
// Kernels (one launch each, in stream order):
//   bc_local_kernel  per (b, h, chunk): Bbar^T diag(d) X and Cbar^T diag(e^Lam)
//                    dY on matrix cores, e^{Lam_tot} and the total rotation.
//   bc_scan_kernel   per (b, h, pair, column): the chunk-start states forward
//                    and the chunk-end adjoints backward (elementwise).
//   bc_grad_kernel   per (b, h, chunk): every gradient of the chunk from its
//                    boundary states; wave w owns operand rows 16w..16w+15.
//   bc_final_kernel  per (b, h): the look-ahead weight's gradient across chunk
//                    boundaries, the state record's gradients, dA shares.
//   bc_dA_kernel     per head: dA summed over the batch in a fixed order.
// Every sum runs in a fixed order: the result is deterministic.
#pragma once

#include "m3_device.hpp"
#include "m3_internal.hpp"
#include "m3_timeline.hpp"

namespace m3 {
namespace bc {

template <typename OP, int N_, int P_, int R_>
struct Cfg {
    using op_t = OP;                             // matrix-core operands and stored boundary states
    static constexpr int N = N_, P = P_, R = R_;
    static constexpr int T = 64;                 // operand rows per chunk (tokens x ranks)
    static constexpr int Q = T / R;              // tokens per chunk
    static constexpr int NPR = N / 2;            // rotation pairs
    static constexpr int E = (int)sizeof(OP);
    static constexpr bool BF = (E == 2);
    static constexpr int PAD = 16 / E;           // 16-byte row padding
    static constexpr int LDN = N + PAD, LDP = P + PAD, LDT = T + PAD, LDH = NPR + 1;
    static constexpr int NT = N / 16, PT = P / 16, NB = N / 32, PB = P / 32;
    static constexpr int VE = 16 / E;            // elements per 16-byte vector
    static constexpr int TS = 72;                // floats per token-scalar slot
    // Output columns split NS ways: wave w owns row tile w % 4 and column part
    // w / 4.  Four parts where the operand tiles leave one workgroup per
    // compute unit (dstate 128), else two.
    static constexpr int NS = (N == 128 && P == 64) ? 4 : 2;
    static constexpr int NW = 4 * NS, NTHR = 64 * NW;   // waves / threads per workgroup
    static_assert(N % 32 == 0 && P % 32 == 0, "K blocks of 32");
    static_assert(NT % NS == 0 && PT % NS == 0, "column parts");
};

// Token-scalar slots (TS floats each).  Partial sums carry one slot per row
// tile (CQ, ZP) or per column part (RS, Diag, E, DD: Cf::NS each, placed
// after the fixed slots by slots<Cf>).
enum { kDt, kLm, kLam, kEL, kW, kGa, kD, kCQ, kTD = kCQ + 4, kCross, kDot, kZP, kFixedSlots = kZP + 4 };
template <class Cf> struct slots {
    static constexpr int RS = kFixedSlots, Diag = RS + Cf::NS, E = Diag + Cf::NS, DD = E + Cf::NS,
                         count = DD + Cf::NS;
};

constexpr size_t a16(size_t x) { return (x + 15) / 16 * 16; }

// LDS carve-up (bytes).  GRAD adds the adjoint operands and the score tiles.
// The chunk-start state, needed only after the (S o M)^T dY product, reuses
// the S o M tile when it fits; the angle gradients of a token reuse that
// token's X rows (X is last read before they are written) when they fit.
template <class Cf, bool GRAD>
struct Lay {
    static constexpr size_t rowsN = a16((size_t)Cf::T * Cf::LDN * Cf::E);
    static constexpr size_t rowsP = a16((size_t)Cf::T * Cf::LDP * Cf::E);
    static constexpr size_t stNP = a16((size_t)Cf::N * Cf::LDP * Cf::E);
    static constexpr size_t sqT = a16((size_t)Cf::T * Cf::LDT * Cf::E);
    static constexpr size_t phi = a16((size_t)Cf::Q * Cf::LDH * 4);
    static constexpr bool ALIAS_G = GRAD && stNP <= sqT;
    static constexpr bool ALIAS_DPHI = GRAD && Cf::NPR * 4 <= Cf::R * Cf::LDP * Cf::E;
    static constexpr int DPS = ALIAS_DPHI ? Cf::R * Cf::LDP * Cf::E / 4 : Cf::LDH;   // dPhi row stride
    static constexpr size_t oBb = 0, oCb = oBb + rowsN, oX = oCb + rowsN, oDY = oX + rowsP;
    static constexpr size_t oDG = oDY + rowsP;
    static constexpr size_t oSM = oDG + (GRAD ? stNP : 0);
    static constexpr size_t odS = oSM + (GRAD ? sqT : 0);
    static constexpr size_t oGi = ALIAS_G ? oSM : odS + (GRAD ? sqT : 0);
    static constexpr size_t oPhi = odS + (GRAD ? sqT : 0) + (GRAD && !ALIAS_G ? stNP : 0);
    static constexpr size_t oDPhi = ALIAS_DPHI ? oX : oPhi + phi;
    static constexpr size_t oTok = oPhi + phi + (GRAD && !ALIAS_DPHI ? phi : 0);
    static constexpr size_t bytes = oTok + (size_t)slots<Cf>::count * Cf::TS * 4;
};

template <typename OP> struct V4T;
template <> struct V4T<bf16> { using type = bf16x4; };
template <> struct V4T<float> { using type = f32x4; };
template <typename OP> __device__ __forceinline__ typename V4T<OP>::type to_v4(const f32x4& v);
template <> __device__ __forceinline__ bf16x4 to_v4<bf16>(const f32x4& v)
{
    bf16x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (bf16)v[e];
    return o;
}
template <> __device__ __forceinline__ f32x4 to_v4<float>(const f32x4& v) { return v; }
// Four consecutive stored-state elements as float32.
__device__ __forceinline__ f32x4 ld4f(const bf16* q)
{
    const bf16x4 v = *reinterpret_cast<const bf16x4*>(q);
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ f32x4 ld4f(const float* q) { return *reinterpret_cast<const f32x4*>(q); }

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename OP> __device__ __forceinline__ void sincos_op(float a, float* s, float* c);
template <> __device__ __forceinline__ void sincos_op<bf16>(float a, float* s, float* c) { __sincosf(a, s, c); }
template <> __device__ __forceinline__ void sincos_op<float>(float a, float* s, float* c) { sincosf(a, s, c); }

// Sum over aligned groups of G lanes (4, 8 or 16) with DPP; every lane of a
// group receives the group's sum.
template <int G>
__device__ __forceinline__ float group_sum(float v)
{
    v += dpp_moved<0xB1, 0xf>(v);    // quad_perm [1,0,3,2]
    v += dpp_moved<0x4E, 0xf>(v);    // quad_perm [2,3,0,1]
    if constexpr (G >= 8) v += dpp_moved<0x141, 0xf>(v);    // row_half_mirror
    if constexpr (G >= 16) v += dpp_moved<0x140, 0xf>(v);   // row_mirror
    return v;
}
// The value of the lane holding the other column of the same rotation pair.
__device__ __forceinline__ float pair_swap(float v) { return dpp_moved<0xB1, 0xf>(v); }

// Matrix-core operand whose K runs along the rows of a row-major LDS array:
// lane (g, l16) takes arr[(r0 + l16) * ld + k0 + 8 g + e], e = 0..7.
template <typename OP>
__device__ __forceinline__ void frag_row(Frag<OP>& f, const OP* arr, int ld, int r0, int k0, int l16, int g)
{
    lds_frag8(f, arr + (r0 + l16) * ld + k0 + 8 * g);
}
// Operand whose K runs down the columns: lane (g, l16) takes
// arr[(k0 + 8 g + e) * ld + c0 + l16] (bf16: two transposing reads).
__device__ __forceinline__ void frag_col(Frag<bf16>& f, const bf16* arr, int ld, int k0, int c0, int l16, int g)
{
    const bf16* q = arr + (k0 + 8 * g + (l16 >> 2)) * ld + c0 + 4 * (l16 & 3);
    const bf16x4 lo = lds_read_tr4(q);
    const bf16x4 hi = lds_read_tr4(q + 4 * ld);
#pragma unroll
    for (int e = 0; e < 4; ++e) { f.v[e] = lo[e]; f.v[4 + e] = hi[e]; }
}
__device__ __forceinline__ void frag_col(Frag<float>& f, const float* arr, int ld, int k0, int c0, int l16, int g)
{
#pragma unroll
    for (int e = 0; e < 8; ++e) f.v[e] = arr[(k0 + 8 * g + e) * ld + c0 + l16];
}

__device__ __forceinline__ void lds_load8(float (&v)[8], const bf16* q)
{
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(q);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (float)a[e];
}
__device__ __forceinline__ void lds_load8(float (&v)[8], const float* q)
{
    const f32x4 a = *reinterpret_cast<const f32x4*>(q);
    const f32x4 b = *reinterpret_cast<const f32x4*>(q + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) { v[e] = a[e]; v[4 + e] = b[e]; }
}
__device__ __forceinline__ void store4_op(bf16* q, const f32x4& v)
{
    bf16x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (bf16)v[e];
    *reinterpret_cast<bf16x4*>(q) = o;
}
__device__ __forceinline__ void store4_op(float* q, const f32x4& v) { *reinterpret_cast<f32x4*>(q) = v; }

// One chunk's global inputs as a thread holds them between issuing the loads
// and writing them to LDS (a workgroup loads the next chunk while it works on
// the current one).
template <class Cf>
struct Raw {
    using V4 = typename V4T<typename Cf::op_t>::type;
    static constexpr int VB = Cf::N / Cf::VE, VX = Cf::P / Cf::VE;      // vectors per B / X row
    static constexpr int IB = (Cf::T * VB + Cf::NTHR - 1) / Cf::NTHR;
    static constexpr int IX = (Cf::T * VX + Cf::NTHR - 1) / Cf::NTHR;
    static constexpr int IT = (Cf::Q * (Cf::NPR / 4) + Cf::NTHR - 1) / Cf::NTHR;
    static constexpr int G4 = Cf::P / 4;                                // lanes per pair in state items
    static constexpr int IG = (Cf::NPR * G4 + Cf::NTHR - 1) / Cf::NTHR;
    uint4 vb[IB], vc[IB], vx[IX], vy[IX];
    f32x4 th[IT];
    float dtv, lmv, av;   // av: the token's decay rate (per token, or the head's)
    V4 sd0[IG], sd1[IG], sg0[IG], sg1[IG];    // state pair items (rows 2i, 2i+1, columns 4q..4q+3)
    float scc[IG], sss[IG];
};

// Values a thread keeps from staging to the end of the gradient: its theta
// items (for sum_i theta_i dphi_i) and its pair items of the chunk-start
// state (written to LDS once its slot there is free).
template <class Cf>
struct Held {
    using V4 = typename V4T<typename Cf::op_t>::type;
    static constexpr int IT = Raw<Cf>::IT, IG = Raw<Cf>::IG;
    f32x4 th[IT];
    V4 g0[IG], g1[IG];
    float av;             // the decay rate of token `lane` (wave 0)
};

__device__ __forceinline__ f32x4 v4f(const bf16x4& v) { return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]}; }
__device__ __forceinline__ f32x4 v4f(const f32x4& v) { return v; }

// Issue the global loads of chunk c of unit bh (zero past the sequence), by
// part: LR_STATE the boundary states (gradient only), LR_BC the B and C rows,
// LR_XT the X and dY rows, theta and the token scalars.
constexpr int LR_STATE = 1, LR_BC = 2, LR_XT = 4, LR_ALL = 7;
template <class Cf, bool GRAD, int PARTS = LR_ALL>
__device__ __forceinline__ void load_raw(const BcParams& p, int bh, int c, Raw<Cf>& rw, int tid)
{
    using op_t = typename Cf::op_t;
    using RW = Raw<Cf>;
    using V4 = typename RW::V4;
    constexpr int T = Cf::T, Q = Cf::Q, R = Cf::R, N = Cf::N, P = Cf::P, NPR = Cf::NPR;
    constexpr int VE = Cf::VE, NTHR = Cf::NTHR, VB = RW::VB, VX = RW::VX, G4 = RW::G4;
    const int64_t L_ = p.L, H = p.H;
    int64_t b, h;
    split_bh(bh, H, b, h);
    const int64_t t0 = (int64_t)c * Q;
    auto tok = [&](int64_t t) -> int64_t { return (b * L_ + t) * H + h; };
    const uint4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int it = 0; it < RW::IB && (PARTS & LR_BC); ++it) {
        const int v = tid + NTHR * it;
        rw.vb[it] = z; rw.vc[it] = z;
        if (v < T * VB) {
            const int rho = v / VB, q = v % VB;
            const int64_t t = t0 + rho / R;
            if (t < L_) {
                const size_t off = ((size_t)tok(t) * R + rho % R) * N + (size_t)q * VE;
                rw.vb[it] = *reinterpret_cast<const uint4*>(reinterpret_cast<const op_t*>(p.B) + off);
                rw.vc[it] = *reinterpret_cast<const uint4*>(reinterpret_cast<const op_t*>(p.C) + off);
            }
        }
    }
#pragma unroll
    for (int it = 0; it < RW::IX && (PARTS & LR_XT); ++it) {
        const int v = tid + NTHR * it;
        rw.vx[it] = z; rw.vy[it] = z;
        if (v < T * VX) {
            const int rho = v / VX, q = v % VX;
            const int64_t t = t0 + rho / R;
            if (t < L_) {
                const size_t off = ((size_t)tok(t) * R + rho % R) * P + (size_t)q * VE;
                rw.vx[it] = *reinterpret_cast<const uint4*>(reinterpret_cast<const op_t*>(p.x) + off);
                rw.vy[it] = *reinterpret_cast<const uint4*>(reinterpret_cast<const op_t*>(p.dy) + off);
            }
        }
    }
#pragma unroll
    for (int it = 0; it < RW::IT && (PARTS & LR_XT); ++it) {
        const int v = tid + NTHR * it;
        rw.th[it] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (v < Q * (NPR / 4)) {
            const int j = v / (NPR / 4), q = v % (NPR / 4);
            if (t0 + j < L_) rw.th[it] = *reinterpret_cast<const f32x4*>(p.theta + tok(t0 + j) * NPR + 4 * q);
        }
    }
    if constexpr ((PARTS & LR_XT) != 0) {
        rw.dtv = 0.f; rw.lmv = 0.f; rw.av = 0.f;
        if (tid <= Q && t0 + tid < L_) { rw.dtv = p.dt[tok(t0 + tid)]; rw.lmv = p.lam[tok(t0 + tid)]; }
        // the decay rate, loaded with the chunk: per token, or the head's one
        // (so that no later phase waits on a load of it)
        if (tid < Q && t0 + tid < L_) rw.av = p.A[p.a_tok ? tok(t0 + tid) : h];
    }
    if constexpr (GRAD && (PARTS & LR_STATE) != 0) {
        const op_t* gin = reinterpret_cast<const op_t*>(p.gst) + ((size_t)bh * (p.nc + 1) + c) * N * P;
        const op_t* dgo = reinterpret_cast<const op_t*>(p.dgst) + ((size_t)bh * (p.nc + 1) + c) * N * P;
        const float* cst = p.csum + ((size_t)bh * p.nc + c) * (1 + N);
#pragma unroll
        for (int it = 0; it < RW::IG; ++it) {
            const int v = tid + NTHR * it;
            const int i = v < NPR * G4 ? v / G4 : 0, q = v < NPR * G4 ? v % G4 : 0;
            rw.sd0[it] = *reinterpret_cast<const V4*>(dgo + (size_t)(2 * i) * P + 4 * q);
            rw.sd1[it] = *reinterpret_cast<const V4*>(dgo + (size_t)(2 * i + 1) * P + 4 * q);
            rw.sg0[it] = *reinterpret_cast<const V4*>(gin + (size_t)(2 * i) * P + 4 * q);
            rw.sg1[it] = *reinterpret_cast<const V4*>(gin + (size_t)(2 * i + 1) * P + 4 * q);
            rw.scc[it] = cst[1 + 2 * i];
            rw.sss[it] = cst[2 + 2 * i];
        }
    }
}

// Stage one chunk from its loaded inputs: token scalars, cumulative angles,
// rotated B and C rows, X and dY rows; for the gradient also the rotated
// end-state adjoint dGbar and, in float32, the chunk-start terms
// e^{Lam_tot} <G_in, dGbar> and per pair e^{Lam_tot} sum_p (G_in,0 dGbar_1 -
// G_in,1 dGbar_0) (the end state's remaining share, sum_k d_k Bbar_k X_k, is
// added from the same per-token products that enter the tokens' own
// gradients, so the two cancel exactly where the reverse prefix sums say they
// must).  The caller has finished with every LDS array of a previous chunk.
template <class Cf, bool GRAD>
__device__ __forceinline__ void stage(const BcParams& p, unsigned char* lds, int bh, int c, const Raw<Cf>& rw,
                                      Held<Cf>& hd, int tid)
{
    using op_t = typename Cf::op_t;
    using L = Lay<Cf, GRAD>;
    using RW = Raw<Cf>;
    constexpr int T = Cf::T, Q = Cf::Q, R = Cf::R, N = Cf::N, P = Cf::P, NPR = Cf::NPR;
    constexpr int LDN = Cf::LDN, LDP = Cf::LDP, LDH = Cf::LDH, VE = Cf::VE, TS = Cf::TS;
    constexpr int NTHR = Cf::NTHR, NW = Cf::NW, VB = RW::VB, VX = RW::VX, G4 = RW::G4;
    const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t H = p.H, h = (int)bh % (int)H;
    op_t* sBb = reinterpret_cast<op_t*>(lds + L::oBb);
    op_t* sCb = reinterpret_cast<op_t*>(lds + L::oCb);
    op_t* sX = reinterpret_cast<op_t*>(lds + L::oX);
    op_t* sDY = reinterpret_cast<op_t*>(lds + L::oDY);
    float* sPhi = reinterpret_cast<float*>(lds + L::oPhi);
    float* sT = reinterpret_cast<float*>(lds + L::oTok);

    // ---- S1: raw rows into LDS ----------------------------------------------
#pragma unroll
    for (int it = 0; it < RW::IB; ++it) {
        const int v = tid + NTHR * it;
        if (v < T * VB) {
            const int rho = v / VB, q = v % VB;
            *reinterpret_cast<uint4*>(sBb + rho * LDN + q * VE) = rw.vb[it];
            *reinterpret_cast<uint4*>(sCb + rho * LDN + q * VE) = rw.vc[it];
        }
    }
#pragma unroll
    for (int it = 0; it < RW::IX; ++it) {
        const int v = tid + NTHR * it;
        if (v < T * VX) {
            const int rho = v / VX, q = v % VX;
            *reinterpret_cast<uint4*>(sX + rho * LDP + q * VE) = rw.vx[it];
            *reinterpret_cast<uint4*>(sDY + rho * LDP + q * VE) = rw.vy[it];
        }
    }
#pragma unroll
    for (int it = 0; it < RW::IT; ++it) {
        const int v = tid + NTHR * it;
        hd.th[it] = rw.th[it];
        if (v < Q * (NPR / 4)) {
            const int j = v / (NPR / 4), q = v % (NPR / 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) sPhi[j * LDH + 4 * q + e] = rw.th[it][e];
        }
    }
    if (tid <= Q) { sT[kDt * TS + tid] = rw.dtv; sT[kLm * TS + tid] = rw.lmv; }
    __syncthreads();

    // ---- S2: token scalars (wave 0) and cumulative angles (all waves) ------
    if (wv == 0) {
        const int j = lane;
        const float dtj = j < Q ? sT[kDt * TS + j] : 0.f;
        const float lmj = j < Q ? sT[kLm * TS + j] : 0.f;
        const float lam_j = wave_inclusive_sum(dtj * rw.av);
        hd.av = rw.av;
        const float lam_tot = wave_read_lane(lam_j, 63);
        const float dtn = sT[kDt * TS + j + 1], lmn = sT[kLm * TS + j + 1];
        const float ga = lmj * dtj;
        const float w = ga + (1.f - lmn) * dtn;
        if (j < Q) {
            sT[kLam * TS + j] = lam_j;
            sT[kEL * TS + j] = ex2(lam_j * kLog2e);
            sT[kW * TS + j] = w;
            sT[kGa * TS + j] = ga;
            sT[kD * TS + j] = w * ex2((lam_tot - lam_j) * kLog2e);
        }
    }
    {
        // this wave's NPR / NW pairs as independent scans (their DPP chains
        // interleave)
        static_assert(NPR % NW == 0, "pairs split evenly over the waves");
        constexpr int KW = NPR / NW;
        const float dtj = lane < Q ? sT[kDt * TS + lane] : 0.f;
        float v[KW];
#pragma unroll
        for (int k = 0; k < KW; ++k) v[k] = lane < Q ? dtj * sPhi[lane * LDH + wv + NW * k] : 0.f;
#pragma unroll
        for (int k = 0; k < KW; ++k) v[k] = wave_inclusive_sum(v[k]);
#pragma unroll
        for (int k = 0; k < KW; ++k)
            if (lane < Q) sPhi[lane * LDH + wv + NW * k] = v[k];
    }
    __syncthreads();

    // ---- S3: rotate B and C rows by R(Phi)^T in place ------------------------
    {
        constexpr int NI = T * (NPR / 4);
        for (int v = tid; v < NI; v += NTHR) {
            const int rho = v / (NPR / 4), qd = v % (NPR / 4);
            const int j = rho / R;
            float cs[4], sn[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) sincos_op<op_t>(sPhi[j * LDH + 4 * qd + e], &sn[e], &cs[e]);
            float bv[8], cv[8], o[8];
            lds_load8(bv, sBb + rho * LDN + 8 * qd);
            lds_load8(cv, sCb + rho * LDN + 8 * qd);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                o[2 * e] = cs[e] * bv[2 * e] + sn[e] * bv[2 * e + 1];
                o[2 * e + 1] = cs[e] * bv[2 * e + 1] - sn[e] * bv[2 * e];
            }
            lds_store8(sBb + rho * LDN + 8 * qd, o);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                o[2 * e] = cs[e] * cv[2 * e] + sn[e] * cv[2 * e + 1];
                o[2 * e + 1] = cs[e] * cv[2 * e + 1] - sn[e] * cv[2 * e];
            }
            lds_store8(sCb + rho * LDN + 8 * qd, o);
        }
    }
    if constexpr (GRAD) {
        op_t* sDG = reinterpret_cast<op_t*>(lds + L::oDG);
        const float el_tot = sT[kEL * TS + Q - 1];
        float dot = 0.f;
#pragma unroll
        for (int it = 0; it < RW::IG; ++it) {
            const int v = tid + NTHR * it;
            const bool ok = v < NPR * G4;
            const f32x4 d0 = v4f(rw.sd0[it]), d1 = v4f(rw.sd1[it]);
            const f32x4 g0 = v4f(rw.sg0[it]), g1 = v4f(rw.sg1[it]);
            float cr = 0.f;
            f32x4 r0, r1;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                r0[e] = rw.scc[it] * d0[e] + rw.sss[it] * d1[e];
                r1[e] = rw.scc[it] * d1[e] - rw.sss[it] * d0[e];
                cr += g0[e] * r1[e] - g1[e] * r0[e];
                dot += ok ? g0[e] * r0[e] + g1[e] * r1[e] : 0.f;
            }
            hd.g0[it] = rw.sg0[it];
            hd.g1[it] = rw.sg1[it];
            if (ok) {
                const int i = v / G4, q = v % G4;
                *reinterpret_cast<typename V4T<op_t>::type*>(sDG + (2 * i) * LDP + 4 * q) = to_v4<op_t>(r0);
                *reinterpret_cast<typename V4T<op_t>::type*>(sDG + (2 * i + 1) * LDP + 4 * q) = to_v4<op_t>(r1);
            }
            cr = group_sum<G4>(cr);
            if (ok && (v % G4) == 0) sT[kCross * TS + v / G4] = el_tot * cr;
        }
        dot = wave_read_lane(wave_inclusive_sum(dot), 63);
        if (lane == 0) sT[kDot * TS + wv] = el_tot * dot;
    }
}

// The chunk-start state from the thread's held items into LDS.
template <class Cf>
__device__ __forceinline__ void put_gin(typename Cf::op_t* sGi, const Held<Cf>& hd, int tid)
{
    using HD = Held<Cf>;
    constexpr int G4 = Cf::P / 4, LDP = Cf::LDP;
#pragma unroll
    for (int it = 0; it < HD::IG; ++it) {
        const int v = tid + Cf::NTHR * it;
        if (v < Cf::NPR * G4) {
            const int i = v / G4, q = v % G4;
            *reinterpret_cast<typename V4T<typename Cf::op_t>::type*>(sGi + (2 * i) * LDP + 4 * q) = hd.g0[it];
            *reinterpret_cast<typename V4T<typename Cf::op_t>::type*>(sGi + (2 * i + 1) * LDP + 4 * q) = hd.g1[it];
        }
    }
}

// ---------------------------------------------------------------------------
// Chunk-local sums: Gloc = Bbar^T diag(d) X and V = Cbar^T diag(e^Lam) dY
// (N x P each, chunk-local frame, stored in the operand type), e^{Lam_tot},
// cos/sin of Phi_tot.
template <class Cf>
__global__ __launch_bounds__(Cf::NTHR) void bc_local_kernel(const BcParams p)
{
    using op_t = typename Cf::op_t;
    using L = Lay<Cf, false>;
    constexpr int T = Cf::T, Q = Cf::Q, R = Cf::R, N = Cf::N, P = Cf::P, NPR = Cf::NPR;
    constexpr int LDN = Cf::LDN, LDP = Cf::LDP, LDH = Cf::LDH, TS = Cf::TS, NT = Cf::NT, PT = Cf::PT;
    constexpr int NTHR = Cf::NTHR, NW = Cf::NW;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    const int bh = blockIdx.x / p.nc, c = blockIdx.x % p.nc;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, l16 = lane & 15, g = lane >> 4;
    Raw<Cf> rw;
    Held<Cf> hd;
    load_raw<Cf, false>(p, bh, c, rw, tid);
    stage<Cf, false>(p, lds, bh, c, rw, hd, tid);
    op_t* sBb = reinterpret_cast<op_t*>(lds + L::oBb);
    op_t* sCb = reinterpret_cast<op_t*>(lds + L::oCb);
    op_t* sX = reinterpret_cast<op_t*>(lds + L::oX);
    op_t* sDY = reinterpret_cast<op_t*>(lds + L::oDY);
    const float* sPhi = reinterpret_cast<const float*>(lds + L::oPhi);
    const float* sT = reinterpret_cast<const float*>(lds + L::oTok);
    // scale X rows by d and dY rows by e^{Lam} in place
    for (int v = tid; v < T * (P / 8); v += NTHR) {
        const int rho = v / (P / 8), q = v % (P / 8);
        const int j = rho / R;
        const float d = sT[kD * TS + j], el = sT[kEL * TS + j];
        float xv[8], yv[8];
        lds_load8(xv, sX + rho * LDP + 8 * q);
        lds_load8(yv, sDY + rho * LDP + 8 * q);
#pragma unroll
        for (int e = 0; e < 8; ++e) { xv[e] *= d; yv[e] *= el; }
        lds_store8(sX + rho * LDP + 8 * q, xv);
        lds_store8(sDY + rho * LDP + 8 * q, yv);
    }
    __syncthreads();
    op_t* out = reinterpret_cast<op_t*>(p.loc) + ((size_t)bh * p.nc + c) * 2 * N * P;
    constexpr int NTILE = 2 * NT * PT;
    for (int tl = wv; tl < NTILE; tl += NW) {
        const int prod = tl / (NT * PT), nt = (tl % (NT * PT)) / PT, pt = tl % PT;
        const op_t* sa = prod ? sCb : sBb;
        const op_t* sb = prod ? sDY : sX;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < T / 32; ++kb) {
            Frag<op_t> a, bb;
            frag_col(a, sa, LDN, 32 * kb, 16 * nt, l16, g);
            frag_col(bb, sb, LDP, 32 * kb, 16 * pt, l16, g);
            mma(a, bb, acc);
        }
        op_t* o = out + (size_t)prod * N * P + (size_t)(16 * nt + 4 * g) * P + 16 * pt + l16;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[(size_t)i * P] = (op_t)acc[i];
    }
    if (tid <= NPR) {
        float* cs = p.csum + ((size_t)bh * p.nc + c) * (1 + N);
        if (tid == 0) {
            cs[0] = ex2(sT[kLam * TS + Q - 1] * kLog2e);
        } else {
            float sn, cn;
            sincosf(sPhi[(Q - 1) * LDH + tid - 1], &sn, &cn);
            cs[2 * tid - 1] = cn;
            cs[2 * tid] = sn;
        }
    }
}

// ---------------------------------------------------------------------------
// Chunk-boundary states: forward G_in(c+1) = R(Phi_tot)(e^{Lam_tot} G_in(c) +
// Gloc(c)) from G_in(0) = h_in + bhat_0 B_prev x_prev; backward
// dG_in(c) = e^{Lam_tot} R(Phi_tot)^T dG_out(c) + V(c) from dG_out = dh_out.
// One thread per (b, h, pair, two columns), float32 recurrence, states stored
// in ST; blockIdx.y picks the direction.  Each batch of U chunks issues all its
// loads (indices clamped into range) before the first use.
template <typename ST> struct ST2T;
template <> struct ST2T<bf16> { using type = bf16x2; };
template <> struct ST2T<float> { using type = float2; };
__device__ __forceinline__ float2 f2(const bf16x2 v) { return make_float2((float)v[0], (float)v[1]); }
__device__ __forceinline__ float2 f2(const float2 v) { return v; }
template <typename ST> __device__ __forceinline__ typename ST2T<ST>::type st2(float a, float b);
template <> __device__ __forceinline__ bf16x2 st2<bf16>(float a, float b)
{
    bf16x2 v;
    v[0] = (bf16)a;
    v[1] = (bf16)b;
    return v;
}
template <> __device__ __forceinline__ float2 st2<float>(float a, float b) { return make_float2(a, b); }

template <typename IO, typename ST>
__global__ __launch_bounds__(256) void bc_scan_kernel(const BcParams p)
{
    using V2 = typename ST2T<ST>::type;
    const int N = p.N, P = p.P, R = p.R, NPR = N / 2, nc = p.nc, P2 = P / 2;
    const int64_t per = (int64_t)NPR * P2;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)p.nbh * per) return;
    const int bh = (int)(idx / per);
    const int rem = (int)(idx % per), i = rem / P2, q = 2 * (rem % P2);
    const size_t NP = (size_t)N * P;
    const size_t o0 = (size_t)(2 * i) * P + q, o1 = o0 + P;
    const float* cs = p.csum + (size_t)bh * nc * (1 + N);
    const ST* lc = reinterpret_cast<const ST*>(p.loc) + (size_t)bh * nc * 2 * NP;
    constexpr int U = 8;
    if (blockIdx.y == 0) {
        float2 g0 = make_float2(0.f, 0.f), g1 = g0;
        if (p.h_in != nullptr) {
            g0 = *reinterpret_cast<const float2*>(p.h_in + bh * NP + o0);
            g1 = *reinterpret_cast<const float2*>(p.h_in + bh * NP + o1);
        }
        if (p.Bp_in != nullptr && p.L > 0) {
            int64_t b, h;
            split_bh(bh, p.H, b, h);
            const int64_t k0 = (b * p.L) * p.H + h;
            const float bhat = (1.f - p.lam[k0]) * p.dt[k0];
            const IO* Bp = reinterpret_cast<const IO*>(p.Bp_in) + (size_t)bh * R * N;
            const IO* xp = reinterpret_cast<const IO*>(p.xp_in) + (size_t)bh * R * P;
            for (int r = 0; r < R; ++r) {
                const float xa = to_f32(xp[r * P + q]), xb = to_f32(xp[r * P + q + 1]);
                const float b0 = bhat * to_f32(Bp[r * N + 2 * i]), b1 = bhat * to_f32(Bp[r * N + 2 * i + 1]);
                g0.x += b0 * xa; g0.y += b0 * xb;
                g1.x += b1 * xa; g1.y += b1 * xb;
            }
        }
        ST* G = reinterpret_cast<ST*>(p.gst) + (size_t)bh * (nc + 1) * NP;
        for (int c0 = 0; c0 < nc; c0 += U) {
            float2 l0[U], l1[U];
            float e[U], cc[U], ss[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + u < nc ? c0 + u : nc - 1;
                l0[u] = f2(*reinterpret_cast<const V2*>(lc + (size_t)c * 2 * NP + o0));
                l1[u] = f2(*reinterpret_cast<const V2*>(lc + (size_t)c * 2 * NP + o1));
                e[u] = cs[(size_t)c * (1 + N)];
                cc[u] = cs[(size_t)c * (1 + N) + 1 + 2 * i];
                ss[u] = cs[(size_t)c * (1 + N) + 2 + 2 * i];
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + u;
                if (c < nc) {
                    *reinterpret_cast<V2*>(G + c * NP + o0) = st2<ST>(g0.x, g0.y);
                    *reinterpret_cast<V2*>(G + c * NP + o1) = st2<ST>(g1.x, g1.y);
                    const float a0x = e[u] * g0.x + l0[u].x, a0y = e[u] * g0.y + l0[u].y;
                    const float a1x = e[u] * g1.x + l1[u].x, a1y = e[u] * g1.y + l1[u].y;
                    g0 = make_float2(cc[u] * a0x - ss[u] * a1x, cc[u] * a0y - ss[u] * a1y);
                    g1 = make_float2(ss[u] * a0x + cc[u] * a1x, ss[u] * a0y + cc[u] * a1y);
                }
            }
        }
    } else {
        float2 d0 = make_float2(0.f, 0.f), d1 = d0;
        if (p.dh_out != nullptr) {
            d0 = *reinterpret_cast<const float2*>(p.dh_out + bh * NP + o0);
            d1 = *reinterpret_cast<const float2*>(p.dh_out + bh * NP + o1);
        }
        ST* D = reinterpret_cast<ST*>(p.dgst) + (size_t)bh * (nc + 1) * NP;
        for (int c0 = nc - 1; c0 >= 0; c0 -= U) {
            float2 v0[U], v1[U];
            float e[U], cc[U], ss[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 - u >= 0 ? c0 - u : 0;
                v0[u] = f2(*reinterpret_cast<const V2*>(lc + ((size_t)c * 2 + 1) * NP + o0));
                v1[u] = f2(*reinterpret_cast<const V2*>(lc + ((size_t)c * 2 + 1) * NP + o1));
                e[u] = cs[(size_t)c * (1 + N)];
                cc[u] = cs[(size_t)c * (1 + N) + 1 + 2 * i];
                ss[u] = cs[(size_t)c * (1 + N) + 2 + 2 * i];
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 - u;
                if (c >= 0) {
                    *reinterpret_cast<V2*>(D + c * NP + o0) = st2<ST>(d0.x, d0.y);
                    *reinterpret_cast<V2*>(D + c * NP + o1) = st2<ST>(d1.x, d1.y);
                    const float r0x = cc[u] * d0.x + ss[u] * d1.x, r0y = cc[u] * d0.y + ss[u] * d1.y;
                    const float r1x = cc[u] * d1.x - ss[u] * d0.x, r1y = cc[u] * d1.y - ss[u] * d0.y;
                    d0 = make_float2(e[u] * r0x + v0[u].x, e[u] * r0y + v0[u].y);
                    d1 = make_float2(e[u] * r1x + v1[u].x, e[u] * r1y + v1[u].y);
                }
            }
        }
        *reinterpret_cast<V2*>(D + nc * NP + o0) = st2<ST>(d0.x, d0.y);
        *reinterpret_cast<V2*>(D + nc * NP + o1) = st2<ST>(d1.x, d1.y);
        if (p.dh_in != nullptr) {
            *reinterpret_cast<float2*>(p.dh_in + bh * NP + o0) = d0;
            *reinterpret_cast<float2*>(p.dh_in + bh * NP + o1) = d1;
        }
    }
}

// ---------------------------------------------------------------------------
// Every gradient of one chunk.  Wave w owns operand rows 16 (w % 4) ..
// 16 (w % 4) + 15 and part w / 4 of the output columns (of the key tiles in
// the score phase).
template <class Cf>
__global__ __launch_bounds__(Cf::NTHR) void bc_grad_kernel(const BcParams p)
{
    using op_t = typename Cf::op_t;
    using L = Lay<Cf, true>;
    using HD = Held<Cf>;
    constexpr int T = Cf::T, Q = Cf::Q, R = Cf::R, N = Cf::N, P = Cf::P, NPR = Cf::NPR;
    constexpr int LDN = Cf::LDN, LDP = Cf::LDP, LDT = Cf::LDT, LDH = Cf::LDH, TS = Cf::TS;
    constexpr int NT = Cf::NT, PT = Cf::PT, NB = Cf::NB, PB = Cf::PB, NTHR = Cf::NTHR, NW = Cf::NW;
    constexpr int NS = Cf::NS;
    constexpr int NH = NT / NS, PH = PT / NS;     // output column tiles per part
    constexpr int kRS = slots<Cf>::RS, kDiag = slots<Cf>::Diag, kE = slots<Cf>::E, kDD = slots<Cf>::DD;
    constexpr int TPR = 4 / R;                    // tokens among a lane's 4 rows
    constexpr int DPS = L::DPS;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    const int64_t L_ = p.L, H = p.H;
    const int nunits = p.nbh * p.nc;
    // Persistent: this workgroup takes units blockIdx.x, + gridDim.x, ...,
    // loading the next one's inputs while it works on the current one.
    Raw<Cf> rw;
    TlRow tlr;   // per-wave phase stamps (instrumented builds)
    tlr.open(p.tl, (size_t)blockIdx.x * NW + (threadIdx.x >> 6), threadIdx.x & 63,
             kTlBackward | ((unsigned long long)(threadIdx.x >> 6) << 48) | blockIdx.x);
    if ((int)blockIdx.x < nunits) load_raw<Cf, true>(p, blockIdx.x / p.nc, blockIdx.x % p.nc, rw, threadIdx.x);
    for (int unit = blockIdx.x; unit < nunits; unit += gridDim.x) {
    tlr.stamp(kTlUnit, threadIdx.x & 63);
    // The lane's indices are made opaque per unit, so that the compiler
    // recomputes the (cheap) LDS addresses inside the loop instead of keeping
    // them all live across it.
    int tid_v = threadIdx.x;
    asm volatile("" : "+v"(tid_v));
    const int tid = tid_v, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6), rt = wv & 3, hf = wv >> 2;
    const int bh = unit / p.nc, c = unit % p.nc;
    int64_t b, h;
    split_bh(bh, H, b, h);
    const int64_t t0 = (int64_t)c * Q;
    auto tok = [&](int64_t t) -> int64_t { return (b * L_ + t) * H + h; };
    Held<Cf> hd;
    stage<Cf, true>(p, lds, bh, c, rw, hd, tid);
    // The next unit's loads go out in three parts, after staging and after
    // the first two product phases, so that the waves' load issue does not
    // all fall in one burst ahead of the first phase.
    const bool more = unit + (int)gridDim.x < nunits;
    const int un = unit + gridDim.x;
    if (more) load_raw<Cf, true, LR_STATE>(p, un / p.nc, un % p.nc, rw, tid);
    const op_t* sBb = reinterpret_cast<const op_t*>(lds + L::oBb);
    const op_t* sCb = reinterpret_cast<const op_t*>(lds + L::oCb);
    const op_t* sX = reinterpret_cast<const op_t*>(lds + L::oX);
    const op_t* sDY = reinterpret_cast<const op_t*>(lds + L::oDY);
    const op_t* sDG = reinterpret_cast<const op_t*>(lds + L::oDG);
    op_t* sGi = reinterpret_cast<op_t*>(lds + L::oGi);
    op_t* sSM = reinterpret_cast<op_t*>(lds + L::oSM);
    op_t* sdS = reinterpret_cast<op_t*>(lds + L::odS);
    const float* sPhi = reinterpret_cast<const float*>(lds + L::oPhi);
    float* sDPhi = reinterpret_cast<float*>(lds + L::oDPhi);
    float* sT = reinterpret_cast<float*>(lds + L::oTok);
    __syncthreads();
    tlr.stamp(kTlStaged, lane);

    const int r0w = 16 * rt;                      // this wave's operand rows
    // ---- phase 1: S = Cbar Bbar^T, dSc = dY X^T on key tiles kt = hf (mod NS) --
    {
        float rowacc[4] = {0.f, 0.f, 0.f, 0.f}, diagacc[4] = {0.f, 0.f, 0.f, 0.f};
        float lam_r[4], ga_r[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tj = (r0w + 4 * g + i) / R;
            lam_r[i] = sT[kLam * TS + tj];
            ga_r[i] = sT[kGa * TS + tj];
        }
#pragma unroll
        for (int k2 = 0; k2 < 4 / NS; ++k2) {
            const int kt = hf + NS * k2;
            const int ck = 16 * kt + l16;
            if (kt > rt) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    sSM[(r0w + 4 * g + i) * LDT + ck] = (op_t)0.f;
                    sdS[(r0w + 4 * g + i) * LDT + ck] = (op_t)0.f;
                }
                if (g == 0) sT[(kCQ + rt) * TS + ck] = 0.f;
                continue;
            }
            f32x4 S = {0.f, 0.f, 0.f, 0.f}, D = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                Frag<op_t> a, bb;
                frag_row(a, sCb, LDN, r0w, 32 * nb, l16, g);
                frag_row(bb, sBb, LDN, 16 * kt, 32 * nb, l16, g);
                mma(a, bb, S);
            }
#pragma unroll
            for (int pb = 0; pb < PB; ++pb) {
                Frag<op_t> a, bb;
                frag_row(a, sDY, LDP, r0w, 32 * pb, l16, g);
                frag_row(bb, sX, LDP, 16 * kt, 32 * pb, l16, g);
                mma(a, bb, D);
            }
            const int tk = ck / R;
            const float lk = sT[kLam * TS + tk], wk = sT[kW * TS + tk];
            float colacc = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rj = r0w + 4 * g + i, tj = rj / R;
                const float v = S[i] * D[i];
                float m = 0.f;
                if (tk < tj) {
                    const float e = ex2((lam_r[i] - lk) * kLog2e);
                    m = e * wk;
                    rowacc[i] += v * m;
                    colacc += v * e;
                } else if (tk == tj) {
                    m = ga_r[i];
                    diagacc[i] += v;
                }
                sSM[rj * LDT + ck] = (op_t)(S[i] * m);
                sdS[rj * LDT + ck] = (op_t)(D[i] * m);
            }
            colacc += __shfl_xor(colacc, 16, 64);
            colacc += __shfl_xor(colacc, 32, 64);
            if (g == 0) sT[(kCQ + rt) * TS + ck] = colacc;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float rs = group_sum<16>(rowacc[i]);
            const float dg = group_sum<16>(diagacc[i]);
            if (l16 == 0) {
                sT[(kRS + hf) * TS + r0w + 4 * g + i] = rs;
                sT[(kDiag + hf) * TS + r0w + 4 * g + i] = dg;
            }
        }
    }
    __syncthreads();
    tlr.stamp(kTlScores, lane);
    if (more) load_raw<Cf, true, LR_BC>(p, un / p.nc, un % p.nc, rw, tid);

    // ---- phase 2a: dX = (S o M)^T dY + diag(d) Bbar dGbar^T ------------------
    {
        f32x4 ax[PH], axs[PH];
#pragma unroll
        for (int u = 0; u < PH; ++u) { ax[u] = f32x4{0.f, 0.f, 0.f, 0.f}; axs[u] = ax[u]; }
        for (int jb = rt >> 1; jb < T / 32; ++jb) {
            Frag<op_t> a;
            frag_col(a, sSM, LDT, 32 * jb, r0w, l16, g);
#pragma unroll
            for (int u = 0; u < PH; ++u) {
                Frag<op_t> bb;
                frag_col(bb, sDY, LDP, 32 * jb, 16 * (hf * PH + u), l16, g);
                mma(a, bb, ax[u]);
            }
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            Frag<op_t> a;
            frag_row(a, sBb, LDN, r0w, 32 * nb, l16, g);
#pragma unroll
            for (int u = 0; u < PH; ++u) {
                Frag<op_t> bb;
                frag_col(bb, sDG, LDP, 32 * nb, 16 * (hf * PH + u), l16, g);
                mma(a, bb, axs[u]);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rk = r0w + 4 * g + i, tk = rk / R;
            if (t0 + tk < L_) {
                const float dk = sT[kD * TS + tk];
                float* o = p.dx + ((size_t)tok(t0 + tk) * R + rk % R) * P + 16 * hf * PH + l16;
#pragma unroll
                for (int u = 0; u < PH; ++u) o[16 * u] = ax[u][i] + dk * axs[u][i];
            }
        }
    }
    __syncthreads();                              // the S o M tile is free
    tlr.stamp(kTlGradX, lane);
    if (more) load_raw<Cf, true, LR_XT>(p, un / p.nc, un % p.nc, rw, tid);
    put_gin<Cf>(sGi, hd, tid);

    // Back-rotation of dBbar / dCbar rows held in accumulators (lane: column
    // n = 16 nt + l16, rows 4 g + i) to dB / dC, and the angle gradient of
    // each (token, pair) summed over ranks into sDPhi (ADD: accumulate).
    auto back_rotate = [&](f32x4 (&acc)[NH], const op_t* sBar, float* gout, bool add) {
#pragma unroll
        for (int u = 0; u < NH; ++u) {
            const int n = 16 * (hf * NH + u) + l16, pr = n >> 1;
            const bool odd = (l16 & 1) != 0;
            float dps[TPR], snv[TPR], csv[TPR];
            // the lane's 4 rows hold TPR tokens: one sine/cosine per token
#pragma unroll
            for (int v = 0; v < TPR; ++v) {
                dps[v] = 0.f;
                sincos_op<op_t>(sPhi[((r0w + 4 * g) / R + v) * LDH + pr], &snv[v], &csv[v]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rk = r0w + 4 * g + i, tk = rk / R;
                const float own = acc[u][i];
                const float oth = pair_swap(own);
                const float d0 = odd ? oth : own, d1 = odd ? own : oth;
                const float bo = to_f32(sBar[rk * LDN + n]);
                const float bx = pair_swap(bo);
                const float b0 = odd ? bx : bo, b1 = odd ? bo : bx;
                const float sn = snv[i / R], cs = csv[i / R];
                dps[i / R] += d0 * b1 - d1 * b0;
                if (t0 + tk < L_)
                    gout[((size_t)tok(t0 + tk) * R + rk % R) * N + n] = odd ? sn * d0 + cs * d1 : cs * d0 - sn * d1;
            }
            if (!odd) {
#pragma unroll
                for (int v = 0; v < TPR; ++v) {
                    const int tk = (r0w + 4 * g) / R + v;
                    float* dp = sDPhi + tk * DPS + pr;
                    *dp = add ? *dp + dps[v] : dps[v];
                }
            }
        }
    };

    // ---- phase 2b: dBbar = dS^T Cbar + diag(d) Zb, Zb = X dGbar^T -------------
    {
        f32x4 ab[NH], zb[NH];
#pragma unroll
        for (int u = 0; u < NH; ++u) { ab[u] = f32x4{0.f, 0.f, 0.f, 0.f}; zb[u] = ab[u]; }
        for (int jb = rt >> 1; jb < T / 32; ++jb) {
            Frag<op_t> a;
            frag_col(a, sdS, LDT, 32 * jb, r0w, l16, g);
#pragma unroll
            for (int u = 0; u < NH; ++u) {
                Frag<op_t> bb;
                frag_col(bb, sCb, LDN, 32 * jb, 16 * (hf * NH + u), l16, g);
                mma(a, bb, ab[u]);
            }
        }
#pragma unroll
        for (int pb = 0; pb < PB; ++pb) {
            Frag<op_t> a;
            frag_row(a, sX, LDP, r0w, 32 * pb, l16, g);
#pragma unroll
            for (int u = 0; u < NH; ++u) {
                Frag<op_t> bb;
                frag_row(bb, sDG, LDP, 16 * (hf * NH + u), 32 * pb, l16, g);
                mma(a, bb, zb[u]);
            }
        }
        __syncthreads();                          // X is free (angle gradients); G_in is staged
        tlr.stamp(kTlGradB, lane);
        // dd_k = <Bbar_k, Zb_k> per row over this half's columns, and per pair
        // the sum over this wave's rows of d_k (Zb_0 Bbar_1 - Zb_1 Bbar_0)
        // (the state term's share of the angle gradient)
        float ddp[4] = {0.f, 0.f, 0.f, 0.f};
        float zp[NH];
#pragma unroll
        for (int u = 0; u < NH; ++u) zp[u] = 0.f;
        const bool odd = (l16 & 1) != 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rk = r0w + 4 * g + i;
            const float dk = sT[kD * TS + rk / R];
#pragma unroll
            for (int u = 0; u < NH; ++u) {
                const float bo = to_f32(sBb[rk * LDN + 16 * (hf * NH + u) + l16]);
                const float bx = pair_swap(bo), zx = pair_swap(zb[u][i]);
                const float z0 = odd ? zx : zb[u][i], z1 = odd ? zb[u][i] : zx;
                const float b0 = odd ? bx : bo, b1 = odd ? bo : bx;
                zp[u] += dk * (z0 * b1 - z1 * b0);
                ddp[i] += zb[u][i] * bo;
                ab[u][i] += dk * zb[u][i];
            }
        }
#pragma unroll
        for (int u = 0; u < NH; ++u) {
            float zz = zp[u];
            zz += __shfl_xor(zz, 16, 64);
            zz += __shfl_xor(zz, 32, 64);
            if (g == 0 && !odd) sT[(kZP + rt) * TS + ((16 * (hf * NH + u) + l16) >> 1)] = zz;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float sm = group_sum<16>(ddp[i]);
            if (l16 == 0) sT[(kDD + hf) * TS + r0w + 4 * g + i] = sm;
        }
        back_rotate(ab, sBb, p.dB, false);
        tlr.stamp(kTlGradBStored, lane);
    }

    // ---- phase 2c: dCbar = dS Bbar + diag(e^Lam) Zc, Zc = dY G_in^T -----------
    {
        f32x4 ac[NH], zc[NH];
#pragma unroll
        for (int u = 0; u < NH; ++u) { ac[u] = f32x4{0.f, 0.f, 0.f, 0.f}; zc[u] = ac[u]; }
        for (int kb = 0; kb <= (rt >> 1); ++kb) {
            Frag<op_t> a;
            frag_row(a, sdS, LDT, r0w, 32 * kb, l16, g);
#pragma unroll
            for (int u = 0; u < NH; ++u) {
                Frag<op_t> bb;
                frag_col(bb, sBb, LDN, 32 * kb, 16 * (hf * NH + u), l16, g);
                mma(a, bb, ac[u]);
            }
        }
#pragma unroll
        for (int pb = 0; pb < PB; ++pb) {
            Frag<op_t> a;
            frag_row(a, sDY, LDP, r0w, 32 * pb, l16, g);
#pragma unroll
            for (int u = 0; u < NH; ++u) {
                Frag<op_t> bb;
                frag_row(bb, sGi, LDP, 16 * (hf * NH + u), 32 * pb, l16, g);
                mma(a, bb, zc[u]);
            }
        }
        tlr.stamp(kTlGradCProducts, lane);
        float ep[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rj = r0w + 4 * g + i;
            const float el = sT[kEL * TS + rj / R];
#pragma unroll
            for (int u = 0; u < NH; ++u) {
                ep[i] += zc[u][i] * to_f32(sCb[rj * LDN + 16 * (hf * NH + u) + l16]);
                ac[u][i] += el * zc[u][i];
            }
            ep[i] *= el;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float sm = group_sum<16>(ep[i]);
            if (l16 == 0) sT[(kE + hf) * TS + r0w + 4 * g + i] = sm;
        }
        back_rotate(ac, sCb, p.dC, true);
    }
    __syncthreads();

    tlr.stamp(kTlGradC, lane);
    // ---- phase 3a: dphi = suffix sums of dPhi over the chunk's tokens ---------
    {
        // this wave's NPR / NW pairs as independent scans (their DPP chains
        // interleave)
        constexpr int KW = NPR / NW;
        float v[KW], inc[KW];
#pragma unroll
        for (int k = 0; k < KW; ++k) {
            const int i = wv + NW * k;
            v[k] = 0.f;
            if (lane < Q) {
                v[k] = sDPhi[lane * DPS + i];
                if (lane == Q - 1)
                    v[k] += sT[kCross * TS + i] - (sT[kZP * TS + i] + sT[(kZP + 1) * TS + i] +
                                                   sT[(kZP + 2) * TS + i] + sT[(kZP + 3) * TS + i]);
            }
        }
#pragma unroll
        for (int k = 0; k < KW; ++k) inc[k] = wave_inclusive_sum(v[k]);
#pragma unroll
        for (int k = 0; k < KW; ++k) {
            const float tot = wave_read_lane(inc[k], 63);
            if (lane < Q) sDPhi[lane * DPS + wv + NW * k] = tot - inc[k] + v[k];
        }
    }
    __syncthreads();

    tlr.stamp(kTlAngleSuffix, lane);
    // ---- phase 3b: dtheta = dt dphi; sum_i theta_i dphi_i per token ------------
    {
        constexpr int G4 = NPR / 4;               // lanes per token (4, 8 or 16)
        constexpr int NI = Q * G4;
#pragma unroll
        for (int it = 0; it < HD::IT; ++it) {
            const int v = tid + NTHR * it;
            float td = 0.f;
            if (v < NI) {
                const int j = v / G4, q = v % G4;
                if (t0 + j < L_) {
                    const int64_t k = tok(t0 + j);
                    const float dtj = sT[kDt * TS + j];
                    f32x4 o;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float dph = sDPhi[j * DPS + 4 * q + e];
                        o[e] = dtj * dph;
                        td += hd.th[it][e] * dph;
                    }
                    *reinterpret_cast<f32x4*>(p.dtheta + k * NPR + 4 * q) = o;
                }
            }
            td = group_sum<G4>(td);
            if (v < NI && (v % G4) == 0) sT[kTD * TS + v / G4] = td;
        }
    }
    __syncthreads();

    tlr.stamp(kTlGradTheta, lane);
    // ---- phase 3c: decay and weight gradients per token (wave 0) --------------
    if (wv == 0) {
        const int t = lane;
        float dlam = 0.f, dw = 0.f, dgt = 0.f, ddk = 0.f;
        if (t < Q) {
            float rs = 0.f, q = 0.f, dg = 0.f, e = 0.f, dd = 0.f;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int rho = t * R + r;
#pragma unroll
                for (int u = 0; u < NS; ++u) {
                    rs += sT[(kRS + u) * TS + rho];
                    dg += sT[(kDiag + u) * TS + rho];
                    e += sT[(kE + u) * TS + rho];
                    dd += sT[(kDD + u) * TS + rho];
                }
#pragma unroll
                for (int w = 0; w < 4; ++w) q += sT[(kCQ + w) * TS + rho];
            }
            const float wt = sT[kW * TS + t];
            ddk = sT[kD * TS + t] * dd;
            dlam = rs - wt * q + e - ddk;
            const float lam_tot = sT[kLam * TS + Q - 1];
            dw = q + dd * ex2((lam_tot - sT[kLam * TS + t]) * kLog2e);
            dgt = dg + dw;
        }
        // the end state's decay term: e^{Lam_tot} <G_in, dGbar> + sum_k d_k dd_k
        const float ddsum = wave_read_lane(wave_inclusive_sum(ddk), 63);
        if (t == Q - 1) {
            float dsum = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) dsum += sT[kDot * TS + w];
            dlam += dsum + ddsum;
        }
        const float inc = wave_inclusive_sum(dlam);
        const float da = wave_read_lane(inc, 63) - inc + dlam;
        const float dw_prev = __shfl_up(dw, 1, 64);
        float dAc = 0.f;
        if (t < Q && t0 + t < L_) {
            const float dtt = sT[kDt * TS + t], lm = sT[kLm * TS + t];
            const float dwp = t > 0 ? dw_prev : 0.f;
            const int64_t k = tok(t0 + t);
            const float A = hd.av;
            p.ddt[k] = A * da + sT[kTD * TS + t] + lm * dgt + (1.f - lm) * dwp;
            p.dlam[k] = dtt * (dgt - dwp);
            dAc = dtt * da;
            if (p.a_tok) p.dA[k] = dAc;      // a per-token rate: its own gradient
        }
        const float dAs = wave_read_lane(wave_inclusive_sum(dAc), 63);
        if (lane == 0) p.dA_part[(size_t)bh * p.nc + c] = dAs;
        if (lane == Q - 1) p.dw_last[(size_t)bh * p.nc + c] = dw;
    }
    __syncthreads();                              // LDS is reused by the next unit
    tlr.stamp(kTlGradDecay, lane);
    }
    tlr.close(threadIdx.x & 63);
}

// ---------------------------------------------------------------------------
// Per (b, h): the look-ahead weight of the last token of chunk c - 1 reaches
// bhat of the first token of chunk c (and the state record's bhat_0 term for
// chunk 0); the record's gradients; this unit's dA share.
template <typename IO, typename ST>
__global__ __launch_bounds__(256) void bc_final_kernel(const BcParams p)
{
    const int bh = blockIdx.x, tid = threadIdx.x;
    const int64_t H = p.H;
    int64_t b, h;
    split_bh(bh, H, b, h);
    const int N = p.N, P = p.P, R = p.R, nc = p.nc, Q = 64 / R;
    auto tok = [&](int64_t t) -> int64_t { return (b * p.L + t) * H + h; };
    __shared__ float red[256];
    const ST* dG0 = reinterpret_cast<const ST*>(p.dgst) + ((size_t)bh * (nc + 1) + nc) * N * P;
    const float bhat0 = p.L > 0 ? (1.f - p.lam[tok(0)]) * p.dt[tok(0)] : 0.f;
    float part = 0.f;
    if (p.Bp_in != nullptr) {
        const IO* Bp = reinterpret_cast<const IO*>(p.Bp_in) + (size_t)bh * R * N;
        const IO* xp = reinterpret_cast<const IO*>(p.xp_in) + (size_t)bh * R * P;
        for (int v = tid; v < R * N; v += 256) {
            const int r = v / N, n = v % N;
            float z = 0.f;
            for (int q = 0; q < P; ++q) z += to_f32(dG0[(size_t)n * P + q]) * to_f32(xp[r * P + q]);
            part += to_f32(Bp[r * N + n]) * z;
            if (p.dBp != nullptr) p.dBp[(size_t)bh * R * N + v] = bhat0 * z;
        }
        if (p.dxp != nullptr) {
            for (int v = tid; v < R * P; v += 256) {
                const int r = v / P, q = v % P;
                float s = 0.f;
                for (int n = 0; n < N; ++n) s += to_f32(Bp[r * N + n]) * to_f32(dG0[(size_t)n * P + q]);
                p.dxp[(size_t)bh * R * P + v] = bhat0 * s;
            }
        }
    } else {
        if (p.dBp != nullptr)
            for (int v = tid; v < R * N; v += 256) p.dBp[(size_t)bh * R * N + v] = 0.f;
        if (p.dxp != nullptr)
            for (int v = tid; v < R * P; v += 256) p.dxp[(size_t)bh * R * P + v] = 0.f;
    }
    red[tid] = part;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (tid < w) red[tid] += red[tid + w];
        __syncthreads();
    }
    const float dbhat0 = red[0];
    __syncthreads();
    for (int c = tid; c < nc; c += 256) {
        const int64_t t = (int64_t)c * Q;
        if (t >= p.L) continue;
        const float dwp = c == 0 ? dbhat0 : p.dw_last[(size_t)bh * nc + c - 1];
        const int64_t k = tok(t);
        p.ddt[k] += (1.f - p.lam[k]) * dwp;
        p.dlam[k] -= p.dt[k] * dwp;
    }
    float s = 0.f;
    for (int c = tid; c < nc; c += 256) s += p.dA_part[(size_t)bh * nc + c];
    red[tid] = s;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (tid < w) red[tid] += red[tid + w];
        __syncthreads();
    }
    if (tid == 0) p.dA_bh[bh] = red[0];
}

// dA[h] = sum over the batch rows of the units' shares (fixed order).
static __global__ void bc_dA_kernel(const float* part, float* dA, int64_t batch, int64_t H)
{
    const int64_t h = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (h >= H) return;
    float s = 0.f;
    for (int64_t b = 0; b < batch; ++b) s += part[b * H + h];
    dA[h] = s;
}

template <class Cf> constexpr size_t local_lds() { return Lay<Cf, false>::bytes; }
template <class Cf> constexpr size_t grad_lds() { return Lay<Cf, true>::bytes; }

template <class Cf>
hipError_t launch_cfg(const BcParams& p, hipStream_t stream)
{
    using IO = typename Cf::op_t;
    auto* k1 = &bc_local_kernel<Cf>;
    auto* k3 = &bc_grad_kernel<Cf>;
    static const hipError_t a1 = hipFuncSetAttribute(reinterpret_cast<const void*>(k1),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    static const hipError_t a3 = hipFuncSetAttribute(reinterpret_cast<const void*>(k3),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (a1 != hipSuccess) return a1;
    if (a3 != hipSuccess) return a3;
    (void)hipGetLastError();
    const unsigned nunits = (unsigned)((int64_t)p.nbh * p.nc);
    if (nunits > 0) {
        hipLaunchKernelGGL(k1, dim3(nunits), dim3(Cf::NTHR), local_lds<Cf>(), stream, p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t nthr = (int64_t)p.nbh * (p.N / 2) * (p.P / 2);
    hipLaunchKernelGGL((bc_scan_kernel<IO, IO>), dim3((unsigned)((nthr + 255) / 256), 2), dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (nunits > 0) {
        // persistent grid: as many workgroups as fit on the device at once
        static int occ = -1;
        if (occ < 0) {
            int o = 0;
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, reinterpret_cast<const void*>(k3), Cf::NTHR,
                                                             grad_lds<Cf>()) != hipSuccess || o < 1)
                o = 1;
            occ = o;
        }
        int dev = 0, ncu = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu < 1)
            ncu = 256;
        (void)hipGetLastError();
        const unsigned ngrid = nunits < (unsigned)(occ * ncu) ? nunits : (unsigned)(occ * ncu);
        if (p.tl != nullptr && (int64_t)ngrid * Cf::NW > p.tl_rows) {
            // instrumented builds: no stamps unless every wave has a row
            BcParams q = p;
            q.tl = nullptr;
            hipLaunchKernelGGL(k3, dim3(ngrid), dim3(Cf::NTHR), grad_lds<Cf>(), stream, q);
        } else {
            hipLaunchKernelGGL(k3, dim3(ngrid), dim3(Cf::NTHR), grad_lds<Cf>(), stream, p);
        }
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((bc_final_kernel<IO, IO>), dim3((unsigned)p.nbh), dim3(256), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (p.a_tok) return hipSuccess;               // dA was written per token
    const int64_t batch = p.nbh / p.H;
    hipLaunchKernelGGL(bc_dA_kernel, dim3((unsigned)((p.H + 63) / 64)), dim3(64), 0, stream,
                       (const float*)p.dA_bh, p.dA, batch, p.H);
    return hipGetLastError();
}

}  // namespace bc
}  // namespace m3

namespace m3 {
namespace bc {

// Dispatch over headdim and rank for one (operand type, dstate).
template <typename OP, int N>
hipError_t launch_pr(const BcParams& p, hipStream_t s)
{
    if (p.P == 32) {
        switch (p.R) {
        case 1: return launch_cfg<Cfg<OP, N, 32, 1>>(p, s);
        case 2: return launch_cfg<Cfg<OP, N, 32, 2>>(p, s);
        default: return launch_cfg<Cfg<OP, N, 32, 4>>(p, s);
        }
    }
    switch (p.R) {
    case 1: return launch_cfg<Cfg<OP, N, 64, 1>>(p, s);
    case 2: return launch_cfg<Cfg<OP, N, 64, 2>>(p, s);
    default: return launch_cfg<Cfg<OP, N, 64, 4>>(p, s);
    }
}

// One translation unit per (operand type, dstate) set.
hipError_t launch_bf16_n32(const BcParams& p, hipStream_t s);
hipError_t launch_bf16_n64(const BcParams& p, hipStream_t s);
hipError_t launch_bf16_n128(const BcParams& p, hipStream_t s);
hipError_t launch_f32_n32(const BcParams& p, hipStream_t s);
hipError_t launch_f32_n64(const BcParams& p, hipStream_t s);

}  // namespace bc
}  // namespace m3
