// Fused chunked prefill of the Mamba-3 mixer on gfx950.
//
// Method (per batch row b, head h):
//   h_t = alpha_t R_t h_{t-1} + beta_t R_t U_{t-1} + gamma_t U_t,  U_t = B_t X_t,
//   y_t = C_t^T h_t,  alpha_t = exp(dt_t A), beta_t = (1-lam_t) dt_t alpha_t,
//   gamma_t = lam_t dt_t, R_t = blockdiag_i R(dt_t theta_t[i]).
// (Mamba-3 summary on b-lab.team: section 1, exponential-trapezoidal
// recurrence; section 2, block-rotation form and the RoPE trick; section 3,
// MIMO input/readout.)
//
// Exact rewrite that this kernel evaluates:
//  * Augmented state g_t = h_t + bhat_{t+1} U_t, bhat_t = (1-lam_t) dt_t, obeys
//    g_t = alpha_t R_t g_{t-1} + w_t U_t with look-ahead weight
//    w_t = gamma_t + bhat_{t+1} (bhat_{L+1} = 0, so g_L = h_L), and
//    y_t = C_t^T alpha_t R_t g_{t-1} + gamma_t C_t^T U_t.
//  * Within a chunk, with chunk-local prefix sums Lam_j = sum_{k<=j} dt_k A and
//    Phi_j = sum_{k<=j} dt_k theta_k (per pair), rotating B and C by
//    R(Phi_j)^T (data-dependent RoPE, Proposition 3) removes the rotation:
//      y_j = e^{Lam_j} Cbar_j^T G_in
//            + sum_{k<j} e^{Lam_j-Lam_k} w_k (Cbar_j^T Bbar_k) X_k
//            + gamma_j (Cbar_j^T Bbar_j) X_j
//    i.e. the SSD quadratic form whose mask is the decay mask times the
//    two-band (width-2 convolution) mask: the "decay mask multiplied by a
//    size-two convolutional mask" of the Towards AI explainer, section II.
//  * Chunk end (true frame): G_out = R(Phi_tot) (e^{Lam_tot} G_in
//      + sum_k e^{Lam_tot-Lam_k} w_k Bbar_k X_k).
//
// Work decomposition: one workgroup per (b, h, headdim slice of PS columns)
// walks the chunks in order.  The fp32 state G (N x PS) stays in matrix-core
// accumulator registers for the whole sequence, so the only HBM traffic is the
// inputs read once and y written once.  Each thread loads its share of chunk
// c+1's raw inputs (dt, lam, theta, B/C pairs, X rows) into registers as soon
// as chunk c's have been moved to LDS, so those loads are in flight while
// chunk c's matrix-core phases run.  Per chunk (Q tokens, T = Q*R rows):
//   A0  one wave: inclusive wavefront prefix scan of dt*A, weights w, gamma,
//       and d_k = w_k e^{Lam_tot-Lam_k}.
//   A1  all threads: angle prefix sums per (pair quad, token block) -- in
//       registers, across a wave's blocks with shuffles, across waves through
//       LDS -- sine/cosine, and rotation of B and C rows (16 bytes per lane)
//       into LDS (Bbar, Cbar as matrix-core operand rows).
//   A2  X slice into LDS: bf16 as rows, read transposed (ds_read_tr16_b64)
//       by both matrix-core products that contract over keys; fp32 as X^T.
//   C   each wave takes 16-row query tiles: S^T = Bbar Cbar^T on matrix
//       cores, two-band decay mask in fp32 registers, (S o M)^T cast to the
//       operand type, Y^T += X^T (S o M)^T, plus the state term
//       e^{Lam_j} G^T Cbar^T; y written straight from the accumulators.
//   D   each wave owns state tiles: G <- R(Phi_tot)(e^{Lam_tot} G + Bbar_d^T X)
//       on matrix cores; the new state is staged in LDS (in the operand type)
//       as the next chunk's state-term operand.  The stage
//       is double-buffered, so C and D of one chunk need no barrier between
//       them.
//
// Sequence segments (more workgroups when batch*heads*slices is small): a
// state pass walks segments 0..S-2 without outputs and records each one's end
// state (segment 0 from the true initial state, the others from zero) with
// its total decay and angle; the output pass then starts segment s from
//   G = R(Phi_{s-1})(e^{Lam_{s-1}} ... ) + G_{s-1}
// (the chunk-summary operator (a2,Phi2,S2)o(a1,Phi1,S1) =
// (a1+a2, Phi1+Phi2, e^{a2} R(Phi2) S1 + S2) applied across segments).
#pragma once

#include "m3_device.hpp"
#include "m3_internal.hpp"

namespace m3 {

struct ScanParams {
    const void *x, *B, *C;
    const float *dt, *A, *theta, *lam;
    const float *h_in;
    const void *Bp_in, *xp_in;
    void *y;
    float *h_out;
    void *Bp_out, *xp_out;
    float *ws;          // segment records: written by the state pass, read by the output pass
    int64_t batch, L, H, P;
    int p_split;
    int nbh;
    int nseg;           // sequence segments (1 = single pass)
    int seg_chunks;     // chunks per segment
};

template <typename IO, int N_, int PS_, int R_, int Q_, int NW_>
struct ScanCfg {
    using io_t = IO;
    using op_t = IO;
    static constexpr int N = N_, PS = PS_, R = R_, Q = Q_, NW = NW_;
    static constexpr int NP = N < 32 ? 32 : N;      // state rows padded to the K block
    static constexpr int NPR = N / 2;                // rotation pairs
    static constexpr int NPR4 = NPR / 4;             // pair quads (8 state rows, 16 B of bf16)
    static constexpr int T = Q * R;                  // operand rows per chunk
    static constexpr int NT = 64 * NW;
    static constexpr int E = (int)sizeof(op_t);
    static constexpr bool BF = (E == 2);
    static constexpr int PADE = 16 / E;              // 16-byte row padding
    static constexpr int LDB = NP + PADE;
    static constexpr int LDX = T + PADE;             // fp32: X^T rows
    static constexpr int LDXR = PS + PADE;           // bf16: X rows
    static constexpr int LDH = NP + PADE;
    // The state-term operand is the state rounded once to the operand type
    // (bf16 relative error 2^-9 on that term).  A hi + lo split halves the
    // error at twice the state-term matrix-core work; it is off.
    static constexpr bool HILO = false;
    static constexpr int NHT = HILO ? 2 : 1;
    static constexpr int TBA = NT / NPR4 < Q ? NT / NPR4 : Q;   // angle-scan token blocks
    static constexpr int TPB = Q / TBA;              // tokens per block
    static constexpr int BW = 64 / NPR4;             // angle blocks per wave
    static constexpr int QT = T / 16;                // 16-row query/key tiles
    static constexpr int KB = T / 32;                // 32-row key blocks
    static constexpr int PT = PS / 16;
    static constexpr int NTL = NP / 16;
    static constexpr int NTILES = NTL * PT;          // 16x16 state tiles
    static constexpr int TPW = (NTILES + NW - 1) / NW;
    static constexpr int QPW = (QT + NW - 1) / NW;
    static constexpr int QPL = (Q + 63) / 64;        // tokens per lane in A0
    static constexpr int XITEMS = T * (PS / 8);      // 8-element X row pieces
    static constexpr int XI = (XITEMS + NT - 1) / NT;
    static constexpr size_t sz_B = (size_t)T * LDB * E;
    static constexpr size_t sz_X = BF ? (size_t)T * LDXR * E : (size_t)PS * LDX * E;
    static constexpr size_t off_B = 0;
    static constexpr size_t off_C = off_B + sz_B;
    static constexpr size_t off_X = off_C + sz_B;
    static constexpr size_t off_H = off_X + sz_X;
    static constexpr size_t sz_H1 = (size_t)NHT * PS * LDH * E;   // one state stage
    static constexpr size_t off_F = off_H + 2 * sz_H1;
    static constexpr size_t nF = 4 * (size_t)Q + (size_t)NW * NPR + 2 * (size_t)NPR + 4;
    static constexpr size_t lds_bytes = off_F + nF * 4;
    // The state-only pass needs no Cbar and no state stage.
    static constexpr size_t off_X1 = off_C;
    static constexpr size_t off_F1 = off_X1 + sz_X;
    static constexpr size_t lds_bytes_state = off_F1 + nF * 4;
    // Segment record: G [N][P] fp32, then Lam_seg*log2(e), then Phi_seg[N/2].
    __host__ __device__ static int64_t rec_floats(int64_t P) { return ((int64_t)N * P + 1 + NPR + 3) / 4 * 4; }
    static_assert(T % 32 == 0, "Q*R must be a multiple of 32");
    static_assert(PS % 16 == 0, "headdim slice must be a multiple of 16");
    static_assert(N % 8 == 0 && NPR4 <= 64 && NT % NPR4 == 0, "bad dstate");
    static_assert(Q % TBA == 0, "");
    static_assert(lds_bytes <= 160 * 1024, "LDS budget");
};

// One thread's share of a chunk's raw inputs, loaded a chunk ahead.
template <class Cf> struct ChunkStage {
    using io_t = typename Cf::io_t;
    float a_dt[Cf::QPL], a_lm[Cf::QPL], a_dn[Cf::QPL], a_ln[Cf::QPL];  // dt, lam at t, t+1
    float dtv[Cf::TPB];                                                 // angle block: dt
    f32x4 thv[Cf::TPB];                                                 //   theta, 4 pairs
    IoRow8<io_t> bq[Cf::TPB][Cf::R], cq[Cf::TPB][Cf::R];                //   B, C: 4 pairs
    IoRow8<io_t> xq[Cf::XI];                                            // X row pieces
};

template <typename OP> __device__ __forceinline__ void rope_sincos(float a, float* s, float* c);
// bf16 operands carry 8 mantissa bits: the hardware sine/cosine suffices.
template <> __device__ __forceinline__ void rope_sincos<bf16>(float a, float* s, float* c)
{
    __sincosf(a, s, c);
}
template <> __device__ __forceinline__ void rope_sincos<float>(float a, float* s, float* c)
{
    sincosf(a, s, c);
}

// 2^x with the hardware exp (results below 2^-126 flush to zero; every
// argument here is <= 0).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// FULL: outputs y (and the state record when this is the last segment).
// !FULL: state pass -- each segment except the last writes its end state
// (from a zero start, except segment 0 which starts from the true state).
template <class Cf, bool FULL>
__global__ __launch_bounds__(Cf::NT) void scan_kernel(const ScanParams p)
{
    using io_t = typename Cf::io_t;
    using op_t = typename Cf::op_t;
    constexpr int N = Cf::N, NP = Cf::NP, NPR = Cf::NPR, NPR4 = Cf::NPR4, PS = Cf::PS, R = Cf::R;
    constexpr int Q = Cf::Q, T = Cf::T, NW = Cf::NW, NT = Cf::NT;
    constexpr int LDB = Cf::LDB, LDX = Cf::LDX, LDXR = Cf::LDXR, LDH = Cf::LDH;
    constexpr int TBA = Cf::TBA, TPB = Cf::TPB, BW = Cf::BW, QT = Cf::QT, KB = Cf::KB, PT = Cf::PT;
    constexpr int NTILES = Cf::NTILES, TPW = Cf::TPW, QPW = Cf::QPW, QPL = Cf::QPL;
    constexpr int NTL = Cf::NTL;
    constexpr int XI = Cf::XI, XITEMS = Cf::XITEMS;
    constexpr bool BF = Cf::BF;
    constexpr int HSTAGE = Cf::NHT * PS * LDH;   // elements of one state stage

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    op_t* sB = reinterpret_cast<op_t*>(smem + Cf::off_B);   // [T][LDB]   Bbar rows
    op_t* sC = reinterpret_cast<op_t*>(smem + Cf::off_C);   // [T][LDB]   Cbar rows
    // X slice: bf16 rows [T][LDXR] (read transposed), fp32 X^T [PS][LDX]
    op_t* sX = reinterpret_cast<op_t*>(smem + (FULL ? Cf::off_X : Cf::off_X1));
    op_t* sH = reinterpret_cast<op_t*>(smem + Cf::off_H);   // [2][NHT][PS][LDH] G^T
    float* sLW = reinterpret_cast<float*>(smem + (FULL ? Cf::off_F : Cf::off_F1));
    //   sLW: [Q][2] = (Lam_j * log2(e), w_j)
    float* sG = sLW + 2 * Q;                                 // [Q] gamma_j
    float* sD = sG + Q;                                      // [Q] w_j e^{Lam_tot-Lam_j}
    float* sWt = sD + Q;                                     // [NW][NPR] per-wave angle sums
    float* sCSt = sWt + NW * NPR;                            // [NPR][2] cos/sin Phi_tot
    float* sMisc = sCSt + 2 * NPR;                           // [0] = Lam_tot * log2(e)

    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int l16 = lane & 15, g = lane >> 4;

    // Workgroup -> (segment, b, h, headdim slice).  Consecutive workgroup ids
    // go to different XCDs (round robin over 8), so the slices of one (b, h)
    // are given ids 8 apart: they share an XCD and its L2 for B/C/theta.
    const int per_seg = (p.nbh + 7) / 8 * 8 * p.p_split;
    const int seg = blockIdx.x / per_seg;
    const int bid = blockIdx.x % per_seg;
    const int bh = (bid >> 3) / p.p_split * 8 + (bid & 7);
    const int ps = (bid >> 3) % p.p_split;
    if (bh >= p.nbh) return;
    const int64_t H = p.H, L = p.L, P = p.P;
    const int64_t b = bh / H, h = bh % H;
    const int p0 = ps * PS;
    const float Ah = p.A[h];

    const int64_t nchunks_all = (L + Q - 1) / Q;
    const int64_t c_begin = (int64_t)seg * p.seg_chunks;
    const int64_t c_end = c_begin + p.seg_chunks < nchunks_all ? c_begin + p.seg_chunks : nchunks_all;
    const bool last_seg = seg == p.nseg - 1;

    // Per-(b, h) base pointers at the segment's first token; advanced by one
    // chunk per iteration.  Offsets inside a chunk are 32-bit.
    const int sDT = (int)H, sTH = (int)(H * NPR), sBN = (int)(H * R * N), sXP = (int)(H * R * P);
    const int64_t tok0 = (b * L + c_begin * Q) * H + h;
    const float* __restrict__ dtc = p.dt + tok0;
    const float* __restrict__ lamc = p.lam + tok0;
    const float* __restrict__ thc = p.theta + tok0 * NPR;
    const io_t* __restrict__ Bc = reinterpret_cast<const io_t*>(p.B) + tok0 * R * N;
    const io_t* __restrict__ Cc = reinterpret_cast<const io_t*>(p.C) + tok0 * R * N;
    const io_t* __restrict__ Xc = reinterpret_cast<const io_t*>(p.x) + tok0 * R * P + p0;
    io_t* __restrict__ Yc = reinterpret_cast<io_t*>(p.y) + tok0 * R * P + p0;

    // Angle / rotation role: pair quad aq (pairs 4aq .. 4aq+3, state rows
    // 8aq .. 8aq+7) of the tokens of block ablk.  Consecutive lanes take
    // consecutive quads of one row, so theta, B and C load 16 bytes per lane,
    // coalesced.  Threads beyond the TBA blocks repeat the last block and
    // neither contribute to the scan nor store.
    const int aq = tid % NPR4;
    const bool aact = tid / NPR4 < TBA;
    const int ablk = aact ? tid / NPR4 : TBA - 1;

    // X piece of item `it`: (row rho, 8-column group cg).
    auto xmap = [](int it, int& rho, int& cg) {
        if constexpr (BF) { rho = it / (PS / 8); cg = it % (PS / 8); }   // rows: coalesced
        else { rho = it % T; cg = it / T; }                               // X^T: conflict-free
    };

    // Padded state columns (N < NP) are constant zeros.
    if constexpr (NP > N) {
        for (int idx = tid; idx < T * (NP - N); idx += NT) {
            const int row = idx / (NP - N), col = N + idx % (NP - N);
            sB[row * LDB + col] = from_f32<op_t>(0.f);
            if constexpr (FULL) sC[row * LDB + col] = from_f32<op_t>(0.f);
        }
    }

    // ---- chunk input loads -------------------------------------------------
    // Token indices are clamped to the last valid token (values past it are
    // masked on use).  Loads are issued in the order the next iteration
    // consumes them, every one unconditional, so the in-order load counter
    // lets each phase wait only for its own data.
    ChunkStage<Cf> st;
    auto issue_loads = [&](int64_t c) {
        const int64_t t0 = c * Q;
        const int jl = (int)((L - 1 - t0) < (Q - 1) ? (L - 1 - t0) : (Q - 1));  // last valid j
        const int jn = (int)((L - 1 - t0) < Q ? (L - 1 - t0) : Q);              // last valid j+1
#pragma unroll
        for (int kk = 0; kk < QPL; ++kk) {
            const int j = lane * QPL + kk;
            const int jc = j < jl ? j : jl;
            const int jnc = j + 1 < jn ? j + 1 : jn;
            st.a_dt[kk] = dtc[jc * sDT];
            st.a_lm[kk] = lamc[jc * sDT];
            st.a_dn[kk] = dtc[jnc * sDT];
            st.a_ln[kk] = lamc[jnc * sDT];
        }
#pragma unroll
        for (int k = 0; k < XI; ++k) {
            int it = tid + k * NT;
            if (XITEMS % NT != 0 && it >= XITEMS) it = XITEMS - 1;   // duplicate
            int rho, cg;
            xmap(it, rho, cg);
            const int j = rho / R < jl ? rho / R : jl;
            st.xq[k].load(Xc + j * sXP + (rho % R) * (int)P + 8 * cg);
        }
#pragma unroll
        for (int kk = 0; kk < TPB; ++kk) {
            const int j = ablk * TPB + kk < jl ? ablk * TPB + kk : jl;
            st.dtv[kk] = dtc[j * sDT];
            st.thv[kk] = *reinterpret_cast<const f32x4*>(thc + j * sTH + 4 * aq);
        }
#pragma unroll
        for (int kk = 0; kk < TPB; ++kk) {
            const int j = ablk * TPB + kk < jl ? ablk * TPB + kk : jl;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int off = j * sBN + r * N + 8 * aq;
                st.bq[kk][r].load(Bc + off);
                if constexpr (FULL) st.cq[kk][r].load(Cc + off);
            }
        }
    };

    // The first chunk's loads go out before the initial state is formed.
    if (c_begin < c_end) issue_loads(c_begin);

    // ---- initial state ------------------------------------------------------
    // Wave wv owns state tiles tau = wv*TPW + k, p-tile major (pt = tau / NTL,
    // nt = tau % NTL): rows 16*nt + 4*g + i, column p0 + 16*pt + l16 of the
    // N x P state.  A wave's tiles then share one d-scaled X operand in D.
    f32x4 hacc[TPW];
    const int64_t rec_sz = Cf::rec_floats(P);
    float* recs = p.ws + (int64_t)bh * (p.nseg - 1) * rec_sz;   // this (b, h)'s records
    if (seg == 0) {
        // G_0 = h_0 + bhat_1 B_prev X_prev.  All loads first, then arithmetic.
        float hv[TPW][4], bv[TPW][4][R], xv[TPW][R];
        const io_t* Bp = reinterpret_cast<const io_t*>(p.Bp_in);
        const io_t* xp = reinterpret_cast<const io_t*>(p.xp_in);
        const float* hsrc = p.h_in;
        float bhat1 = 0.f;
        if (hsrc != nullptr) {
#pragma unroll
            for (int k = 0; k < TPW; ++k) {
                const int tau = wv * TPW + k < NTILES ? wv * TPW + k : NTILES - 1;
                const int pt = tau / NTL, nt = tau % NTL;
                const int64_t col = p0 + 16 * pt + l16;
#pragma unroll
                for (int r = 0; r < R; ++r) xv[k][r] = to_f32(xp[((int64_t)bh * R + r) * P + col]);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int n = 16 * nt + 4 * g + i < N ? 16 * nt + 4 * g + i : N - 1;
                    hv[k][i] = hsrc[((int64_t)bh * N + n) * P + col];
#pragma unroll
                    for (int r = 0; r < R; ++r) bv[k][i][r] = to_f32(Bp[((int64_t)bh * R + r) * N + n]);
                }
            }
            if (L > 0) bhat1 = (1.f - p.lam[(b * L) * H + h]) * p.dt[(b * L) * H + h];
        } else {
#pragma unroll
            for (int k = 0; k < TPW; ++k) {
#pragma unroll
                for (int r = 0; r < R; ++r) xv[k][r] = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    hv[k][i] = 0.f;
#pragma unroll
                    for (int r = 0; r < R; ++r) bv[k][i][r] = 0.f;
                }
            }
        }
#pragma unroll
        for (int k = 0; k < TPW; ++k) {
            const int tau = wv * TPW + k;
            const int nt = tau % NTL;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float u = 0.f;
#pragma unroll
                for (int r = 0; r < R; ++r) u += bv[k][i][r] * xv[k][r];
                const bool ok = tau < NTILES && 16 * nt + 4 * g + i < N;
                hacc[k][i] = ok ? hv[k][i] + bhat1 * u : 0.f;
            }
        }
    } else if constexpr (FULL) {
        // Combine the end states of the earlier segments (associative
        // operator of the chunk summaries): G = R(Phi_s)(2^{l2_s} G) + G_s.
#pragma unroll
        for (int k = 0; k < TPW; ++k) {
            const int tau = wv * TPW + k < NTILES ? wv * TPW + k : NTILES - 1;
            const int pt = tau / NTL, nt = tau % NTL;
            const int64_t col = p0 + 16 * pt + l16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int n = 16 * nt + 4 * g + i < N ? 16 * nt + 4 * g + i : N - 1;
                hacc[k][i] = recs[(int64_t)n * P + col];
            }
        }
        // Records are folded in order; the next record's values are loaded
        // while the current one is applied (one round trip per record would
        // otherwise serialise the prologue).
        float nv[TPW][4], nphi[TPW][2], nl2 = 0.f;
        auto load_rec = [&](int s) {
            const float* rec = recs + (int64_t)s * rec_sz;
            nl2 = rec[(int64_t)N * P];
#pragma unroll
            for (int k = 0; k < TPW; ++k) {
                const int tau = wv * TPW + k < NTILES ? wv * TPW + k : NTILES - 1;
                const int pt = tau / NTL, nt = tau % NTL;
                const int64_t col = p0 + 16 * pt + l16;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int n = 16 * nt + 4 * g + i < N ? 16 * nt + 4 * g + i : N - 2 + (i & 1);
                    nv[k][i] = rec[(int64_t)n * P + col];
                }
#pragma unroll
                for (int ip = 0; ip < 2; ++ip) {
                    const int n = 16 * nt + 4 * g + 2 * ip < N ? 16 * nt + 4 * g + 2 * ip : N - 2;
                    nphi[k][ip] = rec[(int64_t)N * P + 1 + n / 2];
                }
            }
        };
        if (seg > 1) load_rec(1);
        for (int s = 1; s < seg; ++s) {
            float cv[TPW][4], cphi[TPW][2];
#pragma unroll
            for (int k = 0; k < TPW; ++k) {
#pragma unroll
                for (int i = 0; i < 4; ++i) cv[k][i] = nv[k][i];
                cphi[k][0] = nphi[k][0];
                cphi[k][1] = nphi[k][1];
            }
            const float sc = fast_exp2(nl2);
            if (s + 1 < seg) load_rec(s + 1);
#pragma unroll
            for (int k = 0; k < TPW; ++k) {
#pragma unroll
                for (int ip = 0; ip < 2; ++ip) {
                    float sn, cs;
                    sincosf(cphi[k][ip], &sn, &cs);
                    const float a0 = sc * hacc[k][2 * ip], a1 = sc * hacc[k][2 * ip + 1];
                    hacc[k][2 * ip] = cs * a0 - sn * a1 + cv[k][2 * ip];
                    hacc[k][2 * ip + 1] = sn * a0 + cs * a1 + cv[k][2 * ip + 1];
                }
            }
        }
#pragma unroll
        for (int k = 0; k < TPW; ++k) {
            const int tau = wv * TPW + k;
            const int nt = tau % NTL;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (!(tau < NTILES && 16 * nt + 4 * g + i < N)) hacc[k][i] = 0.f;
        }
    } else {
#pragma unroll
        for (int k = 0; k < TPW; ++k) hacc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // Stage G^T (operand type; optionally hi + lo) into state buffer `buf`.
    auto stage_state = [&](int buf) {
        op_t* base = sH + buf * HSTAGE;
#pragma unroll
        for (int k = 0; k < TPW; ++k) {
            const int tau = wv * TPW + k;
            if (tau < NTILES) {
                const int pt = tau / NTL, nt = tau % NTL;
                op_t* dst = base + (16 * pt + l16) * LDH + 16 * nt + 4 * g;
                const f32x4 v = hacc[k];
                lds_store4(dst, v[0], v[1], v[2], v[3]);
                if constexpr (Cf::HILO) {
                    float lo[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) lo[i] = v[i] - to_f32(from_f32<op_t>(v[i]));
                    lds_store4(dst + PS * LDH, lo[0], lo[1], lo[2], lo[3]);
                }
            }
        }
    };
    int hbuf = 0;
    if constexpr (FULL) stage_state(hbuf);

    double l2seg = 0.0, phiseg[4] = {0.0, 0.0, 0.0, 0.0};   // segment totals (state pass)

    for (int64_t c = c_begin; c < c_end; ++c) {
        const int64_t t0 = c * Q;
        const int jl = (int)((L - 1 - t0) < (Q - 1) ? (L - 1 - t0) : (Q - 1));

        // ---- A0: decay prefix scan and trapezoid weights --------------------
        // Every wave evaluates it (uniform load/consume pattern); wave 0 stores.
        {
            float a[QPL], wt[QPL], gm[QPL];
            float run = 0.f;
#pragma unroll
            for (int kk = 0; kk < QPL; ++kk) {
                const int j = lane * QPL + kk;
                const bool ok = j < Q && j <= jl;
                const bool okn = j < Q && t0 + j + 1 < L;
                const float d = ok ? st.a_dt[kk] : 0.f;
                const float lm = ok ? st.a_lm[kk] : 0.f;
                const float dn = okn ? st.a_dn[kk] : 0.f;
                const float ln = okn ? st.a_ln[kk] : 0.f;
                gm[kk] = lm * d;
                wt[kk] = gm[kk] + (1.f - ln) * dn;
                run += d * Ah;
                a[kk] = run;
            }
            const float incl = wave_inclusive_sum(run);
            const float excl = incl - run;
            const float l2tot = wave_read_lane(incl, (Q - 1) / QPL) * kLog2e;
#pragma unroll
            for (int kk = 0; kk < QPL; ++kk) {
                const int j = lane * QPL + kk;
                if (wv == 0 && j < Q) {
                    const float l2 = (excl + a[kk]) * kLog2e;
                    *reinterpret_cast<float2*>(sLW + 2 * j) = make_float2(l2, wt[kk]);
                    sG[j] = gm[kk];
                    sD[j] = wt[kk] * fast_exp2(l2tot - l2);
                }
            }
            if (wv == 0 && lane == 0) sMisc[0] = l2tot;
            if constexpr (!FULL) l2seg += (double)l2tot;
        }

        // ---- A2: X slice into LDS ----------------------------------------------
#pragma unroll
        for (int k = 0; k < XI; ++k) {
            int it = tid + k * NT;
            if (XITEMS % NT != 0 && it >= XITEMS) it = XITEMS - 1;   // identical duplicate
            int rho, cg;
            xmap(it, rho, cg);
            const bool ok = rho / R <= jl;
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = ok ? st.xq[k].get(e) : 0.f;
            if constexpr (BF) {
                lds_store8(sX + rho * LDXR + 8 * cg, v);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) sX[(8 * cg + e) * LDX + rho] = v[e];
            }
        }

        // ---- A1: angle prefix per (pair quad, token block), rotate B and C --
        f32x4 loc[TPB], aoff;
        {
            f32x4 run = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < TPB; ++kk) {
                const bool ok = ablk * TPB + kk <= jl;
#pragma unroll
                for (int e = 0; e < 4; ++e) run[e] += ok ? st.dtv[kk] * st.thv[kk][e] : 0.f;
                loc[kk] = run;
            }
            // Exclusive scan of the block sums over the blocks of this wave
            // (lanes aq, aq + NPR4, ...), then across waves through LDS.
            const f32x4 tot = aact ? run : f32x4{0.f, 0.f, 0.f, 0.f};
            f32x4 inc = tot;
#pragma unroll
            for (int d = 1; d < BW; d <<= 1) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float v = __shfl_up(inc[e], d * NPR4, 64);
                    if (lane >= d * NPR4) inc[e] += v;
                }
            }
            aoff = inc - tot;
            if (lane / NPR4 == BW - 1) *reinterpret_cast<f32x4*>(sWt + wv * NPR + 4 * aq) = inc;
        }
        __syncthreads();
        {
#pragma unroll
            for (int w2 = 0; w2 < NW - 1; ++w2) {
                const f32x4 v = *reinterpret_cast<const f32x4*>(sWt + w2 * NPR + 4 * aq);
                if (w2 < wv) aoff += v;
            }
#pragma unroll
            for (int kk = 0; kk < TPB; ++kk) {
                const int j = ablk * TPB + kk;
                const bool ok = j <= jl;
                float cs[4], sn[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) rope_sincos<op_t>(aoff[e] + loc[kk][e], &sn[e], &cs[e]);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const int rho = j * R + r;
                    // R(Phi)^T applied to each pair
                    float o[8];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float b0 = ok ? st.bq[kk][r].get(2 * e) : 0.f;
                        const float b1 = ok ? st.bq[kk][r].get(2 * e + 1) : 0.f;
                        o[2 * e] = cs[e] * b0 + sn[e] * b1;
                        o[2 * e + 1] = cs[e] * b1 - sn[e] * b0;
                    }
                    if (aact) lds_store8(sB + rho * LDB + 8 * aq, o);
                    if constexpr (FULL) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float c0 = ok ? st.cq[kk][r].get(2 * e) : 0.f;
                            const float c1 = ok ? st.cq[kk][r].get(2 * e + 1) : 0.f;
                            o[2 * e] = cs[e] * c0 + sn[e] * c1;
                            o[2 * e + 1] = cs[e] * c1 - sn[e] * c0;
                        }
                        if (aact) lds_store8(sC + rho * LDB + 8 * aq, o);
                    }
                }
            }
            if (aact && ablk == TBA - 1) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float phi = aoff[e] + loc[TPB - 1][e];
                    float sn, cs;
                    sincosf(phi, &sn, &cs);
                    sCSt[2 * (4 * aq + e)] = cs;
                    sCSt[2 * (4 * aq + e) + 1] = sn;
                    if constexpr (!FULL) phiseg[e] += (double)phi;
                }
            }
        }
        // This chunk's raw inputs now live in LDS: fetch the next chunk's.
        dtc += Q * sDT; lamc += Q * sDT; thc += Q * sTH;
        Bc += Q * sBN; Cc += Q * sBN; Xc += Q * sXP;
        if (c + 1 < c_end) issue_loads(c + 1);
        __syncthreads();

        // ---- C: outputs of this chunk --------------------------------------
        if constexpr (FULL) {
            const op_t* sHc = sH + hbuf * HSTAGE;
#pragma unroll 1
            for (int qi = 0; qi < QPW; ++qi) {
                const int qt = (qi & 1) ? qi * NW + (NW - 1 - wv) : qi * NW + wv;
                if (qt >= QT) continue;
                const int rq = 16 * qt + l16;
                const int jq = rq / R;
                const float2 lwq = *reinterpret_cast<const float2*>(sLW + 2 * jq);
                const float l2q = lwq.x;
                const float gq = sG[jq];

                Frag<op_t> cf[NP / 32];
#pragma unroll
                for (int s = 0; s < NP / 32; ++s) lds_frag8(cf[s], sC + rq * LDB + 32 * s + 8 * g);

                f32x4 yacc[PT];
                const float sq = fast_exp2(l2q);
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) {
                    yacc[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < NP / 32; ++s) {
                        Frag<op_t> a;
                        lds_frag8(a, sHc + (16 * pt + l16) * LDH + 32 * s + 8 * g);
                        mma(a, cf[s], yacc[pt]);
                        if constexpr (Cf::HILO) {
                            lds_frag8(a, sHc + PS * LDH + (16 * pt + l16) * LDH + 32 * s + 8 * g);
                            mma(a, cf[s], yacc[pt]);
                        }
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) yacc[pt][i] *= sq;
                }

#pragma unroll 1
                for (int kp = 0; kp <= qt; kp += 2) {
                    Frag<op_t> pf;
                    const bool second = kp + 1 <= qt;   // wave-uniform
#pragma unroll
                    for (int half = 0; half < 2; ++half) {
                        const int kt = kp + half;
                        if (kt <= qt) {
                            f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                            for (int s = 0; s < NP / 32; ++s) {
                                Frag<op_t> a;
                                lds_frag8(a, sB + (16 * kt + l16) * LDB + 32 * s + 8 * g);
                                mma(a, cf[s], sacc);
                            }
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const int jk = (16 * kt + 4 * g) / R + i / R;
                                const float2 lw = *reinterpret_cast<const float2*>(sLW + 2 * jk);
                                const float m = jk < jq ? lw.y * fast_exp2(l2q - lw.x)
                                                        : (jk == jq ? gq : 0.f);
                                pf.set(4 * half + i, jk <= jq ? sacc[i] * m : 0.f);
                            }
                        } else {
#pragma unroll
                            for (int i = 0; i < 4; ++i) pf.set(4 * half + i, 0.f);
                        }
                    }
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt) {
                        Frag<op_t> xa;
                        if constexpr (BF) {
                            // X^T[p][keys]: keys 16*kp + 4*g + 0..3 (slots 0..3) and
                            // 16*(kp+1) + 4*g + 0..3 (slots 4..7), column p = 16*pt + l16.
                            const bf16* xr = sX + (16 * kp + 4 * g + (l16 >> 2)) * LDXR + 16 * pt
                                             + 4 * (l16 & 3);
                            const bf16x4 lo = lds_read_tr4(xr);
                            bf16x4 hi = {(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
                            if (second) hi = lds_read_tr4(xr + 16 * LDXR);
#pragma unroll
                            for (int e = 0; e < 4; ++e) { xa.v[e] = lo[e]; xa.v[4 + e] = hi[e]; }
                        } else {
                            const op_t* xr = sX + (16 * pt + l16) * LDX;
                            if (second) lds_frag4x2(xa, xr + 16 * kp + 4 * g, xr + 16 * (kp + 1) + 4 * g);
                            else lds_frag4(xa, xr + 16 * kp + 4 * g);
                        }
                        mma(xa, pf, yacc[pt]);
                    }
                }

                if (jq <= jl) {
                    io_t* yrow = Yc + jq * sXP + (rq % R) * (int)P;
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt) gstore4(yrow + 16 * pt + 4 * g, yacc[pt]);
                }
            }
            Yc += Q * sXP;
        }

        // ---- D: state update  G <- R(Phi_tot)(e^{Lam_tot} G + Bbar_d^T X) --
        {
            const float aT = fast_exp2(sMisc[0]);
            // Tiles of a wave: tau = wv*TPW + k -> (nt, pt).  The d-scaled X
            // operand depends only on (pt, kb) and the Bbar^T operand only on
            // (nt, kb); each is rebuilt only when its index changes.
            Frag<op_t> bfr[KB], xfr[KB];
            int cur_nt = -1, cur_pt = -1;
#pragma unroll
            for (int k = 0; k < TPW; ++k) {
                const int tau = wv * TPW + k;
                if (tau < NTILES) {
                    const int pt = tau / NTL, nt = tau % NTL;
                    if (nt != cur_nt) {
                        // A operand Bbar^T: rows n = 16*nt + l16, K-slots keys 32*kb + 8*g + e.
#pragma unroll
                        for (int kb = 0; kb < KB; ++kb) {
                            if constexpr (BF) {
                                const bf16* br = sB + (32 * kb + 8 * g + (l16 >> 2)) * LDB + 16 * nt
                                                 + 4 * (l16 & 3);
                                const bf16x4 lo = lds_read_tr4(br);
                                const bf16x4 hi = lds_read_tr4(br + 4 * LDB);
#pragma unroll
                                for (int e = 0; e < 4; ++e) { bfr[kb].v[e] = lo[e]; bfr[kb].v[4 + e] = hi[e]; }
                            } else {
#pragma unroll
                                for (int e = 0; e < 8; ++e)
                                    bfr[kb].set(e, sB[(32 * kb + 8 * g + e) * LDB + 16 * nt + l16]);
                            }
                        }
                        cur_nt = nt;
                    }
                    if (pt != cur_pt) {
                        // B operand X_d[keys][p] = d_key X[key][p]: column p = 16*pt + l16.
#pragma unroll
                        for (int kb = 0; kb < KB; ++kb) {
                            float xv[8];
                            if constexpr (BF) {
                                const bf16* xr = sX + (32 * kb + 8 * g + (l16 >> 2)) * LDXR + 16 * pt
                                                 + 4 * (l16 & 3);
                                const bf16x4 lo = lds_read_tr4(xr);
                                const bf16x4 hi = lds_read_tr4(xr + 4 * LDXR);
#pragma unroll
                                for (int e = 0; e < 4; ++e) { xv[e] = (float)lo[e]; xv[4 + e] = (float)hi[e]; }
                            } else {
#pragma unroll
                                for (int e = 0; e < 8; ++e) xv[e] = sX[(16 * pt + l16) * LDX + 32 * kb + 8 * g + e];
                            }
#pragma unroll
                            for (int e = 0; e < 8; ++e) xfr[kb].set(e, xv[e] * sD[(32 * kb + 8 * g + e) / R]);
                        }
                        cur_pt = pt;
                    }
                    f32x4 acc = hacc[k];
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[i] *= aT;
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) mma(bfr[kb], xfr[kb], acc);
#pragma unroll
                    for (int ip = 0; ip < 2; ++ip) {
                        const int n = 16 * nt + 4 * g + 2 * ip;
                        if (n < N) {
                            const float cs = sCSt[n], sn = sCSt[n + 1];
                            const float a0 = acc[2 * ip], a1 = acc[2 * ip + 1];
                            acc[2 * ip] = cs * a0 - sn * a1;
                            acc[2 * ip + 1] = sn * a0 + cs * a1;
                        }
                    }
                    hacc[k] = acc;
                }
            }
            if constexpr (FULL) {
                hbuf ^= 1;
                stage_state(hbuf);
            }
        }
        __syncthreads();
    }

    if constexpr (!FULL) {
        // End state of this segment and its decay / angle totals.
        float* rec = recs + (int64_t)seg * rec_sz;
#pragma unroll
        for (int k = 0; k < TPW; ++k) {
            const int tau = wv * TPW + k;
            if (tau < NTILES) {
                const int pt = tau / NTL, nt = tau % NTL;
                const int64_t col = p0 + 16 * pt + l16;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int n = 16 * nt + 4 * g + i;
                    if (n < N) rec[(int64_t)n * P + col] = hacc[k][i];
                }
            }
        }
        if (ps == 0) {
            if (tid == 0) rec[(int64_t)N * P] = (float)l2seg;
            if (aact && ablk == TBA - 1) {
                const double twopi = 6.283185307179586;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    rec[(int64_t)N * P + 1 + 4 * aq + e] =
                        (float)(phiseg[e] - twopi * floor(phiseg[e] / twopi));
            }
        }
        return;
    }

    // ---- final state record (last segment) ----------------------------------
    if (FULL && last_seg && p.h_out != nullptr) {
#pragma unroll
        for (int k = 0; k < TPW; ++k) {
            const int tau = wv * TPW + k;
            if (tau < NTILES) {
                const int pt = tau / NTL, nt = tau % NTL;
                const int64_t col = p0 + 16 * pt + l16;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int n = 16 * nt + 4 * g + i;
                    if (n < N) p.h_out[((int64_t)bh * N + n) * P + col] = hacc[k][i];
                }
            }
        }
        if (ps == 0) {
            const io_t* Bm = reinterpret_cast<const io_t*>(p.B);
            const io_t* X = reinterpret_cast<const io_t*>(p.x);
            io_t* Bo = reinterpret_cast<io_t*>(p.Bp_out) + (int64_t)bh * R * N;
            io_t* xo = reinterpret_cast<io_t*>(p.xp_out) + (int64_t)bh * R * P;
            const io_t* Bi = reinterpret_cast<const io_t*>(p.Bp_in);
            const io_t* xi = reinterpret_cast<const io_t*>(p.xp_in);
            const int64_t tl = (b * L + (L - 1)) * H + h;
            for (int idx = tid; idx < R * N; idx += NT) {
                io_t v = from_f32<io_t>(0.f);
                if (L > 0) v = Bm[tl * R * N + idx];
                else if (Bi != nullptr) v = Bi[(int64_t)bh * R * N + idx];
                Bo[idx] = v;
            }
            for (int64_t idx = tid; idx < R * P; idx += NT) {
                io_t v = from_f32<io_t>(0.f);
                if (L > 0) v = X[tl * R * P + idx];
                else if (xi != nullptr) v = xi[(int64_t)bh * R * P + idx];
                xo[idx] = v;
            }
        }
    }
}

template <class Cf>
size_t scan_workspace_bytes(int64_t nbh, int64_t P, int nseg)
{
    return nseg > 1 ? (size_t)nbh * (size_t)(nseg - 1) * (size_t)Cf::rec_floats(P) * 4 : 0;
}

// Raise the dynamic-LDS limit of one kernel once per process.
template <class Cf, bool FULL>
hipError_t scan_set_lds_limit()
{
    static hipError_t status = [] {
        const void* f = reinterpret_cast<const void*>(&scan_kernel<Cf, FULL>);
        return hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize,
                                   (int)(FULL ? Cf::lds_bytes : Cf::lds_bytes_state));
    }();
    return status;
}

template <class Cf>
hipError_t launch_scan(const ScanParams& p, hipStream_t stream)
{
    const int64_t per_seg = (int64_t)((p.nbh + 7) / 8) * 8 * p.p_split;
    hipError_t e;
    (void)hipGetLastError();
    if (p.nseg > 1) {
        e = scan_set_lds_limit<Cf, false>();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((scan_kernel<Cf, false>), dim3((unsigned)(per_seg * (p.nseg - 1))),
                           dim3(Cf::NT), Cf::lds_bytes_state, stream, p);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    e = scan_set_lds_limit<Cf, true>();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((scan_kernel<Cf, true>), dim3((unsigned)(per_seg * p.nseg)), dim3(Cf::NT),
                       Cf::lds_bytes, stream, p);
    return hipGetLastError();
}

}  // namespace m3
