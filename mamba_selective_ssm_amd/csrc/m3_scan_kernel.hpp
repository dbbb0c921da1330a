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
// Work decomposition: one workgroup per (sequence segment, b, h, headdim
// slice of PS columns) walks the segment's chunks in order.  Its waves have
// two roles:
//   math waves (NWM) hold the fp32 state G (N x PS) in matrix-core
//     accumulator registers for the whole segment and run the matrix-core
//     phases of chunk c:
//     C  outputs: per 16-row query tile, S^T = Bbar Cbar^T, the two-band decay
//        mask in fp32 registers, Y^T += X^T (S o M)^T, plus the state term
//        e^{Lam_j} G^T Cbar^T; y stored straight from the accumulators.  A
//        wave owns whole headdim tiles of y (recomputing the score tiles it
//        needs), so no wave waits for another inside a chunk.
//     D  state update G <- R(Phi_tot)(e^{Lam_tot} G + Bbar_d^T X) on matrix
//        cores; the new G^T is staged in LDS (operand type) for the next
//        chunk's state term.
//   prep waves (NWP) meanwhile turn chunk c+1's raw inputs (loaded into
//     registers one chunk earlier) into matrix-core operands in the other LDS
//     buffer, issuing the loads of chunk c+2 part by part as the registers
//     they refill are consumed:
//     A0 one wave: wavefront prefix scan of dt*A (DPP), weights w, gamma and
//        d_k = w_k e^{Lam_tot-Lam_k}.
//     A1 row-coalesced: a prep wave owns a contiguous run of the chunk's
//        operand rows and a lane one pair quad (4 rotation pairs, 16 bytes of
//        bf16 B/C/theta) of some of them, so one load instruction covers
//        whole rows; the angle prefix is a sum over the lane's rows, a scan
//        across the wave's lane groups and, through LDS, across the prep
//        waves; then sine/cosine and the rotation of B and C rows into LDS.
//        (Shapes whose rows do not split that way: a wave owns pair quads
//        over all rows and scans the angles with DPP inside the wave.)
//     A2 the X slice into LDS (bf16 as rows, read transposed by
//        ds_read_tr16_b64; fp32 as X^T).
// One barrier per chunk separates producer and consumer buffers.
//
// Sequence segments (more workgroups when batch*heads*slices is small): a
// state pass walks segments 0..S-2 without outputs and records each one's end
// state (segment 0 from the true initial state, the others from zero) with
// its total decay and the cosine/sine of its total angle; the output pass
// starts segment s from the fold of records 0..s-1 under the chunk-summary
// operator (a2,Phi2,S2)o(a1,Phi1,S1) = (a1+a2, Phi1+Phi2, e^{a2} R(Phi2) S1 + S2),
// computed by its math waves while the prep waves wait for the first chunk.
// (The kernel boundary orders the two passes; any hand-off between
// workgroups of one pass would need device-scope fences, which write back
// and invalidate the L2 under every workgroup still streaming.)
#pragma once

#include <type_traits>

#include "m3_device.hpp"
#include "m3_internal.hpp"
#include "m3_timeline.hpp"

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
    OptParams opt;      // head groups, per-token decay, phase mode, pre-mixer
    int64_t batch, L, H, P;
    int p_split;
    int nbh;
    int nseg;           // sequence segments (1 = single pass); per-sequence mode: the most
                        // any sequence has (the record stride)
    int seg_chunks;     // chunks per segment
    int nslots;         // packed sequences, per-sequence segments: (sequence, segment) slots
                        // launched (an upper bound); 0: nseg segments of every sequence
    int young_from;     // compute units of the device: with two workgroups per CU, the ids
                        // from here on are the second workgroup on their CU
    unsigned long long* tl;   // per-wave phase stamps (instrumented builds only), else null
    int64_t tl_rows;          // rows of kTlSlots entries that tl holds
};

// (The per-wave phase timeline of instrumented builds: m3_timeline.hpp.)

// NBUF_ = 2: two chunk buffers in LDS (the prep waves fill one while the
// math waves read the other); 1: one chunk buffer for chunks too long for two
// (128 operand rows at dstate 128): the prep waves keep chunk c+1's prepared
// operands in registers while the math waves run chunk c, and store them
// after a second barrier per chunk.
template <typename IO, int N_, int PS_, int R_, int Q_, int NWM_, int NWP_, int OCC_, int NBUF_ = 2>
struct ScanCfg {
    using io_t = IO;
    using op_t = IO;
    static constexpr int N = N_, PS = PS_, R = R_, Q = Q_, NWM = NWM_, NWP = NWP_, OCC = OCC_;
    static constexpr int NBUF = NBUF_;
    // raised issue priority for the younger half of the prep waves (the
    // dstate-128, rank-1 variant with two chunk buffers, where it was measured
    // to help)
    static constexpr bool YOUNG_PRIO = NWP_ == 8 && R_ == 1 && N_ == 128 && NBUF_ == 2;
    static constexpr int NW = NWM + NWP;
    static constexpr int NT = 64 * NW;
    static constexpr int NP = N < 32 ? 32 : N;      // state rows padded to the K block
    static constexpr int NPR = N / 2;                // rotation pairs
    static constexpr int NPR4 = NPR / 4;             // pair quads (8 state rows, 16 B of bf16)
    static constexpr int T = Q * R;                  // operand rows per chunk
    static constexpr int E = (int)sizeof(op_t);
    static constexpr bool BF = (E == 2);
    static constexpr int PADE = 16 / E;              // 16-byte row padding
#ifndef M3_PAD_BC_BYTES
#define M3_PAD_BC_BYTES 16
#endif
#ifndef M3_PAD_X_BYTES
#define M3_PAD_X_BYTES 16
#endif
    static constexpr int LDB = NP + M3_PAD_BC_BYTES / E;   // Bbar, Cbar rows
    static constexpr int LDX = T + PADE;             // fp32: X^T rows
    static constexpr int LDXR = PS + M3_PAD_X_BYTES / E;   // bf16: X rows
    static constexpr int LDH = NP + PADE;
    // prep waves: pair quads per wave, lanes per quad, tokens per lane
    static constexpr int QPWV = NPR4 >= NWP ? NPR4 / NWP : 1;
    static constexpr int WA = NPR4 / QPWV;           // prep waves with quads
    static constexpr int LQ = 64 / QPWV;
    static constexpr int TPL = (Q + LQ - 1) / LQ;
    static constexpr int QPL = (Q + 63) / 64;        // tokens per lane in A0
    // Row-coalesced prep (CL): prep wave w owns the operand rows
    // [RPW w, RPW (w+1)) of a chunk, and lane l takes pair quad l % NPR4 of
    // rows RPW w + KP (l / NPR4) + k, k < KP, so that the lanes of one load
    // instruction cover MQ whole rows of B, C and theta.  The angle prefix
    // over the rows is then a sum within the lane, a scan across the wave's
    // MQ lane groups and a scan across the prep waves (their totals
    // exchanged in LDS).  Otherwise a prep wave owns pair quads over all rows
    // (16-byte pieces of many rows per load instruction).
    static constexpr int RPW = T / NWP;              // operand rows per prep wave
    static constexpr int MQ = 64 / NPR4;             // rows per load instruction
    static constexpr bool CL = (64 % NPR4 == 0) && (T % NWP == 0) && (RPW % MQ == 0);
    static constexpr int KP = CL ? RPW / MQ : 1;     // rows per lane
    static constexpr int SL = CL ? KP : TPL;         // raw B/C/theta slots per prep lane
    static constexpr int SRK = CL ? 1 : R;           // ranks per slot
    static constexpr int XITEMS = T * (PS / 8);      // 8-element X row pieces
    static constexpr int XI = (XITEMS + 64 * NWP - 1) / (64 * NWP);
    // math waves
    static constexpr int QT = T / 16;                // 16-row query/key tiles
    static constexpr int KB = T / 32;                // 32-row key blocks
    static constexpr int PT = PS / 16;
    static constexpr int NTL = NP / 16;
    static constexpr int NTILES = NTL * PT;          // 16x16 state tiles
    static constexpr int TPW = (NTILES + NWM - 1) / NWM;
    // Math waves split C into PG headdim groups x QG query groups; query
    // tiles are dealt out in pairs (qt, QT-1-qt) so every wave gets the same
    // number of score tiles, and each score tile is computed by PG waves.
    static constexpr int PG = PT < 2 ? PT : 2;       // headdim-tile groups of math waves
    static constexpr int QG = NWM / PG;              // query-tile groups
    static constexpr int PPW = PT / PG;              // headdim tiles per math wave
    static constexpr int QPW = (QT + QG - 1) / QG;   // query tiles per math wave
    // When every math wave reads in C only the state rows it writes itself in
    // D, one state stage suffices (LDS operations of a wave stay in order).
    static constexpr bool SH1 = (QG == 1) && (NTILES % NWM == 0);
    // Segment records folded per round trip in the output pass prologue
    // (8*TPW + 1 registers each).
    static constexpr int FB = TPW <= 2 ? 4 : (TPW <= 4 || OCC == 1 ? 2 : 1);
    // LDS: two chunk buffers {Bbar, Cbar, X, scalars} and the state stage(s).
    static constexpr size_t sz_B = (size_t)T * LDB * E;
    static constexpr size_t sz_X = BF ? (size_t)T * LDXR * E : (size_t)PS * LDX * E;
    // chunk scalars: (l2, w)[Q], gamma[Q], d[Q], (cos, sin) of Phi_tot [NPR],
    // misc[4], u[Q] (w_k relative to its key tile's last token)
    static constexpr size_t nF = 5 * (size_t)Q + 2 * (size_t)NPR + 4;
    static constexpr size_t sz_H1 = (size_t)PS * LDH * E;
    // Pre-mixer (PM): gains [2][N] and biases [2][R][N] (each prep wave stages
    // the entries of its own pair quads), partial row sums of squares
    // [WA][2][T] exchanged between the prep waves, and their counter.
    static constexpr size_t sz_PMW = 2 * (size_t)(R + 1) * N * 4;
    static constexpr size_t sz_SS = (size_t)WA * 2 * T * 4;
    // CL: each prep wave's angle totals per pair, exchanged once per chunk.
    static constexpr size_t sz_XW = (size_t)NWP * NPR * 4;
    template <bool FULL, bool PM = false> struct Lay {
        // single chunk buffer (the state pass, without Cbar, keeps two)
        static constexpr bool SB = NBUF == 1 && FULL;
        static constexpr size_t oB = 0;
        static constexpr size_t oC = sz_B;
        static constexpr size_t oX = oC + (FULL ? sz_B : 0);
        static constexpr size_t oF = oX + sz_X;
        static constexpr size_t BUF = (oF + nF * 4 + 15) / 16 * 16;
        static constexpr size_t FST = (nF * 4 + 15) / 16 * 16;
        // stride between the two buffers of {Bbar, Cbar, X} and of the scalars
        static constexpr size_t BSTR = SB ? 0 : BUF;
        static constexpr size_t FSTR = SB ? FST : BUF;
        static constexpr size_t oH = SB ? oF + 2 * FST : 2 * BUF;
        static constexpr size_t oPW = oH + (FULL ? (SH1 ? 1 : 2) * sz_H1 : 0);
        static constexpr size_t oSS = oPW + (PM ? sz_PMW : 0);
        static constexpr size_t oXW = oSS + ((PM && !CL) ? sz_SS : 0);
        static constexpr size_t oCNT = oXW + (CL ? sz_XW : 0);
        static constexpr size_t bytes = oCNT + ((PM || CL) ? 16 : 0);
    };
    static constexpr size_t lds_bytes = Lay<true>::bytes;
    static constexpr size_t lds_bytes_state = Lay<false>::bytes;
    static constexpr size_t lds_bytes_pm = Lay<true, true>::bytes;
    static constexpr size_t lds_bytes_state_pm = Lay<false, true>::bytes;
    // Segment record: G (fp32, NP x P) in the math waves' tile order -- tile
    // slot (slice, tau) holds 64 lanes x 4 rows, one 16-byte access per lane
    // -- then Lam_seg*log2(e) (padded to 4 floats), then (cos, sin) of the
    // segment's total angle per pair.
    __host__ __device__ static int64_t rec_floats(int64_t P) { return (int64_t)NP * P + 4 + N; }
    static_assert(T % 32 == 0, "Q*R must be a multiple of 32");
    static_assert(R == 1 || R == 2 || R == 4, "rank must be 1, 2 or 4");
    static_assert(PS % 16 == 0, "headdim slice must be a multiple of 16");
    static_assert(N % 8 == 0 && LQ >= 16 && LQ <= 64, "unsupported dstate");
    static_assert(NPR4 < NWP || NPR4 % NWP == 0, "pair quads must split evenly over prep waves");
    static_assert(PT % PG == 0 && NWM % PG == 0, "headdim tiles must split evenly over math waves");
    static_assert(lds_bytes <= 160 * 1024 && lds_bytes_pm <= 160 * 1024, "LDS budget");
    static_assert(NBUF == 2 || (NBUF == 1 && BF && CL), "one chunk buffer: bf16 row-coalesced prep only");
};

// One prep thread's share of a chunk's raw inputs, loaded a chunk ahead.
template <class Cf> struct PrepStage {
    using io_t = typename Cf::io_t;
    float a_dt[Cf::QPL], a_lm[Cf::QPL], a_dn[Cf::QPL], a_ln[Cf::QPL];  // dt, lam at t, t+1
    float a_A[Cf::QPL];                                                 // decay rate at t
    float dtv[Cf::SL];                                                  // dt of the lane's tokens
    f32x4 thv[Cf::SL];                                                  // theta, 4 pairs
    IoRow8<io_t> bq[Cf::SL][Cf::SRK], cq[Cf::SL][Cf::SRK];              // B, C: 4 pairs
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

// Inclusive prefix sum over aligned groups of LQ lanes (16, 32 or 64).
template <int LQ>
__device__ __forceinline__ float group_inclusive_sum(float v)
{
    v += dpp_moved<0x111, 0xf>(v);   // row_shr:1
    v += dpp_moved<0x112, 0xf>(v);   // row_shr:2
    v += dpp_moved<0x114, 0xf>(v);   // row_shr:4
    v += dpp_moved<0x118, 0xf>(v);   // row_shr:8
    if constexpr (LQ >= 32) v += dpp_moved<0x142, 0xa>(v);   // row_bcast:15 into rows 1, 3
    if constexpr (LQ >= 64) v += dpp_moved<0x143, 0xc>(v);   // row_bcast:31 into rows 2, 3
    return v;
}

// The value of the lane 16 places below (the previous row of 16 lanes; 0 in
// row 0) and 32 places below (0 in rows 0 and 1), by the row-swapping
// permutes of gfx950: permlane16_swap(v, v) gives rows (v0, v0, v2, v2) and
// (v1, v1, v3, v3), permlane32_swap(v, v) gives rows (v0, v1, v0, v1).  Every
// lane of the wave must be active.
__device__ __forceinline__ float lanes_up16(float v, int lane)
{
    const unsigned u = __float_as_uint(v);
    const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const auto q = __builtin_amdgcn_permlane32_swap(p[1], p[1], false, false);
    const int row = lane >> 4;
    return row == 0 ? 0.f : __uint_as_float(row == 2 ? q[0] : p[0]);
}
__device__ __forceinline__ float lanes_up32(float v, int lane)
{
    const unsigned u = __float_as_uint(v);
    const auto q = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return lane < 32 ? 0.f : __uint_as_float(q[0]);
}
// Inclusive prefix sum over lanes l, l - S, l - 2S, ... (M lane groups of S
// lanes: lanes with equal l % S form one sequence, ordered by l / S), as a
// Hillis-Steele scan with lane shifts S, 2S, 4S, ...  With whole rows as the
// groups (S = 16: dstate 128) the shifts run on the row permutes above (long
// prefill 732 -> 712 us); otherwise through LDS (ds_bpermute), which measured
// faster there than the permutes (dstate 64: 36.6 against 37.5 us per call
// with them for the 16- and 32-lane shifts, 36.5 with DPP row shifts and
// rotations for the 8-lane one as well).
template <int S, int M, int D = 1>
__device__ __forceinline__ float strided_inclusive_sum(float v, int lane)
{
    constexpr int SH = D * S;
    if constexpr (D >= M) {
        return v;
    } else {
        if constexpr (S == 16 && SH == 16) {
            v += lanes_up16(v, lane);
        } else if constexpr (S == 16 && SH == 32) {
            v += lanes_up32(v, lane);
        } else {
            const float u = __shfl_up(v, (unsigned)SH, 64);
            v += lane >= SH ? u : 0.f;
        }
        return strided_inclusive_sum<S, M, 2 * D>(v, lane);
    }
}

// Wait until the workgroup-shared counter *cnt reaches target (the other
// waves of the workgroup publish before they wait, so it always does), with
// a bound of 2^22 polls so that a defect can never hang the device.  Returns
// false only if the bound ran out; the caller then poisons its results.
#ifndef M3_WAIT_SLEEP
#define M3_WAIT_SLEEP 1
#endif
__device__ __forceinline__ bool bounded_wait_at_least(int* cnt, int target)
{
    for (int it = 0; it < (1 << 22); ++it) {
        const int v = __builtin_amdgcn_readfirstlane(
            __hip_atomic_load(cnt, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP));
        if (v >= target) return true;
        if constexpr (M3_WAIT_SLEEP > 0) __builtin_amdgcn_s_sleep(M3_WAIT_SLEEP);
    }
    return false;
}

// FULL: outputs y (and the state record when this is the last segment).
// !FULL: state pass -- each segment except the last writes its end state
// (from a zero start, except segment 0 which starts from the true state).
// softplus(z) = log(1 + e^z) (z itself above 20, where the difference is
// below float32 resolution) and sigmoid(z) = 1 / (1 + e^-z): the pre-mixer's
// maps of the raw dt and lam projections.
// Calls f(std::integral_constant<int, v>) for the runtime value v in [I, NV)
// (a scalar branch per candidate when v is wave-uniform).
template <int I, int NV, class F>
__device__ __forceinline__ void static_dispatch(int v, F&& f)
{
    if constexpr (I < NV) {
        if (v == I) f(std::integral_constant<int, I>{});
        else static_dispatch<I + 1, NV>(v, f);
    }
}

// softplus(z) = max(z, 0) + log1p(e), e = e^{-|z|} in (0, 1], on the hardware
// exp2/log2: for e < 2^-10 the series e (1 - e/2 + e^2/3) (truncation below
// 2^-32 relative), otherwise log(u) with u = 1 + e corrected for the rounding
// of u (log1p(e) = log(u) - ((u - 1) - e) / u to first order).
__device__ __forceinline__ float softplus_f(float z)
{
    const float e = __builtin_amdgcn_exp2f(-fabsf(z) * kLog2e);
    const float u = 1.f + e;
    const float lp = e < 0x1p-10f ? e * (1.f - e * (0.5f - e * (1.f / 3.f)))
                                  : __builtin_amdgcn_logf(u) * 0.6931471805599453f - ((u - 1.f) - e) / u;
    return fmaxf(z, 0.f) + lp;
}
__device__ __forceinline__ float sigmoid_f(float z) { return 1.f / (1.f + expf(-z)); }

// PM: pre-mixer on (the raw dt, lam, B and C are normalised in the prep waves).
template <class Cf, bool FULL, bool PM>
__global__ __launch_bounds__(Cf::NT, Cf::OCC * Cf::NW / 4) void scan_kernel(const ScanParams p)
{
    using io_t = typename Cf::io_t;
    using op_t = typename Cf::op_t;
    using Lay = typename Cf::template Lay<FULL, PM>;
    constexpr int N = Cf::N, NP = Cf::NP, NPR = Cf::NPR, PS = Cf::PS, R = Cf::R;
    constexpr int Q = Cf::Q, T = Cf::T, NWM = Cf::NWM, NWP = Cf::NWP, NT = Cf::NT;
    constexpr int LDB = Cf::LDB, LDX = Cf::LDX, LDXR = Cf::LDXR, LDH = Cf::LDH;
    constexpr int QPWV = Cf::QPWV, WA = Cf::WA, LQ = Cf::LQ, TPL = Cf::TPL, QPL = Cf::QPL;
    constexpr int XI = Cf::XI, XITEMS = Cf::XITEMS;
    constexpr int QT = Cf::QT, KB = Cf::KB, NTL = Cf::NTL, NTILES = Cf::NTILES, TPW = Cf::TPW;
    constexpr int PG = Cf::PG, QG = Cf::QG, PPW = Cf::PPW, QPW = Cf::QPW, FB = Cf::FB;
    constexpr bool BF = Cf::BF;
    constexpr int HSTAGE = PS * LDH;   // elements of one state stage

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    // One word of every 64-byte line of the kernel arguments, read at once:
    // the set-up below reads the arguments in dependent steps, and each line
    // it touches first would otherwise cost a round trip of its own.
    {
        const unsigned* kp = reinterpret_cast<const unsigned*>(&p);
        constexpr int NLINE = (int)((sizeof(ScanParams) + 63) / 64);
#pragma unroll
        for (int i = 0; i < NLINE; ++i) {
            const unsigned t = kp[16 * i];
            asm volatile("" ::"s"(t));
        }
    }
    op_t* sH = reinterpret_cast<op_t*>(smem + Lay::oH);   // [1 or 2][PS][LDH] G^T
    constexpr bool SBUF = Lay::SB;
    auto buf_B = [&](int s) { return reinterpret_cast<op_t*>(smem + s * Lay::BSTR + Lay::oB); };
    auto buf_C = [&](int s) { return reinterpret_cast<op_t*>(smem + s * Lay::BSTR + Lay::oC); };
    auto buf_X = [&](int s) { return reinterpret_cast<op_t*>(smem + s * Lay::BSTR + Lay::oX); };
    //   scalars: [Q][2] = (Lam_j * log2(e), w_j), [Q] gamma_j, [Q] w_j e^{Lam_tot-Lam_j},
    //   [NPR][2] cos/sin Phi_tot, [0] = Lam_tot * log2(e)
    auto buf_F = [&](int s) { return reinterpret_cast<float*>(smem + s * Lay::FSTR + Lay::oF); };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // scalar: role branches are uniform
    const int l16 = lane & 15, g = lane >> 4;
    const bool is_math = wv < NWM;   // wave-uniform role

    // Workgroup -> (segment, b, h, headdim slice): the grid's y index is the
    // segment (or packed slot), x the (b, h, slice) (no division by a runtime
    // value: sixteen waves per CU computing the same scalar set-up share the
    // CU's scalar unit ahead of their first loads).  Consecutive linear
    // workgroup ids go to different XCDs (round robin over 8), so the slices
    // and segments of one (b, h) are given ids that are multiples of 8 apart:
    // they share an XCD and its L2.
    const int64_t H = p.H, P = p.P;
    int seg, bh, ps, nseg_u = p.nseg;
    int pk_lo = 0, pk_len = 0;   // per-sequence slots: the sequence's first token and length
    if (p.nslots == 0) {
        seg = blockIdx.y;
        const int bid = blockIdx.x;
        if (p.p_split == 1) {
            bh = bid;
            ps = 0;
        } else {
            bh = (bid >> 3) / p.p_split * 8 + (bid & 7);
            ps = (bid >> 3) % p.p_split;
        }
        if (bh >= p.nbh) return;
    } else {
        // Packed sequences with segments sized per sequence: sequence b has
        // max(1, ceil(chunks_b / seg_chunks)) segments, numbered in sequence
        // order; a slot of heads x slices per (sequence, segment).  Slots
        // past the last sequence's last segment have no work.  The slot is
        // found without a walk: lane i loads sequence b0 + i's offsets and
        // takes its segment count, a prefix sum over the lanes gives each
        // sequence's first slot, and a ballot picks the sequence whose slots
        // hold this one (64 sequences per round; one round trip to memory for
        // up to 64 sequences instead of one per sequence).
        const int slot = blockIdx.y;
        const int bid = blockIdx.x;
        const int hh = (bid >> 3) / p.p_split * 8 + (bid & 7);
        ps = (bid >> 3) % p.p_split;
        if (hh >= H) return;
        int first = 0;
        int64_t bsel = -1;
        for (int64_t b0 = 0; b0 < p.batch; b0 += 64) {
            const int64_t bb = b0 + lane;
            int ns = 0, lo_i = 0, len_i = 0;
            if (bb < p.batch) {
                int64_t lo = p.opt.cu[bb], hi = p.opt.cu[bb + 1];
                lo = lo < 0 ? 0 : (lo > p.L ? p.L : lo);
                hi = hi < lo ? lo : (hi > p.L ? p.L : hi);
                const int64_t len = hi - lo < p.opt.max_len ? hi - lo : p.opt.max_len;
                const int64_t nch = (len + Q - 1) / Q;
                const int64_t n = (nch + p.seg_chunks - 1) / p.seg_chunks;
                ns = n < 1 ? 1 : (int)n;
                lo_i = (int)lo;       // offsets are int32 on input
                len_i = (int)len;
            }
            const int incl = wave_inclusive_sum_i(ns);
            const int start = first + incl - ns;            // this lane's sequence: its first slot
            const unsigned long long hit = __ballot(bb < p.batch && slot >= start && slot < start + ns);
            if (hit != 0) {
                const int l = __builtin_ctzll(hit);
                bsel = b0 + l;
                first = __builtin_amdgcn_readlane(start, l);
                nseg_u = __builtin_amdgcn_readlane(ns, l);
                pk_lo = __builtin_amdgcn_readlane(lo_i, l);
                pk_len = __builtin_amdgcn_readlane(len_i, l);
                break;
            }
            first += __builtin_amdgcn_readlane(incl, 63);
        }
        if (bsel < 0) return;
        seg = (int)(slot - first);
        bh = (int)(bsel * H + hh);
    }
    // a state pass has no work in a sequence's last segment
    if (!FULL && seg == nseg_u - 1) return;
    // 32-bit division: batch x heads < 2^28 (checked on the host); a 64-bit
    // one is a long software sequence ahead of every workgroup's first load
    const int Hi = (int)H;
    const int bi = bh / Hi;
    const int64_t b = bi, h = bh - bi * Hi;
    const int p0 = ps * PS;
    // This unit's sequence: tokens base .. base+L-1 of the token arrays.  A
    // dense batch has L = p.L and base = b * p.L; packed sequences take them
    // from cu_seqlens (clamped into the arrays and to max_seqlen).
    int64_t L = p.L, base = b * p.L;
    if (p.nslots != 0) {
        base = pk_lo;
        L = pk_len;
    } else if (p.opt.cu != nullptr) {
        int64_t lo = p.opt.cu[b], hi = p.opt.cu[b + 1];
        lo = lo < 0 ? 0 : (lo > p.L ? p.L : lo);
        hi = hi < lo ? lo : (hi > p.L ? p.L : hi);
        base = lo;
        L = hi - lo < p.opt.max_len ? hi - lo : p.opt.max_len;
    }

    const int64_t nchunks_all = (L + Q - 1) / Q;
    const int64_t c_begin = (int64_t)seg * p.seg_chunks;
    const int64_t c_end = c_begin + p.seg_chunks < nchunks_all ? c_begin + p.seg_chunks : nchunks_all;
    const bool last_seg = seg == nseg_u - 1;

    const int64_t G = p.opt.groups;                 // B/C head groups
    const int64_t hg = (int)h / (Hi / (int)G);       // this head's group
    const int sDT = (int)H, sTH = (int)(H * NPR), sBN = (int)(G * R * N), sXP = (int)(H * R * P);
    const int64_t tok0 = (base + c_begin * Q) * H + h;
    const int64_t tok0g = (base + c_begin * Q) * G + hg;   // B, C rows
    const int64_t rec_sz = Cf::rec_floats(P);
    float* recs = p.ws + (int64_t)bh * (p.nseg - 1) * rec_sz;   // this (b, h)'s records

    // Padded state columns (N < NP) are constant zeros in both buffers.
    if constexpr (NP > N) {
        for (int idx = tid; idx < 2 * T * (NP - N); idx += NT) {
            const int s = idx / (T * (NP - N)), r2 = idx % (T * (NP - N));
            const int row = r2 / (NP - N), col = N + r2 % (NP - N);
            buf_B(s)[row * LDB + col] = from_f32<op_t>(0.f);
            if constexpr (FULL) buf_C(s)[row * LDB + col] = from_f32<op_t>(0.f);
        }
    }

    // ========================= prep waves ===================================
    const int pw = wv - NWM;
    const int ptid = tid - 64 * NWM;
    const bool arole = !is_math && pw < WA;
    const int qd = (arole ? pw : 0) * QPWV + lane / LQ;   // pair quad: rows 8qd .. 8qd+7
    const int li = lane % LQ;                              // lane within the quad's group
    // CL layout: this lane's pair quad and its first operand row
    constexpr bool CL = Cf::CL;
    constexpr int KP = Cf::KP, MQ = Cf::MQ, RPW = Cf::RPW, NPR4 = Cf::NPR4;
    const int lq = lane % NPR4;
    const int lr0 = pw * RPW + (lane / NPR4) * KP;
    // the lanes that hold a chunk's total angle (pair quad tq)
    const bool tlane = CL ? (pw == NWP - 1 && lane >= (MQ - 1) * NPR4) : (arole && li == LQ - 1);
    const int tq = CL ? lq : qd;

    // Pre-mixer state: gains and biases of this lane's pair quad in LDS
    // (staged and read by the same wave), the prep waves' exchange of row
    // sums of squares, and the exchange counter (zeroed before any wave can
    // add to it).
    float* const sPW = reinterpret_cast<float*>(smem + Lay::oPW);   // [2][N] gains, [2][R][N] biases
    float* const sSS = reinterpret_cast<float*>(smem + Lay::oSS);   // [WA][2][T]
    float* const sXW = reinterpret_cast<float*>(smem + Lay::oXW);   // CL: [NWP][NPR] angle totals
    int* const sCnt = reinterpret_cast<int*>(smem + Lay::oCNT);
    int pcall = 0;                                                 // prep calls of this wave
    unsigned long long* tlw = nullptr;   // this wave's timeline row (instrumented builds)
    int tln = 0;
    if constexpr (M3_TIMELINE) {
        if (p.tl != nullptr) {
            tlw = p.tl + ((size_t)(blockIdx.y * gridDim.x + blockIdx.x) * Cf::NW + wv) * kTlSlots;
            const unsigned long long rt = __builtin_amdgcn_s_memrealtime();
            const unsigned long long t0 = __builtin_amdgcn_s_memtime();
            if (lane == 0) {
                tlw[0] = rt;
                tlw[1] = t0;
                // pass (bit 63: outputs), role (bit 62: matrix-core wave), wave
                // index (bits 48-55), segment (bits 32-47), unit
                tlw[2] = ((unsigned long long)FULL << 63) | ((unsigned long long)is_math << 62) |
                         ((unsigned long long)(unsigned)wv << 48) |
                         ((unsigned long long)((unsigned)seg & 0xffffu) << 32) | (unsigned)bh;
            }
            tln = 3;
        }
    }
    auto stamp = [&](int code) {
        if constexpr (M3_TIMELINE) {
            if (tlw != nullptr && tln < kTlSlots - 2) {
                const unsigned long long t = __builtin_amdgcn_s_memtime();
                if (lane == 0) tlw[tln] = ((unsigned long long)code << 56) | (t & ((1ull << 56) - 1));
                ++tln;
            }
        }
    };
    auto stamp_exit = [&]() {
        if constexpr (M3_TIMELINE) {
            if (tlw != nullptr) {
                const unsigned long long t = __builtin_amdgcn_s_memtime();
                const unsigned long long rt = __builtin_amdgcn_s_memrealtime();
                if (lane == 0) {
                    tlw[kTlSlots - 2] = t;
                    tlw[kTlSlots - 1] = rt;
                    if (tln < kTlSlots - 2) tlw[tln] = (unsigned long long)kTlExit << 56;
                }
            }
        }
    };
    if constexpr (PM && CL) {
        // every gain and bias (a prep lane reads its own pair quad's)
        for (int idx = tid; idx < 2 * (R + 1) * N; idx += NT) {
            const int m = idx / ((R + 1) * N), rem = idx % ((R + 1) * N), k = rem / N, n = rem % N;
            const float* W = m == 0 ? p.opt.Bw : p.opt.Cw;
            const float* Bb = m == 0 ? p.opt.Bb : p.opt.Cb;
            if (k == 0) sPW[m * N + n] = W != nullptr ? W[n] : 1.f;
            else sPW[2 * N + (m * R + k - 1) * N + n] =
                     Bb != nullptr ? Bb[((int64_t)h * R + (k - 1)) * N + n] : 0.f;
        }
    }
    if constexpr (PM || CL) {
        if (!CL && arole) {
            constexpr int PER = 8 * (R + 1);   // gains and R bias rows, 8 entries each
            for (int idx = li; idx < 2 * PER; idx += LQ) {
                const int m = idx / PER, rem = idx % PER, k = rem / 8, n = 8 * qd + rem % 8;
                const float* W = m == 0 ? p.opt.Bw : p.opt.Cw;
                const float* Bb = m == 0 ? p.opt.Bb : p.opt.Cb;
                if (k == 0) sPW[m * N + n] = W != nullptr ? W[n] : 1.f;
                else sPW[2 * N + (m * R + k - 1) * N + n] =
                         Bb != nullptr ? Bb[((int64_t)h * R + (k - 1)) * N + n] : 0.f;
            }
        }
        if (tid == 0) *sCnt = 0;
        __syncthreads();
    }
    stamp(kTlSetup);
    double l2seg = 0.0, phiseg[4] = {0.0, 0.0, 0.0, 0.0};   // segment totals (state pass)
    const int phase = p.opt.phase;
    const float dtb_h = (PM && p.opt.dtb != nullptr) ? p.opt.dtb[h] : 0.f;

    // Load pointers at the next chunk to be loaded; advanced by every issue.
    const float* __restrict__ ldt = p.dt + tok0;
    const float* __restrict__ llam = p.lam + tok0;
    const float* __restrict__ lth = p.theta + (phase != 1 ? tok0 * NPR : 0);
    const io_t* __restrict__ lB = reinterpret_cast<const io_t*>(p.B) + tok0g * R * N;
    const io_t* __restrict__ lC = reinterpret_cast<const io_t*>(p.C) + tok0g * R * N;
    // decay rate: per token (stride dt's) or one per head (stride 0)
    const float* __restrict__ lA = p.A + (p.opt.a_tok ? tok0 : h);
    const int sA = p.opt.a_tok ? sDT : 0;
    const io_t* __restrict__ lX = reinterpret_cast<const io_t*>(p.x) + tok0 * R * P + p0;

    auto xmap = [](int it, int& rho, int& cg) {
        if constexpr (BF) { rho = it / (PS / 8); cg = it % (PS / 8); }   // rows: coalesced
        else { rho = it % T; cg = it / T; }                               // X^T: conflict-free
    };

    // Token indices are clamped to the last valid token (values past it are
    // masked on use).  Every load is unconditional and issued in the order
    // prep consumes it, so the in-order load counter lets each step wait only
    // for its own data.
    // Offsets inside a chunk are 32-bit byte offsets (token index times the
    // per-token byte stride, < 2^24, via the 24-bit multiplier) added to the
    // wave-uniform chunk base: no 64-bit vector address arithmetic.
    const unsigned bDT = 4u * (unsigned)sDT, bTH = 4u * (unsigned)sTH, bA = 4u * (unsigned)sA;
    const unsigned bBN = (unsigned)sizeof(io_t) * (unsigned)sBN, bXP = (unsigned)sizeof(io_t) * (unsigned)sXP;
    const unsigned bcq = (unsigned)sizeof(io_t) * 8u * (unsigned)qd;       // B/C quad
    // Shuffled phases: the four source pairs of this lane's pair quad (fixed
    // for the kernel), read once and packed one byte each (pair indices are
    // below 128), so that no theta load waits on a load of the permutation
    // (prefill_bf16 with shuffled phases 41.1 -> 39.0 us).  The pre-mixer
    // variants read the permutation with each load instead: holding it cost
    // them 2%.
    unsigned shf = 0u;
    if (!PM && p.opt.phase == 3 && !is_math) {
        const int q = CL ? lane % NPR4 : qd;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            int src = p.opt.perm[4 * q + e];
            src = src < 0 ? 0 : (src >= NPR ? NPR - 1 : src);
            shf |= (unsigned)src << (8 * e);
        }
    }
    auto at = [](const auto* base, unsigned off) {
        return reinterpret_cast<decltype(base)>(reinterpret_cast<const char*>(base) + off);
    };
    PrepStage<Cf> st;
    // One chunk buffer: chunk c+1's rotated Bbar, Cbar rows and X rows,
    // held here until the math waves are done with chunk c.
    // (The X rows stay in the raw stage until then: the next chunk's X loads
    // are issued after they are stored.)
    IoRow8<io_t> pend_b[SBUF ? KP : 1], pend_c[SBUF ? KP : 1];
    // Loads of chunk c into the prep stage, by part (LD_A0: per-token dt, lam
    // and decay rate for A0; LD_X: the X slice; LD_TH: dt and theta of the
    // lane's rows; LD_BC: B and C); `advance` then moves the pointers to the
    // next chunk.
    constexpr int LD_A0 = 1, LD_X = 2, LD_TH = 4, LD_BC = 8;
    // State pass, bf16 row-coalesced prep: the matrix-core waves, which have
    // only the state update to do there, load and store the X rows
    // themselves (off the prep waves' critical path).
    constexpr bool MX = !FULL && BF && CL && !SBUF;
    auto issue_part = [&](int64_t c, auto partc) {
        constexpr int part = decltype(partc)::value;
        const int64_t t0 = c * Q;
        const int jl = (int)((L - 1 - t0) < (Q - 1) ? (L - 1 - t0) : (Q - 1));  // last valid j
        const int jn = (int)((L - 1 - t0) < Q ? (L - 1 - t0) : Q);              // last valid j+1
        // per-token dt / lam (at t and t+1) for A0: only the wave that runs A0
        // (each lane reads its own token's cache line)
        if ((part & LD_A0) && pw == 0) {
#pragma unroll
            for (int kk = 0; kk < QPL; ++kk) {
                const int j = lane * QPL + kk;
                const unsigned jc = (unsigned)(j < jl ? j : jl);
                const unsigned jnc = (unsigned)(j + 1 < jn ? j + 1 : jn);
                st.a_dt[kk] = *at(ldt, __umul24(jc, bDT));
                st.a_A[kk] = *at(lA, __umul24(jc, bA));
                st.a_lm[kk] = *at(llam, __umul24(jc, bDT));
                st.a_dn[kk] = *at(ldt, __umul24(jnc, bDT));
                st.a_ln[kk] = *at(llam, __umul24(jnc, bDT));
            }
        }
        if constexpr ((part & LD_X) != 0 && !MX) {
#pragma unroll
            for (int k = 0; k < XI; ++k) {
                int it = ptid + k * 64 * NWP;
                if (XITEMS % (64 * NWP) != 0 && it >= XITEMS) it = XITEMS - 1;   // duplicate
                int rho, cg;
                xmap(it, rho, cg);
                const unsigned j = (unsigned)(rho / R < jl ? rho / R : jl);
                const unsigned lo = (unsigned)sizeof(io_t) * ((unsigned)(rho % R) * (unsigned)P + 8u * (unsigned)cg);
                st.xq[k].load(at(lX, __umul24(j, bXP) + lo));
            }
        }
        // theta (by phase mode) of 4 pairs from quad q of token j
        auto load_theta = [&](unsigned j, int q, f32x4& th) {
            const unsigned tq16 = 16u * (unsigned)q;
            if (phase == 0) {
                th = *reinterpret_cast<const f32x4*>(at(lth, __umul24(j, bTH) + tq16));
            } else if (phase == 1) {        // zero: theta is not read
                th = f32x4{0.f, 0.f, 0.f, 0.f};
            } else if (phase == 2) {        // reverse
                th = -*reinterpret_cast<const f32x4*>(at(lth, __umul24(j, bTH) + tq16));
            } else if constexpr (!PM) {     // shuffle: pair i reads pair perm[i] (of quad q, in shf)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    th[e] = *at(lth, __umul24(j, bTH) + 4u * ((shf >> (8 * e)) & 0xffu));
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    int src = p.opt.perm[4 * q + e];
                    src = src < 0 ? 0 : (src >= NPR ? NPR - 1 : src);
                    th[e] = *at(lth, __umul24(j, bTH) + 4u * (unsigned)src);
                }
            }
        };
        if constexpr (CL) {
            // whole rows per instruction: row lr0 + k of token (lr0 + k) / R
            if constexpr ((part & LD_TH) != 0) {
#pragma unroll
                for (int k = 0; k < KP; ++k) {
                    const int jj = (lr0 + k) / R;
                    const unsigned j = (unsigned)(jj < jl ? jj : jl);
                    st.dtv[k] = *at(ldt, __umul24(j, bDT));
                    load_theta(j, lq, st.thv[k]);
                }
            }
            if constexpr ((part & LD_BC) != 0) {
#pragma unroll
                for (int k = 0; k < KP; ++k) {
                    const int rho = lr0 + k, jj = rho / R;
                    const unsigned j = (unsigned)(jj < jl ? jj : jl);
                    const unsigned off = __umul24(j, bBN)
                                         + (unsigned)sizeof(io_t) * (unsigned)((rho % R) * N + 8 * lq);
                    st.bq[k][0].load(at(lB, off));
                    if constexpr (FULL) st.cq[k][0].load(at(lC, off));
                }
            }
        } else {
            if constexpr ((part & LD_TH) != 0) {
#pragma unroll
                for (int kk = 0; kk < TPL; ++kk) {
                    const unsigned j = (unsigned)(li * TPL + kk < jl ? li * TPL + kk : jl);
                    st.dtv[kk] = *at(ldt, __umul24(j, bDT));
                    load_theta(j, qd, st.thv[kk]);
                }
            }
            if constexpr ((part & LD_BC) != 0) {
#pragma unroll
                for (int kk = 0; kk < TPL; ++kk) {
                    const unsigned j = (unsigned)(li * TPL + kk < jl ? li * TPL + kk : jl);
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const unsigned off = __umul24(j, bBN) + (unsigned)sizeof(io_t) * (unsigned)(r * N) + bcq;
                        st.bq[kk][r].load(at(lB, off));
                        if constexpr (FULL) st.cq[kk][r].load(at(lC, off));
                    }
                }
            }
        }
    };
    auto advance = [&]() {
        ldt += Q * sDT; llam += Q * sDT; lA += Q * sA;
        if (phase != 1) lth += Q * sTH;
        lB += Q * sBN; lC += Q * sBN; lX += Q * sXP;
    };
    using ld_th = std::integral_constant<int, LD_TH>;
    using ld_a0 = std::integral_constant<int, LD_A0>;
    using ld_x = std::integral_constant<int, LD_X>;
    using ld_bc = std::integral_constant<int, LD_BC>;
    // Part-wise early issue inside prep (row-coalesced layout; not with the
    // pre-mixer, whose prep step has no registers to spare for it).
    constexpr bool EARLY = CL && !PM;
    // Every part of chunk c, in the order prep consumes them, then advance.
    auto issue_loads = [&](int64_t c) {
        if constexpr (CL) {
            issue_part(c, ld_th{});
            issue_part(c, ld_a0{});
            issue_part(c, ld_x{});
            issue_part(c, ld_bc{});
        } else {
            issue_part(c, std::integral_constant<int, LD_A0 | LD_X | LD_TH | LD_BC>{});
        }
        advance();
    };

    // Raw inputs of chunk c (in st) -> operands and scalars in buffer s.
    // CL with nx: each part of chunk c+1's loads is issued as soon as this
    // step has consumed the registers it refills (a longer prefetch distance
    // than issuing them all at the end).
    auto prep = [&](int64_t c, int s, bool nx) {
        ++pcall;
        stamp(kTlPrepStart);
        op_t* sB = buf_B(s);
        op_t* sC = buf_C(s);
        op_t* sX = buf_X(s);
        float* sLW = buf_F(s);
        float* sG = sLW + 2 * Q;
        float* sD = sG + Q;
        float* sCSt = sD + Q;
        float* sMisc = sCSt + 2 * NPR;
        float* sU = sMisc + 4;
        const int64_t t0 = c * Q;
        const int jl = (int)((L - 1 - t0) < (Q - 1) ? (L - 1 - t0) : (Q - 1));

        // ---- CL, A1 part 1: angle increments of the lane's rows, their scan
        // within the wave, and the wave's totals published to the other prep
        // waves (before A0 and A2, so that the totals are there when needed).
        f32x4 cl_loc[KP];     // lane: angle at each of its rows, relative to the wave's first row
        if constexpr (CL) {
            f32x4 run = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < KP; ++k) {
                // one increment per token (its rank-0 row); none past the sequence
                const int rho = lr0 + k;
                const bool ok = rho / R <= jl && rho % R == 0;
                const float dv = PM ? softplus_f(st.dtv[k] + dtb_h) : st.dtv[k];
#pragma unroll
                for (int e = 0; e < 4; ++e) run[e] += ok ? dv * st.thv[k][e] : 0.f;
                cl_loc[k] = run;
            }
            if constexpr (M3_TIMELINE) asm volatile("" ::"v"(run[0]));   // (the stamp after the data)
            stamp(kTlAngleIn);
            f32x4 inc;
#pragma unroll
            for (int e = 0; e < 4; ++e) inc[e] = strided_inclusive_sum<NPR4, MQ>(run[e], lane);
            if constexpr (M3_TIMELINE) asm volatile("" ::"v"(inc[0]));
            stamp(kTlAngleScanned);
            const f32x4 ex = inc - run;
#pragma unroll
            for (int k = 0; k < KP; ++k) cl_loc[k] += ex;   // (cl_loc[KP-1] is now inc)
            if (lane >= (MQ - 1) * NPR4) *reinterpret_cast<f32x4*>(sXW + pw * NPR + 4 * lq) = inc;
            if (lane == 0) __hip_atomic_fetch_add(sCnt, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
            // (one chunk buffer: issued after the rotation, so that these
            // registers are free while the rotated rows are held)
            if (nx && !SBUF) issue_part(c + 1, ld_th{});
            stamp(kTlAngleScan);
        }

        // ---- A0: decay prefix scan and trapezoid weights (one wave) -------
        if (pw == 0) {
            float a[QPL], wt[QPL], gm[QPL];
            float run = 0.f;
#pragma unroll
            for (int kk = 0; kk < QPL; ++kk) {
                const int j = lane * QPL + kk;
                const bool ok = j < Q && j <= jl;
                const bool okn = j < Q && t0 + j + 1 < L;
                float d = st.a_dt[kk], lm = st.a_lm[kk], dn = st.a_dn[kk], ln = st.a_ln[kk];
                if constexpr (PM) {
                    d = softplus_f(d + dtb_h);
                    lm = sigmoid_f(lm);
                    dn = softplus_f(dn + dtb_h);
                    ln = sigmoid_f(ln);
                }
                d = ok ? d : 0.f;
                lm = ok ? lm : 0.f;
                dn = okn ? dn : 0.f;
                ln = okn ? ln : 0.f;
                gm[kk] = lm * d;
                wt[kk] = gm[kk] + (1.f - ln) * dn;
                run += d * st.a_A[kk];
                a[kk] = run;
            }
            const float incl = wave_inclusive_sum(run);
            const float excl = incl - run;
            const float l2tot = wave_read_lane(incl, (Q - 1) / QPL) * kLog2e;
            float l2v[QPL];
#pragma unroll
            for (int kk = 0; kk < QPL; ++kk) l2v[kk] = (excl + a[kk]) * kLog2e;
            // l2 at the last token of each token's 16-row key tile
            constexpr int TM = 16 / R - 1;
            const float l2te = __shfl(l2v[QPL - 1], ((lane * QPL) | TM) / QPL, 64);
#pragma unroll
            for (int kk = 0; kk < QPL; ++kk) {
                const int j = lane * QPL + kk;
                if (j < Q) {
                    const float l2 = l2v[kk];
                    *reinterpret_cast<float2*>(sLW + 2 * j) = make_float2(l2, wt[kk]);
                    sG[j] = gm[kk];
                    sD[j] = wt[kk] * fast_exp2(l2tot - l2);
                    sU[j] = wt[kk] * fast_exp2(l2te - l2);
                }
            }
            if (lane == 0) sMisc[0] = l2tot;
            if constexpr (!FULL) l2seg += (double)l2tot;
        }
        if (CL && nx) issue_part(c + 1, ld_a0{});
        stamp(kTlDecayScan);

        // ---- A2: X slice into LDS ------------------------------------------
        if constexpr (MX) {
            // (the matrix-core waves stage X in this pass)
        } else if (BF && jl == Q - 1) {
            // full chunk: the raw bf16 rows go to LDS as loaded
#pragma unroll
            for (int k = 0; k < XI; ++k) {
                int it = ptid + k * 64 * NWP;
                if (XITEMS % (64 * NWP) != 0 && it >= XITEMS) it = XITEMS - 1;
                int rho, cg;
                xmap(it, rho, cg);
                if constexpr (!SBUF) st.xq[k].store_raw(sX + rho * LDXR + 8 * cg);
            }
        } else {
#pragma unroll
        for (int k = 0; k < XI; ++k) {
            int it = ptid + k * 64 * NWP;
            if (XITEMS % (64 * NWP) != 0 && it >= XITEMS) it = XITEMS - 1;   // identical duplicate
            int rho, cg;
            xmap(it, rho, cg);
            const bool ok = rho / R <= jl;
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = ok ? st.xq[k].get(e) : 0.f;
            if constexpr (SBUF) {
                st.xq[k].set8(v);   // masked rows, stored by the flush
            } else if constexpr (BF) {
                lds_store8(sX + rho * LDXR + 8 * cg, v);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) sX[(8 * cg + e) * LDX + rho] = v[e];
            }
        }
        }
        if (CL && nx && !SBUF) issue_part(c + 1, ld_x{});
        stamp(kTlXRows);

        // ---- A1: angle prefix per pair quad, rotate B and C ----------------
        if constexpr (CL) {
            // Wait until every prep wave has published this chunk's totals (a
            // bounded wait: the waves reach it together), then this wave's
            // offset is the sum of the totals of the waves before it.
            const int target = NWP * pcall;
            const bool waited = bounded_wait_at_least(sCnt, target);
            f32x4 off = {0.f, 0.f, 0.f, 0.f};
            for (int w = 0; w < pw; ++w) off += *reinterpret_cast<const f32x4*>(sXW + w * NPR + 4 * lq);
            // A wait that ran out (never observed: every prep wave publishes
            // before it waits) poisons the rotated operands, so y and the
            // state of this unit come out NaN instead of silently wrong.
            if (!waited) off = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""),
                                     __builtin_nanf("")};
            stamp(kTlWaitTotals);
            auto rotate_cl = [&](auto fullc) {
                constexpr bool FULLC = decltype(fullc)::value;
                // Pre-mixer: each row's RMS scale from the NPR4 lanes that hold it.
                float scB[KP], scC[KP];
                if constexpr (PM) {
                    const float rn = 1.f / (float)N;
#pragma unroll
                    for (int k = 0; k < KP; ++k) {
                        float sb = 0.f, sc = 0.f;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float vb = st.bq[k][0].get(e);
                            sb += vb * vb;
                            if constexpr (FULL) {
                                const float vc = st.cq[k][0].get(e);
                                sc += vc * vc;
                            }
                        }
                        sb = lane_group_sum<NPR4>(sb);
                        if constexpr (FULL) sc = lane_group_sum<NPR4>(sc);
                        scB[k] = rsqrtf(sb * rn + p.opt.eps);
                        scC[k] = FULL ? rsqrtf(sc * rn + p.opt.eps) : 0.f;
                    }
                }
                // the 8 entries of row piece q as the mixer uses them
                auto entries = [&](const IoRow8<io_t>& q, float sc, int m, int r, float (&v)[8]) {
                    if constexpr (!PM) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) v[e] = q.get(e);
                    } else {
                        const float* gp = sPW + m * N + 8 * lq;
                        const float* bp = sPW + 2 * N + (m * R + r) * N + 8 * lq;
                        const f32x4 g0 = *reinterpret_cast<const f32x4*>(gp);
                        const f32x4 g1 = *reinterpret_cast<const f32x4*>(gp + 4);
                        const f32x4 b0 = *reinterpret_cast<const f32x4*>(bp);
                        const f32x4 b1 = *reinterpret_cast<const f32x4*>(bp + 4);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            v[e] = q.get(e) * sc * g0[e] + b0[e];
                            v[4 + e] = q.get(4 + e) * sc * g1[e] + b1[e];
                        }
                    }
                };
                // The rows of one token (its R ranks) share its angle: the
                // sine and cosine are taken once per token.  A lane's first
                // row starts a token (RPW and KP are multiples of R, or KP
                // divides R), so token starts are the rows k % R == 0.
                static_assert(RPW % R == 0 && (KP % R == 0 || R % KP == 0), "row groups must align with tokens");
                float cs[4], sn[4];
#pragma unroll
                for (int k = 0; k < KP; ++k) {
                    const int rho = lr0 + k, r = rho % R;
                    const bool ok = FULLC || rho / R <= jl;
                    if (k % R == 0) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) rope_sincos<op_t>(off[e] + cl_loc[k][e], &sn[e], &cs[e]);
                    }
                    // R(Phi)^T applied to each pair
                    float o[8], v[8];
                    entries(st.bq[k][0], PM ? scB[k] : 1.f, 0, r, v);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float b0 = ok ? v[2 * e] : 0.f;
                        const float b1 = ok ? v[2 * e + 1] : 0.f;
                        o[2 * e] = cs[e] * b0 + sn[e] * b1;
                        o[2 * e + 1] = cs[e] * b1 - sn[e] * b0;
                    }
                    if constexpr (SBUF) pend_b[k].set8(o);
                    else lds_store8(sB + rho * LDB + 8 * lq, o);
                    if constexpr (FULL) {
                        entries(st.cq[k][0], PM ? scC[k] : 1.f, 1, r, v);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float c0 = ok ? v[2 * e] : 0.f;
                            const float c1 = ok ? v[2 * e + 1] : 0.f;
                            o[2 * e] = cs[e] * c0 + sn[e] * c1;
                            o[2 * e + 1] = cs[e] * c1 - sn[e] * c0;
                        }
                        if constexpr (SBUF) pend_c[k].set8(o);
                        else lds_store8(sC + rho * LDB + 8 * lq, o);
                    }
                }
            };
            if (jl == Q - 1) rotate_cl(std::true_type{});
            else rotate_cl(std::false_type{});
            if (nx) {
                if constexpr (SBUF) issue_part(c + 1, ld_th{});
                issue_part(c + 1, ld_bc{});
                advance();
            }
            stamp(kTlRotate);
            // The last wave's last lane group holds the chunk's total angle.
            if (pw == NWP - 1) {
                const f32x4 tot = off + cl_loc[KP - 1];
                if constexpr (BF) {
                    float cs[4], sn[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) __sincosf(tot[e], &sn[e], &cs[e]);
                    if (tlane) {
                        *reinterpret_cast<f32x4*>(sCSt + 8 * lq) = f32x4{cs[0], sn[0], cs[1], sn[1]};
                        *reinterpret_cast<f32x4*>(sCSt + 8 * lq + 4) = f32x4{cs[2], sn[2], cs[3], sn[3]};
                    }
                } else if (tlane) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float sn, cs;
                        sincosf(tot[e], &sn, &cs);
                        sCSt[2 * (4 * lq + e)] = cs;
                        sCSt[2 * (4 * lq + e) + 1] = sn;
                    }
                }
                if constexpr (!FULL) {
                    if (tlane) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) phiseg[e] += (double)tot[e];
                    }
                }
            }
        } else if (arole) {
            // FULLC: every token of the chunk is valid (no masking needed)
            auto rotate_all = [&](auto fullc) {
                constexpr bool FULLC = decltype(fullc)::value;
                // Pre-mixer, step 1: this wave's share of every row's sum of
                // squares (its pair quads), summed over the wave's quads and
                // published to the other prep waves.
                float scB[TPL][R], scC[TPL][R];
                if constexpr (PM) {
#pragma unroll
                    for (int kk = 0; kk < TPL; ++kk)
#pragma unroll
                        for (int r = 0; r < R; ++r) {
                            float sb = 0.f, sc = 0.f;
#pragma unroll
                            for (int e = 0; e < 8; ++e) {
                                const float vb = st.bq[kk][r].get(e);
                                sb += vb * vb;
                                if constexpr (FULL) {
                                    const float vc = st.cq[kk][r].get(e);
                                    sc += vc * vc;
                                }
                            }
#pragma unroll
                            for (int off = LQ; off < 64; off <<= 1) {
                                sb += __shfl_xor(sb, off, 64);
                                if constexpr (FULL) sc += __shfl_xor(sc, off, 64);
                            }
                            scB[kk][r] = sb;
                            scC[kk][r] = sc;
                        }
                    if (lane < LQ) {
#pragma unroll
                        for (int kk = 0; kk < TPL; ++kk) {
                            const int j = li * TPL + kk;
                            if (LQ * TPL == Q || j < Q) {
#pragma unroll
                                for (int r = 0; r < R; ++r) {
                                    sSS[(pw * 2 + 0) * T + j * R + r] = scB[kk][r];
                                    if constexpr (FULL) sSS[(pw * 2 + 1) * T + j * R + r] = scC[kk][r];
                                }
                            }
                        }
                    }
                    if (lane == 0) __hip_atomic_fetch_add(sCnt, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
                }
                f32x4 loc[TPL];
                f32x4 run = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < TPL; ++kk) {
                    // lanes past the chunk (LQ * TPL > Q) never contribute
                    const int j = li * TPL + kk;
                    const bool ok = FULLC ? (LQ * TPL == Q || j < Q) : j <= jl;
                    const float dv = PM ? softplus_f(st.dtv[kk] + dtb_h) : st.dtv[kk];
#pragma unroll
                    for (int e = 0; e < 4; ++e) run[e] += ok ? dv * st.thv[kk][e] : 0.f;
                    loc[kk] = run;
                }
                f32x4 inc;
#pragma unroll
                for (int e = 0; e < 4; ++e) inc[e] = group_inclusive_sum<LQ>(run[e]);
                const f32x4 ex = inc - run;
                // Pre-mixer, step 2: wait until every prep wave with pair quads
                // has published this chunk's partial sums (a bounded wait: the
                // waves reach it together), then the rows' RMS scales.
                if constexpr (PM) {
                    const int target = WA * pcall;
                    // a wait that ran out poisons the row scales (NaN outputs)
                    const float rn = bounded_wait_at_least(sCnt, target) ? 1.f / (float)N
                                                                         : __builtin_nanf("");
#pragma unroll
                    for (int kk = 0; kk < TPL; ++kk) {
                        int j = li * TPL + kk;
                        j = j < Q ? j : Q - 1;
#pragma unroll
                        for (int r = 0; r < R; ++r) {
                            float tb = 0.f, tc = 0.f;
#pragma unroll
                            for (int w = 0; w < WA; ++w) {
                                tb += sSS[(w * 2 + 0) * T + j * R + r];
                                if constexpr (FULL) tc += sSS[(w * 2 + 1) * T + j * R + r];
                            }
                            scB[kk][r] = rsqrtf(tb * rn + p.opt.eps);
                            scC[kk][r] = FULL ? rsqrtf(tc * rn + p.opt.eps) : 0.f;
                        }
                    }
                }
                // The 8 entries of a B (m = 0) or C (m = 1) row piece as the
                // mixer uses them: raw, or scaled, gained and biased (gains
                // and biases read from LDS where they are used).
                auto entries = [&](const IoRow8<io_t>& q, float sc, int m, int r, float (&v)[8]) {
                    if constexpr (!PM) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) v[e] = q.get(e);
                    } else {
                        const float* gp = sPW + m * N + 8 * qd;
                        const float* bp = sPW + 2 * N + (m * R + r) * N + 8 * qd;
                        const f32x4 g0 = *reinterpret_cast<const f32x4*>(gp);
                        const f32x4 g1 = *reinterpret_cast<const f32x4*>(gp + 4);
                        const f32x4 b0 = *reinterpret_cast<const f32x4*>(bp);
                        const f32x4 b1 = *reinterpret_cast<const f32x4*>(bp + 4);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            v[e] = q.get(e) * sc * g0[e] + b0[e];
                            v[4 + e] = q.get(4 + e) * sc * g1[e] + b1[e];
                        }
                    }
                };
#pragma unroll
                for (int kk = 0; kk < TPL; ++kk) {
                    const int j = li * TPL + kk;
                    const bool ok = FULLC || j <= jl;
                    if (LQ * TPL == Q || j < Q) {
                        float cs[4], sn[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) rope_sincos<op_t>(ex[e] + loc[kk][e], &sn[e], &cs[e]);
#pragma unroll
                        for (int r = 0; r < R; ++r) {
                            const int rho = j * R + r;
                            // R(Phi)^T applied to each pair
                            float o[8], v[8];
                            entries(st.bq[kk][r], PM ? scB[kk][r] : 1.f, 0, r, v);
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const float b0 = ok ? v[2 * e] : 0.f;
                                const float b1 = ok ? v[2 * e + 1] : 0.f;
                                o[2 * e] = cs[e] * b0 + sn[e] * b1;
                                o[2 * e + 1] = cs[e] * b1 - sn[e] * b0;
                            }
                            lds_store8(sB + rho * LDB + 8 * qd, o);
                            if constexpr (FULL) {
                                entries(st.cq[kk][r], PM ? scC[kk][r] : 1.f, 1, r, v);
#pragma unroll
                                for (int e = 0; e < 4; ++e) {
                                    const float c0 = ok ? v[2 * e] : 0.f;
                                    const float c1 = ok ? v[2 * e + 1] : 0.f;
                                    o[2 * e] = cs[e] * c0 + sn[e] * c1;
                                    o[2 * e + 1] = cs[e] * c1 - sn[e] * c0;
                                }
                                lds_store8(sC + rho * LDB + 8 * qd, o);
                            }
                        }
                    }
                }
                // The group's last lane holds the chunk's total angle per pair.
                if constexpr (BF) {
                    // hardware sine/cosine in every lane (no divergent branch)
                    float cs[4], sn[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) __sincosf(inc[e], &sn[e], &cs[e]);
                    if (li == LQ - 1) {
                        *reinterpret_cast<f32x4*>(sCSt + 8 * qd) = f32x4{cs[0], sn[0], cs[1], sn[1]};
                        *reinterpret_cast<f32x4*>(sCSt + 8 * qd + 4) = f32x4{cs[2], sn[2], cs[3], sn[3]};
                    }
                } else if (li == LQ - 1) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float sn, cs;
                        sincosf(inc[e], &sn, &cs);
                        sCSt[2 * (4 * qd + e)] = cs;
                        sCSt[2 * (4 * qd + e) + 1] = sn;
                    }
                }
                if constexpr (!FULL) {
                    if (li == LQ - 1) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) phiseg[e] += (double)inc[e];
                    }
                }
            };
            if (jl == Q - 1) rotate_all(std::true_type{});
            else rotate_all(std::false_type{});
        }
    };

    // One chunk buffer: the held operands of prepared chunk c into LDS, then
    // (cn: chunk c+1 exists) chunk c+1's X loads into the raw stage.  The
    // other parts of chunk c+1 were issued during its prep step, after which
    // the load pointers moved on; X is addressed one chunk back.
    auto flush = [&](int64_t c, bool cn) {
        if constexpr (SBUF) {
            op_t* sB = buf_B(0);
            op_t* sC = buf_C(0);
            op_t* sX = buf_X(0);
#pragma unroll
            for (int k = 0; k < KP; ++k) {
                const int rho = lr0 + k;
                pend_b[k].store_raw(sB + rho * LDB + 8 * lq);
                pend_c[k].store_raw(sC + rho * LDB + 8 * lq);
            }
#pragma unroll
            for (int k = 0; k < XI; ++k) {
                int it = ptid + k * 64 * NWP;
                if (XITEMS % (64 * NWP) != 0 && it >= XITEMS) it = XITEMS - 1;
                int rho, cg;
                xmap(it, rho, cg);
                st.xq[k].store_raw(sX + rho * LDXR + 8 * cg);
            }
            if (cn) {
                if constexpr (EARLY) {
                    lX -= Q * sXP;
                    issue_part(c + 1, ld_x{});
                    lX += Q * sXP;
                } else {
                    issue_loads(c + 1);
                }
            }
        }
    };

    // State pass (MX): the X rows of chunk c, loaded by the matrix-core waves
    // into registers a chunk ahead and stored into a chunk buffer (rows past
    // the sequence zeroed), with the same item map as the prep waves' A2.
    constexpr int XIM = (XITEMS + 64 * NWM - 1) / (64 * NWM);
    IoRow8<io_t> xm[MX ? XIM : 1];
    const io_t* __restrict__ const lX0 = lX;
    auto x_issue = [&](int64_t c) {
        if constexpr (MX) {
            const int64_t t0 = c * Q;
            const int jl = (int)((L - 1 - t0) < (Q - 1) ? (L - 1 - t0) : (Q - 1));
            const io_t* xb = lX0 + (c - c_begin) * Q * sXP;
#pragma unroll
            for (int k = 0; k < XIM; ++k) {
                int it = tid + k * 64 * NWM;
                if (XITEMS % (64 * NWM) != 0 && it >= XITEMS) it = XITEMS - 1;   // identical duplicate
                int rho, cg;
                xmap(it, rho, cg);
                const unsigned j = (unsigned)(rho / R < jl ? rho / R : jl);
                const unsigned lo = (unsigned)sizeof(io_t) * ((unsigned)(rho % R) * (unsigned)P + 8u * (unsigned)cg);
                xm[k].load(at(xb, __umul24(j, bXP) + lo));
            }
        }
    };
    auto x_store = [&](int64_t c, int s) {
        if constexpr (MX) {
            const int64_t t0 = c * Q;
            const int jl = (int)((L - 1 - t0) < (Q - 1) ? (L - 1 - t0) : (Q - 1));
            op_t* sX = buf_X(s);
#pragma unroll
            for (int k = 0; k < XIM; ++k) {
                int it = tid + k * 64 * NWM;
                if (XITEMS % (64 * NWM) != 0 && it >= XITEMS) it = XITEMS - 1;
                int rho, cg;
                xmap(it, rho, cg);
                if (jl == Q - 1) {
                    xm[k].store_raw(sX + rho * LDXR + 8 * cg);
                } else {
                    const bool ok = rho / R <= jl;
                    float v[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] = ok ? xm[k].get(e) : 0.f;
                    lds_store8(sX + rho * LDXR + 8 * cg, v);
                }
            }
        }
    };

    // ========================= math waves ===================================
    // Math wave wv owns state tiles tau = wv*TPW + k, p-tile major
    // (pt = tau / NTL, nt = tau % NTL): rows 16*nt + 4*g + i, column
    // p0 + 16*pt + l16 of the N x P state.
    f32x4 hacc[TPW];
    io_t* __restrict__ Y0 = reinterpret_cast<io_t*>(p.y) + tok0 * R * P + p0;

    // Float offset of this lane's 4 rows of tile k in a segment record.
    auto rec_slot = [&](int k) -> int64_t {
        int tau = wv * TPW + k;
        if (tau >= NTILES) tau = NTILES - 1;
        return ((int64_t)(ps * NTILES + tau) * 64 + lane) * 4;
    };
    auto tile_of = [&](int k, int& pt, int& nt) {
        int tau = wv * TPW + k;
        if (tau >= NTILES) tau = NTILES - 1;
        pt = tau / NTL;
        nt = tau % NTL;
    };

    auto initial_state = [&]() {
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
                    int pt, nt;
                    tile_of(k, pt, nt);
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
                if (L > 0) {
                    float d0 = p.dt[base * H + h], l0 = p.lam[base * H + h];
                    if constexpr (PM) {
                        d0 = softplus_f(d0 + (p.opt.dtb != nullptr ? p.opt.dtb[h] : 0.f));
                        l0 = sigmoid_f(l0);
                    }
                    bhat1 = (1.f - l0) * d0;
                }
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
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float u = 0.f;
#pragma unroll
                    for (int r = 0; r < R; ++r) u += bv[k][i][r] * xv[k][r];
                    hacc[k][i] = hv[k][i] + bhat1 * u;
                }
            }
        } else if constexpr (FULL) {
            // The state entering segment seg: fold of records 0..seg-1 under
            // the chunk-summary operator, G <- R(Phi_s)(2^{l2_s} G) + G_s.
            // FB records per round trip; this overlaps the prep waves' wait
            // for the first chunk's inputs.
#pragma unroll 1
            for (int s0 = 0; s0 < seg; s0 += FB) {
                float gv[FB][TPW][4], cz[FB][TPW][4], l2v[FB];
#pragma unroll
                for (int f = 0; f < FB; ++f) {
                    const float* rec = recs + (int64_t)(s0 + f < seg ? s0 + f : seg - 1) * rec_sz;
                    l2v[f] = rec[(int64_t)NP * P];
#pragma unroll
                    for (int k = 0; k < TPW; ++k) {
                        int pt, nt;
                        tile_of(k, pt, nt);
                        const f32x4 g4 = *reinterpret_cast<const f32x4*>(rec + rec_slot(k));
#pragma unroll
                        for (int i = 0; i < 4; ++i) gv[f][k][i] = g4[i];
                        // (cos, sin) of pairs n0/2 and n0/2 + 1
                        const int n0 = 16 * nt + 4 * g < N ? 16 * nt + 4 * g : N - 4;
                        const f32x4 c4 = *reinterpret_cast<const f32x4*>(rec + (int64_t)NP * P + 4 + n0);
#pragma unroll
                        for (int i = 0; i < 4; ++i) cz[f][k][i] = c4[i];
                    }
                }
#pragma unroll
                for (int f = 0; f < FB; ++f) {
                    const int s = s0 + f;
                    if (s == 0) {
#pragma unroll
                        for (int k = 0; k < TPW; ++k)
#pragma unroll
                            for (int i = 0; i < 4; ++i) hacc[k][i] = gv[f][k][i];
                    } else if (s < seg) {
                        const float sc = fast_exp2(l2v[f]);
#pragma unroll
                        for (int k = 0; k < TPW; ++k) {
#pragma unroll
                            for (int ip = 0; ip < 2; ++ip) {
                                const float cs = cz[f][k][2 * ip], sn = cz[f][k][2 * ip + 1];
                                const float a0 = sc * hacc[k][2 * ip], a1 = sc * hacc[k][2 * ip + 1];
                                hacc[k][2 * ip] = cs * a0 - sn * a1 + gv[f][k][2 * ip];
                                hacc[k][2 * ip + 1] = sn * a0 + cs * a1 + gv[f][k][2 * ip + 1];
                            }
                        }
                    }
                }
            }
        } else {
#pragma unroll
            for (int k = 0; k < TPW; ++k) hacc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        // Padded rows and duplicate tiles are zero.
#pragma unroll
        for (int k = 0; k < TPW; ++k) {
            const int tau = wv * TPW + k;
            const int nt = tau % NTL;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (!(tau < NTILES && 16 * nt + 4 * g + i < N)) hacc[k][i] = 0.f;
        }
    };

    // Stage G^T (operand type) into state stage `hs`.
    auto stage_state = [&](int hs) {
        op_t* base = sH + hs * HSTAGE;
#pragma unroll
        for (int k = 0; k < TPW; ++k) {
            const int tau = wv * TPW + k;
            if (tau < NTILES) {
                const int pt = tau / NTL, nt = tau % NTL;
                const f32x4 v = hacc[k];
                lds_store4(base + (16 * pt + l16) * LDH + 16 * nt + 4 * g, v[0], v[1], v[2], v[3]);
            }
        }
    };

    // ---- C: outputs of chunk c from buffer s, state stage sHc -------------
    auto phase_C = [&](int64_t c, int s, const op_t* sHc) {
        const op_t* sB = buf_B(s);
        const op_t* sC = buf_C(s);
        const op_t* sX = buf_X(s);
        const float* sLW = buf_F(s);
        const float* sG = sLW + 2 * Q;
        const float* sU = sLW + 4 * Q + 2 * NPR + 4;
        const int64_t t0 = c * Q;
        const int jl = (int)((L - 1 - t0) < (Q - 1) ? (L - 1 - t0) : (Q - 1));
        io_t* __restrict__ Yc = Y0 + (c - c_begin) * Q * (int64_t)sXP;
        const int pg = wv % PG;
        // A operands G^T of this wave's headdim tiles, shared by its query tiles
        Frag<op_t> gfr[PPW][NP / 32];
#pragma unroll
        for (int k = 0; k < PPW; ++k)
#pragma unroll
            for (int s2 = 0; s2 < NP / 32; ++s2)
                lds_frag8(gfr[k][s2], sHc + (16 * (pg * PPW + k) + l16) * LDH + 32 * s2 + 8 * g);
        // The wave's query group as a compile-time constant (one copy of the
        // body per group): its query tiles and their key ranges are then
        // known, and the tile loops unroll with constant bounds.
        static_dispatch<0, QG>(wv / PG, [&](auto qgc) {
        constexpr int qg = decltype(qgc)::value;
        // (up to two query tiles per wave the loop unrolls, so the tiles'
        // key ranges are compile-time constants; more are walked in a loop,
        // which keeps the register footprint of one tile)
#pragma unroll (QPW <= 2 ? QPW : 1)
        for (int qi = 0; qi < QPW; ++qi) {
            // query tiles of this wave; with several query groups, alternate
            // direction so that long and short key ranges pair up
            const int qt = QG == 1 ? qi : ((qi & 1) ? qi * QG + (QG - 1 - qg) : qi * QG + qg);
            if (qt < QT) {
                const int rq = 16 * qt + l16;
                const int jq = rq / R;
                const float2 lwq = *reinterpret_cast<const float2*>(sLW + 2 * jq);
                const float l2q = lwq.x;
                const float gq = sG[jq];

                Frag<op_t> cf[NP / 32];
#pragma unroll
                for (int s2 = 0; s2 < NP / 32; ++s2) lds_frag8(cf[s2], sC + rq * LDB + 32 * s2 + 8 * g);

                f32x4 yacc[PPW];
                const float sq = fast_exp2(l2q);
#pragma unroll
                for (int k = 0; k < PPW; ++k) {
                    yacc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s2 = 0; s2 < NP / 32; ++s2) mma(gfr[k][s2], cf[s2], yacc[k]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) yacc[k][i] *= sq;
                }

#pragma unroll
                for (int kp = 0; kp < QT; kp += 2) {
                    if (kp <= qt) {
                        Frag<op_t> pf;
                        const bool second = kp + 1 <= qt;
#pragma unroll
                        for (int half = 0; half < 2; ++half) {
                            const int kt = kp + half;
                            if (kt < qt) {
                                // Key tile wholly before the query token: the mask
                                // factors as u_k * 2^{l2_q - l2_te} (te = the tile's
                                // last token, both factors <= 1).
                                const int jk0 = (16 * kt + 4 * g) / R;
                                float uk[4 / R];
                                if constexpr (R == 1) {
                                    const f32x4 u4 = *reinterpret_cast<const f32x4*>(sU + jk0);
#pragma unroll
                                    for (int e = 0; e < 4; ++e) uk[e] = u4[e];
                                } else if constexpr (R == 2) {
                                    const float2 u2 = *reinterpret_cast<const float2*>(sU + jk0);
                                    uk[0] = u2.x; uk[1] = u2.y;
                                } else {
                                    uk[0] = sU[jk0];
                                }
                                const float l2te = sLW[2 * ((16 * kt + 15) / R)];
                                f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                                for (int s2 = 0; s2 < NP / 32; ++s2) {
                                    Frag<op_t> a;
                                    lds_frag8(a, sB + (16 * kt + l16) * LDB + 32 * s2 + 8 * g);
                                    mma(a, cf[s2], sacc);
                                }
                                const float vq = fast_exp2(l2q - l2te);
#pragma unroll
                                for (int i = 0; i < 4; ++i) pf.set(4 * half + i, sacc[i] * (uk[i / R] * vq));
                            } else if (kt == qt) {
                                // diagonal tile: exact two-band mask per element
                                // ((Lam_k log2 e, w_k) of this lane's 4 / R distinct keys,
                                // loaded before the products that they scale)
                                const int jk0 = (16 * kt + 4 * g) / R;
                                float kl[8];
                                if constexpr (R == 1) {
                                    const f32x4 u0 = *reinterpret_cast<const f32x4*>(sLW + 2 * jk0);
                                    const f32x4 u1 = *reinterpret_cast<const f32x4*>(sLW + 2 * jk0 + 4);
#pragma unroll
                                    for (int e = 0; e < 4; ++e) { kl[e] = u0[e]; kl[4 + e] = u1[e]; }
                                } else if constexpr (R == 2) {
                                    const f32x4 u0 = *reinterpret_cast<const f32x4*>(sLW + 2 * jk0);
#pragma unroll
                                    for (int e = 0; e < 4; ++e) kl[e] = u0[e];
                                } else {
                                    const float2 u0 = *reinterpret_cast<const float2*>(sLW + 2 * jk0);
                                    kl[0] = u0.x; kl[1] = u0.y;
                                }
                                f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                                for (int s2 = 0; s2 < NP / 32; ++s2) {
                                    Frag<op_t> a;
                                    lds_frag8(a, sB + (16 * kt + l16) * LDB + 32 * s2 + 8 * g);
                                    mma(a, cf[s2], sacc);
                                }
                                // two-band decay mask, branch-free: w_k 2^{l2_q - l2_k}
                                // below the diagonal, gamma_q on it, 0 above
#pragma unroll
                                for (int i = 0; i < 4; ++i) {
                                    const int jk = jk0 + i / R;
                                    const float l2k = kl[2 * (i / R)], wk = kl[2 * (i / R) + 1];
                                    const float dec = wk * fast_exp2(fminf(l2q - l2k, 0.f));
                                    const float m = jk < jq ? dec : (jk == jq ? gq : 0.f);
                                    pf.set(4 * half + i, sacc[i] * m);
                                }
                            } else {
#pragma unroll
                                for (int i = 0; i < 4; ++i) pf.set(4 * half + i, 0.f);
                            }
                        }
#pragma unroll
                        for (int k = 0; k < PPW; ++k) {
                            const int pt = pg * PPW + k;
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
                            mma(xa, pf, yacc[k]);
                        }
                    }
                }

                if (jq <= jl) {
                    io_t* yrow = Yc + jq * sXP + (rq % R) * (int)P;
#pragma unroll
                    for (int k = 0; k < PPW; ++k) gstore4(yrow + 16 * (pg * PPW + k) + 4 * g, yacc[k]);
                }
            }
        }
        });
    };

    // ---- D: state update  G <- R(Phi_tot)(e^{Lam_tot} G + Bbar_d^T X) ------
    // A operand Bbar^T (rows n = 16*nt + l16, K-slots keys 32*kb + 8*g + e)
    // and B operand X_d[keys][p] = d_key X[key][p] (column p = 16*pt + l16).
    auto load_bt = [&](const op_t* sB, int nt, int kb, Frag<op_t>& f) {
        if constexpr (BF) {
            const bf16* br = sB + (32 * kb + 8 * g + (l16 >> 2)) * LDB + 16 * nt + 4 * (l16 & 3);
            const bf16x4 lo = lds_read_tr4(br);
            const bf16x4 hi = lds_read_tr4(br + 4 * LDB);
#pragma unroll
            for (int e = 0; e < 4; ++e) { f.v[e] = lo[e]; f.v[4 + e] = hi[e]; }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) f.set(e, sB[(32 * kb + 8 * g + e) * LDB + 16 * nt + l16]);
        }
    };
    auto load_xd = [&](const op_t* sX, const float* sD, int pt, int kb, Frag<op_t>& f) {
        float xv[8];
        if constexpr (BF) {
            const bf16* xr = sX + (32 * kb + 8 * g + (l16 >> 2)) * LDXR + 16 * pt + 4 * (l16 & 3);
            const bf16x4 lo = lds_read_tr4(xr);
            const bf16x4 hi = lds_read_tr4(xr + 4 * LDXR);
#pragma unroll
            for (int e = 0; e < 4; ++e) { xv[e] = (float)lo[e]; xv[4 + e] = (float)hi[e]; }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) xv[e] = sX[(16 * pt + l16) * LDX + 32 * kb + 8 * g + e];
        }
        // d of the 8 / R tokens behind the 8 K-slots (naturally aligned loads)
        float dv[8 / R];
        if constexpr (R == 1) {
            const f32x4 d0 = *reinterpret_cast<const f32x4*>(sD + 32 * kb + 8 * g);
            const f32x4 d1 = *reinterpret_cast<const f32x4*>(sD + 32 * kb + 8 * g + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) { dv[e] = d0[e]; dv[4 + e] = d1[e]; }
        } else if constexpr (R == 2) {
            const f32x4 d0 = *reinterpret_cast<const f32x4*>(sD + 16 * kb + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e) dv[e] = d0[e];
        } else {
            const float2 d0 = *reinterpret_cast<const float2*>(sD + 8 * kb + 2 * g);
            dv[0] = d0.x;
            dv[1] = d0.y;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) f.set(e, xv[e] * dv[e / R]);
    };
    auto update_tile = [&](f32x4& hk, int nt, const Frag<op_t>* bfr, const Frag<op_t>* xfr,
                           float aT, const float* sCSt) {
        f32x4 acc = hk;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] *= aT;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) mma(bfr[kb], xfr[kb], acc);
        const f32x4 csn = *reinterpret_cast<const f32x4*>(sCSt + 16 * nt + 4 * g);
#pragma unroll
        for (int ip = 0; ip < 2; ++ip) {
            if (16 * nt + 4 * g + 2 * ip < N) {
                const float cs = csn[2 * ip], sn = csn[2 * ip + 1];
                const float a0 = acc[2 * ip], a1 = acc[2 * ip + 1];
                acc[2 * ip] = cs * a0 - sn * a1;
                acc[2 * ip + 1] = sn * a0 + cs * a1;
            }
        }
        hk = acc;
    };
    auto phase_D = [&](int s) {
        const op_t* sB = buf_B(s);
        const op_t* sX = buf_X(s);
        const float* sD = buf_F(s) + 3 * Q;
        const float* sCSt = sD + Q;
        const float aT = fast_exp2(sCSt[2 * NPR]);
        if constexpr (TPW % NTL == 0 && NTILES % NWM == 0 && KB <= 2) {
            // A wave owns whole columns of tiles: every Bbar^T operand is
            // loaded once, up front, and reused for each of its p tiles.
            constexpr int PPD = TPW / NTL;
            Frag<op_t> bfr[NTL][KB];
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt)
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) load_bt(sB, nt, kb, bfr[nt][kb]);
#pragma unroll
            for (int pp = 0; pp < PPD; ++pp) {
                const int pt = wv * PPD + pp;
                Frag<op_t> xfr[KB];
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) load_xd(sX, sD, pt, kb, xfr[kb]);
#pragma unroll
                for (int nt = 0; nt < NTL; ++nt) update_tile(hacc[pp * NTL + nt], nt, bfr[nt], xfr, aT, sCSt);
            }
        } else {
            // Generic layout: operands rebuilt only when their tile index changes.
            Frag<op_t> bfr[KB], xfr[KB];
            int cur_nt = -1, cur_pt = -1;
#pragma unroll
            for (int k = 0; k < TPW; ++k) {
                const int tau = wv * TPW + k;
                if (tau < NTILES) {
                    const int pt = tau / NTL, nt = tau % NTL;
                    if (nt != cur_nt) {
#pragma unroll
                        for (int kb = 0; kb < KB; ++kb) load_bt(sB, nt, kb, bfr[kb]);
                        cur_nt = nt;
                    }
                    if (pt != cur_pt) {
#pragma unroll
                        for (int kb = 0; kb < KB; ++kb) load_xd(sX, sD, pt, kb, xfr[kb]);
                        cur_pt = pt;
                    }
                    update_tile(hacc[k], nt, bfr, xfr, aT, sCSt);
                }
            }
        }
    };

    // Two workgroups per CU: the instruction arbiter favours the older
    // workgroup's waves, so the younger one (dispatched in the second round)
    // finishes 15-18% later and sets the pass's time (a per-wave timeline of
    // prefill_bf16).  In the output pass its waves take a raised priority
    // (prefill_bf16 37.8 -> 36.9 us; in the state pass it did not help).
    const bool young_wg = FULL && Cf::OCC == 2 && (int)(blockIdx.y * gridDim.x + blockIdx.x) >= p.young_from;

    // ========================= schedule =====================================
    // Each role runs its own loop with the same number of barriers: one after
    // the prologue and one per chunk.  (The role test is a scalar branch, so a
    // wave only ever executes its own loop.)
    // A workgroup in its prologue (first chunk's inputs, state fold) issues
    // ahead of other workgroups' steady-state loops on the same CU, so that
    // workgroups that start together also reach their loops together.
    __builtin_amdgcn_s_setprio(1);
    if (!is_math) {
        // prologue: chunk c_begin into buffer 0, chunk c_begin+1's loads out
        if (c_begin < c_end) {
            if constexpr (CL) {
                // Every workgroup starts at once, so the first chunk's loads
                // arrive as one burst across the chip.  The angle and decay
                // inputs go first and alone (a fifth of the bytes); the rows
                // of X, B and C are issued once they have arrived, so that the
                // angle prefix and A0 run while the larger burst is in flight.
                issue_part(c_begin, ld_th{});
                issue_part(c_begin, ld_a0{});
                stamp(kTlFirstIssue);
                __builtin_amdgcn_s_waitcnt(0);
                stamp(kTlFirstArrived);
                issue_part(c_begin, ld_x{});
                issue_part(c_begin, ld_bc{});
                advance();
            } else {
                issue_loads(c_begin);
            }
            prep(c_begin, 0, EARLY && c_begin + 1 < c_end);
            if (!EARLY && !SBUF && c_begin + 1 < c_end) issue_loads(c_begin + 1);
            flush(c_begin, c_begin + 1 < c_end);
            stamp(kTlProloguePrep);
        }
        __syncthreads();
        stamp(kTlPrologueBarrier);
        // With 8 prep waves and one matrix-core wave per SIMD, the youngest
        // prep waves lose instruction issue to the older waves of the
        // workgroup and become the critical path (a per-wave timeline of the
        // long prefill: their rotation and load issue run 30-50% longer and
        // they reach the chunk barrier last); a raised priority for them
        // balances the prep side: long prefill 754 -> 730 us.  (At rank 4 the
        // matrix-core waves are as loaded and it costs 1%; with the pre-mixer
        // at dstate 64, 3%.)
        __builtin_amdgcn_s_setprio(0);
        if (Cf::YOUNG_PRIO && pw >= NWP / 2) __builtin_amdgcn_s_setprio(1);
        if (young_wg) __builtin_amdgcn_s_setprio(1);
        for (int64_t c = c_begin; c < c_end; ++c) {
            const int s = (int)((c - c_begin) & 1);
            if (c + 1 < c_end) {
                prep(c + 1, s ^ 1, EARLY && c + 2 < c_end);
                if (!EARLY && !SBUF && c + 2 < c_end) issue_loads(c + 2);
            }
            if constexpr (SBUF) {
                // one chunk buffer: store chunk c+1's operands once the math
                // waves are done reading chunk c's
                __syncthreads();
                if (c + 1 < c_end) flush(c + 1, c + 2 < c_end);
            }
            __syncthreads();
            stamp(kTlBarrier);
        }
        stamp_exit();
        if constexpr (!FULL) {
            // decay and angle totals of this segment
            float* rec = recs + (int64_t)seg * rec_sz;
            if (ps == 0) {
                if (pw == 0 && lane == 0) rec[(int64_t)NP * P] = (float)l2seg;
                if (tlane) {
                    const double twopi = 6.283185307179586;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float phi = (float)(phiseg[e] - twopi * floor(phiseg[e] / twopi));
                        float sn, cs;
                        sincosf(phi, &sn, &cs);
                        rec[(int64_t)NP * P + 4 + 2 * (4 * tq + e)] = cs;
                        rec[(int64_t)NP * P + 5 + 2 * (4 * tq + e)] = sn;
                    }
                }
            }
        }
    } else {
        int hs = 0;
        if (MX && c_begin < c_end) x_issue(c_begin);
        initial_state();
        if (MX && c_begin < c_end) {
            x_store(c_begin, 0);
            if (c_begin + 1 < c_end) x_issue(c_begin + 1);
        }
        stamp(kTlFold);
        if constexpr (FULL) stage_state(0);
        stamp(kTlStage0);
        __syncthreads();
        stamp(kTlPrologueBarrier);
        __builtin_amdgcn_s_setprio(0);
        if (young_wg) __builtin_amdgcn_s_setprio(1);
        for (int64_t c = c_begin; c < c_end; ++c) {
            const int s = (int)((c - c_begin) & 1);
            if constexpr (FULL) {
                phase_C(c, s, sH + hs * HSTAGE);
                stamp(kTlPhaseC);
                phase_D(s);
                stamp(kTlPhaseD);
                if constexpr (SBUF) __syncthreads();   // the operands may now be overwritten
                if constexpr (!Cf::SH1) hs ^= 1;
                stage_state(hs);
                stamp(kTlStage);
            } else {
                phase_D(s);
                stamp(kTlPhaseD);
                if (MX && c + 1 < c_end) {
                    // chunk c+1's X rows into the other buffer (last read by
                    // phase D of chunk c-1, before the previous barrier)
                    x_store(c + 1, s ^ 1);
                    if (c + 2 < c_end) x_issue(c + 2);
                }
            }
            __syncthreads();
            stamp(kTlBarrier);
        }
        stamp_exit();
        if constexpr (!FULL) {
            // end state of this segment
            float* rec = recs + (int64_t)seg * rec_sz;
#pragma unroll
            for (int k = 0; k < TPW; ++k)
                if (wv * TPW + k < NTILES) *reinterpret_cast<f32x4*>(rec + rec_slot(k)) = hacc[k];
        } else if (last_seg && p.h_out != nullptr) {
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
        }
    }
    if constexpr (!FULL) return;

    // ---- state record copies (last segment) --------------------------------
    if (last_seg && p.h_out != nullptr) {
        if (ps == 0) {
            const io_t* Bm = reinterpret_cast<const io_t*>(p.B);
            const io_t* X = reinterpret_cast<const io_t*>(p.x);
            io_t* Bo = reinterpret_cast<io_t*>(p.Bp_out) + (int64_t)bh * R * N;
            io_t* xo = reinterpret_cast<io_t*>(p.xp_out) + (int64_t)bh * R * P;
            const io_t* Bi = reinterpret_cast<const io_t*>(p.Bp_in);
            const io_t* xi = reinterpret_cast<const io_t*>(p.xp_in);
            const int64_t tl = (base + (L - 1)) * H + h;
            const int64_t tlg = (base + (L - 1)) * G + hg;
            if (PM && L > 0) {
                // the last token's B through the pre-mixer (wave 0)
                if (wv == 0) {
                    for (int r = 0; r < R; ++r) {
                        const io_t* row = Bm + (tlg * R + r) * N;
                        float ss = 0.f;
                        for (int n = lane; n < N; n += 64) {
                            const float v = to_f32(row[n]);
                            ss += v * v;
                        }
#pragma unroll
                        for (int off = 1; off < 64; off <<= 1) ss += __shfl_xor(ss, off, 64);
                        const float sc = rsqrtf(ss / (float)N + p.opt.eps);
                        for (int n = lane; n < N; n += 64) {
                            const float w = p.opt.Bw != nullptr ? p.opt.Bw[n] : 1.f;
                            const float bb = p.opt.Bb != nullptr ? p.opt.Bb[((int64_t)h * R + r) * N + n] : 0.f;
                            Bo[r * N + n] = from_f32<io_t>(to_f32(row[n]) * sc * w + bb);
                        }
                    }
                }
            } else {
                for (int idx = tid; idx < R * N; idx += NT) {
                    io_t v = from_f32<io_t>(0.f);
                    if (L > 0) v = Bm[tlg * R * N + idx];
                    else if (Bi != nullptr) v = Bi[(int64_t)bh * R * N + idx];
                    Bo[idx] = v;
                }
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
template <class Cf, bool FULL, bool PM>
hipError_t scan_set_lds_limit()
{
    static hipError_t status = [] {
        const void* f = reinterpret_cast<const void*>(&scan_kernel<Cf, FULL, PM>);
        return hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize,
                                   (int)Cf::template Lay<FULL, PM>::bytes);
    }();
    return status;
}

template <class Cf, bool PM>
hipError_t launch_scan_t(const ScanParams& p, hipStream_t stream)
{
    const int64_t per_seg = (int64_t)((p.nbh + 7) / 8) * 8 * p.p_split;
    const int64_t per_slot = (p.H + 7) / 8 * 8 * p.p_split;
    // grid of each pass: (b, h, slice) x segments, or (h, slice) x (sequence,
    // segment) slots; a state pass's blocks in a last segment return
    const dim3 grid_state(p.nslots ? (unsigned)per_slot : (unsigned)per_seg,
                          p.nslots ? (unsigned)p.nslots : (unsigned)(p.nseg - 1));
    const dim3 grid_full(p.nslots ? (unsigned)per_slot : (unsigned)per_seg,
                         p.nslots ? (unsigned)p.nslots : (unsigned)p.nseg);
    constexpr size_t lds_state = Cf::template Lay<false, PM>::bytes;
    constexpr size_t lds_full = Cf::template Lay<true, PM>::bytes;
    auto* const k_state = &scan_kernel<Cf, false, PM>;
    auto* const k_full = &scan_kernel<Cf, true, PM>;
    hipError_t e;
    (void)hipGetLastError();
    // instrumented builds: stamps only when the buffer holds a row for every
    // wave of both passes
    const int64_t state_rows = p.nseg > 1 ? (int64_t)grid_state.x * grid_state.y * Cf::NW : 0;
    if (p.tl != nullptr && state_rows + (int64_t)grid_full.x * grid_full.y * Cf::NW > p.tl_rows) {
        ScanParams q = p;
        q.tl = nullptr;
        return launch_scan_t<Cf, PM>(q, stream);
    }
    if (p.nseg > 1) {
        e = scan_set_lds_limit<Cf, false, PM>();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(k_state, grid_state, dim3(Cf::NT), lds_state, stream, p);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    e = scan_set_lds_limit<Cf, true, PM>();
    if (e != hipSuccess) return e;
    if (p.tl != nullptr && p.nseg > 1) {
        // instrumented builds: the output pass's rows follow the state pass's
        ScanParams q = p;
        q.tl += (size_t)state_rows * kTlSlots;
        hipLaunchKernelGGL(k_full, grid_full, dim3(Cf::NT), lds_full, stream, q);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(k_full, grid_full, dim3(Cf::NT), lds_full, stream, p);
    return hipGetLastError();
}

template <class Cf>
hipError_t launch_scan(const ScanParams& p, hipStream_t stream)
{
    return p.opt.premix ? launch_scan_t<Cf, true>(p, stream) : launch_scan_t<Cf, false>(p, stream);
}

}  // namespace m3
