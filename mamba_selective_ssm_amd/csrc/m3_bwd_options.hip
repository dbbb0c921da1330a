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
// Every kernel here is bound by HBM bytes and runs once per call.  Rows of
// dstate values are processed by groups of lanes, 4 consecutive entries per
// lane (LPR = the power of two >= dstate/4 lanes per row, 64/LPR rows per wave
// at once).  Sums over tokens run in two fixed-order stages (partials per
// block of rows, then the partials in block order): the result is
// deterministic.
#include "m3scan.h"

#include "m3_device.hpp"
#include "m3_internal.hpp"

namespace m3 {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxPairs = 128;
constexpr int kMaxBlocks = 2048;     // grid-stride kernels: enough to fill 256 CUs
constexpr int kFinalLanes = 16;      // partial lanes per column in the final sum

__device__ __forceinline__ void ld4(const float* p, float (&v)[4])
{
    const float4 t = *reinterpret_cast<const float4*>(p);
    v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
}
__device__ __forceinline__ void ld4(const bf16* p, float (&v)[4])
{
    const bf16x4 t = *reinterpret_cast<const bf16x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (float)t[i];
}
__device__ __forceinline__ void st4(float* p, const float (&v)[4])
{
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void st4(bf16* p, const float (&v)[4])
{
    bf16x4 t;
#pragma unroll
    for (int i = 0; i < 4; ++i) t[i] = (bf16)v[i];
    *reinterpret_cast<bf16x4*>(p) = t;
}

// Sum over the aligned group of `lpr` lanes (a power of two); every lane of
// the group ends with the same value (each butterfly step adds a commutative
// pair).
__device__ __forceinline__ float group_sum(float v, int lpr)
{
    for (int off = lpr >> 1; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
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

__device__ __forceinline__ int clamp_pair(int s, int npr) { return s < 0 ? 0 : (s >= npr ? npr - 1 : s); }

// Lane layout of the row kernels.
struct RowLanes {
    int lpr, sub, c;       // lanes per row, row within the wave's group, first entry
    int64_t stride;        // rows advanced per grid-stride iteration
    __device__ RowLanes(int N, int lane)
    {
        lpr = 1;
        while (lpr * 4 < N) lpr <<= 1;
        sub = lane / lpr;
        c = (lane % lpr) * 4;
        stride = (int64_t)gridDim.x * kWaves * (64 / lpr);
    }
    __device__ int64_t first(int wave) const { return ((int64_t)blockIdx.x * kWaves + wave) * (64 / lpr); }
};

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

__device__ __forceinline__ void gain4(const float* w, int c, bool ok, float (&wv)[4])
{
    if (w != nullptr && ok) ld4(w + c, wv);
    else wv[0] = wv[1] = wv[2] = wv[3] = 1.f;
}

// B' and C' for every head of a row's group: rows are (token, group, rank);
// blockIdx.y picks B (0) or C (1).
template <typename IO>
__global__ void __launch_bounds__(kThreads) bo_prep_bc_kernel(BwdOptParams p)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const RowLanes rl(p.N, lane);
    const bool isC = blockIdx.y != 0;
    const IO* src = static_cast<const IO*>(isC ? p.C : p.B);
    IO* dst = static_cast<IO*>(isC ? p.Ce : p.Be);
    const float* bias = isC ? p.opt.Cb : p.opt.Bb;
    const bool colok = rl.c < p.N;
    float wv[4];
    gain4(isC ? p.opt.Cw : p.opt.Bw, rl.c, colok, wv);
    const int64_t rows = p.BtL * p.G * p.R, hpg = p.H / p.G;
    for (int64_t r0 = rl.first(wave); r0 < rows; r0 += rl.stride) {
        const int64_t row = r0 + rl.sub;
        const bool ok = colok && row < rows;
        float v[4] = {0.f, 0.f, 0.f, 0.f};
        if (ok) ld4(src + row * p.N + rl.c, v);
        float sc = 1.f;
        if (p.opt.premix) {
            const float ss = group_sum(v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3], rl.lpr);
            sc = rsqrtf(ss / (float)p.N + p.opt.eps);
        }
        if (!ok) continue;
        const RowIdx ri = row_index(p, row);
        for (int64_t j = 0; j < hpg; ++j) {
            const int64_t h = ri.g * hpg + j;
            float o[4] = {v[0], v[1], v[2], v[3]};
            if (p.opt.premix) {
                float b[4] = {0.f, 0.f, 0.f, 0.f};
                if (bias) ld4(bias + (h * p.R + ri.r) * p.N + rl.c, b);
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i] = v[i] * sc * wv[i] + b[i];
            }
            st4(dst + ((ri.bt * p.H + h) * p.R + ri.r) * p.N + rl.c, o);
        }
    }
}

// Thread layout of the per-token maps: with theta rows, nq threads per token
// (4 pairs each) and 256/nq tokens per block step; else one token per thread.
struct TokLanes {
    int rpb, lr, q4;
    bool ok;
    __device__ TokLanes(bool th, int nq)
    {
        rpb = th ? kThreads / nq : kThreads;
        lr = th ? (int)threadIdx.x / nq : (int)threadIdx.x;
        q4 = th ? ((int)threadIdx.x % nq) * 4 : 0;
        ok = lr < rpb;
    }
};

// Per-token maps before the gradient, 4 rotary pairs per thread (dstate is a
// multiple of 8): theta after the phase map (zero mode: theta is not read)
// and, with the pre-mixer, dt = softplus(dt_raw + dt_bias_h) and
// lam = sigmoid(lam_raw) (by the thread holding the token's first pairs).
__global__ void __launch_bounds__(kThreads) bo_prep_tok_kernel(BwdOptParams p)
{
    __shared__ int sperm[kMaxPairs];
    const int npr = p.N / 2, nq = npr / 4;
    const bool shuffle = p.opt.phase == M3_PHASE_SHUFFLE, th = p.thetae != nullptr;
    if (shuffle) {
        for (int j = threadIdx.x; j < npr; j += kThreads) sperm[j] = clamp_pair(p.opt.perm[j], npr);
        __syncthreads();
    }
    const int64_t tok = p.BtL * p.H;
    const TokLanes tl(th, nq);
    for (int64_t r0 = (int64_t)blockIdx.x * tl.rpb; r0 < tok; r0 += (int64_t)gridDim.x * tl.rpb) {
        const int64_t row = r0 + tl.lr;
        if (!tl.ok || row >= tok) continue;
        const int q4 = tl.q4;
        if (th) {
            float o[4] = {0.f, 0.f, 0.f, 0.f};
            const float* src = p.theta + row * npr;
            if (p.opt.phase == M3_PHASE_REVERSE) {
                ld4(src + q4, o);
#pragma unroll
                for (int k = 0; k < 4; ++k) o[k] = -o[k];
            } else if (shuffle) {
#pragma unroll
                for (int k = 0; k < 4; ++k) o[k] = src[sperm[q4 + k]];
            }
            st4(p.thetae + row * npr + q4, o);
        }
        if (p.dte != nullptr && q4 == 0) {
            p.dte[row] = softplus_acc(p.dt[row] + (p.opt.dtb ? p.opt.dtb[row % p.H] : 0.f));
            p.lame[row] = sigmoid_acc(p.lam[row]);
        }
    }
}

// Group sums of dB', dC' and, with the pre-mixer, the RMSNorm backward; the
// gain terms G xh are summed over this block's rows into qpart[y][block][N]
// (lanes' row sums, then the block's lanes in fixed order).
template <typename IO>
__global__ void __launch_bounds__(kThreads) bo_post_bc_kernel(BwdOptParams p)
{
    __shared__ float red[kWaves][64][4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const RowLanes rl(p.N, lane);
    const bool isC = blockIdx.y != 0;
    const float* dsrc = isC ? p.dCe : p.dBe;
    float* dout = isC ? p.dC : p.dB;
    const IO* src = static_cast<const IO*>(isC ? p.C : p.B);
    const bool colok = rl.c < p.N;
    float wv[4];
    gain4(isC ? p.opt.Cw : p.opt.Bw, rl.c, colok, wv);
    const int64_t rows = p.BtL * p.G * p.R, hpg = p.H / p.G;
    float qacc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int64_t r0 = rl.first(wave); r0 < rows; r0 += rl.stride) {
        const int64_t row = r0 + rl.sub;
        const bool ok = colok && row < rows;
        float G[4] = {0.f, 0.f, 0.f, 0.f};
        if (ok) {
            const RowIdx ri = row_index(p, row);
            for (int64_t j = 0; j < hpg; ++j) {
                float d[4];
                ld4(dsrc + ((ri.bt * p.H + ri.g * hpg + j) * p.R + ri.r) * p.N + rl.c, d);
#pragma unroll
                for (int i = 0; i < 4; ++i) G[i] += d[i];
            }
        }
        if (!p.opt.premix) {
            if (ok) st4(dout + row * p.N + rl.c, G);
            continue;
        }
        float v[4] = {0.f, 0.f, 0.f, 0.f};
        if (ok) ld4(src + row * p.N + rl.c, v);
        const float ss = group_sum(v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3], rl.lpr);
        const float sc = rsqrtf(ss / (float)p.N + p.opt.eps);
        float gx = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) gx += G[i] * wv[i] * (v[i] * sc);
        gx = group_sum(gx, rl.lpr) / (float)p.N;
        if (!ok) continue;
        float o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float xh = v[i] * sc;
            o[i] = sc * (G[i] * wv[i] - xh * gx);
            qacc[i] += G[i] * xh;
        }
        st4(dout + row * p.N + rl.c, o);
    }
    if (!p.opt.premix || p.qpart == nullptr) return;   // uniform over the block
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][lane][i] = qacc[i];
    __syncthreads();
    // column quad t: the block's lanes holding it, wave by wave, group by group
    for (int t = threadIdx.x; t < rl.lpr; t += kThreads) {
        if (t * 4 >= p.N) continue;
        float s[4] = {0.f, 0.f, 0.f, 0.f};
        for (int w = 0; w < kWaves; ++w)
            for (int g = 0; g < 64 / rl.lpr; ++g)
#pragma unroll
                for (int i = 0; i < 4; ++i) s[i] += red[w][g * rl.lpr + t][i];
        st4(p.qpart + ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * p.N + t * 4, s);
    }
}

// Per-token maps after the gradient, 4 rotary pairs per thread: dtheta from
// the gradient of the mapped theta and, with the pre-mixer, ddt and dlam
// through softplus and sigmoid (in place).  Shuffle: each block lists, per
// pair j, the pairs i with perm[i] = j in increasing order (a chain first[j]
// -> next[i] -> ...); every i is on exactly one chain.
__global__ void __launch_bounds__(kThreads) bo_post_tok_kernel(BwdOptParams p)
{
    __shared__ int sperm[kMaxPairs], first[kMaxPairs], next[kMaxPairs];
    const int npr = p.N / 2, nq = npr / 4;
    const bool shuffle = p.opt.phase == M3_PHASE_SHUFFLE;
    const bool th = p.dthetae != nullptr && p.dtheta != nullptr;
    if (shuffle && th) {
        for (int j = threadIdx.x; j < npr; j += kThreads) sperm[j] = clamp_pair(p.opt.perm[j], npr);
        __syncthreads();
        for (int j = threadIdx.x; j < npr; j += kThreads) {
            int prev = -1;
            first[j] = -1;
            for (int i = 0; i < npr; ++i) {
                if (sperm[i] != j) continue;
                if (prev < 0) first[j] = i;
                else next[prev] = i;
                prev = i;
            }
            if (prev >= 0) next[prev] = -1;
        }
        __syncthreads();
    }
    const int64_t tok = p.BtL * p.H;
    const TokLanes tl(th, nq);
    for (int64_t r0 = (int64_t)blockIdx.x * tl.rpb; r0 < tok; r0 += (int64_t)gridDim.x * tl.rpb) {
        const int64_t row = r0 + tl.lr;
        if (!tl.ok || row >= tok) continue;
        const int q4 = tl.q4;
        if (th) {
            float o[4] = {0.f, 0.f, 0.f, 0.f};
            const float* d = p.dthetae + row * npr;
            if (p.opt.phase == M3_PHASE_REVERSE) {
                ld4(d + q4, o);
#pragma unroll
                for (int k = 0; k < 4; ++k) o[k] = -o[k];
            } else if (shuffle) {
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    for (int c = first[q4 + k]; c >= 0; c = next[c]) o[k] += d[c];
            }
            st4(p.dtheta + row * npr + q4, o);
        }
        if (p.opt.premix && q4 == 0) {
            p.ddt[row] *= sigmoid_acc(p.dt[row] + (p.opt.dtb ? p.opt.dtb[row % p.H] : 0.f));
            const float sg = sigmoid_acc(p.lam[row]);
            p.dlam[row] *= sg * (1.f - sg);
        }
    }
}

// Token rows between packed and padded layouts: one block per padded token
// (s, t); a sequence's offsets are clamped into [0, T] and its length to maxL
// (bad offsets give wrong results, never accesses outside the arrays).
__global__ void __launch_bounds__(kThreads) bo_pack_kernel(PackParams q)
{
    const int64_t ntok = q.nseq * q.maxL;
    for (int64_t i = blockIdx.x; i < ntok; i += gridDim.x) {
        const int64_t s = i / q.maxL, t = i % q.maxL;
        int64_t st = q.cu[s], en = q.cu[s + 1];
        st = st < 0 ? 0 : (st > q.T ? q.T : st);
        en = en < st ? st : (en > q.T ? q.T : en);
        const int64_t len = en - st < q.maxL ? en - st : q.maxL;
        const bool real = t < len;
        if (q.unpack && !real) continue;                // uniform over the block
        for (int k = 0; k < q.n; ++k) {
            const int W = q.words[k];
            const uint32_t* src = static_cast<const uint32_t*>(q.src[k]);
            uint32_t* dst = static_cast<uint32_t*>(q.dst[k]);
            const int64_t pad = i * W, pk = (st + t) * W;
            for (int w = threadIdx.x; w < W; w += kThreads) {
                if (q.unpack) dst[pk + w] = src[pad + w];
                else dst[pad + w] = real ? src[pk + w] : 0u;
            }
        }
    }
}

// Column sums of [rows][cols] float32 arrays, one or two per launch
// (blockIdx.z picks the array; a NULL destination is skipped).
struct ColPair {
    const float* src[2];
    float* dst[2];
};

// Stage 1: block (x, y) = 64 columns x 4 row lanes over rows y*rpc .. y*rpc +
// rpc - 1; lane k takes every 4th row from k, then the 4 lanes are added in
// order into part[z][y][cols].
__global__ void __launch_bounds__(kThreads) bo_colsum_partial_kernel(ColPair cp, int64_t rows,
                                                                      int64_t cols, int64_t rpc,
                                                                      float* part, int64_t pstride)
{
    __shared__ float red[kWaves][64];
    const int z = blockIdx.z;
    if (cp.dst[z] == nullptr) return;                   // uniform over the block
    const float* src = cp.src[z];
    const int cl = threadIdx.x & 63, k = threadIdx.x >> 6;
    const int64_t c = (int64_t)blockIdx.x * 64 + cl;
    const int64_t r0 = (int64_t)blockIdx.y * rpc;
    const int64_t r1 = r0 + rpc < rows ? r0 + rpc : rows;
    float acc = 0.f;
    if (c < cols) {
#pragma unroll 8
        for (int64_t r = r0 + k; r < r1; r += kWaves) acc += src[r * cols + c];
    }
    red[k][cl] = acc;
    __syncthreads();
    if (k == 0 && c < cols)
        part[z * pstride + (int64_t)blockIdx.y * cols + c] =
            ((red[0][cl] + red[1][cl]) + red[2][cl]) + red[3][cl];
}

// Stage 2: block = 64 columns x 16 partial lanes; lane k adds partials k,
// k + 16, ... in order, then the 16 lanes are added in order.
__global__ void __launch_bounds__(64 * kFinalLanes) bo_colsum_final_kernel(const float* part, int64_t pstride,
                                                                          int nchunk, int64_t cols,
                                                                          ColPair cp)
{
    __shared__ float red[kFinalLanes][64];
    const int z = blockIdx.z;
    float* dst = cp.dst[z];
    if (dst == nullptr) return;                         // uniform over the block
    part += z * pstride;
    const int cl = threadIdx.x & 63, k = threadIdx.x >> 6;
    const int64_t c = (int64_t)blockIdx.x * 64 + cl;
    float acc = 0.f;
    if (c < cols) {
#pragma unroll 8
        for (int q = k; q < nchunk; q += kFinalLanes) acc += part[(int64_t)q * cols + c];
    }
    red[k][cl] = acc;
    __syncthreads();
    if (k == 0 && c < cols) {
        float s = 0.f;
        for (int q = 0; q < kFinalLanes; ++q) s += red[q][cl];
        dst[c] = s;
    }
}

// Row chunks of a stage-1 column sum: about 2048 blocks in all, at least 16
// rows per chunk, at most 4 Mi partial values.
void colsum_plan(int64_t rows, int64_t cols, int64_t* rpc, int* nchunk)
{
    const int64_t tiles = (cols + 63) / 64 > 0 ? (cols + 63) / 64 : 1;
    int64_t nc = kMaxBlocks / tiles;
    const int64_t by_rows = (rows + 15) / 16;
    if (nc > by_rows) nc = by_rows;
    const int64_t cap = ((int64_t)1 << 22) / (cols > 0 ? cols : 1);
    if (nc > cap) nc = cap;
    if (nc < 1) nc = 1;
    int64_t r = (rows + nc - 1) / nc;
    if (r < 1) r = 1;
    *rpc = r;
    *nchunk = (int)((rows + r - 1) / r);
    if (*nchunk < 1) *nchunk = 1;
}

size_t colsum_partial_floats(int64_t rows, int64_t cols)
{
    int64_t rpc;
    int nchunk;
    colsum_plan(rows, cols, &rpc, &nchunk);
    return (size_t)nchunk * (size_t)(cols > 0 ? cols : 0);
}

hipError_t colsum_final(const float* part, int64_t pstride, int nchunk, int64_t cols,
                        const ColPair& cp, hipStream_t s)
{
    hipLaunchKernelGGL(bo_colsum_final_kernel, dim3((unsigned)((cols + 63) / 64), 1, 2),
                       dim3(64 * kFinalLanes), 0, s, part, pstride, nchunk, cols, cp);
    return hipGetLastError();
}

// Column sums of one or two [rows][cols] arrays; `part` holds two partial
// sets of colsum_partial_floats(rows, cols) values.
hipError_t colsum(const ColPair& cp, int64_t rows, int64_t cols, float* part, hipStream_t s)
{
    if (cols <= 0) return hipSuccess;
    int64_t rpc;
    int nchunk;
    colsum_plan(rows, cols, &rpc, &nchunk);
    const int64_t pstride = (int64_t)nchunk * cols;
    hipLaunchKernelGGL(bo_colsum_partial_kernel, dim3((unsigned)((cols + 63) / 64), nchunk, 2),
                       dim3(kThreads), 0, s, cp, rows, cols, rpc, part, pstride);
    const hipError_t e = hipGetLastError();
    return e != hipSuccess ? e : colsum_final(part, pstride, nchunk, cols, cp, s);
}

unsigned stride_grid_n(int64_t n)
{
    const int64_t b = (n + kThreads - 1) / kThreads;
    return (unsigned)(b < 1 ? 1 : (b < kMaxBlocks ? b : kMaxBlocks));
}

// Blocks of the per-token maps (TokLanes: 256/nq tokens per block step).
unsigned tok_grid(int64_t tok, bool th, int N)
{
    const int64_t rpb = th ? kThreads / (N / 8) : kThreads;
    const int64_t b = (tok + rpb - 1) / rpb;
    return (unsigned)(b < 1 ? 1 : (b < kMaxBlocks ? b : kMaxBlocks));
}

// Blocks of the row kernels: 4 waves, 64/LPR rows per wave at once.
unsigned row_grid(int64_t rows, int N)
{
    int lpr = 1;
    while (lpr * 4 < N) lpr <<= 1;
    const int64_t per_block = (int64_t)kWaves * (64 / lpr);
    const int64_t b = (rows + per_block - 1) / per_block;
    return (unsigned)(b < 1 ? 1 : (b < kMaxBlocks ? b : kMaxBlocks));
}

template <typename IO>
hipError_t pre_impl(const BwdOptParams& p, hipStream_t s)
{
    const int64_t rows = p.BtL * p.G * p.R, tok = p.BtL * p.H;
    if (p.Be != nullptr && rows > 0)
        hipLaunchKernelGGL(bo_prep_bc_kernel<IO>, dim3(row_grid(rows, p.N), 2), dim3(kThreads), 0, s, p);
    if ((p.thetae != nullptr || p.dte != nullptr) && tok > 0)
        hipLaunchKernelGGL(bo_prep_tok_kernel, dim3(tok_grid(tok, p.thetae != nullptr, p.N)), dim3(kThreads),
                           0, s, p);
    return hipGetLastError();
}

template <typename IO>
hipError_t post_impl(const BwdOptParams& p, hipStream_t s)
{
    const int64_t rows = p.BtL * p.G * p.R, tok = p.BtL * p.H;
    const unsigned gbc = row_grid(rows, p.N);
    if (p.dBe != nullptr && rows > 0)
        hipLaunchKernelGGL(bo_post_bc_kernel<IO>, dim3(gbc, 2), dim3(kThreads), 0, s, p);
    const bool th = p.dthetae != nullptr && p.dtheta != nullptr;
    if ((th || p.opt.premix) && tok > 0)
        hipLaunchKernelGGL(bo_post_tok_kernel, dim3(tok_grid(tok, th, p.N)), dim3(kThreads), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !p.opt.premix) return e;
    // gain gradients: the row kernel's per-block partials (none written when
    // there are no rows: the sums are then zero)
    const ColPair gains = {{nullptr, nullptr}, {p.dBw, p.dCw}};
    if ((p.dBw || p.dCw) &&
        (e = colsum_final(p.qpart, (int64_t)gbc * p.N, rows > 0 ? (int)gbc : 0, p.N, gains, s)) != hipSuccess)
        return e;
    const ColPair dtb = {{p.ddt, nullptr}, {p.ddtb, nullptr}};
    if (p.ddtb && (e = colsum(dtb, p.BtL, p.H, p.part, s)) != hipSuccess) return e;
    const ColPair bias = {{p.dBe, p.dCe}, {p.dBb, p.dCb}};
    if ((p.dBb || p.dCb) && (e = colsum(bias, p.BtL, p.H * p.R * p.N, p.part, s)) != hipSuccess) return e;
    return hipSuccess;
}

}  // namespace

size_t bwd_options_partial_floats(int64_t BtL, int64_t H, int64_t G, int N, int R)
{
    // two partial sets (B and C) of the larger of the two column sums
    size_t a = colsum_partial_floats(BtL, H), b = colsum_partial_floats(BtL, H * R * N);
    return 2 * (a > b ? a : b);
}

size_t bwd_options_gain_floats(int64_t BtL, int64_t G, int N, int R)
{
    return 2 * (size_t)row_grid(BtL * G * R, N) * (size_t)N;
}

hipError_t launch_bwd_pack(const PackParams& p, hipStream_t stream)
{
    const int64_t ntok = p.nseq * p.maxL;
    if (ntok <= 0 || p.n <= 0) return hipSuccess;
    const unsigned grid = (unsigned)(ntok < 8192 ? ntok : 8192);
    hipLaunchKernelGGL(bo_pack_kernel, dim3(grid), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

// One thread per (sequence, head, rank, entry) of the record gradient.
__global__ void __launch_bounds__(kThreads) bo_record_grad_kernel(RecGradParams q)
{
    const int64_t per = (int64_t)q.R * (q.N + q.P);
    const int64_t total = q.batch * q.H * per;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * kThreads) {
        const int64_t bh = i / per, b = bh / q.H, h = bh % q.H;
        const int64_t e = i % per;
        const bool isB = e < (int64_t)q.R * q.N;
        const int64_t k = isB ? e : e - (int64_t)q.R * q.N;     // (r, n) or (r, p)
        const int W = isB ? q.N : q.P;
        const float g = isB ? q.dBL[bh * q.R * q.N + k] : q.dxL[bh * q.R * q.P + k];
        int64_t last = -1;                                       // token row of the last token
        if (q.cu != nullptr) {
            // offsets clamped and the length capped at max_seqlen, as the
            // forward and the padding kernel do: the record holds token
            // st + len - 1
            int64_t st = q.cu[b], en = q.cu[b + 1];
            st = st < 0 ? 0 : (st > q.L ? q.L : st);
            en = en < st ? st : (en > q.L ? q.L : en);
            const int64_t len = en - st < q.max_len ? en - st : q.max_len;
            if (len > 0) last = st + len - 1;
        } else if (q.L > 0) {
            last = b * q.L + q.L - 1;
        }
        if (last >= 0) {
            float* dst = isB ? q.dB : q.dx;
            dst[(last * q.H + h) * q.R * W + k] += g;
        } else {
            float* dst = isB ? q.dBp : q.dxp;
            if (dst != nullptr) dst[bh * q.R * W + k] += g;
        }
    }
}

hipError_t launch_bwd_record_grad(const RecGradParams& p, hipStream_t stream)
{
    const int64_t total = p.batch * p.H * (int64_t)p.R * (p.N + p.P);
    if (total <= 0) return hipSuccess;
    hipLaunchKernelGGL(bo_record_grad_kernel, dim3(stride_grid_n(total)), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
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
