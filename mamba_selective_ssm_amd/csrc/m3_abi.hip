// C ABI of libm3scan: argument validation (complete before any HIP call),
// variant selection and launch.  See include/m3scan.h for the contract.
#include "m3scan.h"

#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "m3_internal.hpp"
#include "m3_scan_kernel.hpp"

namespace {

#if M3_TIMELINE
// Instrumented builds: the device buffer that scan kernels write their
// per-wave phase stamps into (set by m3_timeline_buffer; null: no stamps).
unsigned long long* g_timeline = nullptr;
int64_t g_timeline_rows = 0;
#endif


thread_local int g_last_hip_error = 0;

struct Range {
    uintptr_t lo, hi;   // [lo, hi)
};

Range range_of(const void* p, int64_t bytes)
{
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    if (p == nullptr) return Range{0, 0};   // absent pointers overlap nothing
    return Range{a, a + static_cast<uintptr_t>(bytes > 0 ? bytes : 0)};
}

bool overlaps(const Range& a, const Range& b)
{
    if (a.lo == a.hi || b.lo == b.hi) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int io_size(int dt) { return dt == M3_F32 ? 4 : 2; }

// Default chunk length: 64 operand rows (tokens x rank) for bf16, 32 for fp32
// (whose double-buffered tiles take twice the LDS).
int default_chunk(int64_t R, int io) { return io == M3_BF16 ? (int)(64 / R) : (int)(32 / R); }

template <typename F>
void for_each_variant(F&& f)
{
    using table_fn = const m3::ScanVariant* (*)(int*);
    const table_fn tables[] = {m3::scan_variants_f32, m3::scan_variants_bf16a,
                               m3::scan_variants_bf16b};
    for (table_fn t : tables) {
        int n = 0;
        const m3::ScanVariant* v = t(&n);
        for (int i = 0; i < n; ++i) f(v[i]);
    }
}

// The compiled variant for these sizes.  chunk / p_split 0 = library choice:
// the widest headdim slice (no work repeated across slices); sequence
// segments then supply the parallelism.
const m3::ScanVariant* pick_scan(int io, int64_t N, int64_t R, int64_t P, int chunk,
                                 int p_split, int64_t nbh, int premix = 0)
{
    const int Q = chunk ? chunk : default_chunk(R, io);
    const m3::ScanVariant* best = nullptr;
    for_each_variant([&](const m3::ScanVariant& v) {
        if (v.io != io || v.N != N || v.R != R || v.Q != Q) return;
        if (P % v.PS != 0) return;
        if (p_split != 0 && P / v.PS != p_split) return;
        if (v.pm && !premix) return;                          // pre-mixer-only variant
        (void)nbh;
        // first of the widest; with the pre-mixer a pre-mixer variant of
        // the same width wins
        if (best == nullptr || v.PS > best->PS || (v.PS == best->PS && v.pm && !best->pm)) best = &v;
    });
    return best;
}

m3_status hip_status(hipError_t e)
{
    if (e == hipSuccess) return M3_OK;
    g_last_hip_error = static_cast<int>(e);
    return M3_ERR_HIP;
}

// Options common to both entry points: ranges, required pointers, alignment.
// Fills the kernel-side fields; `ntok` is the scan's seqlen (the bound of
// packed-sequence lengths), or -1 for a decode step (no packed sequences).
m3_status check_options(const m3_options& o, int64_t H, int64_t N, int64_t R, int64_t ntok,
                        m3::OptParams* k)
{
    // packed sequences: scan calls only (a decode step passes ntok < 0)
    if (o.cu_seqlens != nullptr && (ntok < 0 || o.max_seqlen < 0 || o.max_seqlen > ntok))
        return M3_ERR_OPTION;
    if (o.ngroups < 0 || (o.ngroups > 0 && H > 0 && H % o.ngroups != 0)) return M3_ERR_OPTION;
    if (o.A_per_token != 0 && o.A_per_token != 1) return M3_ERR_OPTION;
    if (o.phase_mode < M3_PHASE_NATIVE || o.phase_mode > M3_PHASE_NO_WRITE_READ) return M3_ERR_OPTION;
    // rotation removed from writing / readout: decode steps only
    if (o.phase_mode >= M3_PHASE_NO_WRITE && ntok >= 0) return M3_ERR_OPTION;
    if (o.premix != 0 && o.premix != 1) return M3_ERR_OPTION;
    if (o.premix && !(o.norm_eps >= 0.f && o.norm_eps < 3.0e38f)) return M3_ERR_OPTION;
    if (o.phase_mode == M3_PHASE_SHUFFLE && o.phase_perm == nullptr) return M3_ERR_NULL;
    const void* ptrs[] = {o.phase_perm, o.B_norm_w, o.C_norm_w, o.B_bias, o.C_bias, o.dt_bias,
                          o.cu_seqlens, o.phase_in, o.phase_out};
    for (const void* q : ptrs)
        if (q != nullptr && !aligned16(q)) return M3_ERR_ALIGN;
    (void)N; (void)R;
    k->groups = o.ngroups > 0 ? o.ngroups : H;
    k->a_tok = o.A_per_token;
    k->phase = o.phase_mode;
    k->perm = o.phase_mode == M3_PHASE_SHUFFLE ? o.phase_perm : nullptr;
    k->premix = o.premix;
    k->eps = o.norm_eps;
    k->Bw = o.premix ? o.B_norm_w : nullptr;
    k->Cw = o.premix ? o.C_norm_w : nullptr;
    k->Bb = o.premix ? o.B_bias : nullptr;
    k->Cb = o.premix ? o.C_bias : nullptr;
    k->dtb = o.premix ? o.dt_bias : nullptr;
    k->cu = o.cu_seqlens;
    k->max_len = o.max_seqlen;
    k->phase_in = o.phase_in;
    k->phase_out = o.phase_out;
    return M3_OK;
}

// Byte ranges of the option arrays (inputs of the call).
void option_ranges(const m3_options& o, int64_t Bt, int64_t H, int64_t N, int64_t R, Range* out)
{
    out[6] = range_of(o.cu_seqlens, (Bt + 1) * 4);
    out[0] = range_of(o.phase_mode == M3_PHASE_SHUFFLE ? o.phase_perm : nullptr, (N / 2) * 4);
    out[1] = range_of(o.premix ? o.B_norm_w : nullptr, N * 4);
    out[2] = range_of(o.premix ? o.C_norm_w : nullptr, N * 4);
    out[3] = range_of(o.premix ? o.B_bias : nullptr, H * R * N * 4);
    out[4] = range_of(o.premix ? o.C_bias : nullptr, H * R * N * 4);
    out[5] = range_of(o.premix ? o.dt_bias : nullptr, H * 4);
    out[7] = range_of(o.phase_in != o.phase_out ? o.phase_in : nullptr, Bt * H * (N / 2) * 4);
}

struct ScanPlan {
    const m3::ScanVariant* v;
    int p_split, nseg, seg_chunks;
    int nslots;                // packed sequences with per-sequence segments (0: uniform)
    int64_t phase_blocks;      // 64-token blocks per sequence (accumulated angle)
    size_t phase_off;          // workspace offset of the angle's partial sums
    bool rec_alias;            // the output state record is the input record
    size_t snap_off;           // workspace offset of the input record's copy (rec_alias)
    size_t snap_h, snap_b;     // its h and B_prev parts in bytes (x_prev follows)
    size_t ws;
};

// The output state record is exactly the input record (updated in place).
bool record_in_place(const m3_scan_args* a)
{
    return a->h_in != nullptr && a->h_out == a->h_in && a->B_prev_out == a->B_prev_in &&
           a->x_prev_out == a->x_prev_in;
}

// Everything about a call that depends only on sizes: the compiled variant,
// the headdim split, the sequence segments and the workspace they need.
m3_status plan_scan(const m3_scan_args* a, ScanPlan* out)
{
    if (a == nullptr) return M3_ERR_NULL;
    const int64_t Bt = a->batch, L = a->seqlen, H = a->nheads;
    const int64_t P = a->headdim, N = a->dstate, R = a->rank;
    if (Bt < 0 || L < 0 || H < 0 || P < 1 || N < 1 || R < 1 || (N % 2) != 0) return M3_ERR_SHAPE;
    if (a->chunk < 0 || a->p_split < 0 || a->segments < 0) return M3_ERR_SHAPE;
    if (a->io_dtype != M3_F32 && a->io_dtype != M3_BF16) return M3_ERR_DTYPE;
    const int64_t nbh = Bt * H;
    if (nbh > (int64_t)1 << 28) return M3_ERR_UNSUPPORTED;
    const m3::ScanVariant* v = pick_scan(a->io_dtype, N, R, P, a->chunk, a->p_split,
                                         nbh > 0 ? nbh : 1, a->opt.premix == 1);
    if (v == nullptr) return M3_ERR_UNSUPPORTED;
    // In-chunk offsets are 32-bit: a chunk's span of every tensor must fit,
    // and a token's byte stride must fit the 24-bit multiplier.
    const int64_t wide = (N > P ? N : P) * R;
    if ((int64_t)v->Q * H * wide >= ((int64_t)1 << 31)) return M3_ERR_UNSUPPORTED;
    if (H * wide * 4 >= ((int64_t)1 << 24)) return M3_ERR_UNSUPPORTED;
    const int p_split = (int)(P / v->PS);
    // the launch grid's x dimension, (b, h, slice) slots, counts work items in 32 bits
    if (((nbh + 7) / 8 * 8 + 8) * p_split * (int64_t)v->NW * 64 >= ((int64_t)1 << 32)) return M3_ERR_UNSUPPORTED;
    // packed sequences: the launch is sized for the longest one
    const int64_t Lrun = a->opt.cu_seqlens != nullptr ? (a->opt.max_seqlen >= 0 ? a->opt.max_seqlen : 0) : L;
    const int64_t nchunks = (Lrun + v->Q - 1) / v->Q;
    int64_t nseg = a->segments;
    if (nseg == 0) {
        // Fill the chip: about `occ` workgroups per compute unit (256 CUs),
        // with at least three chunks per segment.
        const int64_t per_seg = (nbh > 0 ? (nbh + 7) / 8 * 8 : 8) * p_split;
        const int64_t target = 256 * (int64_t)v->occ;
        nseg = (target + per_seg - 1) / per_seg;
        if (nseg > nchunks / 3) nseg = nchunks / 3;
        if (nseg > 64) nseg = 64;
    }
    if (nseg > nchunks) nseg = nchunks;
    if (nseg < 1) nseg = 1;
    int64_t seg_chunks = nchunks > 0 ? (nchunks + nseg - 1) / nseg : 1;
    nseg = nchunks > 0 ? (nchunks + seg_chunks - 1) / seg_chunks : 1;
    if (nseg * ((nbh + 7) / 8 * 8) * p_split >= ((int64_t)1 << 31)) return M3_ERR_UNSUPPORTED;
    int64_t nslots = 0;
    if (a->opt.cu_seqlens != nullptr && a->segments == 0 && nbh > 0 && Bt <= 65536) {
        // Packed sequences, library's segmentation: segments of a fixed
        // number of chunks per sequence (a short sequence takes fewer), about
        // `occ` workgroups per compute unit in all, at least three chunks per
        // segment.  Each workgroup finds its (sequence, segment) on the device;
        // the launch covers an upper bound of such slots.
        const int64_t per_slot = (H + 7) / 8 * 8 * p_split;
        int64_t tslots = 256 * (int64_t)v->occ / per_slot;
        tslots = tslots < 1 ? 1 : tslots;
        const int64_t tchunks = (L + v->Q - 1) / v->Q;
        int64_t sc = (tchunks + tslots - 1) / tslots;
        sc = sc < 3 ? 3 : sc;
        const int64_t maxseg = nchunks > 0 ? (nchunks + sc - 1) / sc : 1;
        if (maxseg > 1) {
            // sum_b max(1, ceil(ceil(len_b / Q) / sc)) <= L / (Q sc) + 2 nseq
            // when the offsets rise (others only give wrong results)
            nslots = (tchunks + sc - 1) / sc + 2 * Bt + 1;
            if (nslots * per_slot >= ((int64_t)1 << 31)) return M3_ERR_UNSUPPORTED;
            nseg = maxseg;
            seg_chunks = sc;
        }
    }
    out->v = v;
    out->p_split = p_split;
    out->nseg = (int)nseg;
    out->seg_chunks = (int)seg_chunks;
    out->nslots = (int)nslots;
    out->ws = v->ws_bytes(nbh, P, (int)nseg);
    out->phase_blocks = 0;
    out->phase_off = 0;
    if (a->opt.phase_out != nullptr) {
        // float64 partial sums of the accumulated angle, per (row, head, block, pair)
        out->phase_blocks = (Lrun + m3::kPhaseBlock - 1) / m3::kPhaseBlock;
        if (out->phase_blocks > 65535) return M3_ERR_UNSUPPORTED;
        out->phase_off = (out->ws + 255) / 256 * 256;
        out->ws = out->phase_off + (size_t)nbh * out->phase_blocks * (N / 2) * 8;
    }
    // An in-place record: the kernels read a copy of the input record taken
    // at the start of the call (the last segment's workgroups write the new
    // record while others may still be about to read the old one).
    out->rec_alias = record_in_place(a);
    out->snap_off = out->snap_h = out->snap_b = 0;
    if (out->rec_alias && nbh > 0) {
        const size_t e = a->io_dtype == M3_F32 ? 4 : 2;
        out->snap_off = (out->ws + 255) / 256 * 256;
        out->snap_h = (size_t)nbh * N * P * 4;
        out->snap_b = ((size_t)nbh * R * N * e + 15) / 16 * 16;
        out->ws = out->snap_off + out->snap_h + out->snap_b + (size_t)nbh * R * P * e;
    }
    return M3_OK;
}

// Backward.  Step method: sub-block length TB, sub-blocks per checkpoint K,
// checkpoints per (b, h) and the workspace carve-up (checkpoints, scratch,
// dA shares).  Chunked method: chunks per (b, h) and its carve-up.
struct BwdPlan {
    int method;                 // M3_BWD_STEP or M3_BWD_CHUNKED
    int TB, K, parts;
    int64_t nsup;
    size_t unit_floats, ck_bytes, scr_bytes, dx_bytes, scal_bytes, dxp_bytes, part_bytes;
    int64_t nc;
    size_t loc_bytes, cs_bytes, st_bytes, chunk_bytes, bh_bytes;
    size_t core_ws;             // the plain gradient's workspace
    // Options: the maps around the plain gradient and their workspace, which
    // follows the plain gradient's.
    bool opt_bc, opt_scal, opt_theta;
    int64_t groups;
    size_t be_bytes, dbe_bytes, se_bytes, te_bytes, q_bytes, sum_bytes;
    // Packed sequences: the plain gradient runs on a padded batch of
    // [batch][max_seqlen] tokens (inputs and gradients), packed <-> padded
    // around it.
    bool packed;
    int64_t Lp;                 // max_seqlen
    size_t px_bytes, pb_bytes, ps_bytes, pt_bytes;        // io rows x, B; float rows dt, theta
    size_t gx_bytes, gb_bytes, gs_bytes;                  // float32 gradient rows
    size_t ws;
};

size_t round256(size_t v) { return (v + 255) / 256 * 256; }

bool bwd_method_ok(int method, int64_t N, int64_t P, int64_t R, int io)
{
    if (method == M3_BWD_STEP) return m3::bwd_supported(N, P, R, io);
    if (method == M3_BWD_CHUNKED) return m3::bwd_chunked_supported(N, P, R, io);
    return m3::bwd_chunked_supported(N, P, R, io) || m3::bwd_supported(N, P, R, io);
}

m3_status plan_bwd_core(const m3_scan_bwd_args* a, BwdPlan* out);

// The options a gradient call supports (per-token decay, head groups, the
// phase maps of a scan, the pre-mixer, packed sequences) and the workspace of
// their maps.
m3_status plan_bwd_options(const m3_scan_bwd_args* a, BwdPlan* out)
{
    const m3_options& o = a->opt;
    const int64_t Bt = a->batch, L = a->seqlen, H = a->nheads;
    const int64_t P = a->headdim, N = a->dstate, R = a->rank;
    if (o.phase_in != nullptr || o.phase_out != nullptr) return M3_ERR_UNSUPPORTED;
    if (o.A_per_token != 0 && o.A_per_token != 1) return M3_ERR_OPTION;
    if (o.phase_mode < M3_PHASE_NATIVE || o.phase_mode > M3_PHASE_SHUFFLE) return M3_ERR_OPTION;
    if (o.ngroups < 0 || (o.ngroups > 0 && H > 0 && H % o.ngroups != 0)) return M3_ERR_OPTION;
    if (o.premix != 0 && o.premix != 1) return M3_ERR_OPTION;
    if (o.premix && !(o.norm_eps >= 0.f && o.norm_eps < 3.0e38f)) return M3_ERR_OPTION;
    const float* pg[] = {a->dB_norm_w, a->dC_norm_w, a->dB_bias, a->dC_bias, a->ddt_bias};
    for (const float* q : pg)
        if (q != nullptr && !o.premix) return M3_ERR_OPTION;
    out->groups = o.ngroups > 0 ? o.ngroups : H;
    out->opt_bc = o.premix || out->groups != H;
    out->opt_scal = o.premix != 0;
    out->opt_theta = o.phase_mode != M3_PHASE_NATIVE;
    // the option maps move rows of dstate values and of rotary pairs 4 at a
    // time, pairs through LDS
    if ((out->opt_bc || out->opt_scal || out->opt_theta) && (N > 256 || N % 8 != 0))
        return M3_ERR_UNSUPPORTED;
    // token rows of the caller's arrays (packed: one row of seqlen tokens)
    const int64_t BtL = (out->packed ? 1 : Bt) * L;
    const size_t tok = (size_t)BtL * H, es = (size_t)io_size(a->io_dtype);
    if (out->opt_bc) {
        out->be_bytes = round256(tok * R * N * es);
        out->dbe_bytes = round256(tok * R * N * 4);
    }
    if (out->opt_scal) {
        out->se_bytes = round256(tok * 4);
        out->q_bytes = round256(m3::bwd_options_gain_floats(BtL, out->groups, (int)N, (int)R) * 4);
        out->sum_bytes = round256(m3::bwd_options_partial_floats(BtL, H, out->groups, (int)N,
                                                                  (int)R) * 4);
    }
    if (out->opt_theta) out->te_bytes = round256(tok * (N / 2) * 4);
    if (out->packed) {
        const size_t tp = (size_t)Bt * out->Lp * H;
        out->px_bytes = round256(tp * R * P * es);
        out->pb_bytes = round256(tp * R * N * es);
        out->ps_bytes = round256(tp * 4);
        out->pt_bytes = round256(tp * (N / 2) * 4);
        out->gx_bytes = round256(tp * R * P * 4);
        out->gb_bytes = round256(tp * R * N * 4);
        out->gs_bytes = round256(tp * 4);
    }
    if (Bt * H == 0) return M3_OK;
    // padded: x, dy; B, C; dt, lam, A; theta; dx; dB, dC; ddt, dlam, dA; dtheta
    out->ws = out->core_ws + 2 * out->be_bytes + 2 * out->dbe_bytes + 2 * out->se_bytes +
              2 * out->te_bytes + out->q_bytes + out->sum_bytes + 2 * out->px_bytes +
              2 * out->pb_bytes + 3 * out->ps_bytes + 2 * out->pt_bytes + out->gx_bytes +
              2 * out->gb_bytes + 3 * out->gs_bytes;
    return M3_OK;
}

m3_status plan_bwd(const m3_scan_bwd_args* a, BwdPlan* out)
{
    if (a == nullptr) return M3_ERR_NULL;
    // packed sequences: the plain gradient's part is that of the padded batch
    m3_scan_bwd_args core = *a;
    const bool packed = a->opt.cu_seqlens != nullptr;
    if (packed) {
        if (a->opt.max_seqlen < 0 || a->opt.max_seqlen > a->seqlen) return M3_ERR_OPTION;
        core.seqlen = a->opt.max_seqlen;
    }
    const m3_status s = plan_bwd_core(&core, out);
    if (s != M3_OK) return s;
    out->core_ws = out->ws;
    out->packed = packed;
    out->Lp = packed ? a->opt.max_seqlen : a->seqlen;
    return plan_bwd_options(a, out);
}

m3_status plan_bwd_core(const m3_scan_bwd_args* a, BwdPlan* out)
{
    if (a == nullptr) return M3_ERR_NULL;
    const int64_t Bt = a->batch, L = a->seqlen, H = a->nheads;
    const int64_t P = a->headdim, N = a->dstate, R = a->rank;
    if (Bt < 0 || L < 0 || H < 0 || P < 1 || N < 1 || R < 1 || (N % 2) != 0) return M3_ERR_SHAPE;
    if (a->io_dtype != M3_F32 && a->io_dtype != M3_BF16) return M3_ERR_DTYPE;
    if (a->method != M3_BWD_AUTO && a->method != M3_BWD_STEP && a->method != M3_BWD_CHUNKED)
        return M3_ERR_OPTION;
    if (!bwd_method_ok(a->method, N, P, R, a->io_dtype)) return M3_ERR_UNSUPPORTED;
    const int64_t nbh = Bt * H;
    if (nbh > (int64_t)1 << 24) return M3_ERR_UNSUPPORTED;
    memset(out, 0, sizeof(*out));
    out->method = a->method;
    if (out->method == M3_BWD_AUTO)
        out->method = m3::bwd_chunked_supported(N, P, R, a->io_dtype) ? M3_BWD_CHUNKED : M3_BWD_STEP;
    if (out->method == M3_BWD_CHUNKED) {
        const int64_t Q = m3::bwd_chunk_tokens(R);
        out->nc = (L + Q - 1) / Q;
        if (nbh * out->nc >= ((int64_t)1 << 31)) return M3_ERR_UNSUPPORTED;
        const size_t NP = (size_t)N * P, es = (size_t)io_size(a->io_dtype);
        out->loc_bytes = round256((size_t)nbh * out->nc * 2 * NP * es);
        out->cs_bytes = round256((size_t)nbh * out->nc * (1 + N) * 4);
        out->st_bytes = round256((size_t)nbh * (out->nc + 1) * NP * es);
        out->chunk_bytes = round256((size_t)nbh * out->nc * 4);
        out->bh_bytes = round256((size_t)nbh * 4);
        out->ws = nbh > 0 ? out->loc_bytes + out->cs_bytes + 2 * out->st_bytes + 2 * out->chunk_bytes +
                                out->bh_bytes : 0;
        return M3_OK;
    }
    out->TB = m3::bwd_sub_steps(N);
    out->K = m3::bwd_blocks_per_checkpoint(N, P, R, a->io_dtype);
    out->parts = m3::bwd_pair_parts(N);
    const int64_t T1 = (int64_t)out->TB * out->K;
    out->nsup = (L + T1 - 1) / T1;
    const size_t units = (size_t)nbh * out->parts, ntok = (size_t)Bt * L * H;
    out->unit_floats = (size_t)P * 32;                       // 16 pairs x P of one part
    out->ck_bytes = round256(units * (size_t)(out->nsup > 0 ? out->nsup : 1) * out->unit_floats * 4);
    out->scr_bytes = round256(units * out->K * out->unit_floats * 4);
    out->dx_bytes = round256((size_t)out->parts * ntok * R * P * 4);
    out->scal_bytes = round256((size_t)out->parts * ntok * 16);
    out->dxp_bytes = round256((size_t)out->parts * nbh * R * P * 4);
    out->part_bytes = round256((size_t)nbh * 4);
    out->ws = nbh > 0 ? out->ck_bytes + out->scr_bytes + out->dx_bytes + out->scal_bytes +
                            out->dxp_bytes + out->part_bytes : 0;
    return M3_OK;
}

// Scratch memory of m3_scan_fwd_noalloc: one file-scope device array that
// each GPU the library runs on holds until the process ends.  In host code
// `scratch` is only a stand-in for the symbol; its device address on each
// device comes from hipGetSymbolAddress, taken once per device (with that
// device current) on the first call there, and only that address is used.
constexpr size_t kScratchBytes = M3_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Compute units of the current device (cached per device; 256 when unknown):
// on a launch with two workgroups per CU, the second workgroup of each CU has
// an id from here on.
int cu_count()
{
    static std::atomic<int> cache[kMaxDevices];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Device address of the scratch array on the current device, which must be
// the device of `stream` (NULL: the current device's default stream).
m3_status scratch_address(void* stream, void** out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    if (stream != nullptr) {
        int sdev = -1;
        e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev);
        if (e != hipSuccess) return hip_status(e);
        if (sdev != dev) return hip_status(hipErrorInvalidDevice);
    }
    if (dev < 0 || dev >= kMaxDevices) return hip_status(hipErrorInvalidDevice);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e);
        if (ptr == nullptr || (reinterpret_cast<uintptr_t>(ptr) & 255u) != 0)
            return hip_status(hipErrorInvalidSymbol);
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return M3_OK;
}

}  // namespace

extern "C" {

size_t m3_scan_bwd_workspace_bytes(const m3_scan_bwd_args* a)
{
    BwdPlan plan;
    if (plan_bwd(a, &plan) != M3_OK) return 0;
    return plan.ws;
}

int m3_scan_bwd_supported(int64_t dstate, int64_t headdim, int64_t rank, int32_t io_dtype)
{
    return bwd_method_ok(M3_BWD_AUTO, dstate, headdim, rank, io_dtype) ? 1 : 0;
}

int m3_scan_bwd_method_supported(int64_t dstate, int64_t headdim, int64_t rank, int32_t io_dtype,
                                 int32_t method)
{
    if (method != M3_BWD_AUTO && method != M3_BWD_STEP && method != M3_BWD_CHUNKED) return 0;
    return bwd_method_ok(method, dstate, headdim, rank, io_dtype) ? 1 : 0;
}

m3_status m3_scan_bwd(const m3_scan_bwd_args* a, void* stream)
{
    BwdPlan plan;
    const m3_status ps = plan_bwd(a, &plan);
    if (ps != M3_OK) return ps;
    const int64_t Bt = a->batch, L = a->seqlen, H = a->nheads;
    const int64_t P = a->headdim, N = a->dstate, R = a->rank;
    const int64_t nbh = Bt * H;
    if (nbh == 0) return M3_OK;
    m3::OptParams op;
    const m3_status os = check_options(a->opt, H, N, R, L, &op);
    if (os != M3_OK) return os;
    const bool zero_phase = a->opt.phase_mode == M3_PHASE_ZERO;
    const bool st_in = a->h_in || a->B_prev_in || a->x_prev_in;
    const bool st_out = a->dh_in || a->dB_prev || a->dx_prev;
    if (st_in && !(a->h_in && a->B_prev_in && a->x_prev_in)) return M3_ERR_NULL;
    if (st_out && !(a->dh_in && a->dB_prev && a->dx_prev)) return M3_ERR_NULL;
    const bool rec_g = a->dB_prev_out || a->dx_prev_out;      // output record's gradient
    if (rec_g && !(a->dB_prev_out && a->dx_prev_out)) return M3_ERR_NULL;
    // per-token A and dA are empty when there are no tokens
    if ((a->A == nullptr || a->dA == nullptr) && !(a->opt.A_per_token && L == 0)) return M3_ERR_NULL;
    if (L > 0 && (!a->x || !a->B || !a->C || !a->dt || (!zero_phase && !a->theta) || !a->lam ||
                  !a->dy || !a->dx || !a->dB || !a->dC || !a->ddt ||
                  (!zero_phase && !a->dtheta) || !a->dlam))
        return M3_ERR_NULL;
    const float* theta_in = zero_phase ? nullptr : a->theta;
    const void* ptrs[] = {a->x, a->B, a->C, a->dt, a->A, theta_in, a->lam, a->h_in,
                          a->B_prev_in, a->x_prev_in, a->dy, a->dh_out, a->dx, a->dB, a->dC,
                          a->ddt, a->dA, a->dtheta, a->dlam, a->dh_in, a->dB_prev, a->dx_prev,
                          a->dB_norm_w, a->dC_norm_w, a->dB_bias, a->dC_bias, a->ddt_bias,
                          a->dB_prev_out, a->dx_prev_out};
    for (const void* q : ptrs)
        if (q != nullptr && !aligned16(q)) return M3_ERR_ALIGN;
    const int e = io_size(a->io_dtype);
    // token arrays: batch rows x seqlen, or one row of seqlen packed tokens
    const int64_t rowsL = (plan.packed ? 1 : Bt) * L;
    const int64_t tok = rowsL * H, tokg = rowsL * plan.groups;
    const int64_t nA = a->opt.A_per_token ? tok : H;       // A and dA
    Range in[22] = {
        range_of(a->x, tok * R * P * e),         range_of(a->B, tokg * R * N * e),
        range_of(a->C, tokg * R * N * e),        range_of(a->dt, tok * 4),
        range_of(a->A, nA * 4),                  range_of(theta_in, tok * (N / 2) * 4),
        range_of(a->lam, tok * 4),               range_of(a->h_in, nbh * N * P * 4),
        range_of(a->B_prev_in, nbh * R * N * e), range_of(a->x_prev_in, nbh * R * P * e),
        range_of(a->dy, tok * R * P * e),        range_of(a->dh_out, nbh * N * P * 4),
    };
    option_ranges(a->opt, Bt, H, N, R, in + 12);
    in[20] = range_of(a->dB_prev_out, nbh * R * N * 4);
    in[21] = range_of(a->dx_prev_out, nbh * R * P * 4);
    const Range out[] = {
        range_of(a->dx, tok * R * P * 4),        range_of(a->dB, tokg * R * N * 4),
        range_of(a->dC, tokg * R * N * 4),       range_of(a->ddt, tok * 4),
        range_of(a->dA, nA * 4),                 range_of(a->dtheta, tok * (N / 2) * 4),
        range_of(a->dlam, tok * 4),              range_of(a->dh_in, nbh * N * P * 4),
        range_of(a->dB_prev, nbh * R * N * 4),   range_of(a->dx_prev, nbh * R * P * 4),
        range_of(a->dB_norm_w, N * 4),           range_of(a->dC_norm_w, N * 4),
        range_of(a->dB_bias, H * R * N * 4),     range_of(a->dC_bias, H * R * N * 4),
        range_of(a->ddt_bias, H * 4),            range_of(a->workspace, (int64_t)plan.ws),
    };
    const int nout = sizeof(out) / sizeof(out[0]);
    for (const Range& o : out)
        for (const Range& i : in)
            if (overlaps(o, i)) return M3_ERR_ALIAS;
    for (int i = 0; i < nout; ++i)
        for (int j = i + 1; j < nout; ++j)
            if (overlaps(out[i], out[j])) return M3_ERR_ALIAS;
    if (a->workspace == nullptr || a->workspace_bytes < plan.ws) return M3_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(a->workspace) & 255u) != 0) return M3_ERR_ALIGN;
    const hipStream_t st = static_cast<hipStream_t>(stream);

    // With options the plain gradient runs on the inputs as the recurrence
    // uses them (materialised behind its workspace) and writes the gradients
    // with respect to those there; the option maps carry them back after it.
    const void *Bx = a->B, *Cx = a->C;
    const float *dtx = a->dt, *lamx = a->lam, *thx = a->theta;
    float *dBx = a->dB, *dCx = a->dC, *dthx = a->dtheta;
    m3::BwdOptParams bo;
    memset(&bo, 0, sizeof(bo));
    const bool opts = plan.opt_bc || plan.opt_scal || plan.opt_theta;
    char* w = static_cast<char*>(a->workspace) + plan.core_ws;
    auto take = [&w](size_t bytes) { char* q = bytes ? w : nullptr; w += bytes; return q; };
    if (opts) {
        bo.B = a->B; bo.C = a->C; bo.dt = a->dt; bo.lam = a->lam; bo.theta = theta_in;
        bo.opt = op;
        bo.Be = take(plan.be_bytes);
        bo.Ce = take(plan.be_bytes);
        float* dBe = reinterpret_cast<float*>(take(plan.dbe_bytes));
        float* dCe = reinterpret_cast<float*>(take(plan.dbe_bytes));
        bo.dBe = dBe; bo.dCe = dCe;
        bo.dte = reinterpret_cast<float*>(take(plan.se_bytes));
        bo.lame = reinterpret_cast<float*>(take(plan.se_bytes));
        bo.thetae = reinterpret_cast<float*>(take(plan.te_bytes));
        float* dthe = reinterpret_cast<float*>(take(plan.te_bytes));
        bo.dthetae = dthe;
        bo.qpart = reinterpret_cast<float*>(take(plan.q_bytes));
        bo.part = reinterpret_cast<float*>(take(plan.sum_bytes));
        bo.dB = a->dB; bo.dC = a->dC; bo.ddt = a->ddt; bo.dlam = a->dlam; bo.dtheta = a->dtheta;
        bo.dBw = a->dB_norm_w; bo.dCw = a->dC_norm_w; bo.dBb = a->dB_bias; bo.dCb = a->dC_bias;
        bo.ddtb = a->ddt_bias;
        bo.BtL = rowsL; bo.H = H; bo.G = plan.groups; bo.N = (int)N; bo.R = (int)R;
        if (plan.opt_bc) { Bx = bo.Be; Cx = bo.Ce; dBx = dBe; dCx = dCe; }
        if (plan.opt_scal) { dtx = bo.dte; lamx = bo.lame; }
        if (plan.opt_theta) { thx = bo.thetae; dthx = dthe; }
        const hipError_t e0 = m3::launch_bwd_options_pre(bo, a->io_dtype, st);
        if (e0 != hipSuccess) return hip_status(e0);
    }

    // The plain gradient's operands: as above, or (packed sequences) those
    // moved into a padded batch of max_seqlen tokens per sequence, zero past
    // each sequence's end -- a zero step dt_t makes a padding step the
    // identity (no decay, rotation or input), so the padded batch has the
    // packed sequences' gradients.
    const void *xc = a->x, *Bc = Bx, *Cc = Cx, *dyc = a->dy;
    const float *dtc = dtx, *lamc = lamx, *thc = thx, *Ac = a->A;
    float *dxc = a->dx, *dBc = dBx, *dCc = dCx, *ddtc = a->ddt, *dlamc = a->dlam, *dthc = dthx;
    float* dAc = a->dA;
    const int64_t Lc = plan.Lp;
    m3::PackParams un;
    memset(&un, 0, sizeof(un));
    if (plan.packed) {
        m3::PackParams pk;
        memset(&pk, 0, sizeof(pk));
        pk.cu = a->opt.cu_seqlens; pk.nseq = Bt; pk.T = L; pk.maxL = plan.Lp;
        un = pk;
        un.unpack = 1;
        const int wx = (int)(H * R * P * e / 4), wb = (int)(H * R * N * e / 4), ws = (int)H;
        const int wt = (int)(H * (N / 2)), wgx = (int)(H * R * P), wgb = (int)(H * R * N);
        auto move = [](m3::PackParams& q, const void* s, void* d, int words) {
            q.src[q.n] = s; q.dst[q.n] = d; q.words[q.n] = words; ++q.n;
        };
        void* px = take(plan.px_bytes); void* pdy = take(plan.px_bytes);
        void* pB = take(plan.pb_bytes); void* pC = take(plan.pb_bytes);
        float* pdt = reinterpret_cast<float*>(take(plan.ps_bytes));
        float* plam = reinterpret_cast<float*>(take(plan.ps_bytes));
        float* pA = reinterpret_cast<float*>(take(plan.ps_bytes));
        float* pth = reinterpret_cast<float*>(take(plan.pt_bytes));
        float* gth = reinterpret_cast<float*>(take(plan.pt_bytes));
        float* gx = reinterpret_cast<float*>(take(plan.gx_bytes));
        float* gB = reinterpret_cast<float*>(take(plan.gb_bytes));
        float* gC = reinterpret_cast<float*>(take(plan.gb_bytes));
        float* gdt = reinterpret_cast<float*>(take(plan.gs_bytes));
        float* glam = reinterpret_cast<float*>(take(plan.gs_bytes));
        float* gA = reinterpret_cast<float*>(take(plan.gs_bytes));
        move(pk, a->x, px, wx); move(pk, a->dy, pdy, wx);
        move(pk, Bx, pB, wb); move(pk, Cx, pC, wb);
        move(pk, dtx, pdt, ws); move(pk, lamx, plam, ws); move(pk, thx, pth, wt);
        move(un, gx, a->dx, wgx); move(un, gB, dBx, wgb); move(un, gC, dCx, wgb);
        move(un, gdt, a->ddt, ws); move(un, glam, a->dlam, ws); move(un, gth, dthx, wt);
        if (a->opt.A_per_token) { move(pk, a->A, pA, ws); move(un, gA, a->dA, ws); Ac = pA; dAc = gA; }
        xc = px; dyc = pdy; Bc = pB; Cc = pC; dtc = pdt; lamc = plam; thc = pth;
        dxc = gx; dBc = gB; dCc = gC; ddtc = gdt; dlamc = glam; dthc = gth;
        const hipError_t e1 = m3::launch_bwd_pack(pk, st);
        if (e1 != hipSuccess) return hip_status(e1);
    }

    hipError_t err;
    if (plan.method == M3_BWD_CHUNKED) {
        m3::BcParams q;
        memset(&q, 0, sizeof(q));
        q.x = xc; q.B = Bc; q.C = Cc; q.dy = dyc;
        q.dt = dtc; q.A = Ac; q.theta = thc; q.lam = lamc;
        q.h_in = a->h_in; q.Bp_in = a->B_prev_in; q.xp_in = a->x_prev_in; q.dh_out = a->dh_out;
        q.dx = dxc; q.dB = dBc; q.dC = dCc; q.ddt = ddtc; q.dtheta = dthc;
        q.dlam = dlamc; q.dh_in = a->dh_in; q.dBp = a->dB_prev; q.dxp = a->dx_prev; q.dA = dAc;
        char* w = static_cast<char*>(a->workspace);
        q.loc = w;
        w += plan.loc_bytes;
        q.csum = reinterpret_cast<float*>(w);
        w += plan.cs_bytes;
        q.gst = w;
        w += plan.st_bytes;
        q.dgst = w;
        w += plan.st_bytes;
        q.dA_part = reinterpret_cast<float*>(w);
        w += plan.chunk_bytes;
        q.dw_last = reinterpret_cast<float*>(w);
        w += plan.chunk_bytes;
        q.dA_bh = reinterpret_cast<float*>(w);
        q.a_tok = a->opt.A_per_token;
        q.L = Lc; q.H = H; q.N = (int)N; q.P = (int)P; q.R = (int)R;
        q.nbh = (int)nbh;
        q.nc = (int)plan.nc;
#if M3_TIMELINE
        q.tl = g_timeline;
        q.tl_rows = g_timeline_rows;
#endif
        err = m3::launch_bwd_chunked(q, a->io_dtype, st);
    } else {
        m3::BwdParams p;
        memset(&p, 0, sizeof(p));
        p.x = xc; p.B = Bc; p.C = Cc; p.dy = dyc;
        p.dt = dtc; p.A = Ac; p.theta = thc; p.lam = lamc;
        p.h_in = a->h_in; p.Bp_in = a->B_prev_in; p.xp_in = a->x_prev_in; p.dh_out = a->dh_out;
        p.dx = dxc; p.dB = dBc; p.dC = dCc; p.ddt = ddtc; p.dtheta = dthc;
        p.dlam = dlamc; p.dh_in = a->dh_in; p.dBp = a->dB_prev; p.dxp = a->dx_prev;
        char* ws = static_cast<char*>(a->workspace);
        p.ckpt = reinterpret_cast<float*>(ws);
        ws += plan.ck_bytes;
        p.scr = reinterpret_cast<float*>(ws);
        ws += plan.scr_bytes;
        p.dx_part = reinterpret_cast<float*>(ws);
        ws += plan.dx_bytes;
        p.scal = reinterpret_cast<float*>(ws);
        ws += plan.scal_bytes;
        p.dxprev_part = reinterpret_cast<float*>(ws);
        ws += plan.dxp_bytes;
        p.dA_part = reinterpret_cast<float*>(ws);
        p.a_tok = a->opt.A_per_token;
        p.dAt = dAc;
        p.L = Lc; p.H = H; p.N = (int)N; p.P = (int)P; p.R = (int)R;
        p.ntok = Bt * Lc * H;
        p.nbh = (int)nbh;
        p.parts = plan.parts;
        p.TB = plan.TB; p.K = plan.K;
        err = m3::launch_bwd(p, a->io_dtype, a->dA, st);
    }
    if (err == hipSuccess && plan.packed) err = m3::launch_bwd_pack(un, st);
    if (err == hipSuccess && rec_g) {
        // the output record's (B_L, x_L) are the last token's B (as used) and x
        m3::RecGradParams rg;
        memset(&rg, 0, sizeof(rg));
        rg.dBL = a->dB_prev_out; rg.dxL = a->dx_prev_out;
        rg.dB = dBx; rg.dx = a->dx; rg.dBp = a->dB_prev; rg.dxp = a->dx_prev;
        rg.cu = a->opt.cu_seqlens;
        rg.max_len = a->opt.max_seqlen;
        rg.batch = Bt; rg.L = L; rg.H = H; rg.N = (int)N; rg.P = (int)P; rg.R = (int)R;
        err = m3::launch_bwd_record_grad(rg, st);
    }
    if (err != hipSuccess || !opts) return hip_status(err);
    return hip_status(m3::launch_bwd_options_post(bo, a->io_dtype, st));
}


int m3_abi_version(void) { return M3_ABI_VERSION; }

#if M3_TIMELINE
// Instrumented builds only (not part of the ABI): the device buffer of
// per-wave phase stamps for the following scan calls (rows of kTlSlots
// 64-bit entries, one per wave of both passes' grids), or NULL.  A call whose
// waves need more rows than `rows` runs without stamps.
void m3_timeline_buffer(void* buf, int64_t rows)
{
    g_timeline = static_cast<unsigned long long*>(buf);
    g_timeline_rows = buf != nullptr ? rows : 0;
}
#endif

int m3_last_hip_error(void) { return g_last_hip_error; }

const char* m3_status_string(m3_status s)
{
    switch (s) {
    case M3_OK: return "ok";
    case M3_ERR_NULL: return "required pointer is NULL or state record incomplete";
    case M3_ERR_SHAPE: return "invalid shape (negative or zero size, odd dstate)";
    case M3_ERR_UNSUPPORTED: return "dstate/headdim/rank/chunk outside the compiled set";
    case M3_ERR_DTYPE: return "unknown io dtype";
    case M3_ERR_ALIGN: return "pointer not 16-byte aligned";
    case M3_ERR_WORKSPACE: return "workspace missing or too small";
    case M3_ERR_ALIAS: return "output overlaps an input";
    case M3_ERR_HIP: return "HIP call failed";
    case M3_ERR_OPTION: return "option out of range (groups, phase mode, premix, eps)";
    case M3_ERR_SCRATCH: return "call needs more scratch than M3_NOALLOC_SCRATCH_BYTES";
    }
    return "unknown status";
}

int m3_scan_supported(int64_t dstate, int64_t headdim, int64_t rank, int32_t chunk,
                      int32_t io_dtype)
{
    if (io_dtype != M3_F32 && io_dtype != M3_BF16) return 0;
    if (dstate < 2 || headdim < 1 || rank < 1 || chunk < 0) return 0;
    return pick_scan(io_dtype, dstate, rank, headdim, chunk, 0, 1 << 20) != nullptr;
}

int m3_decode_supported(int64_t dstate, int64_t headdim, int64_t rank, int32_t io_dtype)
{
    return m3::decode_supported(dstate, headdim, rank, io_dtype) ? 1 : 0;
}

size_t m3_scan_workspace_bytes(const m3_scan_args* a)
{
    ScanPlan plan;
    if (plan_scan(a, &plan) != M3_OK) return 0;
    return plan.ws;
}

}  // extern "C"

namespace {

// Every argument check of m3_scan_fwd (no HIP call).  Without `own_ws` the
// workspace is the library's scratch array: the caller's workspace fields are
// not used and the plan's size is checked against the array instead.
m3_status scan_check(const m3_scan_args* a, bool own_ws, ScanPlan* planp, m3::OptParams* opp)
{
    ScanPlan& plan = *planp;
    const m3_status ps = plan_scan(a, &plan);
    if (ps != M3_OK) return ps;
    const int64_t Bt = a->batch, L = a->seqlen, H = a->nheads;
    const int64_t P = a->headdim, N = a->dstate, R = a->rank;
    const int64_t nbh = Bt * H;
    if (nbh == 0) return M3_OK;

    m3::OptParams& op = *opp;
    const m3_status os = check_options(a->opt, H, N, R, L, &op);
    if (os != M3_OK) return os;
    const bool packed = a->opt.cu_seqlens != nullptr;
    const bool st_in = a->h_in || a->B_prev_in || a->x_prev_in;
    const bool st_out = a->h_out || a->B_prev_out || a->x_prev_out;
    if (st_in && !(a->h_in && a->B_prev_in && a->x_prev_in)) return M3_ERR_NULL;
    if (st_out && !(a->h_out && a->B_prev_out && a->x_prev_out)) return M3_ERR_NULL;
    if (a->A == nullptr && !(a->opt.A_per_token && L == 0)) return M3_ERR_NULL;
    const bool need_theta = a->opt.phase_mode != M3_PHASE_ZERO;
    if (L > 0 && (!a->x || !a->B || !a->C || !a->dt || (need_theta && !a->theta) || !a->lam || !a->y))
        return M3_ERR_NULL;
    const void* theta = need_theta ? a->theta : nullptr;

    const void* ptrs[] = {a->x, a->B, a->C, a->dt, a->A, theta, a->lam, a->h_in,
                          a->B_prev_in, a->x_prev_in, a->y, a->h_out, a->B_prev_out,
                          a->x_prev_out};
    for (const void* q : ptrs)
        if (q != nullptr && !aligned16(q)) return M3_ERR_ALIGN;

    const int e = io_size(a->io_dtype);
    const int64_t tok = (packed ? 1 : Bt) * L * H;             // token arrays: rows x heads
    const int64_t tokg = (packed ? 1 : Bt) * L * op.groups;
    Range in[18] = {
        range_of(a->x, tok * R * P * e),         range_of(a->B, tokg * R * N * e),
        range_of(a->C, tokg * R * N * e),        range_of(a->dt, tok * 4),
        range_of(a->A, (a->opt.A_per_token ? tok : H) * 4),
        range_of(theta, tok * (N / 2) * 4),
        range_of(a->lam, tok * 4),               range_of(a->h_in, nbh * N * P * 4),
        range_of(a->B_prev_in, nbh * R * N * e), range_of(a->x_prev_in, nbh * R * P * e),
    };
    option_ranges(a->opt, Bt, H, N, R, in + 10);
    const Range out[] = {
        range_of(a->y, tok * R * P * e),         range_of(a->h_out, nbh * N * P * 4),
        range_of(a->B_prev_out, nbh * R * N * e), range_of(a->x_prev_out, nbh * R * P * e),
        range_of(own_ws ? a->workspace : nullptr, (int64_t)plan.ws),
        range_of(a->opt.phase_out, nbh * (N / 2) * 4),
    };
    const int nout = sizeof(out) / sizeof(out[0]);
    // out[1..3] may be exactly the input record in[7..9] (updated in place);
    // any other overlap is rejected.
    for (int k = 0; k < nout; ++k) {
        for (int i = 0; i < 18; ++i) {
            if (plan.rec_alias && k >= 1 && k <= 3 && i >= 7 && i <= 9) continue;
            if (overlaps(out[k], in[i])) return M3_ERR_ALIAS;
        }
    }
    for (int i = 0; i < nout; ++i)
        for (int j = i + 1; j < nout; ++j)
            if (overlaps(out[i], out[j])) return M3_ERR_ALIAS;
    if (plan.ws > 0 && own_ws) {
        if (a->workspace == nullptr || a->workspace_bytes < plan.ws) return M3_ERR_WORKSPACE;
        if ((reinterpret_cast<uintptr_t>(a->workspace) & 255u) != 0) return M3_ERR_ALIGN;
    }
    if (plan.ws > kScratchBytes && !own_ws) return M3_ERR_SCRATCH;
    return M3_OK;
}

// The launches of a checked m3_scan_fwd call, with workspace `ws`.
m3_status scan_launch(const m3_scan_args* a, const ScanPlan& plan, const m3::OptParams& op, void* ws,
                      void* stream)
{
    const int64_t Bt = a->batch, L = a->seqlen, H = a->nheads;
    const int64_t P = a->headdim, N = a->dstate, R = a->rank;
    const int64_t nbh = Bt * H;
    if (nbh == 0) return M3_OK;
    const int e = io_size(a->io_dtype);
    const void* theta = a->opt.phase_mode != M3_PHASE_ZERO ? a->theta : nullptr;

    m3::ScanParams p;
    memset(&p, 0, sizeof(p));
    p.x = a->x; p.B = a->B; p.C = a->C;
    p.dt = a->dt; p.A = a->A; p.theta = a->theta; p.lam = a->lam;
    p.h_in = a->h_in; p.Bp_in = a->B_prev_in; p.xp_in = a->x_prev_in;
    if (plan.rec_alias) {
        // copy the input record to the workspace; the kernels read the copy
        char* snap = static_cast<char*>(ws) + plan.snap_off;
        const hipStream_t s0 = static_cast<hipStream_t>(stream);
        const size_t bx = (size_t)nbh * R * P * e;
        hipError_t ec = hipMemcpyAsync(snap, a->h_in, plan.snap_h, hipMemcpyDeviceToDevice, s0);
        if (ec == hipSuccess)
            ec = hipMemcpyAsync(snap + plan.snap_h, a->B_prev_in, (size_t)nbh * R * N * e,
                                hipMemcpyDeviceToDevice, s0);
        if (ec == hipSuccess)
            ec = hipMemcpyAsync(snap + plan.snap_h + plan.snap_b, a->x_prev_in, bx,
                                hipMemcpyDeviceToDevice, s0);
        if (ec != hipSuccess) return hip_status(ec);
        p.h_in = reinterpret_cast<const float*>(snap);
        p.Bp_in = snap + plan.snap_h;
        p.xp_in = snap + plan.snap_h + plan.snap_b;
    }
    p.y = a->y; p.h_out = a->h_out; p.Bp_out = a->B_prev_out; p.xp_out = a->x_prev_out;
    p.ws = static_cast<float*>(ws);
    p.opt = op;
    p.theta = static_cast<const float*>(theta);
    p.batch = Bt; p.L = L; p.H = H; p.P = P;
    p.p_split = plan.p_split;
    p.nbh = (int)nbh;
    p.nseg = plan.nseg;
    p.seg_chunks = plan.seg_chunks;
    p.nslots = plan.nslots;
    p.young_from = cu_count();
#if M3_TIMELINE
    p.tl = g_timeline;
    p.tl_rows = g_timeline_rows;
#endif
    const hipError_t e1 = plan.v->fn(p, static_cast<hipStream_t>(stream));
    if (e1 != hipSuccess || a->opt.phase_out == nullptr) return hip_status(e1);
    m3::PhaseParams q;
    memset(&q, 0, sizeof(q));
    q.dt = a->dt;
    q.theta = static_cast<const float*>(theta);
    q.opt = op;
    q.rows = Bt; q.L = L; q.H = H; q.NPR = (int)(N / 2);
    q.nblk = plan.phase_blocks;
    q.part = reinterpret_cast<double*>(static_cast<char*>(ws) + plan.phase_off);
    return hip_status(m3::launch_phase_accumulate(q, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

m3_status m3_scan_fwd(const m3_scan_args* a, void* stream)
{
    ScanPlan plan;
    m3::OptParams op;
    const m3_status st = scan_check(a, true, &plan, &op);
    if (st != M3_OK) return st;
    return scan_launch(a, plan, op, a->workspace, stream);
}

m3_status m3_scan_fwd_noalloc(const m3_scan_args* a, void* stream)
{
    ScanPlan plan;
    m3::OptParams op;
    const m3_status st = scan_check(a, false, &plan, &op);
    if (st != M3_OK) return st;
    void* ws = nullptr;
    if (plan.ws > 0 && a->batch * a->nheads > 0) {
        const m3_status ss = scratch_address(stream, &ws);
        if (ss != M3_OK) return ss;
    }
    return scan_launch(a, plan, op, ws, stream);
}

m3_status m3_decode_step(const m3_decode_args* a, void* stream)
{
    if (a == nullptr) return M3_ERR_NULL;
    const int64_t Bt = a->batch, H = a->nheads, P = a->headdim, N = a->dstate, R = a->rank;
    if (Bt < 0 || H < 0 || P < 1 || N < 1 || R < 1 || (N % 2) != 0) return M3_ERR_SHAPE;
    if (a->io_dtype != M3_F32 && a->io_dtype != M3_BF16) return M3_ERR_DTYPE;
    if (!m3::decode_supported(N, P, R, a->io_dtype)) return M3_ERR_UNSUPPORTED;
    const int64_t nbh = Bt * H;
    if (nbh > (int64_t)1 << 30) return M3_ERR_UNSUPPORTED;
    m3::OptParams op;
    const m3_status os = check_options(a->opt, H, N, R, -1, &op);
    if (os != M3_OK) return os;
    if (nbh == 0) return M3_OK;
    const void* theta = a->opt.phase_mode != M3_PHASE_ZERO ? a->theta : nullptr;
    const void* ptrs[] = {a->x, a->B, a->C, a->dt, a->A, theta, a->lam,
                          a->h, a->B_prev, a->x_prev, a->y};
    for (int i = 0; i < 11; ++i)
        if (ptrs[i] == nullptr && !(i == 5 && a->opt.phase_mode == M3_PHASE_ZERO)) return M3_ERR_NULL;
    for (const void* q : ptrs)
        if (q != nullptr && !aligned16(q)) return M3_ERR_ALIGN;
    const int e = io_size(a->io_dtype);
    const int64_t nbg = Bt * op.groups;
    Range in[15] = {
        range_of(a->x, nbh * R * P * e), range_of(a->B, nbg * R * N * e),
        range_of(a->C, nbg * R * N * e), range_of(a->dt, nbh * 4),
        range_of(a->A, (a->opt.A_per_token ? nbh : H) * 4),
        range_of(theta, nbh * (N / 2) * 4), range_of(a->lam, nbh * 4),
    };
    option_ranges(a->opt, Bt, H, N, R, in + 7);
    const Range rec[] = {
        range_of(a->h, nbh * N * P * 4), range_of(a->B_prev, nbh * R * N * e),
        range_of(a->x_prev, nbh * R * P * e),
    };
    const Range y = range_of(a->y, nbh * R * P * e);
    const Range ph = range_of(a->opt.phase_out, nbh * (N / 2) * 4);
    for (const Range& r : rec) {
        if (overlaps(y, r) || overlaps(ph, r)) return M3_ERR_ALIAS;
        for (const Range& i : in)
            if (overlaps(r, i)) return M3_ERR_ALIAS;
    }
    for (const Range& i : in)
        if (overlaps(y, i) || overlaps(ph, i)) return M3_ERR_ALIAS;
    if (overlaps(y, ph)) return M3_ERR_ALIAS;
    for (int i = 0; i < 3; ++i)
        for (int j = i + 1; j < 3; ++j)
            if (overlaps(rec[i], rec[j])) return M3_ERR_ALIAS;

    m3::DecodeParams p;
    p.x = a->x; p.B = a->B; p.C = a->C;
    p.dt = a->dt; p.A = a->A; p.theta = static_cast<const float*>(theta); p.lam = a->lam;
    p.opt = op;
    p.h = a->h; p.Bp = a->B_prev; p.xp = a->x_prev; p.y = a->y;
    p.H = H; p.N = (int)N; p.P = (int)P; p.R = (int)R; p.nbh = nbh;
    return hip_status(m3::launch_decode(p, a->io_dtype, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
