// Internal (non-ABI) declarations shared by the libm3scan translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace m3 {

struct ScanParams;

// Options of both entry points, resolved for the kernels.
struct OptParams {
    int64_t groups;        // B/C head groups (nheads when not grouped)
    int a_tok;             // A per (batch, token, head) instead of per head
    int phase;             // m3_phase_mode
    const int* perm;       // [N/2] pair permutation (shuffle only)
    int premix;            // dt/lam raw, B/C RMS-normalised with gains and biases
    float eps;
    const float *Bw, *Cw;  // [N] or NULL (ones)
    const float *Bb, *Cb;  // [H, R, N] or NULL (zeros)
    const float *dtb;      // [H] or NULL (zeros)
    const int* cu;         // [batch + 1] packed-sequence offsets, or NULL (dense batch)
    int64_t max_len;       // longest packed sequence
    const float* phase_in; // [batch, H, N/2] accumulated angle before the call, or NULL (zero)
    float* phase_out;      // [batch, H, N/2] accumulated angle after the call, or NULL
};

struct DecodeParams {
    const void *x, *B, *C;
    const float *dt, *A, *theta, *lam;
    float *h;
    void *Bp, *xp;
    void *y;
    int64_t H;
    int N, P, R;
    int64_t nbh;
    OptParams opt;
};

// Gradient of the scan (reverse-time recurrence with checkpointed recompute).
struct BwdParams {
    const void *x, *B, *C, *dy;
    const float *dt, *A, *theta, *lam;
    const float *h_in;
    const void *Bp_in, *xp_in;
    const float *dh_out;
    float *dx, *dB, *dC, *ddt, *dtheta, *dlam;
    float *dh_in, *dBp, *dxp;
    float *ckpt;      // [B*H*parts][nsup][32 P] states every T1 steps
    float *scr;       // [B*H*parts][K][32 P] sub-block start states of one superblock
    float *dx_part;   // [parts][B*L*H][R][P] each pair part's share of dX
    float *scal;      // [parts][B*L*H][4] each part's dalpha, dbeta, dgamma, theta.dphi
    float *dxprev_part;  // [parts][B*H][R][P]
    float *dA_part;   // [B*H] this unit's share of dA
    float *dAt;       // [B*L*H] dA per token (a_tok), else unused
    int a_tok;        // A given per (batch, token, head)
    int64_t L, H, ntok;
    int N, P, R;
    int nbh, parts;   // (b, h) units; pair parts (16 pairs) per unit
    int TB, K;        // sub-block steps, sub-blocks per superblock (T1 = K * TB)
};

bool bwd_supported(int64_t N, int64_t P, int64_t R, int io_dtype);
int bwd_sub_steps(int64_t N);
int bwd_blocks_per_checkpoint(int64_t N, int64_t P, int64_t R, int io_dtype);
int bwd_pair_parts(int64_t N);
hipError_t launch_bwd(const BwdParams& p, int io_dtype, float* dA, hipStream_t stream);

// Gradient of the scan in chunked (SSD) form: per-chunk local sums, a scan of
// the chunk-boundary states forward and of their adjoints backward, then
// every gradient of a chunk from its two boundary states on matrix cores.
struct BcParams {
    const void *x, *B, *C, *dy;
    const float *dt, *A, *theta, *lam;
    const float *h_in;
    const void *Bp_in, *xp_in;
    const float *dh_out;
    float *dx, *dB, *dC, *ddt, *dtheta, *dlam;
    float *dh_in, *dBp, *dxp, *dA;
    // Chunk-boundary arrays, stored in the io type (bf16 or float32):
    void *loc;        // [B*H][nc][2][N][P] chunk-local state and adjoint sums
    float *csum;      // [B*H][nc][1 + N] e^{Lam_tot}, then cos, sin of Phi_tot per pair
    void *gst;        // [B*H][nc + 1][N][P] state at each chunk start (last slot unused)
    void *dgst;       // [B*H][nc + 1][N][P] adjoint of each chunk's end state, then of the initial state
    float *dA_part;   // [B*H][nc] each chunk's share of dA
    float *dw_last;   // [B*H][nc] gradient of the look-ahead weight of a chunk's last token
    float *dA_bh;     // [B*H] each unit's share of dA
    int a_tok;        // A (and dA) per (batch, token, head)
    int64_t L, H;
    int N, P, R;
    int nbh, nc;      // (b, h) units; chunks per unit
    unsigned long long* tl;   // per-wave phase stamps (instrumented builds only), else null
    int64_t tl_rows;          // rows that tl holds
};

bool bwd_chunked_supported(int64_t N, int64_t P, int64_t R, int io_dtype);
int bwd_chunk_tokens(int64_t R);
hipError_t launch_bwd_chunked(const BcParams& p, int io_dtype, hipStream_t stream);

// Options of the scan gradient, as maps around the plain gradient: the
// inputs materialised as the recurrence uses them before it (B, C repeated
// per head and pre-mixed, theta after the phase map, dt and lam through
// softplus and sigmoid), the gradients carried back to the caller's inputs
// and the pre-mixer's parameters after it.
struct BwdOptParams {
    const void *B, *C;             // caller's [B*L*G*R][N] io type
    const float *dt, *lam, *theta; // caller's (raw with the pre-mixer)
    OptParams opt;
    void *Be, *Ce;                 // [B*L*H*R][N] io type (groups or pre-mixer)
    float *dte, *lame;             // [B*L*H] (pre-mixer)
    float *thetae;                 // [B*L*H][N/2] (phase map)
    const float *dBe, *dCe;        // gradients with respect to Be, Ce
    const float *dthetae;          // gradient with respect to thetae
    float *dB, *dC;                // caller's [B*L*G*R][N]
    float *ddt, *dlam;             // caller's, mapped in place (pre-mixer)
    float *dtheta;                 // caller's or NULL
    float *dBw, *dCw, *dBb, *dCb, *ddtb;   // parameter gradients or NULL
    float *qpart;                  // [2][row blocks][N] gain-gradient partials (workspace)
    float *part;                   // column-sum partials (workspace)
    int64_t BtL, H, G;
    int N, R;
};
// Packed sequences around the gradient: token rows moved between the packed
// arrays ([T] token rows, sequence s = rows cu[s] .. cu[s+1]-1) and a padded
// batch ([nseq][maxL] token rows, zero past each sequence's end).
struct PackParams {
    const int* cu;            // [nseq + 1], clamped on the device
    int64_t nseq, T, maxL;
    int n;                    // arrays moved by one launch
    int unpack;               // 0: packed -> padded; 1: padded -> packed (real tokens only)
    const void* src[8];
    void* dst[8];
    int words[8];             // 4-byte words per token row
};
hipError_t launch_bwd_pack(const PackParams& p, hipStream_t stream);

// The gradient of the output record (B_L, x_L) added to each sequence's last
// token's dB (per head) and dx, or to the input record's dB_prev, dx_prev for a
// sequence without tokens.
struct RecGradParams {
    const float *dBL, *dxL;   // [B*H][R][N], [B*H][R][P]
    float *dB, *dx;           // token gradients [rows][L or T][H][R][N or P]
    float *dBp, *dxp;         // input record gradients, or NULL
    const int* cu;            // packed: [batch + 1], else NULL
    int64_t max_len;          // packed: the length cap (max_seqlen)
    int64_t batch, L, H;      // L: tokens per row (dense) or the packed length
    int N, P, R;
};
hipError_t launch_bwd_record_grad(const RecGradParams& p, hipStream_t stream);
size_t bwd_options_partial_floats(int64_t BtL, int64_t H, int64_t G, int N, int R);
size_t bwd_options_gain_floats(int64_t BtL, int64_t G, int N, int R);
hipError_t launch_bwd_options_pre(const BwdOptParams& p, int io_dtype, hipStream_t stream);
hipError_t launch_bwd_options_post(const BwdOptParams& p, int io_dtype, hipStream_t stream);

// Accumulated rotation angle of a scan: per (row, head, 64-token block) the
// float64 partial sums of dt theta per pair into `part`, then per (row, head,
// pair) their sum in block order plus phase_in, reduced into [-pi, pi).
struct PhaseParams {
    const float *dt, *theta;
    OptParams opt;
    int64_t rows, L, H;    // batch rows (sequences when packed), token rows per sequence bound
    int NPR;
    int64_t nblk;          // 64-token blocks per sequence
    double* part;          // [rows * H][nblk][NPR]
};
constexpr int kPhaseBlock = 64;
hipError_t launch_phase_accumulate(const PhaseParams& p, hipStream_t stream);

bool decode_supported(int64_t N, int64_t P, int64_t R, int io_dtype);
hipError_t launch_decode(const DecodeParams& p, int io_dtype, hipStream_t stream);

typedef hipError_t (*scan_launcher)(const ScanParams&, hipStream_t);
typedef size_t (*scan_ws_fn)(int64_t nbh, int64_t P, int nseg);

// One compiled instantiation of the fused scan kernel.
struct ScanVariant {
    int io;        // m3_dtype
    int N, R, Q, PS, NW;
    int occ;       // workgroups per compute unit the launch bounds aim for
    size_t lds_bytes;
    scan_launcher fn;
    scan_ws_fn ws_bytes;   // workspace bytes for a segmented call
    int pm;                // 1: used only with the pre-mixer, and preferred then
};

// Tables defined by the instantiation units (host functions, so that the
// device pass never sees host function pointers).
const ScanVariant* scan_variants_f32(int* count);
const ScanVariant* scan_variants_bf16a(int* count);
const ScanVariant* scan_variants_bf16b(int* count);

}  // namespace m3
