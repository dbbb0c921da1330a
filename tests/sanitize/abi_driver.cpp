// Driver for the host side of libm3scan (argument validation, variant
// selection, workspace sizing: csrc/m3_abi.hip) built with AddressSanitizer
// and UndefinedBehaviorSanitizer on the host code.  Every call here is
// rejected or sized before any HIP call -- fake device pointers are never
// dereferenced -- so it runs without a GPU.  Sizes include extreme values
// (2^40 tokens, 2^31 heads) so that any overflow in the size arithmetic is
// caught by the sanitizer.  Exit status 0: every check held.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "m3scan.h"

static int failures = 0;
#define CHECK(c, ...)                                      \
    do {                                                   \
        if (!(c)) {                                        \
            ++failures;                                    \
            fprintf(stderr, "check failed (line %d): ", __LINE__); \
            fprintf(stderr, __VA_ARGS__);                  \
            fprintf(stderr, "\n");                         \
        }                                                  \
    } while (0)

static const uintptr_t FAKE = 0x7F0000000000ull;
static void* fake(int i, int off = 0) { return reinterpret_cast<void*>(FAKE + ((uintptr_t)i << 32) + off); }

static m3_scan_args scan_args()
{
    m3_scan_args a;
    memset(&a, 0, sizeof(a));
    a.batch = 2; a.seqlen = 10; a.nheads = 3; a.headdim = 32; a.dstate = 64; a.rank = 1;
    a.io_dtype = M3_BF16;
    a.x = fake(0); a.B = fake(1); a.C = fake(2);
    a.dt = (const float*)fake(3); a.A = (const float*)fake(4); a.theta = (const float*)fake(5);
    a.lam = (const float*)fake(6); a.y = fake(7);
    return a;
}

static m3_decode_args decode_args()
{
    m3_decode_args a;
    memset(&a, 0, sizeof(a));
    a.batch = 4; a.nheads = 2; a.headdim = 64; a.dstate = 128; a.rank = 4; a.io_dtype = M3_BF16;
    a.x = fake(0); a.B = fake(1); a.C = fake(2);
    a.dt = (const float*)fake(3); a.A = (const float*)fake(4); a.theta = (const float*)fake(5);
    a.lam = (const float*)fake(6); a.h = (float*)fake(7); a.B_prev = fake(8); a.x_prev = fake(9);
    a.y = fake(10);
    return a;
}

static m3_scan_bwd_args bwd_args()
{
    m3_scan_bwd_args a;
    memset(&a, 0, sizeof(a));
    a.batch = 2; a.seqlen = 100; a.nheads = 3; a.headdim = 64; a.dstate = 64; a.rank = 1;
    a.io_dtype = M3_BF16; a.method = M3_BWD_AUTO;
    a.x = fake(0); a.B = fake(1); a.C = fake(2);
    a.dt = (const float*)fake(3); a.A = (const float*)fake(4); a.theta = (const float*)fake(5);
    a.lam = (const float*)fake(6); a.dy = fake(7);
    a.dx = (float*)fake(8); a.dB = (float*)fake(9); a.dC = (float*)fake(10); a.ddt = (float*)fake(11);
    a.dA = (float*)fake(12); a.dtheta = (float*)fake(13); a.dlam = (float*)fake(14);
    return a;
}

int main()
{
    // ---- scan: validation codes ------------------------------------------
    CHECK(m3_scan_fwd(nullptr, nullptr) == M3_ERR_NULL, "null args");
    CHECK(m3_scan_fwd_noalloc(nullptr, nullptr) == M3_ERR_NULL, "noalloc null args");
    struct ScanCase { void (*edit)(m3_scan_args&); m3_status code; const char* what; };
    const ScanCase cases[] = {
        {[](m3_scan_args& a) { a.dstate = 63; }, M3_ERR_SHAPE, "odd dstate"},
        {[](m3_scan_args& a) { a.batch = -1; }, M3_ERR_SHAPE, "negative batch"},
        {[](m3_scan_args& a) { a.chunk = -1; }, M3_ERR_SHAPE, "negative chunk"},
        {[](m3_scan_args& a) { a.io_dtype = 7; }, M3_ERR_DTYPE, "dtype"},
        {[](m3_scan_args& a) { a.dstate = 48; }, M3_ERR_UNSUPPORTED, "dstate 48"},
        {[](m3_scan_args& a) { a.chunk = 24; }, M3_ERR_UNSUPPORTED, "chunk 24"},
        {[](m3_scan_args& a) { a.x = nullptr; }, M3_ERR_NULL, "x null"},
        {[](m3_scan_args& a) { a.x = fake(0, 8); }, M3_ERR_ALIGN, "x misaligned"},
        {[](m3_scan_args& a) { a.y = fake(0); }, M3_ERR_ALIAS, "y aliases x"},
        {[](m3_scan_args& a) { a.seqlen = 1000; a.segments = 4; }, M3_ERR_WORKSPACE, "no workspace"},
        {[](m3_scan_args& a) { a.opt.ngroups = 2; }, M3_ERR_OPTION, "groups"},
        {[](m3_scan_args& a) { a.opt.phase_mode = 3; }, M3_ERR_NULL, "shuffle without perm"},
        {[](m3_scan_args& a) { a.opt.premix = 1; a.opt.norm_eps = -1.f; }, M3_ERR_OPTION, "eps"},
        {[](m3_scan_args& a) { a.opt.cu_seqlens = (const int32_t*)fake(42); a.opt.max_seqlen = 11; },
         M3_ERR_OPTION, "max_seqlen"},
        {[](m3_scan_args& a) { a.opt.phase_out = (float*)fake(43); }, M3_ERR_WORKSPACE, "phase_out ws"},
        // extreme sizes: rejected (or sized) without overflow
        {[](m3_scan_args& a) { a.batch = (int64_t)1 << 40; }, M3_ERR_UNSUPPORTED, "2^40 rows"},
        {[](m3_scan_args& a) { a.nheads = (int64_t)1 << 31; }, M3_ERR_UNSUPPORTED, "2^31 heads"},
        {[](m3_scan_args& a) { a.headdim = (int64_t)1 << 40; }, M3_ERR_UNSUPPORTED, "2^40 headdim"},
        {[](m3_scan_args& a) { a.rank = (int64_t)1 << 40; }, M3_ERR_UNSUPPORTED, "2^40 rank"},
        // (its fake arrays, 2^40 tokens long, overlap one another)
        {[](m3_scan_args& a) { a.seqlen = (int64_t)1 << 40; a.segments = 64; }, M3_ERR_ALIAS,
         "2^40 tokens, 64 segments"},
    };
    for (const ScanCase& c : cases) {
        m3_scan_args a = scan_args();
        c.edit(a);
        const m3_status st = m3_scan_fwd(&a, nullptr);
        CHECK(st == c.code, "scan %s: got %d, want %d", c.what, (int)st, (int)c.code);
        (void)m3_scan_workspace_bytes(&a);
    }
    // the state record in place needs the workspace that holds its copy
    {
        m3_scan_args a = scan_args();
        a.h_in = a.h_out = (float*)fake(20);
        a.B_prev_in = a.B_prev_out = fake(21);
        a.x_prev_in = a.x_prev_out = fake(22);
        const size_t ws = m3_scan_workspace_bytes(&a);
        CHECK(ws >= (size_t)6 * 64 * 32 * 4, "in-place workspace %zu", ws);
        CHECK(m3_scan_fwd(&a, nullptr) == M3_ERR_WORKSPACE, "in place without workspace");
        a.h_out = (float*)fake(20, 16);
        CHECK(m3_scan_fwd(&a, nullptr) == M3_ERR_ALIAS, "partial overlap");
    }
    // the allocation-free scan: a call beyond its scratch
    {
        m3_scan_args a = scan_args();
        a.batch = 64; a.nheads = 16; a.seqlen = 1 << 16; a.headdim = 64; a.segments = 64;
        CHECK(m3_scan_fwd_noalloc(&a, nullptr) == M3_ERR_SCRATCH, "noalloc scratch limit");
    }
    // zero work needs no pointers
    {
        m3_scan_args a;
        memset(&a, 0, sizeof(a));
        a.seqlen = 100; a.nheads = 4; a.headdim = 64; a.dstate = 64; a.rank = 1; a.io_dtype = M3_BF16;
        CHECK(m3_scan_fwd(&a, nullptr) == M3_OK, "zero batch");
    }

    // ---- decode -----------------------------------------------------------
    CHECK(m3_decode_step(nullptr, nullptr) == M3_ERR_NULL, "decode null");
    struct DecCase { void (*edit)(m3_decode_args&); m3_status code; const char* what; };
    const DecCase dcases[] = {
        {[](m3_decode_args& a) { a.dstate = 5; }, M3_ERR_SHAPE, "odd dstate"},
        {[](m3_decode_args& a) { a.rank = 3; }, M3_ERR_UNSUPPORTED, "rank 3"},
        {[](m3_decode_args& a) { a.h = nullptr; }, M3_ERR_NULL, "h null"},
        {[](m3_decode_args& a) { a.y = fake(7); }, M3_ERR_ALIAS, "y aliases h"},
        {[](m3_decode_args& a) { a.opt.phase_mode = 9; }, M3_ERR_OPTION, "phase mode"},
        {[](m3_decode_args& a) { a.batch = (int64_t)1 << 40; }, M3_ERR_UNSUPPORTED, "2^40 rows"},
    };
    for (const DecCase& c : dcases) {
        m3_decode_args a = decode_args();
        c.edit(a);
        const m3_status st = m3_decode_step(&a, nullptr);
        CHECK(st == c.code, "decode %s: got %d, want %d", c.what, (int)st, (int)c.code);
    }

    // ---- gradient ---------------------------------------------------------
    CHECK(m3_scan_bwd(nullptr, nullptr) == M3_ERR_NULL, "bwd null");
    {
        m3_scan_bwd_args a = bwd_args();
        const size_t ws = m3_scan_bwd_workspace_bytes(&a);
        CHECK(ws > 0, "bwd workspace");
        CHECK(m3_scan_bwd(&a, nullptr) == M3_ERR_WORKSPACE, "bwd without workspace");
        a.method = 7;
        CHECK(m3_scan_bwd(&a, nullptr) == M3_ERR_OPTION, "bwd method");
        a = bwd_args();
        a.dx = (float*)fake(0);
        CHECK(m3_scan_bwd(&a, nullptr) == M3_ERR_ALIAS, "dx aliases x");
        a = bwd_args();
        a.batch = (int64_t)1 << 40;
        (void)m3_scan_bwd_workspace_bytes(&a);
        CHECK(m3_scan_bwd(&a, nullptr) < 0, "bwd 2^40 rows");
        for (int m = 0; m < 3; ++m) {
            a = bwd_args();
            a.method = m;
            a.seqlen = (int64_t)1 << 30;
            (void)m3_scan_bwd_workspace_bytes(&a);
        }
    }

    // ---- helpers ----------------------------------------------------------
    CHECK(m3_abi_version() == M3_ABI_VERSION, "abi version");
    for (int s = 1; s >= -12; --s) CHECK(m3_status_string((m3_status)s) != nullptr, "status string");
    CHECK(m3_scan_supported(64, 64, 1, 0, M3_BF16) == 1, "supported");
    CHECK(m3_scan_supported(96, 64, 1, 0, M3_BF16) == 0, "unsupported");
    CHECK(m3_decode_supported(128, 64, 4, M3_BF16) == 1, "decode supported");
    CHECK(m3_scan_bwd_supported(128, 64, 4, M3_BF16) == 1, "bwd supported");
    CHECK(m3_last_hip_error() == 0, "no HIP error");

    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("abi driver: all checks passed\n");
    return 0;
}
