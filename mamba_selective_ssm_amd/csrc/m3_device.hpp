// Device-side helpers for libm3scan (gfx950 only): operand fragments for the
// 16x16 matrix-core tiles, element conversions, vector loads.
//
// Matrix-core tile conventions used throughout (wave64, 16x16 output tile):
//   A operand (16 x K): lane l supplies row (l % 16), K-slots g*8 + e (g = l/16,
//                       e = 0..7) -- 8 values per lane per 32-wide K block.
//   B operand (K x 16): lane l supplies column (l % 16), the same K-slots.
//   D (16 x 16 fp32):   lane l holds column (l % 16), rows g*4 + i, i = 0..3.
// Which physical K index a slot carries is up to the caller, as long as A and
// B use the same assignment; the kernels exploit that to avoid transposes.
// bf16 operands use one v_mfma_f32_16x16x32_bf16 per 32-wide K block; fp32
// operands use eight v_mfma_f32_16x16x4_f32 (slot e of every lane group forms
// the 4-wide K block of the e-th instruction).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace m3 {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

// 8 K-slots of one lane.
template <typename OP> struct Frag;
template <> struct Frag<bf16> {
    bf16x8 v;
    __device__ __forceinline__ void set(int e, float x) { v[e] = (bf16)x; }
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (bf16)0.0f;
    }
};
template <> struct Frag<float> {
    float v[8];
    __device__ __forceinline__ void set(int e, float x) { v[e] = x; }
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = 0.0f;
    }
};

__device__ __forceinline__ void mma(const Frag<bf16>& a, const Frag<bf16>& b, f32x4& c) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ void mma(const Frag<float>& a, const Frag<float>& b, f32x4& c) {
#pragma unroll
    for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], c, 0, 0, 0);
}

// 8 contiguous operand elements from LDS (16-byte aligned for bf16, 32 for fp32).
__device__ __forceinline__ void lds_frag8(Frag<bf16>& f, const bf16* p) {
    f.v = *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ void lds_frag8(Frag<float>& f, const float* p) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) { f.v[e] = a[e]; f.v[4 + e] = b[e]; }
}
// Two runs of 4 contiguous elements: slots 0..3 from p0, slots 4..7 from p1.
__device__ __forceinline__ void lds_frag4x2(Frag<bf16>& f, const bf16* p0, const bf16* p1) {
    const bf16x4 a = *reinterpret_cast<const bf16x4*>(p0);
    const bf16x4 b = *reinterpret_cast<const bf16x4*>(p1);
#pragma unroll
    for (int e = 0; e < 4; ++e) { f.v[e] = a[e]; f.v[4 + e] = b[e]; }
}
__device__ __forceinline__ void lds_frag4x2(Frag<float>& f, const float* p0, const float* p1) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p0);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p1);
#pragma unroll
    for (int e = 0; e < 4; ++e) { f.v[e] = a[e]; f.v[4 + e] = b[e]; }
}
__device__ __forceinline__ void lds_frag4(Frag<bf16>& f, const bf16* p0) {
    const bf16x4 a = *reinterpret_cast<const bf16x4*>(p0);
#pragma unroll
    for (int e = 0; e < 4; ++e) { f.v[e] = a[e]; f.v[4 + e] = (bf16)0.0f; }
}
__device__ __forceinline__ void lds_frag4(Frag<float>& f, const float* p0) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p0);
#pragma unroll
    for (int e = 0; e < 4; ++e) { f.v[e] = a[e]; f.v[4 + e] = 0.0f; }
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// 8 contiguous io elements from global memory as floats.
__device__ __forceinline__ void gload8(float (&d)[8], const bf16* p) {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) d[e] = (float)v[e];
}
__device__ __forceinline__ void gload8(float (&d)[8], const float* p) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) { d[e] = a[e]; d[4 + e] = b[e]; }
}
// A pair of adjacent io elements (one rotation pair) from global memory.
__device__ __forceinline__ void gload2(float& a, float& b, const bf16* p) {
    const bf16x2 v = *reinterpret_cast<const bf16x2*>(p);
    a = (float)v[0]; b = (float)v[1];
}
__device__ __forceinline__ void gload2(float& a, float& b, const float* p) {
    const float2 v = *reinterpret_cast<const float2*>(p);
    a = v.x; b = v.y;
}
__device__ __forceinline__ void sstore2(bf16* p, float a, float b) {
    bf16x2 v; v[0] = (bf16)a; v[1] = (bf16)b;
    *reinterpret_cast<bf16x2*>(p) = v;
}
__device__ __forceinline__ void sstore2(float* p, float a, float b) {
    *reinterpret_cast<float2*>(p) = make_float2(a, b);
}
// 4 contiguous io elements to global memory.
__device__ __forceinline__ void gstore4(bf16* p, const f32x4& v) {
    bf16x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (bf16)v[e];
    *reinterpret_cast<bf16x4*>(p) = o;
}
__device__ __forceinline__ void gstore4(float* p, const f32x4& v) {
    *reinterpret_cast<f32x4*>(p) = v;
}

constexpr float kLog2e = 1.4426950408889634f;

}  // namespace m3

namespace m3 {

// A rotation pair (two adjacent io elements) held in registers.
template <typename T> struct IoPair;
template <> struct IoPair<bf16> {
    bf16x2 v;
    __device__ __forceinline__ void load(const bf16* p) { v = *reinterpret_cast<const bf16x2*>(p); }
    __device__ __forceinline__ float lo() const { return (float)v[0]; }
    __device__ __forceinline__ float hi() const { return (float)v[1]; }
};
template <> struct IoPair<float> {
    float2 v;
    __device__ __forceinline__ void load(const float* p) { v = *reinterpret_cast<const float2*>(p); }
    __device__ __forceinline__ float lo() const { return v.x; }
    __device__ __forceinline__ float hi() const { return v.y; }
};

// 8 contiguous io elements held in registers.
template <typename T> struct IoRow8;
template <> struct IoRow8<bf16> {
    bf16x8 v;
    __device__ __forceinline__ void load(const bf16* p) { v = *reinterpret_cast<const bf16x8*>(p); }
    __device__ __forceinline__ float get(int e) const { return (float)v[e]; }
    __device__ __forceinline__ void store_raw(bf16* p) const { *reinterpret_cast<bf16x8*>(p) = v; }
    __device__ __forceinline__ void set8(const float (&x)[8]) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (bf16)x[e];
    }
};
template <> struct IoRow8<float> {
    f32x4 a, b;
    __device__ __forceinline__ void load(const float* p) {
        a = *reinterpret_cast<const f32x4*>(p);
        b = *reinterpret_cast<const f32x4*>(p + 4);
    }
    __device__ __forceinline__ float get(int e) const { return e < 4 ? a[e] : b[e - 4]; }
    __device__ __forceinline__ void store_raw(float* p) const {
        *reinterpret_cast<f32x4*>(p) = a;
        *reinterpret_cast<f32x4*>(p + 4) = b;
    }
};

// Four operand elements to LDS in one store.
__device__ __forceinline__ void lds_store4(bf16* p, float a, float b, float c, float d) {
    bf16x4 v; v[0] = (bf16)a; v[1] = (bf16)b; v[2] = (bf16)c; v[3] = (bf16)d;
    *reinterpret_cast<bf16x4*>(p) = v;
}
__device__ __forceinline__ void lds_store4(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
}

}  // namespace m3

namespace m3 {

// Inclusive prefix sum across the 64 lanes of a wavefront with DPP moves:
// row shifts by 1, 2, 4, 8 scan each row of 16 lanes, then the row
// broadcasts of lanes 15 and 31 carry row totals upward.  Lanes with no DPP
// source add the old value 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_moved(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                                 ROW_MASK, 0xf, false));
}

__device__ __forceinline__ float wave_inclusive_sum(float v)
{
    v += dpp_moved<0x111, 0xf>(v);   // row_shr:1
    v += dpp_moved<0x112, 0xf>(v);   // row_shr:2
    v += dpp_moved<0x114, 0xf>(v);   // row_shr:4
    v += dpp_moved<0x118, 0xf>(v);   // row_shr:8
    v += dpp_moved<0x142, 0xa>(v);   // row_bcast:15 into rows 1 and 3
    v += dpp_moved<0x143, 0xc>(v);   // row_bcast:31 into rows 2 and 3
    return v;
}

// (b, h) of a flattened (batch, head) index in 32-bit arithmetic: the callers
// keep batch x heads below 2^31, and a 64-bit division is a long software
// sequence at the start of every wave that needs it.
__device__ __forceinline__ void split_bh(int64_t bh, int64_t H, int64_t& b, int64_t& h)
{
    const int q = (int)bh / (int)H;
    b = q;
    h = (int)bh - q * (int)H;
}

// The same for 32-bit integers.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_moved_i(int x)
{
    return __builtin_amdgcn_update_dpp(0, x, CTRL, ROW_MASK, 0xf, false);
}
__device__ __forceinline__ int wave_inclusive_sum_i(int v)
{
    v += dpp_moved_i<0x111, 0xf>(v);
    v += dpp_moved_i<0x112, 0xf>(v);
    v += dpp_moved_i<0x114, 0xf>(v);
    v += dpp_moved_i<0x118, 0xf>(v);
    v += dpp_moved_i<0x142, 0xa>(v);
    v += dpp_moved_i<0x143, 0xc>(v);
    return v;
}

// Sum over aligned groups of G consecutive lanes (4, 8 or 16), every lane of a
// group receiving its group's sum: a butterfly of DPP lane moves inside each
// row of 16 lanes (no LDS round trip).
template <int G>
__device__ __forceinline__ float lane_group_sum(float v)
{
    static_assert(G == 4 || G == 8 || G == 16, "lane groups of 4, 8 or 16");
    v += dpp_moved<0xB1, 0xf>(v);                            // quad_perm [1,0,3,2]
    v += dpp_moved<0x4E, 0xf>(v);                            // quad_perm [2,3,0,1]
    if constexpr (G >= 8) v += dpp_moved<0x141, 0xf>(v);     // row_half_mirror
    if constexpr (G >= 16) v += dpp_moved<0x140, 0xf>(v);    // row_mirror
    return v;
}

__device__ __forceinline__ float wave_read_lane(float v, int lane)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

}  // namespace m3

namespace m3 {

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// Transposing LDS read (gfx950 ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane j supplies the address of 4 consecutive bf16 values; lane i then
// receives element (i % 4) of the values supplied by lanes (i / 4), 4 + (i / 4),
// 8 + (i / 4) and 12 + (i / 4).  With lane j pointing at row k0 + j / 4,
// columns c0 + 4 * (j % 4) .. + 3 of a row-major bf16 block, lane i gets rows
// k0 .. k0 + 3 of column c0 + i: four consecutive keys of one column, the
// K-slots of a matrix-core operand read from a key-major array.
__device__ __forceinline__ bf16x4 lds_read_tr4(const bf16* p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

}  // namespace m3

namespace m3 {

// Eight operand elements to LDS (16 B for bf16, 32 B for fp32).
__device__ __forceinline__ void lds_store8(bf16* p, const float (&v)[8])
{
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (bf16)v[e];
    *reinterpret_cast<bf16x8*>(p) = o;
}
__device__ __forceinline__ void lds_store8(float* p, const float (&v)[8])
{
    *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
}

}  // namespace m3
