// gfx950.hpp -- device-side building blocks for the libtfla kernels (CDNA4,
// 64-lane wavefronts, matrix-core instructions with fp32 accumulation).
//
// Fragment conventions.  A 16x16 output tile is produced
// by v_mfma_f32_16x16x32_bf16 from:
//   A (16 x 32, M x K): lane l holds A[l%16][8*(l/16) + e], e = 0..7
//   B (32 x 16, K x N): lane l holds B[8*(l/16) + e][l%16], e = 0..7
//   D (16 x 16)       : lane l holds D[4*(l/16) + r][l%16], r = 0..3
// The fp32 path keeps the same per-lane data (8 K-elements per lane) and
// issues eight v_mfma_f32_16x16x4_f32, the e-th one contracting the K
// indices {e, 8+e, 16+e, 24+e}; the sum over e is the same contraction, so a
// kernel written once serves both element types.
//
// 32x32 tiles (v_mfma_f32_32x32x16_bf16; fp32: eight v_mfma_f32_32x32x2_f32):
//   A (32 x 16): lane l holds A[l%32][8*(l/32) + e], e = 0..7
//   B (16 x 32): lane l holds B[8*(l/32) + e][l%32]
//   D (32 x 32): lane l holds D[8*(r/4) + 4*(l/32) + r%4][l%32], r = 0..15
//
// LDS transpose read (ds_read_b64_tr_b16): within each 16-lane group, output
// lane j element r is element j%4 of the 8 bytes addressed by lane 4r + j/4.
// With lane i of a group pointing at row (base + i/4), column (c0 + 4*(i%4))
// of a row-major 16-bit tile, lane j receives column c0 + j, rows base..base+3:
// a matrix-core operand fragment read straight from a row-major tile.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tfla {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
// Floor of the log forget gate: a gate below e^-100 acts as e^-100, which
// keeps chunk-local log-decay differences finite (also for a gate of 0).
constexpr float kLogForgetFloor = -100.0f;

// ---- element traits --------------------------------------------------------
template <typename T> struct Elem;
template <> struct Elem<bf16> {
    typedef bf16x8 frag;                 // 8 K-elements per lane
    static constexpr int vec = 8;        // elements per 16-byte vector
};
template <> struct Elem<float> {
    struct frag { f32x4 lo, hi; };       // 8 fp32 K-elements per lane
    static constexpr int vec = 4;
};

__device__ __forceinline__ bf16 to_bf16(float x) { return (bf16)x; }   // RNE (v_cvt_pk_bf16_f32)

template <typename T> __device__ __forceinline__ T from_float(float x);
template <> __device__ __forceinline__ bf16 from_float<bf16>(float x) { return to_bf16(x); }
template <> __device__ __forceinline__ float from_float<float>(float x) { return x; }

__device__ __forceinline__ float to_float(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_float(float x) { return x; }

// ---- matrix-core step: acc += A * B over K = 32 ----------------------------
__device__ __forceinline__ f32x4 mma(const bf16x8& a, const bf16x8& b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const Elem<float>::frag& a, const Elem<float>::frag& b, f32x4 c)
{
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[0], b.lo[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[1], b.lo[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[2], b.lo[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[3], b.lo[3], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[0], b.hi[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[1], b.hi[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[2], b.hi[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[3], b.hi[3], c, 0, 0, 0);
    return c;
}

// ---- matrix-core step on a 32x32 tile: acc += A * B over K = 16 ----------
__device__ __forceinline__ f32x16 mma32(const bf16x8& a, const bf16x8& b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma32(const Elem<float>::frag& a, const Elem<float>::frag& b, f32x16 c)
{
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[0], b.lo[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[1], b.lo[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[2], b.lo[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[3], b.lo[3], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[0], b.hi[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[1], b.hi[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[2], b.hi[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[3], b.hi[3], c, 0, 0, 0);
    return c;
}

// ---- LDS transpose read ------------------------------------------------------
// Four 16-bit elements of a row-major LDS tile, transposed across the lane's
// 16-lane group (see the convention above).  `p` must point into LDS.
__device__ __forceinline__ bf16x4 tr_read4(const bf16* p)
{
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
    return __builtin_bit_cast(bf16x4, r);
}

// Operand fragment of a 32x32x16 product read from a row-major LDS tile
// whose rows run along the contraction index (e.g. V[step][value] as the B
// operand of P V, or both operands of V^T K): the 16-row block at `row0`,
// the 32 columns at `col0`.  Element e of lane l holds row
// row0 + 4h + e (e < 4) or row0 + 8 + 4h + (e - 4) (e >= 4), h = l/32, and
// column col0 + l%32 -- the order in which a 32x32 accumulator holds its
// rows, so an accumulator reused as the other operand contracts consistently.
template <int LD>
__device__ __forceinline__ bf16x8 frag_tr(const bf16 (*t)[LD], int row0, int col0, int lane)
{
    const int G = lane >> 4, i = lane & 15, h = G >> 1;
    const int col = col0 + 16 * (G & 1) + 4 * (i & 3);
    const int r = row0 + 4 * h + (i >> 2);
    const bf16x4 lo = tr_read4(&t[r][col]);
    const bf16x4 hi = tr_read4(&t[r + 8][col]);
    bf16x8 f;
    f[0] = lo[0]; f[1] = lo[1]; f[2] = lo[2]; f[3] = lo[3];
    f[4] = hi[0]; f[5] = hi[1]; f[6] = hi[2]; f[7] = hi[3];
    return f;
}
template <int LD>
__device__ __forceinline__ Elem<float>::frag frag_tr(const float (*t)[LD], int row0, int col0, int lane)
{
    const int h = lane >> 5, col = col0 + (lane & 31);
    Elem<float>::frag f;
    for (int e = 0; e < 4; ++e) {
        f.lo[e] = t[row0 + 4 * h + e][col];
        f.hi[e] = t[row0 + 8 + 4 * h + e][col];
    }
    return f;
}

// ---- fragment element access ----------------------------------------------
__device__ __forceinline__ void frag_set(bf16x8& f, int e, float x) { f[e] = to_bf16(x); }
__device__ __forceinline__ void frag_set(Elem<float>::frag& f, int e, float x)
{
    if (e < 4) f.lo[e] = x; else f.hi[e - 4] = x;
}
__device__ __forceinline__ float frag_get(const bf16x8& f, int e) { return (float)f[e]; }
__device__ __forceinline__ float frag_get(const Elem<float>::frag& f, int e)
{
    return e < 4 ? f.lo[e] : f.hi[e - 4];
}

// 8 contiguous elements (16-byte aligned for bf16, 16-byte aligned halves for fp32)
__device__ __forceinline__ bf16x8 load8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ Elem<float>::frag load8(const float* p)
{
    Elem<float>::frag f;
    f.lo = *reinterpret_cast<const f32x4*>(p);
    f.hi = *reinterpret_cast<const f32x4*>(p + 4);
    return f;
}
// two runs of 4 contiguous elements: p[0..3] and p2[0..3]
__device__ __forceinline__ bf16x8 load4x2(const bf16* p, const bf16* p2)
{
    bf16x4 a = *reinterpret_cast<const bf16x4*>(p);
    bf16x4 b = *reinterpret_cast<const bf16x4*>(p2);
    bf16x8 f;
    f[0] = a[0]; f[1] = a[1]; f[2] = a[2]; f[3] = a[3];
    f[4] = b[0]; f[5] = b[1]; f[6] = b[2]; f[7] = b[3];
    return f;
}
__device__ __forceinline__ Elem<float>::frag load4x2(const float* p, const float* p2)
{
    Elem<float>::frag f;
    f.lo = *reinterpret_cast<const f32x4*>(p);
    f.hi = *reinterpret_cast<const f32x4*>(p2);
    return f;
}

// 16 bytes of global memory as floats (VEC elements of T)
template <typename T> struct Vec16;
template <> struct Vec16<bf16> {
    bf16x8 v;
    __device__ __forceinline__ void load(const bf16* p) { v = *reinterpret_cast<const bf16x8*>(p); }
    __device__ __forceinline__ float get(int e) const { return (float)v[e]; }
    __device__ __forceinline__ void set(int e, float x) { v[e] = to_bf16(x); }
    __device__ __forceinline__ void zero() { for (int e = 0; e < 8; ++e) v[e] = (bf16)0.0f; }
    __device__ __forceinline__ void store(bf16* p) const { *reinterpret_cast<bf16x8*>(p) = v; }
    // non-temporal: for results this launch and the next do not read again
    __device__ __forceinline__ void store_nt(bf16* p) const { __builtin_nontemporal_store(v, reinterpret_cast<bf16x8*>(p)); }
};
template <> struct Vec16<float> {
    f32x4 v;
    __device__ __forceinline__ void load(const float* p) { v = *reinterpret_cast<const f32x4*>(p); }
    __device__ __forceinline__ float get(int e) const { return v[e]; }
    __device__ __forceinline__ void set(int e, float x) { v[e] = x; }
    __device__ __forceinline__ void zero() { v = f32x4{0.f, 0.f, 0.f, 0.f}; }
    __device__ __forceinline__ void store(float* p) const { *reinterpret_cast<f32x4*>(p) = v; }
    __device__ __forceinline__ void store_nt(float* p) const { __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p)); }
};

// store two consecutive elements (x at p[0], y at p[1])
__device__ __forceinline__ void store2(bf16* p, float x, float y)
{
    bf16x2 t;
    t[0] = to_bf16(x);
    t[1] = to_bf16(y);
    *reinterpret_cast<bf16x2*>(p) = t;
}
__device__ __forceinline__ void store2(float* p, float x, float y)
{
    *reinterpret_cast<f32x2*>(p) = f32x2{x, y};
}

// store four consecutive elements (8-byte aligned for bf16, 16 for fp32)
__device__ __forceinline__ void store4(bf16* p, float x, float y, float z, float w)
{
    bf16x4 t;
    t[0] = to_bf16(x);
    t[1] = to_bf16(y);
    t[2] = to_bf16(z);
    t[3] = to_bf16(w);
    *reinterpret_cast<bf16x4*>(p) = t;
}
__device__ __forceinline__ void store4(float* p, float x, float y, float z, float w)
{
    *reinterpret_cast<f32x4*>(p) = f32x4{x, y, z, w};
}

// ---- scalar math -----------------------------------------------------------
// 2^x on the transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// log(sigmoid(x)) = min(x,0) - log1p(exp(-|x|)), accurate library calls
__device__ __forceinline__ float log_sigmoid(float x)
{
    return fminf(x, 0.0f) - log1pf(expf(-fabsf(x)));
}

// The same on the transcendental unit, for kernels that evaluate it per
// element of large tensors: y = e^{-|x|} = 2^{-|x| log2 e} (v_exp_f32), and
// log1p(y) by D. Goldberg, "What every computer scientist should know about
// floating-point arithmetic" (1991), Theorem 4: with u = 1 + y rounded,
// log1p(y) = y if u = 1, else ln(u) y / (u - 1) -- the rounding of u cancels
// between ln(u) and u - 1, so small y keep their relative accuracy.  ln(u) =
// log2(u) ln 2 (v_log_f32), 1 / (u - 1) by v_rcp_f32.  A few ulp against
// the library calls.
__device__ __forceinline__ float log_sigmoid_fast(float x)
{
    constexpr float kLn2 = 0.6931471805599453f;
    const float y = exp2_fast(-fabsf(x) * kLog2e);
    const float u = 1.0f + y;
    const float l1p = u == 1.0f ? y : __builtin_amdgcn_logf(u) * kLn2 * (y * __builtin_amdgcn_rcpf(u - 1.0f));
    return fminf(x, 0.0f) - l1p;
}

// Block index remap so that consecutive logical tiles land on one XCD:
// the dispatcher places workgroup b on XCD b % 8, so logical tile
// (b % 8) * (n / 8) + b / 8 keeps neighbours (which share K/V rows and
// states) inside one XCD's L2.  Identity when n is not a multiple of 8.
__device__ __forceinline__ int xcd_remap(int b, int n)
{
    if ((n & 7) != 0) return b;
    return (b & 7) * (n >> 3) + (b >> 3);
}

}  // namespace tfla
