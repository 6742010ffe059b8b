// gdn_device.h -- device helpers shared by the gfx950 kernels of libgdn:
// element types, conversions and the 16x16 MFMA fragment convention.
//
// Fragment convention.  Every MFMA here is a 16x16 output tile
// (v_mfma_f32_16x16x32_{bf16,f16} or v_mfma_f32_16x16x4_f32).  A lane
// l = x + 16*q (x in 0..15, q in 0..3) holds
//   * of an accumulator tile D[16 rows][16 cols]: column x, rows 4q..4q+3
//     in its four f32 registers;
//   * of an operand over a contraction of length K (a multiple of 16): for
//     each 16-wide block kb of the contraction, the four elements at
//     contraction indices 16*kb + 4q + (0..3) of row (A) or column (B) x.
// The hardware multiplies operand slot s of lane group q of A with slot s of
// lane group q of B, so any fixed assignment of contraction indices to
// (q, s) gives the right sum as long as A and B share it.  With this one, an
// accumulator tile is already an operand fragment over its rows: its column
// becomes the operand's row (A) or column (B) and its rows the contraction
// index.  Matrices staged in LDS row-major along the contraction index give
// their fragments with one 8-byte (16-bit types) or 16-byte (f32) read.
#pragma once

#include "gdn_internal.h"
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// The decay a gate input stands for: the value itself, or exp of it when
// the caller passes log-decays (the ferrox-core gdn_chunk.rs page's host
// body takes the gate in that form and exponentiates it).
__device__ __forceinline__ float decay_of(float g, int flags) {
    return (flags & kLogGate) ? expf(g) : g;
}

// Key head read by value head hv: grouped (hv / (Hv / Hk), the layout of the
// metaltile-std gated_delta_wy.rs page) or tiled (hv mod Hk).
__device__ __forceinline__ int key_head(int hv, int Hk, int Hv, int flags) {
    return (flags & kTiledHeads) ? hv % Hk : hv / (Hv / Hk);
}

// Value head of the r-th slot of a batch element when slots are counted with
// the value heads of each key head adjacent (key head r / (Hv / Hk)).
__device__ __forceinline__ int value_head_of_rank(int r, int Hk, int Hv, int flags) {
    const int group = Hv / Hk;
    return (flags & kTiledHeads) ? (r % group) * Hk + r / group : r;
}

template <typename T> struct Vec;
template <> struct Vec<float> { using x4 = f32x4; };
template <> struct Vec<__bf16> { using x4 = bf16x4; using x8 = bf16x8; };
template <> struct Vec<_Float16> { using x4 = f16x4; using x8 = f16x8; };

template <typename T> __device__ __forceinline__ float to_f32(T x) { return static_cast<float>(x); }
template <typename T> __device__ __forceinline__ T from_f32(float x) { return static_cast<T>(x); }

template <typename T>
__device__ __forceinline__ typename Vec<T>::x4 cvt4(f32x4 a) {
    typename Vec<T>::x4 r;
    r[0] = from_f32<T>(a[0]);
    r[1] = from_f32<T>(a[1]);
    r[2] = from_f32<T>(a[2]);
    r[3] = from_f32<T>(a[3]);
    return r;
}

// bfloat16: converted in pairs and packed through 32-bit words.  Written
// element by element, a result that feeds a matrix-core operand is
// converted one value per instruction and repacked with byte permutes
// (three times the vector-ALU work); pairs keep one packed conversion per
// two values.  Rounding is the same (to nearest even).
template <>
__device__ __forceinline__ bf16x4 cvt4<__bf16>(f32x4 a) {
    typedef float f32x2_ __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_ __attribute__((ext_vector_type(2)));
    typedef unsigned u32x2_ __attribute__((ext_vector_type(2)));
    const bf16x2_ lo = __builtin_convertvector(f32x2_{a[0], a[1]}, bf16x2_);
    const bf16x2_ hi = __builtin_convertvector(f32x2_{a[2], a[3]}, bf16x2_);
    const u32x2_ w = {__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
    return __builtin_bit_cast(bf16x4, w);
}

template <typename T>
__device__ __forceinline__ f32x4 to_f32x4(typename Vec<T>::x4 a) {
    f32x4 r;
    r[0] = to_f32(a[0]);
    r[1] = to_f32(a[1]);
    r[2] = to_f32(a[2]);
    r[3] = to_f32(a[3]);
    return r;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// A row of zeros read in place of state_in when it is NULL, so that the state
// loads are unconditional (a branch around each load made the compiler wait
// for every load before issuing the next).  Pointers into it and into
// state_in are global-memory pointers (address space 1), so that the loads
// stay global loads after the select.
static __device__ const float kZeroRow[128] = {};
typedef const float __attribute__((address_space(1))) gfloat;
typedef const f32x4 __attribute__((address_space(1))) gf32x4;

// One 16x16 MFMA step over 32 (16-bit types) or 4 (f32) contraction
// indices: acc += A_frag * B_frag.
__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// 16x16x16 steps (one 16-wide contraction block) for 16-bit types.
__device__ __forceinline__ f32x4 mfma(bf16x4 a, bf16x4 b, f32x4 c) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma(f16x4 a, f16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <typename T>
__device__ __forceinline__ typename Vec<T>::x8 cat8(typename Vec<T>::x4 lo, typename Vec<T>::x4 hi) {
    typename Vec<T>::x8 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
}

// acc += sum over contraction blocks kb in [kb0, kb1) of A(kb) * B(kb), where
// fa(kb) / fb(kb) return the lane's four operand elements of block kb
// (type Vec<T>::x4).  For 16-bit types blocks are paired into one MFMA; an
// odd last block is paired with zeros.
template <typename T, typename FA, typename FB>
__device__ __forceinline__ f32x4 mma_range(f32x4 acc, int kb0, int kb1, FA fa, FB fb) {
    if constexpr (sizeof(T) == 4) {
        for (int kb = kb0; kb < kb1; ++kb) {
            f32x4 a = fa(kb), b = fb(kb);
            acc = mfma(a[0], b[0], acc);
            acc = mfma(a[1], b[1], acc);
            acc = mfma(a[2], b[2], acc);
            acc = mfma(a[3], b[3], acc);
        }
    } else {
        using X4 = typename Vec<T>::x4;
        int kb = kb0;
        for (; kb + 1 < kb1; kb += 2)
            acc = mfma(cat8<T>(fa(kb), fa(kb + 1)), cat8<T>(fb(kb), fb(kb + 1)), acc);
        if (kb < kb1) {
            X4 z = cvt4<T>(zero4());
            acc = mfma(cat8<T>(fa(kb), z), cat8<T>(fb(kb), z), acc);
        }
    }
    return acc;
}

// Vector load/store of four elements (8 bytes for 16-bit types, 16 for f32).
template <typename T>
__device__ __forceinline__ typename Vec<T>::x4 ld4(const T *p) {
    return *reinterpret_cast<const typename Vec<T>::x4 *>(p);
}
template <typename T>
__device__ __forceinline__ void st4(T *p, typename Vec<T>::x4 v) {
    *reinterpret_cast<typename Vec<T>::x4 *>(p) = v;
}

}  // namespace gdn
