// Device-side building blocks shared by the gfx950 kernels: MFMA fragments,
// the LDS operand layout and small wave-level helpers.
//
// Matrix-core conventions (v_mfma_f32_32x32x16_bf16 on a wave64, verified on
// gfx950; the fp32 path issues eight v_mfma_f32_32x32x2_f32 with the same
// fragment contents):
//   lane l:  n = l & 31 (column of the output / row of an A operand), g = l >> 5
//   accumulator (f32x16) register r holds element (rho(g, r), n) of a 32x32
//   tile with rho(g, r) = 8*(r>>2) + 4*g + (r&3).
//   A fragment for one 16-wide k-step ks: lane (m, g) holds A[m][kappa(ks, g, j)],
//   j = 0..7, and B fragment lane (n, g) holds B[kappa(ks, g, j)][n], with
//   kappa(ks, g, j) = 16*ks + 8*(j>>2) + 4*g + (j&3).
// Because kappa(ks, g, j) = 32*(ks>>1) + rho(g, 8*(ks&1) + j), the eight
// accumulator registers 8*(ks&1)..+7 of tile ks>>1 ARE the B fragment of k-step
// ks when the product contracts over the accumulator's row index.  Every chain
// of products in the kernels is arranged that way, so results never leave
// registers between dependent products.
//
// LDS tiles are natural row-major (see toff); A fragments are two 4-element
// reads, and fragments of a transposed tile come from the gfx950 transposing
// LDS read (tfrag), so no transposed copy of any tile is ever stored.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kChunk = 64;   // tokens per chunk (talk summary, paragraph 3, gives 64 as the usual length)
constexpr int kDk = 128;
constexpr int kDv = 128;

template <typename T> struct FragOf;
template <> struct FragOf<__bf16> { using type = bf16x8; };
template <> struct FragOf<float> { using type = f32x8; };

// One 32x32x16 step: acc += A(32x16) * B(16x32).
__device__ __forceinline__ f32x16 mma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma(const f32x8& a, const f32x8& b, f32x16 c) {
#pragma unroll
    for (int i = 0; i < 8; ++i) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[i], c, 0, 0, 0);
    return c;
}

__device__ __forceinline__ int rho(int g, int r) { return ((r >> 2) << 3) + (g << 2) + (r & 3); }

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}

// Convert eight accumulator registers (half = 0: regs 0..7, 1: regs 8..15) to a fragment.
template <typename T>
__device__ __forceinline__ typename FragOf<T>::type acc_frag(const f32x16& acc, int half) {
    typename FragOf<T>::type f;
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = (T)acc[8 * half + j];
    return f;
}
// The same, with a per-register scale.
// A bf16 fragment taken from accumulator rows carries contraction indices
// 16h + 8(j>>2) + 4g + (j&3) (the accumulator's row order); a 16-byte tile read
// carries 16h + 8g + j.  Reordering one into the other moves elements 4..7 of
// the g = 0 half-wave and elements 0..3 of the g = 1 half-wave across: two
// v_permlane32_swap, each exchanging the upper half-wave of its first operand
// with the lower half-wave of its second.  Float32 fragments are unchanged.
template <typename T>
__device__ __forceinline__ typename FragOf<T>::type nat_frag(const typename FragOf<T>::type& f) {
    if constexpr (sizeof(T) == 2) {
        typedef uint32_t u4 __attribute__((ext_vector_type(4)));
        const u4 u = __builtin_bit_cast(u4, f);   // u[0], u[1]: elements 0..3; u[2], u[3]: 4..7
        const auto r0 = __builtin_amdgcn_permlane32_swap(u[0], u[2], false, false);
        const auto r1 = __builtin_amdgcn_permlane32_swap(u[1], u[3], false, false);
        const u4 o = {r0[0], r1[0], r0[1], r1[1]};
        return __builtin_bit_cast(typename FragOf<T>::type, o);
    } else {
        return f;
    }
}

template <typename T>
__device__ __forceinline__ typename FragOf<T>::type acc_frag_scaled(const f32x16& acc, int half,
                                                                     const float* s) {
    typename FragOf<T>::type f;
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = (T)(acc[8 * half + j] * s[8 * half + j]);
    return f;
}

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int swz4(int row) { return (row ^ (row >> 2)) & 3; }
// Rows of 16 or more slots (a 256-byte bf16 row spans all 64 LDS banks): the
// slot index is XORed with a 4-bit value that differs for any 16 consecutive
// rows, and whose top two bits differ for any 4 consecutive rows.  gfx950
// serves a 64-bit LDS read in two 32-lane halves: 32 rows reading the same
// 8-byte column then fall on 16 distinct bank pairs (two lanes per bank, the
// fewest possible), and a transposing read, whose 32 lanes cover 4 rows x 64
// bytes, touches 4 disjoint 16-bank groups (no conflict).
__device__ __forceinline__ int swz16(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }
template <int CPR>
__device__ __forceinline__ int slot_swz(int row) {
    return CPR >= 16 ? swz16(row) : CPR >= 8 ? swz(row) : swz4(row);
}

// Natural row-major tiles in LDS: a row of `Cols` elements is stored as 16-byte
// chunks; chunk c of row r sits at slot c ^ slot_swz(r) (swz16 for rows of
// sixteen or more chunks, swz for eight, swz4 for four), so rows read together
// at the same column land in different bank groups.  Element offset of (row, col):
template <typename T, int Cols>
__device__ __forceinline__ int toff(int row, int col) {
    constexpr int EPC = 16 / (int)sizeof(T);   // elements per 16-byte chunk
    constexpr int CPR = Cols / EPC;             // chunks per row
    const int s = slot_swz<CPR>(row);
    return row * Cols + (((col / EPC) ^ s) * EPC) + (col % EPC);
}

template <typename T> struct Quad;
template <> struct Quad<__bf16> { typedef __bf16 type __attribute__((ext_vector_type(4))); };
template <> struct Quad<float> { typedef float type __attribute__((ext_vector_type(4))); };

// A fragment of a row-major tile: lane (m, g) gets A[m][kappa(ks, g, 0..7)], i.e.
// columns 16ks+4g..+3 and 16ks+8+4g..+3 of row m (two 4-element reads).
template <typename T, int Cols>
__device__ __forceinline__ typename FragOf<T>::type afrag(const T* tile, int row, int ks, int g) {
    typedef typename Quad<T>::type Q4;
    Q4 lo = *reinterpret_cast<const Q4*>(tile + toff<T, Cols>(row, 16 * ks + 4 * g));
    Q4 hi = *reinterpret_cast<const Q4*>(tile + toff<T, Cols>(row, 16 * ks + 8 + 4 * g));
    typename FragOf<T>::type f;
#pragma unroll
    for (int j = 0; j < 4; ++j) { f[j] = lo[j]; f[4 + j] = hi[j]; }
    return f;
}
template <typename T, int Cols>
__device__ __forceinline__ void st_afrag(T* tile, int row, int ks, int g,
                                         const typename FragOf<T>::type& f) {
    typedef typename Quad<T>::type Q4;
    Q4 lo, hi;
#pragma unroll
    for (int j = 0; j < 4; ++j) { lo[j] = f[j]; hi[j] = f[4 + j]; }
    *reinterpret_cast<Q4*>(tile + toff<T, Cols>(row, 16 * ks + 4 * g)) = lo;
    *reinterpret_cast<Q4*>(tile + toff<T, Cols>(row, 16 * ks + 8 + 4 * g)) = hi;
}

// Transposed fragment of a row-major tile M[k][n]: lane (m, g), m = lane & 31,
// gets M[kappa(ks, g, 0..7)][nbase + m].  For bf16 this is two ds_read_b64_tr_b16:
// within each 16-lane group, lane L points at row k0 + L/4, columns
// n0 + 4(L%4)..+3, and lane i then holds M[k0 + j][n0 + i] for j = 0..3
// (verified on gfx950).  The float32 build reads the eight elements one by one.
template <typename T, int Cols>
__device__ __forceinline__ typename FragOf<T>::type tfrag(const T* tile, int nbase, int ks, int lane) {
    const int g = lane >> 5;
    typename FragOf<T>::type f;
    if constexpr (sizeof(T) == 2) {
        typedef short s4 __attribute__((ext_vector_type(4)));
        const int i = lane & 15;
        const int n0 = nbase + (lane & 16);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int k0 = 16 * ks + 8 * h + 4 * g;
            const T* p = tile + toff<T, Cols>(k0 + (i >> 2), n0 + 4 * (i & 3));
            s4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s4*)(__attribute__((address_space(3))) void*)p);
            // reinterpret the whole vector (per-element casts of the result were
            // miscompiled into a splat of element 0 by this toolchain)
            typename Quad<T>::type q = __builtin_bit_cast(typename Quad<T>::type, r);
#pragma unroll
            for (int j = 0; j < 4; ++j) f[4 * h + j] = q[j];
        }
    } else {
        const int n = nbase + (lane & 31);
#pragma unroll
        for (int j = 0; j < 8; ++j) f[j] = tile[toff<T, Cols>(16 * ks + 8 * (j >> 2) + 4 * g + (j & 3), n)];
    }
    return f;
}

// x of lane l, as a wave-uniform value (v_readlane: no LDS round trip).
__device__ __forceinline__ float lane_value(float x, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}

// The value of the lane that DPP control CTRL selects (0 where it selects none
// or where ROWS masks the row out).
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_take(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROWS, 0xf, true));
}

// Inclusive prefix sum across the 64 lanes of a wave, on the DPP paths alone:
// shifts by 1, 2, 4 and 8 lanes scan each row of 16, then the last lane of row
// 0 (and of row 2) is added to row 1 (row 3), and the last lane of row 1 to rows
// 2 and 3.
__device__ __forceinline__ float wave_inclusive_scan(float x) {
    x += dpp_take<0x111, 0xf>(x);   // row_shr:1
    x += dpp_take<0x112, 0xf>(x);   // row_shr:2
    x += dpp_take<0x114, 0xf>(x);   // row_shr:4
    x += dpp_take<0x118, 0xf>(x);   // row_shr:8
    x += dpp_take<0x142, 0xa>(x);   // row_bcast:15 into rows 1 and 3
    x += dpp_take<0x143, 0xc>(x);   // row_bcast:31 into rows 2 and 3
    return x;
}

}  // namespace gdn
