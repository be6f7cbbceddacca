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
// LDS operand layout ("A layout"): a matrix with rows m and Kc contraction
// columns is stored row-major in fragments of 8 elements; fragment f = 2*ks + g
// of row m holds the elements kappa(ks, g, 0..7), and sits at slot
// f ^ swz(m) of the row so that 8 consecutive rows read by one instruction hit
// distinct bank groups.  One A (or B) fragment is then a single 16-byte read.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kChunk = 64;   // tokens per chunk (talk summary, paragraph 3: "usually 64")
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
template <typename T>
__device__ __forceinline__ typename FragOf<T>::type acc_frag_scaled(const f32x16& acc, int half,
                                                                     const float* s) {
    typename FragOf<T>::type f;
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = (T)(acc[8 * half + j] * s[8 * half + j]);
    return f;
}

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

// Element offset of (row, col) in an A-layout matrix with Kc contraction columns.
__device__ __forceinline__ int lds_elem(int row, int col, int Kc) {
    int f = ((col >> 4) << 1) | ((col >> 2) & 1);
    int j = (((col >> 3) & 1) << 2) | (col & 3);
    return row * Kc + ((f ^ swz(row)) << 3) + j;
}
// Element offset of fragment (row, ks, g).
__device__ __forceinline__ int lds_frag(int row, int ks, int g, int Kc) {
    return row * Kc + (((2 * ks + g) ^ swz(row)) << 3);
}

template <typename T>
__device__ __forceinline__ typename FragOf<T>::type ld_frag(const T* base, int row, int ks, int g,
                                                            int Kc) {
    return *reinterpret_cast<const typename FragOf<T>::type*>(base + lds_frag(row, ks, g, Kc));
}
template <typename T>
__device__ __forceinline__ void st_frag(T* base, int row, int ks, int g, int Kc,
                                        const typename FragOf<T>::type& f) {
    *reinterpret_cast<typename FragOf<T>::type*>(base + lds_frag(row, ks, g, Kc)) = f;
}

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ float wave_inclusive_scan(float x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        float y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    return x;
}

}  // namespace gdn
