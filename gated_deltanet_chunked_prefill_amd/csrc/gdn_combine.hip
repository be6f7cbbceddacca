// Segment combine of the intra-GPU sequence split (FlashQLA talk summary,
// onedev.kr, paragraph 4: the state difference across a chunk is one dk x dk
// matrix product, so by associativity each segment's correction is composed
// once; only each segment's last correction is kept).
//
// For an exact head split into P segments, pass-1 left, per segment p >= 1,
// its zero-start final state bz_p, the gate-free transition Mt_p and the gate
// sum G_p, so that the segment maps an entering state H to
//     H -> exp(G_p) Mt_p H + bz_p.
// Segment 0 already ran from the true initial state and stored the true state
// entering segment 1 (hs_1).  This kernel walks p = 2..P-1 sequentially:
//     hs_p = exp(G_{p-1}) Mt_{p-1} hs_{p-1} + bz_{p-1}.
// Grid: (B*H, 4); workgroup (bh, cb) owns state columns [32cb, 32cb+32) and its
// four waves own dk row tiles.  The 128x128x32 products run on the bf16 matrix
// cores with a three-term hi/lo split (a_hi b_hi + a_hi b_lo + a_lo b_hi), which
// keeps them close to float32 accuracy.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

__device__ __forceinline__ void split_bf16(const f32x8& x, bf16x8& hi, bf16x8& lo) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        __bf16 h = (__bf16)x[j];
        hi[j] = h;
        lo[j] = (__bf16)(x[j] - (float)h);
    }
}

__global__ __launch_bounds__(256, 1) void combine_kernel(FwdParams prm) {
    __shared__ float xs[4][64][16];
    const int bh = blockIdx.x, cb = blockIdx.y;
    if (prm.flags && prm.flags[bh] != 0) return;  // window head: no correction
    const int P = prm.P;
    if (P < 3) return;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 31, g = lane >> 5;
    const size_t SS = (size_t)kDk * kDv;
    const int col = 32 * cb + n;

    f32x16 cur;
    const float* h1 = prm.hs + ((size_t)bh * P + 1) * SS;
#pragma unroll
    for (int r = 0; r < 16; ++r) cur[r] = h1[(32 * w + rho(g, r)) * kDv + col];

    for (int p = 2; p < P; ++p) {
#pragma unroll
        for (int r = 0; r < 16; ++r) xs[w][lane][r] = cur[r];
        __syncthreads();
        const float* mt = prm.mt + ((size_t)bh * P + p - 1) * SS;
        const float* bz = prm.bz + ((size_t)bh * P + p - 1) * SS;
        const float eG = __expf(prm.gsum[(size_t)bh * P + p - 1]);
        f32x16 acc = zero16();
        const float* arow = mt + (size_t)(32 * w + n) * kDk;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            f32x4 a0 = *(const f32x4*)(arow + 16 * ks + 4 * g);
            f32x4 a1 = *(const f32x4*)(arow + 16 * ks + 8 + 4 * g);
            f32x8 a, bb;
#pragma unroll
            for (int j = 0; j < 4; ++j) { a[j] = a0[j]; a[4 + j] = a1[j]; }
#pragma unroll
            for (int j = 0; j < 8; ++j) bb[j] = xs[ks >> 1][lane][8 * (ks & 1) + j];
            bf16x8 ah, al, bhi, blo;
            split_bf16(a, ah, al);
            split_bf16(bb, bhi, blo);
            acc = mma(ah, bhi, acc);
            acc = mma(ah, blo, acc);
            acc = mma(al, bhi, acc);
        }
        float* dst = prm.hs + ((size_t)bh * P + p) * SS;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int idx = (32 * w + rho(g, r)) * kDv + col;
            cur[r] = eG * acc[r] + bz[idx];
            dst[idx] = cur[r];
        }
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_combine(const FwdParams& p, hipStream_t s) {
    hipLaunchKernelGGL(combine_kernel, dim3(p.B * p.H, 4), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace gdn
