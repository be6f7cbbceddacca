// Sequential composition of segment maps S_next = M S + b (the chain step of an
// exact sequence split, talk summary paragraph 4: each segment acts on the state
// entering it as an affine map, so the states entering all segments follow from
// the maps in order).  Used by the KDA forward (states forward in time) and by
// the backward's state-gradient sweep (gradients backward in time).
//
// Workspace: per batch-head bh, `slots` slots of kStateSlot floats; slot i holds
// a map's M ([dk][dk], row-major) and then b ([dk][dv]).  The chain starts from
// the b field of slot `start` and, for i = 1 .. count, composes cur = start +
// i * step: S = M_cur S + b_cur, written over b_cur.  In float32 on the vector
// units: columns of S never mix, so workgroup (batch-head, column block cb) owns
// 16 of the 128 columns, its S block stays in LDS across the links, and thread t
// owns row t >> 1, columns 16 cb + 8 (t & 1) .. +7 of every product; each thread
// holds its row of M_cur in registers, fetched one link ahead with its entries
// of b_cur.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int kChainCols = 16;
constexpr int kChainThreads = 2 * kDk;

__global__ __launch_bounds__(kChainThreads, 1) void state_chain_kernel(ChainParams prm) {
    __shared__ __attribute__((aligned(16))) float Sl[kDk * kChainCols];   // [k][16 columns]
    constexpr int CB = kDv / kChainCols;
    const int bh = (int)blockIdx.x / CB, cb = (int)blockIdx.x % CB, t = threadIdx.x;
    const int i = t >> 1, jl = 8 * (t & 1), j0 = kChainCols * cb + jl;
    const size_t MM = (size_t)kDk * kDk;
    float* const base = prm.ws + (size_t)bh * prm.slots * kStateSlot;
    const float* const S0 = base + (size_t)prm.start * kStateSlot + MM;
#pragma unroll
    for (int c = 0; c < 8; ++c) Sl[i * kChainCols + jl + c] = S0[(size_t)i * kDv + j0 + c];
    f32x4 mnext[kDk / 4];
    float bnext[8];
    if (prm.count > 0) {
        const float* const M1 = base + (size_t)(prm.start + prm.step) * kStateSlot;
#pragma unroll
        for (int q = 0; q < kDk / 4; ++q) mnext[q] = *reinterpret_cast<const f32x4*>(M1 + (size_t)i * kDk + 4 * q);
#pragma unroll
        for (int c = 0; c < 8; ++c) bnext[c] = M1[MM + (size_t)i * kDv + j0 + c];
    }
    __syncthreads();
    for (int n = 1; n <= prm.count; ++n) {
        float* const bp = base + (size_t)(prm.start + n * prm.step) * kStateSlot + MM;
        float acc[8];
        f32x4 m[kDk / 4];
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = bnext[c];
#pragma unroll
        for (int q = 0; q < kDk / 4; ++q) m[q] = mnext[q];
        if (n < prm.count) {
            const float* const Mn = base + (size_t)(prm.start + (n + 1) * prm.step) * kStateSlot;
#pragma unroll
            for (int q = 0; q < kDk / 4; ++q) mnext[q] = *reinterpret_cast<const f32x4*>(Mn + (size_t)i * kDk + 4 * q);
#pragma unroll
            for (int c = 0; c < 8; ++c) bnext[c] = Mn[MM + (size_t)i * kDv + j0 + c];
        }
#pragma unroll
        for (int k = 0; k < kDk; ++k) {
            const float mk = m[k >> 2][k & 3];
            const f32x4 s0 = *reinterpret_cast<const f32x4*>(Sl + k * kChainCols + jl);
            const f32x4 s1 = *reinterpret_cast<const f32x4*>(Sl + k * kChainCols + jl + 4);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                acc[c] = __builtin_fmaf(mk, s0[c], acc[c]);
                acc[4 + c] = __builtin_fmaf(mk, s1[c], acc[4 + c]);
            }
        }
        __syncthreads();   // every product has read S
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            Sl[i * kChainCols + jl + c] = acc[c];
            bp[(size_t)i * kDv + j0 + c] = acc[c];
        }
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_state_chain(const ChainParams& p, int nbh, hipStream_t s) {
    if (p.count <= 0) return hipSuccess;
    hipLaunchKernelGGL(state_chain_kernel, dim3(nbh * (kDv / kChainCols)), dim3(kChainThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace gdn
