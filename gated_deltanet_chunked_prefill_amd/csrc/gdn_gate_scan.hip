// Gate scan for gfx950 (FlashQLA talk summary, onedev.kr, paragraph 5: one
// light kernel scans the gate distribution and marks the heads whose
// alpha-powers fall below a threshold within a window, so those heads can skip
// the sequence-split correction and warm up over one window instead).
//
// Two small launches, both bound by one read of g:
//   1. chunk sums s[b][c][h] = sum of g over the (up to) 64 tokens of chunk c;
//   2. per head (one workgroup): W_c = s_{c-w+1} + ... + s_c for c >= w-1 (each
//      window summed directly), its maximum over c, and flag = N >= w && max <= log_eps.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

// One workgroup per (chunk, batch).  The chunk's g values are one contiguous
// block of 64 x H floats; thread t reads the elements of head t % H in token
// order (group t / H takes every G-th token, G = 256 / H), so loads are
// coalesced, and the G partial sums of a head are added in a fixed order
// (results do not depend on scheduling).
__global__ __launch_bounds__(256) void chunk_sums_kernel(const float* __restrict__ g, int T, int H,
                                                         int N, float* __restrict__ sums) {
    __shared__ float part[256];
    const int c = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int t0 = c * kChunk;
    const int nt = T - t0 < kChunk ? T - t0 : kChunk;
    const float* src = g + ((size_t)b * T + t0) * H;
    for (int h0 = 0; h0 < H; h0 += 256) {
        const int hw = H - h0 < 256 ? H - h0 : 256;   // heads in this pass
        const int G = 256 / hw;                        // token groups
        const int h = h0 + tid % hw, grp = tid / hw;
        float acc = 0.f;
        if (grp < G)
            for (int t = grp; t < nt; t += G) acc += src[(size_t)t * H + h];
        part[tid] = acc;
        __syncthreads();
        if (tid < hw) {
            float s = 0.f;
            for (int q = 0; q < G; ++q) s += part[q * hw + tid];
            sums[((size_t)b * N + c) * H + h0 + tid] = s;
        }
        __syncthreads();
    }
}

// One workgroup per head: each thread sums the windows ending at its chunks,
// then the workgroup takes the maximum.
__global__ __launch_bounds__(256) void window_flags_kernel(const float* __restrict__ sums, int B,
                                                           int H, int N, int w, float log_eps,
                                                           int32_t* __restrict__ flags,
                                                           float* __restrict__ maxwin) {
    __shared__ float red[256];
    const int bh = blockIdx.x;
    const int b = bh / H, h = bh % H;
    float best = -INFINITY;
    for (int c = w - 1 + (int)threadIdx.x; c < N; c += blockDim.x) {
        float acc = 0.f;
        for (int j = c - w + 1; j <= c; ++j) acc += sums[((size_t)b * N + j) * H + h];
        best = acc > best ? acc : best;
    }
    red[threadIdx.x] = best;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + s]);
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        best = red[0];
        flags[bh] = (N >= w && best <= log_eps) ? 1 : 0;
        if (maxwin) maxwin[bh] = best;
    }
}

}  // namespace

hipError_t launch_chunk_sums(const float* g, int B, int T, int H, float* chunk_sums, hipStream_t s) {
    const int N = (T + kChunk - 1) / kChunk;
    dim3 grid(N, B);
    hipLaunchKernelGGL(chunk_sums_kernel, grid, dim3(256), 0, s, g, T, H, N, chunk_sums);
    return hipGetLastError();
}

hipError_t launch_window_flags(const float* chunk_sums, int B, int T, int H, int w, float log_eps,
                               int32_t* flags, float* maxwin, hipStream_t s) {
    const int N = (T + kChunk - 1) / kChunk;
    dim3 grid(B * H);
    hipLaunchKernelGGL(window_flags_kernel, grid, dim3(256), 0, s, chunk_sums, B, H, N, w,
                       log_eps, flags, maxwin);
    return hipGetLastError();
}

}  // namespace gdn
