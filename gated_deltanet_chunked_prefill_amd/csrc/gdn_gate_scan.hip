// Gate scan for gfx950 (FlashQLA talk summary, onedev.kr, paragraph 5: one
// light kernel scans the gate distribution and marks the heads whose
// alpha-powers fall below a threshold within a window, so those heads can skip
// the sequence-split correction and warm up over one window instead).
//
// Two small launches, both bound by one read of g:
//   1. chunk sums s[b][c][h] = sum of g over the (up to) 64 tokens of chunk c;
//   2. per head (one workgroup): W_c = s_{c-w+1} + ... + s_c for c >= w-1 (each
//      window summed directly), its maximum over c, and flag = N >= w && max <= log_eps.
// The split forward forms the same chunk sums (fwd_sums_kernel) and window
// sums per group of chunks and window length (fwd_window_kernel) for its
// planner.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

// One workgroup per (chunk, batch).  The chunk's g values are one contiguous
// block of 64 x H floats; thread t reads the elements of head t % H in token
// order (group t / H takes every G-th token, G = 256 / H), so loads are
// coalesced, and the G partial sums of a head are added in a fixed order
// (results do not depend on scheduling).
__device__ void chunk_sums_wg(const float* __restrict__ g, int T, int H, int N, int c, int b,
                              float* __restrict__ sums) {
    __shared__ float part[256];
    const int tid = threadIdx.x;
    const int t0 = c * kChunk;
    const int nt = T - t0 < kChunk ? T - t0 : kChunk;
    const float* src = g + ((size_t)b * T + t0) * H;
    for (int h0 = 0; h0 < H; h0 += 256) {
        const int hw = H - h0 < 256 ? H - h0 : 256;   // heads in this pass
        const int G = 256 / hw;                        // token groups
        const int h = h0 + tid % hw, grp = tid / hw;
        float acc = 0.f;
        if (G >= 4 && grp < G) {
            // at most 16 tokens per thread: every load issued before the sum
            // (tokens past the chunk read as zero, which leaves the sum unchanged)
            float v[16];
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                const int t = grp + m * G;
                v[m] = t < nt ? src[(size_t)t * H + h] : 0.f;
            }
#pragma unroll
            for (int m = 0; m < 16; ++m) acc += v[m];
        } else if (grp < G) {
            for (int t = grp; t < nt; t += G) acc += src[(size_t)t * H + h];
        }
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

__global__ __launch_bounds__(256) void chunk_sums_kernel(const float* __restrict__ g, int T, int H,
                                                         int N, float* __restrict__ sums) {
    chunk_sums_wg(g, T, H, N, blockIdx.x, blockIdx.y, sums);
}

// First launch of the split forward: the reset of the planner's words and
// hand-off counters, which the persistent launch relies on, and (when window
// heads are considered) the chunk sums of g, one workgroup per chunk, in the
// arrangement and summation order of chunk_sums_kernel.
__global__ __launch_bounds__(256) void fwd_sums_kernel(const float* __restrict__ g, int T, int H, int N,
                                                       float* __restrict__ sums, int* __restrict__ zero,
                                                       int nzero, int* __restrict__ plan_words,
                                                       int* __restrict__ wmax, int nwmax) {
    const int tid = threadIdx.x;
    const int wg = blockIdx.y * gridDim.x + blockIdx.x, nwg = gridDim.x * gridDim.y;
    for (int i = wg * 256 + tid; i < nzero; i += nwg * 256) zero[i] = 0;
    for (int i = wg * 256 + tid; i < nwmax; i += nwg * 256) wmax[i] = float_key(-INFINITY);
    if (wg == 0 && tid < 16) plan_words[tid] = 0;   // the planner's words (at most 16)
    if (sums) chunk_sums_wg(g, T, H, N, blockIdx.x, blockIdx.y, sums);
}

// Second launch (window heads considered): window maxima per group of
// kWinGroup chunks for the window lengths W = m*w, m = 1 .. levels.  Workgroup
// (grp, b) stages the chunk sums of its chunks and of the levels*w - 1 chunks
// before them, then per head and length takes the largest window sum
// s_{c-W+1} + ... + s_c (summed in that order) over the windows ending in the
// group, folded into wmax[(m-1)*B*H + b*H + h] with an atomic maximum of
// order-preserving integer keys (the first launch set every entry to -inf).  At
// m = 1 the sums are those of window_flags_kernel, term for term.
constexpr int kWinGroup = 8;
constexpr int kWinMaxSums = 8192;   // LDS floats for the group's chunk sums
constexpr int kWinThreads = 512;    // one pass over the (head, length, end) triples of 32 heads
__global__ __launch_bounds__(kWinThreads) void fwd_window_kernel(const float* __restrict__ sums, int H, int N, int w,
                                                         int levels, int* __restrict__ wmax) {
    __shared__ float s_sum[kWinMaxSums];
    const int grp = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int c0 = grp * kWinGroup;
    const int c1 = c0 + kWinGroup < N ? c0 + kWinGroup : N;
    const int wl = levels * w;                          // longest window
    const int cs = c0 - wl + 1 > 0 ? c0 - wl + 1 : 0;   // first chunk a window needs
    const int nc = c1 - cs;
    const int hpass = kWinMaxSums / nc < H ? kWinMaxSums / nc : H;   // >= 1: nc <= kWinMaxSums
    for (int h0 = 0; h0 < H; h0 += hpass) {
        const int hn = H - h0 < hpass ? H - h0 : hpass;
        for (int i = tid; i < nc * hn; i += kWinThreads) {
            const int c = cs + i / hn, hl = i % hn;
            s_sum[(c - cs) * hpass + hl] = sums[((size_t)b * N + c) * H + h0 + hl];
        }
        __syncthreads();
        // one thread per (head, length, window end); the kWinGroup ends of a
        // (head, length) pair sit in adjacent lanes and are reduced by shuffles
        const int ntask = hn * levels * kWinGroup;
        for (int x0 = 0; x0 < ntask; x0 += kWinThreads) {
            const int x = x0 + tid, e = x % kWinGroup, pr = x / kWinGroup;
            const int hl = pr % hn, m = 1 + pr / hn, W = m * w, c = c0 + e;
            float acc = -INFINITY;
            if (x < ntask && c < c1 && c >= W - 1) {
                // summed left to right; the unrolled loop issues the LDS reads
                // ahead of the dependent additions
                acc = 0.f;
                const float* src = s_sum + (c - W + 1 - cs) * hpass + hl;
#pragma unroll 8
                for (int j = 0; j < W; ++j) acc += src[j * hpass];
            }
#pragma unroll
            for (int d = 1; d < kWinGroup; d <<= 1) {
                const float o = __shfl_xor(acc, d, 64);
                acc = o > acc ? o : acc;
            }
            if (x < ntask && e == 0 && acc > -INFINITY)
                atomicMax(&wmax[((size_t)(m - 1) * gridDim.y + b) * H + h0 + hl], float_key(acc));
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

int window_groups(int T) { return ((T + kChunk - 1) / kChunk + kWinGroup - 1) / kWinGroup; }
int max_window_chunks() { return kWinMaxSums - kWinGroup + 1; }

hipError_t launch_fwd_sums(const float* g, int B, int T, int H, float* sums, int* zero, int nzero,
                           int* plan_words, int* wmax, int nwmax, hipStream_t s) {
    const int N = (T + kChunk - 1) / kChunk;
    dim3 grid(sums ? N : 1, sums ? B : 1);
    hipLaunchKernelGGL(fwd_sums_kernel, grid, dim3(256), 0, s, g, T, H, N, sums, zero, nzero, plan_words, wmax,
                       nwmax);
    return hipGetLastError();
}
hipError_t launch_fwd_windows(const float* sums, int B, int T, int H, int w, int levels, int* wmax,
                              hipStream_t s) {
    const int N = (T + kChunk - 1) / kChunk;
    dim3 grid(window_groups(T), B);
    hipLaunchKernelGGL(fwd_window_kernel, grid, dim3(kWinThreads), 0, s, sums, H, N, w, levels, wmax);
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
