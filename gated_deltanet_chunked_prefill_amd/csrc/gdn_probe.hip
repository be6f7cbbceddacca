// Streaming probe of the fused forward's memory pattern (a measurement aid, not
// part of the operator).  The talk summary (FlashQLA, onedev.kr, paragraph 7)
// argues the fused forward is bound by memory traffic; this kernel moves the
// forward's bytes in the forward's layout with no arithmetic, so the bandwidth it
// reaches is the ceiling that layout and this hardware leave to the real kernel.
//
// One workgroup (eight waves) per (head, segment) walks the segment's 64-token
// chunks in order.  Per chunk it copies the K, Q and V tiles (64 rows of 256
// bytes, rows H*256 bytes apart in a [T, H, 128] bf16 tensor) into LDS with
// direct loads, waits for them, and writes the previous chunk's V tile back as
// that chunk's 64 x 128 output tile with 16-byte stores: three reads and one
// write per token-head, as the forward.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int kProbeThreads = 512;
constexpr int kProbeTile = kChunk * kDk;   // elements of one 64 x 128 tile

__global__ __launch_bounds__(kProbeThreads, 1) void gdn_stream_probe_kernel(const __bf16* k, const __bf16* q,
                                                                          const __bf16* v, __bf16* o, int H,
                                                                          int chunks_per_wg) {
    extern __shared__ __attribute__((aligned(16))) char smem_raw[];
    __bf16* const lds = reinterpret_cast<__bf16*>(smem_raw);   // [2 buffers][K, Q, V tiles]
    const int h = (int)blockIdx.x % H, seg = (int)blockIdx.x / H;
    const int tid = threadIdx.x;
    const int c0 = seg * chunks_per_wg;
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    for (int i = 0; i < chunks_per_wg; ++i) {
        const int c = c0 + i;
        __bf16* const buf = lds + (i & 1) * 3 * kProbeTile;
        // 1024 pieces of 16 bytes per tile: two rounds of 512 threads
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int L = r * kProbeThreads + tid, row = L >> 4, piece = L & 15;
            const size_t off = ((size_t)(c * kChunk + row) * H + h) * kDk + 8 * piece;
            // wave-uniform LDS base: this wave's 64 pieces are consecutive
            __bf16* const dst = buf + (r * kProbeThreads + (tid & ~63)) * 8;
            __builtin_amdgcn_global_load_lds((const void*)(k + off), (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
            __builtin_amdgcn_global_load_lds((const void*)(q + off),
                                             (__attribute__((address_space(3))) void*)(dst + kProbeTile), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((const void*)(v + off),
                                             (__attribute__((address_space(3))) void*)(dst + 2 * kProbeTile), 16, 0, 0);
        }
        if (i > 0) {
            // the previous chunk's output tile, from its V tile in the other buffer
            const __bf16* const src = lds + ((i - 1) & 1) * 3 * kProbeTile + 2 * kProbeTile;
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int L = r * kProbeThreads + tid, row = L >> 4, piece = L & 15;
                const size_t off = ((size_t)((c - 1) * kChunk + row) * H + h) * kDk + 8 * piece;
                const u4 x = *reinterpret_cast<const u4*>(src + L * 8);
                *(__attribute__((address_space(1))) u4*)(o + off) = x;
            }
        }
        __builtin_amdgcn_s_waitcnt(0x3f70);   // vmcnt(0): this chunk's tiles are in LDS
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_stream_probe(const void* k, const void* q, const void* v, void* o, int T, int H, int segments,
                               hipStream_t s) {
    const size_t lds = 2 * 3 * kProbeTile * sizeof(__bf16);
    static bool configured = false;
    if (!configured) {
        const hipError_t e = hipFuncSetAttribute((const void*)gdn_stream_probe_kernel,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        configured = true;
    }
    const int chunks_per_wg = T / kChunk / segments;
    hipLaunchKernelGGL(gdn_stream_probe_kernel, dim3(H * segments), dim3(kProbeThreads), lds, s,
                       (const __bf16*)k, (const __bf16*)q, (const __bf16*)v, (__bf16*)o, H, chunks_per_wg);
    return hipGetLastError();
}

}  // namespace gdn
