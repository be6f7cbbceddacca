// Host/device shared parameter blocks and the internal launchers behind the C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

// Workspace of the split forward, per head bh = b*H + h and segment p
// (all float32, 256-byte aligned sub-buffers):
//   chunk_sums [B, N, H]          gate scan scratch
//   flags      [B*H] int32        1 = window head
//   maxwin     [B*H]              max window log-decay
//   hs         [B*H, P, dk, dv]   true state entering segment p (p >= 1)
//   bz         [B*H, P, dk, dv]   final state of segment p run from zero
//   mt         [B*H, P, dk, dk]   gate-free segment transition (prod of I - K^T T0 diag(beta) K)
//   gsum       [B*H, P]           sum of g over segment p
struct FwdParams {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    const float* h0;   // nullable
    void* o;
    float* ht;         // nullable
    int B, T, H, N;    // N = number of 64-token chunks
    int P;             // segments per head (1 = no split)
    int w;             // window length in chunks
    float scale;
    const int32_t* flags;  // nullable: all heads exact
    float* hs;
    float* bz;
    float* mt;
    float* gsum;
    float* hstore;     // nullable: [B*H, N+1, dk, dv] state entering each chunk, then the final state
};

// PHASE_STATES: the unsplit forward that only stores the state entering every
// chunk (into hstore), for the backward.
enum FwdPhase { PHASE_SINGLE = 0, PHASE_A = 1, PHASE_C = 2, PHASE_STATES = 3 };

hipError_t launch_fwd(const FwdParams& p, int phase, bool bf16, hipStream_t s);
hipError_t launch_combine(const FwdParams& p, hipStream_t s);
hipError_t launch_chunk_sums(const float* g, int B, int T, int H, float* chunk_sums, hipStream_t s);
hipError_t launch_window_flags(const float* chunk_sums, int B, int T, int H, int w, float log_eps,
                               int32_t* flags, float* maxwin, hipStream_t s);

struct BwdParams {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    const float* h0;
    const void* dout;
    const float* dht;     // nullable: no gradient on the final state
    void* dq;
    void* dk;
    void* dv;
    float* dg;
    float* dbeta;
    float* dh0;           // nullable
    int B, T, H, N;
    float scale;
    const float* hstore;  // [B*H, N+1, dk, dv] state entering each chunk, then the final state
    float* dhstore;       // [B*H, N, dk, dv] gradient reaching the end of each chunk
};
hipError_t launch_bwd_dh(const BwdParams& p, bool bf16, hipStream_t s);
hipError_t launch_bwd_local(const BwdParams& p, bool bf16, hipStream_t s);

}  // namespace gdn
