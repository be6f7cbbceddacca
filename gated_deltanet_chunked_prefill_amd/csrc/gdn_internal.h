// Host/device shared parameter blocks and the internal launchers behind the C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

// Workspace of the split forward, per head bh = b*H + h and segment slot p < P
// (P = the largest segment count the call may use; 256-byte aligned sub-buffers):
//   csum       [B, N, H]          sums of g per chunk (gate scan)
//   wmax       [LV, B*H] int32    largest window sum per window length level and head,
//                                 as order-preserving integer keys (LV = kMaxWindowLevels slots)
//   flags      [B*H] int32        0 = exact head, m >= 1 = window head of m*w chunks
//   maxwin     [B*H]              max window log-decay
//   hs         [B*H, P, dk, dv]   true state entering segment p (p >= 1) of an exact head
//   hs_cnt     [B*H, P] int32     parts of hs[bh, p] published (complete at 16)
//              (hs_cnt and tr_cnt are one block, reset by the first launch)
//   bz         [B*H, P, dk, dv]   final state of segment p run from a zero state
//   mt         [B*H, P, 2, dk, dk] bf16  gate-free transition of segment p, as hi and lo parts
//   eg         [B*H, P]           exp(sum of g over segment p)
//   tr_cnt     [B*H, P] int32     number of waves that have published bz, mt, eg of segment p
//   head_map   [2*B*H] int32      heads by exact rank, then by window rank
//   plan       FwdPlan            segment counts, job count, job counter
//   jobs       [B*H*(2P+3)] TaskRec  the work queue of the split forward
//
// A job is one run of the fused chunk loop over chunks [c_begin, c_end) of head
// bh, with outputs from chunk c_out on, or (mode = chain) the composition of
// the states entering segments seg+1 .. c_end of head bh.
constexpr int kMaxSegments = 1024;   // the device planner's limit on segments per head
constexpr int kMaxWindowLevels = 8;  // window lengths w, 2w, ..., 8w chunks at most

struct TaskRec {
    int bh, seg, c_begin, c_out, c_end, mode, init, dst;
};
struct FwdPlan {
    int P_e, P_w;      // segments of an exact head / the most segments of a window head
    int n_exact, n_window;
    int n_jobs;
    int next;          // next job to hand out (atomic counter)
    int error;         // set when a wait for another job's state ran out (never expected)
    int ready;         // job count + 1 once the job list is written
};

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
    int P;             // segment slots per head (1 = no split)
    int w;             // window length in chunks (level 1)
    int levels;        // window lengths tried: w, 2w, ..., levels * w (0 with no window heads)
    float scale;
    const int* wmax;       // split forward with window heads: largest window sum per window
                           // length and head [levels, B*H], as order-preserving integer keys
                           // (null: all heads exact)
    int* head_map;         // [2*B*H] planner scratch: heads by exact rank, then by window rank
    int32_t* flags;        // written by the planner: 0 = exact head, m = window head of m*w chunks
    float* maxwin;         // the largest window sum at length w
    float log_eps;
    float* hs;
    int* hs_cnt;
    float* bz;
    __bf16* mt;
    float* eg;
    int* tr_cnt;
    __bf16* hstore;    // nullable: [B*H, N+1, dv, dk] bf16, transposed: state entering each chunk,
                       // then the final state
    FwdPlan* plan;     // split forward: written by the plan kernel
    TaskRec* jobs;
    int cus;           // compute units of the device
    int forced;        // 1: every head uses exactly P segments of equal length
    const int* cu;     // packed sequences (PHASE_VARLEN, PHASE_STATES_VARLEN): token offsets
                       // [B+1] of the B sequences in a [1, T, H, d] batch; null otherwise
    int cmax;          // packed sequences: chunk slots per head, ceil(T/64) + B (bounds the
                       // chunks of all sequences together)
    const int* cstart; // packed sequences with kept states: chunk prefix [B+1], then the
                       // sequence bounds [B+1] (seq_span)
    int vseg;          // packed sequences without kept states: target chunks per segment
                       // (0 = one workgroup per sequence and head); P = segments at most
};

// Packed sequences: sequence s holds tokens [t0, t0 + len).  Without the chunk
// prefix, t0 = cu[s] and t0 + len = cu[s+1], both clamped to [0, T] (and the end
// to at least t0).  With it (the backward, cstart != null), the bounds are the
// ones the prefix launch wrote after the prefix, cstart[nseq + 1 + s] =
// max(0, clamp(cu[0]), .., clamp(cu[s])): non-decreasing, so the sequences are
// disjoint and their chunks fit the per-head slots even when cu_seqlens
// decreases.  nch = ceil(len / 64) chunks; c0 = cstart[s], the chunks of the
// sequences before it (its first chunk in a numbering of all chunks of the
// batch).
struct SeqSpan {
    int t0, len, nch, c0;
};
__host__ __device__ inline int clamp_tok(int x, int lo, int T) { return x < lo ? lo : (x > T ? T : x); }
__device__ inline SeqSpan seq_span(const int* cu, const int* cstart, int nseq, int T, int s) {
    SeqSpan r;
    if (cstart) {
        const int* const bnd = cstart + nseq + 1;
        r.t0 = __builtin_amdgcn_readfirstlane(bnd[s]);
        r.len = __builtin_amdgcn_readfirstlane(bnd[s + 1]) - r.t0;
        r.c0 = __builtin_amdgcn_readfirstlane(cstart[s]);
    } else {
        r.t0 = clamp_tok(__builtin_amdgcn_readfirstlane(cu[s]), 0, T);
        r.len = clamp_tok(__builtin_amdgcn_readfirstlane(cu[s + 1]), r.t0, T) - r.t0;
        r.c0 = 0;
    }
    r.nch = (r.len + 63) / 64;
    return r;
}

// PHASE_SINGLE: one workgroup per head, the whole sequence.
// PHASE_QUEUE: persistent workgroups running the jobs of the split forward.
// PHASE_QUEUE_STATES: the same, keeping the state entering every chunk (hstore,
// as PHASE_STATES) from the jobs that own the chunk's output.
// PHASE_STATES: the unsplit forward that only stores the state entering every
// chunk (into hstore), for the backward.
// PHASE_VARLEN: one workgroup per (sequence, head) of a packed batch (cu).
// PHASE_STATES_VARLEN: PHASE_STATES over a packed batch.
enum FwdPhase { PHASE_SINGLE = 0, PHASE_QUEUE = 1, PHASE_STATES = 2, PHASE_VARLEN = 3, PHASE_STATES_VARLEN = 4,
                PHASE_QUEUE_STATES = 5 };

hipError_t launch_fwd(const FwdParams& p, int phase, bool bf16, hipStream_t s);
// The forward's fixed scratch array (gdn_chunk_fwd_noalloc): its size, and its
// device address on the current device (looked up on the first call per device).
constexpr size_t kFwdScratchBytes = (size_t)64 << 20;
hipError_t fwd_scratch(void** ptr);
hipError_t launch_chunk_sums(const float* g, int B, int T, int H, float* chunk_sums, hipStream_t s);
int window_groups(int T);
int max_window_chunks();
hipError_t launch_fwd_sums(const float* g, int B, int T, int H, float* sums, int* zero, int nzero,
                           int* plan_words, int* wmax, int nwmax, hipStream_t s);
hipError_t launch_fwd_windows(const float* sums, int B, int T, int H, int w, int levels, int* wmax,
                              hipStream_t s);
// Order-preserving integer key of a float (signed comparison of keys = comparison
// of the floats), and back.
__host__ __device__ inline int float_key(float x) {
    const int b = __builtin_bit_cast(int, x);
    return b >= 0 ? b : b ^ 0x7FFFFFFF;
}
__host__ __device__ inline float key_float(int k) {
    return __builtin_bit_cast(float, k >= 0 ? k : k ^ 0x7FFFFFFF);
}
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
    const __bf16* hstore;  // [B*H, N+1, dv, dk] bf16, transposed: state entering each chunk, then
                           // the final state
    __bf16* dhstore;       // [B*H, N, dv, dk] bf16, transposed: gradient reaching the end of each chunk
    const int* cu;         // packed sequences: token offsets [B+1] (null: B sequences of length T)
    int cmax;              // packed sequences: chunk slots per head (see FwdParams)
    const int* cstart;     // packed sequences: chunk prefix [B+1], then the sequence bounds [B+1]
    // split state-gradient sweep: P segments of S chunks (the last shorter); ws:
    // per batch-head P slots of kStateSlot floats: slot s (1 <= s <= P-2) holds
    // segment s's map from the gradient at its end to the gradient at its start
    // (M, then b), and after the chain its b field holds the gradient at the end
    // of segment s - 1; slot P-1's b field receives the gradient at the start of
    // segment P-1, which runs from dht
    int P, S;
    float* ws;
};
// sweep launches: DH_FULL one workgroup per head over all chunks; DH_FIRST
// segment P-1 (from dht) beside the maps of segments 1 .. P-2; DH_REST segments
// 0 .. P-2 from the gradients the chain left
enum { DH_FULL = 0, DH_FIRST = 1, DH_REST = 2 };
// Per-key-channel-decay variant (KDA): g is [B, T, H, dk] float32 (one log-decay
// per key channel), q, k, v, o bf16; one workgroup per (batch, head).
struct KdaParams {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    const float* h0;   // nullable
    void* o;
    float* ht;         // nullable
    int B, T, H, N;
    float scale;
    // sequence split: P segments of S chunks (the last one shorter); P = 1 runs
    // unsplit.  ws: per batch-head bh, P - 1 slots (slot bh (P - 1) + p) of
    // kKdaSlot floats: for p >= 1 segment p's transition M (its linear state map,
    // [dk][dk]) and its state b from a zero start ([dk][dv]); the chain overwrites
    // each b field with the state entering segment p + 1; slot 0's b field
    // receives the final state of segment 0, which runs from h0 (float32,
    // row-major).
    int P, S;
    float* ws;
};
// one segment map of an exact split: M ([dk][dk]) then b ([dk][dv]), float32
constexpr size_t kStateSlot = 2 * 128 * 128;
constexpr size_t kKdaSlot = kStateSlot;
// The chain of segment maps (gdn_chain.hip): per batch-head `slots` slots; from
// the b field of slot `start`, for i = 1 .. count, slot cur = start + i * step:
// S = M_cur S + b_cur, written over b_cur.
struct ChainParams {
    float* ws;
    int slots, start, step, count;
};
hipError_t launch_state_chain(const ChainParams& p, int nbh, hipStream_t s);
// KDA_FULL: one segment per head (P = 1).  KDA_FIRST: segment 0 with outputs
// beside the transitions of segments 1 .. P-2 (P - 1 workgroups per head).
// KDA_REST: segments 1 .. P-1 with outputs from the states the chain left.
enum { KDA_FULL = 0, KDA_FIRST = 1, KDA_REST = 2 };
// Streaming probe of the forward's memory pattern (gdn_probe.hip).
hipError_t launch_stream_probe(const void* k, const void* q, const void* v, void* o, int T, int H, int segments,
                               hipStream_t s);
hipError_t launch_kda_fwd(const KdaParams& p, int mode, hipStream_t s);
// the states entering segments 2 .. P-1 from segment 0's final state and the
// transitions (segments in order; 16 state columns per workgroup)
hipError_t launch_kda_chain(const KdaParams& p, hipStream_t s);
size_t kda_smem_bytes();

// Packed sequences: the stored states of sequence s, head h sit at per-head slots
// h * (cmax + B) + c0 + s + c (c = 0 .. nch, the last being its final state) and
// the state gradients at h * cmax + c0 + c (c < nch).
hipError_t launch_bwd_dh(const BwdParams& p, bool bf16, hipStream_t s, int mode = DH_FULL);
// Packed sequences: cstart[s] = chunks of sequences 0 .. s-1, s = 0 .. B, then
// the bounds cstart[B + 1 + s] = max(0, clamp(cu[0]), .., clamp(cu[s])), s = 0 .. B.
hipError_t launch_seq_chunk_prefix(const int* cu, int B, int T, int* cstart, hipStream_t s);
hipError_t launch_bwd_local(const BwdParams& p, bool bf16, hipStream_t s);

}  // namespace gdn
