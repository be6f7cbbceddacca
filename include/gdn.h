/*
 * gdn.h - C ABI of the MI355X (gfx950) Gated DeltaNet chunked-prefill library.
 *
 * The operator (per batch b and head h, tokens t = 0..T-1):
 *     S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,
 *     o_t = scale * S_t^T q_t,         alpha_t = exp(g_t),
 * the gated delta rule of Gated DeltaNet.  The FlashQLA pages describe it as
 * linear attention with a d x d state updated token by token (talk summary,
 * onedev.kr, paragraph 2), a forget gate alpha in (0,1) and L2-normalised keys
 * (paragraph 5), evaluated chunk-wise in WY form (paragraph 3).  The state S is
 * stored as a dk x dv matrix ("h"), so o_t[j] = scale * sum_i q_t[i] h_t[i][j].
 *
 * Conventions for every entry point below
 *   - Tensor pointers are DEVICE pointers to contiguous row-major arrays;
 *     q, k, v, o, dout, dq, dk, dv must be 16-byte aligned, the float32 tensors
 *     4-byte aligned:
 *         q, k, dq, dk          [B, T, H, dk]   in the I/O dtype
 *         v, o, dout, dv        [B, T, H, dv]   in the I/O dtype
 *         g, beta, dg, dbeta    [B, T, H]       float32 (g = log alpha <= 0)
 *         h0, ht, dht, dh0      [B, H, dk, dv]  float32
 *   - Only dk = dv = 128 is supported (GDN_ERR_UNSUPPORTED otherwise).  T >= 1 is
 *     arbitrary: the last 64-token chunk may be short.  B*T*H*128 <= 2^40, and the
 *     64 rows of one chunk of one head must span less than 2^31 bytes
 *     (64 * H * 128 * element size < 2^31: H < 131072 for bfloat16, H < 65536 for
 *     float32); larger shapes are rejected with GDN_ERR_INVALID_ARG.
 *   - The op neither normalises q, k nor squashes beta.  The sliding-window
 *     shortcut assumes ||k_t|| <= 1 and 0 <= beta_t <= 2 (then each per-token map
 *     I - beta k k^T has spectral norm <= 1).
 *   - Ownership: the caller owns every buffer, including the workspace.  The
 *     library allocates no device memory and keeps no pointer after returning.
 *   - Asynchrony: all work is enqueued on `stream` (a hipStream_t; NULL = the
 *     default stream) and the call returns without synchronising.  The launch
 *     plan depends on the shapes only; per-head choices read device data.
 *   - Errors: arguments are validated before anything is launched; a non-OK
 *     status means nothing was enqueued, except GDN_ERR_HIP, which reports a
 *     failed launch (hipGetLastError) after earlier launches of the same call
 *     may have been enqueued.  gdn_last_error() returns a thread-local message
 *     for the last non-OK status on the calling thread.  No C++ exception
 *     crosses this boundary.
 *   - Calls that share a workspace or outputs must be ordered by the caller
 *     (e.g. the same stream).
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDN_OK = 0,
    GDN_ERR_INVALID_ARG = 1, /* null required pointer, non-positive size, misalignment, bad option */
    GDN_ERR_UNSUPPORTED = 2, /* dk or dv != 128, unknown dtype                                       */
    GDN_ERR_WORKSPACE = 3,   /* workspace smaller than the matching *_workspace_size() query         */
    GDN_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed                           */
} gdn_status;

typedef enum {
    GDN_F32 = 0,  /* q, k, v, o (and dout, dq, dk, dv) in float32  */
    GDN_BF16 = 1  /* the same tensors in bfloat16                   */
} gdn_dtype;

/* Forward options.  Pass NULL for the defaults (gdn_default_options). */
typedef struct {
    /* Intra-GPU sequence split (talk summary, paragraph 4: split the sequence
     * so that few heads still fill the GPU; each segment recurs from a zero
     * state and a dk x dk correction is composed associatively).
     *   0 = automatic segment count from the shapes (paragraph 8: a square-root
     *       rule on the chunk count; see gdn_plan_segments),
     *   1 = off (one segment per head),
     *   2 = use n_segments. */
    int split_mode;
    int n_segments;     /* used when split_mode == 2; 1 <= n_segments <= min(number of chunks, 1024) */
    /* Sliding-window heads (paragraph 5): when 1 and the sequence is split, heads
     * whose every window of window_chunks chunks decays by at least exp(log_eps)
     * skip the correction and warm up from a zero state over the previous
     * window_chunks chunks.  0 = always exact. */
    int use_window;
    int window_chunks;  /* w >= 1, default 8 (the page 1 commentary quotes a 6-8 chunk warm-up) */
    float log_eps;      /* default log(2^-24)                                                    */
    /* Per-head window length (talk summary, paragraph 8, lists fixed window
     * rules as an open problem): the forward tries the lengths w, 2w, ...,
     * window_levels * w chunks and gives each head the shortest one whose every
     * window decays by at least exp(log_eps); a head that none satisfies stays
     * exact.  1 = the single length w.  1 <= window_levels <= 8, default 4;
     * lengths beyond the first launch's staging limit are not tried. */
    int window_levels;
} gdn_options;

/* Fill *opt with the defaults: automatic split, window shortcut on, w = 8,
 * log_eps = log(2^-24), window_levels = 4. */
void gdn_default_options(gdn_options* opt);

/* Segment slots per head of the forward for these shapes on a device with
 * num_cus compute units (the host-side planner; no device access): 1 when the
 * sequence is not split; n_segments (at most the chunk count) when
 * split_mode == 2; otherwise 1 when B*H >= num_cus or N < 2 * window_chunks, else
 * the most segments the device-side planner may give a head,
 * min(32, floor(sqrt(N)), N/2) for N chunks (its makespan model may still keep
 * heads unsplit).  That planner reads the
 * window flags and picks the counts of exact and window heads per call (see
 * gdn_chunk_fwd_plan_info).  Returns 0 for invalid arguments. */
int gdn_plan_segments(int B, int T, int H, int num_cus, const gdn_options* opt);

/* Read back the plan the last split forward with these shapes, options and
 * workspace used (synchronises `stream`).  info[0..7]: segments of an exact
 * head, segments of a window head, number of exact heads, number of window
 * heads, number of jobs, requests made to the job counter (a workgroup's first
 * job is its index; each later request, including one final empty request per
 * workgroup that ran a job, goes through the counter), error flag (nonzero: a
 * wait for another job's state ran out; the outputs are then invalid), and the
 * number of jobs + 1 once the plan was written.  Without a split:
 * {1, 1, B*H, 0, B*H, 0, 0, 0}; the workspace is not read then. */
gdn_status gdn_chunk_fwd_plan_info(int B, int T, int H, const gdn_options* opt, const void* workspace,
                                   int32_t* info, void* stream);

/* Workspace bytes gdn_chunk_fwd needs for these shapes on the current device
 * (0 when the sequence is not split).  Returns (size_t)-1 for invalid arguments. */
size_t gdn_chunk_fwd_workspace_size(int B, int T, int H, int dk, int dv, gdn_dtype dtype,
                                    const gdn_options* opt);

/* Fused chunked forward (talk summary, paragraph 3: per 64-token chunk, the
 * K K^T inverse, W and U, the state pass and the output, fused so that W, U and
 * the state never reach HBM; paragraphs 4-6: sequence split, window heads and
 * gate scaling pulled outside the inverse).
 *   q, k, v, g, beta  inputs (required)
 *   h0                initial state or NULL (zero state)
 *   o                 output [B,T,H,dv] (required)
 *   ht                final state or NULL (not written)
 *   scale             multiplies every output (1.0 for the plain operator)
 *   opt               NULL for defaults
 *   workspace         device memory of at least gdn_chunk_fwd_workspace_size()
 *                     bytes, 256-byte aligned (may be NULL when that size is 0)
 * Returns GDN_OK or an error status (see the conventions above). */
gdn_status gdn_chunk_fwd(const void* q, const void* k, const void* v, const float* g,
                         const float* beta, const float* h0, void* o, float* ht, int B, int T,
                         int H, int dk, int dv, gdn_dtype dtype, float scale,
                         const gdn_options* opt, void* workspace, size_t workspace_bytes,
                         void* stream);

/* Bytes of the fixed scratch array gdn_chunk_fwd_noalloc uses on each GPU. */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* gdn_chunk_fwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same arguments and results without a workspace argument.  The call makes no
 * hipMalloc, hipFree or other allocating call.  The split forward's scratch
 * (what gdn_chunk_fwd keeps in its workspace) lives in a fixed device array of
 * GDN_NOALLOC_SCRATCH_BYTES bytes that the library holds on every GPU it runs on
 * until the process ends; its address is looked up once per device, on the
 * first call with that device current.  Everything the kernels need cleared is
 * cleared by the call's own first kernel.
 * Limit: with split_mode == 2, a segment count whose scratch exceeds the array
 * is rejected with GDN_ERR_WORKSPACE; the automatic plan uses at most as many
 * segment slots per head as fit (none, i.e. the unsplit forward, if even two do
 * not), so its results can differ from gdn_chunk_fwd's by rounding only.
 * Every call on one GPU shares that GPU's array: calls that overlap in time on
 * the same GPU (different streams, or threads without ordering) race and give
 * wrong results; order them (e.g. one stream).  Errors as for gdn_chunk_fwd. */
gdn_status gdn_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* g,
                                 const float* beta, const float* h0, void* o, float* ht, int B, int T,
                                 int H, int dk, int dv, gdn_dtype dtype, float scale,
                                 const gdn_options* opt, void* stream);

/* Fused chunked forward over a packed batch of variable-length sequences (the
 * chunked-prefill serving shape: several prompts of different lengths in one
 * call; the same chunk-wise computation as gdn_chunk_fwd, talk summary
 * paragraph 3, applied to each sequence on its own).
 *   q, k, v, o        [T, H, dk|dv] in the I/O dtype: the sequences one after another
 *   g, beta           [T, H] float32
 *   cu_seqlens        DEVICE pointer, int32 [n_seqs + 1]: sequence s holds tokens
 *                     cu_seqlens[s] .. cu_seqlens[s+1] - 1 (required: non-decreasing,
 *                     cu_seqlens[0] = 0, cu_seqlens[n_seqs] = T).  The values are read
 *                     on the device and clamped to [0, T] (the end of a sequence to at
 *                     least its start), so no access leaves the tensors whatever they
 *                     hold; a decreasing cu_seqlens makes sequences overlap, and the
 *                     output rows they share are then written more than once
 *                     (unspecified values).  An empty sequence leaves its final state
 *                     equal to its initial state.
 *   h0                initial states [n_seqs, H, dk, dv] float32, or NULL (zero)
 *   ht                final states [n_seqs, H, dk, dv] float32, or NULL (not written)
 *   scale             multiplies every output
 * Chunks never cross a sequence boundary (each sequence's last chunk may be
 * short).  A sequence longer than the per-CU share of all chunks
 * (max(2 * window_chunks, ceil(ceil(T/64) * H / CUs)) chunks, default options) is
 * cut into up to 16 segments of about that length (talk summary, paragraph 4);
 * the cut is taken on the device from the sequence's length.  A later segment
 * starts from the zero state m * window_chunks chunks before its first output
 * chunk, for the smallest m in 1, 2, 4, 8 whose sum of g over those chunks (this
 * head, this sequence) is at most log_eps (the window shortcut of paragraph 5,
 * decided per segment), and otherwise runs from the sequence's start (exact).
 * One workgroup per (segment, sequence, head).  No workspace.  Errors as for
 * gdn_chunk_fwd; tokens outside every sequence are neither read nor written. */
gdn_status gdn_chunk_fwd_varlen(const void* q, const void* k, const void* v, const float* g,
                                const float* beta, const float* h0, void* o, float* ht,
                                const int32_t* cu_seqlens, int n_seqs, int T, int H, int dk, int dv,
                                gdn_dtype dtype, float scale, void* stream);

/* Chunked forward of the per-key-channel-decay variant (KDA; the FlashQLA
 * commentary names it, in its "kernel innovation" section, as the library's
 * sibling operator of GDN, without printing its recurrence).  The reading:
 *     S_t = (I - beta_t k_t k_t^T) diag(exp(g_t)) S_{t-1} + beta_t k_t v_t^T,
 *     o_t = scale * S_t^T q_t,
 * with one log-decay per key channel, g_t in R^dk, applied to the state before
 * the delta correction; with equal channels it is gdn_chunk_fwd's operator.
 *   q, k, v, o        as for gdn_chunk_fwd, bfloat16 only (GDN_ERR_UNSUPPORTED otherwise)
 *   g                 [B, T, H, dk] float32, log-decays (<= 0) per key channel;
 *                     H at most 65535 (GDN_ERR_INVALID_ARG beyond: 64 rows of
 *                     gates are addressed with 32-bit byte offsets)
 *   beta, h0, ht      as for gdn_chunk_fwd (h0, ht nullable)
 *   n_segments        sequence split (talk summary, paragraph 4): 1 = one
 *                     workgroup per (batch, head) over all chunks in order;
 *                     k >= 2 = k segments of ceil(N / k) chunks (N = ceil(T/64),
 *                     fewer when the last ones would be empty); 0 = automatic
 *                     (gdn_kda_plan_segments with the current device's CU count).
 *                     At most 1024.
 *   workspace         device memory of gdn_kda_fwd_workspace_size() bytes,
 *                     256-byte aligned (NULL allowed when that size is 0)
 * The chunk step applies the per-channel decay factors to the K and Q tiles
 * (re-centred per 32-token half, and at the half boundary for the block that
 * couples the halves), so results are finite as long as no key channel decays
 * by more than exp(-88) (the float32 exponent range) over 16 consecutive tokens
 * of a 64-token chunk.
 * With P > 1 segments the split is exact (no window shortcut): the chunk map is
 * affine in the state, S_out = M S_in + b.  A first launch runs segment 0 with
 * outputs from h0 (its final state goes to the workspace) beside segments
 * 1 .. P-2 from the identity and from zero, which give each segment's M (dk x
 * dk) and b (float32, in the workspace); a second composes them in order into
 * the state entering every segment; the third runs segments 1 .. P-1 with
 * outputs from those states.  Results differ from the unsplit call by rounding
 * only.
 * Errors as for gdn_chunk_fwd; GDN_ERR_WORKSPACE when the workspace is missing
 * or too small. */
gdn_status gdn_kda_fwd(const void* q, const void* k, const void* v, const float* g, const float* beta,
                       const float* h0, void* o, float* ht, int B, int T, int H, int dk, int dv, gdn_dtype dtype,
                       float scale, int n_segments, void* workspace, size_t workspace_bytes, void* stream);

/* Segments per head gdn_kda_fwd uses for these shapes on a device with num_cus
 * compute units (host only), N = ceil(T/64): 1 for n_segments = 1;
 * min(n_segments, N) reduced to ceil(N / ceil(N / n_segments)) for
 * n_segments >= 2; for n_segments = 0, a + 1 reduced the same way, with
 * a = min(16, floor(num_cus / (B H)), floor(N / 8) - 1), when a >= 2, else 1 (a
 * workgroups per head then run in each launch with outputs).  Returns 0 for
 * invalid arguments (num_cus is read only when n_segments = 0). */
int gdn_kda_plan_segments(int B, int T, int H, int num_cus, int n_segments);

/* Workspace bytes gdn_kda_fwd needs on the current device: B H (P - 1) x 2 x
 * 128 x 128 float32 values for P segments per head (0 when P = 1).  Returns
 * (size_t)-1 for invalid arguments. */
size_t gdn_kda_fwd_workspace_size(int B, int T, int H, int dk, int dv, int n_segments);

/* Workspace bytes for gdn_chunk_bwd_varlen ((size_t)-1 for invalid arguments):
 * the chunk prefix and bounds of the sequences, and per head (ceil(T/64) + 2 n_seqs)
 * bfloat16 128 x 128 states plus (ceil(T/64) + n_seqs) state gradients. */
size_t gdn_chunk_bwd_varlen_workspace_size(int n_seqs, int T, int H, int dk, int dv, gdn_dtype dtype);

/* Backward of gdn_chunk_fwd_varlen (packed variable-length sequences, same
 * layouts): gradients of L given dL/do = dout [T, H, dv] and dL/dht = dht
 * [n_seqs, H, dk, dv] (NULL = 0), each sequence on its own as in
 * gdn_chunk_bwd.  grad_q, grad_k, grad_v [T, H, ..] (I/O dtype), grad_g,
 * grad_beta [T, H] float32, grad_h0 [n_seqs, H, dk, dv] float32 or NULL.
 * cu_seqlens as for gdn_chunk_fwd_varlen (device, read on the device; tokens
 * outside every sequence are not written).  Here the bounds are made
 * non-decreasing on the device before use: sequence s runs from
 * max(cu_seqlens[0..s]) to max(cu_seqlens[0..s+1]) (each value clamped to [0, T]),
 * which is the given sequence whenever cu_seqlens is valid and keeps every
 * workspace slot in bounds when it is not.  bf16 I/O only.  workspace: at
 * least gdn_chunk_bwd_varlen_workspace_size() bytes, 256-byte aligned.  Runs a
 * one-workgroup chunk-prefix launch, then the launches of gdn_chunk_bwd (the
 * state store and the state-gradient sweep side by side on the library's side
 * stream) with one workgroup per (sequence, head) or per (head, chunk). */
gdn_status gdn_chunk_bwd_varlen(const void* q, const void* k, const void* v, const float* g,
                                const float* beta, const float* h0, const void* dout, const float* dht,
                                void* grad_q, void* grad_k, void* grad_v, float* grad_g,
                                float* grad_beta, float* grad_h0, const int32_t* cu_seqlens, int n_seqs,
                                int T, int H, int dk, int dv, gdn_dtype dtype, float scale,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes for gdn_chunk_bwd on the current device ((size_t)-1 for
 * invalid arguments): B*H*(2N+1) bfloat16 128 x 128 matrices (N = number of
 * 64-token chunks), the state entering every chunk plus the final state, and the
 * state gradient reaching the end of every chunk; when the sweep is split
 * (gdn_chunk_bwd_plan_segments > 1) also the split forward's workspace and
 * B*H*P slots of 2 x 128 x 128 float32 values.  Without a device: the unsplit
 * size. */
size_t gdn_chunk_bwd_workspace_size(int B, int T, int H, int dk, int dv, gdn_dtype dtype);

/* Segments per head of gdn_chunk_bwd's state-gradient sweep on a device with
 * num_cus compute units (the same rule as the forward's sequence split, talk
 * summary paragraph 4, applied to the reverse recurrence, whose chunk map is the
 * transposed forward map): with few heads, 2 B H < num_cus, the sweep is cut
 * into P = a + 1 segments, a = min(16, floor(num_cus / (B H)), floor(N / 8) - 1),
 * when a >= 2 (then S = ceil(N / P) chunks each and P = ceil(N / S)); else 1
 * (unsplit).  A split sweep also stores the states through the split forward.
 * Returns 0 for invalid arguments, 1 when num_cus <= 0. */
int gdn_chunk_bwd_plan_segments(int B, int T, int H, int num_cus);

/* Fused chunked backward (page 1 lede and talk summary paragraph 6: the
 * backward of GDN chunked prefill; the gradient of the K K^T term is formed as
 * (dA + dA^T) K in one product).  Gradients of L given dL/do = dout and
 * dL/dht = dht (NULL = 0):
 *   grad_q, grad_k, grad_v  [.., dk|dv] in the I/O dtype (required)
 *   grad_g, grad_beta       [B,T,H] float32 (required); grad_g is dL/d(log alpha)
 *   grad_h0                 [B,H,dk,dv] float32 or NULL
 * The forward inputs (q, k, v, g, beta, h0) must be the ones of the forward.
 * Only bf16 I/O is supported (GDN_ERR_UNSUPPORTED for float32).  workspace:
 * at least gdn_chunk_bwd_workspace_size() bytes, 256-byte aligned (required).
 * Runs three launches: the forward kernel storing the state entering every
 * chunk (on `stream`) and, side by side with it, the state gradient from the
 * last chunk to the first (on a library-owned side stream of the current
 * device, created on first use with default priority, joined back through an
 * event); then the local gradients of all chunks in parallel on `stream`.
 * With few heads (gdn_chunk_bwd_plan_segments > 1) and a workspace of the
 * size gdn_chunk_bwd_workspace_size reports, everything runs on `stream`: the
 * states through the split forward, then the sweep's last segment from dht
 * beside the other segments' maps (dH_in = M dH_out + b), a chain composing
 * the gradients entering the segments, the other segments from those, and the
 * local gradients; with the unsplit size the call runs unsplit.
 * The call is ordered after earlier work on `stream` and later work on
 * `stream` is ordered after it, as with a single stream. */
gdn_status gdn_chunk_bwd(const void* q, const void* k, const void* v, const float* g,
                         const float* beta, const float* h0, const void* dout, const float* dht,
                         void* grad_q, void* grad_k, void* grad_v, float* grad_g,
                         float* grad_beta, float* grad_h0, int B, int T, int H, int dk, int dv,
                         gdn_dtype dtype, float scale, void* workspace, size_t workspace_bytes,
                         void* stream);

/* Workspace bytes for gdn_gate_scan ((size_t)-1 for invalid arguments). */
size_t gdn_gate_scan_workspace_size(int B, int T, int H);

/* Gate scan (talk summary, paragraph 5: one light kernel scans the gate
 * distribution to find the heads with an effective sliding window).  With
 * chunks of 64 tokens (the last may be short), s_c = sum of g over chunk c and
 * W_c = s_{c-w+1} + ... + s_c for c >= w-1:
 *   flags[b*H+h]               = 1 if N >= w and max_c W_c <= log_eps, else 0
 *   max_window_logdecay[b*H+h] = max_c W_c (-inf when N < w); may be NULL.
 * g is a device pointer [B,T,H] float32; flags / max are device pointers. */
gdn_status gdn_gate_scan(const float* g, int B, int T, int H, int window_chunks, float log_eps,
                         int32_t* flags, float* max_window_logdecay, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Measurement aid, not part of the operator: the memory pattern of the fused
 * forward with no arithmetic (the talk summary, paragraph 7, argues the fused
 * forward is memory-bound; this measures what its layout can stream).  One
 * workgroup per (head, segment) of T / (64 * segments) chunks copies each
 * chunk's K, Q, V tiles (rows of 256 bytes, H * 256 bytes apart) into LDS and
 * writes the previous chunk's V tile to o at that chunk's rows, so every call
 * reads k, q, v once and writes o except each segment's last chunk.  Its time
 * bounds the forward's from below for the same bytes.
 *   k, q, v, o   DEVICE pointers, [T, H, 128] bfloat16, 16-byte aligned
 *   T            a positive multiple of 64 * segments;  H >= 1;  segments >= 1
 * GDN_ERR_INVALID_ARG for other shapes or null pointers; no workspace. */
gdn_status gdn_stream_probe(const void* k, const void* q, const void* v, void* o, int T, int H, int segments,
                            void* stream);

/* Kinds of kernel launch reported by gdn_profile_events. */
typedef enum {
    GDN_LAUNCH_GATE_SUMS = 0,   /* gate scan: per-chunk sums of g                     */
    GDN_LAUNCH_GATE_FLAGS = 1,  /* gate scan: window maxima and flags                 */
    GDN_LAUNCH_FWD_SINGLE = 2,  /* fused forward, unsplit                             */
    GDN_LAUNCH_FWD_WINDOWS = 3, /* split forward: window maxima per group of chunks   */
    GDN_LAUNCH_FWD_QUEUE = 4,   /* split forward: planner, then persistent workgroups over the jobs */
    GDN_LAUNCH_BWD_STATES = 5,  /* backward: state entering every chunk (forward kernel) */
    GDN_LAUNCH_BWD_DH = 6,      /* backward: state gradient, end to start             */
    GDN_LAUNCH_BWD_LOCAL = 7,   /* backward: local gradients of every chunk           */
    GDN_LAUNCH_FWD_SUMS = 8,    /* split forward: chunk sums of g, planner reset      */
    GDN_LAUNCH_KDA_FWD = 9,     /* KDA forward (with outputs)                         */
    GDN_LAUNCH_STREAM_PROBE = 10, /* measurement aid: the forward's memory pattern    */
    GDN_LAUNCH_KDA_PASS1 = 11,  /* KDA split: segment 0, and the other segments' transitions */
    GDN_LAUNCH_KDA_CHAIN = 12,  /* KDA split: states entering the segments            */
    GDN_LAUNCH_BWD_CHAIN = 13   /* backward, few heads: gradients entering the sweep's segments */
} gdn_launch_kind;

/* Measurement hook (the talk summary, paragraph 7, argues the fused operator
 * stays memory-bound; timing each launch is how that is checked).  While set,
 * every kernel launch the library makes from this thread is bracketed by
 * hipEventRecord(events[2i]) and hipEventRecord(events[2i+1]) on the launch
 * stream, and labels[i] receives its gdn_launch_kind, for i = 0..capacity-1;
 * later launches are not recorded.  events holds 2*capacity hipEvent_t created
 * by the caller.  Passing events == NULL clears the hook.  Returns the number of
 * launches recorded since the hook was last set.  Host-only bookkeeping: no
 * device memory is touched. */
int gdn_profile_events(void** events, int* labels, int capacity);

/* Restrict the hook to the launch kinds whose bit (1u << gdn_launch_kind) is set
 * in mask (all kinds by default); launches of other kinds are neither bracketed
 * nor counted.  Each event record costs the stream a few microseconds, so a
 * caller timing one kernel keeps the others unbracketed.  Thread-local; returns
 * the previous mask. */
uint32_t gdn_profile_kinds(uint32_t mask);

/* Thread-local text describing the last non-OK status on this thread ("" if none). */
const char* gdn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
