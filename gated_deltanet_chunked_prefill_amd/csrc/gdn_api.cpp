// C ABI of the gfx950 Gated DeltaNet chunked-prefill library: argument
// validation, the launch planner, the workspace carve-up and the launches.
// Declarations and the contract of every entry point are in include/gdn.h.
#include "gdn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "gdn_internal.h"

namespace {

thread_local char g_err[512];

// Launch-event profiling hook (gdn_profile_events).
struct Profile {
    hipEvent_t* events = nullptr;
    int* labels = nullptr;
    int capacity = 0;
    int used = 0;
};
thread_local Profile g_prof;
thread_local uint32_t g_prof_kinds = 0xffffffffu;   // gdn_profile_kinds

// Run one launcher, bracketed by profiling events when the hook is set.
template <typename F>
hipError_t recorded(int label, hipStream_t s, F&& launch) {
    Profile& p = g_prof;
    const bool rec = p.events && p.used < p.capacity && ((g_prof_kinds >> label) & 1u);
    if (rec) {
        hipError_t e = hipEventRecord(p.events[2 * p.used], s);
        if (e != hipSuccess) return e;
    }
    hipError_t e = launch();
    if (e != hipSuccess) return e;
    if (rec) {
        e = hipEventRecord(p.events[2 * p.used + 1], s);
        if (e != hipSuccess) return e;
        p.labels[p.used] = label;
        ++p.used;
    }
    return hipSuccess;
}

gdn_status fail(gdn_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

gdn_status hip_fail(hipError_t e, const char* what) {
    return fail(GDN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// A side stream per device (default priority, non-blocking), created on first
// use and kept until the process ends: the backward forks its two independent
// sweeps onto it and joins them back through events.
constexpr int kMaxDevices = 64;
hipStream_t g_side[kMaxDevices];
std::mutex g_side_mu;

hipError_t side_stream(hipStream_t* out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_side_mu);
    if (!g_side[dev]) {
        e = hipStreamCreateWithFlags(&g_side[dev], hipStreamNonBlocking);
        if (e != hipSuccess) {
            g_side[dev] = nullptr;
            return e;
        }
    }
    *out = g_side[dev];
    return hipSuccess;
}

// Make `waiter` wait for the work enqueued so far on `producer` (a fresh event
// per hand-over, released once enqueued).
hipError_t stream_wait(hipStream_t waiter, hipStream_t producer) {
    hipEvent_t ev;
    hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
    if (e != hipSuccess) return e;
    e = hipEventRecord(ev, producer);
    if (e == hipSuccess) e = hipStreamWaitEvent(waiter, ev, 0);
    const hipError_t d = hipEventDestroy(ev);
    return e != hipSuccess ? e : d;
}

constexpr int kChunk = 64;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

gdn_options resolve(const gdn_options* opt) {
    gdn_options o;
    gdn_default_options(&o);
    if (opt) o = *opt;
    return o;
}

gdn_status check_options(const gdn_options& o, int N) {
    if (o.split_mode < 0 || o.split_mode > 2)
        return fail(GDN_ERR_INVALID_ARG, "split_mode must be 0, 1 or 2 (got %d)", o.split_mode);
    const int pmax = N < gdn::kMaxSegments ? N : gdn::kMaxSegments;
    if (o.split_mode == 2 && (o.n_segments < 1 || o.n_segments > pmax))
        return fail(GDN_ERR_INVALID_ARG, "n_segments must be in [1, %d] (got %d)", pmax, o.n_segments);
    if (o.window_chunks < 1) return fail(GDN_ERR_INVALID_ARG, "window_chunks must be >= 1");
    if (!(o.log_eps < 0.f)) return fail(GDN_ERR_INVALID_ARG, "log_eps must be negative");
    if (o.window_levels < 1 || o.window_levels > gdn::kMaxWindowLevels)
        return fail(GDN_ERR_INVALID_ARG, "window_levels must be in [1, %d] (got %d)", gdn::kMaxWindowLevels,
                    o.window_levels);
    return GDN_OK;
}

constexpr long long kChunkRows = 64;   // tokens per chunk

gdn_status check_shapes(int B, int T, int H, int dk, int dv, gdn_dtype dt) {
    if (B <= 0 || T <= 0 || H <= 0)
        return fail(GDN_ERR_INVALID_ARG, "B, T, H must be positive (got %d, %d, %d)", B, T, H);
    if (dk != 128 || dv != 128)
        return fail(GDN_ERR_UNSUPPORTED, "only dk = dv = 128 is supported (got %d, %d)", dk, dv);
    if (dt != GDN_F32 && dt != GDN_BF16) return fail(GDN_ERR_UNSUPPORTED, "unknown dtype %d", (int)dt);
    if ((long long)B * T * H * 128 > (1LL << 40))
        return fail(GDN_ERR_INVALID_ARG, "tensor too large");
    // The tile loaders address the 64 rows of one chunk of one head (stride
    // H * 128 elements) with 32-bit per-lane byte offsets: reject head counts
    // whose 64-row span does not fit.
    const long long elem = dt == GDN_F32 ? 4 : 2;
    if ((long long)kChunkRows * H * 128 * elem > (long long)INT32_MAX)
        return fail(GDN_ERR_INVALID_ARG, "H = %d too large for %s I/O (at most %lld heads)", H,
                    dt == GDN_F32 ? "float32" : "bfloat16", (long long)INT32_MAX / (kChunkRows * 128 * elem));
    return GDN_OK;
}

int num_chunks(int T) { return (T + kChunk - 1) / kChunk; }

// Segment slots per head: 1 = no split.  In the automatic mode this is the
// most segments the device-side planner may give a head (talk summary,
// paragraph 8: a square-root rule on the chunk count bounds the split); the
// planner picks the counts per call from the number of exact and window heads,
// with its makespan model deciding between no split (one candidate) and the
// split ones whenever there are fewer heads than compute units (paragraph 8
// calls a fixed activation boundary crude).
int plan(int B, int T, int H, int num_cus, const gdn_options& o) {
    const int N = num_chunks(T);
    if (o.split_mode == 1) return 1;
    if (o.split_mode == 2) return o.n_segments < N ? o.n_segments : N;
    const long long heads = (long long)B * H;
    if (heads >= num_cus || N < 2 * o.window_chunks) return 1;
    long long p = (long long)std::floor(std::sqrt((double)N));
    if (p > 32) p = 32;
    if (p > N / 2) p = N / 2;
    return p < 2 ? 1 : (int)p;
}

struct FwdLayout {
    size_t csum, wmax, flags, maxwin, head_map, hs, counters, bz, mt, eg, plan, jobs, total;
};

FwdLayout fwd_layout(int B, int T, int H, int P) {
    FwdLayout L{};
    if (P <= 1) return L;
    const size_t N = num_chunks(T), bh = (size_t)B * H, SS = 128 * 128;
    size_t off = 0;
    L.csum = off;       off += align_up((size_t)B * N * H * sizeof(float));
    L.wmax = off;       off += align_up((size_t)gdn::kMaxWindowLevels * bh * sizeof(int32_t));
    L.flags = off;      off += align_up(bh * sizeof(int32_t));
    L.maxwin = off;     off += align_up(bh * sizeof(float));
    L.head_map = off;   off += align_up(2 * bh * sizeof(int32_t));
    L.hs = off;         off += align_up(bh * P * SS * sizeof(float));
    L.counters = off;   off += align_up(2 * bh * P * sizeof(int32_t));   // hs_cnt, then tr_cnt
    L.bz = off;         off += align_up(bh * P * SS * sizeof(float));
    L.mt = off;         off += align_up(bh * P * 2 * SS * sizeof(uint16_t));
    L.eg = off;         off += align_up(bh * P * sizeof(float));
    L.plan = off;       off += align_up(sizeof(gdn::FwdPlan));
    L.jobs = off;       off += align_up(bh * (2 * P + 3) * sizeof(gdn::TaskRec));
    L.total = off;
    return L;
}

struct BwdLayout {
    size_t hstore, dhstore, total;
};

BwdLayout bwd_layout(int B, int T, int H) {
    BwdLayout L{};
    const size_t N = num_chunks(T), bh = (size_t)B * H, SS = 128 * 128;
    size_t off = 0;
    L.hstore = off;  off += align_up(bh * (N + 1) * SS * sizeof(uint16_t));   // bf16
    L.dhstore = off; off += align_up(bh * N * SS * sizeof(uint16_t));
    L.total = off;
    return L;
}

// Backward for few heads (talk summary, paragraph 4, applied to both serial
// passes): when 2 B H < CUs, the state store runs through the split forward on
// every CU (P_f segment slots per head, its workspace after the unsplit layout)
// and the state-gradient sweep is split into P_s segments (their maps in P_s
// slots per head after that): a = min(16, CUs / (B H), N / 8 - 1) workgroups per
// head, P_s = a + 1 when a >= 2 (as for KDA: segment P_s - 1 runs beside the maps
// of the others).  P_s = 1 means the unsplit backward.
struct BwdSplit {
    int pf, ps, ss;          // forward segment slots, sweep segments, chunks per sweep segment
    size_t fwd, slots, total;   // offsets of the forward's workspace and the sweep slots; total bytes
};
BwdSplit bwd_split(int B, int T, int H, int cus) {
    BwdSplit sp{};
    sp.ps = 1;
    const int N = num_chunks(T);
    const long long bh = (long long)B * H;
    if (cus > 0 && 2 * bh < cus) {
        long long a = cus / bh;
        if (a > 16) a = 16;
        if (a > N / 8 - 1) a = N / 8 - 1;
        if (a >= 2) {
            const int p = (int)a + 1;
            sp.ss = (N + p - 1) / p;
            sp.ps = (N + sp.ss - 1) / sp.ss;
        }
    }
    if (sp.ps == 1) return sp;
    gdn_options o;
    gdn_default_options(&o);
    sp.pf = plan(B, T, H, cus, o);
    size_t off = bwd_layout(B, T, H).total;
    sp.fwd = off;
    if (sp.pf > 1) off += align_up(fwd_layout(B, T, H, sp.pf).total);
    sp.slots = off;
    off += align_up((size_t)bh * sp.ps * gdn::kStateSlot * sizeof(float));
    sp.total = off;
    return sp;
}

// Packed-sequence backward workspace: the chunk prefix and the sequence bounds
// (cu_seqlens clamped to [0, T] and made non-decreasing), then states and state
// gradients in per-head slots (cmax = ceil(T/64) + S bounds the chunks of all
// sequences together, which holds because the bounded sequences are disjoint).
struct BwdVarlenLayout {
    size_t cstart, hstore, dhstore, total;
    int cmax;
};

BwdVarlenLayout bwd_varlen_layout(int S, int T, int H) {
    BwdVarlenLayout L{};
    L.cmax = num_chunks(T) + S;
    const size_t SS = 128 * 128;
    size_t off = 0;
    L.cstart = off;  off += align_up(2 * ((size_t)S + 1) * sizeof(int32_t));   // chunk prefix, then bounds
    L.hstore = off;  off += align_up((size_t)H * (L.cmax + S) * SS * sizeof(uint16_t));   // bf16
    L.dhstore = off; off += align_up((size_t)H * L.cmax * SS * sizeof(uint16_t));
    L.total = off;
    return L;
}

// KDA sequence split: P segments of S chunks per head (the last one shorter).
// n_segments = 1: unsplit; n_segments >= 2: that many (at most the chunk count);
// 0: one segment more than the workgroups per head that fill the device, a =
// min(16, cus / (B H), N / 8 - 1), when a >= 2, else unsplit (both launches with
// outputs then hold a workgroups per head: segment 0 runs beside the
// transitions of segments 1 .. P-2, segments 1 .. P-1 after the chain).
// S = ceil(N / P), then P = ceil(N / S) so that no segment is empty.
constexpr int kKdaMaxSegments = 1024;
void kda_plan(int B, int T, int H, int cus, int n_segments, int* P, int* S) {
    const int N = num_chunks(T);
    int p = 1;
    if (n_segments >= 2) {
        p = n_segments < N ? n_segments : N;
    } else if (n_segments == 0) {
        const long bh = (long)B * H;
        long a = cus / bh;
        if (a > 16) a = 16;
        if (a > N / 8 - 1) a = N / 8 - 1;
        p = a >= 2 ? (int)a + 1 : 1;
    }
    if (p < 1) p = 1;
    const int s = (N + p - 1) / p;
    *S = s;
    *P = (N + s - 1) / s;
}

// Workspace of the KDA split: (P - 1) slots of gdn::kKdaSlot floats per head.
size_t kda_workspace_bytes(int B, int H, int P) {
    return P > 1 ? (size_t)B * H * (P - 1) * gdn::kKdaSlot * sizeof(float) : 0;
}

gdn_status device_cus(int* cus) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    return GDN_OK;
}

// Packed sequences: a sequence longer than the per-CU share of all chunks (at
// least two windows) is cut into segments of about that many chunks, at most 16,
// each later one warming up over a window (talk summary, paragraphs 4 and 5).
// The cut is taken on the device from each sequence's length; here only its
// target length and the segment bound follow from the shapes.
void varlen_segments(int n_seqs, int T, int H, int cus, gdn::FwdParams& p) {
    const gdn_options d = resolve(nullptr);
    const long long nch = num_chunks(T);
    long long target = (nch * H + cus - 1) / (cus > 0 ? cus : 1);
    if (target < 2LL * d.window_chunks) target = 2LL * d.window_chunks;
    long long P = (nch + target - 1) / target;
    if (P > 16) P = 16;
    if (P <= 1 || (long long)n_seqs * H * P > (1LL << 30)) {
        p.vseg = 0;
        p.P = 1;
        return;
    }
    p.vseg = (int)target;
    p.P = (int)P;
    p.w = d.window_chunks;
    p.log_eps = d.log_eps;
}

}  // namespace

extern "C" {

void gdn_default_options(gdn_options* opt) {
    if (!opt) return;
    opt->split_mode = 0;
    opt->n_segments = 1;
    opt->use_window = 1;
    opt->window_chunks = 8;
    opt->log_eps = std::log(std::ldexp(1.0f, -24));
    opt->window_levels = 4;
}

const char* gdn_last_error(void) { return g_err; }

uint32_t gdn_profile_kinds(uint32_t mask) {
    const uint32_t prev = g_prof_kinds;
    g_prof_kinds = mask;
    return prev;
}

int gdn_profile_events(void** events, int* labels, int capacity) {
    const int used = g_prof.used;
    if (!events || !labels || capacity <= 0) {
        g_prof = Profile{};
    } else {
        g_prof.events = (hipEvent_t*)events;
        g_prof.labels = labels;
        g_prof.capacity = capacity;
        g_prof.used = 0;
    }
    return used;
}

int gdn_plan_segments(int B, int T, int H, int num_cus, const gdn_options* opt) {
    if (B <= 0 || T <= 0 || H <= 0 || num_cus <= 0) return 0;
    gdn_options o = resolve(opt);
    if (check_options(o, num_chunks(T)) != GDN_OK) return 0;
    return plan(B, T, H, num_cus, o);
}

size_t gdn_chunk_fwd_workspace_size(int B, int T, int H, int dk, int dv, gdn_dtype dtype,
                                    const gdn_options* opt) {
    if (check_shapes(B, T, H, dk, dv, dtype) != GDN_OK) return (size_t)-1;
    gdn_options o = resolve(opt);
    if (check_options(o, num_chunks(T)) != GDN_OK) return (size_t)-1;
    int cus = 0;
    if (device_cus(&cus) != GDN_OK) return (size_t)-1;
    return fwd_layout(B, T, H, plan(B, T, H, cus, o)).total;
}

}  // extern "C"

namespace {

// Checks of the forward's tensors and sizes, shared by both forward entry points.
gdn_status check_fwd_args(const void* q, const void* k, const void* v, const float* g, const float* beta,
                          const float* h0, const void* o, const float* ht, int B, int T, int H, int dk, int dv,
                          gdn_dtype dtype, float scale) {
    if (!q || !k || !v || !g || !beta || !o)
        return fail(GDN_ERR_INVALID_ARG, "q, k, v, g, beta and o are required");
    gdn_status st = check_shapes(B, T, H, dk, dv, dtype);
    if (st != GDN_OK) return st;
    const void* vec_ptrs[] = {q, k, v, o};
    for (const void* p : vec_ptrs)
        if (!aligned16(p)) return fail(GDN_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
    const void* f32_ptrs[] = {g, beta, h0, ht};
    for (const void* p : f32_ptrs)
        if (p && !aligned4(p)) return fail(GDN_ERR_INVALID_ARG, "g, beta, h0 and ht must be 4-byte aligned");
    if (!std::isfinite(scale)) return fail(GDN_ERR_INVALID_ARG, "scale must be finite");
    return GDN_OK;
}

// The forward's launches with P segment slots per head, in a workspace of at
// least fwd_layout(B, T, H, P).total bytes (unused when P = 1).
gdn_status fwd_launch(const void* q, const void* k, const void* v, const float* g, const float* beta,
                      const float* h0, void* o, float* ht, int B, int T, int H, gdn_dtype dtype, float scale,
                      const gdn_options& op, int cus, int P, void* workspace, hipStream_t s,
                      __bf16* hstore = nullptr) {
    const int N = num_chunks(T);
    const FwdLayout L = fwd_layout(B, T, H, P);
    gdn::FwdParams p{};
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta; p.h0 = h0; p.o = o; p.ht = ht;
    p.B = B; p.T = T; p.H = H; p.N = N; p.P = P; p.w = op.window_chunks; p.scale = scale;
    p.wmax = nullptr;
    p.hstore = hstore;   // keep the state entering every chunk (the backward's state store)
    const bool bf16 = dtype == GDN_BF16;
    hipError_t e;
    if (P == 1) {
        if (hstore)
            e = recorded(GDN_LAUNCH_BWD_STATES, s, [&] { return gdn::launch_fwd(p, gdn::PHASE_STATES, bf16, s); });
        else
            e = recorded(GDN_LAUNCH_FWD_SINGLE, s, [&] { return gdn::launch_fwd(p, gdn::PHASE_SINGLE, bf16, s); });
        if (e != hipSuccess) return hip_fail(e, "forward launch");
        return GDN_OK;
    }
    char* ws = (char*)workspace;
    const int nbh = B * H;
    p.hs = (float*)(ws + L.hs);
    p.hs_cnt = (int*)(ws + L.counters);
    p.tr_cnt = p.hs_cnt + (size_t)nbh * P;
    p.bz = (float*)(ws + L.bz);
    p.mt = (__bf16*)(ws + L.mt);
    p.eg = (float*)(ws + L.eg);
    p.plan = (gdn::FwdPlan*)(ws + L.plan);
    p.jobs = (gdn::TaskRec*)(ws + L.jobs);
    p.cus = cus;
    p.forced = op.split_mode == 2 ? 1 : 0;
    p.flags = (int32_t*)(ws + L.flags);
    p.maxwin = (float*)(ws + L.maxwin);
    p.head_map = (int*)(ws + L.head_map);
    p.log_eps = op.log_eps;
    // window heads only when a window fits the sequence (no head qualifies
    // otherwise) and the first launch can stage it
    // (longer windows are tried only while they fit the sequence and the staging)
    p.levels = 0;
    if (op.use_window && op.window_chunks <= N && op.window_chunks <= gdn::max_window_chunks()) {
        p.wmax = (const int*)(ws + L.wmax);
        p.levels = 1;
        while (p.levels < op.window_levels && (p.levels + 1) * op.window_chunks <= N &&
               (p.levels + 1) * op.window_chunks <= gdn::max_window_chunks())
            ++p.levels;
    }
    float* const csum = p.wmax ? (float*)(ws + L.csum) : nullptr;
    int* const wmax = const_cast<int*>(p.wmax);
    e = recorded(GDN_LAUNCH_FWD_SUMS, s, [&] {
        return gdn::launch_fwd_sums(g, B, T, H, csum, p.hs_cnt, 2 * nbh * P, (int*)p.plan, wmax,
                                    wmax ? p.levels * nbh : 0, s);
    });
    if (e != hipSuccess) return hip_fail(e, "forward preparation launch");
    if (p.wmax) {
        e = recorded(GDN_LAUNCH_FWD_WINDOWS, s, [&] {
            return gdn::launch_fwd_windows(csum, B, T, H, op.window_chunks, p.levels, wmax, s);
        });
        if (e != hipSuccess) return hip_fail(e, "forward window launch");
    }
    if (hstore)
        e = recorded(GDN_LAUNCH_BWD_STATES, s,
                     [&] { return gdn::launch_fwd(p, gdn::PHASE_QUEUE_STATES, bf16, s); });
    else
        e = recorded(GDN_LAUNCH_FWD_QUEUE, s, [&] { return gdn::launch_fwd(p, gdn::PHASE_QUEUE, bf16, s); });
    if (e != hipSuccess) return hip_fail(e, "forward launch");
    return GDN_OK;
}

}  // namespace

extern "C" {

gdn_status gdn_chunk_fwd(const void* q, const void* k, const void* v, const float* g,
                         const float* beta, const float* h0, void* o, float* ht, int B, int T,
                         int H, int dk, int dv, gdn_dtype dtype, float scale,
                         const gdn_options* opt, void* workspace, size_t workspace_bytes,
                         void* stream) {
    g_err[0] = 0;
    gdn_status st = check_fwd_args(q, k, v, g, beta, h0, o, ht, B, T, H, dk, dv, dtype, scale);
    if (st != GDN_OK) return st;
    gdn_options op = resolve(opt);
    st = check_options(op, num_chunks(T));
    if (st != GDN_OK) return st;
    int cus = 0;
    st = device_cus(&cus);
    if (st != GDN_OK) return st;
    const int P = plan(B, T, H, cus, op);
    const FwdLayout L = fwd_layout(B, T, H, P);
    if (L.total > 0) {
        if (!workspace) return fail(GDN_ERR_WORKSPACE, "a workspace of %zu bytes is required", L.total);
        if (workspace_bytes < L.total)
            return fail(GDN_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes, L.total);
        if (((uintptr_t)workspace & (kAlign - 1)) != 0)
            return fail(GDN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    }
    return fwd_launch(q, k, v, g, beta, h0, o, ht, B, T, H, dtype, scale, op, cus, P, workspace,
                      (hipStream_t)stream);
}

static_assert(gdn::kFwdScratchBytes == GDN_NOALLOC_SCRATCH_BYTES, "scratch size declared in gdn.h");

gdn_status gdn_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* g,
                                 const float* beta, const float* h0, void* o, float* ht, int B, int T,
                                 int H, int dk, int dv, gdn_dtype dtype, float scale,
                                 const gdn_options* opt, void* stream) {
    g_err[0] = 0;
    gdn_status st = check_fwd_args(q, k, v, g, beta, h0, o, ht, B, T, H, dk, dv, dtype, scale);
    if (st != GDN_OK) return st;
    gdn_options op = resolve(opt);
    st = check_options(op, num_chunks(T));
    if (st != GDN_OK) return st;
    int cus = 0;
    st = device_cus(&cus);
    if (st != GDN_OK) return st;
    int P = plan(B, T, H, cus, op);
    const size_t cap = gdn::kFwdScratchBytes;
    if (fwd_layout(B, T, H, P).total > cap) {
        if (op.split_mode == 2)
            return fail(GDN_ERR_WORKSPACE,
                        "%d segments per head need %zu bytes of scratch; the fixed scratch holds %zu bytes",
                        P, fwd_layout(B, T, H, P).total, cap);
        // automatic split: fewer segment slots, down to none
        while (P > 1 && fwd_layout(B, T, H, P).total > cap) --P;
    }
    void* scratch = nullptr;
    if (P > 1) {
        const hipError_t e = gdn::fwd_scratch(&scratch);
        if (e != hipSuccess) return hip_fail(e, "scratch address lookup");
    }
    return fwd_launch(q, k, v, g, beta, h0, o, ht, B, T, H, dtype, scale, op, cus, P, scratch,
                      (hipStream_t)stream);
}

gdn_status gdn_kda_fwd(const void* q, const void* k, const void* v, const float* g, const float* beta,
                       const float* h0, void* o, float* ht, int B, int T, int H, int dk, int dv, gdn_dtype dtype,
                       float scale, int n_segments, void* workspace, size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    gdn_status st = check_fwd_args(q, k, v, g, beta, h0, o, ht, B, T, H, dk, dv, dtype, scale);
    if (st != GDN_OK) return st;
    if (dtype != GDN_BF16) return fail(GDN_ERR_UNSUPPORTED, "the KDA forward supports bf16 I/O only");
    // the per-channel gates (128 float32 per token-head) are addressed like a
    // float32 tile: 64 rows of H * 512 bytes within 32-bit offsets
    if ((long long)kChunkRows * H * 128 * 4 > (long long)INT32_MAX)
        return fail(GDN_ERR_INVALID_ARG, "H = %d too large for the KDA gates (at most %lld heads)", H,
                    (long long)INT32_MAX / (kChunkRows * 128 * 4));
    if (n_segments < 0 || n_segments > kKdaMaxSegments)
        return fail(GDN_ERR_INVALID_ARG, "n_segments must be in [0, %d] (got %d)", kKdaMaxSegments, n_segments);
    int cus = 0;
    if (n_segments == 0 && (st = device_cus(&cus)) != GDN_OK) return st;
    int P = 1, S = 1;
    kda_plan(B, T, H, cus, n_segments, &P, &S);
    const size_t need = kda_workspace_bytes(B, H, P);
    if (need > 0) {
        if (!workspace) return fail(GDN_ERR_WORKSPACE, "%d segments per head need a workspace of %zu bytes", P, need);
        if (workspace_bytes < need)
            return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
        if (((uintptr_t)workspace & (kAlign - 1)) != 0)
            return fail(GDN_ERR_INVALID_ARG, "the workspace must be %zu-byte aligned", kAlign);
    }
    gdn::KdaParams p{};
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta; p.h0 = h0; p.o = o; p.ht = ht;
    p.B = B; p.T = T; p.H = H; p.N = num_chunks(T); p.scale = scale;
    p.P = P; p.S = S; p.ws = (float*)workspace;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = hipSuccess;
    if (P == 1) {
        e = recorded(GDN_LAUNCH_KDA_FWD, s, [&] { return gdn::launch_kda_fwd(p, gdn::KDA_FULL, s); });
        if (e != hipSuccess) return hip_fail(e, "KDA forward launch");
        return GDN_OK;
    }
    e = recorded(GDN_LAUNCH_KDA_PASS1, s, [&] { return gdn::launch_kda_fwd(p, gdn::KDA_FIRST, s); });
    if (e != hipSuccess) return hip_fail(e, "KDA first launch");
    if (P > 2) {
        e = recorded(GDN_LAUNCH_KDA_CHAIN, s, [&] { return gdn::launch_kda_chain(p, s); });
        if (e != hipSuccess) return hip_fail(e, "KDA chain launch");
    }
    e = recorded(GDN_LAUNCH_KDA_FWD, s, [&] { return gdn::launch_kda_fwd(p, gdn::KDA_REST, s); });
    if (e != hipSuccess) return hip_fail(e, "KDA forward launch");
    return GDN_OK;
}

int gdn_kda_plan_segments(int B, int T, int H, int num_cus, int n_segments) {
    if (B <= 0 || T <= 0 || H <= 0 || n_segments < 0 || n_segments > kKdaMaxSegments) return 0;
    if (n_segments == 0 && num_cus <= 0) return 0;
    int P = 1, S = 1;
    kda_plan(B, T, H, num_cus, n_segments, &P, &S);
    return P;
}

size_t gdn_kda_fwd_workspace_size(int B, int T, int H, int dk, int dv, int n_segments) {
    if (check_shapes(B, T, H, dk, dv, GDN_BF16) != GDN_OK) return (size_t)-1;
    if (n_segments < 0 || n_segments > kKdaMaxSegments) return (size_t)-1;
    int cus = 0;
    if (n_segments == 0 && device_cus(&cus) != GDN_OK) return (size_t)-1;
    int P = 1, S = 1;
    kda_plan(B, T, H, cus, n_segments, &P, &S);
    return kda_workspace_bytes(B, H, P);
}

gdn_status gdn_stream_probe(const void* k, const void* q, const void* v, void* o, int T, int H, int segments,
                            void* stream) {
    g_err[0] = 0;
    if (!k || !q || !v || !o) return fail(GDN_ERR_INVALID_ARG, "k, q, v and o are required");
    if (H < 1 || segments < 1 || T < 1) return fail(GDN_ERR_INVALID_ARG, "T, H and segments must be positive");
    if (T % (64LL * segments) != 0)
        return fail(GDN_ERR_INVALID_ARG, "T (%d) must be a multiple of 64 * segments (%d)", T, segments);
    if ((long long)T * H * 128 * 2 >= (1LL << 40) || (long long)H * segments > (1LL << 30))
        return fail(GDN_ERR_INVALID_ARG, "shape too large");
    const void* ptrs[] = {k, q, v, o};
    for (const void* p : ptrs)
        if (!aligned16(p)) return fail(GDN_ERR_INVALID_ARG, "k, q, v and o must be 16-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    const hipError_t e = recorded(GDN_LAUNCH_STREAM_PROBE, s, [&] {
        return gdn::launch_stream_probe(k, q, v, o, T, H, segments, s);
    });
    if (e != hipSuccess) return hip_fail(e, "stream probe launch");
    return GDN_OK;
}

gdn_status gdn_chunk_fwd_varlen(const void* q, const void* k, const void* v, const float* g,
                                const float* beta, const float* h0, void* o, float* ht,
                                const int32_t* cu_seqlens, int n_seqs, int T, int H, int dk, int dv,
                                gdn_dtype dtype, float scale, void* stream) {
    g_err[0] = 0;
    if (!q || !k || !v || !g || !beta || !o || !cu_seqlens)
        return fail(GDN_ERR_INVALID_ARG, "q, k, v, g, beta, o and cu_seqlens are required");
    if (n_seqs <= 0) return fail(GDN_ERR_INVALID_ARG, "n_seqs must be positive (got %d)", n_seqs);
    gdn_status st = check_shapes(1, T, H, dk, dv, dtype);
    if (st != GDN_OK) return st;
    if ((long long)n_seqs * H > (1LL << 30)) return fail(GDN_ERR_INVALID_ARG, "too many sequences");
    const void* vec_ptrs[] = {q, k, v, o};
    for (const void* p : vec_ptrs)
        if (!aligned16(p)) return fail(GDN_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
    const void* i32_ptrs[] = {g, beta, h0, ht, cu_seqlens};
    for (const void* p : i32_ptrs)
        if (p && !aligned4(p))
            return fail(GDN_ERR_INVALID_ARG, "g, beta, h0, ht and cu_seqlens must be 4-byte aligned");
    if (!std::isfinite(scale)) return fail(GDN_ERR_INVALID_ARG, "scale must be finite");
    hipStream_t s = (hipStream_t)stream;
    gdn::FwdParams p{};
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta; p.h0 = h0; p.o = o; p.ht = ht;
    p.B = n_seqs; p.T = T; p.H = H; p.N = num_chunks(T); p.P = 1; p.w = 1; p.scale = scale;
    p.cu = cu_seqlens;
    int cus = 0;
    st = device_cus(&cus);
    if (st != GDN_OK) return st;
    varlen_segments(n_seqs, T, H, cus, p);
    const hipError_t e = recorded(GDN_LAUNCH_FWD_SINGLE, s, [&] {
        return gdn::launch_fwd(p, gdn::PHASE_VARLEN, dtype == GDN_BF16, s);
    });
    if (e != hipSuccess) return hip_fail(e, "forward launch");
    return GDN_OK;
}

size_t gdn_chunk_bwd_varlen_workspace_size(int n_seqs, int T, int H, int dk, int dv, gdn_dtype dtype) {
    if (n_seqs <= 0 || check_shapes(1, T, H, dk, dv, dtype) != GDN_OK) return (size_t)-1;
    if ((long long)n_seqs * H > (1LL << 30)) return (size_t)-1;
    return bwd_varlen_layout(n_seqs, T, H).total;
}

gdn_status gdn_chunk_bwd_varlen(const void* q, const void* k, const void* v, const float* g,
                                const float* beta, const float* h0, const void* dout, const float* dht,
                                void* grad_q, void* grad_k, void* grad_v, float* grad_g,
                                float* grad_beta, float* grad_h0, const int32_t* cu_seqlens, int n_seqs,
                                int T, int H, int dk, int dv, gdn_dtype dtype, float scale,
                                void* workspace, size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    if (!q || !k || !v || !g || !beta || !dout || !grad_q || !grad_k || !grad_v || !grad_g || !grad_beta ||
        !cu_seqlens)
        return fail(GDN_ERR_INVALID_ARG, "q, k, v, g, beta, dout, the gradients of q, k, v, g, beta and "
                                         "cu_seqlens are required");
    if (n_seqs <= 0) return fail(GDN_ERR_INVALID_ARG, "n_seqs must be positive (got %d)", n_seqs);
    gdn_status st = check_shapes(1, T, H, dk, dv, dtype);
    if (st != GDN_OK) return st;
    if ((long long)n_seqs * H > (1LL << 30)) return fail(GDN_ERR_INVALID_ARG, "too many sequences");
    if (dtype != GDN_BF16) return fail(GDN_ERR_UNSUPPORTED, "the backward supports bf16 I/O only");
    const void* vec_ptrs[] = {q, k, v, dout, grad_q, grad_k, grad_v};
    for (const void* p : vec_ptrs)
        if (!aligned16(p))
            return fail(GDN_ERR_INVALID_ARG, "q, k, v, dout and their gradients must be 16-byte aligned");
    const void* i32_ptrs[] = {g, beta, h0, dht, grad_g, grad_beta, grad_h0, cu_seqlens};
    for (const void* p : i32_ptrs)
        if (p && !aligned4(p))
            return fail(GDN_ERR_INVALID_ARG, "float32 tensors and cu_seqlens must be 4-byte aligned");
    if (!std::isfinite(scale)) return fail(GDN_ERR_INVALID_ARG, "scale must be finite");
    const BwdVarlenLayout L = bwd_varlen_layout(n_seqs, T, H);
    if (!workspace) return fail(GDN_ERR_WORKSPACE, "a workspace of %zu bytes is required", L.total);
    if (workspace_bytes < L.total)
        return fail(GDN_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes, L.total);
    if (((uintptr_t)workspace & (kAlign - 1)) != 0)
        return fail(GDN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");

    hipStream_t s = (hipStream_t)stream;
    hipStream_t s2 = nullptr;
    hipError_t e = side_stream(&s2);
    if (e != hipSuccess) return hip_fail(e, "backward side stream");
    char* ws = (char*)workspace;
    int* cstart = (int*)(ws + L.cstart);
    __bf16* hstore = (__bf16*)(ws + L.hstore);
    __bf16* dhstore = (__bf16*)(ws + L.dhstore);
    gdn::FwdParams f{};
    f.q = q; f.k = k; f.v = v; f.g = g; f.beta = beta; f.h0 = h0; f.o = nullptr; f.ht = nullptr;
    f.B = n_seqs; f.T = T; f.H = H; f.N = num_chunks(T); f.P = 1; f.w = 1; f.scale = scale;
    f.hstore = hstore;
    f.cu = cu_seqlens; f.cmax = L.cmax; f.cstart = cstart;
    gdn::BwdParams p{};
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta; p.h0 = h0; p.dout = dout; p.dht = dht;
    p.dq = grad_q; p.dk = grad_k; p.dv = grad_v; p.dg = grad_g; p.dbeta = grad_beta; p.dh0 = grad_h0;
    p.B = n_seqs; p.T = T; p.H = H; p.N = num_chunks(T); p.scale = scale;
    p.hstore = hstore;
    p.dhstore = dhstore;
    p.cu = cu_seqlens; p.cmax = L.cmax; p.cstart = cstart;
    // the chunk prefix, then (as in gdn_chunk_bwd) the state-gradient sweep on the
    // side stream beside the state store, then the local gradients
    e = gdn::launch_seq_chunk_prefix(cu_seqlens, n_seqs, T, cstart, s);
    if (e != hipSuccess) return hip_fail(e, "backward chunk prefix launch");
    e = stream_wait(s2, s);
    if (e != hipSuccess) return hip_fail(e, "backward fork");
    e = recorded(GDN_LAUNCH_BWD_DH, s2, [&] { return gdn::launch_bwd_dh(p, true, s2); });
    if (e != hipSuccess) return hip_fail(e, "backward state-gradient launch");
    e = recorded(GDN_LAUNCH_BWD_STATES, s, [&] { return gdn::launch_fwd(f, gdn::PHASE_STATES_VARLEN, true, s); });
    if (e != hipSuccess) return hip_fail(e, "backward state launch");
    e = stream_wait(s, s2);
    if (e != hipSuccess) return hip_fail(e, "backward join");
    e = recorded(GDN_LAUNCH_BWD_LOCAL, s, [&] { return gdn::launch_bwd_local(p, true, s); });
    if (e != hipSuccess) return hip_fail(e, "backward local-gradient launch");
    return GDN_OK;
}

gdn_status gdn_chunk_fwd_plan_info(int B, int T, int H, const gdn_options* opt, const void* workspace,
                                   int32_t* info, void* stream) {
    g_err[0] = 0;
    if (!info) return fail(GDN_ERR_INVALID_ARG, "info is required");
    if (B <= 0 || T <= 0 || H <= 0)
        return fail(GDN_ERR_INVALID_ARG, "B, T, H must be positive (got %d, %d, %d)", B, T, H);
    gdn_options op = resolve(opt);
    gdn_status st = check_options(op, num_chunks(T));
    if (st != GDN_OK) return st;
    int cus = 0;
    st = device_cus(&cus);
    if (st != GDN_OK) return st;
    const int P = plan(B, T, H, cus, op);
    if (P == 1) {
        const int32_t whole[8] = {1, 1, B * H, 0, B * H, 0, 0, 0};
        std::memcpy(info, whole, sizeof(whole));
        return GDN_OK;
    }
    if (!workspace) return fail(GDN_ERR_WORKSPACE, "the split forward's workspace is required");
    const FwdLayout L = fwd_layout(B, T, H, P);
    hipStream_t s = (hipStream_t)stream;
    static_assert(sizeof(gdn::FwdPlan) >= 8 * sizeof(int32_t) && sizeof(gdn::FwdPlan) <= 16 * sizeof(int32_t),
                  "plan words: eight reported, at most sixteen reset");
    hipError_t e = hipMemcpyAsync(info, (const char*)workspace + L.plan, 8 * sizeof(int32_t),
                                  hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return hip_fail(e, "plan read-back");
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "plan read-back");
    return GDN_OK;
}

size_t gdn_gate_scan_workspace_size(int B, int T, int H) {
    if (B <= 0 || T <= 0 || H <= 0) return (size_t)-1;
    return align_up((size_t)B * num_chunks(T) * H * sizeof(float));
}

gdn_status gdn_gate_scan(const float* g, int B, int T, int H, int window_chunks, float log_eps,
                         int32_t* flags, float* max_window_logdecay, void* workspace,
                         size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    if (!g || !flags || !workspace) return fail(GDN_ERR_INVALID_ARG, "g, flags and workspace are required");
    if (B <= 0 || T <= 0 || H <= 0)
        return fail(GDN_ERR_INVALID_ARG, "B, T, H must be positive (got %d, %d, %d)", B, T, H);
    if (window_chunks < 1) return fail(GDN_ERR_INVALID_ARG, "window_chunks must be >= 1");
    if ((long long)B * H > (long long)INT32_MAX || (long long)B * T * H > (1LL << 40))
        return fail(GDN_ERR_INVALID_ARG, "B * H or B * T * H too large");
    if (!aligned4(g) || !aligned4(flags) || (max_window_logdecay && !aligned4(max_window_logdecay)))
        return fail(GDN_ERR_INVALID_ARG, "pointers must be 4-byte aligned");
    if (((uintptr_t)workspace & 3u) != 0) return fail(GDN_ERR_INVALID_ARG, "workspace must be 4-byte aligned");
    const size_t need = gdn_gate_scan_workspace_size(B, T, H);
    if (workspace_bytes < need)
        return fail(GDN_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes, need);
    hipStream_t s = (hipStream_t)stream;
    float* sums = (float*)workspace;
    hipError_t e = recorded(GDN_LAUNCH_GATE_SUMS, s, [&] { return gdn::launch_chunk_sums(g, B, T, H, sums, s); });
    if (e != hipSuccess) return hip_fail(e, "gate scan launch");
    e = recorded(GDN_LAUNCH_GATE_FLAGS, s, [&] {
        return gdn::launch_window_flags(sums, B, T, H, window_chunks, log_eps, flags,
                                        max_window_logdecay, s);
    });
    if (e != hipSuccess) return hip_fail(e, "gate scan launch");
    return GDN_OK;
}

int gdn_chunk_bwd_plan_segments(int B, int T, int H, int num_cus) {
    if (B <= 0 || T <= 0 || H <= 0 || (long long)B * H > (1LL << 30)) return 0;
    return bwd_split(B, T, H, num_cus).ps;
}

size_t gdn_chunk_bwd_workspace_size(int B, int T, int H, int dk, int dv, gdn_dtype dtype) {
    if (check_shapes(B, T, H, dk, dv, dtype) != GDN_OK) return (size_t)-1;
    int cus = 0;
    if (device_cus(&cus) != GDN_OK) {   // no device: the unsplit backward's size
        g_err[0] = 0;
        return bwd_layout(B, T, H).total;
    }
    const BwdSplit sp = bwd_split(B, T, H, cus);
    return sp.ps > 1 ? sp.total : bwd_layout(B, T, H).total;
}

gdn_status gdn_chunk_bwd(const void* q, const void* k, const void* v, const float* g,
                         const float* beta, const float* h0, const void* dout, const float* dht,
                         void* grad_q, void* grad_k, void* grad_v, float* grad_g,
                         float* grad_beta, float* grad_h0, int B, int T, int H, int dk, int dv,
                         gdn_dtype dtype, float scale, void* workspace, size_t workspace_bytes,
                         void* stream) {
    g_err[0] = 0;
    if (!q || !k || !v || !g || !beta || !dout || !grad_q || !grad_k || !grad_v || !grad_g || !grad_beta)
        return fail(GDN_ERR_INVALID_ARG,
                    "q, k, v, g, beta, dout, grad_q, grad_k, grad_v, grad_g and grad_beta are required");
    gdn_status st = check_shapes(B, T, H, dk, dv, dtype);
    if (st != GDN_OK) return st;
    if (dtype != GDN_BF16) return fail(GDN_ERR_UNSUPPORTED, "the backward supports bf16 I/O only");
    const void* vec_ptrs[] = {q, k, v, dout, grad_q, grad_k, grad_v};
    for (const void* p : vec_ptrs)
        if (!aligned16(p))
            return fail(GDN_ERR_INVALID_ARG, "q, k, v, dout and their gradients must be 16-byte aligned");
    const void* f32_ptrs[] = {g, beta, h0, dht, grad_g, grad_beta, grad_h0};
    for (const void* p : f32_ptrs)
        if (p && !aligned4(p))
            return fail(GDN_ERR_INVALID_ARG, "float32 tensors must be 4-byte aligned");
    if (!std::isfinite(scale)) return fail(GDN_ERR_INVALID_ARG, "scale must be finite");
    const BwdLayout L = bwd_layout(B, T, H);
    if (!workspace) return fail(GDN_ERR_WORKSPACE, "a workspace of %zu bytes is required", L.total);
    if (workspace_bytes < L.total)
        return fail(GDN_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes, L.total);
    if (((uintptr_t)workspace & (kAlign - 1)) != 0)
        return fail(GDN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");

    hipStream_t s = (hipStream_t)stream;
    const int N = num_chunks(T);
    char* ws = (char*)workspace;
    __bf16* hstore = (__bf16*)(ws + L.hstore);
    __bf16* dhstore = (__bf16*)(ws + L.dhstore);
    int cus = 0;
    if ((st = device_cus(&cus)) != GDN_OK) return st;
    const BwdSplit sp = bwd_split(B, T, H, cus);
    if (sp.ps > 1 && workspace_bytes >= sp.total) {
        // few heads: the state store through the split forward on every CU, then
        // the sweep in segments (first launch: the last segment and the others'
        // maps; the chain; the remaining segments), then the local gradients
        gdn_options o;
        gdn_default_options(&o);
        st = fwd_launch(q, k, v, g, beta, h0, nullptr, nullptr, B, T, H, dtype, scale, o, cus, sp.pf,
                        ws + sp.fwd, s, hstore);
        if (st != GDN_OK) return st;
        gdn::BwdParams p{};
        p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta; p.h0 = h0; p.dout = dout; p.dht = dht;
        p.dq = grad_q; p.dk = grad_k; p.dv = grad_v; p.dg = grad_g; p.dbeta = grad_beta; p.dh0 = grad_h0;
        p.B = B; p.T = T; p.H = H; p.N = N; p.scale = scale;
        p.hstore = hstore;
        p.dhstore = dhstore;
        p.P = sp.ps; p.S = sp.ss; p.ws = (float*)(ws + sp.slots);
        hipError_t e = recorded(GDN_LAUNCH_BWD_DH, s, [&] { return gdn::launch_bwd_dh(p, true, s, gdn::DH_FIRST); });
        if (e != hipSuccess) return hip_fail(e, "backward state-gradient launch");
        if (sp.ps > 2) {
            // from the gradient at the start of segment P-1 down to segment 1
            gdn::ChainParams c{p.ws, sp.ps, sp.ps - 1, -1, sp.ps - 2};
            e = recorded(GDN_LAUNCH_BWD_CHAIN, s, [&] { return gdn::launch_state_chain(c, B * H, s); });
            if (e != hipSuccess) return hip_fail(e, "backward chain launch");
        }
        e = recorded(GDN_LAUNCH_BWD_DH, s, [&] { return gdn::launch_bwd_dh(p, true, s, gdn::DH_REST); });
        if (e != hipSuccess) return hip_fail(e, "backward state-gradient launch");
        e = recorded(GDN_LAUNCH_BWD_LOCAL, s, [&] { return gdn::launch_bwd_local(p, true, s); });
        if (e != hipSuccess) return hip_fail(e, "backward local-gradient launch");
        return GDN_OK;
    }
    hipStream_t s2 = nullptr;
    hipError_t e = side_stream(&s2);
    if (e != hipSuccess) return hip_fail(e, "backward side stream");
    gdn::FwdParams f{};
    f.q = q; f.k = k; f.v = v; f.g = g; f.beta = beta; f.h0 = h0; f.o = nullptr; f.ht = nullptr;
    f.B = B; f.T = T; f.H = H; f.N = N; f.P = 1; f.w = 1; f.scale = scale;
    f.hstore = hstore;
    gdn::BwdParams p{};
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta; p.h0 = h0; p.dout = dout; p.dht = dht;
    p.dq = grad_q; p.dk = grad_k; p.dv = grad_v; p.dg = grad_g; p.dbeta = grad_beta; p.dh0 = grad_h0;
    p.B = B; p.T = T; p.H = H; p.N = N; p.scale = scale;
    p.hstore = hstore;
    p.dhstore = dhstore;
    // 1 and 2 are independent (B*H workgroups each) and run side by side: the
    // state gradient, end to start, on the side stream, and the state entering
    // every chunk (the forward kernel, no outputs) on the caller's stream
    e = stream_wait(s2, s);
    if (e != hipSuccess) return hip_fail(e, "backward fork");
    e = recorded(GDN_LAUNCH_BWD_DH, s2, [&] { return gdn::launch_bwd_dh(p, true, s2); });
    if (e != hipSuccess) return hip_fail(e, "backward state-gradient launch");
    e = recorded(GDN_LAUNCH_BWD_STATES, s, [&] { return gdn::launch_fwd(f, gdn::PHASE_STATES, true, s); });
    if (e != hipSuccess) return hip_fail(e, "backward state launch");
    e = stream_wait(s, s2);
    if (e != hipSuccess) return hip_fail(e, "backward join");
    // 3. local gradients of every chunk
    e = recorded(GDN_LAUNCH_BWD_LOCAL, s, [&] { return gdn::launch_bwd_local(p, true, s); });
    if (e != hipSuccess) return hip_fail(e, "backward local-gradient launch");
    return GDN_OK;
}

}  // extern "C"
