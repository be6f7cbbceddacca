// Fused chunked forward of the gated delta rule for gfx950.
//
// One workgroup of four wave64s runs one (batch, head, segment) task over a
// run of 64-token chunks.  Wave w owns dv columns [32w, 32w+32) of the 128x128
// float32 state, which lives in MFMA accumulators for the whole task: the state,
// the W/U-type intermediates and the per-chunk inverse never reach HBM (FlashQLA
// talk summary, onedev.kr, paragraph 3 names the per-chunk steps and criticises
// writing W, U and S to HBM and reading them back).
//
// Per chunk (gamma = in-chunk cumulative sum of g, Gamma = exp(gamma)):
//   prep (chunk-independent, paragraph 3 steps 1-2 and paragraph 6):
//     A0 = diag(beta) strict_lower(K K^T) and T0 = (I + A0)^-1 are gate-free;
//     the gated inverse is T = diag(Gamma) T0 diag(1/Gamma), whose entries
//     T0_rs Gamma_r/Gamma_s come from the 2C+1 exponentials
//     exp(gamma_r - gamma_C/2), exp(gamma_C/2 - gamma_r) and exp(gamma_C/2)
//     (the diagonal scaling pulled outside the inverse);
//     Tt = T diag(beta) and P = (Q K^T) o Mask, Mask_rs = Gamma_r/Gamma_s for s <= r.
//     T0 is built per 32x32 diagonal block as the product series
//     (I+M)(I+M^2)(I+M^4)(I+M^8)(I+M^16), M = -A0_block (exact: M^32 = 0), then
//     merged: T0_10 = -T0_11 A0_10 T0_00.
//   state step (paragraph 3 steps 3-4, serial over chunks):
//     X  = K H,  Y = V - diag(Gamma) X,  V' = Tt Y           (the true new values)
//     O  = scale (diag(Gamma) Q H + P V')
//     H <- Gamma_C H + K^T diag(Gamma_C / Gamma) V'
// Pass-1 of the sequence split (paragraph 4) runs the same step from a zero
// state without Q or O and also carries the gate-free segment transition
//     Mt <- (I - K^T T0 diag(beta) K) Mt,
// i.e. the same step on 128 extra columns with V = 0 and Gamma = 1.
//
// Memory path: the K, Q and V tiles of a chunk are copied from HBM straight
// into LDS (global_load_lds, 16 bytes per lane, double-buffered so the next
// chunk streams in under the current one); K^T and V in accumulator layout are
// read from the same row-major tiles with the transposing LDS read.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

enum { MODE_FULL = 0, MODE_PASS1 = 1 };
enum { INIT_ZERO = 0, INIT_H0 = 1, INIT_HS = 2 };
enum { DST_NONE = 0, DST_HT = 1, DST_HS_NEXT = 2, DST_PASS1 = 3 };

struct Task {
    int bh, seg;
    int c_begin, c_out, c_end;
    int mode, init, dst;
};

__device__ __forceinline__ int seg_start(int p, int N, int P) { return (int)(((long long)p * N) / P); }

// Decode the task of this workgroup.  Returns false when it has nothing to do.
__device__ bool decode_task(const FwdParams& prm, int phase, Task& t) {
    const int P = prm.P;
    if (phase == PHASE_SINGLE) {
        t.bh = blockIdx.x;
        t.seg = 0;
        t.c_begin = 0;
        t.c_out = 0;
        t.c_end = prm.N;
        t.mode = MODE_FULL;
        t.init = prm.h0 ? INIT_H0 : INIT_ZERO;
        t.dst = prm.ht ? DST_HT : DST_NONE;
        return true;
    }
    if (phase == PHASE_A) {
        t.bh = blockIdx.x / P;
        t.seg = blockIdx.x % P;
    } else {
        t.bh = blockIdx.x / (P - 1);
        t.seg = 1 + blockIdx.x % (P - 1);
    }
    const int p = t.seg;
    const bool window = prm.flags && prm.flags[t.bh] != 0;
    const int s = seg_start(p, prm.N, P), e = seg_start(p + 1, prm.N, P);
    t.c_out = s;
    t.c_end = e;
    if (window) {
        // sliding-window head (paragraph 5): warm up over the w chunks before s
        if (phase != PHASE_A) return false;
        t.c_begin = s - prm.w > 0 ? s - prm.w : 0;
        t.mode = MODE_FULL;
        t.init = (t.c_begin == 0 && prm.h0) ? INIT_H0 : INIT_ZERO;
        t.dst = (p == P - 1 && prm.ht) ? DST_HT : DST_NONE;
        return true;
    }
    if (phase == PHASE_A) {
        if (p == 0) {
            t.c_begin = 0;
            t.mode = MODE_FULL;
            t.init = prm.h0 ? INIT_H0 : INIT_ZERO;
            t.dst = DST_HS_NEXT;
            return true;
        }
        if (p == P - 1) return false;
        t.c_begin = s;
        t.c_out = e;  // no outputs
        t.mode = MODE_PASS1;
        t.init = INIT_ZERO;
        t.dst = DST_PASS1;
        return true;
    }
    // PHASE_C: exact head, segment p >= 1 from its true entering state
    t.c_begin = s;
    t.mode = MODE_FULL;
    t.init = INIT_HS;
    t.dst = (p == P - 1 && prm.ht) ? DST_HT : DST_NONE;
    return true;
}

// bf16 tiles are double-buffered; the float32 build (used for the small float32
// workloads only) single-buffers to fit in LDS.
template <typename T> struct NBuf { static constexpr int value = sizeof(T) == 2 ? 2 : 1; };

template <typename T>
struct Smem {
    static constexpr int NB = NBuf<T>::value;
    T kt[NB][kChunk * kDk];   // K, row-major [position][dk]
    T qt[NB][kChunk * kDk];   // Q
    T vt[NB][kChunk * kDv];   // V, row-major [position][dv]
    T tt[kChunk * kChunk];    // Tt = T diag(beta), row-major [r][s]
    T pm[kChunk * kChunk];    // P = (Q K^T) o Mask (full mode) / T0 diag(beta) (pass-1)
    float exch[64 * 16];      // accumulator hand-over between waves 0 and 1
    float gam[kChunk];        // gamma_r
    float gp[kChunk];         // exp(gamma_r - gamma_C/2)
    float gn[kChunk];         // exp(gamma_C/2 - gamma_r)
    float Gam[kChunk];        // Gamma_r
    float E[kChunk];          // Gamma_C / Gamma_r
    float beta[kChunk];
    float scal[4];            // [0] Gamma_C, [1] pairwise-exp flag
};

__device__ __forceinline__ void wait_all_loads() {
    // vmcnt(0) and lgkmcnt(0): this wave's global->LDS copies and LDS writes are done
    __builtin_amdgcn_s_waitcnt(0x0070);
}

// Copy one 64 x 128 tile of chunk rows [t0, t0 + nvalid) of head (b, h) into a
// swizzled row-major LDS tile.  Full chunks go HBM -> LDS directly (each lane's 16
// bytes land at slot base + 16*lane, so the lane fetches the chunk that belongs
// there); a short last chunk goes through registers and is zero-filled.
template <typename T>
__device__ __forceinline__ void load_tile(T* tile, const T* src, int b, int h, int T_, int H, int t0,
                                          int nvalid) {
    constexpr int EPC = 16 / (int)sizeof(T);
    constexpr int CPR = kDk / EPC;                 // 16-byte chunks per row
    constexpr int ROUNDS = kChunk * CPR / 256;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const size_t rowstride = (size_t)H * kDk;
    const T* base = src + (((size_t)b * T_ + t0) * H + h) * kDk;
    if (nvalid == kChunk) {
#pragma unroll
        for (int i = 0; i < ROUNDS; ++i) {
            const int L = (i * 4 + w) * 64 + lane;     // slot index in the tile
            const int row = L / CPR, slot = L % CPR;
            const int c = slot ^ swz(row);
            const T* gp = base + row * rowstride + c * EPC;
            T* lbase = tile + (i * 4 + w) * 64 * EPC;
            __builtin_amdgcn_global_load_lds((const void*)gp,
                                             (__attribute__((address_space(3))) void*)lbase, 16, 0, 0);
        }
    } else {
        typedef uint32_t u4 __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int i = 0; i < ROUNDS; ++i) {
            const int L = (i * 4 + w) * 64 + lane;
            const int row = L / CPR, slot = L % CPR;
            const int c = slot ^ swz(row);
            u4 v = {0u, 0u, 0u, 0u};
            if (row < nvalid) v = *(const u4*)(base + row * rowstride + c * EPC);
            *(u4*)(tile + L * EPC) = v;
        }
    }
}

// Gate vectors of one chunk from g (wave 0) and beta (wave 1): the in-chunk scan
// and the 2C+1 exponentials of the factored gate (paragraph 6), re-centred at
// gamma_C/2 so both factors stay within exp(|gamma_C|/2).  Chunks whose decay
// exceeds that safe range use pairwise exponentials exp(gamma_r - gamma_s).
template <typename T>
__device__ __forceinline__ void gate_vectors(Smem<T>& sm, float gb, float& gsum_acc) {
    const int tid = threadIdx.x, lane = tid & 63;
    if (tid < 64) {
        float gam = wave_inclusive_scan(gb);
        float gC = __shfl(gam, 63, 64);
        float half = 0.5f * gC;
        bool pairwise = gC < -160.f;
        float gp = __expf(gam - half);
        float gn = __expf(half - gam);
        float eh = __expf(half);
        sm.gam[lane] = gam;
        sm.gp[lane] = gp;
        sm.gn[lane] = gn;
        sm.Gam[lane] = pairwise ? __expf(gam) : gp * eh;
        sm.E[lane] = pairwise ? __expf(gC - gam) : gn * eh;
        if (lane == 0) {
            sm.scal[0] = pairwise ? __expf(gC) : eh * eh;
            sm.scal[1] = pairwise ? 1.f : 0.f;
        }
        gsum_acc += gC;
    } else if (tid < 128) {
        sm.beta[lane] = gb;
    }
}

__device__ __forceinline__ float load_gb(const FwdParams& prm, int b, int h, int t0, int nvalid) {
    const int tid = threadIdx.x, pos = tid & 63;
    float x = 0.f;
    if (tid < 128 && pos < nvalid) {
        size_t go = ((size_t)b * prm.T + t0 + pos) * prm.H + h;
        x = tid < 64 ? prm.g[go] : prm.beta[go];
    }
    return x;
}

// threadIdx.x hidden from loop-invariant code motion: the swizzled LDS addresses
// derived from it are then recomputed in each chunk step instead of being
// hoisted out of the chunk loop, where ~200 precomputed addresses would stay
// live and push the state and operands into scratch.
__device__ __forceinline__ int opaque_tid() {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}

// Per-position vector values for the 16 accumulator rows of row tile rt.
__device__ __forceinline__ f32x16 rows_of(const float* vec, int rt, int g) {
    f32x16 out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f32x4 x = *(const f32x4*)(vec + 32 * rt + 8 * i + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) out[4 * i + e] = x[e];
    }
    return out;
}

// Gate factor Gamma_r / Gamma_s for s <= r.
template <typename T>
__device__ __forceinline__ float mask_factor(const Smem<T>& sm, int r, int s, bool pairwise) {
    return pairwise ? __expf(sm.gam[r] - sm.gam[s]) : sm.gp[r] * sm.gn[s];
}

// 32x32 product of two accumulator-form operands: returns c + X Y given
// xt = acc(X^T) (its fragments are the A fragments of X) and y = acc(Y).
template <typename T>
__device__ __forceinline__ f32x16 mm_acc(const f32x16& xt, const f32x16& y, f32x16 c) {
    c = mma(acc_frag<T>(xt, 0), acc_frag<T>(y, 0), c);
    c = mma(acc_frag<T>(xt, 1), acc_frag<T>(y, 1), c);
    return c;
}

// Inverse of (I + Nd) for one 32x32 diagonal block, Nd = diag(beta) strict_lower(S),
// from S = K_p K_p^T (acc form).  Returns acc(T0_pp) in z and acc(T0_pp^T) in zt.
template <typename T>
__device__ __forceinline__ void diag_inverse(const f32x16& S, const float* beta_blk, int n, int g,
                                             f32x16& z, f32x16& zt) {
    f32x16 m, mt;
    const float bn = beta_blk[n];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        int row = rho(g, r);
        m[r] = (n < row) ? -beta_blk[row] * S[r] : 0.f;   // M = -Nd
        mt[r] = (row < n) ? -bn * S[r] : 0.f;             // M^T (S is symmetric)
        float id = (row == n) ? 1.f : 0.f;
        z[r] = id + m[r];
        zt[r] = id + mt[r];
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        f32x16 m2 = mm_acc<T>(mt, m, zero16());    // M^(2^(it+1))
        f32x16 m2t = mm_acc<T>(m, mt, zero16());   // its transpose
        m = m2;
        mt = m2t;
        f32x16 zn = mm_acc<T>(zt, m, z);           // Z (I + M^(2^(it+1)))
        f32x16 ztn = mm_acc<T>(m, zt, zt);         // transpose of the same
        z = zn;
        zt = ztn;
    }
}

// Chunk-independent prep of one chunk: Tt (and T0 diag(beta) in pass-1) and P.
template <typename T, int MODE>
__device__ __forceinline__ void chunk_prep(Smem<T>& sm, int buf, bool emit, bool pairwise) {
    using F = typename FragOf<T>::type;
    const int tid = opaque_tid(), w = tid >> 6, lane = tid & 63, n = lane & 31, g = lane >> 5;
    const T* kt = sm.kt[buf];
    const T* qt = sm.qt[buf];
    f32x16 w1_W;
    if (w < 2) {
        const int p = w;
        f32x16 S = zero16(), x = zero16();
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            F kf = afrag<T, kDk>(kt, 32 * p + n, ks, g);
            S = mma(kf, kf, S);
            // wave 1 also needs K_1 K_0^T: A = K_1 rows, B = K_0^T (its fragment is a K_0 row read)
            if (p == 1) x = mma(kf, afrag<T, kDk>(kt, n, ks, g), x);
        }
        f32x16 z, zt;
        diag_inverse<T>(S, sm.beta + 32 * p, n, g, z, zt);
        // acc(T0^T): lane n holds row 32p+n of T0, registers = columns 32p + rho
        const int row = 32 * p + n;
#pragma unroll
        for (int ksl = 0; ksl < 2; ++ksl) {
            F f, f0;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                int col = 32 * p + rho(g, 8 * ksl + j);
                float t0v = zt[8 * ksl + j] * sm.beta[col];
                f[j] = (T)(col <= row ? t0v * mask_factor(sm, row, col, pairwise) : 0.f);
                f0[j] = (T)t0v;
            }
            st_afrag<T, kChunk>(sm.tt, row, 2 * p + ksl, g, f);
            if (MODE == MODE_PASS1) st_afrag<T, kChunk>(sm.pm, row, 2 * p + ksl, g, f0);
        }
        if (p == 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sm.exch[lane * 16 + r] = z[r];
        } else {
            // acc(A0_10) = diag(beta_1) K_1 K_0^T, then W = A0_10^T T0_11^T
            f32x16 a10;
#pragma unroll
            for (int r = 0; r < 16; ++r) a10[r] = sm.beta[32 + rho(g, r)] * x[r];
            w1_W = mm_acc<T>(a10, zt, zero16());
        }
    } else if (MODE == MODE_FULL && emit) {
        // acc(K_j Q_i^T): lane n holds row 32i+n of Q K^T, registers = columns 32j+rho
        const int ntile = (w == 2) ? 2 : 1;
        for (int tix = 0; tix < ntile; ++tix) {
            const int i = (w == 2) ? tix : 1;
            const int j = (w == 2) ? tix : 0;
            f32x16 x = zero16();
#pragma unroll
            for (int ks = 0; ks < 8; ++ks)
                x = mma(afrag<T, kDk>(kt, 32 * j + n, ks, g), afrag<T, kDk>(qt, 32 * i + n, ks, g), x);
            const int row = 32 * i + n;
#pragma unroll
            for (int ksl = 0; ksl < 2; ++ksl) {
                F f;
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    int col = 32 * j + rho(g, 8 * ksl + jj);
                    f[jj] = (T)(col <= row ? x[8 * ksl + jj] * mask_factor(sm, row, col, pairwise) : 0.f);
                }
                st_afrag<T, kChunk>(sm.pm, row, 2 * j + ksl, g, f);
            }
        }
    }
    __syncthreads();
    if (w == 1) {
        // T0_10^T = -T0_00^T (A0_10^T T0_11^T); the A fragments of T0_00^T are acc(T0_00)
        f32x16 t00;
#pragma unroll
        for (int r = 0; r < 16; ++r) t00[r] = sm.exch[lane * 16 + r];
        f32x16 y = mm_acc<T>(t00, w1_W, zero16());
        const int row = 32 + n;
#pragma unroll
        for (int ksl = 0; ksl < 2; ++ksl) {
            F f, f0;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                int col = rho(g, 8 * ksl + j);
                float t0v = -y[8 * ksl + j] * sm.beta[col];
                f[j] = (T)(t0v * mask_factor(sm, row, col, pairwise));
                f0[j] = (T)t0v;
            }
            st_afrag<T, kChunk>(sm.tt, row, ksl, g, f);
            if (MODE == MODE_PASS1) st_afrag<T, kChunk>(sm.pm, row, ksl, g, f0);
        }
    }
    __syncthreads();
}

// H <- a H + K^T B with B given as four fragments over the chunk positions.
template <typename T>
__device__ __forceinline__ void state_update(const T* kt, f32x16* Hs, float a,
                                             const typename FragOf<T>::type* bf, int lane) {
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
        f32x16 acc = Hs[ht] * a;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc = mma(tfrag<T, kDk>(kt, 32 * ht, ks, lane), bf[ks], acc);
        Hs[ht] = acc;
    }
}

// X = K Hm for the two 32-row position tiles (Hm: the four dk tiles of a state).
template <typename T>
__device__ __forceinline__ void k_times_state(const T* kt, const f32x16* Hm, int n, int g, f32x16* X) {
    using F = typename FragOf<T>::type;
    X[0] = zero16();
    X[1] = zero16();
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        F hf = acc_frag<T>(Hm[ks >> 1], ks & 1);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) X[rt] = mma(afrag<T, kDk>(kt, 32 * rt + n, ks, g), hf, X[rt]);
    }
}

// Lower-triangular 64x64 (row-major tile) times the 64x32 operand given as fragments.
template <typename T>
__device__ __forceinline__ void tri_times(const T* tile, const typename FragOf<T>::type* yf, int n,
                                          int g, f32x16* out) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) out[0] = mma(afrag<T, kChunk>(tile, n, ks, g), yf[ks], out[0]);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) out[1] = mma(afrag<T, kChunk>(tile, 32 + n, ks, g), yf[ks], out[1]);
}

// The serial state step of one chunk for this wave's 32 state columns.
template <typename T, int MODE>
__device__ __forceinline__ void chunk_state(const FwdParams& prm, Smem<T>& sm, int buf, int b, int h,
                                            int t0, int nvalid, bool emit, f32x16* Hs, f32x16* Ms) {
    using F = typename FragOf<T>::type;
    const int tid = opaque_tid(), w = tid >> 6, lane = tid & 63, n = lane & 31, g = lane >> 5;
    const T* kt = sm.kt[buf];
    const T* qt = sm.qt[buf];
    const T* vt = sm.vt[buf];

    f32x16 X[2];
    k_times_state<T>(kt, Hs, n, g, X);
    // Y = V - diag(Gamma) X (V in accumulator layout via the transposing read)
    F yf[4];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        F v0 = tfrag<T, kDv>(vt, 32 * w, 2 * rt, lane);
        F v1 = tfrag<T, kDv>(vt, 32 * w, 2 * rt + 1, lane);
        f32x16 gr = rows_of(sm.Gam, rt, g);
        f32x16 y;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            y[j] = (float)v0[j] - gr[j] * X[rt][j];
            y[8 + j] = (float)v1[j] - gr[8 + j] * X[rt][8 + j];
        }
        yf[2 * rt] = acc_frag<T>(y, 0);
        yf[2 * rt + 1] = acc_frag<T>(y, 1);
    }
    f32x16 Vp[2] = {zero16(), zero16()};
    tri_times<T>(sm.tt, yf, n, g, Vp);

    if (MODE == MODE_FULL && emit) {
        // O = scale (diag(Gamma) Q H + P V')
        f32x16 QH[2] = {zero16(), zero16()};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            F hf = acc_frag<T>(Hs[ks >> 1], ks & 1);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) QH[rt] = mma(afrag<T, kDk>(qt, 32 * rt + n, ks, g), hf, QH[rt]);
        }
        F vf[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) vf[ks] = acc_frag<T>(Vp[ks >> 1], ks & 1);
        f32x16 O[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) O[rt] = rows_of(sm.Gam, rt, g) * QH[rt];
        tri_times<T>(sm.pm, vf, n, g, O);
        T* o = (T*)prm.o;
        const int col = 32 * w + n;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                int pos = 32 * rt + rho(g, r);
                if (pos < nvalid)
                    o[(((size_t)b * prm.T + t0 + pos) * prm.H + h) * kDv + col] = (T)(prm.scale * O[rt][r]);
            }
    }
    // H <- Gamma_C H + K^T diag(E) V'
    F ef[4];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        f32x16 ev = Vp[rt] * rows_of(sm.E, rt, g);
        ef[2 * rt] = acc_frag<T>(ev, 0);
        ef[2 * rt + 1] = acc_frag<T>(ev, 1);
    }
    state_update<T>(kt, Hs, sm.scal[0], ef, lane);

    if (MODE == MODE_PASS1) {
        // Mt <- Mt - K^T T0 diag(beta) K Mt  (V = 0, no gates)
        k_times_state<T>(kt, Ms, n, g, X);
        F mf[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) mf[ks] = acc_frag<T>(-X[ks >> 1], ks & 1);
        f32x16 VpM[2] = {zero16(), zero16()};
        tri_times<T>(sm.pm, mf, n, g, VpM);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) mf[ks] = acc_frag<T>(VpM[ks >> 1], ks & 1);
        state_update<T>(kt, Ms, 1.f, mf, lane);
    }
}

__device__ __forceinline__ void load_state(const float* src, int w, int lane, f32x16* Hs) {
    const int n = lane & 31, g = lane >> 5;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            Hs[ht][r] = src[(32 * ht + rho(g, r)) * kDv + 32 * w + n];
}
__device__ __forceinline__ void store_state(float* dst, int w, int lane, const f32x16* Hs) {
    const int n = lane & 31, g = lane >> 5;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            dst[(32 * ht + rho(g, r)) * kDv + 32 * w + n] = Hs[ht][r];
}

template <typename T>
__device__ __forceinline__ void load_chunk_tiles(const FwdParams& prm, Smem<T>& sm, int buf, int b,
                                                 int h, int c, bool need_q) {
    const int t0 = c * kChunk;
    const int nvalid = prm.T - t0 < kChunk ? prm.T - t0 : kChunk;
    load_tile<T>(sm.kt[buf], (const T*)prm.k, b, h, prm.T, prm.H, t0, nvalid);
    load_tile<T>(sm.vt[buf], (const T*)prm.v, b, h, prm.T, prm.H, t0, nvalid);
    if (need_q) load_tile<T>(sm.qt[buf], (const T*)prm.q, b, h, prm.T, prm.H, t0, nvalid);
}

template <typename T, int MODE>
__device__ void run_task(const FwdParams& prm, Smem<T>& sm, const Task& tk) {
    constexpr int NB = NBuf<T>::value;
    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, g = lane >> 5, n = lane & 31;
    const int b = tk.bh / prm.H, h = tk.bh % prm.H;
    const size_t SS = (size_t)kDk * kDv;

    f32x16 Hs[4], Ms[4];
    if (tk.init == INIT_H0) {
        load_state(prm.h0 + (size_t)tk.bh * SS, w, lane, Hs);
    } else if (tk.init == INIT_HS) {
        load_state(prm.hs + ((size_t)tk.bh * prm.P + tk.seg) * SS, w, lane, Hs);
    } else {
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) Hs[ht] = zero16();
    }
    if (MODE == MODE_PASS1) {
#pragma unroll
        for (int ht = 0; ht < 4; ++ht)
#pragma unroll
            for (int r = 0; r < 16; ++r) Ms[ht][r] = (32 * ht + rho(g, r) == 32 * w + n) ? 1.f : 0.f;
    }
    float gsum = 0.f;

    auto nvalid_of = [&](int c) { return prm.T - c * kChunk < kChunk ? prm.T - c * kChunk : kChunk; };
    float gb = load_gb(prm, b, h, tk.c_begin * kChunk, nvalid_of(tk.c_begin));
    if (NB == 2)
        load_chunk_tiles<T>(prm, sm, 0, b, h, tk.c_begin, MODE == MODE_FULL && tk.c_begin >= tk.c_out);

    for (int c = tk.c_begin; c < tk.c_end; ++c) {
        const bool emit = MODE == MODE_FULL && c >= tk.c_out;
        const int buf = NB == 2 ? ((c - tk.c_begin) & 1) : 0;
        const int t0 = c * kChunk, nvalid = nvalid_of(c);
        if (NB == 1) {
            __syncthreads();   // the previous chunk is done with the single buffer
            load_chunk_tiles<T>(prm, sm, 0, b, h, c, emit);
        }
        wait_all_loads();
        __syncthreads();       // chunk c is in LDS; the previous chunk is done with buffer buf^1
        if (NB == 2 && c + 1 < tk.c_end)
            load_chunk_tiles<T>(prm, sm, buf ^ 1, b, h, c + 1, MODE == MODE_FULL && c + 1 >= tk.c_out);
        gate_vectors<T>(sm, gb, gsum);
        if (c + 1 < tk.c_end) gb = load_gb(prm, b, h, t0 + kChunk, nvalid_of(c + 1));
        __syncthreads();
        const bool pairwise = sm.scal[1] != 0.f;
        chunk_prep<T, MODE>(sm, buf, emit, pairwise);
        chunk_state<T, MODE>(prm, sm, buf, b, h, t0, nvalid, emit, Hs, Ms);
    }

    if (tk.dst == DST_HT) {
        store_state(prm.ht + (size_t)tk.bh * SS, w, lane, Hs);
    } else if (tk.dst == DST_HS_NEXT) {
        store_state(prm.hs + ((size_t)tk.bh * prm.P + tk.seg + 1) * SS, w, lane, Hs);
    } else if (tk.dst == DST_PASS1) {
        const size_t o = ((size_t)tk.bh * prm.P + tk.seg) * SS;
        store_state(prm.bz + o, w, lane, Hs);
        store_state(prm.mt + o, w, lane, Ms);
        if (tid == 0) prm.gsum[(size_t)tk.bh * prm.P + tk.seg] = gsum;
    }
}

template <typename T, int PHASE>
__global__ __launch_bounds__(256, 1) void gdn_fwd_kernel(FwdParams prm) {
    extern __shared__ __attribute__((aligned(16))) char smem_raw[];
    Smem<T>& sm = *reinterpret_cast<Smem<T>*>(smem_raw);
    Task tk;
    if (!decode_task(prm, PHASE, tk)) return;
    // only the first launch of a split forward has pass-1 tasks
    if (PHASE == PHASE_A && tk.mode == MODE_PASS1)
        run_task<T, MODE_PASS1>(prm, sm, tk);
    else
        run_task<T, MODE_FULL>(prm, sm, tk);
}

template <typename T, int PHASE>
hipError_t launch_phase(const FwdParams& p, int grid, hipStream_t s) {
    const size_t lds = sizeof(Smem<T>);
    static bool configured = false;
    if (!configured) {
        hipError_t e = hipFuncSetAttribute((const void*)gdn_fwd_kernel<T, PHASE>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        configured = true;
    }
    hipLaunchKernelGGL((gdn_fwd_kernel<T, PHASE>), dim3(grid), dim3(256), lds, s, p);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_fwd_t(const FwdParams& p, int phase, hipStream_t s) {
    if (phase == PHASE_SINGLE) return launch_phase<T, PHASE_SINGLE>(p, p.B * p.H, s);
    if (phase == PHASE_A) return launch_phase<T, PHASE_A>(p, p.B * p.H * p.P, s);
    return launch_phase<T, PHASE_C>(p, p.B * p.H * (p.P - 1), s);
}

}  // namespace

hipError_t launch_fwd(const FwdParams& p, int phase, bool bf16, hipStream_t s) {
    return bf16 ? launch_fwd_t<__bf16>(p, phase, s) : launch_fwd_t<float>(p, phase, s);
}

}  // namespace gdn
