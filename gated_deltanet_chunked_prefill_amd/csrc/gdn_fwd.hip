// Fused chunked forward of the gated delta rule for gfx950.
//
// One workgroup of four wave64s runs one (batch, head, segment) task over a
// run of 64-token chunks.  Wave w owns dv columns [32w, 32w+32) of the 128x128
// float32 state, which lives in MFMA accumulators for the whole task: the state,
// W/U-type intermediates and the per-chunk inverse never reach HBM (FlashQLA
// talk summary, onedev.kr, paragraph 3 names the per-chunk steps and criticises
// writing W, U and S to HBM and reading them back).
//
// Per chunk (gamma = in-chunk cumulative sum of g, Gamma = exp(gamma)):
//   prep (chunk-independent, paragraph 3 steps 1-2 and paragraph 6):
//     A0 = diag(beta) strict_lower(K K^T) and T0 = (I + A0)^-1 are gate-free;
//     the gated inverse is T = diag(Gamma) T0 diag(1/Gamma), formed from the
//     2C+1 exponentials exp(gamma_r - gamma_C/2), exp(gamma_C/2 - gamma_r) and
//     exp(gamma_C/2) (the diagonal scaling pulled outside the inverse);
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

// V goes through LDS (transposed, read back as accumulator-layout fragments)
// for bf16; the float32 build keeps V in registers so that its tiles fit in LDS.
template <typename T> struct VInLds { static constexpr bool value = sizeof(T) == 2; };

template <typename T>
struct Smem {
    T krm[kChunk * kDk];   // K, A layout, rows = position, contraction = dk
    T qrm[kChunk * kDk];   // Q, same layout
    T ktr[kDk * kChunk];   // K^T, A layout, rows = dk, contraction = position
    T vtr[VInLds<T>::value ? kDv * kChunk : 8];  // V^T, A layout, rows = dv, contraction = position
    T tt[kChunk * kChunk];   // Tt = T diag(beta), rows r, contraction s
    // P = (Q K^T) o Mask in full mode; T0 diag(beta) (gate-free) in pass-1
    T pm[kChunk * kChunk];
    float exch[64 * 16];     // accumulator hand-over between waves
    float gam[kChunk];       // gamma_r
    float gp[kChunk];        // exp(gamma_r - gamma_C/2)
    float gn[kChunk];        // exp(gamma_C/2 - gamma_r)
    float Gam[kChunk];       // Gamma_r
    float E[kChunk];         // Gamma_C / Gamma_r
    float beta[kChunk];
    float scal[4];           // [0] Gamma_C, [1] pairwise-exp flag
};

// Chunk staging registers: one 16-byte vector per thread and row group.
template <typename T> struct Vec;
template <> struct Vec<__bf16> {
    typedef __bf16 v16 __attribute__((ext_vector_type(8)));
    typedef __bf16 v4 __attribute__((ext_vector_type(4)));
};
template <> struct Vec<float> {
    typedef float v16 __attribute__((ext_vector_type(4)));
    typedef float v4 __attribute__((ext_vector_type(4)));
};

template <typename T>
struct Stage {
    static constexpr int VE = 16 / (int)sizeof(T);          // elements per vector
    static constexpr int VPR = kDk / VE;                     // vectors per row
    static constexpr int NV = kChunk * VPR / 256;            // vectors per thread
    typename Vec<T>::v16 kv[NV];
    typename Vec<T>::v16 qv[NV];
    typename Vec<T>::v16 vv[VInLds<T>::value ? NV : 1];
    float gb;     // g (wave 0) or beta (wave 1) of position (tid & 63)
};

// Read the V values this lane needs for the state step, in accumulator layout.
template <typename T>
__device__ __forceinline__ void load_v(const T* v, int b, int h, int H, int T_, int t0, int nvalid,
                                       int col, int g, float* out /*32*/) {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            int pos = 32 * rt + rho(g, r);
            float x = 0.f;
            if (pos < nvalid) x = (float)v[(((size_t)b * T_ + t0 + pos) * H + h) * kDv + col];
            out[16 * rt + r] = x;
        }
}

template <typename T>
__device__ __forceinline__ void load_stage(const FwdParams& prm, int b, int h, int t0, int nvalid,
                                           bool need_q, Stage<T>& st) {
    const int tid = threadIdx.x;
    const T* k = (const T*)prm.k;
    const T* q = (const T*)prm.q;
#pragma unroll
    for (int i = 0; i < Stage<T>::NV; ++i) {
        int vi = tid + 256 * i;
        int row = vi / Stage<T>::VPR, cv = vi % Stage<T>::VPR;
        size_t off = (((size_t)b * prm.T + t0 + row) * prm.H + h) * kDk + cv * Stage<T>::VE;
        typedef typename Vec<T>::v16 V16;
        V16 z;
#pragma unroll
        for (int e = 0; e < Stage<T>::VE; ++e) z[e] = (T)0.f;
        st.kv[i] = row < nvalid ? *(const V16*)(k + off) : z;
        st.qv[i] = (need_q && row < nvalid) ? *(const V16*)(q + off) : z;
        if (VInLds<T>::value) st.vv[i] = row < nvalid ? *(const V16*)((const T*)prm.v + off) : z;
    }
    const int pos = tid & 63;
    float x = 0.f;
    if (tid < 128 && pos < nvalid) {
        size_t go = ((size_t)b * prm.T + t0 + pos) * prm.H + h;
        x = tid < 64 ? prm.g[go] : prm.beta[go];
    }
    st.gb = x;
}

// Write staged K/Q into the A-layout tiles, K^T into its own tile, and the
// per-position gate vectors (wave 0 does the in-chunk scan).
template <typename T>
__device__ __forceinline__ void store_stage(Smem<T>& sm, const Stage<T>& st, bool need_q,
                                            float& gsum_acc) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < Stage<T>::NV; ++i) {
        int vi = tid + 256 * i;
        int row = vi / Stage<T>::VPR, cv = vi % Stage<T>::VPR;
        typedef typename Vec<T>::v4 V4;
        const auto& ke = st.kv[i];
        const auto& qe = st.qv[i];
#pragma unroll
        for (int c4 = 0; c4 < Stage<T>::VE; c4 += 4) {
            int col = cv * Stage<T>::VE + c4;
            int off = lds_elem(row, col, kDk);
            V4 kk, qq;
#pragma unroll
            for (int e = 0; e < 4; ++e) { kk[e] = ke[c4 + e]; qq[e] = qe[c4 + e]; }
            *(V4*)(sm.krm + off) = kk;
            if (need_q) *(V4*)(sm.qrm + off) = qq;
        }
#pragma unroll
        for (int e = 0; e < Stage<T>::VE; ++e) {
            int col = cv * Stage<T>::VE + e;
            sm.ktr[lds_elem(col, row, kChunk)] = ke[e];
            if (VInLds<T>::value) sm.vtr[lds_elem(col, row, kChunk)] = st.vv[i][e];
        }
    }
    const int lane = tid & 63;
    if (tid < 64) {
        // gate prep with the diagonal scaling pulled outside the inverse (paragraph 6):
        // 2C+1 exponentials per chunk, re-centred at gamma_C/2 so that both
        // factors stay within exp(|gamma_C|/2).  Chunks whose decay exceeds the
        // safe range fall back to pairwise exponentials exp(gamma_r - gamma_s).
        float gam = wave_inclusive_scan(st.gb);
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
        sm.beta[lane] = st.gb;
    }
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

// 32x32 product of two accumulator-form operands: returns acc(X Y) given
// xt = acc(X^T) (its fragments are the A fragments of X) and y = acc(Y).
template <typename T>
__device__ __forceinline__ f32x16 mm_acc(const f32x16& xt, const f32x16& y, f32x16 c) {
    c = mma(acc_frag<T>(xt, 0), acc_frag<T>(y, 0), c);
    c = mma(acc_frag<T>(xt, 1), acc_frag<T>(y, 1), c);
    return c;
}

// Inverse of (I + Nd) for one 32x32 diagonal block from S = K_p K_p^T (acc form).
// Returns acc(T0_pp) in z and acc(T0_pp^T) in zt.
template <typename T>
__device__ __forceinline__ void diag_inverse(const f32x16& S, const float* beta_blk, int n, int g,
                                             f32x16& z, f32x16& zt) {
    f32x16 m, mt;
    const float bn = beta_blk[n];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        int row = rho(g, r);
        m[r] = (n < row) ? -beta_blk[row] * S[r] : 0.f;   // M = -diag(beta) strict_lower(S)
        mt[r] = (row < n) ? -bn * S[r] : 0.f;             // M^T
        float id = (row == n) ? 1.f : 0.f;
        z[r] = id + m[r];
        zt[r] = id + mt[r];
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        f32x16 m2 = mm_acc<T>(mt, m, zero16());    // M^2
        f32x16 m2t = mm_acc<T>(m, mt, zero16());   // (M^2)^T = M^T M^T
        m = m2;
        mt = m2t;
        f32x16 zn = mm_acc<T>(zt, m, z);           // Z + Z M^(2^k)
        f32x16 ztn = mm_acc<T>(m, zt, zt);         // Z^T + (M^(2^k))^T Z^T
        z = zn;
        zt = ztn;
    }
}

template <typename T, int MODE>
__device__ __forceinline__ void chunk_step(const FwdParams& prm, Smem<T>& sm, const Task& tk,
                                           int b, int h, int c, bool emit, const float* vreg,
                                           f32x16* Hs, f32x16* Ms) {
    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, n = lane & 31, g = lane >> 5;
    using F = typename FragOf<T>::type;
    const int t0 = c * kChunk;
    const int nvalid = prm.T - t0 < kChunk ? prm.T - t0 : kChunk;
    const bool pairwise = sm.scal[1] != 0.f;

    // ---------------- prep: inverse (waves 0, 1) and P tiles (waves 2, 3) ----------------
    f32x16 w1_W;  // wave 1: W = A0_10^T T0_11^T
    if (w < 2) {
        const int p = w;
        F kf[8];
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) kf[ks] = ld_frag<T>(sm.krm, 32 * p + n, ks, g, kDk);
        f32x16 S = zero16();
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) S = mma(kf[ks], kf[ks], S);
        f32x16 z, zt;
        diag_inverse<T>(S, sm.beta + 32 * p, n, g, z, zt);
        // A-layout fragments of the diagonal block of Tt (and T0 diag(beta)):
        // acc(T0^T) lane n holds row 32p+n of T0, registers = columns.
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
            st_frag<T>(sm.tt, row, 2 * p + ksl, g, kChunk, f);
            if (MODE == MODE_PASS1) st_frag<T>(sm.pm, row, 2 * p + ksl, g, kChunk, f0);
        }
        if (p == 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sm.exch[lane * 16 + r] = z[r];
        } else {
            // acc(A0_10) = diag(beta_1) K_1 K_0^T, then W = A0_10^T T0_11^T
            f32x16 x = zero16();
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) x = mma(kf[ks], ld_frag<T>(sm.krm, n, ks, g, kDk), x);
            f32x16 a10;
#pragma unroll
            for (int r = 0; r < 16; ++r) a10[r] = sm.beta[32 + rho(g, r)] * x[r];
            // NOTE: x = acc(K_1 K_0^T) has lane n = column (block-0 position), rows = block-1 positions.
            w1_W = mm_acc<T>(a10, zt, zero16());
        }
    } else if (emit) {
        // P^T tiles: acc(K_j Q_i^T) lane n holds row 32i+n of Q K^T, registers = columns 32j+rho
        const int ntile = (w == 2) ? 2 : 1;
        for (int tix = 0; tix < ntile; ++tix) {
            int i, j;
            if (w == 2) { i = tix; j = tix; } else { i = 1; j = 0; }
            f32x16 x = zero16();
#pragma unroll
            for (int ks = 0; ks < 8; ++ks)
                x = mma(ld_frag<T>(sm.krm, 32 * j + n, ks, g, kDk),
                        ld_frag<T>(sm.qrm, 32 * i + n, ks, g, kDk), x);
            const int row = 32 * i + n;
#pragma unroll
            for (int ksl = 0; ksl < 2; ++ksl) {
                F f;
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    int col = 32 * j + rho(g, 8 * ksl + jj);
                    f[jj] = (T)(col <= row ? x[8 * ksl + jj] * mask_factor(sm, row, col, pairwise)
                                           : 0.f);
                }
                st_frag<T>(sm.pm, row, 2 * j + ksl, g, kChunk, f);
            }
        }
    }
    __syncthreads();
    if (w == 1) {
        // T0_10^T = -T0_00^T (A0_10^T T0_11^T): A fragments of T0_00^T are acc(T0_00)
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
            st_frag<T>(sm.tt, row, ksl, g, kChunk, f);
            if (MODE == MODE_PASS1) st_frag<T>(sm.pm, row, ksl, g, kChunk, f0);
        }
    }
    __syncthreads();

    // ---------------- state step (every wave, its 32 columns) ----------------
    F hf[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) hf[ks] = acc_frag<T>(Hs[ks >> 1], ks & 1);
    f32x16 X[2] = {zero16(), zero16()};
    f32x16 QH[2] = {zero16(), zero16()};
    f32x16 XM[2] = {zero16(), zero16()};
    F mf[8];
    if (MODE == MODE_PASS1) {
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) mf[ks] = acc_frag<T>(Ms[ks >> 1], ks & 1);
    }
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            F a = ld_frag<T>(sm.krm, 32 * rt + n, ks, g, kDk);
            X[rt] = mma(a, hf[ks], X[rt]);
            if (MODE == MODE_PASS1) XM[rt] = mma(a, mf[ks], XM[rt]);
        }
    }
    if (MODE == MODE_FULL && emit) {
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
                QH[rt] = mma(ld_frag<T>(sm.qrm, 32 * rt + n, ks, g, kDk), hf[ks], QH[rt]);
    }
    // Y = V - diag(Gamma) X
    f32x16 Y[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        f32x16 gr = rows_of(sm.Gam, rt, g);
        f32x16 vr;
        if constexpr (VInLds<T>::value) {
            F v0 = ld_frag<T>(sm.vtr, 32 * w + n, 2 * rt, g, kChunk);
            F v1 = ld_frag<T>(sm.vtr, 32 * w + n, 2 * rt + 1, g, kChunk);
#pragma unroll
            for (int j = 0; j < 8; ++j) { vr[j] = (float)v0[j]; vr[8 + j] = (float)v1[j]; }
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) vr[r] = vreg[16 * rt + r];
        }
        Y[rt] = vr - gr * X[rt];
    }
    F yf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) yf[ks] = acc_frag<T>(Y[ks >> 1], ks & 1);
    // V' = Tt Y (Tt lower triangular: row tile 0 needs k-steps 0-1 only)
    f32x16 Vp[2] = {zero16(), zero16()};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) Vp[0] = mma(ld_frag<T>(sm.tt, n, ks, g, kChunk), yf[ks], Vp[0]);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) Vp[1] = mma(ld_frag<T>(sm.tt, 32 + n, ks, g, kChunk), yf[ks], Vp[1]);
    f32x16 VpM[2] = {zero16(), zero16()};
    if (MODE == MODE_PASS1) {
        F ymf[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            f32x16 t = XM[ks >> 1];
            ymf[ks] = acc_frag<T>(-t, ks & 1);
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            VpM[0] = mma(ld_frag<T>(sm.pm, n, ks, g, kChunk), ymf[ks], VpM[0]);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            VpM[1] = mma(ld_frag<T>(sm.pm, 32 + n, ks, g, kChunk), ymf[ks], VpM[1]);
    }
    if (MODE == MODE_FULL && emit) {
        F vf[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) vf[ks] = acc_frag<T>(Vp[ks >> 1], ks & 1);
        f32x16 O[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) O[rt] = rows_of(sm.Gam, rt, g) * QH[rt];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) O[0] = mma(ld_frag<T>(sm.pm, n, ks, g, kChunk), vf[ks], O[0]);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) O[1] = mma(ld_frag<T>(sm.pm, 32 + n, ks, g, kChunk), vf[ks], O[1]);
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
    const float GC = sm.scal[0];
    F ef[4];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        f32x16 ev = Vp[rt] * rows_of(sm.E, rt, g);
        ef[2 * rt] = acc_frag<T>(ev, 0);
        ef[2 * rt + 1] = acc_frag<T>(ev, 1);
    }
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
        f32x16 acc = Hs[ht] * GC;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc = mma(ld_frag<T>(sm.ktr, 32 * ht + n, ks, g, kChunk), ef[ks], acc);
        Hs[ht] = acc;
    }
    if (MODE == MODE_PASS1) {
        F mvf[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) mvf[ks] = acc_frag<T>(VpM[ks >> 1], ks & 1);
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) {
            f32x16 acc = Ms[ht];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) acc = mma(ld_frag<T>(sm.ktr, 32 * ht + n, ks, g, kChunk), mvf[ks], acc);
            Ms[ht] = acc;
        }
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

template <typename T, int MODE>
__device__ void run_task(const FwdParams& prm, Smem<T>& sm, const Task& tk) {
    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, n = lane & 31, g = lane >> 5;
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

    Stage<T> st;
    constexpr int NVR = VInLds<T>::value ? 1 : 32;
    float vcur[NVR], vnext[NVR];
    {
        const int c = tk.c_begin;
        const int t0 = c * kChunk;
        const int nvalid = prm.T - t0 < kChunk ? prm.T - t0 : kChunk;
        const bool need_q = MODE == MODE_FULL && c >= tk.c_out;
        load_stage<T>(prm, b, h, t0, nvalid, need_q, st);
        if constexpr (!VInLds<T>::value)
            load_v<T>((const T*)prm.v, b, h, prm.H, prm.T, t0, nvalid, 32 * w + n, g, vnext);
    }
    for (int c = tk.c_begin; c < tk.c_end; ++c) {
        const bool emit = MODE == MODE_FULL && c >= tk.c_out;
        __syncthreads();  // the previous chunk's state step is done with the tiles
        store_stage<T>(sm, st, emit, gsum);
        if constexpr (!VInLds<T>::value) {
#pragma unroll
            for (int i = 0; i < NVR; ++i) vcur[i] = vnext[i];
        }
        __syncthreads();
        if (c + 1 < tk.c_end) {
            const int t0 = (c + 1) * kChunk;
            const int nvalid = prm.T - t0 < kChunk ? prm.T - t0 : kChunk;
            const bool need_q = MODE == MODE_FULL && c + 1 >= tk.c_out;
            load_stage<T>(prm, b, h, t0, nvalid, need_q, st);
            if constexpr (!VInLds<T>::value)
                load_v<T>((const T*)prm.v, b, h, prm.H, prm.T, t0, nvalid, 32 * w + n, g, vnext);
        }
        chunk_step<T, MODE>(prm, sm, tk, b, h, c, emit, vcur, Hs, Ms);
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
    __shared__ __attribute__((aligned(16))) Smem<T> sm;
    Task tk;
    if (!decode_task(prm, PHASE, tk)) return;
    // only the first launch of a split forward has pass-1 tasks
    if (PHASE == PHASE_A && tk.mode == MODE_PASS1)
        run_task<T, MODE_PASS1>(prm, sm, tk);
    else
        run_task<T, MODE_FULL>(prm, sm, tk);
}

template <typename T>
hipError_t launch_fwd_t(const FwdParams& p, int phase, hipStream_t s) {
    dim3 block(256);
    if (phase == PHASE_SINGLE) {
        hipLaunchKernelGGL((gdn_fwd_kernel<T, PHASE_SINGLE>), dim3(p.B * p.H), block, 0, s, p);
    } else if (phase == PHASE_A) {
        hipLaunchKernelGGL((gdn_fwd_kernel<T, PHASE_A>), dim3(p.B * p.H * p.P), block, 0, s, p);
    } else {
        hipLaunchKernelGGL((gdn_fwd_kernel<T, PHASE_C>), dim3(p.B * p.H * (p.P - 1)), block, 0, s, p);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const FwdParams& p, int phase, bool bf16, hipStream_t s) {
    return bf16 ? launch_fwd_t<__bf16>(p, phase, s) : launch_fwd_t<float>(p, phase, s);
}

}  // namespace gdn
