// Fused chunked forward of the gated delta rule for gfx950.
//
// One workgroup (eight wave64s, two per SIMD) runs one (batch, head, segment)
// task over a run of 64-token chunks.  The workgroup is split by role:
//   * four state waves: wave w owns dv columns [32w, 32w+32) of the 128x128
//     float32 state, which stays in MFMA accumulators for the whole task, and
//     runs the serial per-chunk state step;
//   * four prep waves: stream the next chunks' K, Q, V tiles from HBM straight
//     into LDS and compute the chunk-independent part of the next chunk (gate
//     scan, intra-chunk inverse, masked Q K^T) while the state waves work on the
//     current one.  A state wave and a prep wave share each SIMD, so the prep's
//     vector work overlaps the state step's matrix work.
// The state, W/U-type intermediates and the per-chunk inverse never reach HBM
// (FlashQLA talk summary, onedev.kr, paragraph 3 names the per-chunk steps and
// criticises writing W, U and S to HBM and reading them back; paragraph 7
// describes splitting loads and the V', O, S work over cooperating groups).
//
// Per chunk (gamma = in-chunk cumulative sum of g, Gamma = exp(gamma)), with
// 32-row blocks 0 and 1 of the chunk:
//   prep (paragraph 3 steps 1-2, paragraph 6):
//     A0 = diag(beta) strict_lower(K K^T); its diagonal blocks are inverted
//     gate-free, T0_pp = (I + A0_pp)^-1, by the product series
//     (I+M)(I+M^2)(I+M^4)(I+M^8)(I+M^16), M = -A0_pp (exact: M^32 = 0);
//     gates enter as the factor Gamma_r/Gamma_s = exp(gamma_r - gamma_C/2) *
//     exp(gamma_C/2 - gamma_s) (2C+1 exponentials: the diagonal scaling pulled
//     outside the inverse), giving Tt_pp = T_pp diag(beta) with
//     T_pp = diag(Gamma) T0_pp diag(1/Gamma), the gated off-diagonal block
//     Ah_10 = (Gamma_r/Gamma_s) K_1 K_0^T and P = (Q K^T) o Mask (s <= r).
//   state step (paragraph 3 steps 3-4, serial over chunks):
//     X = K H,  Y = V - diag(Gamma) X
//     V'_0 = Tt_00 Y_0,  V'_1 = Tt_11 (Y_1 - Ah_10 V'_0)   (block forward substitution
//                                                          of (I + A) V' = diag(beta) Y)
//     O = scale (diag(Gamma) Q H + P V')
//     H <- Gamma_C H + K^T diag(Gamma_C / Gamma) V'
// Pass-1 of the sequence split (paragraph 4) runs the same step from a zero
// state without Q or O and also carries the gate-free segment transition
//     Mt <- (I - K^T T0 diag(beta) K) Mt,
// i.e. the same step on 128 extra columns with V = 0 and no gates.
//
// K^T and V in accumulator layout are read from the row-major tiles with the
// transposing LDS read; O is produced transposed (O^T = H^T Q^T + V'^T P^T) so
// each lane holds a row of O and writes it as 8-byte segments.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

enum { MODE_FULL = 0, MODE_PASS1 = 1 };
enum { INIT_ZERO = 0, INIT_H0 = 1, INIT_HS = 2 };
enum { DST_NONE = 0, DST_HT = 1, DST_HS_NEXT = 2, DST_PASS1 = 3 };

constexpr int kThreads = 512;   // 4 state waves + 4 prep waves

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

// bf16 runs the prep one chunk ahead of the state step (K/Q triple-buffered,
// V and prep outputs double-buffered); the float32 build, used for small
// float32 workloads, runs prep and state step back to back in single buffers.
template <typename T> struct Pipe { static constexpr bool on = sizeof(T) == 2; };

// Prep outputs of one chunk, six 32x32 A-layout tiles:
//   0: Tt_00   1: Tt_11   2: -Ah_10 (gated)
//   3: P_00 | T0_00 diag(beta)   4: P_10 | -K_1 K_0^T   5: P_11 | T0_11 diag(beta)
// (full mode | pass-1 gate-free versions for the segment transition).
constexpr int kT32 = 32 * 32;

template <typename T>
struct Smem {
    static constexpr int NKQ = Pipe<T>::on ? 3 : 1;
    static constexpr int NV = Pipe<T>::on ? 2 : 1;
    static constexpr int NP = Pipe<T>::on ? 2 : 1;
    T kt[NKQ][kChunk * kDk];   // K, row-major [position][dk]
    T qt[NKQ][kChunk * kDk];   // Q
    T vt[NV][kChunk * kDv];    // V, row-major [position][dv]
    T t32[NP][6][kT32];        // prep outputs
    float gam_vec[NP][kChunk]; // Gamma_r for the state step
    float e_vec[NP][kChunk];   // Gamma_C / Gamma_r
    float gc[NP][4];           // [0] Gamma_C
    float pscr[4][4][kChunk];  // per prep wave: gamma, exp(gamma - gC/2), exp(gC/2 - gamma), beta
};

__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x3f70); }   // vmcnt(0)
__device__ __forceinline__ void wait_lgkm() { __builtin_amdgcn_s_waitcnt(0xc07f); } // lgkmcnt(0)

// Workgroup barrier that orders LDS only: outstanding global stores of the
// state waves are not waited for.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// threadIdx.x hidden from loop-invariant code motion (used by the generic
// float32 addressing, whose per-access address arithmetic must not be hoisted
// out of the chunk loop where it would occupy hundreds of registers).
__device__ __forceinline__ int opaque_tid() {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}

// Index of this thread's wave in the workgroup, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

typedef __attribute__((address_space(3))) char lds_t;
__device__ __forceinline__ const lds_t* as_lds(const void* p) { return (const lds_t*)p; }

template <typename V>
__device__ __forceinline__ V lds_ld(const void* base, uint32_t off) {
    return *(const __attribute__((address_space(3))) V*)(as_lds(base) + off);
}
template <typename V>
__device__ __forceinline__ void lds_st(void* base, uint32_t off, const V& v) {
    *(__attribute__((address_space(3))) V*)((lds_t*)as_lds(base) + off) = v;
}

// Per-lane LDS addressing.  For bf16 the swizzled byte offsets a lane needs are
// precomputed once per task into small tables, so every fragment read in the
// chunk loop is a table register plus an immediate offset:
//   * rows 32rt + n of a 64 x 128 tile: slot = (2ks + h) ^ 4rt ^ swz(n), whose
//     low three bits are (c' & 7) ^ swz(n) with c' = (2ks + h) ^ 4rt;
//   * transposing reads of a 64 x 128 tile: lane (i, q, g) of a 16-lane group
//     reads row 16ks + 8h + a (a = 4g + i/4) and column block 2q + (i/2)%2 of its
//     32-column window; the slot's low bits are that block ^ a ^ (2ks + h);
//   * rows n of a 32 x 32 tile: slot = (2ks + h) ^ swz4(n).
template <typename T>
struct Lane {
    int lane, n, g, w;
    uint32_t a128[8];   // bf16: n*256 + 8g + ((j ^ swz(n)) << 4)
    uint32_t a32[4];    // bf16: n*64 + 8g + ((j ^ swz4(n)) << 4)
    uint32_t trk[8];    // bf16: transposing-read offsets for column windows 32ht
    uint32_t trv[8];    // bf16: the same for this wave's V columns 32w

    __device__ void init(int tid) {
        lane = tid & 63;
        n = lane & 31;
        g = lane >> 5;
        w = (tid >> 6) & 3;
        if constexpr (sizeof(T) == 2) {
            const int s = swz(n), s4 = swz4(n);
#pragma unroll
            for (int j = 0; j < 8; ++j) a128[j] = n * 256 + 8 * g + ((j ^ s) << 4);
#pragma unroll
            for (int j = 0; j < 4; ++j) a32[j] = n * 64 + 8 * g + ((j ^ s4) << 4);
            const int i = lane & 15, q = (lane >> 4) & 1;
            const int a = 4 * g + (i >> 2);
            const int lam = (2 * q + ((i >> 1) & 1)) ^ a;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                trk[j] = a * 256 + 8 * (i & 1) + ((j ^ lam) << 4);
                trv[j] = a * 256 + 8 * (i & 1) + ((j ^ lam ^ (4 * (w & 1))) << 4) + 128 * (w >> 1);
            }
        }
    }

    // A fragment of rows 32rt + n of a 64 x 128 tile, contraction k-step ks.
    __device__ __forceinline__ typename FragOf<T>::type f128(const T* tile, int rt, int ks) const {
        if constexpr (sizeof(T) == 2) {
            typedef __bf16 b4 __attribute__((ext_vector_type(4)));
            const int c0 = (2 * ks) ^ (4 * rt), c1 = (2 * ks + 1) ^ (4 * rt);
            b4 lo = lds_ld<b4>(tile, a128[c0 & 7] + rt * 8192 + (c0 & 8) * 16);
            b4 hi = lds_ld<b4>(tile, a128[c1 & 7] + rt * 8192 + (c1 & 8) * 16);
            typename FragOf<T>::type f;
#pragma unroll
            for (int j = 0; j < 4; ++j) { f[j] = lo[j]; f[4 + j] = hi[j]; }
            return f;
        } else {
            const int nn = opaque_tid() & 31;
            return afrag<T, kDk>(tile, 32 * rt + nn, ks, g);
        }
    }
    // A fragment of rows n of a 32 x 32 tile, k-step ks (0 or 1).
    __device__ __forceinline__ typename FragOf<T>::type f32(const T* tile, int ks) const {
        if constexpr (sizeof(T) == 2) {
            typedef __bf16 b4 __attribute__((ext_vector_type(4)));
            b4 lo = lds_ld<b4>(tile, a32[2 * ks]);
            b4 hi = lds_ld<b4>(tile, a32[2 * ks + 1]);
            typename FragOf<T>::type f;
#pragma unroll
            for (int j = 0; j < 4; ++j) { f[j] = lo[j]; f[4 + j] = hi[j]; }
            return f;
        } else {
            const int nn = opaque_tid() & 31;
            return afrag<T, 32>(tile, nn, ks, g);
        }
    }
    __device__ __forceinline__ void st32(T* tile, int ks, const typename FragOf<T>::type& f) const {
        if constexpr (sizeof(T) == 2) {
            typedef __bf16 b4 __attribute__((ext_vector_type(4)));
            b4 lo, hi;
#pragma unroll
            for (int j = 0; j < 4; ++j) { lo[j] = f[j]; hi[j] = f[4 + j]; }
            lds_st<b4>(tile, a32[2 * ks], lo);
            lds_st<b4>(tile, a32[2 * ks + 1], hi);
        } else {
            const int nn = opaque_tid() & 31;
            st_afrag<T, 32>(tile, nn, ks, g, f);
        }
    }
    // Transposed fragment of a 64 x 128 tile: lane (m, g) gets
    // tile[kappa(ks, g, 0..7)][32*cb + m]; cb = column window (compile-time for
    // K, the wave's own window for V).
    __device__ __forceinline__ typename FragOf<T>::type tr(const T* tile, const uint32_t* tab, int cbhi,
                                                           int kappa_lo, int ks) const {
        if constexpr (sizeof(T) == 2) {
            typedef short s4 __attribute__((ext_vector_type(4)));
            typedef __bf16 b4 __attribute__((ext_vector_type(4)));
            typename FragOf<T>::type f;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int b = (2 * ks + h) & 7;
                const uint32_t off = tab[(kappa_lo ^ b) & 7] + (16 * ks + 8 * h) * 256 + 128 * cbhi;
                s4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s4*)(as_lds(tile) + off));
                b4 q = __builtin_bit_cast(b4, r);
#pragma unroll
                for (int j = 0; j < 4; ++j) f[4 * h + j] = q[j];
            }
            return f;
        } else {
            (void)tab; (void)cbhi; (void)kappa_lo;
            return typename FragOf<T>::type{};
        }
    }
    // K^T fragment for dk rows 32ht + m.
    __device__ __forceinline__ typename FragOf<T>::type trK(const T* tile, int ht, int ks) const {
        if constexpr (sizeof(T) == 2) {
            return tr(tile, trk, ht >> 1, 4 * (ht & 1), ks);
        } else {
            return tfrag<T, kDk>(tile, 32 * ht, ks, opaque_tid() & 63);
        }
    }
    // V fragment (accumulator layout) for this wave's dv columns.
    __device__ __forceinline__ typename FragOf<T>::type trV(const T* tile, int ks) const {
        if constexpr (sizeof(T) == 2) {
            return tr(tile, trv, 0, 0, ks);
        } else {
            return tfrag<T, kDv>(tile, 32 * w, ks, opaque_tid() & 63);
        }
    }
};

// Copy one 64 x 128 tile of chunk rows [t0, t0 + nvalid) of head (b, h) into a
// swizzled row-major LDS tile, spread over the 256 lanes of the prep waves
// (pl = 0..255).  Full chunks go HBM -> LDS directly (each lane's 16 bytes land
// at slot base + 16*lane, so the lane fetches the chunk that belongs there); a
// short last chunk goes through registers and is zero-filled.
template <typename T>
__device__ __forceinline__ void load_tile(T* tile, const T* src, int b, int h, int T_, int H, int t0,
                                          int nvalid, int pl) {
    constexpr int EPC = 16 / (int)sizeof(T);
    constexpr int CPR = kDk / EPC;                 // 16-byte chunks per row
    constexpr int ROUNDS = kChunk * CPR / 256;
    const int pw = pl >> 6, lane = pl & 63;
    const size_t rowstride = (size_t)H * kDk;
    const T* base = src + (((size_t)b * T_ + t0) * H + h) * kDk;
    if (nvalid == kChunk) {
#pragma unroll
        for (int i = 0; i < ROUNDS; ++i) {
            const int L = (i * 4 + pw) * 64 + lane;     // slot index in the tile
            const int row = L / CPR, slot = L % CPR;
            const int c = slot ^ swz(row);
            const T* gp = base + row * rowstride + c * EPC;
            T* lbase = tile + (i * 4 + pw) * 64 * EPC;
            __builtin_amdgcn_global_load_lds((const void*)gp,
                                             (__attribute__((address_space(3))) void*)lbase, 16, 0, 0);
        }
    } else {
        typedef uint32_t u4 __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int i = 0; i < ROUNDS; ++i) {
            const int L = (i * 4 + pw) * 64 + lane;
            const int row = L / CPR, slot = L % CPR;
            const int c = slot ^ swz(row);
            u4 v = {0u, 0u, 0u, 0u};
            if (row < nvalid) v = *(const u4*)(base + row * rowstride + c * EPC);
            *(u4*)(tile + L * EPC) = v;
        }
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

// 32x32 product of two accumulator-form operands: returns c + X Y given
// xt = acc(X^T) (its fragments are the A fragments of X) and y = acc(Y).
template <typename T>
__device__ __forceinline__ f32x16 mm_acc(const f32x16& xt, const f32x16& y, f32x16 c) {
    c = mma(acc_frag<T>(xt, 0), acc_frag<T>(y, 0), c);
    c = mma(acc_frag<T>(xt, 1), acc_frag<T>(y, 1), c);
    return c;
}

// Inverse of (I + Nd) for one 32x32 diagonal block, Nd = diag(beta) strict_lower(S),
// from S = K_p K_p^T (acc form).  Returns acc(T0_pp^T) in zt.
template <typename T>
__device__ __forceinline__ f32x16 diag_inverse_t(const f32x16& S, const f32x16& beta_rows,
                                                 float beta_n, int n, int g) {
    f32x16 m, mt, z, zt;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        int row = rho(g, r);
        m[r] = (n < row) ? -beta_rows[r] * S[r] : 0.f;   // M = -Nd
        mt[r] = (row < n) ? -beta_n * S[r] : 0.f;        // M^T (S is symmetric)
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
        f32x16 zn = (it < 3) ? mm_acc<T>(zt, m, z) : z;   // Z is only needed transposed at the end
        f32x16 ztn = mm_acc<T>(m, zt, zt);         // Z^T (I + M^(2^(it+1)))^T
        z = zn;
        zt = ztn;
    }
    return zt;
}

// Gate factor Gamma_r / Gamma_s for lane row r and accumulator-row columns s:
// fr is the row value (gamma_r or exp(gamma_r - gC/2)), fc the column values.
__device__ __forceinline__ float gate_factor(float fr, float fc, bool pairwise) {
    return pairwise ? __expf(fr - fc) : fr * fc;
}

// Diagonal block p of the chunk: S = K_p K_p^T, T0_pp by the series, then the
// gated Tt_pp (and the gate-free T0_pp diag(beta) in pass-1).  p is a template
// parameter so that every per-lane address-table index is a compile-time constant.
template <typename T, int MODE, int p>
__device__ __forceinline__ void diag_block(const Lane<T>& L, const T* kt, T (*t32)[kT32],
                                           const float* s_row, const float* s_col,
                                           const float* s_beta, bool pairwise) {
    using F = typename FragOf<T>::type;
    const int n = L.n, g = L.g;
    f32x16 S = zero16();
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        F kf = L.f128(kt, p, ks);
        S = mma(kf, kf, S);
    }
    const f32x16 brow = rows_of(s_beta, p, g);
    f32x16 zt = diag_inverse_t<T>(S, brow, s_beta[32 * p + n], n, g);
    // acc(T0^T): lane n holds row 32p+n of T0_pp, registers = columns 32p + rho
    const float fr = s_row[32 * p + n];
    const f32x16 fc = rows_of(s_col, p, g);
#pragma unroll
    for (int ksl = 0; ksl < 2; ++ksl) {
        F f, f0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int r = 8 * ksl + j;
            const float t0v = zt[r] * brow[r];
            f[j] = (T)(rho(g, r) <= n ? t0v * gate_factor(fr, fc[r], pairwise) : 0.f);
            f0[j] = (T)t0v;
        }
        L.st32(t32[p], ksl, f);
        if (MODE == MODE_PASS1) L.st32(t32[p == 0 ? 3 : 5], ksl, f0);
    }
}

// Chunk-independent prep of one chunk by prep wave pw.
template <typename T, int MODE>
__device__ __forceinline__ void chunk_prep(Smem<T>& sm, const Lane<T>& L, int pw, const T* kt,
                                           const T* qt, T (*t32)[kT32], float* gam_vec,
                                           float* e_vec, float* gc, float gv, float bv, bool emit,
                                           float& gsum) {
    using F = typename FragOf<T>::type;
    const int lane = L.lane, n = L.n, g = L.g;
    float* scr = &sm.pscr[pw][0][0];
    // in-chunk scan and the 2C+1 exponentials of the factored gate (paragraph 6),
    // re-centred at gamma_C/2 so both factors stay within exp(|gamma_C|/2); chunks
    // whose decay exceeds that safe range use pairwise exponentials.
    const float gam = wave_inclusive_scan(gv);
    const float gC = __builtin_bit_cast(
        float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, __shfl(gam, 63, 64))));  // wave-uniform
    const float half = 0.5f * gC;
    const bool pairwise = gC < -160.f;
    const float gp = __expf(gam - half);
    const float gn = __expf(half - gam);
    const float eh = __expf(half);
    scr[0 * kChunk + lane] = gam;
    scr[1 * kChunk + lane] = gp;
    scr[2 * kChunk + lane] = gn;
    scr[3 * kChunk + lane] = bv;
    if (pw == 3) {
        gam_vec[lane] = pairwise ? __expf(gam) : gp * eh;
        e_vec[lane] = pairwise ? __expf(gC - gam) : gn * eh;
        if (lane == 0) gc[0] = pairwise ? __expf(gC) : eh * eh;
        gsum += gC;
    }
    wait_lgkm();
    const float* s_row = scr + (pairwise ? 0 : 1) * kChunk;   // gamma or exp(gamma - gC/2)
    const float* s_col = scr + (pairwise ? 0 : 2) * kChunk;   // gamma or exp(gC/2 - gamma)
    const float* s_beta = scr + 3 * kChunk;

    if (pw == 0) {
        diag_block<T, MODE, 0>(L, kt, t32, s_row, s_col, s_beta, pairwise);
    } else if (pw == 1) {
        diag_block<T, MODE, 1>(L, kt, t32, s_row, s_col, s_beta, pairwise);
    } else if (pw == 2) {
        // off-diagonal block: acc(K_0 K_1^T) has lane n = row 32+n, registers = columns rho
        f32x16 x = zero16();
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) x = mma(L.f128(kt, 0, ks), L.f128(kt, 1, ks), x);
        const float fr = s_row[32 + n];
        const f32x16 fc = rows_of(s_col, 0, g);
#pragma unroll
        for (int ksl = 0; ksl < 2; ++ksl) {
            F f, f0;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int r = 8 * ksl + j;
                f[j] = (T)(-x[r] * gate_factor(fr, fc[r], pairwise));
                f0[j] = (T)(-x[r]);
            }
            L.st32(t32[2], ksl, f);
            if (MODE == MODE_PASS1) L.st32(t32[4], ksl, f0);
        }
        if (MODE == MODE_FULL && emit) {
            // P_10: acc(K_0 Q_1^T), lane n = row 32+n
            f32x16 y = zero16();
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) y = mma(L.f128(kt, 0, ks), L.f128(qt, 1, ks), y);
#pragma unroll
            for (int ksl = 0; ksl < 2; ++ksl) {
                F f;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int r = 8 * ksl + j;
                    f[j] = (T)(y[r] * gate_factor(fr, fc[r], pairwise));
                }
                L.st32(t32[4], ksl, f);
            }
        }
    } else if (MODE == MODE_FULL && emit) {
        // P_00 and P_11 (s <= r): acc(K_j Q_j^T), lane n = row 32j+n
#pragma unroll
        for (int j2 = 0; j2 < 2; ++j2) {
            f32x16 y = zero16();
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) y = mma(L.f128(kt, j2, ks), L.f128(qt, j2, ks), y);
            const float fr = s_row[32 * j2 + n];
            const f32x16 fc = rows_of(s_col, j2, g);
#pragma unroll
            for (int ksl = 0; ksl < 2; ++ksl) {
                F f;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int r = 8 * ksl + j;
                    f[j] = (T)(rho(g, r) <= n ? y[r] * gate_factor(fr, fc[r], pairwise) : 0.f);
                }
                L.st32(t32[j2 == 0 ? 3 : 5], ksl, f);
            }
        }
    }
}

// X = K Hm for the two 32-row position tiles (Hm: the four dk tiles of a state).
template <typename T>
__device__ __forceinline__ void k_times(const Lane<T>& L, const T* kt, const f32x16* Hm, f32x16* X) {
    X[0] = zero16();
    X[1] = zero16();
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        const typename FragOf<T>::type hf = acc_frag<T>(Hm[ks >> 1], ks & 1);
        X[0] = mma(L.f128(kt, 0, ks), hf, X[0]);
        X[1] = mma(L.f128(kt, 1, ks), hf, X[1]);
    }
}

// V'_0 = Tt_00 Y_0, V'_1 = Tt_11 (Y_1 - Ah_10 V'_0): y0f = fragments of Y_0,
// y1 = Y_1 in accumulator form; tiles t_00, t_11 and -Ah_10.
template <typename T>
__device__ __forceinline__ void block_solve(const Lane<T>& L, const T* t00, const T* t11,
                                            const T* na10, const typename FragOf<T>::type* y0f,
                                            const f32x16& y1, f32x16* Vp) {
    Vp[0] = zero16();
    Vp[0] = mma(L.f32(t00, 0), y0f[0], Vp[0]);
    Vp[0] = mma(L.f32(t00, 1), y0f[1], Vp[0]);
    f32x16 z1 = y1;
    z1 = mma(L.f32(na10, 0), acc_frag<T>(Vp[0], 0), z1);
    z1 = mma(L.f32(na10, 1), acc_frag<T>(Vp[0], 1), z1);
    Vp[1] = zero16();
    Vp[1] = mma(L.f32(t11, 0), acc_frag<T>(z1, 0), Vp[1]);
    Vp[1] = mma(L.f32(t11, 1), acc_frag<T>(z1, 1), Vp[1]);
}

// Hm <- a Hm + K^T B, B given as four fragments over the chunk positions.
template <typename T>
__device__ __forceinline__ void kt_update(const Lane<T>& L, const T* kt, f32x16* Hm, float a,
                                          const typename FragOf<T>::type* bf) {
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
        f32x16 acc = Hm[ht] * a;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc = mma(L.trK(kt, ht, ks), bf[ks], acc);
        Hm[ht] = acc;
    }
}

// The serial state step of one chunk for state wave w (its 32 state columns).
template <typename T, int MODE>
__device__ __forceinline__ void chunk_state(const FwdParams& prm, const Lane<T>& L, const T* kt,
                                            const T* qt, const T* vt, const T (*t32)[kT32],
                                            const float* gam_vec, const float* e_vec, float GC,
                                            int b, int h, int t0, int nvalid, bool emit,
                                            f32x16* Hs, f32x16* Ms) {
    using F = typename FragOf<T>::type;
    const int n = L.n, g = L.g, w = L.w;
    f32x16 X[2];
    f32x16 OT[2] = {zero16(), zero16()};   // (Q H)^T: lane = position, registers = dv
    X[0] = zero16();
    X[1] = zero16();
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        // the state fragment of this k-step is converted right before use (keeps
        // one fragment live instead of eight)
        const F hf = acc_frag<T>(Hs[ks >> 1], ks & 1);
        X[0] = mma(L.f128(kt, 0, ks), hf, X[0]);
        X[1] = mma(L.f128(kt, 1, ks), hf, X[1]);
        if (MODE == MODE_FULL && emit) {
            OT[0] = mma(hf, L.f128(qt, 0, ks), OT[0]);
            OT[1] = mma(hf, L.f128(qt, 1, ks), OT[1]);
        }
    }
    // Y = V - diag(Gamma) X (V in accumulator layout via the transposing read)
    f32x16 Y[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        F v0 = L.trV(vt, 2 * rt), v1 = L.trV(vt, 2 * rt + 1);
        f32x16 gr = rows_of(gam_vec, rt, g);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            Y[rt][j] = (float)v0[j] - gr[j] * X[rt][j];
            Y[rt][8 + j] = (float)v1[j] - gr[8 + j] * X[rt][8 + j];
        }
    }
    F y0f[2] = {acc_frag<T>(Y[0], 0), acc_frag<T>(Y[0], 1)};
    f32x16 Vp[2];
    block_solve<T>(L, t32[0], t32[1], t32[2], y0f, Y[1], Vp);
    F vf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) vf[ks] = acc_frag<T>(Vp[ks >> 1], ks & 1);

    if (MODE == MODE_FULL && emit) {
        // O^T = diag-scaled (Q H)^T + V'^T P^T; P^T's B fragments are rows of P
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) OT[rt] = OT[rt] * gam_vec[32 * rt + n];
        OT[0] = mma(vf[0], L.f32(t32[3], 0), OT[0]);
        OT[0] = mma(vf[1], L.f32(t32[3], 1), OT[0]);
        OT[1] = mma(vf[0], L.f32(t32[4], 0), OT[1]);
        OT[1] = mma(vf[1], L.f32(t32[4], 1), OT[1]);
        OT[1] = mma(vf[2], L.f32(t32[5], 0), OT[1]);
        OT[1] = mma(vf[3], L.f32(t32[5], 1), OT[1]);
        typedef T t4 __attribute__((ext_vector_type(4)));
        T* o = (T*)prm.o;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int pos = 32 * rt + n;
            if (pos < nvalid) {
                T* orow = o + (((size_t)b * prm.T + t0 + pos) * prm.H + h) * kDv + 32 * w + 4 * g;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    t4 v;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = (T)(prm.scale * OT[rt][4 * i + e]);
                    *(t4*)(orow + 8 * i) = v;
                }
            }
        }
    }
    // H <- Gamma_C H + K^T diag(E) V'
    F ef[4];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        f32x16 ev = Vp[rt] * rows_of(e_vec, rt, g);
        ef[2 * rt] = acc_frag<T>(ev, 0);
        ef[2 * rt + 1] = acc_frag<T>(ev, 1);
    }
    kt_update<T>(L, kt, Hs, GC, ef);

    if (MODE == MODE_PASS1) {
        // Mt <- Mt - K^T T0 diag(beta) K Mt  (V = 0, no gates)
        k_times<T>(L, kt, Ms, X);
        const f32x16 y1 = -X[1];
        F ym0[2] = {acc_frag<T>(-X[0], 0), acc_frag<T>(-X[0], 1)};
        block_solve<T>(L, t32[3], t32[5], t32[4], ym0, y1, Vp);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) vf[ks] = acc_frag<T>(Vp[ks >> 1], ks & 1);
        kt_update<T>(L, kt, Ms, 1.f, vf);
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

__device__ __forceinline__ int nvalid_of(const FwdParams& prm, int c) {
    return prm.T - c * kChunk < kChunk ? prm.T - c * kChunk : kChunk;
}

// g (into gv) and beta (into bv) of chunk c at position = lane.
__device__ __forceinline__ void load_gb(const FwdParams& prm, int b, int h, int c, int lane, float& gv,
                                        float& bv) {
    gv = 0.f;
    bv = 0.f;
    if (lane < nvalid_of(prm, c)) {
        const size_t go = ((size_t)b * prm.T + c * kChunk + lane) * prm.H + h;
        gv = prm.g[go];
        bv = prm.beta[go];
    }
}

// State waves: load the entering state, run the serial step of every chunk,
// store the result.  Executes exactly the same barriers as prep_loop.
template <typename T, int MODE>
__device__ __noinline__ void state_loop(const FwdParams& prm, Smem<T>& sm, const Task& tk) {
    constexpr bool kPipe = Pipe<T>::on;
    const int b = tk.bh / prm.H, h = tk.bh % prm.H;
    const size_t SS = (size_t)kDk * kDv;
    const int nch = tk.c_end - tk.c_begin;
    Lane<T> L;
    L.init(threadIdx.x);
    f32x16 Hs[4], Ms[4];
    if (tk.init == INIT_H0) {
        load_state(prm.h0 + (size_t)tk.bh * SS, L.w, L.lane, Hs);
    } else if (tk.init == INIT_HS) {
        load_state(prm.hs + ((size_t)tk.bh * prm.P + tk.seg) * SS, L.w, L.lane, Hs);
    } else {
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) Hs[ht] = zero16();
    }
    if (MODE == MODE_PASS1) {
#pragma unroll
        for (int ht = 0; ht < 4; ++ht)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                Ms[ht][r] = (32 * ht + rho(L.g, r) == 32 * L.w + L.n) ? 1.f : 0.f;
    }
    auto emit = [&](int c) { return MODE == MODE_FULL && c >= tk.c_out; };
    if constexpr (kPipe) {
        lds_barrier();
        lds_barrier();
        for (int i = 0; i < nch; ++i) {
            const int c = tk.c_begin + i;
            const int slot = i % 3, vb = i & 1;
            chunk_state<T, MODE>(prm, L, sm.kt[slot], sm.qt[slot], sm.vt[vb], sm.t32[vb],
                                 sm.gam_vec[vb], sm.e_vec[vb], sm.gc[vb][0], b, h, c * kChunk,
                                 nvalid_of(prm, c), emit(c), Hs, Ms);
            lds_barrier();
        }
    } else {
        for (int i = 0; i < nch; ++i) {
            const int c = tk.c_begin + i;
            lds_barrier();
            lds_barrier();
            lds_barrier();
            chunk_state<T, MODE>(prm, L, sm.kt[0], sm.qt[0], sm.vt[0], sm.t32[0], sm.gam_vec[0],
                                 sm.e_vec[0], sm.gc[0][0], b, h, c * kChunk, nvalid_of(prm, c),
                                 emit(c), Hs, Ms);
        }
    }
    if (tk.dst == DST_HT) {
        store_state(prm.ht + (size_t)tk.bh * SS, L.w, L.lane, Hs);
    } else if (tk.dst == DST_HS_NEXT) {
        store_state(prm.hs + ((size_t)tk.bh * prm.P + tk.seg + 1) * SS, L.w, L.lane, Hs);
    } else if (tk.dst == DST_PASS1) {
        const size_t o = ((size_t)tk.bh * prm.P + tk.seg) * SS;
        store_state(prm.bz + o, L.w, L.lane, Hs);
        store_state(prm.mt + o, L.w, L.lane, Ms);
    }
}

// Prep waves: stream tiles into LDS and prep each chunk one step ahead of the
// state waves.  Executes exactly the same barriers as state_loop.
// Both role loops stay out of line: with this function inlined into the
// single-launch kernel the hipcc (ROCm 7.2) build produced wrong outputs, while
// the out-of-line build matches the reference on every tested shape.
template <typename T, int MODE>
__device__ __noinline__ void prep_loop(const FwdParams& prm, Smem<T>& sm, const Task& tk) {
    constexpr bool kPipe = Pipe<T>::on;
    const int pl = threadIdx.x & 255;     // lane index within the prep group
    const int pw = wave_id() - 4;
    const int b = tk.bh / prm.H, h = tk.bh % prm.H;
    const int nch = tk.c_end - tk.c_begin;
    Lane<T> L;
    L.init(threadIdx.x);
    float gsum = 0.f;
    float g_cur = 0.f, b_cur = 0.f, g_nxt = 0.f, b_nxt = 0.f;
    auto need_q = [&](int c) { return MODE == MODE_FULL && c >= tk.c_out; };
    auto load_kq = [&](int c, int slot) {
        const int t0 = c * kChunk, nv = nvalid_of(prm, c);
        load_tile<T>(sm.kt[slot], (const T*)prm.k, b, h, prm.T, prm.H, t0, nv, pl);
        if (need_q(c)) load_tile<T>(sm.qt[slot], (const T*)prm.q, b, h, prm.T, prm.H, t0, nv, pl);
    };
    auto load_v = [&](int c, int slot) {
        load_tile<T>(sm.vt[slot], (const T*)prm.v, b, h, prm.T, prm.H, c * kChunk, nvalid_of(prm, c), pl);
    };
    if constexpr (kPipe) {
        // prologue: chunk 0 in LDS and prepped; chunk 1's K, Q in flight
        load_kq(tk.c_begin, 0);
        load_v(tk.c_begin, 0);
        if (nch > 1) load_kq(tk.c_begin + 1, 1);
        load_gb(prm, b, h, tk.c_begin, L.lane, g_cur, b_cur);
        if (nch > 1) load_gb(prm, b, h, tk.c_begin + 1, L.lane, g_nxt, b_nxt);
        wait_vm();
        lds_barrier();
        chunk_prep<T, MODE>(sm, L, pw, sm.kt[0], sm.qt[0], sm.t32[0], sm.gam_vec[0], sm.e_vec[0],
                            sm.gc[0], g_cur, b_cur, need_q(tk.c_begin), gsum);
        g_cur = g_nxt;
        b_cur = b_nxt;
        lds_barrier();
        for (int i = 0; i < nch; ++i) {
            const int c = tk.c_begin + i;
            if (i + 1 < nch) {
                if (i + 2 < nch) {
                    load_kq(c + 2, (i + 2) % 3);
                    load_gb(prm, b, h, c + 2, L.lane, g_nxt, b_nxt);
                }
                load_v(c + 1, (i + 1) & 1);
                const int slot = (i + 1) % 3, pb = (i + 1) & 1;
                chunk_prep<T, MODE>(sm, L, pw, sm.kt[slot], sm.qt[slot], sm.t32[pb], sm.gam_vec[pb],
                                    sm.e_vec[pb], sm.gc[pb], g_cur, b_cur, need_q(c + 1), gsum);
                g_cur = g_nxt;
                b_cur = b_nxt;
                wait_vm();
            }
            lds_barrier();
        }
    } else {
        for (int i = 0; i < nch; ++i) {
            const int c = tk.c_begin + i;
            lds_barrier();   // the previous chunk is done with the single buffers
            load_kq(c, 0);
            load_v(c, 0);
            load_gb(prm, b, h, c, L.lane, g_cur, b_cur);
            wait_vm();
            lds_barrier();
            chunk_prep<T, MODE>(sm, L, pw, sm.kt[0], sm.qt[0], sm.t32[0], sm.gam_vec[0], sm.e_vec[0],
                                sm.gc[0], g_cur, b_cur, need_q(c), gsum);
            lds_barrier();
        }
    }
    if (tk.dst == DST_PASS1 && pw == 3 && L.lane == 0) prm.gsum[(size_t)tk.bh * prm.P + tk.seg] = gsum;
}

template <typename T, int MODE>
__device__ __forceinline__ void run_task(const FwdParams& prm, Smem<T>& sm, const Task& tk) {
    // the role branch must be wave-uniform to the compiler: both roles hold
    // s_barrier, and a branch it takes for divergent would be laid out so that a
    // wave also passes through the other role's barriers
    if (wave_id() < 4)
        state_loop<T, MODE>(prm, sm, tk);
    else
        prep_loop<T, MODE>(prm, sm, tk);
}

template <typename T, int PHASE>
__global__ __launch_bounds__(kThreads, 1) void gdn_fwd_kernel(FwdParams prm) {
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
    hipLaunchKernelGGL((gdn_fwd_kernel<T, PHASE>), dim3(grid), dim3(kThreads), lds, s, p);
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
