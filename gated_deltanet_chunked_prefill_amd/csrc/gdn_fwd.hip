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
#include "gdn_chunk.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

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
    if (phase == PHASE_SINGLE || phase == PHASE_STATES) {
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

// The serial state step of one chunk for state wave w (its 32 state columns).
template <typename T, int MODE>
__device__ __forceinline__ void chunk_state(T* o, int Tn, int H, float scale, const Lane<T>& L, const T* kt,
                                            const T* qt, const T* vt, const T (*t32)[kT32],
                                            const float* gam_vec, const float* e_vec, float GC,
                                            int b, int h, int t0, int nvalid, bool emit,
                                            f32x16* Hs) {
    using F = typename FragOf<T>::type;
    const int n = L.n, g = L.g, w = L.w;
    f32x16 X[2];
    f32x16 OT[2] = {zero16(), zero16()};   // (Q H)^T: lane = position, registers = dv
    X[0] = zero16();
    X[1] = zero16();
    // software-pipelined: the LDS fragments of k-step ks+1 are requested before
    // the products of k-step ks are issued
    F ka[2], qa[2];
    ka[0] = L.f128(kt, 0, 0);
    ka[1] = L.f128(kt, 1, 0);
    if (MODE == MODE_FULL && emit) {
        qa[0] = L.f128(qt, 0, 0);
        qa[1] = L.f128(qt, 1, 0);
    }
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        F kn[2], qn[2];
        if (ks + 1 < 8) {
            kn[0] = L.f128(kt, 0, ks + 1);
            kn[1] = L.f128(kt, 1, ks + 1);
            if (MODE == MODE_FULL && emit) {
                qn[0] = L.f128(qt, 0, ks + 1);
                qn[1] = L.f128(qt, 1, ks + 1);
            }
        }
        // the state fragment of this k-step is converted right before use
        const F hf = acc_frag<T>(Hs[ks >> 1], ks & 1);
        X[0] = mma(ka[0], hf, X[0]);
        X[1] = mma(ka[1], hf, X[1]);
        if (MODE == MODE_FULL && emit) {
            OT[0] = mma(hf, qa[0], OT[0]);
            OT[1] = mma(hf, qa[1], OT[1]);
        }
        if (ks + 1 < 8) {
            ka[0] = kn[0];
            ka[1] = kn[1];
            if (MODE == MODE_FULL && emit) {
                qa[0] = qn[0];
                qa[1] = qn[1];
            }
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
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int pos = 32 * rt + n;
            if (pos < nvalid) {
                // global address space: plain vector stores, counted by vmcnt only
                typedef __attribute__((address_space(1))) t4 gt4;
                gt4* orow = (gt4*)(o + (((size_t)b * Tn + t0 + pos) * H + h) * kDv + 32 * w + 4 * g);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    t4 v;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = (T)(scale * OT[rt][4 * i + e]);
                    orow[2 * i] = v;
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
}

// Pass-1 segment transition, carried by the prep waves (prep wave w owns columns
// [32w, 32w+32) of the 128 x 128 product): Mt <- Mt - K^T T0 diag(beta) K Mt, i.e.
// the state step with V = 0 and no gates, through the gate-free blocks
// T0_00 diag(beta), T0_11 diag(beta) and -K_1 K_0^T.
template <typename T>
__device__ __forceinline__ void mt_step(const Lane<T>& L, const T* kt, const T (*t32)[kT32], f32x16* Ms) {
    using F = typename FragOf<T>::type;
    f32x16 X[2], Vp[2];
    k_times<T>(L, kt, Ms, X);
    const f32x16 y1 = -X[1];
    F ym0[2] = {acc_frag<T>(-X[0], 0), acc_frag<T>(-X[0], 1)};
    block_solve<T>(L, t32[3], t32[5], t32[4], ym0, y1, Vp);
    F vf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) vf[ks] = acc_frag<T>(Vp[ks >> 1], ks & 1);
    kt_update<T>(L, kt, Ms, 1.f, vf);
}

// State waves: load the entering state, run the serial step of every chunk,
// store the result.  Executes exactly the same barriers as prep_loop.
template <typename T, int MODE, bool KEEP>
__device__ __noinline__ void state_loop(const FwdParams& prm, Smem<T>& sm, const Task& tk) {
    constexpr bool kPipe = Pipe<T>::on;
    // every parameter read once, into scalar registers
    const int bh = uni(tk.bh), seg = uni(tk.seg), c_begin = uni(tk.c_begin), c_out = uni(tk.c_out);
    const int c_end = uni(tk.c_end), init = uni(tk.init), dst = uni(tk.dst);
    const int Tn = uni(prm.T), H = uni(prm.H), N = uni(prm.N), P = uni(prm.P);
    const float scale = uni(prm.scale);
    T* const o = uni((T*)prm.o);
    float* const hst = KEEP ? uni(prm.hstore) : nullptr;
    const int b = bh / H, h = bh % H;
    const size_t SS = (size_t)kDk * kDv;
    const int nch = c_end - c_begin;
    Lane<T> L;
    L.init(threadIdx.x);
    f32x16 Hs[4];
    if (init == INIT_H0) {
        load_state(uni(prm.h0) + (size_t)bh * SS, L.w, L.lane, Hs);
    } else if (init == INIT_HS) {
        load_state(uni(prm.hs) + ((size_t)bh * P + seg) * SS, L.w, L.lane, Hs);
    } else {
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) Hs[ht] = zero16();
    }
    const size_t hst_base = (size_t)bh * (N + 1);
    auto emit = [&](int c) { return MODE == MODE_FULL && o != nullptr && c >= c_out; };
    // the state entering every chunk this task owns (for the backward)
    auto keep = [&](int c) {
        if (KEEP && c >= c_out) store_state(hst + (hst_base + c) * SS, L.w, L.lane, Hs);
    };
    if constexpr (kPipe) {
        lds_barrier();
        lds_barrier();
        for (int i = 0; i < nch; ++i) {
            const int c = c_begin + i;
            const int slot = i % 3, vb = i & 1;
            keep(c);
            chunk_state<T, MODE>(o, Tn, H, scale, L, sm.kt[slot], sm.qt[slot], sm.vt[vb], sm.t32[vb],
                                 sm.gam_vec[vb], sm.e_vec[vb], sm.gc[vb][0], b, h, c * kChunk,
                                 chunk_len(Tn, c), emit(c), Hs);
            lds_barrier();
        }
    } else {
        for (int i = 0; i < nch; ++i) {
            const int c = c_begin + i;
            lds_barrier();
            lds_barrier();
            lds_barrier();
            keep(c);
            chunk_state<T, MODE>(o, Tn, H, scale, L, sm.kt[0], sm.qt[0], sm.vt[0], sm.t32[0],
                                 sm.gam_vec[0], sm.e_vec[0], sm.gc[0][0], b, h, c * kChunk,
                                 chunk_len(Tn, c), emit(c), Hs);
        }
    }
    if (KEEP && c_end == N) keep(N);
    if (dst == DST_HT) {
        store_state(uni(prm.ht) + (size_t)bh * SS, L.w, L.lane, Hs);
    } else if (dst == DST_HS_NEXT) {
        store_state(uni(prm.hs) + ((size_t)bh * P + seg + 1) * SS, L.w, L.lane, Hs);
    } else if (dst == DST_PASS1) {
        store_state(uni(prm.bz) + ((size_t)bh * P + seg) * SS, L.w, L.lane, Hs);
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
    const int pw = wave_id() - 4;
    // every parameter read once, into scalar registers
    const int bh = uni(tk.bh), seg = uni(tk.seg), c_begin = uni(tk.c_begin), c_out = uni(tk.c_out);
    const int c_end = uni(tk.c_end), dst = uni(tk.dst);
    const int Tn = uni(prm.T), H = uni(prm.H), P = uni(prm.P);
    const T* const kp = uni((const T*)prm.k);
    const T* const qp = uni((const T*)prm.q);
    const T* const vp = uni((const T*)prm.v);
    const float* const gp = uni(prm.g);
    const float* const bp = uni(prm.beta);
    const bool has_o = uni(prm.o) != nullptr;
    const int b = bh / H, h = bh % H;
    const int nch = c_end - c_begin;
    Lane<T> L;
    L.init(threadIdx.x);
    float gsum = 0.f;
    float g_cur = 0.f, b_cur = 0.f, g_nxt = 0.f, b_nxt = 0.f;
    f32x16 Ms[4];
    if (MODE == MODE_PASS1) {
#pragma unroll
        for (int ht = 0; ht < 4; ++ht)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                Ms[ht][r] = (32 * ht + rho(L.g, r) == 32 * L.w + L.n) ? 1.f : 0.f;
    }
    auto need_q = [&](int c) { return MODE == MODE_FULL && has_o && c >= c_out; };
    TileLoader<T> TL;
    TL.init(pw, L.lane, H);
    auto load_kq = [&](int c, int slot) {
        const size_t cb = chunk_base(b, h, Tn, H, c);
        const int nv = chunk_len(Tn, c);
        TL.load(sm.kt[slot], kp + cb, nv);
        if (need_q(c)) TL.load(sm.qt[slot], qp + cb, nv);
    };
    auto load_v = [&](int c, int slot) {
        TL.load(sm.vt[slot], vp + chunk_base(b, h, Tn, H, c), chunk_len(Tn, c));
    };
    auto load_gb = [&](int c, float& gv, float& bv) {
        load_gate_beta(gp, bp, Tn, H, b, h, c, L.lane, gv, bv);
    };
    if constexpr (kPipe) {
        // prologue: chunk 0 in LDS and prepped; chunk 1's K, Q in flight
        load_kq(c_begin, 0);
        load_v(c_begin, 0);
        if (nch > 1) load_kq(c_begin + 1, 1);
        load_gb(c_begin, g_cur, b_cur);
        if (nch > 1) load_gb(c_begin + 1, g_nxt, b_nxt);
        wait_vm();
        lds_barrier();
        chunk_prep<T, MODE>(sm, L, pw, sm.kt[0], sm.qt[0], sm.t32[0], sm.gam_vec[0], sm.e_vec[0],
                            sm.gc[0], g_cur, b_cur, need_q(c_begin), gsum);
        g_cur = g_nxt;
        b_cur = b_nxt;
        lds_barrier();
        for (int i = 0; i < nch; ++i) {
            const int c = c_begin + i;
            // this chunk's segment transition (its prep outputs are in buffer i & 1)
            if (MODE == MODE_PASS1) mt_step<T>(L, sm.kt[i % 3], sm.t32[i & 1], Ms);
            if (i + 1 < nch) {
                if (i + 2 < nch) {
                    load_kq(c + 2, (i + 2) % 3);
                    load_gb(c + 2, g_nxt, b_nxt);
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
            const int c = c_begin + i;
            lds_barrier();   // the previous chunk is done with the single buffers
            load_kq(c, 0);
            load_v(c, 0);
            load_gb(c, g_cur, b_cur);
            wait_vm();
            lds_barrier();
            chunk_prep<T, MODE>(sm, L, pw, sm.kt[0], sm.qt[0], sm.t32[0], sm.gam_vec[0], sm.e_vec[0],
                                sm.gc[0], g_cur, b_cur, need_q(c), gsum);
            lds_barrier();
            if (MODE == MODE_PASS1) mt_step<T>(L, sm.kt[0], sm.t32[0], Ms);
        }
    }
    if (dst == DST_PASS1) {
        store_state(uni(prm.mt) + ((size_t)bh * P + seg) * (size_t)(kDk * kDv), L.w, L.lane, Ms);
        if (pw == 3 && L.lane == 0) uni(prm.gsum)[(size_t)bh * P + seg] = gsum;
    }
}

template <typename T, int MODE, bool KEEP = false>
__device__ __forceinline__ void run_task(const FwdParams& prm, Smem<T>& sm, const Task& tk) {
    // the role branch must be wave-uniform to the compiler: both roles hold
    // s_barrier, and a branch it takes for divergent would be laid out so that a
    // wave also passes through the other role's barriers
    if (wave_id() < 4)
        state_loop<T, MODE, KEEP>(prm, sm, tk);
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
    else if (PHASE == PHASE_STATES)
        run_task<T, MODE_FULL, true>(prm, sm, tk);
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
    if (phase == PHASE_STATES) return launch_phase<T, PHASE_STATES>(p, p.B * p.H, s);
    if (phase == PHASE_A) return launch_phase<T, PHASE_A>(p, p.B * p.H * p.P, s);
    return launch_phase<T, PHASE_C>(p, p.B * p.H * (p.P - 1), s);
}

}  // namespace

hipError_t launch_fwd(const FwdParams& p, int phase, bool bf16, hipStream_t s) {
    return bf16 ? launch_fwd_t<__bf16>(p, phase, s) : launch_fwd_t<float>(p, phase, s);
}

}  // namespace gdn
