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
// Split forward as a work queue.  A one-workgroup plan kernel reads the gate
// flags, chooses the segment counts of exact and window heads from a cost
// model and writes the job list; persistent workgroups (one per CU) then take
// jobs from an atomic counter.  Per exact head with P segments the jobs are
//   seg 0     full run from h0, publishes the state entering segment 1;
//   seg p     (0 < p < P-1) pass-1 from zero, then the composition
//             hs[p+1] = exp(G_p) Mt_p hs[p] + b_p once hs[p] is published, then
//             the full run of segment p from hs[p];
//   seg P-1   full run from hs[P-1] (waits for it), writes ht;
// window heads (paragraph 5) get independent jobs that warm up over the w
// chunks before their segment.  The list is ordered so that every job waits
// only for jobs handed out before it (seg 0 jobs, middle segments in
// increasing p, window jobs, last segments), so the waits end for any number
// of resident workgroups.  A state crosses workgroups through HBM with an
// agent-scope release by each producing wave and an acquire by the consumer.
//
// K^T and V in accumulator layout are read from the row-major tiles with the
// transposing LDS read; O is produced transposed (O^T = H^T Q^T + V'^T P^T) so
// each lane holds a row of O and writes it as 8-byte segments.
#include "gdn_chunk.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

enum { INIT_ZERO = 0, INIT_H0 = 1, INIT_HS = 2, INIT_HS_WAIT = 3 };
enum { DST_NONE = 0, DST_HT = 1, DST_HS_NEXT = 2, DST_COMPOSE = 3 };

constexpr int kThreads = 512;   // 4 state waves + 4 prep waves
constexpr int kMtStride = kDk + 4;   // float row stride of a segment transition staged in LDS
constexpr int kSpinLimit = 1 << 22;  // polls of about 1 us: seconds, far beyond any real wait

struct Task {
    int bh, seg;
    int c_begin, c_out, c_end;
    int mode, init, dst;
};

// The unsplit launches: workgroup = head, the whole sequence.
__device__ void whole_head_task(const FwdParams& prm, Task& t) {
    t.bh = blockIdx.x;
    t.seg = 0;
    t.c_begin = 0;
    t.c_out = 0;
    t.c_end = prm.N;
    t.mode = MODE_FULL;
    t.init = prm.h0 ? INIT_H0 : INIT_ZERO;
    t.dst = prm.ht ? DST_HT : DST_NONE;
}

// Make this wave's global stores visible device-wide, then count the wave in.
__device__ __forceinline__ void publish(int* cnt) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until `target` waves have published (bounded: on running out the plan's
// error flag is raised and the wait ends).
__device__ __forceinline__ void wait_published(const int* cnt, int target, int* error) {
    for (int spin = 0;; ++spin) {
        const int v = __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (uni(v) >= target) break;
        if (spin >= kSpinLimit) {
            if ((threadIdx.x & 63) == 0) __hip_atomic_store(error, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
        __builtin_amdgcn_s_sleep(8);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// acc += a b for float operands: exact float32 products in the float32 build;
// in the bf16 build three bf16 products of the hi/lo split (a_hi b_hi + a_hi b_lo
// + a_lo b_hi), close to float32 accuracy.
template <typename T>
__device__ __forceinline__ f32x16 mma_f32(const f32x8& a, const f32x8& b, f32x16 acc) {
    if constexpr (sizeof(T) == 4) {
        return mma(a, b, acc);
    } else {
        bf16x8 ah, al, bh, bl;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            ah[j] = (__bf16)a[j];
            al[j] = (__bf16)(a[j] - (float)ah[j]);
            bh[j] = (__bf16)b[j];
            bl[j] = (__bf16)(b[j] - (float)bh[j]);
        }
        acc = mma(ah, bh, acc);
        acc = mma(ah, bl, acc);
        return mma(al, bh, acc);
    }
}

// State wave w's 32 columns of the state entering the next segment (talk
// summary, paragraph 4: a segment maps its entering state H to
// exp(G) Mt H + b, with Mt gate-free and b the segment's run from zero):
//     out = eG * Mt * hin + bz,
// Mt row-major float in LDS (row stride kMtStride), hin and out in HBM, bz in
// accumulator layout.
template <typename T>
__device__ __forceinline__ void compose_next(const float* mtl, float eG, const float* hin, float* out,
                                             int w, int lane, const f32x16* bz) {
    const int n = lane & 31, g = lane >> 5;
    f32x16 hp[4];
    load_state(hin, w, lane, hp);
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
        f32x16 acc = zero16();
        const float* row = mtl + (32 * ht + n) * kMtStride + 4 * g;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const f32x4 lo = *reinterpret_cast<const f32x4*>(row + 16 * ks);
            const f32x4 hi = *reinterpret_cast<const f32x4*>(row + 16 * ks + 8);
            f32x8 a, b;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                a[j] = lo[j];
                a[4 + j] = hi[j];
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) b[j] = hp[ks >> 1][8 * (ks & 1) + j];
            acc = mma_f32<T>(a, b, acc);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r)
            out[(32 * ht + rho(g, r)) * kDv + 32 * w + n] = eG * acc[r] + bz[ht][r];
    }
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
    const size_t slot = (size_t)bh * P + seg;   // this segment's state slot
    if (init == INIT_H0) {
        load_state(uni(prm.h0) + (size_t)bh * SS, L.w, L.lane, Hs);
    } else if (init == INIT_HS || init == INIT_HS_WAIT) {
        if (init == INIT_HS_WAIT) wait_published(uni(prm.hs_cnt) + slot, 4, &uni(prm.plan)->error);
        load_state(uni(prm.hs) + slot * SS, L.w, L.lane, Hs);
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
        store_state(uni(prm.hs) + (slot + 1) * SS, L.w, L.lane, Hs);
        publish(uni(prm.hs_cnt) + slot + 1);
    } else if (dst == DST_COMPOSE) {
        // Hs is this segment's run from zero; the prep waves stage Mt and exp(G)
        lds_barrier();   // done with the chunk tiles
        lds_barrier();   // Mt in LDS
        wait_published(uni(prm.hs_cnt) + slot, 4, &uni(prm.plan)->error);
        float* const hs = uni(prm.hs);
        compose_next<T>(reinterpret_cast<const float*>(&sm.kt[0][0]), sm.fslot[0], hs + slot * SS,
                        hs + (slot + 1) * SS, L.w, L.lane, Hs);
        publish(uni(prm.hs_cnt) + slot + 1);
        lds_barrier();   // Mt no longer needed
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
    const int bh = uni(tk.bh), c_begin = uni(tk.c_begin), c_out = uni(tk.c_out);
    const int c_end = uni(tk.c_end), dst = uni(tk.dst);
    const int Tn = uni(prm.T), H = uni(prm.H);
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
    if (dst == DST_COMPOSE) {
        lds_barrier();   // the state waves are done with the chunk tiles
        float* const mtl = reinterpret_cast<float*>(&sm.kt[0][0]);
#pragma unroll
        for (int ht = 0; ht < 4; ++ht)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                mtl[(32 * ht + rho(L.g, r)) * kMtStride + 32 * L.w + L.n] = Ms[ht][r];
        if (pw == 3 && L.lane == 0) sm.fslot[0] = __expf(gsum);
        lds_barrier();   // Mt in LDS
        lds_barrier();   // the state waves have composed
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
    whole_head_task(prm, tk);
    if (PHASE == PHASE_STATES)
        run_task<T, MODE_FULL, true>(prm, sm, tk);
    else
        run_task<T, MODE_FULL>(prm, sm, tk);
}

// Persistent workgroups of the split forward: take jobs until the list is empty.
template <typename T>
__global__ __launch_bounds__(kThreads, 1) void gdn_fwd_queue_kernel(FwdParams prm) {
    extern __shared__ __attribute__((aligned(16))) char smem_raw[];
    Smem<T>& sm = *reinterpret_cast<Smem<T>*>(smem_raw);
    const int n_jobs = uni(prm.plan->n_jobs);
    for (;;) {
        if (threadIdx.x == 0) sm.islot[0] = atomicAdd(&prm.plan->next, 1);
        __syncthreads();
        const int j = uni(sm.islot[0]);
        __syncthreads();
        if (j >= n_jobs) break;
        const TaskRec rec = prm.jobs[j];
        Task tk{rec.bh, rec.seg, rec.c_begin, rec.c_out, rec.c_end, rec.mode, rec.init, rec.dst};
        if (tk.mode == MODE_PASS1) {
            // middle segment of an exact head: pass-1 and composition, then the
            // segment's outputs from its true entering state
            run_task<T, MODE_PASS1>(prm, sm, tk);
            tk.mode = MODE_FULL;
            tk.c_out = tk.c_begin;
            tk.init = INIT_HS;
            tk.dst = DST_NONE;
        }
        run_task<T, MODE_FULL>(prm, sm, tk);
    }
}

// ---------------------------------------------------------------------------
// Planner of the split forward (one workgroup).
//
// Cost model, in units of one fused chunk step: a pass-1 step costs kCostPass1,
// one link of the state chain of an exact head kCostLink.  An exact head with
// P >= 3 segments keeps P - 1 workgroups busy for about
//     L (1 + kCostPass1) + (P - 2) kCostLink,   L = 8 N / (kSeg0Weight + 8 (P - 1)),
// where segment 0 (which only runs full steps and later takes the last
// segment) is kSeg0Weight / 8 times as long as the others.  The remaining
// workgroups share the window heads' segments, each costing N / P_w + w.  The
// planner takes the P (and P_w) with the smallest estimated makespan.
constexpr float kCostPass1 = 1.4f;
constexpr float kCostLink = 1.0f;
constexpr int kSeg0Weight = 11;

__device__ int exact_bound(int p, int P, int N, int w0) {
    if (p <= 0) return 0;
    if (p >= P) return N;
    return (int)(((long long)N * (w0 + 8 * (p - 1))) / (w0 + 8 * (P - 1)));
}

__device__ void choose_segments(int n_e, int n_w, int N, int w, int cus, int pmax, int& Pe, int& Pw) {
    float best = 3.0e38f;
    Pe = 1;
    Pw = 1;
    const int pw_cap = N / w > 1 ? N / w : 1;
    for (int P = 1; P <= (n_e > 0 ? pmax : 1); ++P) {
        if (P == 2) continue;   // two segments only serialise
        const int ecus = n_e * (P == 1 ? 1 : P - 1);
        if (P > 1 && ecus > cus) break;
        float te = 0.f;
        if (n_e > 0)
            te = P == 1 ? (float)N
                        : 8.f * N * (1.f + kCostPass1) / (kSeg0Weight + 8 * (P - 1)) + (P - 2) * kCostLink;
        const int free = cus - ecus > 0 ? cus - ecus : 0;
        int pw = 1;
        float tw = 0.f;
        if (n_w > 0) {
            if (free >= n_w) {
                pw = free / n_w;
                if (pw > pmax) pw = pmax;
                if (pw > pw_cap) pw = pw_cap;
                tw = (float)N / pw + (pw > 1 ? w : 0);
            } else if (free > 0) {
                tw = (float)((n_w + free - 1) / free) * N;
            } else {
                tw = te + N;
            }
        }
        const float t = te > tw ? te : tw;
        if (t < best * 0.999f) {
            best = t;
            Pe = P;
            Pw = pw;
        }
    }
}

__device__ __forceinline__ void put_job(TaskRec* jobs, int j, int bh, int seg, int cb, int co, int ce,
                                        int mode, int init, int dst) {
    TaskRec r;
    r.bh = bh; r.seg = seg; r.c_begin = cb; r.c_out = co; r.c_end = ce;
    r.mode = mode; r.init = init; r.dst = dst;
    jobs[j] = r;
}

__global__ __launch_bounds__(256) void plan_kernel(FwdParams prm) {
    __shared__ int s_rank[256];
    __shared__ int s_par[4];
    const int tid = threadIdx.x;
    const int nbh = prm.B * prm.H, N = prm.N, pmax = prm.P, w = prm.w;
    const int per = (nbh + 255) / 256;
    const int lo = tid * per < nbh ? tid * per : nbh;
    const int hi = lo + per < nbh ? lo + per : nbh;
    auto exact = [&](int bh) { return prm.flags == nullptr || prm.flags[bh] == 0; };
    int ne = 0;
    for (int bh = lo; bh < hi; ++bh) ne += exact(bh) ? 1 : 0;
    s_rank[tid] = ne;
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int i = 0; i < 256; ++i) {
            const int c = s_rank[i];
            s_rank[i] = run;
            run += c;
        }
        const int n_e = run, n_w = nbh - run;
        int Pe = pmax, Pw = pmax;
        if (!prm.forced) choose_segments(n_e, n_w, N, w, prm.cus, pmax, Pe, Pw);
        s_par[0] = n_e;
        s_par[1] = n_w;
        s_par[2] = Pe;
        s_par[3] = Pw;
        FwdPlan* pl = prm.plan;
        pl->P_e = Pe;
        pl->P_w = Pw;
        pl->n_exact = n_e;
        pl->n_window = n_w;
        pl->n_jobs = n_e * Pe + n_w * Pw;
        pl->next = 0;
        pl->error = 0;
    }
    __syncthreads();
    const int n_e = s_par[0], n_w = s_par[1], Pe = s_par[2], Pw = s_par[3];
    // job groups: [seg 0 of exact heads][middle segments, p-major][window jobs][last segments]
    const int g_mid = n_e, g_win = n_e + n_e * (Pe > 2 ? Pe - 2 : 0), g_last = g_win + n_w * Pw;
    const int w0 = prm.forced ? 8 : kSeg0Weight;
    const bool has_h0 = prm.h0 != nullptr, has_ht = prm.ht != nullptr;
    int re = s_rank[tid], rw = lo - s_rank[tid];
    for (int bh = lo; bh < hi; ++bh) {
        if (exact(bh)) {
            const int init0 = has_h0 ? INIT_H0 : INIT_ZERO;
            if (Pe == 1) {
                put_job(prm.jobs, re, bh, 0, 0, 0, N, MODE_FULL, init0, has_ht ? DST_HT : DST_NONE);
            } else {
                put_job(prm.jobs, re, bh, 0, 0, 0, exact_bound(1, Pe, N, w0), MODE_FULL, init0, DST_HS_NEXT);
                for (int p = 1; p + 1 < Pe; ++p) {
                    const int cb = exact_bound(p, Pe, N, w0), ce = exact_bound(p + 1, Pe, N, w0);
                    put_job(prm.jobs, g_mid + (p - 1) * n_e + re, bh, p, cb, ce, ce, MODE_PASS1, INIT_ZERO,
                            DST_COMPOSE);
                }
                const int cb = exact_bound(Pe - 1, Pe, N, w0);
                put_job(prm.jobs, g_last + re, bh, Pe - 1, cb, cb, N, MODE_FULL, INIT_HS_WAIT,
                        has_ht ? DST_HT : DST_NONE);
            }
            ++re;
        } else {
            for (int p = 0; p < Pw; ++p) {
                const int s = (int)(((long long)p * N) / Pw), e = (int)(((long long)(p + 1) * N) / Pw);
                const int cb = s - w > 0 ? s - w : 0;
                put_job(prm.jobs, g_win + p * n_w + rw, bh, p, cb, s, e, MODE_FULL,
                        (cb == 0 && has_h0) ? INIT_H0 : INIT_ZERO,
                        (p == Pw - 1 && has_ht) ? DST_HT : DST_NONE);
            }
            ++rw;
        }
    }
    for (int i = tid; i < nbh * pmax; i += 256) prm.hs_cnt[i] = 0;
}

template <typename K>
hipError_t set_lds(K kernel, size_t lds) {
    return hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

template <typename T, int PHASE>
hipError_t launch_phase(const FwdParams& p, hipStream_t s) {
    const size_t lds = sizeof(Smem<T>);
    static bool configured = false;
    if (!configured) {
        hipError_t e;
        if constexpr (PHASE == PHASE_QUEUE)
            e = set_lds(gdn_fwd_queue_kernel<T>, lds);
        else
            e = set_lds(gdn_fwd_kernel<T, PHASE>, lds);
        if (e != hipSuccess) return e;
        configured = true;
    }
    if constexpr (PHASE == PHASE_QUEUE)
        hipLaunchKernelGGL((gdn_fwd_queue_kernel<T>), dim3(p.cus), dim3(kThreads), lds, s, p);
    else
        hipLaunchKernelGGL((gdn_fwd_kernel<T, PHASE>), dim3(p.B * p.H), dim3(kThreads), lds, s, p);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_fwd_t(const FwdParams& p, int phase, hipStream_t s) {
    if (phase == PHASE_SINGLE) return launch_phase<T, PHASE_SINGLE>(p, s);
    if (phase == PHASE_STATES) return launch_phase<T, PHASE_STATES>(p, s);
    return launch_phase<T, PHASE_QUEUE>(p, s);
}

}  // namespace

hipError_t launch_fwd(const FwdParams& p, int phase, bool bf16, hipStream_t s) {
    return bf16 ? launch_fwd_t<__bf16>(p, phase, s) : launch_fwd_t<float>(p, phase, s);
}

hipError_t launch_plan(const FwdParams& p, hipStream_t s) {
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace gdn
