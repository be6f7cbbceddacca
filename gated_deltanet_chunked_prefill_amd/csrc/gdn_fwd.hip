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
//     gate-free, T0_pp = (I + A0_pp)^-1, by recursive block doubling on
//     MFMA (Z <- Z - Z No Z from 1x1 to 32x32 blocks, stable for any keys);
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
// window maxima, gives every head a window length or marks it exact, chooses
// the segment counts of exact and window heads from a cost model and writes
// the job list; persistent workgroups (one per CU) then take
// jobs from an atomic counter.  An exact head with P segments gets a full run
// of segment 0, pass-1 runs of the middle segments (publishing their
// transitions), one chain job composing the true entering states, and full
// runs of segments 1 .. P-1 from those states; window heads (paragraph 5) get
// independent jobs that warm up over the w chunks before their segment.  The
// list is ordered so that every job waits only for jobs handed out before it,
// so the waits end for any number of resident workgroups.
//
// K^T and V in accumulator layout are read from the row-major tiles with the
// transposing LDS read; O is produced transposed (O^T = H^T Q^T + V'^T P^T) so
// each lane holds a row of O and writes it as 8-byte segments.
#include <mutex>

#include "gdn_chunk.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

enum { INIT_ZERO = 0, INIT_H0 = 1, INIT_HS = 2, INIT_HS_WAIT = 3 };
enum { DST_NONE = 0, DST_HT = 1, DST_HS_NEXT = 2, DST_TRANSITION = 3 };
enum { MODE_CHAIN = 2 };   // job kind beside MODE_FULL and MODE_PASS1

constexpr int kThreads = 512;   // 4 state waves + 4 prep waves
constexpr int kMtStride = kDk + 4;   // float row stride of a segment transition staged in LDS
constexpr int kSpinLimit = 1 << 22;  // polls of about 1 us: seconds, far beyond any real wait
constexpr size_t kSS = (size_t)kDk * kDv;

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

// Hand-off of data between workgroups of one launch.  The producer writes with
// device-coherent stores (the sc1 policy: written through to the level shared
// by all XCDs), waits until its wave's stores are acknowledged, then adds 1 to
// a counter; the consumer polls the counter and reads with device-coherent
// loads.  No cache-wide write-back or invalidation is needed on either side.
// Bulk data moves as 16-byte buffer accesses; a handed-off state is stored
// transposed ([dv][dk]) so that each lane's four consecutive accumulator rows
// are one 16-byte word.
constexpr int kSC1 = 16;   // cache-policy operand: device scope
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t dev_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ void st_dev(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// byte offset of lane (n, g)'s accumulator rows 32ht + 8q + 4g .. +3 of state
// column 32w + n in the transposed layout
__device__ __forceinline__ int state_t_off(int w, int lane, int ht, int q) {
    return ((32 * w + (lane & 31)) * kDk + 32 * ht + 8 * q + 4 * (lane >> 5)) * 4;
}
__device__ __forceinline__ void store_state_t_dev(float* dst, int w, int lane, const f32x16* Hs) {
    const __amdgpu_buffer_rsrc_t rs = dev_rsrc(dst, (int)(kSS * 4));
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f32x4 v = {Hs[ht][4 * q], Hs[ht][4 * q + 1], Hs[ht][4 * q + 2], Hs[ht][4 * q + 3]};
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, state_t_off(w, lane, ht, q), 0,
                                                   kSC1);
        }
}
__device__ __forceinline__ void load_state_t_dev(const float* src, int w, int lane, f32x16* Hs) {
    const __amdgpu_buffer_rsrc_t rs = dev_rsrc(src, (int)(kSS * 4));
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f32x4 v = __builtin_bit_cast(
                f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, state_t_off(w, lane, ht, q), 0, kSC1));
#pragma unroll
            for (int j = 0; j < 4; ++j) Hs[ht][4 * q + j] = v[j];
        }
}
// Count this wave in (by `amount`) once all its earlier stores are acknowledged.
__device__ __forceinline__ void publish(int* cnt, int amount = 1) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    wait_vm();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_add(cnt, amount, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A handed-off state is complete when its counter reaches kStateParts: the
// four state waves of a full run add 4 each, the 16 waves of the four chain
// jobs (one per 32-column block) 1 each.
constexpr int kStateParts = 16;
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
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// The serial state step of one chunk for state wave w (its 32 state columns).
// EMIT (output chunk or not) is a compile-time choice: a run-time flag inside
// the unrolled product loops made every k-step branch and copy the (Q H)^T
// accumulators, waiting on each product's result.
template <typename T, int MODE, bool EMIT>
__device__ __forceinline__ void chunk_state(T* o, int Tn, int H, float scale, const Lane<T>& L, const T* kt,
                                            const T* qt, const T* vt, const T (*t32)[kT32],
                                            const float* gam_vec, const float* e_vec, float GC,
                                            int b, int h, int t0, int nvalid,
                                            f32x16* Hs) {
    constexpr bool emit = MODE == MODE_FULL && EMIT;
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
        // the state fragment of this k-step is converted right before use (into
        // the column order of the K and Q fragments)
        const F hf = nat_frag<T>(acc_frag<T>(Hs[ks >> 1], ks & 1));
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
    }
    // H <- Gamma_C H + K^T diag(E) V', issued before the output is converted and
    // stored so that those instructions overlap the update's products
    F ef[4];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        f32x16 ev = Vp[rt] * rows_of(e_vec, rt, g);
        ef[2 * rt] = acc_frag<T>(ev, 0);
        ef[2 * rt + 1] = acc_frag<T>(ev, 1);
    }
    kt_update<T>(L, kt, Hs, GC, ef);
    if (MODE == MODE_FULL && emit) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int pos = 32 * rt + n;
            // global address space: plain vector stores, counted by vmcnt only
            T* const orow = o + (((size_t)b * Tn + t0 + pos) * H + h) * kDv + 32 * w;
            if constexpr (sizeof(T) == 2) {
                // lane (n, g) holds state columns 8i + 4g .. +3 (i = 0..3) of row pos;
                // two lane swaps between the half-waves give it columns 8g .. +7 and
                // 16 + 8g .. +7, two 16-byte pieces
                uint32_t pk[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
                    const b2 pr = {(__bf16)(scale * OT[rt][2 * k]), (__bf16)(scale * OT[rt][2 * k + 1])};
                    pk[k] = __builtin_bit_cast(uint32_t, pr);
                }
#pragma unroll
                for (int q = 0; q < 2; ++q) {
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const auto r = __builtin_amdgcn_permlane32_swap(pk[4 * q + e], pk[4 * q + 2 + e], false, false);
                        pk[4 * q + e] = r[0];
                        pk[4 * q + 2 + e] = r[1];
                    }
                }
                if (pos < nvalid) {
                    typedef __attribute__((address_space(1))) u32x4 gu4;
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        const u32x4 v = {pk[4 * q], pk[4 * q + 1], pk[4 * q + 2], pk[4 * q + 3]};
                        *(gu4*)(orow + 16 * q + 8 * g) = v;
                    }
                }
            } else {
                if (pos < nvalid) {
                    typedef T t4 __attribute__((ext_vector_type(4)));
                    typedef __attribute__((address_space(1))) t4 gt4;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        t4 v;
#pragma unroll
                        for (int e = 0; e < 4; ++e) v[e] = (T)(scale * OT[rt][4 * i + e]);
                        *(gt4*)(orow + 8 * i + 4 * g) = v;
                    }
                }
            }
        }
    }
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
    __bf16* const hst = KEEP ? uni(prm.hstore) : nullptr;
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
        if (init == INIT_HS_WAIT) wait_published(uni(prm.hs_cnt) + slot, kStateParts, &uni(prm.plan)->error);
        load_state_t_dev(uni(prm.hs) + slot * SS, L.w, L.lane, Hs);
    } else {
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) Hs[ht] = zero16();
    }
    const size_t hst_base = (size_t)bh * (N + 1);
    // chunks before i_out only warm the state up; from i_out on they emit outputs
    // (two loops, each with its step compiled for its kind of chunk)
    const int i_out = (MODE == MODE_FULL && o != nullptr) ? (c_out > c_begin ? c_out - c_begin : 0) : nch;
    // the state entering every chunk this task owns (for the backward)
    auto keep = [&](int c) {
        if (KEEP && c >= c_out) store_state_bf16t(hst + (hst_base + c) * SS, L.w, L.lane, Hs);
    };
    if constexpr (kPipe) {
        lds_barrier();
        lds_barrier();
        for (int i = 0; i < i_out && i < nch; ++i) {
            const int c = c_begin + i;
            const int slot = i % 3, vb = i & 1;
            keep(c);
            chunk_state<T, MODE, false>(o, Tn, H, scale, L, sm.kt[slot], sm.qt[slot], sm.vt[vb], sm.t32[vb],
                                        sm.gam_vec[vb], sm.e_vec[vb], sm.gc[vb][0], b, h, c * kChunk,
                                        chunk_len(Tn, c), Hs);
            lds_barrier();
        }
        for (int i = i_out; i < nch; ++i) {
            const int c = c_begin + i;
            const int slot = i % 3, vb = i & 1;
            keep(c);
            chunk_state<T, MODE, true>(o, Tn, H, scale, L, sm.kt[slot], sm.qt[slot], sm.vt[vb], sm.t32[vb],
                                       sm.gam_vec[vb], sm.e_vec[vb], sm.gc[vb][0], b, h, c * kChunk,
                                       chunk_len(Tn, c), Hs);
            lds_barrier();
        }
    } else {
        for (int i = 0; i < nch; ++i) {
            const int c = c_begin + i;
            lds_barrier();
            lds_barrier();
            lds_barrier();
            keep(c);
            if (i >= i_out)
                chunk_state<T, MODE, true>(o, Tn, H, scale, L, sm.kt[0], sm.qt[0], sm.vt[0], sm.t32[0],
                                           sm.gam_vec[0], sm.e_vec[0], sm.gc[0][0], b, h, c * kChunk,
                                           chunk_len(Tn, c), Hs);
            else
                chunk_state<T, MODE, false>(o, Tn, H, scale, L, sm.kt[0], sm.qt[0], sm.vt[0], sm.t32[0],
                                            sm.gam_vec[0], sm.e_vec[0], sm.gc[0][0], b, h, c * kChunk,
                                            chunk_len(Tn, c), Hs);
        }
    }
    if (KEEP && c_end == N) keep(N);
    if (dst == DST_HT) {
        store_state(uni(prm.ht) + (size_t)bh * SS, L.w, L.lane, Hs);
    } else if (dst == DST_HS_NEXT) {
        store_state_t_dev(uni(prm.hs) + (slot + 1) * SS, L.w, L.lane, Hs);
        publish(uni(prm.hs_cnt) + slot + 1, kStateParts / 4);
    } else if (dst == DST_TRANSITION) {
        // Hs is this segment's run from a zero state; the prep waves publish Mt
        store_state_t_dev(uni(prm.bz) + slot * SS, L.w, L.lane, Hs);
        publish(uni(prm.tr_cnt) + slot);
        lds_barrier();   // done with the chunk tiles
        lds_barrier();   // Mt staged in LDS
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
    float g_cur = 0.f, b_cur = 0.f;
    f32x16 Ms[4];
    if (MODE == MODE_PASS1) {
#pragma unroll
        for (int ht = 0; ht < 4; ++ht)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                Ms[ht][r] = (32 * ht + rho(L.g, r) == 32 * L.w + L.n) ? 1.f : 0.f;
    }
    auto need_q = [&](int c) { return MODE == MODE_FULL && has_o && c >= c_out; };
    // bf16: prep waves 2 and 3 issue every load of the chunk tiles and stage g and
    // beta in LDS, so waves 0 and 1 (the diagonal inverses, the longest prep work)
    // never wait on the memory pipeline; float32: all four load their quarter.
    constexpr int kLoaders = kPipe ? 2 : 4;
    const bool loader = pw >= 4 - kLoaders;
    TileLoader<T, kLoaders> TL;
    if (loader) TL.init(pw - (4 - kLoaders), L.lane, H);
    auto load_kq = [&](int c, int slot) {
        if (!loader) return;
        const size_t cb = chunk_base(b, h, Tn, H, c);
        const int nv = chunk_len(Tn, c);
        TL.load(sm.kt[slot], kp + cb, nv);
        if (need_q(c)) TL.load(sm.qt[slot], qp + cb, nv);
    };
    auto load_v = [&](int c, int slot) {
        if (!loader) return;
        TL.load(sm.vt[slot], vp + chunk_base(b, h, Tn, H, c), chunk_len(Tn, c));
    };
    auto load_gb = [&](int c, float& gv, float& bv) {
        load_gate_beta(gp, bp, Tn, H, b, h, c, L.lane, gv, bv);
    };
    // g (wave 2) and beta (wave 3) of chunk c into LDS slot `slot`, zero past the
    // end of the sequence (a short chunk goes through registers)
    auto stage_gb = [&](int c, int slot) {
        if (pw < 2) return;
        const float* const src = pw == 2 ? gp : bp;
        float* const dst = &sm.gbt[slot][pw - 2][0];
        const size_t e0 = ((size_t)b * Tn + (size_t)c * kChunk) * H + h;
        const int nv = chunk_len(Tn, c);
        if (nv == kChunk) {
            __builtin_amdgcn_global_load_lds((const void*)(src + e0 + (size_t)L.lane * H),
                                             (__attribute__((address_space(3))) void*)dst, 4, 0, kCpolStream);
        } else {
            typedef __attribute__((address_space(1))) const float gfloat;
            dst[L.lane] = L.lane < nv ? ((gfloat*)src)[e0 + (size_t)L.lane * H] : 0.f;
        }
    };
    if constexpr (kPipe) {
        // prologue: chunk 0 in LDS and prepped; chunk 1's K, Q, g, beta in flight
        load_kq(c_begin, 0);
        load_v(c_begin, 0);
        stage_gb(c_begin, 0);
        if (nch > 1) {
            load_kq(c_begin + 1, 1);
            stage_gb(c_begin + 1, 1);
        }
        wait_vm();
        lds_barrier();
        chunk_prep<T, MODE>(sm, L, pw, sm.kt[0], sm.qt[0], sm.t32[0], sm.gam_vec[0], sm.e_vec[0],
                            sm.gc[0], sm.gbt[0][0][L.lane], sm.gbt[0][1][L.lane], need_q(c_begin), gsum);
        lds_barrier();
        for (int i = 0; i < nch; ++i) {
            const int c = c_begin + i;
            // this chunk's segment transition (its prep outputs are in buffer i & 1)
            if (MODE == MODE_PASS1) mt_step<T>(L, sm.kt[i % 3], sm.t32[i & 1], Ms);
            if (i + 1 < nch) {
                if (i + 2 < nch) {
                    load_kq(c + 2, (i + 2) % 3);
                    stage_gb(c + 2, (i + 2) % 3);
                }
                load_v(c + 1, (i + 1) & 1);
                const int slot = (i + 1) % 3, pb = (i + 1) & 1;
                chunk_prep<T, MODE>(sm, L, pw, sm.kt[slot], sm.qt[slot], sm.t32[pb], sm.gam_vec[pb],
                                    sm.e_vec[pb], sm.gc[pb], sm.gbt[slot][0][L.lane], sm.gbt[slot][1][L.lane],
                                    need_q(c + 1), gsum);
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
    if (dst == DST_TRANSITION) {
        // publish the segment's gate-free transition Mt as bf16 hi and lo parts
        // (row-major [128][128] each) and exp(G), staged through LDS as floats
        lds_barrier();   // the state waves are done with the chunk tiles
        float* const mtl = reinterpret_cast<float*>(&sm.kt[0][0]);
#pragma unroll
        for (int ht = 0; ht < 4; ++ht)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                mtl[(32 * ht + rho(L.g, r)) * kMtStride + 32 * L.w + L.n] = Ms[ht][r];
        lds_barrier();   // Mt staged
        const size_t slot = (size_t)bh * uni(prm.P) + uni(tk.seg);
        const __amdgpu_buffer_rsrc_t rs = dev_rsrc(uni(prm.mt) + slot * 2 * kSS, (int)(2 * kSS * 2));
        const int row = 32 * pw + (L.lane >> 1), c0 = 64 * (L.lane & 1);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float* src = mtl + row * kMtStride + c0 + 8 * i;
            const f32x4 x0 = *reinterpret_cast<const f32x4*>(src);
            const f32x4 x1 = *reinterpret_cast<const f32x4*>(src + 4);
            bf16x8 hi, lo;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float x = j < 4 ? x0[j] : x1[j - 4];
                hi[j] = (__bf16)x;
                lo[j] = (__bf16)(x - (float)hi[j]);
            }
            const int off = (row * kDk + c0 + 8 * i) * 2;
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, hi), rs, off, 0, kSC1);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, lo), rs, off + (int)kSS * 2, 0, kSC1);
        }
        if (pw == 3 && L.lane == 0) st_dev(uni(prm.eg) + slot, __expf(gsum));
        publish(uni(prm.tr_cnt) + slot);
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

// Chain jobs of an exact head (talk summary, paragraph 4: segment p maps the
// state entering it, H, to exp(G_p) Mt_p H + b_p, so the true entering states
// follow from the first one by one dk x dk product per segment):
//     hs[p+1] = exp(G_p) Mt_p hs[p] + b_p,   p = seg .. c_end - 1.
// Columns of the state evolve independently, so four jobs share a head, job c
// owning state columns [32c, 32c+32); its state wave w forms the 32 x 32 tile
// of rows [32w, 32w+32) per link (24 split-precision MFMAs: a_hi b_hi + a_hi
// b_lo + a_lo b_hi), publishes it, and the four tiles are exchanged through LDS
// for the next link.  The prep waves stream each Mt_p (bf16 hi and lo parts,
// published by the pass-1 job of segment p) into LDS one link ahead; each
// wave's part of b_p is loaded one link ahead, and a tile's publication is
// counted one link late, once the wave's later loads show its stores done.
template <typename T>
struct ChainBuf {
    // Mt double-buffered when both buffers fit in front of the prep outputs
    static constexpr bool two = 2 * 4 * kChunk * kDk * 2 <= (int)offsetof(Smem<T>, t32);
    static __device__ __forceinline__ __bf16* tiles(Smem<T>& sm, int buf) {
        return reinterpret_cast<__bf16*>(&sm) + (two ? buf : 0) * 4 * kChunk * kDk;
    }
    // exchange of the four 32 x 32 float tiles of a column block (16 KiB)
    static __device__ __forceinline__ float* exch(Smem<T>& sm) {
        return reinterpret_cast<float*>(&sm.t32[0][0][0]);
    }
};
static_assert(sizeof(((Smem<float>*)0)->t32) >= 16384 && sizeof(((Smem<__bf16>*)0)->t32) >= 16384,
              "the chain's tile exchange lives in the prep-output area");

// byte offset of lane (n, g)'s rows 32ht + 8q + 4g .. +3 of state column 32c + n
// (transposed layout), as in state_t_off
__device__ __forceinline__ void load_tile_t_dev(const float* src, int c, int ht, int lane, f32x16& t) {
    const __amdgpu_buffer_rsrc_t rs = dev_rsrc(src, (int)(kSS * 4));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const f32x4 v = __builtin_bit_cast(
            f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, state_t_off(c, lane, ht, q), 0, kSC1));
#pragma unroll
        for (int j = 0; j < 4; ++j) t[4 * q + j] = v[j];
    }
}
__device__ __forceinline__ void store_tile_t_dev(float* dst, int c, int ht, int lane, const f32x16& t) {
    const __amdgpu_buffer_rsrc_t rs = dev_rsrc(dst, (int)(kSS * 4));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const f32x4 v = {t[4 * q], t[4 * q + 1], t[4 * q + 2], t[4 * q + 3]};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, state_t_off(c, lane, ht, q), 0,
                                               kSC1);
    }
}

template <typename T>
__device__ __noinline__ void chain_state(const FwdParams& prm, Smem<T>& sm, const Task& tk) {
    using CB = ChainBuf<T>;
    const int bh = uni(tk.bh), p0 = uni(tk.seg), p_end = uni(tk.c_end), c = uni(tk.c_begin);
    const int P = uni(prm.P);
    float* const hs = uni(prm.hs);
    const float* const bz = uni(prm.bz);
    const float* const eg = uni(prm.eg);
    int* const hs_cnt = uni(prm.hs_cnt);
    int* const err = &uni(prm.plan)->error;
    Lane<__bf16> L;
    L.init(threadIdx.x);
    const int w = L.w, lane = L.lane;
    const size_t base = (size_t)bh * P;
    float* const ex = CB::exch(sm);
    // the column block of the first state, all four row tiles
    f32x16 Hc[4];
    wait_published(hs_cnt + base + p0, kStateParts, err);
    load_state_t_dev(hs + (base + p0) * kSS, c, lane, Hc);
    // this wave's tile of b_p and exp(G_p): read after a barrier behind which the
    // prep waves have seen transition p published (one link ahead when
    // double-buffered)
    f32x16 Bt;
    float e = 0.f;
    if (CB::two) {
        lds_barrier();   // X: Mt_p0 in LDS
        load_tile_t_dev(bz + (base + p0) * kSS, c, w, lane, Bt);
        e = ld_dev(eg + base + p0);
    }
    for (int p = p0; p < p_end; ++p) {
        if (!CB::two) {
            lds_barrier();   // A: Mt_p in LDS
            load_tile_t_dev(bz + (base + p) * kSS, c, w, lane, Bt);
            e = ld_dev(eg + base + p);
        }
        // H column block split into bf16 hi and lo parts (the B operands, in the
        // column order of the Mt fragments)
        bf16x8 hh[8], hl[8];
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float x = Hc[ks >> 1][8 * (ks & 1) + j];
                hh[ks][j] = (__bf16)x;
                hl[ks][j] = (__bf16)(x - (float)hh[ks][j]);
            }
            hh[ks] = nat_frag<__bf16>(hh[ks]);
            hl[ks] = nat_frag<__bf16>(hl[ks]);
        }
        if (CB::two) lds_barrier();   // Y: the exchange has been read; Mt_p+1 in LDS
        const __bf16* const thi = CB::tiles(sm, (p - p0) & 1) + (w >> 1) * kChunk * kDk;
        const __bf16* const tlo = thi + 2 * kChunk * kDk;
        f32x16 acc0 = zero16(), acc1 = zero16();
#pragma unroll
        for (int ks = 0; ks < 8; ks += 2) {
            const bf16x8 ah0 = L.f128(thi, w & 1, ks), al0 = L.f128(tlo, w & 1, ks);
            const bf16x8 ah1 = L.f128(thi, w & 1, ks + 1), al1 = L.f128(tlo, w & 1, ks + 1);
            acc0 = mma(ah0, hh[ks], acc0);
            acc1 = mma(ah1, hh[ks + 1], acc1);
            acc0 = mma(ah0, hl[ks], acc0);
            acc1 = mma(ah1, hl[ks + 1], acc1);
            acc0 = mma(al0, hh[ks], acc0);
            acc1 = mma(al1, hh[ks + 1], acc1);
            __builtin_amdgcn_sched_barrier(0);   // bound the LDS reads in flight (registers)
        }
        // b_p arrived (and, memory operations of a wave completing in order, the
        // previous link's tile stores with it): count that tile in
        wait_vm();
        if (p > p0) publish(hs_cnt + base + p);
        f32x16 Hn;
#pragma unroll
        for (int r = 0; r < 16; ++r) Hn[r] = e * (acc0[r] + acc1[r]) + Bt[r];
        store_tile_t_dev(hs + (base + p + 1) * kSS, c, w, lane, Hn);
#pragma unroll
        for (int r = 0; r < 16; ++r) ex[(w * 16 + r) * 64 + lane] = Hn[r];
        if (CB::two && p + 1 < p_end) {
            // the prep waves saw transition p+1 published before barrier Y
            load_tile_t_dev(bz + (base + p + 1) * kSS, c, w, lane, Bt);
            e = ld_dev(eg + base + p + 1);
        }
        lds_barrier();   // X (two) / B: the exchange is written, Mt_p is done with
#pragma unroll
        for (int ht = 0; ht < 4; ++ht)
#pragma unroll
            for (int r = 0; r < 16; ++r) Hc[ht][r] = ex[(ht * 16 + r) * 64 + lane];
        if (!CB::two) lds_barrier();   // C: the exchange has been read
    }
    publish(hs_cnt + base + p_end);
}

template <typename T>
__device__ __noinline__ void chain_prep(const FwdParams& prm, Smem<T>& sm, const Task& tk) {
    using CB = ChainBuf<T>;
    const int pw = wave_id() - 4, lane = threadIdx.x & 63;
    const int bh = uni(tk.bh), p0 = uni(tk.seg), p_end = uni(tk.c_end), P = uni(prm.P);
    const __bf16* const mt = uni(prm.mt);
    const int* const tr_cnt = uni(prm.tr_cnt);
    int* const err = &uni(prm.plan)->error;
    const size_t base = (size_t)bh * P;
    TileLoader<__bf16> TL;
    TL.init(pw, lane, 1);
    auto load = [&](int p) {
        wait_published(tr_cnt + base + p, 8, err);
        const __bf16* const src = mt + (base + p) * 2 * kSS;
        __bf16* const dst = CB::tiles(sm, (p - p0) & 1);
#pragma unroll
        for (int q = 0; q < 4; ++q) TL.template load<16>(dst + q * kChunk * kDk, src + q * kChunk * kDk, kChunk);
        wait_vm();
    };
    if (CB::two) {
        // Mt_p+1 goes into the buffer link p-1 used; its readers finished before
        // the X barrier that ends link p-1
        load(p0);
        lds_barrier();   // X
        for (int p = p0; p < p_end; ++p) {
            if (p + 1 < p_end) load(p + 1);
            lds_barrier();   // Y
            lds_barrier();   // X
        }
    } else {
        for (int p = p0; p < p_end; ++p) {
            load(p);
            lds_barrier();   // A
            lds_barrier();   // B
            lds_barrier();   // C
        }
    }
}

// Sum of g over tokens [t_lo, t_hi) of row bh of a [B, T, H] gate tensor (token
// index b*T + t), by the whole workgroup; every thread returns the total.
template <typename T>
__device__ float gate_sum(const FwdParams& p, Smem<T>& sm, int bh, int t_lo, int t_hi) {
    const int b = bh / p.H, h = bh % p.H;
    float x = 0.f;
    for (int t = t_lo + (int)threadIdx.x; t < t_hi; t += kThreads)
        x += p.g[((size_t)b * p.T + t) * p.H + h];
    x = lane_value(wave_inclusive_scan(x), 63);
    float* const part = &sm.pscr[0][0][0];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int i = 0; i < kThreads / 64; ++i) tot += part[i];
    __syncthreads();   // the partials are read before the task reuses the scratch
    return tot;
}

// First chunk of a later segment's warm-up (window path, talk summary paragraph 5,
// commentary paragraph 8): starting from the zero state m*w chunks before the
// segment's first output chunk c_out is within a factor exp(sum of g over those
// chunks) of the true state, so the shortest of m = 1, 2, 4, 8 whose window sum
// is at most log eps is taken; with none, the segment runs from the sequence's
// first chunk (its h0), which is exact.
template <typename T>
__device__ int varlen_warmup_start(const FwdParams& p, Smem<T>& sm, int bh, int c_out) {
    float acc = 0.f;
    int done = 0;   // chunks summed so far, counted back from c_out
    for (int m = 1; m <= 8; m *= 2) {
        const int L = m * p.w;
        if (c_out - L <= 0) return 0;
        acc += gate_sum(p, sm, bh, (c_out - L) * kChunk, (c_out - done) * kChunk);
        done = L;
        if (acc <= p.log_eps) return c_out - L;
    }
    return 0;
}

template <typename T, int PHASE>
__global__ __launch_bounds__(kThreads, 1) void gdn_fwd_kernel(FwdParams prm) {
    extern __shared__ __attribute__((aligned(16))) char smem_raw[];
    Smem<T>& sm = *reinterpret_cast<Smem<T>*>(smem_raw);
    Task tk;
    if constexpr (PHASE == PHASE_VARLEN || PHASE == PHASE_STATES_VARLEN) {
        // Packed sequences: workgroup = (segment p, sequence s, head h), p slowest
        // and descending (later segments, which carry a warm-up and belong to the
        // longest sequences, are dispatched first); sequence s holds tokens
        // [t0, t0 + len).  The task runs as sequence s of
        // a batch of sequences of length len, with every token pointer shifted by
        // t0 - s*len, so that the loops' token index s*len + t addresses token
        // t0 + t (and, when the states are kept, the state slot bh*(nch+1) + c
        // addresses the sequence's own slots).
        const int SH = prm.B * prm.H;
        int pi = (int)blockIdx.x / SH;
        const int sh = (int)blockIdx.x % SH;
        if (PHASE == PHASE_VARLEN && prm.vseg > 0) pi = prm.P - 1 - pi;
        const int s = sh / prm.H, h = sh % prm.H;
        const SeqSpan sp = seq_span(prm.cu, prm.cstart, prm.B, prm.T, s);
        // a long sequence is cut into segments of about vseg chunks (talk summary,
        // paragraph 4); every workgroup derives the same cut from the sequence's length
        int nseg = 1;
        if (PHASE == PHASE_VARLEN && prm.vseg > 0) {
            nseg = (sp.nch + prm.vseg - 1) / prm.vseg;
            nseg = nseg < 1 ? 1 : (nseg > prm.P ? prm.P : nseg);
        }
        if (pi >= nseg) return;   // workgroup-uniform, before any barrier
        const long long shift = ((long long)sp.t0 - (long long)s * sp.len) * prm.H;   // token-head rows
        FwdParams p = prm;
        p.q = (const T*)prm.q + shift * kDk;
        p.k = (const T*)prm.k + shift * kDk;
        p.v = (const T*)prm.v + shift * kDv;
        if (prm.o) p.o = (T*)prm.o + shift * kDv;
        p.g = prm.g + shift;
        p.beta = prm.beta + shift;
        p.T = sp.len;
        p.N = sp.nch;
        if constexpr (PHASE == PHASE_STATES_VARLEN) {
            const long long slot = (long long)h * (prm.cmax + prm.B) + sp.c0 + s -
                                   (long long)sh * (sp.nch + 1);
            p.hstore = prm.hstore + slot * (long long)(kDk * kDv);
        }
        tk.bh = sh;
        tk.seg = 0;
        tk.c_out = (int)((long long)sp.nch * pi / nseg);
        tk.c_end = (int)((long long)sp.nch * (pi + 1) / nseg);
        tk.c_begin = pi == 0 ? 0 : varlen_warmup_start(p, sm, sh, tk.c_out);
        tk.mode = MODE_FULL;
        tk.init = (tk.c_begin == 0 && prm.h0) ? INIT_H0 : INIT_ZERO;
        tk.dst = (tk.c_end == sp.nch && prm.ht) ? DST_HT : DST_NONE;
        run_task<T, MODE_FULL, PHASE == PHASE_STATES_VARLEN>(p, sm, tk);
    } else {
        whole_head_task(prm, tk);
        if (PHASE == PHASE_STATES)
            run_task<T, MODE_FULL, true>(prm, sm, tk);
        else
            run_task<T, MODE_FULL>(prm, sm, tk);
    }
}

// Per-head tables of the planner live in LDS up to this many heads (always, for
// the automatic split, which needs B*H < CUs), in the workspace beyond.
constexpr int kPlanHeads = 4096;

// The persistent kernel's parameters read straight from the kernel-argument
// segment (they are its only argument, at offset 0), with scalar loads.  The
// kernel's own copy, which the job functions take by reference, sits in scratch
// memory; reading that back would put a scratch round trip before the
// planner's first loads.
using KParams = const __attribute__((address_space(4))) FwdParams;
__device__ __forceinline__ KParams& launch_params() {
    return *(KParams*)__builtin_amdgcn_kernarg_segment_ptr();
}

template <typename T>
__device__ __forceinline__ void plan_wg(const FwdParams& prm, Smem<T>& sm, bool publish);

// Persistent workgroups of the split forward: take jobs until the list is empty.
// KEEP: every job with outputs also stores the state entering each of its output
// chunks (the backward's state store for few heads).
template <typename T, bool KEEP>
__global__ __launch_bounds__(kThreads, 1) void gdn_fwd_queue_kernel(FwdParams prm) {
    extern __shared__ __attribute__((aligned(16))) char smem_raw[];
    Smem<T>& sm = *reinterpret_cast<Smem<T>*>(smem_raw);
    // The plan is a deterministic function of the launch's inputs.  With the
    // per-head tables in LDS every workgroup plans for itself and starts its
    // first job (its own index) at once; workgroup 0 also writes the job list
    // for the jobs handed out later and releases it through the ready word
    // (cleared by the preceding launch, it becomes n_jobs + 1; the records are
    // written back before it and read with device-coherent loads).  With more
    // heads than the LDS tables hold, workgroup 0 plans alone in the workspace
    // and the others wait for the list.
    int* const ready = &prm.plan->ready;
    int* const err = &prm.plan->error;
    const bool local = launch_params().B * launch_params().H <= kPlanHeads;
    const bool publish = blockIdx.x == 0;
    if (local || publish) {
        plan_wg<T>(prm, sm, publish);
        if (publish) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            __syncthreads();
            if (threadIdx.x == 0)
                __hip_atomic_store(ready, sm.islot[1] + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    } else if (threadIdx.x < 64) {
        wait_published(ready, 1, err);
        if (threadIdx.x == 0)
            sm.islot[1] = __hip_atomic_load(ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - 1;
    }
    __syncthreads();
    const int n_jobs = uni(sm.islot[1]);
    // the first job of every workgroup is its index; later ones come from the counter
    int j = blockIdx.x;
    bool first = true, listed = !local || publish;   // listed: the job list is known to be written
    for (;; ) {
        if (j >= n_jobs) break;
        int f[8];
        if (first && local) {
#pragma unroll
            for (int i = 0; i < 8; ++i) f[i] = uni(sm.jrec[i]);
        } else {
            if (!listed) {
                if (threadIdx.x < 64) wait_published(ready, 1, err);
                __syncthreads();
                listed = true;
            }
            // job records read with device-coherent vector loads (written this launch)
            const int* const jr = reinterpret_cast<const int*>(prm.jobs + j);
#pragma unroll
            for (int i = 0; i < 8; ++i) f[i] = uni(__hip_atomic_load(jr + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        }
        first = false;
        const Task tk{f[0], f[1], f[2], f[3], f[4], f[5], f[6], f[7]};
        if (tk.mode == MODE_CHAIN) {
            if (wave_id() < 4)
                chain_state<T>(prm, sm, tk);
            else
                chain_prep<T>(prm, sm, tk);
        } else if (tk.mode == MODE_PASS1) {
            run_task<T, MODE_PASS1>(prm, sm, tk);
        } else {
            run_task<T, MODE_FULL, KEEP>(prm, sm, tk);
        }
        if (threadIdx.x == 0) sm.islot[0] = (int)gridDim.x + atomicAdd(&prm.plan->next, 1);
        __syncthreads();
        j = uni(sm.islot[0]);
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Planner of the split forward (one workgroup).
//
// Jobs of an exact head split into P >= 3 segments (chunk bounds b_0 = 0 <
// b_1 < ... < b_P = N):
//   seg 0           full run of [0, b_1) from h0, publishes hs[1];
//   pass-1 p        run of [b_p, b_p+1) from a zero state (p = 1 .. P-2),
//                   publishes b_p, Mt_p and exp(G_p);
//   chain           hs[p+1] = exp(G_p) Mt_p hs[p] + b_p for p = 1 .. P-2;
//   pass-3 p        full run of [b_p, b_p+1) from hs[p] (p = 1 .. P-1), the
//                   last one writes ht.
// With P = 2 only seg 0 and one pass-3 job remain, with P = 1 one full run.
// A window head of level m (window of m*w chunks) gets P_m independent jobs,
// each warming up over the m*w chunks before its segment.  Queue order: seg 0
// jobs, pass-1 jobs, window jobs (longest windows first), chain jobs, pass-3
// jobs (segment-major), so that every job waits only for jobs handed out
// before it.
//
// Cost model, in units of one full chunk step under load: a pass-1 step costs
// kCostPass1, one link of the chain kCostLink, a warm-up step kCostWarm.  An
// exact head keeps P - 1 workgroups busy for about
//     L (1 + kCostPass1) + (P - 2) kCostLink,   L = 8 N / (kSeg0Weight + 8 (P - 1)),
// segment 0 being kSeg0Weight / 8 times as long as the others so that it ends
// with the pass-1 jobs.  The remaining workgroups share the window heads: a
// level-m head in P segments costs (N + (P - 1) c_m) / P per job, c_m =
// kCostWarm m w, when its first segment (which has no warm-up) is longer by
// c_m; the planner finds the smallest job cost M whose segment counts fit the
// free workgroups.  It takes the P with the smallest estimated makespan.
constexpr float kCostPass1 = 1.35f;
constexpr float kCostLink = 0.8f;
constexpr float kCostWarm = 0.7f;
constexpr int kSeg0Weight = 11;

constexpr int kCandP = 32;   // segment counts tried per kept window level: P = 1, 3, .., 32
constexpr int kMaxCand = (kMaxWindowLevels + 1) * (kCandP - 1);

// Job cost of a head of warm-up cost c in P segments: (N + (P - 1) c) / P.
__device__ __forceinline__ float win_job_cost(int N, float c, int P) {
    return ((float)N + (float)(P - 1) * c) / (float)P;
}

// Segments of a window head of warm-up cost c so that each job costs at most M:
// the smallest P with (N + (P - 1) c) / P <= M; `bad` is set when none up to
// `cap` exists.
__device__ __forceinline__ int win_segments(int N, float c, int cap, float M, bool& bad) {
    const float q = ((float)N - c) * __builtin_amdgcn_rcpf(M - c);
    int p = (int)ceilf(q);
    p = M >= (float)N ? 1 : p;
    bad = M < (float)N && (M <= c || p > cap);
    return bad ? 1 : p;
}

// A store through a global-address-space pointer.  The same store through a
// generic pointer is a flat store, which the wave also counts as an LDS
// operation: the next LDS barrier would wait until it reached memory.
template <typename V>
__device__ __forceinline__ void gstore(V* p, const V& v) {
    *(__attribute__((address_space(1))) V*)p = v;
}

// Job j: into the job list when publishing, and into the workgroup's LDS slot
// when it is the workgroup's first job.
__device__ __forceinline__ void put_job(TaskRec* jobs, int* jrec, bool publish, int j, int bh, int seg, int cb,
                                        int co, int ce, int mode, int init, int dst) {
    using i32x4 = int __attribute__((ext_vector_type(4)));
    static_assert(sizeof(TaskRec) == 2 * sizeof(i32x4), "job record layout");
    // the record's fields in declaration order, as two 16-byte stores
    const i32x4 lo = {bh, seg, cb, co}, hi = {ce, mode, init, dst};
    if (publish) {
        i32x4* const dst4 = reinterpret_cast<i32x4*>(jobs + j);
        gstore(dst4, lo);
        gstore(dst4 + 1, hi);
    }
    if (j == (int)blockIdx.x) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            jrec[i] = lo[i];
            jrec[4 + i] = hi[i];
        }
    }
}

__device__ int seg_bound(long long num, long long den, int N) {
    return (int)(((double)N * (double)num) / (double)den);
}

// Start of segment p of a level-m window head with P segments: the first
// segment is longer by c = kCostWarm m w so that every job costs the same.
// Equal segments when forced, or when the others would be shorter than 1.5
// chunks (the rounded bounds then still increase strictly).
__device__ int win_bound(int p, int P, int N, float c, bool forced) {
    if (p <= 0) return 0;
    if (p >= P) return N;
    int s;
    if (forced || (float)N - c < 1.5f * P) {
        s = (int)(((long long)p * N) / P);
    } else {
        const float L0 = ((float)N + (P - 1) * c) / P;
        s = (int)floorf(p * L0 - (p - 1) * c + 0.5f);
    }
    s = s < p ? p : s;
    return s > N - (P - p) ? N - (P - p) : s;
}

// Planner scratch in the workgroup's LDS (used before any job runs).
constexpr int kMaxBp = kMaxWindowLevels * kCandP;   // job-cost breakpoints: (level, P <= 32)

struct PlanLds {
    int bound[kMaxSegments + 1];
    int lcnt[1 + kMaxWindowLevels];   // heads per window level (0 = exact)
    float cw[kMaxWindowLevels];       // warm-up cost kCostWarm m w per level
    int cap[kMaxWindowLevels];        // most segments per level: min(pmax, max(1, N / (m w)))
    int cum[1 + kMaxWindowLevels];    // window heads of levels 1..m
    int off[1 + kMaxWindowLevels];    // breakpoints of levels 1..m (level m's start at off[m-1])
    int cnt[1 + kMaxWindowLevels];    // candidates per cutoff Lc
    int pm[kMaxWindowLevels];         // chosen segments of a window head per level
    int kb[kMaxWindowLevels];         // heads of a level given one segment more (the first ones)
    int pe, lc;                       // chosen exact segment count and longest level kept
    int tmin, win;                    // smallest estimated makespan (key) and the chosen candidate
    int rc[kThreads / 64][1 + kMaxWindowLevels];   // heads per wave and class in one round
    int cand_lc[kMaxCand], cand_p[kMaxCand], cand_fr[kMaxCand];   // candidate: cutoff, P, free workgroups
    int bkey[kMaxBp];                 // breakpoints, level by level (levels with heads): job cost (key)
    int need[kMaxWindowLevels][kMaxBp + 1];   // [Lc-1][b]: workgroups the window heads need at
                                              // breakpoint b (rows padded: no bank conflicts)
    int lev[kPlanHeads];              // window level per head (0 = exact)
    int hmap[kPlanHeads];             // heads by class
};

// q = floor(a / b) for 0 <= a < 2^20 and 1 <= b < 2^12 through the reciprocal:
// (a + 1/2) / b lies at least 1/(2b) from an integer, and the single-precision
// product is off by at most (a / b) 2^-22 < 1/(4b).
__device__ __forceinline__ int small_div(int a, int b) {
    return (int)(((float)a + 0.5f) * __builtin_amdgcn_rcpf((float)b));
}

// The planner, run by every workgroup of the persistent launch before its first
// job (by workgroup 0 alone when the per-head tables exceed the LDS), with the
// same result in each: it is on every workgroup's path to its first job, so
// every step is a short parallel pass with small code (it runs once per
// launch, from a cold instruction cache).  Workgroup 0 (`publish`) also writes
// the job list, the per-head levels and the plan record; every workgroup keeps
// its own first job in LDS.
//
// Candidates (Lc, P): window levels above Lc run as exact heads, exact heads
// take P segments.  Per Lc (from the highest level down, only where level
// Lc + 1 has heads or Lc is the highest) they are P = 1 and P = 3 .. the
// largest P whose exact jobs fit the workgroups (P = 1 alone when no head is
// exact).  The window heads' job cost M of a candidate is the smallest M at
// which their segment counts fit the free workgroups; a level's count only
// changes where M equals its job cost at some P, so M is the smallest feasible
// such breakpoint (each evaluated just above the breakpoint).  The makespan
// estimate is the larger of the exact heads' time and M; the earliest
// candidate within 0.1 % of the smallest wins (fewer segments, more window
// heads on near-ties).
template <typename T>
__device__ __forceinline__ void plan_wg(const FwdParams& prm_copy, Smem<T>& sm, bool publish) {
    KParams& prm = launch_params();
    (void)prm_copy;
    static_assert(sizeof(PlanLds) <= offsetof(Smem<T>, islot), "planner scratch overlaps the job slots");
    PlanLds& pl = *reinterpret_cast<PlanLds*>(&sm);
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int B = uni(prm.B), H = uni(prm.H), nbh = B * H, N = uni(prm.N), pmax = uni(prm.P), w = uni(prm.w);
    const int cus = uni(prm.cus), forced = uni(prm.forced);
    const int* const wmax = uni(prm.wmax);
    const int LV = wmax ? uni(prm.levels) : 0;
    const float log_eps = uni(prm.log_eps);
    int* const flags = uni(prm.flags);
    int* const head_map = uni(prm.head_map);
    float* const maxwin = uni(prm.maxwin);
    FwdPlan* const fp = uni(prm.plan);
    TaskRec* const jobs = uni(prm.jobs);
    const bool has_h0 = prm.h0 != nullptr, has_ht = prm.ht != nullptr;
    const bool in_lds = nbh <= kPlanHeads;
    // the group maxima of the thread's first head, loaded first: their latency
    // (data another launch wrote) overlaps the set-up below
    int key0[kMaxWindowLevels];
#pragma unroll
    for (int m = 0; m < kMaxWindowLevels; ++m) key0[m] = (wmax && m < LV && tid < nbh) ? wmax[(size_t)m * nbh + tid] : 0;
    if (tid <= kMaxWindowLevels) pl.lcnt[tid] = 0;
    if (tid < kMaxWindowLevels) {
        const int m = tid + 1;
        pl.cw[tid] = kCostWarm * (float)(m * w);
        int cp = N / (m * w);
        cp = cp < 1 ? 1 : cp;
        pl.cap[tid] = cp < pmax ? cp : pmax;
    }
    if (tid == 0) {
        pl.tmin = 0x7FFFFFFF;
        pl.win = 0x7FFFFFFF;
    }
    lds_barrier();
    // 1. window levels (talk summary, paragraph 5): a head is a window head of
    //    level m when its largest sum of g over m*w consecutive chunks is at
    //    most log_eps, for the smallest such m; the preceding launch left that
    //    largest sum per length and head
    if (wmax) {
        for (int bh = tid; bh < nbh; bh += kThreads) {
            int key[kMaxWindowLevels];
#pragma unroll
            for (int m = 0; m < kMaxWindowLevels; ++m)
                key[m] = bh == tid ? key0[m] : (m < LV ? wmax[(size_t)m * nbh + bh] : 0);
            int lev = 0;
#pragma unroll
            for (int m = kMaxWindowLevels; m >= 1; --m)
                if (m <= LV && N >= m * w && key_float(key[m - 1]) <= log_eps) lev = m;
            if (maxwin && publish) gstore(maxwin + bh, key_float(key[0]));
            if (in_lds)
                pl.lev[bh] = lev;
            else
                gstore(flags + bh, lev);
            atomicAdd(&pl.lcnt[lev], 1);
        }
    } else if (tid == 0) {
        pl.lcnt[0] = nbh;
    }
    lds_barrier();
    // per-level values in registers (loops over the levels are unrolled; a
    // level picked at run time is read from LDS); cum[m]: window heads of
    // levels 1..m; off[m]: breakpoints of levels 1..m (cap of each level with
    // heads), so that level m's breakpoints start at off[m-1]
    int lcnt[kMaxWindowLevels + 1], cap[kMaxWindowLevels], cum[kMaxWindowLevels + 1], off[kMaxWindowLevels + 1];
    float cw[kMaxWindowLevels];
    lcnt[0] = pl.lcnt[0];
    cum[0] = 0;
    off[0] = 0;
#pragma unroll
    for (int m = 1; m <= kMaxWindowLevels; ++m) {
        lcnt[m] = pl.lcnt[m];   // zero above LV
        cap[m - 1] = pl.cap[m - 1];
        cw[m - 1] = pl.cw[m - 1];
        cum[m] = cum[m - 1] + lcnt[m];
        off[m] = off[m - 1] + (lcnt[m] > 0 ? cap[m - 1] : 0);
    }
    if (tid <= kMaxWindowLevels) {
        int cv = 0, ov = 0;
#pragma unroll
        for (int m = 1; m <= kMaxWindowLevels; ++m) {
            cv = m == tid ? cum[m] : cv;
            ov = m == tid ? off[m] : ov;
        }
        pl.cum[tid] = cv;
        pl.off[tid] = ov;
    }
    lds_barrier();
    if (!forced) {
        // 2. candidate counts per cutoff (one thread per Lc) and the breakpoint
        //    list (one thread per (level, P))
        if (tid <= kMaxWindowLevels) {
            const int lc = tid, ne = nbh - pl.cum[lc];
            const bool distinct = lc <= LV && (lc == LV || pl.lcnt[lc + 1] > 0);
            int pok = ne > 0 ? 1 + small_div(cus, ne) : 1;   // largest P with ne (P - 1) <= cus
            pok = pok < pmax ? pok : pmax;
            pok = pok < kCandP ? pok : kCandP;
            pl.cnt[lc] = !distinct ? 0 : (ne == 0 ? 1 : 1 + (pok >= 3 ? pok - 2 : 0));
        }
        if (tid < kMaxBp) {
            const int m = 1 + (tid >> 5), p = 1 + (tid & 31);
            if (m <= LV && pl.lcnt[m] > 0 && p <= pl.cap[m - 1])
                pl.bkey[pl.off[m - 1] + p - 1] = float_key(win_job_cost(N, pl.cw[m - 1], p) * (1.f + 1e-5f));
        }
        lds_barrier();
        int cbase[kMaxWindowLevels + 1];   // first candidate of each cutoff (cutoffs from high to low)
        int ncand = 0;
#pragma unroll
        for (int lc = kMaxWindowLevels; lc >= 0; --lc) {
            cbase[lc] = ncand;
            ncand += pl.cnt[lc];
        }
        // 3. candidate i: its cutoff, P and free workgroups (one thread each);
        //    workgroups the window heads need at each breakpoint, per cutoff
        if (tid < ncand) {
            int lc = 0, ci = 0;
#pragma unroll
            for (int l = kMaxWindowLevels; l >= 0; --l) {
                const bool in = tid >= cbase[l] && tid < cbase[l] + pl.cnt[l];
                lc = in ? l : lc;
                ci = in ? tid - cbase[l] : ci;
            }
            const int P = ci == 0 ? 1 : ci + 2;
            const int ne = nbh - pl.cum[lc];
            const int fr = cus - ne * (P == 1 ? 1 : P - 1);
            pl.cand_lc[tid] = lc;
            pl.cand_p[tid] = P;
            pl.cand_fr[tid] = fr > 0 ? fr : 0;
        }
        for (int it = tid; it < LV * kMaxBp; it += kThreads) {
            const int lc = 1 + it / kMaxBp, b = it % kMaxBp;
            if (b < pl.off[lc]) {
                const float M = key_float(pl.bkey[b]);
                int need = 0;
                bool ok = true;
#pragma unroll
                for (int m = 1; m <= kMaxWindowLevels; ++m) {
                    const bool act = m <= lc && lcnt[m] > 0;
                    bool bad;
                    const int p = win_segments(N, cw[m - 1], cap[m - 1], M, bad);
                    ok = ok && !(act && bad);
                    need += act ? lcnt[m] * p : 0;
                }
                pl.need[lc - 1][b] = ok ? need : 0x7FFFFFFF;
            }
        }
        lds_barrier();
        // 4. per candidate (one thread each): the smallest feasible breakpoint of
        //    its cutoff and the estimated makespan, in full chunk steps
        int lc = 0, P = 1;
        int pmv[kMaxWindowLevels];
        float t = 3.0e38f;
#pragma unroll
        for (int m = 0; m < kMaxWindowLevels; ++m) pmv[m] = 1;
        if (tid < ncand) {
            lc = pl.cand_lc[tid];
            P = pl.cand_p[tid];
            const int fr = pl.cand_fr[tid];
            const int ne = nbh - pl.cum[lc];
            const int nw = nbh - ne;   // window heads kept
            float te = 0.f;
            if (ne > 0)
                te = P == 1 ? (float)N
                            : 8.f * N * (1.f + kCostPass1) / (kSeg0Weight + 8 * (P - 1)) + (P - 2) * kCostLink;
            float tw = 0.f;
            if (nw > 0 && fr < nw) {
                // fewer workgroups than window heads: one job per head, in rounds;
                // with none free the window heads run after the exact ones
                tw = fr > 0 ? (float)((nw + fr - 1) / fr) * N : te + N;
            } else if (nw > 0) {
                // the breakpoints of levels 1 .. lc; the one with all heads in
                // one segment each is always feasible here (fr >= nw)
                const int* const nd = pl.need[lc - 1];
                const int nb = pl.off[lc];
                int best = 0x7FFFFFFF;
#pragma unroll 8
                for (int b = 0; b < nb; ++b) {
                    const int kk = pl.bkey[b];
                    best = (nd[b] <= fr && kk < best) ? kk : best;
                }
                const float M = key_float(best);
#pragma unroll
                for (int m = 1; m <= kMaxWindowLevels; ++m) {
                    bool bad;
                    const int p = win_segments(N, cw[m - 1], cap[m - 1], M, bad);
                    if (m <= lc && lcnt[m] > 0) {
                        pmv[m - 1] = p;
                        const float f = win_job_cost(N, cw[m - 1], p);
                        tw = f > tw ? f : tw;
                    }
                }
            }
            t = te > tw ? te : tw;
            atomicMin(&pl.tmin, float_key(t));
        }
        lds_barrier();
        if (tid < ncand && t <= key_float(pl.tmin) * 1.001f) atomicMin(&pl.win, tid);
        lds_barrier();
        if (tid == pl.win) {
            pl.pe = P;
            pl.lc = lc;
#pragma unroll
            for (int m = 0; m < kMaxWindowLevels; ++m) pl.pm[m] = pmv[m];
        }
    } else if (tid == 0) {
        pl.pe = pmax;
        pl.lc = LV;
#pragma unroll
        for (int m = 0; m < kMaxWindowLevels; ++m) pl.pm[m] = pmax;
    }
    lds_barrier();
    const int Pe = uni(pl.pe), Lc = uni(pl.lc);
    int pmr[kMaxWindowLevels], nl[kMaxWindowLevels];
#pragma unroll
    for (int m = 1; m <= kMaxWindowLevels; ++m) {
        pmr[m - 1] = pl.pm[m - 1];
        nl[m - 1] = m <= Lc ? lcnt[m] : 0;
    }
    const int n_e = nbh - pl.cum[Lc];
    const int n_w = nbh - n_e;
    // 5. workgroups the window heads leave free go, one segment more per head,
    //    to the heads of the levels whose jobs cost most (levels by job cost,
    //    highest first, ties to the lower level; each takes what is left, up to
    //    its head count): the makespan estimate stays, but far fewer jobs run at
    //    it (job times vary from workgroup to workgroup, so the slowest of many
    //    such jobs sets the end of the launch).  One thread per level.
    if (tid < kMaxWindowLevels) {
        int spare = cus - (n_e == 0 ? 0 : n_e * (Pe == 1 ? 1 : Pe - 1));
        float f[kMaxWindowLevels];
        bool el[kMaxWindowLevels];
#pragma unroll
        for (int m = 1; m <= kMaxWindowLevels; ++m) {
            spare -= nl[m - 1] * pmr[m - 1];
            el[m - 1] = nl[m - 1] > 0 && pmr[m - 1] + 1 <= cap[m - 1];
            f[m - 1] = win_job_cost(N, cw[m - 1], pmr[m - 1]);
        }
        const int m = tid + 1;
        bool mine = el[0];
        float fm = f[0];
#pragma unroll
        for (int k = 1; k < kMaxWindowLevels; ++k) {
            mine = k == tid ? el[k] : mine;
            fm = k == tid ? f[k] : fm;
        }
        int before = 0;
#pragma unroll
        for (int k = 1; k <= kMaxWindowLevels; ++k)
            before += (el[k - 1] && (f[k - 1] > fm || (f[k - 1] == fm && k < m))) ? nl[k - 1] : 0;
        int k = spare - before;
        const int nm = m <= Lc ? pl.lcnt[m] : 0;
        k = k < nm ? k : nm;
        pl.kb[tid] = (forced || !mine || k < 0) ? 0 : k;
    }
    lds_barrier();
    int kbr[kMaxWindowLevels];
    int n_win_jobs = 0, pw = 1;
#pragma unroll
    for (int m = 1; m <= kMaxWindowLevels; ++m) {
        kbr[m - 1] = pl.kb[m - 1];
        n_win_jobs += nl[m - 1] * pmr[m - 1] + kbr[m - 1];
        const int p = pmr[m - 1] + (kbr[m - 1] > 0 ? 1 : 0);
        pw = (nl[m - 1] > 0 && p > pw) ? p : pw;
    }
    // 6. rank the heads by class (exact heads with the levels above Lc, then
    //    levels Lc, .., 1), each class in head order: rounds of one head per
    //    thread, ranks inside a wave from ballots; record the levels that ran
    //    (0 = exact)
    int* const hm = in_lds ? pl.hmap : head_map;
    int cst[kMaxWindowLevels + 1];   // next free slot per class
    cst[0] = 0;
#pragma unroll
    for (int c = 1; c <= kMaxWindowLevels; ++c) cst[c] = n_e + (c <= Lc ? n_w - pl.cum[Lc - c + 1] : 0);
    for (int r0 = 0; r0 < nbh; r0 += kThreads) {
        const int bh = r0 + tid;
        const bool valid = bh < nbh;
        const int m = (valid && wmax) ? (in_lds ? pl.lev[bh] : flags[bh]) : 0;
        const int c = (m == 0 || m > Lc) ? 0 : 1 + Lc - m;
        int rank = 0;
        for (int cc = 0; cc <= Lc; ++cc) {
            const unsigned long long mask = __ballot(valid && c == cc);
            if (lane == 0) pl.rc[wv][cc] = __popcll(mask);
            if (c == cc)
                rank = __builtin_amdgcn_mbcnt_hi((unsigned)(mask >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)mask, 0u));
        }
        lds_barrier();
        int before = 0;
#pragma unroll
        for (int w2 = 0; w2 < kThreads / 64; ++w2) before += w2 < wv ? pl.rc[w2][c] : 0;
        if (valid) {
            int slot = cst[0];
#pragma unroll
            for (int k = 1; k <= kMaxWindowLevels; ++k) slot = k == c ? cst[k] : slot;
            if (in_lds)
                pl.hmap[slot + before + rank] = bh;
            else
                gstore(head_map + slot + before + rank, bh);
            if (wmax && publish) gstore(flags + bh, m > Lc ? 0 : m);
        }
        if (r0 + kThreads < nbh) {
            // the next round's heads come after this round's in every class
            for (int cc = 0; cc <= Lc; ++cc) {
                int n = 0;
#pragma unroll
                for (int w2 = 0; w2 < kThreads / 64; ++w2) n += pl.rc[w2][cc];
#pragma unroll
                for (int k = 0; k <= kMaxWindowLevels; ++k) cst[k] += k == cc ? n : 0;
            }
        }
        lds_barrier();
    }
    const int g_win = n_e + (Pe >= 3 ? n_e * (Pe - 2) : 0);
    const int g_chain = g_win + n_win_jobs;
    const int g_p3 = g_chain + (Pe >= 3 ? 4 * n_e : 0);
    const int n_jobs = g_p3 + (Pe >= 2 ? n_e * (Pe - 1) : 0);
    if (tid == 0) sm.islot[1] = n_jobs;
    if (tid == 0 && publish) {
        gstore(&fp->P_e, Pe);
        gstore(&fp->P_w, pw);
        gstore(&fp->n_exact, n_e);
        gstore(&fp->n_window, n_w);
        gstore(&fp->n_jobs, n_jobs);
    }
    // 7. the job list, one job per thread (segment bounds of exact heads once);
    //    a workgroup that does not publish forms only its own first job
    const int w0 = forced ? 8 : kSeg0Weight;
    const long long den = w0 + 8 * (Pe - 1);
    for (int p = tid; p <= Pe; p += kThreads)
        pl.bound[p] = p <= 0 ? 0 : p >= Pe ? N : seg_bound(w0 + 8 * (p - 1), den, N);
    __syncthreads();
    const int dst_last = has_ht ? DST_HT : DST_NONE;
    const int init0 = has_h0 ? INIT_H0 : INIT_ZERO;
    for (int j = tid; j < n_jobs; j += kThreads) {
        if (!publish && j != (int)blockIdx.x) continue;   // only the workgroup's own first job
        if (j < n_e) {   // segment 0 (or the whole sequence)
            const int bh = hm[j];
            if (Pe == 1)
                put_job(jobs, sm.jrec, publish, j, bh, 0, 0, 0, N, MODE_FULL, init0, dst_last);
            else
                put_job(jobs, sm.jrec, publish, j, bh, 0, 0, 0, pl.bound[1], MODE_FULL, init0, DST_HS_NEXT);
        } else if (j < g_win) {   // pass-1 of segment p, segment-major
            const int p = 1 + (j - n_e) / n_e, e = (j - n_e) % n_e;
            put_job(jobs, sm.jrec, publish, j, hm[e], p, pl.bound[p], pl.bound[p + 1], pl.bound[p + 1], MODE_PASS1,
                    INIT_ZERO, DST_TRANSITION);
        } else if (j < g_chain) {   // window segments, level by level (longest first), head-major
            int jw = j - g_win, hbase = n_e, m = 1;
            bool fnd = false;
#pragma unroll
            for (int mm = kMaxWindowLevels; mm >= 2; --mm) {
                if (mm <= Lc && !fnd) {
                    const int nj = nl[mm - 1] * pmr[mm - 1] + kbr[mm - 1];
                    if (jw < nj) {
                        m = mm;
                        fnd = true;
                    } else {
                        jw -= nj;
                        hbase += nl[mm - 1];
                    }
                }
            }
            int Pm = pmr[0], kb = kbr[0];
            float c = cw[0];
#pragma unroll
            for (int mm = 2; mm <= kMaxWindowLevels; ++mm) {
                Pm = mm == m ? pmr[mm - 1] : Pm;
                kb = mm == m ? kbr[mm - 1] : kb;
                c = mm == m ? cw[mm - 1] : c;
            }
            // the first kb heads of the level have one segment more
            const int W = m * w;
            int P, r, p;
            if (jw < kb * (Pm + 1)) {
                P = Pm + 1;
                r = jw / P;
                p = jw % P;
            } else {
                P = Pm;
                r = kb + (jw - kb * (Pm + 1)) / Pm;
                p = (jw - kb * (Pm + 1)) % Pm;
            }
            const int sb = win_bound(p, P, N, c, forced != 0), e = win_bound(p + 1, P, N, c, forced != 0);
            const int cb = sb - W > 0 ? sb - W : 0;
            put_job(jobs, sm.jrec, publish, j, hm[hbase + r], p, cb, sb, e, MODE_FULL,
                    (cb == 0 && has_h0) ? INIT_H0 : INIT_ZERO, p == P - 1 ? dst_last : DST_NONE);
        } else if (j < g_p3) {   // chain, one job per 32-column block
            const int e = (j - g_chain) / 4, cb = (j - g_chain) % 4;
            put_job(jobs, sm.jrec, publish, j, hm[e], 1, cb, 0, Pe - 1, MODE_CHAIN, 0, 0);
        } else {   // pass-3 of segment p, segment-major
            const int p = 1 + (j - g_p3) / n_e, e = (j - g_p3) % n_e;
            put_job(jobs, sm.jrec, publish, j, hm[e], p, pl.bound[p], pl.bound[p], pl.bound[p + 1], MODE_FULL,
                    INIT_HS_WAIT, p == Pe - 1 ? dst_last : DST_NONE);
        }
    }
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
            e = set_lds(gdn_fwd_queue_kernel<T, false>, lds);
        else if constexpr (PHASE == PHASE_QUEUE_STATES)
            e = set_lds(gdn_fwd_queue_kernel<T, true>, lds);
        else
            e = set_lds(gdn_fwd_kernel<T, PHASE>, lds);
        if (e != hipSuccess) return e;
        configured = true;
    }
    if constexpr (PHASE == PHASE_QUEUE)
        hipLaunchKernelGGL((gdn_fwd_queue_kernel<T, false>), dim3(p.cus), dim3(kThreads), lds, s, p);
    else if constexpr (PHASE == PHASE_QUEUE_STATES)
        hipLaunchKernelGGL((gdn_fwd_queue_kernel<T, true>), dim3(p.cus), dim3(kThreads), lds, s, p);
    else if constexpr (PHASE == PHASE_VARLEN)
        hipLaunchKernelGGL((gdn_fwd_kernel<T, PHASE>), dim3(p.B * p.H * (p.vseg > 0 ? p.P : 1)),
                           dim3(kThreads), lds, s, p);
    else
        hipLaunchKernelGGL((gdn_fwd_kernel<T, PHASE>), dim3(p.B * p.H), dim3(kThreads), lds, s, p);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_fwd_t(const FwdParams& p, int phase, hipStream_t s) {
    if (phase == PHASE_SINGLE) return launch_phase<T, PHASE_SINGLE>(p, s);
    if (phase == PHASE_STATES) return launch_phase<T, PHASE_STATES>(p, s);
    if (phase == PHASE_VARLEN) return launch_phase<T, PHASE_VARLEN>(p, s);
    if (phase == PHASE_STATES_VARLEN) return launch_phase<T, PHASE_STATES_VARLEN>(p, s);
    if (phase == PHASE_QUEUE_STATES) return launch_phase<T, PHASE_QUEUE_STATES>(p, s);
    return launch_phase<T, PHASE_QUEUE>(p, s);
}

}  // namespace

hipError_t launch_fwd(const FwdParams& p, int phase, bool bf16, hipStream_t s) {
    return bf16 ? launch_fwd_t<__bf16>(p, phase, s) : launch_fwd_t<float>(p, phase, s);
}

// Scratch of the forward entry point that allocates nothing
// (gdn_chunk_fwd_noalloc): a fixed array in device memory, one copy per GPU,
// held until the process ends.  In host code `scratch` names a host-side
// stand-in, never the device array: its device address is looked up once per
// device (with that device current) and only that address is handed to
// kernels.
static __device__ __align__(256) unsigned char scratch[kFwdScratchBytes];

namespace {
constexpr int kScratchDevices = 64;
void* g_scratch_ptr[kScratchDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t fwd_scratch(void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr || ((uintptr_t)p & 255u) != 0) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}



}  // namespace gdn
