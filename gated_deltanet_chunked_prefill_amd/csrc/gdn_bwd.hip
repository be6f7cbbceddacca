// Chunked backward of the gated delta rule for gfx950.
//
// Three launches (the first is the forward kernel storing the state entering
// every chunk, see gdn_fwd.hip):
//
//   1. state gradient sweep, one workgroup per head, chunks in reverse order.
//      With dHn the gradient reaching the end of chunk c, the chunk's state step
//      H' = Gamma_C H + K^T diag(E) V' (E_r = Gamma_C / Gamma_r) and output
//      O = scale (diag(Gamma) Q H + P V') give the gradient reaching its start:
//        dV' = scale P^T dO + diag(E) K dHn
//        dY  = Tt^T dV'        (Tt = T diag(beta), transposed block substitution:
//                               dY_1 = Tt_11^T dV'_1, dY_0 = Tt_00^T (dV'_0 - Ah_10^T dY_1))
//        dH  = Gamma_C dHn + scale Q^T diag(Gamma) dO - K^T diag(Gamma) dY
//      The chunk prep (gate scan, inverse blocks, masked Q K^T blocks) is the
//      forward's, run by four prep waves one chunk ahead of the four waves that
//      carry dH in MFMA accumulators.  dHn of every chunk is stored for launch 2.
//
//   2. local gradients, one workgroup per (head, chunk), all chunks at once.
//      From the chunk's entering state H and dHn it recomputes
//      the chunk's forward in gated-matrix form (Sg_rs = Gamma_r / Gamma_s, s <= r;
//      Pm = tril(Q K^T) o Sg, Mg = strict_lower(K K^T) o Sg, T = (I + diag(beta) Mg)^-1,
//      Y = V - diag(Gamma) K H, V' = T diag(beta) Y) and runs reverse mode:
//        dY, dZ as above (dZ = dY / beta before the beta scaling)
//        dPm = scale tril(dO V'^T),  dMg = -strict_lower(dY V'^T)
//        dq  = (dPm o Sg) K + scale diag(Gamma) dO H^T
//        dk  = (dPm o Sg)^T Q + (dMg o Sg + (dMg o Sg)^T) K - diag(Gamma) dY H^T
//              + diag(E) V' dHn^T
//        dv  = dY
//        dbeta_r = dZ_r . (Y - Mg V')_r
//        dgamma_r = sum_s X_rs - sum_s X_sr + q_r . dq2_r + k_r . dk3_r - k_r . dk4_r
//                   (+ <dHn, Hn> for the last position),  X = dPm o Pm + dMg o Mg,
//                   with Hn = Gamma_C H + K^T diag(E) V' the chunk's final state, so
//                   <dHn, Hn> = Gamma_C <dHn, H> + sum_r E_r (K dHn)_r . V'_r
//        dg = reverse cumulative sum of dgamma inside the chunk.
//      The K K^T gradient is bundled as (dA + dA^T) K (FlashQLA talk summary,
//      onedev.kr, paragraph 6); the four chunk steps being inverted are those of
//      paragraph 3.  Exponentials of gamma differences are taken pairwise here
//      (each Sg entry is at most 1), which keeps every factor bounded.
#include "gdn_chunk.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int kDhThreads = 512;     // 4 gradient waves + 4 prep waves
// The reverse sweep runs prep and gradient step back to back, two barriers per
// chunk, with the next chunk's K, Q, dO tiles and gates fetched into a second
// slot during the prep (kDhLoadAhead; deterministic and bit-identical to the
// three-barrier sweep without the fetch ahead).  The fully pipelined schedule
// (prep one chunk ahead of the step, as in the forward) gave run-to-run
// different state gradients from the second chunk on, and is off.
constexpr bool kDhPipelined = false;
constexpr bool kDhLoadAhead = true;
constexpr int kLocalThreads = 256;  // 4 waves
// direct state loads per wave in the local-gradient kernel (four 64 x 128 tiles)
constexpr int kStateLoads = 16;

// ---------------------------------------------------------------------------
// Launch 1: reverse sweep of the state gradient.

// One chunk for gradient wave w (its 32 dv columns of dH).
template <typename T>
__device__ __forceinline__ void dh_chunk_step(const Lane<T>& L, const T* kt, const T* qt, const T* dot,
                                              const T (*t32)[kT32], const float* gam_vec,
                                              const float* e_vec, float GC, float scale, f32x16* dH) {
    using F = typename FragOf<T>::type;
    const int g = L.g, lane = L.lane;
    f32x16 X[2];
    k_times<T>(L, kt, dH, X);   // K dHn
    // P^T dO: (P^T)_00 = P_00^T, (P^T)_01 = P_10^T, (P^T)_11 = P_11^T
    f32x16 pd0 = zero16(), pd1 = zero16();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const F d_lo = L.trV(dot, ks), d_hi = L.trV(dot, 2 + ks);
        pd0 = mma(tfrag<T, 32>(t32[3], 0, ks, lane), d_lo, pd0);
        pd0 = mma(tfrag<T, 32>(t32[4], 0, ks, lane), d_hi, pd0);
        pd1 = mma(tfrag<T, 32>(t32[5], 0, ks, lane), d_hi, pd1);
    }
    const f32x16 e0 = rows_of(e_vec, 0, g), e1 = rows_of(e_vec, 1, g);
    f32x16 dvp0, dvp1;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        dvp0[r] = scale * pd0[r] + e0[r] * X[0][r];
        dvp1[r] = scale * pd1[r] + e1[r] * X[1][r];
    }
    // transposed block substitution through Tt = T diag(beta)
    f32x16 dy1 = zero16();
    dy1 = mma(tfrag<T, 32>(t32[1], 0, 0, lane), acc_frag<T>(dvp1, 0), dy1);
    dy1 = mma(tfrag<T, 32>(t32[1], 0, 1, lane), acc_frag<T>(dvp1, 1), dy1);
    f32x16 z0 = dvp0;   // + (-Ah_10)^T dY_1
    z0 = mma(tfrag<T, 32>(t32[2], 0, 0, lane), acc_frag<T>(dy1, 0), z0);
    z0 = mma(tfrag<T, 32>(t32[2], 0, 1, lane), acc_frag<T>(dy1, 1), z0);
    f32x16 dy0 = zero16();
    dy0 = mma(tfrag<T, 32>(t32[0], 0, 0, lane), acc_frag<T>(z0, 0), dy0);
    dy0 = mma(tfrag<T, 32>(t32[0], 0, 1, lane), acc_frag<T>(z0, 1), dy0);
    // dH <- Gamma_C dH - K^T diag(Gamma) dY + scale Q^T diag(Gamma) dO
    F bk[4], bq[4];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const f32x16 gr = rows_of(gam_vec, rt, g);
        const f32x16& dy = rt ? dy1 : dy0;
        const F d0 = L.trV(dot, 2 * rt), d1 = L.trV(dot, 2 * rt + 1);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            bk[2 * rt][j] = (T)(-gr[j] * dy[j]);
            bk[2 * rt + 1][j] = (T)(-gr[8 + j] * dy[8 + j]);
            bq[2 * rt][j] = (T)(scale * gr[j] * (float)d0[j]);
            bq[2 * rt + 1][j] = (T)(scale * gr[8 + j] * (float)d1[j]);
        }
    }
    kt_update<T>(L, kt, dH, GC, bk);
    kt_update<T>(L, qt, dH, 1.f, bq);
}

// The linear part of one chunk's step, for the segment maps of the split sweep:
// dH <- Gamma_C dH - K^T diag(Gamma) dY with dY from dV' = diag(E) K dH alone
// (the chunk map of dh_chunk_step with dO = 0).
template <typename T>
__device__ __forceinline__ void dh_map_step(const Lane<T>& L, const T* kt, const T (*t32)[kT32],
                                            const float* gam_vec, const float* e_vec, float GC, f32x16* M) {
    using F = typename FragOf<T>::type;
    const int g = L.g, lane = L.lane;
    f32x16 X[2];
    k_times<T>(L, kt, M, X);   // K M
    const f32x16 e0 = rows_of(e_vec, 0, g), e1 = rows_of(e_vec, 1, g);
    f32x16 dvp0, dvp1;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        dvp0[r] = e0[r] * X[0][r];
        dvp1[r] = e1[r] * X[1][r];
    }
    f32x16 dy1 = zero16();
    dy1 = mma(tfrag<T, 32>(t32[1], 0, 0, lane), acc_frag<T>(dvp1, 0), dy1);
    dy1 = mma(tfrag<T, 32>(t32[1], 0, 1, lane), acc_frag<T>(dvp1, 1), dy1);
    f32x16 z0 = dvp0;
    z0 = mma(tfrag<T, 32>(t32[2], 0, 0, lane), acc_frag<T>(dy1, 0), z0);
    z0 = mma(tfrag<T, 32>(t32[2], 0, 1, lane), acc_frag<T>(dy1, 1), z0);
    f32x16 dy0 = zero16();
    dy0 = mma(tfrag<T, 32>(t32[0], 0, 0, lane), acc_frag<T>(z0, 0), dy0);
    dy0 = mma(tfrag<T, 32>(t32[0], 0, 1, lane), acc_frag<T>(z0, 1), dy0);
    F bk[4];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const f32x16 gr = rows_of(gam_vec, rt, g);
        const f32x16& dy = rt ? dy1 : dy0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            bk[2 * rt][j] = (T)(-gr[j] * dy[j]);
            bk[2 * rt + 1][j] = (T)(-gr[8 + j] * dy[8 + j]);
        }
    }
    kt_update<T>(L, kt, M, GC, bk);
}

// Chunk tile for loader wave lw (0, 1) of the sweep's segment maps, by buffer
// loads into LDS with the lane offsets formed per call: no offset registers stay
// live across the chunk loop, where the prep waves also hold their 32 columns of
// M (the fetch-ahead loader's offsets were spilled there).  The same slots as
// TileLoader<T, 2>; a short chunk goes through registers, zero past its end.
template <typename T>
__device__ __forceinline__ void dh_load_tile(T* tile, const T* chunk, int nv, int H, int lw) {
    static_assert(sizeof(T) == 2, "bf16 tiles");
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));   // offsets per call, not hoisted out of the chunk loop
    const int rb = H * kDk * (int)sizeof(T);   // bytes between rows
    if (nv == kChunk) {
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(chunk), (short)0, kChunk * rb, 0x00020000);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            // slots (2 i + lw) * 64 + lane: row 8 i + 4 lw + lane / 16, piece lane % 16
            const int row = 8 * i + 4 * lw + (lane >> 4);
            const int voff = (4 * lw + (lane >> 4)) * rb + (((lane & 15) ^ swz16(row)) << 4);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs, (__attribute__((address_space(3))) void*)(tile + (2 * i + lw) * 64 * 8), 16, voff, 8 * i * rb, 0,
                kCpolStream);
        }
    } else {
        typedef uint32_t u4 __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int L = (2 * i + lw) * 64 + lane, row = L >> 4, slot = L & 15;
            u4 v = {0u, 0u, 0u, 0u};
            if (row < nv)
                v = *(const __attribute__((address_space(1))) u4*)((const char*)chunk + (size_t)row * rb +
                                                                    ((slot ^ swz16(row)) << 4));
            *(u4*)(tile + L * 8) = v;
        }
    }
}

// Gradient waves: carry dH over chunks c1 - 1 down to c0 of head bh.  The start
// is dht (in_slot < 0) or the b field of workspace slot in_slot; PASS1 starts
// from zero and stores no per-chunk gradients (the segment's b).  At the end the
// gradient goes to the b field of slot out_slot (>= 0), to dh0 (-1) or nowhere
// (-2).  Executes exactly the same barriers as dh_prep_loop.
template <typename T, bool PASS1 = false>
__device__ __noinline__ void dh_state_loop(const BwdParams& prm, Smem<T>& sm, int bh, int c0, int c1, int in_slot,
                                           int out_slot) {
    static_assert(!PASS1 || kDhLoadAhead, "segment maps are built with the fetch-ahead sweep only");
    bh = uni(bh), c0 = uni(c0), c1 = uni(c1), in_slot = uni(in_slot), out_slot = uni(out_slot);
    constexpr bool kPipe = kDhPipelined;
    const size_t SS = (size_t)kDk * kDv;
    const int N = uni(prm.N);
    const int n = c1 - c0;
    const float scale = uni(prm.scale);
    __bf16* const dst = uni(prm.dhstore) + (size_t)bh * N * SS;
    const float* const dht = uni(prm.dht);
    float* const dh0 = uni(prm.dh0);
    float* const ws = uni(prm.ws);
    const int P = uni(prm.P);
    Lane<T> L;
    L.init(threadIdx.x);
    f32x16 dH[4];
    if (!PASS1 && in_slot >= 0) {
        load_state(ws + ((size_t)bh * P + in_slot) * kStateSlot + kDk * kDk, L.w, L.lane, dH);
    } else if (!PASS1 && dht) {
        load_state(dht + (size_t)bh * SS, L.w, L.lane, dH);
    } else {
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) dH[ht] = zero16();
    }
    if constexpr (kPipe) {
        lds_barrier();
        lds_barrier();
        for (int i = 0; i < n; ++i) {
            const int c = c1 - 1 - i;
            const int slot = i % 3, vb = i & 1;
            store_state_bf16t(uni(dst + (size_t)c * SS), L.w, L.lane, dH);
            dh_chunk_step<T>(L, sm.kt[slot], sm.qt[slot], sm.vt[vb], sm.t32[vb], sm.gam_vec[vb],
                             sm.e_vec[vb], sm.gc[vb][0], scale, dH);
            lds_barrier();
        }
    } else if constexpr (kDhLoadAhead) {
        for (int i = 0; i < n; ++i) {
            const int c = c1 - 1 - i;
            const int slot = i & 1;
            lds_barrier();   // A
            lds_barrier();   // B
            if (!PASS1) store_state_bf16t(uni(dst + (size_t)c * SS), L.w, L.lane, dH);
            dh_chunk_step<T>(L, sm.kt[slot], sm.qt[slot], sm.vt[slot], sm.t32[0], sm.gam_vec[0], sm.e_vec[0],
                             sm.gc[0][0], scale, dH);
        }
    } else {
        for (int i = 0; i < n; ++i) {
            const int c = c1 - 1 - i;
            lds_barrier();
            lds_barrier();
            lds_barrier();
            store_state_bf16t(uni(dst + (size_t)c * SS), L.w, L.lane, dH);
            dh_chunk_step<T>(L, sm.kt[0], sm.qt[0], sm.vt[0], sm.t32[0], sm.gam_vec[0], sm.e_vec[0],
                             sm.gc[0][0], scale, dH);
        }
    }
    if (out_slot >= 0)
        store_state(ws + ((size_t)bh * P + out_slot) * kStateSlot + kDk * kDk, L.w, L.lane, dH);
    else if (out_slot == -1 && dh0)
        store_state(uni(dh0 + (size_t)bh * SS), L.w, L.lane, dH);
}

// Prep waves: stream K, Q, dO of chunks c1 - 1 down to c0 and prep each one
// ahead of the gradient waves.  In PASS1 they also carry the segment's map M
// from the identity, 32 columns each, after the blocks of a chunk are written
// (the gradient waves' step reads the same buffers), and store it in the M
// field of slot out_slot.  Executes exactly the same barriers as dh_state_loop.
template <typename T, bool PASS1 = false>
__device__ __noinline__ void dh_prep_loop(const BwdParams& prm, Smem<T>& sm, int bh, int c0, int c1, int out_slot) {
    static_assert(!PASS1 || kDhLoadAhead, "segment maps are built with the fetch-ahead sweep only");
    bh = uni(bh), c0 = uni(c0), c1 = uni(c1), out_slot = uni(out_slot);
    constexpr bool kPipe = kDhPipelined;
    const int pw = wave_id() - 4;
    const int H = uni(prm.H), Tn = uni(prm.T);
    const int N = c1 - c0;   // chunks of this range
    const int b = bh / H, h = bh % H;
    const T* const q = uni((const T*)prm.q);
    const T* const k = uni((const T*)prm.k);
    const T* const dout = uni((const T*)prm.dout);
    const float* const gp = uni(prm.g);
    const float* const bp = uni(prm.beta);
    Lane<T> L;
    L.init(threadIdx.x);
    float gsum = 0.f;
    float g_cur = 0.f, b_cur = 0.f, g_nxt = 0.f, b_nxt = 0.f;
    auto cidx = [&](int i) { return c1 - 1 - i; };
    f32x16 Ms[4];
    if (PASS1) {
#pragma unroll
        for (int ht = 0; ht < 4; ++ht)
#pragma unroll
            for (int r = 0; r < 16; ++r) Ms[ht][r] = (32 * ht + rho(L.g, r) == 32 * L.w + L.n) ? 1.f : 0.f;
    }
    // with the fetch ahead, prep waves 2 and 3 issue every tile load, so waves 0
    // and 1 (the diagonal inverses, the longest prep work) never wait on the
    // memory pipeline; otherwise all four load their quarter
    constexpr int kLoaders = kDhLoadAhead ? 2 : 4;
    const bool loader = pw >= 4 - kLoaders;
    TileLoader<T, kLoaders> TL;
    if (!PASS1 && loader) TL.init(pw - (4 - kLoaders), L.lane, H);
    auto load_kq = [&](int c, int slot) {
        if (!loader) return;
        const size_t cb = chunk_base(b, h, Tn, H, c);
        const int nv = chunk_len(Tn, c);
        if constexpr (PASS1) {
            dh_load_tile<T>(sm.kt[slot], k + cb, nv, H, pw - 2);
            dh_load_tile<T>(sm.qt[slot], q + cb, nv, H, pw - 2);
        } else {
            TL.load(sm.kt[slot], k + cb, nv);
            TL.load(sm.qt[slot], q + cb, nv);
        }
    };
    auto load_do = [&](int c, int slot) {
        if (!loader) return;
        if constexpr (PASS1)
            dh_load_tile<T>(sm.vt[slot], dout + chunk_base(b, h, Tn, H, c), chunk_len(Tn, c), H, pw - 2);
        else
            TL.load(sm.vt[slot], dout + chunk_base(b, h, Tn, H, c), chunk_len(Tn, c));
    };
    if constexpr (kPipe) {
        load_kq(cidx(0), 0);
        load_do(cidx(0), 0);
        if (N > 1) load_kq(cidx(1), 1);
        load_gate_beta(gp, bp, Tn, H, b, h, cidx(0), L.lane, g_cur, b_cur);
        if (N > 1) load_gate_beta(gp, bp, Tn, H, b, h, cidx(1), L.lane, g_nxt, b_nxt);
        wait_vm();
        lds_barrier();
        chunk_prep<T, MODE_FULL>(sm, L, pw, sm.kt[0], sm.qt[0], sm.t32[0], sm.gam_vec[0], sm.e_vec[0],
                                 sm.gc[0], g_cur, b_cur, true, gsum);
        g_cur = g_nxt;
        b_cur = b_nxt;
        lds_barrier();
        for (int i = 0; i < N; ++i) {
            if (i + 1 < N) {
                if (i + 2 < N) {
                    load_kq(cidx(i + 2), (i + 2) % 3);
                    load_gate_beta(gp, bp, Tn, H, b, h, cidx(i + 2), L.lane, g_nxt, b_nxt);
                }
                load_do(cidx(i + 1), (i + 1) & 1);
                const int slot = (i + 1) % 3, pb = (i + 1) & 1;
                chunk_prep<T, MODE_FULL>(sm, L, pw, sm.kt[slot], sm.qt[slot], sm.t32[pb],
                                         sm.gam_vec[pb], sm.e_vec[pb], sm.gc[pb], g_cur, b_cur, true,
                                         gsum);
                g_cur = g_nxt;
                b_cur = b_nxt;
                wait_vm();
            }
            lds_barrier();
        }
    } else if constexpr (kDhLoadAhead) {
        // chunk i + 1's tiles and gates are fetched into the other slot while
        // chunk i is prepped; prep and gradient step stay in sequence
        if (N > 0) {
            load_kq(cidx(0), 0);
            load_do(cidx(0), 0);
            load_gate_beta(gp, bp, Tn, H, b, h, cidx(0), L.lane, g_nxt, b_nxt);
            wait_vm();
        }
        for (int i = 0; i < N; ++i) {
            const int slot = i & 1;
            lds_barrier();   // A: the gradient step of chunk i - 1 is done with the buffers
            g_cur = g_nxt;
            b_cur = b_nxt;
            if (i + 1 < N) {
                load_kq(cidx(i + 1), slot ^ 1);
                load_do(cidx(i + 1), slot ^ 1);
                load_gate_beta(gp, bp, Tn, H, b, h, cidx(i + 1), L.lane, g_nxt, b_nxt);
            }
            chunk_prep<T, MODE_FULL>(sm, L, pw, sm.kt[slot], sm.qt[slot], sm.t32[0], sm.gam_vec[0],
                                     sm.e_vec[0], sm.gc[0], g_cur, b_cur, true, gsum);
            wait_vm();
            lds_barrier();   // B: prep of chunk i and the tiles of chunk i + 1 are in LDS
            if (PASS1) dh_map_step<T>(L, sm.kt[slot], sm.t32[0], sm.gam_vec[0], sm.e_vec[0], sm.gc[0][0], Ms);
        }
    } else {
        for (int i = 0; i < N; ++i) {
            const int c = cidx(i);
            lds_barrier();
            load_kq(c, 0);
            load_do(c, 0);
            load_gate_beta(gp, bp, Tn, H, b, h, c, L.lane, g_cur, b_cur);
            wait_vm();
            lds_barrier();
            chunk_prep<T, MODE_FULL>(sm, L, pw, sm.kt[0], sm.qt[0], sm.t32[0], sm.gam_vec[0],
                                     sm.e_vec[0], sm.gc[0], g_cur, b_cur, true, gsum);
            lds_barrier();
        }
    }
    if (PASS1) store_state(uni(prm.ws) + ((size_t)bh * uni(prm.P) + out_slot) * kStateSlot, L.w, L.lane, Ms);
}

// DH_FULL: workgroup = head, all chunks.  DH_FIRST: per head P - 1 workgroups;
// j = 0 runs segment P-1 from dht (its gradients stored, the gradient at its
// start to slot P-1), j >= 1 builds the map of segment P-1-j.  DH_REST: per head
// P - 1 workgroups; j runs segment j from the gradient at its end (slot j + 1).
template <typename T, int MODE>
__global__ __launch_bounds__(kDhThreads, 1) void gdn_bwd_dh_kernel(BwdParams prm) {
    extern __shared__ __attribute__((aligned(16))) char smem_raw[];
    Smem<T>& sm = *reinterpret_cast<Smem<T>*>(smem_raw);
    const int groups = MODE == DH_FULL ? 1 : prm.P - 1;
    const int bh = (int)blockIdx.x / groups, j = (int)blockIdx.x % groups;
    int seg = 0, c0 = 0, c1 = prm.N, in_slot = -1, out_slot = -1;
    if (MODE == DH_FIRST) {
        seg = prm.P - 1 - j;
        out_slot = seg;
    } else if (MODE == DH_REST) {
        seg = j;
        in_slot = seg + 1;
        out_slot = seg == 0 ? -1 : -2;
    }
    if (MODE != DH_FULL) {
        c0 = seg * prm.S;
        c1 = min(c0 + prm.S, prm.N);
    }
    const bool map = MODE == DH_FIRST && j > 0;
    // wave-uniform role branch: both roles hold barriers
    if (wave_id() < 4) {
        if (map)
            dh_state_loop<T, true>(prm, sm, bh, c0, c1, in_slot, out_slot);
        else
            dh_state_loop<T>(prm, sm, bh, c0, c1, in_slot, out_slot);
    } else {
        if (map)
            dh_prep_loop<T, true>(prm, sm, bh, c0, c1, out_slot);
        else
            dh_prep_loop<T>(prm, sm, bh, c0, c1, out_slot);
    }
}

// Packed sequences: parameters of sequence s, head h as one sequence of a batch
// of sequences of its length.  Every token pointer is shifted by t0 - s*len
// tokens (the kernels' token index s*len + t then addresses token t0 + t), and
// the stored-state pointers so that slot bh*(nch+1) + c (states) and bh*nch + c
// (state gradients) address the sequence's own slots.
__device__ __forceinline__ void varlen_bwd_params(BwdParams& p, int s, int h, size_t elem) {
    const SeqSpan sp = seq_span(p.cu, p.cstart, p.B, p.T, s);
    const long long rows = ((long long)sp.t0 - (long long)s * sp.len) * p.H;   // token-head rows
    const long long vb = rows * kDk * (long long)elem;                          // bytes of q, k, v rows
    p.q = (const char*)p.q + vb;
    p.k = (const char*)p.k + vb;
    p.v = (const char*)p.v + vb;
    p.dout = (const char*)p.dout + vb;
    p.dq = (char*)p.dq + vb;
    p.dk = (char*)p.dk + vb;
    p.dv = (char*)p.dv + vb;
    p.g += rows;
    p.beta += rows;
    p.dg += rows;
    p.dbeta += rows;
    const long long bh = (long long)s * p.H + h;
    const long long SS = (long long)kDk * kDv;
    p.hstore += ((long long)h * (p.cmax + p.B) + sp.c0 + s - bh * (sp.nch + 1)) * SS;
    p.dhstore += ((long long)h * p.cmax + sp.c0 - bh * sp.nch) * SS;
    p.T = sp.len;
    p.N = sp.nch;
}

template <typename T>
__global__ __launch_bounds__(kDhThreads, 1) void gdn_bwd_dh_varlen_kernel(BwdParams prm_in) {
    extern __shared__ __attribute__((aligned(16))) char smem_raw[];
    Smem<T>& sm = *reinterpret_cast<Smem<T>*>(smem_raw);
    const int bh = blockIdx.x;
    BwdParams prm = prm_in;
    varlen_bwd_params(prm, bh / prm_in.H, bh % prm_in.H, sizeof(T));
    if (wave_id() < 4)
        dh_state_loop<T>(prm, sm, bh, 0, prm.N, -1, -1);
    else
        dh_prep_loop<T>(prm, sm, bh, 0, prm.N, -1);
}

// Packed sequences, one workgroup, 256 bounds per round with running carries:
// the bounds bnd[s] = max(0, clamp(cu[0]), .., clamp(cu[s])) (s = 0 .. B, a
// prefix maximum, so sequence s = [bnd[s], bnd[s+1]) never overlaps another)
// into cstart[B + 1 + s], and the chunk prefix cstart[s] = chunks of sequences
// 0 .. s-1 (s = 0 .. B).
__global__ __launch_bounds__(256) void seq_chunk_prefix_kernel(const int* __restrict__ cu, int B, int T,
                                                               int* __restrict__ cstart) {
    __shared__ int part[256];
    __shared__ int bnd[257];
    int* const bout = cstart + B + 1;
    const int tid = threadIdx.x;
    int carry = 0, lastb = 0;   // chunks before this round; the bound before this round
    for (int s0 = 0; s0 <= B; s0 += 256) {
        const int s = s0 + tid;   // bound index; sequence s - 1 ends at bound s
        part[tid] = s <= B ? clamp_tok(cu[s], 0, T) : 0;
        __syncthreads();
        for (int d = 1; d < 256; d <<= 1) {   // inclusive maximum scan
            const int x = tid >= d ? part[tid - d] : 0;
            __syncthreads();
            part[tid] = part[tid] > x ? part[tid] : x;
            __syncthreads();
        }
        const int b = part[tid] > lastb ? part[tid] : lastb;
        if (s <= B) bout[s] = b;
        bnd[tid + 1] = b;
        if (tid == 0) bnd[0] = lastb;
        __syncthreads();
        const int nch = (s >= 1 && s <= B) ? (bnd[tid + 1] - bnd[tid] + 63) / 64 : 0;
        part[tid] = nch;
        __syncthreads();
        for (int d = 1; d < 256; d <<= 1) {   // inclusive scan
            const int x = tid >= d ? part[tid - d] : 0;
            __syncthreads();
            part[tid] += x;
            __syncthreads();
        }
        if (s >= 1 && s <= B) cstart[s - 1] = carry + part[tid] - nch;
        carry += part[255];
        lastb = bnd[256];
        __syncthreads();
    }
    if (tid == 0) cstart[B] = carry;
}

// ---------------------------------------------------------------------------
// Launch 2: local gradients of every chunk.

constexpr int kT64 = 64 * 64;

template <typename T>
struct LocalSmem {
    T qt[kChunk * kDk];     // 64 x 128 tiles (swizzled row-major, as in the forward)
    T kt[kChunk * kDk];
    T vt[kChunk * kDv];     // V, then V'
    T dot[kChunk * kDv];    // dO
    // the 64 x 64 score tiles Pm, Mg and the diagonal blocks of the gated
    // inverse (phases 1-2), then dY as a 64 x 128 tile
    T sc[3 * kT64];
    // the chunk's entering state and its gradient, stored layout [dv][dk], as
    // four 64 x 128 tiles (rows dv 0-63, 64-127 of each), then the gradient
    // tiles dPm o Sg, dMg o Sg
    T stt[4 * kChunk * kDk];
    float gst[2][kChunk];           // g and beta of the chunk as loaded (zero past the end)
    float gam[kChunk];
    float Gam[kChunk];
    float E[kChunk];
    float beta[kChunk];
    float part[4][4][kChunk];       // per wave: dbeta, q.dq2, k.dk3, k.dk4 partial row sums
    float xrow[4][32];              // per wave: row sums of its 32 x 32 tile of X = dPm o Pm + dMg o Mg
    float xcol[4][32];              // per wave: column sums of that tile
    float red[4];
    __device__ T* pm() { return sc; }
    __device__ T* mg() { return sc + kT64; }
    __device__ T* tg() { return sc + 2 * kT64; }    // diagonal blocks of the gated inverse T (beta-free)
    __device__ T* dyt() { return sc; }
    __device__ T* st(int i) { return stt + i * kChunk * kDk; }   // 0, 1: H; 2, 3: dHn
    __device__ T* dpg() { return stt; }             // dPm o Sg
    __device__ T* dmg() { return stt + kT64; }      // dMg o Sg
    __device__ const T* pm() const { return sc; }
    __device__ const T* mg() const { return sc + kT64; }
    __device__ const T* tg() const { return sc + 2 * kT64; }
};
static_assert(sizeof(LocalSmem<__bf16>) <= 160 * 1024, "local-gradient LDS exceeds a CU's 160 KB");

// B fragment of a stored state (bf16, transposed [dv][dk]), contraction over
// its dk rows, in the column order of the 16-byte tile fragments: lane (n, g)
// gets S[16ks + 8g + j][col], j = 0..7, one 16-byte load.
template <typename T>
__device__ __forceinline__ typename FragOf<T>::type state_colfrag(const __bf16* St, int ks, int g, int col) {
    static_assert(sizeof(T) == 2, "the backward is built for bf16 only");
    typedef __attribute__((address_space(1))) const typename FragOf<T>::type gfrag;
    return *(gfrag*)(St + (size_t)col * kDk + 16 * ks + 8 * g);
}
// Transposed fragment of a 64 x 128 LDS tile in the contraction order of the
// 16-byte tile fragments: lane (n, g) gets tile[16 ks + 8 g + j][nbase + n],
// j = 0..7 (two ds_read_b64_tr_b16, each giving four consecutive rows).
template <typename T>
__device__ __forceinline__ typename FragOf<T>::type tfrag_nat(const T* tile, int nbase, int ks, int lane) {
    static_assert(sizeof(T) == 2, "the backward is built for bf16 only");
    typedef short s4 __attribute__((ext_vector_type(4)));
    const int g = lane >> 5, i = lane & 15, n0 = nbase + (lane & 16);
    typename FragOf<T>::type f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const T* p = tile + toff<T, kDk>(16 * ks + 8 * g + 4 * h + (i >> 2), n0 + 4 * (i & 3));
        const s4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s4*)(__attribute__((address_space(3))) void*)p);
        const typename Quad<T>::type q = __builtin_bit_cast(typename Quad<T>::type, r);
#pragma unroll
        for (int j = 0; j < 4; ++j) f[4 * h + j] = q[j];
    }
    return f;
}

// Sum of each accumulator row over the 32 lanes of its half-wave, written to
// dst[32 rt + rho(g, r)].  A reduce-scatter: each exchange halves the registers a
// lane carries (it keeps the half its partner does not), so 16 rows cost 8
// v_permlane16_swap (lanes n, n ^ 16) and 15 DPP moves (partners n ^ 8, n ^ 7,
// n ^ 2, n ^ 1) instead of a five-step butterfly per row.  Afterwards lanes
// n and n ^ 1 hold the sum of register n >> 1; the even lane writes it.
__device__ __forceinline__ void row_sums(float* dst, const f32x16& v, int rt, int g, int n) {
    float a[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        // even rows of 16 keep registers 0..7, odd rows 8..15: the swap hands the
        // odd row its partner's register i + 8 and the even row its partner's i
        // (__builtin_bit_cast of a vector element reads element 0 with this
        // toolchain; the intrinsic conversions take the element's value)
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]), __float_as_uint(v[i + 8]),
                                                        false, false);
        a[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    const bool b3 = (n >> 3) & 1, b2 = (n >> 2) & 1, b1 = (n >> 1) & 1;
    float b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float send = b3 ? a[i] : a[i + 4];
        const float keep = b3 ? a[i + 4] : a[i];
        b[i] = keep + dpp_take<0x128, 0xf>(send);   // row_ror:8, lane n ^ 8
    }
    float c[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const float send = b2 ? b[i] : b[i + 2];
        const float keep = b2 ? b[i + 2] : b[i];
        c[i] = keep + dpp_take<0x141, 0xf>(send);   // row_half_mirror, lane n ^ 7
    }
    const float send = b1 ? c[0] : c[1];
    const float keep = b1 ? c[1] : c[0];
    float d = keep + dpp_take<0x4e, 0xf>(send);     // quad_perm [2,3,0,1], lane n ^ 2
    d += dpp_take<0xb1, 0xf>(d);                    // quad_perm [1,0,3,2], lane n ^ 1
    if ((n & 1) == 0) dst[32 * rt + rho(g, n >> 1)] = d;
}

// Column sums of an accumulator tile (over its 32 rows, both half-waves):
// written by the g = 0 half to dst[n].
__device__ __forceinline__ void col_sums(float* dst, const f32x16& v, int g, int n) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += v[r];
    const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
    // x[0] holds, in the upper half-wave, the lower half's value; x[1] the reverse
    const float other = __uint_as_float(g ? x[0] : x[1]);
    if (g == 0) dst[n] = s + other;
}

// Store an accumulator tile (rows 32 ti + rho, column 32 tj + n) into a 64 x 64 tile.
template <typename T>
__device__ __forceinline__ void st_tile64(T* tile, const f32x16& v, int ti, int tj, int g, int n) {
#pragma unroll
    for (int r = 0; r < 16; ++r) tile[toff<T, 64>(32 * ti + rho(g, r), 32 * tj + n)] = (T)v[r];
}

// Store accumulator tile rt of a 64 x 128 result (this wave's 32 columns) into a
// swizzled 64 x 128 LDS tile.
template <typename T>
__device__ __forceinline__ void st_rows_lds(T* tile, const f32x16& v, int rt, int g, int n, int w) {
#pragma unroll
    for (int r = 0; r < 16; ++r) tile[toff<T, kDv>(32 * rt + rho(g, r), 32 * w + n)] = (T)v[r];
}

// Store the 32 values of a transposed accumulator tile that belong to one row:
// lane (n, g) holds columns 8i + 4g .. +3 (i = 0..3) of its row; two lane swaps
// between the half-waves give it columns 8g .. +7 and 16 + 8g .. +7, stored as
// two 16-byte pieces at row + 8g and row + 16 + 8g (when valid).
template <typename T>
__device__ __forceinline__ void store_row_pieces(T* row, const f32x16& v, int g, bool valid) {
    static_assert(sizeof(T) == 2, "the backward is built for bf16 only");
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    uint32_t pk[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const b2 pr = {(__bf16)v[2 * k], (__bf16)v[2 * k + 1]};
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
    if (valid) {
        typedef uint32_t u4 __attribute__((ext_vector_type(4)));
        typedef __attribute__((address_space(1))) u4 gu4;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const u4 x = {pk[4 * q], pk[4 * q + 1], pk[4 * q + 2], pk[4 * q + 3]};
            *(gu4*)(row + 16 * q + 8 * g) = x;
        }
    }
}

// Copy the first nv rows of a swizzled 64 x 128 LDS tile to the rows of a
// [.., T, H, 128] tensor (dst = the chunk's first row of this head), as
// 16-byte row pieces: 1024 pieces over the workgroup's threads.
template <typename T>
__device__ __forceinline__ void copy_tile_rows(T* dst, const T* tile, int H, int nv, int tid) {
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(1))) u4 gu4;
#pragma unroll
    for (int i = tid; i < kChunk * 16; i += kLocalThreads) {
        const int row = i >> 4, ch = i & 15;
        if (row < nv) {
            const u4 x = *reinterpret_cast<const u4*>(tile + toff<T, kDv>(row, 8 * ch));
            *(gu4*)(dst + (size_t)row * H * kDv + 8 * ch) = x;
        }
    }
}

// Tile (ti, tj) of the gated score matrices, ti >= tj: Pm = tril(Q K^T) o Sg and
// Mg = strict_lower(K K^T) o Sg with Sg_rs = exp(gamma_r - gamma_s) (s <= r), in
// accumulator form (rows 32 ti + rho, column 32 tj + n); skk returns the raw K K^T
// tile.  Recomputed where needed rather than carried in registers between phases.
template <typename T>
__device__ __forceinline__ void score_tiles(const Lane<T>& L, const LocalSmem<T>& sm, int ti, int tj,
                                            f32x16& Pm, f32x16& Mg, f32x16& SG, f32x16& skk) {
    using F = typename FragOf<T>::type;
    const int n = L.n, g = L.g;
    f32x16 sqk = zero16();
    skk = zero16();
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        const F kf = L.f128(sm.kt, tj, ks);
        sqk = mma(L.f128(sm.qt, ti, ks), kf, sqk);
        skk = mma(L.f128(sm.kt, ti, ks), kf, skk);
    }
    const f32x16 gr = rows_of(sm.gam, ti, g);
    const float gs = sm.gam[32 * tj + n];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int R = 32 * ti + rho(g, r), S = 32 * tj + n;
        const float sg = R >= S ? __expf(gr[r] - gs) : 0.f;
        SG[r] = sg;
        Pm[r] = sqk[r] * sg;
        Mg[r] = R > S ? skk[r] * sg : 0.f;
    }
}

// The local gradients of chunk c of head bh (one workgroup).
template <typename T>
__device__ __forceinline__ void local_body(const BwdParams& prm, int bh, int c) {
    using F = typename FragOf<T>::type;
    extern __shared__ __attribute__((aligned(16))) char smem_raw[];
    LocalSmem<T>& sm = *reinterpret_cast<LocalSmem<T>*>(smem_raw);
    const int H = prm.H, Tn = prm.T, N = prm.N;
    const int b = bh / H, h = bh % H;
    const int t0 = c * kChunk, nv = chunk_len(Tn, c);
    const int tid = threadIdx.x;
    const int w = wave_id();
    Lane<T> L;
    L.init(tid);
    const int lane = L.lane, n = L.n, g = L.g;
    const float scale = prm.scale;
    const size_t SS = (size_t)kDk * kDv;
    const __bf16* const Hc = prm.hstore + ((size_t)bh * (N + 1) + c) * SS;
    const __bf16* const dHn = prm.dhstore + ((size_t)bh * N + c) * SS;

    // ---- phase 0: g and beta, the tiles, then the entering state and its
    // gradient (not read before phase 2: their latency runs under phase 1).
    // Every full-chunk load goes straight to LDS, so no register waits on them.
    if (w == 0) {
        const size_t e0 = ((size_t)b * Tn + t0) * H + h;
        if (nv == kChunk) {
            __builtin_amdgcn_global_load_lds((const void*)(prm.g + e0 + (size_t)lane * H),
                                             (__attribute__((address_space(3))) void*)&sm.gst[0][0], 4, 0,
                                             kCpolStream);
            __builtin_amdgcn_global_load_lds((const void*)(prm.beta + e0 + (size_t)lane * H),
                                             (__attribute__((address_space(3))) void*)&sm.gst[1][0], 4, 0,
                                             kCpolStream);
        } else {
            float gv = 0.f, bv = 0.f;
            load_gate_beta(prm.g, prm.beta, Tn, H, b, h, c, lane, gv, bv);
            sm.gst[0][lane] = gv;
            sm.gst[1][lane] = bv;
        }
    }
    {
        TileLoader<T> TL;
        TL.init(w, lane, H);
        const size_t cb = chunk_base(b, h, Tn, H, c);
        TL.load(sm.qt, (const T*)prm.q + cb, nv);
        TL.load(sm.kt, (const T*)prm.k + cb, nv);
        TL.load(sm.vt, (const T*)prm.v + cb, nv);
        TL.load(sm.dot, (const T*)prm.dout + cb, nv);
        TileLoader<T> TS;
        TS.init(w, lane, 1);   // rows of 128 contiguous elements
        static_assert(4 * TileLoader<T>::ROUNDS == kStateLoads, "state loads per wave");
        TS.load(sm.st(0), (const T*)Hc, kChunk);
        TS.load(sm.st(1), (const T*)Hc + kChunk * kDk, kChunk);
        TS.load(sm.st(2), (const T*)dHn, kChunk);
        TS.load(sm.st(3), (const T*)dHn + kChunk * kDk, kChunk);
    }
    // Memory operations complete in issue order: all but the last kStateLoads
    // (this wave's state loads) done means g, beta and the tiles are in LDS.  The
    // barrier is spelled out: an LDS release fence would also wait for the state
    // loads (direct loads write LDS).
    __builtin_amdgcn_s_waitcnt(vmcnt_wait(kStateLoads) & ~(0x3f << 8));   // and lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    {
        // the in-chunk gate scan, by every wave (each writes the same values and
        // reads back only its own writes)
        const float gam = wave_inclusive_scan(sm.gst[0][lane]);
        const float gC = lane_value(gam, 63);
        sm.gam[lane] = gam;
        sm.Gam[lane] = __expf(gam);
        sm.E[lane] = __expf(gC - gam);
        sm.beta[lane] = sm.gst[1][lane];
    }

    // ---- phase 1: 64 x 64 tile (ti, tj) of the score matrices
    const int ti = w >> 1, tj = w & 1;
    {
    f32x16 Pm = zero16(), Mg = zero16(), SG, skk;
    if (ti >= tj) {
        score_tiles<T>(L, sm, ti, tj, Pm, Mg, SG, skk);
        const f32x16 gr = rows_of(sm.gam, ti, g);
        if (ti == tj) {
            // diagonal block p: T_pp = diag(Gamma) T0_pp diag(1/Gamma), T0_pp gate-free
            const int p = ti;
            const f32x16 brow = rows_of(sm.beta, p, g);
            const f32x16 zt = diag_inverse_t<T>(skk, skk, brow, sm.beta[32 * p + n], n, g);
            // zt = acc(T0_pp^T): lane n holds row 32p + n, registers columns 32p + rho
            const float gn = sm.gam[32 * p + n];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int col = rho(g, r);
                const float t = col <= n ? zt[r] * __expf(gn - gr[r]) : 0.f;
                sm.tg()[toff<T, 64>(32 * p + n, 32 * p + col)] = (T)t;
            }
        }
    }
    st_tile64<T>(sm.pm(), Pm, ti, tj, g, n);
    st_tile64<T>(sm.mg(), Mg, ti, tj, g, n);
    }
    lds_barrier();

    wait_vm();       // the staged states
    lds_barrier();

    // ---- phase 2: this wave's 32 dv columns of Y, V', dV', dY
    f32x16 Y[2], Vp[2], dZ[2], dY[2];
    // this lane's part of <dHn, Hn>, with Hn = Gamma_C Hc + K^T diag(E) V' the
    // chunk's final state: <dHn, Hn> = Gamma_C <dHn, Hc> + sum_r E_r (K dHn)_r . V'_r,
    // both terms over this wave's columns
    float hn_dot = 0.f, hc_dot = 0.f;
    {
        f32x16 KH[2] = {zero16(), zero16()};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const F hf = L.f128(sm.st(w >> 1), w & 1, ks);   // H rows 32w + n of [dv][dk]
            KH[0] = mma(L.f128(sm.kt, 0, ks), hf, KH[0]);
            KH[1] = mma(L.f128(sm.kt, 1, ks), hf, KH[1]);
            // <dHn, Hc> over this wave's columns (the same elements of dHn)
            const F df = L.f128(sm.st(2 + (w >> 1)), w & 1, ks);
#pragma unroll
            for (int j = 0; j < 8; ++j) hc_dot += (float)hf[j] * (float)df[j];
        }
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const F v0 = L.trV(sm.vt, 2 * rt), v1 = L.trV(sm.vt, 2 * rt + 1);
            const f32x16 G = rows_of(sm.Gam, rt, g);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                Y[rt][j] = (float)v0[j] - G[j] * KH[rt][j];
                Y[rt][8 + j] = (float)v1[j] - G[8 + j] * KH[rt][8 + j];
            }
        }
    }
    const f32x16 be0 = rows_of(sm.beta, 0, g), be1 = rows_of(sm.beta, 1, g);
    f32x16 MgV0 = zero16(), MgV1 = zero16();

    {
        // V'_0 = T_00 diag(beta_0) Y_0 ; V'_1 = T_11 diag(beta_1) (Y_1 - Mg_10 V'_0)
        const f32x16 z0 = Y[0] * be0;
        Vp[0] = zero16();
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) Vp[0] = mma(afrag<T, 64>(sm.tg(), n, ks, g), acc_frag<T>(z0, ks), Vp[0]);
        f32x16 w10 = zero16();
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const F vf = acc_frag<T>(Vp[0], ks);
            w10 = mma(afrag<T, 64>(sm.mg(), 32 + n, ks, g), vf, w10);
            MgV0 = mma(afrag<T, 64>(sm.mg(), n, ks, g), vf, MgV0);
        }
        const f32x16 z1 = (Y[1] - w10) * be1;
        Vp[1] = zero16();
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            Vp[1] = mma(afrag<T, 64>(sm.tg(), 32 + n, 2 + ks, g), acc_frag<T>(z1, ks), Vp[1]);
        MgV1 = w10;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            MgV1 = mma(afrag<T, 64>(sm.mg(), 32 + n, 2 + ks, g), acc_frag<T>(Vp[1], ks), MgV1);
    }
    {
        // dV' = scale Pm^T dO + diag(E) K dHn
        f32x16 KdH[2] = {zero16(), zero16()};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const F hf = L.f128(sm.st(2 + (w >> 1)), w & 1, ks);
            KdH[0] = mma(L.f128(sm.kt, 0, ks), hf, KdH[0]);
            KdH[1] = mma(L.f128(sm.kt, 1, ks), hf, KdH[1]);
        }
        f32x16 PdO[2] = {zero16(), zero16()};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const F df = L.trV(sm.dot, ks);
            PdO[0] = mma(tfrag<T, 64>(sm.pm(), 0, ks, lane), df, PdO[0]);
            if (ks >= 2) PdO[1] = mma(tfrag<T, 64>(sm.pm(), 32, ks, lane), df, PdO[1]);
        }
        f32x16 dVp[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const f32x16 e = rows_of(sm.E, rt, g);
            dVp[rt] = PdO[rt] * scale + e * KdH[rt];
#pragma unroll
            for (int r = 0; r < 16; ++r) hn_dot += e[r] * KdH[rt][r] * Vp[rt][r];
        }
        // dZ_1 = T_11^T dV'_1 ; dZ_0 = T_00^T (dV'_0 - Mg_10^T diag(beta_1) dZ_1)
        dZ[1] = zero16();
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            dZ[1] = mma(tfrag<T, 64>(sm.tg(), 32, 2 + ks, lane), acc_frag<T>(dVp[1], ks), dZ[1]);
        dY[1] = dZ[1] * be1;
        f32x16 u = zero16();
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) u = mma(tfrag<T, 64>(sm.mg(), 0, 2 + ks, lane), acc_frag<T>(dY[1], ks), u);
        const f32x16 t0v = dVp[0] - u;
        dZ[0] = zero16();
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) dZ[0] = mma(tfrag<T, 64>(sm.tg(), 0, ks, lane), acc_frag<T>(t0v, ks), dZ[0]);
        dY[0] = dZ[0] * be0;
    }
    // dbeta partial over this wave's columns; V' and dY to LDS (dv = dY goes to
    // HBM from there, as row pieces)
    {
        const f32x16 r0 = dZ[0] * (Y[0] - MgV0), r1 = dZ[1] * (Y[1] - MgV1);
        row_sums(sm.part[w][0], r0, 0, g, n);
        row_sums(sm.part[w][0], r1, 1, g, n);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) st_rows_lds<T>(sm.vt, Vp[rt], rt, g, n, w);
        lds_barrier();   // the score tiles are dead: dY takes their place
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) st_rows_lds<T>(sm.dyt(), dY[rt], rt, g, n, w);
    }
    lds_barrier();

    // ---- phase 3: 64 x 64 gradient tiles, kept in registers until the staged
    // states are no longer read
    copy_tile_rows<T>((T*)prm.dv + (((size_t)b * Tn + t0) * H + h) * kDv, sm.dyt(), H, nv, tid);
    f32x16 dpS, dmS;   // dPm o Sg, dMg o Sg
    {
        f32x16 dPm = zero16(), dMg = zero16(), Pm = zero16(), Mg = zero16(), SG = zero16();
        if (ti >= tj) {
            f32x16 skk;
            score_tiles<T>(L, sm, ti, tj, Pm, Mg, SG, skk);
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const F vf = L.f128(sm.vt, tj, ks);
                dPm = mma(L.f128(sm.dot, ti, ks), vf, dPm);
                dMg = mma(L.f128(sm.dyt(), ti, ks), vf, dMg);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int R = 32 * ti + rho(g, r), S = 32 * tj + n;
                dPm[r] = R >= S ? scale * dPm[r] : 0.f;
                dMg[r] = R > S ? -dMg[r] : 0.f;
            }
        }
        const f32x16 X = dPm * Pm + dMg * Mg;
        row_sums(sm.xrow[w], X, 0, g, n);
        col_sums(sm.xcol[w], X, g, n);
        dpS = dPm * SG;
        dmS = dMg * SG;
    }

    // ---- phase 4: this wave's 32 dk columns of dq and dk, accumulated transposed
    // (swapped MFMA operands: lane n = position 32 rt + n, registers = dk rows
    // 32 w + rho), so that a lane holds row pieces of its position
    {
        f32x16 a2[2] = {zero16(), zero16()}, a3[2] = {zero16(), zero16()}, a4[2] = {zero16(), zero16()};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            // state rows 32w + n over dv = 16 ks + 8 g + j (the stored layout is [dv][dk])
            const F hr = tfrag_nat<T>(sm.st(ks >> 2), 32 * w, ks & 3, lane);
            const F dr = tfrag_nat<T>(sm.st(2 + (ks >> 2)), 32 * w, ks & 3, lane);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                a2[rt] = mma(hr, L.f128(sm.dot, rt, ks), a2[rt]);   // (dO H^T)^T
                a3[rt] = mma(hr, L.f128(sm.dyt(), rt, ks), a3[rt]); // (dY H^T)^T
                a4[rt] = mma(dr, L.f128(sm.vt, rt, ks), a4[rt]);    // (V' dHn^T)^T
            }
        }
        lds_barrier();   // the states are dead: the gradient tiles take the region
        st_tile64<T>(sm.dpg(), dpS, ti, tj, g, n);
        st_tile64<T>(sm.dmg(), dmS, ti, tj, g, n);
        lds_barrier();
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int pos = 32 * rt + n;
            f32x16 dqt = zero16(), dkt = zero16();
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const F kf = L.trK(sm.kt, w, ks);
                const F qf = L.trK(sm.qt, w, ks);
                dqt = mma(kf, afrag<T, 64>(sm.dpg(), pos, ks, g), dqt);        // (dPm o Sg  K)^T
                dkt = mma(qf, tfrag<T, 64>(sm.dpg(), 32 * rt, ks, lane), dkt); // ((dPm o Sg)^T Q)^T
                dkt = mma(kf, afrag<T, 64>(sm.dmg(), pos, ks, g), dkt);        // (dMg o Sg  K)^T
                dkt = mma(kf, tfrag<T, 64>(sm.dmg(), 32 * rt, ks, lane), dkt); // ((dMg o Sg)^T K)^T
            }
            const float G = sm.Gam[pos], E = sm.E[pos];
            const f32x16 dq2 = a2[rt] * (G * scale);
            const f32x16 dk3 = a3[rt] * (-G);
            const f32x16 dk4 = a4[rt] * E;
            dqt = dqt + dq2;
            dkt = dkt + dk3 + dk4;
            // q and k of this position at dk rows 32w + rho(g, r): four 4-element reads
            f32x16 pq, pk3, pk4;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                typedef typename Quad<T>::type Q4;
                const Q4 qv = *reinterpret_cast<const Q4*>(sm.qt + toff<T, kDk>(pos, 32 * w + 8 * i + 4 * g));
                const Q4 kv = *reinterpret_cast<const Q4*>(sm.kt + toff<T, kDk>(pos, 32 * w + 8 * i + 4 * g));
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    pq[4 * i + e] = (float)qv[e] * dq2[4 * i + e];
                    pk3[4 * i + e] = (float)kv[e] * dk3[4 * i + e];
                    pk4[4 * i + e] = (float)kv[e] * dk4[4 * i + e];
                }
            }
            col_sums(sm.part[w][1] + 32 * rt, pq, g, n);
            col_sums(sm.part[w][2] + 32 * rt, pk3, g, n);
            col_sums(sm.part[w][3] + 32 * rt, pk4, g, n);
            const size_t row = (((size_t)b * Tn + t0 + pos) * H + h) * kDk + 32 * w;
            store_row_pieces<T>((T*)prm.dq + row, dqt, g, pos < nv);
            store_row_pieces<T>((T*)prm.dk + row, dkt, g, pos < nv);
        }
    }
    // ---- phase 5: <dHn, Hn> for the gradient of gamma_C, this wave's part
    {
        float acc = sm.Gam[kChunk - 1] * hc_dot + hn_dot;   // Gamma_{63} = Gamma_C
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) acc += __shfl_xor(acc, d, 64);
        if (lane == 0) sm.red[w] = acc;
    }
    lds_barrier();

    // ---- phase 6: dgamma, reverse cumulative sum, dbeta
    if (w == 0) {
        const int r = lane, rl = r & 31;
        // wave 2 ti + tj holds the tile (ti, tj): rows of tile ti come from waves
        // 2 ti and 2 ti + 1, columns of tile tj from waves tj and 2 + tj
        const float rs = r < 32 ? sm.xrow[0][rl] + sm.xrow[1][rl] : sm.xrow[2][rl] + sm.xrow[3][rl];
        const float cs = r < 32 ? sm.xcol[0][rl] + sm.xcol[2][rl] : sm.xcol[1][rl] + sm.xcol[3][rl];
        float dgam = rs - cs, db = 0.f;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
            dgam += sm.part[ww][1][r] + sm.part[ww][2][r] - sm.part[ww][3][r];
            db += sm.part[ww][0][r];
        }
        if (r == kChunk - 1) dgam += sm.red[0] + sm.red[1] + sm.red[2] + sm.red[3];
        // suffix sum over positions r..63
        const float rev = __shfl(dgam, kChunk - 1 - r, 64);
        const float sc = wave_inclusive_scan(rev);
        const float dgv = __shfl(sc, kChunk - 1 - r, 64);
        if (r < nv) {
            const size_t go = ((size_t)b * Tn + t0 + r) * H + h;
            prm.dg[go] = dgv;
            prm.dbeta[go] = db;
        }
    }
}

template <typename T>
__global__ __launch_bounds__(kLocalThreads, 1) void gdn_bwd_local_kernel(BwdParams prm) {
    local_body<T>(prm, blockIdx.x / prm.N, blockIdx.x % prm.N);
}

// Packed sequences: workgroup (h, gc) takes chunk gc of all the batch's chunks
// of head h (none past the last chunk); a binary search of the chunk prefix
// finds its sequence.
template <typename T>
__global__ __launch_bounds__(kLocalThreads, 1) void gdn_bwd_local_varlen_kernel(BwdParams prm_in) {
    const int h = (int)blockIdx.x / prm_in.cmax, gc = (int)blockIdx.x % prm_in.cmax;
    const int* const cs = prm_in.cstart;
    if (gc >= __builtin_amdgcn_readfirstlane(cs[prm_in.B])) return;   // whole workgroup
    int lo = 0, hi = prm_in.B;   // cs[lo] <= gc < cs[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (__builtin_amdgcn_readfirstlane(cs[mid]) <= gc)
            lo = mid;
        else
            hi = mid;
    }
    BwdParams prm = prm_in;
    varlen_bwd_params(prm, lo, h, sizeof(T));
    local_body<T>(prm, lo * prm_in.H + h, gc - __builtin_amdgcn_readfirstlane(cs[lo]));
}

template <typename K>
hipError_t set_lds(K kernel, size_t bytes) {
    return hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <typename T>
hipError_t launch_dh_t(const BwdParams& p, hipStream_t s, int mode) {
    static bool configured = false;
    const size_t lds = sizeof(Smem<T>);
    if (!configured) {
        hipError_t e = set_lds(gdn_bwd_dh_kernel<T, DH_FULL>, lds);
        if (e == hipSuccess) e = set_lds(gdn_bwd_dh_kernel<T, DH_FIRST>, lds);
        if (e == hipSuccess) e = set_lds(gdn_bwd_dh_kernel<T, DH_REST>, lds);
        if (e == hipSuccess) e = set_lds(gdn_bwd_dh_varlen_kernel<T>, lds);
        if (e != hipSuccess) return e;
        configured = true;
    }
    const unsigned nbh = (unsigned)(p.B * p.H);
    if (p.cu)
        hipLaunchKernelGGL((gdn_bwd_dh_varlen_kernel<T>), dim3(nbh), dim3(kDhThreads), lds, s, p);
    else if (mode == DH_FIRST)
        hipLaunchKernelGGL((gdn_bwd_dh_kernel<T, DH_FIRST>), dim3(nbh * (p.P - 1)), dim3(kDhThreads), lds, s, p);
    else if (mode == DH_REST)
        hipLaunchKernelGGL((gdn_bwd_dh_kernel<T, DH_REST>), dim3(nbh * (p.P - 1)), dim3(kDhThreads), lds, s, p);
    else
        hipLaunchKernelGGL((gdn_bwd_dh_kernel<T, DH_FULL>), dim3(nbh), dim3(kDhThreads), lds, s, p);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_local_t(const BwdParams& p, hipStream_t s) {
    static bool configured = false;
    const size_t lds = sizeof(LocalSmem<T>);
    if (!configured) {
        hipError_t e = set_lds(gdn_bwd_local_kernel<T>, lds);
        if (e == hipSuccess) e = set_lds(gdn_bwd_local_varlen_kernel<T>, lds);
        if (e != hipSuccess) return e;
        configured = true;
    }
    if (p.cu)
        hipLaunchKernelGGL((gdn_bwd_local_varlen_kernel<T>), dim3(p.H * p.cmax), dim3(kLocalThreads), lds, s,
                           p);
    else
        hipLaunchKernelGGL((gdn_bwd_local_kernel<T>), dim3(p.B * p.H * p.N), dim3(kLocalThreads), lds, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_dh(const BwdParams& p, bool bf16, hipStream_t s, int mode) {
    return bf16 ? launch_dh_t<__bf16>(p, s, mode) : hipErrorNotSupported;
}

hipError_t launch_bwd_local(const BwdParams& p, bool bf16, hipStream_t s) {
    return bf16 ? launch_local_t<__bf16>(p, s) : hipErrorNotSupported;
}

hipError_t launch_seq_chunk_prefix(const int* cu, int B, int T, int* cstart, hipStream_t s) {
    hipLaunchKernelGGL(seq_chunk_prefix_kernel, dim3(1), dim3(256), 0, s, cu, B, T, cstart);
    return hipGetLastError();
}

}  // namespace gdn
