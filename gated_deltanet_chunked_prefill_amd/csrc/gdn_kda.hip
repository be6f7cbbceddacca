// Chunked forward of the per-key-channel-decay variant (KDA) for gfx950.
//
// The FlashQLA commentary names GDN and KDA as the sibling operators of the
// library (its "kernel innovation" section); the pages never print KDA's
// recurrence.  The reading taken here: one decay per key channel, applied to
// the state before the delta correction,
//     S_t = (I - beta_t k_t k_t^T) diag(exp(g_t)) S_{t-1} + beta_t k_t v_t^T,
//     o_t = scale * S_t^T q_t,                 g_t in R^dk,
// which is the gated delta rule when every channel decays alike.
//
// Chunk form (chunks of 64 tokens, G_r = in-chunk cumulative sum of g per key
// channel, H = the dk x dv state entering the chunk):
//     U  = (I + strict_lower(diag(beta) Kt Kh^T))^-1 diag(beta) (V - Kt H)
//     O  = scale (Qt H + lower(Qt Kh^T) U)
//     H' = diag(exp(G_C)) H + (K o exp(G_C - G))^T U
// with Kt = K o exp(G), Kh = K o exp(-G), Qt = Q o exp(G) row by row: the
// scalar gate factors of the GDN chunk step become per-channel factors inside
// the operands, so they are applied to the K and Q tiles before the products
// instead of as row and column scalings after them (the talk summary's EXP
// consolidation, paragraph 6, does not carry over: exp(G_r - G_s) no longer
// factors into one number per row and column).
//
// Range: Kt Kh^T only enters for s <= r, where every factor exp(G_r - G_s) is
// at most 1, but the two operands carry exp(G) and exp(-G) separately.  Each
// 32-token half of the chunk is therefore re-centred at the cumulative decay of
// its middle token (diagonal blocks: factors within exp(|decay over 16
// tokens|)), and the off-diagonal block (rows in the second half, columns in the
// first) at the decay of token 31, the boundary, where both factors are at most
// 1.  The exact products Kt H and Qt H use the re-centred tiles against state
// rows scaled by exp(centre) (at most 1).  The largest factor is exp(decay over
// the 16 tokens between a half's centre and its end), so results are finite
// whenever no key channel decays by more than exp(-88) (the float32 exponent
// range) over 16 consecutive tokens of a chunk.
//
// One workgroup (eight waves) per (batch, head) runs the chunks in order; per
// chunk: all waves load the K, Q, V tiles and form the re-centred tiles in LDS;
// waves 4-7 then build the inverse blocks and the masked score blocks while
// waves 0-3, each owning 32 state columns in MFMA accumulators, form Kt H and
// Qt H; after a barrier the state waves solve for U by block forward
// substitution, write the outputs and update the state.
#include "gdn_chunk.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int kKdaThreads = 512;

struct KdaSmem {
    __bf16 ku[kChunk * kDk];   // raw K, then K o exp(G_C - G)
    __bf16 qc[kChunk * kDk];   // raw Q, then Q o exp(G - c_half)
    __bf16 kc[kChunk * kDk];   // K o exp(G - c_half)
    __bf16 kd[kChunk * kDk];   // K o exp(c_half - G)
    __bf16 bnd[kChunk * kDk];  // rows 0-31: K o exp(G_31 - G); rows 32-63: K o exp(G - G_31)
    __bf16 bq[kChunk * kDk];   // rows 0-31: Q of tokens 32-63 o exp(G - G_31)
    __bf16 vt[kChunk * kDv];   // V
    __bf16 t32[6][kT32];       // Tt_00, Tt_11, -Ah_10, P_00, P_10, P_11 (A-layout 32 x 32 tiles)
    float ec0[kDk];            // exp(c_0) per key channel (c_0 = G at token 15)
    float ec1[kDk];            // exp(c_1) (c_1 = G at token 47)
    float eC[kDk];             // exp(G_C)
    float beta[kChunk];
    float gst[kChunk * kDk];   // the next chunk's gates [token][channel], staged by direct loads
    float bst[kChunk];         // the next chunk's beta, staged likewise
};
static_assert(sizeof(KdaSmem) <= 160 * 1024, "KDA LDS exceeds a CU's 160 KB");

// Workgroup barrier ordering LDS only: the prep waves' direct loads into the
// other buffers stay in flight (a release fence on LDS would wait for them,
// since they write LDS); their readers wait for them explicitly.
__device__ __forceinline__ void bar() {
    wait_lgkm();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// A 32 x 32 block written as an A-layout tile (lane n = row n): values x[r] at
// row n, column rho(g, r), times `s` and masked to columns <= n when `lower`.
__device__ __forceinline__ void put_block(const Lane<__bf16>& L, __bf16* tile, const f32x16& x, float s,
                                          bool lower) {
#pragma unroll
    for (int ksl = 0; ksl < 2; ++ksl) {
        bf16x8 f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int r = 8 * ksl + j;
            f[j] = (__bf16)((!lower || rho(L.g, r) <= L.n) ? s * x[r] : 0.f);
        }
        L.st32(tile, ksl, f);
    }
}

// acc(X Y^T) for rows 32 xr + (0..31) of tile X and rows 32 yr + (0..31) of tile
// Y (both 64 x 128 row-major): lane n holds (Y X^T)[n][rho].
__device__ __forceinline__ f32x16 rows_product(const Lane<__bf16>& L, const __bf16* X, int xr, const __bf16* Y,
                                               int yr) {
    f32x16 a = zero16();
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) a = mma(L.f128(X, xr, ks), L.f128(Y, yr, ks), a);
    return a;
}

// Prep wave pw (0..3) of one chunk.
__device__ __forceinline__ void kda_prep(const Lane<__bf16>& L, KdaSmem& sm, int pw) {
    const int n = L.n, g = L.g;
    if (pw < 2) {
        // diagonal block p: S = Kc_p Kd_p^T, T0_pp by recursive block inversion,
        // Tt_pp = T0_pp diag(beta)
        const int p = pw;
        const f32x16 S = rows_product(L, sm.kc, p, sm.kd, p);    // acc(Kc Kd^T): [rho][n] = kc_rho . kd_n
        const f32x16 St = rows_product(L, sm.kd, p, sm.kc, p);   // acc(S^T)
        const f32x16 brow = rows_of(sm.beta, p, g);
        const f32x16 zt = diag_inverse_t<__bf16>(S, St, brow, sm.beta[32 * p + n], n, g);
        f32x16 tt;
#pragma unroll
        for (int r = 0; r < 16; ++r) tt[r] = zt[r] * brow[r];
        put_block(L, sm.t32[p], tt, 1.f, true);
    } else if (pw == 2) {
        // off-diagonal block, rows 32-63 by columns 0-31, centred at token 31:
        // lane n holds Ah_10[n][rho] = kt_(32+n) . kh_rho
        const f32x16 x = rows_product(L, sm.bnd, 0, sm.bnd, 1);
        put_block(L, sm.t32[2], x, -1.f, false);
    } else {
        // masked score blocks: P_jj[n][rho] = qt_n . kh_rho (rho <= n), P_10 at the boundary
        put_block(L, sm.t32[3], rows_product(L, sm.kd, 0, sm.qc, 0), 1.f, true);
        put_block(L, sm.t32[5], rows_product(L, sm.kd, 1, sm.qc, 1), 1.f, true);
        put_block(L, sm.t32[4], rows_product(L, sm.bnd, 0, sm.bq, 0), 1.f, false);
    }
}

// Loads of chunk c, issued by prep wave pw (0..3) as direct buffer loads into
// LDS, which are waited for only where their data is read.  Each tensor's
// buffer descriptor starts at the chunk's first row and ends after its last
// row in the sequence, so rows past the sequence's end read as zero.  The fp32
// gates and beta go to the staging area; the raw K, Q, V tiles go to kd, kc and
// bnd (swizzled rows as toff), buffers whose previous contents are dead once
// the chunk before has written its blocks.  In pass 1 of the sequence split Q
// is not needed.
// The launch's input pointers and sizes, read once per workgroup into scalar
// registers: a read of the parameter block inside the chunk loop is a vector
// memory load, whose wait would also wait for every prefetch issued before it.
struct KdaIO {
    const __bf16 *k, *q, *v;
    const float *g, *beta;
    int T, H;
    __device__ __forceinline__ void init(const KdaParams& prm) {
        k = uni((const __bf16*)prm.k);
        q = uni((const __bf16*)prm.q);
        v = uni((const __bf16*)prm.v);
        g = uni(prm.g);
        beta = uni(prm.beta);
        T = uni(prm.T);
        H = uni(prm.H);
    }
};

constexpr int kKdaGateLoads = kChunk * kDk * 4 / (4 * 1024);   // 1 KB per wave instruction: 8 per wave
__device__ __forceinline__ __amdgpu_buffer_rsrc_t kda_rows(const void* first_row, int rows, int row_bytes) {
    // at most 64 rows of at most 2^31 / 64 bytes (the entry point bounds H)
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(first_row), (short)0, rows * row_bytes, 0x00020000);
}
__device__ __forceinline__ void kda_stage_gates(const KdaIO& io, KdaSmem& sm, int pw, int lane, int b, int h, int c) {
    const int Tn = io.T, H = io.H;
    const int nv = chunk_len(Tn, c);
    const size_t row0 = ((size_t)b * Tn + (size_t)c * kChunk) * H + h;
    const __amdgpu_buffer_rsrc_t rg = kda_rows(io.g + row0 * kDk, nv, H * kDk * 4);
    // rows 2R, 2R + 1 for R = 4 i + pw: 1 KB, lane-contiguous in LDS
    const int voff = (2 * pw + (lane >> 5)) * H * kDk * 4 + 16 * (lane & 31);
#pragma unroll
    for (int i = 0; i < kKdaGateLoads; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rg, (__attribute__((address_space(3))) void*)(sm.gst + 2 * (4 * i + pw) * kDk),
                                                 16, voff, i * 8 * H * kDk * 4, 0, kCpolStream);
    // every prep wave writes the same 256 bytes of beta (with the load under a
    // wave-index branch this compiler's gfx950 back end rejects the kernel)
    const __amdgpu_buffer_rsrc_t rb = kda_rows(io.beta + row0, nv, H * 4);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (__attribute__((address_space(3))) void*)sm.bst, 4, lane * H * 4, 0, 0,
                                             kCpolStream);
}
template <bool PASS1>
__device__ __forceinline__ void kda_stage_tiles(const KdaIO& io, KdaSmem& sm, int pw, int lane, int b, int h, int c) {
    const int Tn = io.T, H = io.H;
    const int nv = chunk_len(Tn, c);
    const size_t cb = chunk_base(b, h, Tn, H, c);
    const int rb = H * kDk * 2;   // bytes between rows
    const __amdgpu_buffer_rsrc_t rk = kda_rows(io.k + cb, nv, rb);
    const __amdgpu_buffer_rsrc_t rq = kda_rows(io.q + cb, nv, rb);
    const __amdgpu_buffer_rsrc_t rv = kda_rows(io.v + cb, nv, rb);
    // round i: tile slots (4 i + pw) * 64 + lane, i.e. row 16 i + 4 pw + lane / 16
    // and 16-byte piece lane % 16 (stored at slot piece ^ swz16(row), which does
    // not depend on i)
    const int row = 4 * pw + (lane >> 4);
    const int voff = row * rb + (((lane & 15) ^ swz16(row)) << 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int so = 16 * i * rb, lo = (4 * i + pw) * 64 * 8;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)(sm.kd + lo), 16, voff, so,
                                                 0, kCpolStream);
        if (!PASS1)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (__attribute__((address_space(3))) void*)(sm.kc + lo), 16, voff,
                                                     so, 0, kCpolStream);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void*)(sm.bnd + lo), 16, voff,
                                                 so, 0, kCpolStream);
    }
}
// direct loads of kda_stage_tiles per prep wave
template <bool PASS1>
constexpr int kda_tile_loads() { return (PASS1 ? 2 : 3) * kChunk * kDk * 2 / (4 * 1024); }

// Steps 1 and 2 run with thread (pair pr = tid % 64, group grp = tid / 64)
// owning key channels 2 pr, 2 pr + 1 and tokens 8 grp .. 8 grp + 7 (a wave
// covers one group: whole 256-byte rows, two channels per 4-byte LDS access).
// Cumulative gates are kept in base-2 units (times log2 e), so each factor is
// one exp2 of a difference.
typedef float kf2 __attribute__((ext_vector_type(2)));
typedef __bf16 kb2 __attribute__((ext_vector_type(2)));
constexpr float kLog2e = 1.4426950408889634f;
// the eight group sums per channel pass from step 1 to step 2 through the
// inverse and score blocks' space, dead from the end of one chunk step until
// the next chunk's blocks are written
__device__ __forceinline__ float* kda_group_sums(KdaSmem& sm) { return reinterpret_cast<float*>(&sm.t32[0][0]); }
static_assert(sizeof(KdaSmem::t32) >= 8 * kDk * sizeof(float), "group sums need 4 KB");

// Step 1 of chunk c, by every wave, from the staged gates: the in-chunk
// cumulative sums of this thread's 8 tokens for its two channels (base 2); the
// group sums go to LDS, beta to its slot.  A barrier follows.
__device__ __forceinline__ void kda_gates(int Tn, KdaSmem& sm, int c, kf2 (&gl)[8]) {
    const int nv = chunk_len(Tn, c);
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));   // per-chunk addressing, not hoisted out of the chunk loop
    const int pr = tid & 63, grp = tid >> 6;
    kf2 run = {0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int t = 8 * grp + j;
        const kf2 x = *reinterpret_cast<const kf2*>(sm.gst + t * kDk + 2 * pr);
        run += t < nv ? x * kLog2e : kf2{0.f, 0.f};
        gl[j] = run;
    }
    *reinterpret_cast<kf2*>(kda_group_sums(sm) + grp * kDk + 2 * pr) = run;
    if (tid < kChunk) {
        const float x = sm.bst[tid];
        sm.beta[tid] = tid < nv ? x : 0.f;
    }
}

// Step 2 of chunk c, by every wave: the re-centred tiles from the raw K, Q, V
// tiles (each thread reads and then overwrites only its own elements of kd, kc
// and bnd, so the in-place reuse is race-free); rows past the sequence's end
// are zeroed here, whatever the buffer loads left in them.  A barrier follows.
template <bool PASS1>
__device__ __forceinline__ void kda_scale(KdaSmem& sm, const kf2 (&gl)[8], int nv) {
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));   // per-chunk addressing, not hoisted out of the chunk loop
    const int pr = tid & 63, grp = tid >> 6;
    const float* const gs = kda_group_sums(sm);
    kf2 cum[8];   // cumulative group sums: G at tokens 7, 15, .., 63 (base 2)
    cum[0] = *reinterpret_cast<const kf2*>(gs + 2 * pr);
#pragma unroll
    for (int i = 1; i < 8; ++i) cum[i] = cum[i - 1] + *reinterpret_cast<const kf2*>(gs + i * kDk + 2 * pr);
    kf2 off = {0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 7; ++i)
        if (i < grp) off = cum[i];
    const kf2 c0 = cum[1], gb = cum[3], c1 = cum[5], gC = cum[7];
    const kf2 centre = grp < 4 ? c0 : c1;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int t = 8 * grp + j;
        const int e = toff<__bf16, kDk>(t, 2 * pr);   // channels 2 pr, 2 pr + 1: adjacent
        const bool in = t < nv;
        const kb2 kr = *reinterpret_cast<const kb2*>(sm.kd + e);
        const kb2 qr = *reinterpret_cast<const kb2*>(sm.kc + e);
        const kb2 vr = *reinterpret_cast<const kb2*>(sm.bnd + e);
        *reinterpret_cast<kb2*>(sm.vt + e) = in ? vr : kb2{(__bf16)0.f, (__bf16)0.f};
        kb2 okc, okd, oqc, oku, obn, obq;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const float G = off[i] + gl[j][i];
            const float kv = in ? (float)kr[i] : 0.f;
            const float qv = PASS1 || !in ? 0.f : (float)qr[i];
            const float ec = __builtin_amdgcn_exp2f(G - centre[i]), ed = __builtin_amdgcn_exp2f(centre[i] - G);
            okc[i] = (__bf16)(kv * ec);
            okd[i] = (__bf16)(kv * ed);
            oqc[i] = (__bf16)(qv * ec);
            oku[i] = (__bf16)(kv * __builtin_amdgcn_exp2f(gC[i] - G));
            const float eb = __builtin_amdgcn_exp2f(grp < 4 ? gb[i] - G : G - gb[i]);
            obn[i] = (__bf16)(kv * eb);
            obq[i] = (__bf16)(qv * eb);
        }
        *reinterpret_cast<kb2*>(sm.kc + e) = okc;
        *reinterpret_cast<kb2*>(sm.kd + e) = okd;
        if (!PASS1) *reinterpret_cast<kb2*>(sm.qc + e) = oqc;
        *reinterpret_cast<kb2*>(sm.ku + e) = oku;
        *reinterpret_cast<kb2*>(sm.bnd + e) = obn;
        if (!PASS1 && grp >= 4) *reinterpret_cast<kb2*>(sm.bq + toff<__bf16, kDk>(t - 32, 2 * pr)) = obq;
    }
    if (grp == 0) {
        *reinterpret_cast<kf2*>(sm.ec0 + 2 * pr) = kf2{__builtin_amdgcn_exp2f(c0[0]), __builtin_amdgcn_exp2f(c0[1])};
        *reinterpret_cast<kf2*>(sm.ec1 + 2 * pr) = kf2{__builtin_amdgcn_exp2f(c1[0]), __builtin_amdgcn_exp2f(c1[1])};
        *reinterpret_cast<kf2*>(sm.eC + 2 * pr) = kf2{__builtin_amdgcn_exp2f(gC[0]), __builtin_amdgcn_exp2f(gC[1])};
    }
}

// Waves 4-7: per chunk the shared steps, then the inverse and score blocks.  In
// pass 1 of the sequence split (segment p < P - 1, no outputs, so no score
// blocks) they also carry the segment's transition M from the identity, 32
// columns each: the chunk step with no values (the chunk map is linear in the
// state), after the blocks are written; M goes to the segment's slot.
// Executes exactly the barriers of kda_state_loop.
template <bool PASS1>
__device__ __noinline__ void kda_prep_loop(const KdaParams& prm, KdaSmem& sm, int bh, int p, int c0, int c1) {
    // arguments arrive in vector registers: make them wave-uniform
    bh = uni(bh), p = uni(p), c0 = uni(c0), c1 = uni(c1);
    using F = bf16x8;
    KdaIO io;
    io.init(prm);
    const int H = io.H;
    const int b = bh / H, h = bh % H;
    const int lane = threadIdx.x & 63;
    Lane<__bf16> L;
    L.init(threadIdx.x);
    const int pw = wave_id() - 4;
    const int n = L.n, gg = L.g, w = L.w;
    f32x16 Ms[4];
    if (PASS1) {
#pragma unroll
        for (int ht = 0; ht < 4; ++ht)
#pragma unroll
            for (int r = 0; r < 16; ++r) Ms[ht][r] = (32 * ht + rho(gg, r) == 32 * w + n) ? 1.f : 0.f;
    }
    // the first chunk's loads; later chunks' are issued one chunk ahead
    kda_stage_gates(io, sm, pw, lane, b, h, c0);
    kda_stage_tiles<PASS1>(io, sm, pw, lane, b, h, c0);
    wait_vm();
    bar();
    for (int c = c0; c < c1; ++c) {
        kf2 gl[8];
        kda_gates(io.T, sm, c, gl);
        wait_vm();   // this chunk's raw tiles
        bar();       // gates scanned: the staging area is free
        if (c + 1 < c1) kda_stage_gates(io, sm, pw, lane, b, h, c + 1);
        kda_scale<PASS1>(sm, gl, chunk_len(io.T, c));
        bar();       // tiles formed
        if (!PASS1 || pw < 3) kda_prep(L, sm, pw);
        bar();       // blocks written: kd, kc (full pass) and bnd are free
        if (c + 1 < c1) kda_stage_tiles<PASS1>(io, sm, pw, lane, b, h, c + 1);
        if (PASS1) {
            // X = Kt M (state rows scaled by each half's exp(centre)), U = T (-X)
            f32x16 X[2] = {zero16(), zero16()};
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const f32x16 s0 = rows_of(sm.ec0, ks >> 1, gg), s1 = rows_of(sm.ec1, ks >> 1, gg);
                F m0f, m1f;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int r = 8 * (ks & 1) + j;
                    m0f[j] = (__bf16)(-Ms[ks >> 1][r] * s0[r]);
                    m1f[j] = (__bf16)(-Ms[ks >> 1][r] * s1[r]);
                }
                m0f = nat_frag<__bf16>(m0f);
                m1f = nat_frag<__bf16>(m1f);
                X[0] = mma(L.f128(sm.kc, 0, ks), m0f, X[0]);
                X[1] = mma(L.f128(sm.kc, 1, ks), m1f, X[1]);
            }
            const F y0f[2] = {acc_frag<__bf16>(X[0], 0), acc_frag<__bf16>(X[0], 1)};
            f32x16 Vp[2];
            block_solve<__bf16>(L, sm.t32[0], sm.t32[1], sm.t32[2], y0f, X[1], Vp);
            F vf[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) vf[ks] = acc_frag<__bf16>(Vp[ks >> 1], ks & 1);
#pragma unroll
            for (int ht = 0; ht < 4; ++ht) Ms[ht] = Ms[ht] * rows_of(sm.eC, ht, gg);
            kt_update<__bf16>(L, sm.ku, Ms, 1.f, vf);
        }
        // the next chunk's gates (issued before its tiles) have landed
        __builtin_amdgcn_s_waitcnt(vmcnt_wait(kda_tile_loads<PASS1>()));
        bar();       // the state step is done with the tiles
    }
    if (PASS1) store_state(uni(prm.ws) + ((size_t)bh * (uni(prm.P) - 1) + p) * kKdaSlot, w, lane, Ms);
}

// Waves 0-3: the state (32 columns per wave, in MFMA accumulators) and the
// serial chunk step over chunks c0 .. c1-1 of segment p, with outputs; the
// segment starts from h0 (p = 0) or from the state the chain left for it, and the
// last segment writes ht.  Executes exactly the barriers of kda_prep_loop.
template <bool PASS1>
__device__ __noinline__ void kda_state_loop(const KdaParams& prm, KdaSmem& sm, int bh, int p, int c0, int c1) {
    // arguments arrive in vector registers: make them wave-uniform
    bh = uni(bh), p = uni(p), c0 = uni(c0), c1 = uni(c1);
    using F = bf16x8;
    const int Tn = uni(prm.T), H = uni(prm.H);
    const int b = bh / H, h = bh % H;
    const int lane = threadIdx.x & 63;
    const float scale = uni(prm.scale);
    __bf16* const op = uni((__bf16*)prm.o);
    Lane<__bf16> L;
    L.init(threadIdx.x);
    const int n = L.n, gg = L.g, w = L.w;
    f32x16 Hs[4];
    if (PASS1) {
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) Hs[ht] = zero16();
    } else if (p > 0) {
        load_state(uni(prm.ws) + ((size_t)bh * (prm.P - 1) + p - 1) * kKdaSlot + kDk * kDk, w, lane, Hs);
    } else if (prm.h0) {
        load_state(uni(prm.h0) + (size_t)bh * kDk * kDv, w, lane, Hs);
    } else {
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) Hs[ht] = zero16();
    }
    bar();   // the first chunk's loads have landed
    for (int c = c0; c < c1; ++c) {
        const int nv = chunk_len(Tn, c);
        {
            kf2 gl[8];
            kda_gates(Tn, sm, c, gl);
            bar();
            kda_scale<PASS1>(sm, gl, nv);
            bar();
        }
        // Kt H and (Qt H)^T: state rows of each k-step scaled by each half's exp(centre)
        f32x16 X[2], OT[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            X[rt] = zero16();
            OT[rt] = zero16();
        }
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const f32x16 s0 = rows_of(sm.ec0, ks >> 1, gg), s1 = rows_of(sm.ec1, ks >> 1, gg);
            F h0f, h1f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int r = 8 * (ks & 1) + j;
                h0f[j] = (__bf16)(Hs[ks >> 1][r] * s0[r]);
                h1f[j] = (__bf16)(Hs[ks >> 1][r] * s1[r]);
            }
            h0f = nat_frag<__bf16>(h0f);
            h1f = nat_frag<__bf16>(h1f);
            X[0] = mma(L.f128(sm.kc, 0, ks), h0f, X[0]);
            X[1] = mma(L.f128(sm.kc, 1, ks), h1f, X[1]);
            if (!PASS1) {
                OT[0] = mma(h0f, L.f128(sm.qc, 0, ks), OT[0]);
                OT[1] = mma(h1f, L.f128(sm.qc, 1, ks), OT[1]);
            }
        }
        bar();   // blocks written
        // Y = V - Kt H, U by block substitution
        f32x16 Y[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const F v0 = L.trV(sm.vt, 2 * rt), v1 = L.trV(sm.vt, 2 * rt + 1);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                Y[rt][j] = (float)v0[j] - X[rt][j];
                Y[rt][8 + j] = (float)v1[j] - X[rt][8 + j];
            }
        }
        const F y0f[2] = {acc_frag<__bf16>(Y[0], 0), acc_frag<__bf16>(Y[0], 1)};
        f32x16 Vp[2];
        block_solve<__bf16>(L, sm.t32[0], sm.t32[1], sm.t32[2], y0f, Y[1], Vp);
        F vf[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) vf[ks] = acc_frag<__bf16>(Vp[ks >> 1], ks & 1);
        if (PASS1) {
#pragma unroll
            for (int ht = 0; ht < 4; ++ht) Hs[ht] = Hs[ht] * rows_of(sm.eC, ht, gg);
            kt_update<__bf16>(L, sm.ku, Hs, 1.f, vf);
            bar();   // the tiles are free for the next chunk
            continue;
        }
        // O^T = (Qt H)^T + U^T P^T; P^T's B fragments are rows of P
        OT[0] = mma(vf[0], L.f32(sm.t32[3], 0), OT[0]);
        OT[0] = mma(vf[1], L.f32(sm.t32[3], 1), OT[0]);
        OT[1] = mma(vf[0], L.f32(sm.t32[4], 0), OT[1]);
        OT[1] = mma(vf[1], L.f32(sm.t32[4], 1), OT[1]);
        OT[1] = mma(vf[2], L.f32(sm.t32[5], 0), OT[1]);
        OT[1] = mma(vf[3], L.f32(sm.t32[5], 1), OT[1]);
        // H <- diag(exp(G_C)) H + (K o exp(G_C - G))^T U
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) Hs[ht] = Hs[ht] * rows_of(sm.eC, ht, gg);
        kt_update<__bf16>(L, sm.ku, Hs, 1.f, vf);
        // outputs: lane (n, g) holds state columns 8i + 4g .. +3 of row 32rt + n;
        // two half-wave lane swaps give it columns 8g .. +7 and 16 + 8g .. +7
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int pos = 32 * rt + n;
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
            if (pos < nv) {
                typedef uint32_t u4 __attribute__((ext_vector_type(4)));
                typedef __attribute__((address_space(1))) u4 gu4;
                __bf16* const orow = op + (((size_t)b * Tn + (size_t)c * kChunk + pos) * H + h) * kDv + 32 * w;
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const u4 v = {pk[4 * q], pk[4 * q + 1], pk[4 * q + 2], pk[4 * q + 3]};
                    *(gu4*)(orow + 16 * q + 8 * gg) = v;
                }
            }
        }
        bar();   // the tiles are free for the next chunk
    }
    const int P = uni(prm.P);
    if (PASS1 || (p == 0 && P > 1))   // b of segment p, or the state entering segment 1
        store_state(uni(prm.ws) + ((size_t)bh * (P - 1) + p) * kKdaSlot + kDk * kDk, w, lane, Hs);
    else if (prm.ht && p == P - 1)
        store_state(uni(prm.ht) + (size_t)bh * kDk * kDv, w, lane, Hs);
}

template <int MODE>
__global__ __launch_bounds__(kKdaThreads, 1) void gdn_kda_fwd_kernel(KdaParams prm) {
    extern __shared__ __attribute__((aligned(16))) char smem_raw[];
    KdaSmem& sm = *reinterpret_cast<KdaSmem*>(smem_raw);
    const int groups = MODE == KDA_FULL ? 1 : prm.P - 1;
    const int bh = (int)blockIdx.x / groups, j = (int)blockIdx.x % groups;
    const int p = MODE == KDA_REST ? j + 1 : j;
    const int c0 = p * prm.S, c1 = MODE == KDA_FULL ? prm.N : min(c0 + prm.S, prm.N);
    // the role branch is wave-uniform (both roles hold barriers); in KDA_FIRST
    // workgroup j = 0 runs segment 0 with outputs, the others pass 1
    const bool pass1 = MODE == KDA_FIRST && j > 0;
    if (wave_id() < 4) {
        if (pass1)
            kda_state_loop<true>(prm, sm, bh, p, c0, c1);
        else
            kda_state_loop<false>(prm, sm, bh, p, c0, c1);
    } else {
        if (pass1)
            kda_prep_loop<true>(prm, sm, bh, p, c0, c1);
        else
            kda_prep_loop<false>(prm, sm, bh, p, c0, c1);
    }
}

}  // namespace

size_t kda_smem_bytes() { return sizeof(KdaSmem); }

hipError_t launch_kda_fwd(const KdaParams& p, int mode, hipStream_t s) {
    static bool configured = false;
    const size_t lds = sizeof(KdaSmem);
    if (!configured) {
        hipError_t e = hipFuncSetAttribute((const void*)gdn_kda_fwd_kernel<KDA_FULL>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e == hipSuccess)
            e = hipFuncSetAttribute((const void*)gdn_kda_fwd_kernel<KDA_FIRST>,
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e == hipSuccess)
            e = hipFuncSetAttribute((const void*)gdn_kda_fwd_kernel<KDA_REST>,
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        configured = true;
    }
    const unsigned bh = (unsigned)(p.B * p.H);
    if (mode == KDA_FIRST)
        hipLaunchKernelGGL(gdn_kda_fwd_kernel<KDA_FIRST>, dim3(bh * (p.P - 1)), dim3(kKdaThreads), lds, s, p);
    else if (mode == KDA_REST)
        hipLaunchKernelGGL(gdn_kda_fwd_kernel<KDA_REST>, dim3(bh * (p.P - 1)), dim3(kKdaThreads), lds, s, p);
    else
        hipLaunchKernelGGL(gdn_kda_fwd_kernel<KDA_FULL>, dim3(bh), dim3(kKdaThreads), lds, s, p);
    return hipGetLastError();
}

hipError_t launch_kda_chain(const KdaParams& p, hipStream_t s) {
    // S_1 in slot 0 (segment 0's final state), then slots 1 .. P-2 in order
    ChainParams c{p.ws, p.P - 1, 0, 1, p.P - 2};
    return launch_state_chain(c, p.B * p.H, s);
}

}  // namespace gdn
