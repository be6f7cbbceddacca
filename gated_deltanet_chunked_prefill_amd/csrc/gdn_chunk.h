// Chunk-level device building blocks of the chunked gated delta rule for gfx950,
// shared by the fused forward and the backward kernels: the LDS layout of one
// workgroup (K/Q/V tiles and the chunk prep outputs), per-lane fragment
// addressing, the tile loader, the chunk prep (gate scan, 2C+1 exponentials,
// intra-chunk inverse blocks, masked Q K^T blocks) and the state-side products.
// Every function is inlined into the kernel that uses it.
#pragma once
#include "gdn_device.h"

namespace gdn {
namespace {

enum { MODE_FULL = 0, MODE_PASS1 = 1 };

// bf16 runs the prep one chunk ahead of the state step (K/Q triple-buffered,
// V and prep outputs double-buffered); the float32 build, used for small
// float32 workloads, runs prep and state step back to back in single buffers.
template <typename T> struct Pipe { static constexpr bool on = sizeof(T) == 2; };

// Prep outputs of one chunk, six 32x32 A-layout tiles:
//   0: Tt_00   1: Tt_11   2: -Ah_10 (gated)
//   3: P_00 | T0_00 diag(beta)   4: P_10 | -K_1 K_0^T   5: P_11 | T0_11 diag(beta)
// (full mode | pass-1 gate-free versions for the segment transition).
constexpr int kT32 = 32 * 32;
// Cache policy of the direct loads of data a call reads once (the chunk tiles
// and gates): non-temporal.  Measured: the forward's memory pattern streams 5 %
// faster with non-temporal loads (gdn_stream_probe), the forward 0.5 % and the
// backward 1 %.  Stores stay ordinary: the forward's output rows leave in 64-byte
// pieces per wave, and non-temporal stores of such partial lines made it 10 %
// slower.
constexpr int kCpolStream = 2;

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
    float gbt[3][2][kChunk];   // bf16 pipeline: g and beta of a chunk, staged with its K/Q slot
    int islot[4];              // workgroup-wide scalars: [0] job index, [1] job count
    float fslot[4];            // [0] exp(sum of g over a segment)
    int jrec[8];               // split forward: the workgroup's first job, planned in the workgroup
};

__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x3f70); }   // vmcnt(0)
// s_waitcnt immediate for vmcnt(n) alone, n < 64 (vmcnt in bits 3:0 and 15:14;
// expcnt and lgkmcnt at their maxima, as in vmcnt(0) = 0x3f70)
constexpr int vmcnt_wait(int n) { return 0x3f70 | (n & 15) | (((n >> 4) & 3) << 14); }
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

// Wave-uniform copies of values every lane holds alike: the compiler keeps them
// in scalar registers, so loops bounded by them are scalar loops and values read
// once through a generic pointer are not re-read (each such read would wait for
// every outstanding memory operation of the wave).
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ float uni(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}
template <typename P>
__device__ __forceinline__ P* uni(P* p) {
    const uint64_t v = (uint64_t)p;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
    return (P*)(((uint64_t)hi << 32) | lo);
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
//   * rows 32rt + n of a 64 x 128 tile, one 16-byte read of columns 16ks + 8g ..
//     +7: slot = (2ks + g) ^ swz16(n) (swz16 of row 32rt + n equals swz16(n)); the
//     16 lanes a 128-bit read serves per cycle hit 16 distinct slots;
//   * transposing reads of a 64 x 128 tile: lane (i, q, g) of a 16-lane group
//     reads row r = 16ks + 8h + a (a = 4g + i/4), columns 32ht + 16q + 4(i%4)..+3,
//     i.e. slot 4ht + x with x = 2q + (i/2)%2; swz16(r) = 4(a%4) + 2h + g, so the
//     stored slot is 4(ht ^ a%4) + (x ^ (2h + g)) for every ks;
//   * rows n of a 32 x 32 tile: slot = (2ks + h) ^ swz4(n).
template <typename T>
struct Lane {
    int lane, n, g, w;
    uint32_t a128[8];   // bf16: n*256 + (((2ks + g) ^ swz16(n)) << 4), entry ks
    uint32_t a32[4];    // bf16: n*64 + 8g + ((j ^ swz4(n)) << 4)
    uint32_t trk[8];    // bf16: transposing-read offsets, entry 2ht + h (column window 32ht)
    uint32_t trv[2];    // bf16: the same for this wave's V columns 32w, entry h

    __device__ void init(int tid) {
        lane = tid & 63;
        n = lane & 31;
        g = lane >> 5;
        w = (tid >> 6) & 3;
        if constexpr (sizeof(T) == 2) {
            const int s = swz16(n), s4 = swz4(n);
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) a128[ks] = n * 256 + (((2 * ks + g) ^ s) << 4);
#pragma unroll
            for (int j = 0; j < 4; ++j) a32[j] = n * 64 + 8 * g + ((j ^ s4) << 4);
            const int i = lane & 15, q = (lane >> 4) & 1;
            const int a = 4 * g + (i >> 2);
            const int x = 2 * q + ((i >> 1) & 1);
            const uint32_t base = a * 256 + 8 * (i & 1);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int lo = x ^ (2 * h + g);
#pragma unroll
                for (int ht = 0; ht < 4; ++ht) trk[2 * ht + h] = base + ((((ht ^ (a & 3)) << 2) | lo) << 4);
                trv[h] = base + ((((w ^ (a & 3)) << 2) | lo) << 4);
            }
        }
    }

    // A fragment of rows 32rt + n of a 64 x 128 tile, contraction k-step ks.  For
    // bf16 the lane gets columns 16ks + 8g .. +7 in order (one 16-byte read): a
    // fragment in accumulator row order meets it only through nat_frag.
    __device__ __forceinline__ typename FragOf<T>::type f128(const T* tile, int rt, int ks) const {
        if constexpr (sizeof(T) == 2) {
            return lds_ld<typename FragOf<T>::type>(tile, a128[ks] + rt * 8192);
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
    // tile[kappa(ks, g, 0..7)][32*cb + m]; tab2 = the two table entries (h = 0, 1)
    // of column window cb (compile-time for K, the wave's own window for V).
    __device__ __forceinline__ typename FragOf<T>::type tr(const T* tile, const uint32_t* tab2, int ks) const {
        if constexpr (sizeof(T) == 2) {
            typedef short s4 __attribute__((ext_vector_type(4)));
            typedef __bf16 b4 __attribute__((ext_vector_type(4)));
            typename FragOf<T>::type f;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t off = tab2[h] + (16 * ks + 8 * h) * 256;
                s4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s4*)(as_lds(tile) + off));
                b4 q = __builtin_bit_cast(b4, r);
#pragma unroll
                for (int j = 0; j < 4; ++j) f[4 * h + j] = q[j];
            }
            return f;
        } else {
            (void)tab2;
            return typename FragOf<T>::type{};
        }
    }
    // K^T fragment for dk rows 32ht + m.
    __device__ __forceinline__ typename FragOf<T>::type trK(const T* tile, int ht, int ks) const {
        if constexpr (sizeof(T) == 2) {
            return tr(tile, trk + 2 * ht, ks);
        } else {
            return tfrag<T, kDk>(tile, 32 * ht, ks, opaque_tid() & 63);
        }
    }
    // V fragment (accumulator layout) for this wave's dv columns.
    __device__ __forceinline__ typename FragOf<T>::type trV(const T* tile, int ks) const {
        if constexpr (sizeof(T) == 2) {
            return tr(tile, trv, ks);
        } else {
            return tfrag<T, kDv>(tile, 32 * w, ks, opaque_tid() & 63);
        }
    }
};

// Copy of one 64 x 128 chunk tile of a head into a swizzled row-major LDS tile,
// spread over the 64 NW lanes of NW loading waves.  Full chunks go HBM -> LDS
// directly (each lane's 16 bytes land at slot base + 16*lane, so the lane fetches
// the chunk that belongs there); a short last chunk goes through registers and
// is zero-filled.
template <typename T, int NW = 4>
struct TileLoader {
    static constexpr int EPC = 16 / (int)sizeof(T);     // elements per 16-byte chunk
    static constexpr int CPR = kDk / EPC;               // 16-byte chunks per row
    static constexpr int ROUNDS = kChunk * CPR / (64 * NW);
    uint32_t off[ROUNDS];   // byte offset of this lane's 16 bytes from the chunk's first row
    int pw, lane;           // loading wave (0..NW-1, wave-uniform) and lane

    // Computed once per task: round i covers tile slots (NW i + pw) * 64 + lane.
    __device__ __forceinline__ void init(int pw_, int lane_, int H) {
        pw = pw_;
        lane = lane_;
#pragma unroll
        for (int i = 0; i < ROUNDS; ++i) {
            const int L = (i * NW + pw) * 64 + lane;
            const int row = L / CPR, slot = L % CPR;
            off[i] = (uint32_t)((row * H * kDk + (slot ^ slot_swz<CPR>(row)) * EPC) * (int)sizeof(T));
        }
    }
    // Copy the chunk whose first row (for this head) is `chunk` into `tile`.
    // CPOL: cache policy of the direct loads (streaming by default; 16 =
    // device-coherent, for data another workgroup published during the launch).
    template <int CPOL = kCpolStream>
    __device__ __forceinline__ void load(T* tile, const T* chunk, int nvalid) const {
        const char* base = (const char*)chunk;
        if (nvalid == kChunk) {
#pragma unroll
            for (int i = 0; i < ROUNDS; ++i) {
                T* lbase = tile + (i * NW + pw) * 64 * EPC;   // wave-uniform LDS destination
                __builtin_amdgcn_global_load_lds((const void*)(base + off[i]),
                                                 (__attribute__((address_space(3))) void*)lbase, 16, 0, CPOL);
            }
        } else {
            typedef uint32_t u4 __attribute__((ext_vector_type(4)));
#pragma unroll
            for (int i = 0; i < ROUNDS; ++i) {
                const int L = (i * NW + pw) * 64 + lane;
                u4 v = {0u, 0u, 0u, 0u};
                if (L / CPR < nvalid) v = *(const __attribute__((address_space(1))) u4*)(base + off[i]);
                *(u4*)(tile + L * EPC) = v;
            }
        }
    }
};

// Element offset of the first row of chunk c of head (b, h) in a [B, T, H, 128] tensor.
__device__ __forceinline__ size_t chunk_base(int b, int h, int T, int H, int c) {
    return (((size_t)b * T + (size_t)c * kChunk) * H + h) * kDk;
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

// c + X Y to about float32 accuracy from bf16 MFMAs: X and Y split into bf16
// high and low parts, the three products that matter accumulated separately
// (the low x low term is below float32 rounding); float32 operands need no split.
template <typename T>
__device__ __forceinline__ f32x16 mm_acc_split(const f32x16& xt, const f32x16& y, f32x16 c) {
    if constexpr (sizeof(T) == 2) {
        f32x16 xl, yl;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            xl[r] = xt[r] - (float)(T)xt[r];
            yl[r] = y[r] - (float)(T)y[r];
        }
        c = mm_acc<T>(xt, yl, c);
        c = mm_acc<T>(xl, y, c);
    }
    return mm_acc<T>(xt, y, c);
}

// Whether entry (row, n), row = rho(g, r), of acc(No^T) at doubling step LEV is
// an entry of Nd joining two blocks of 2^LEV: No[n][row] with n in an odd block
// and row in the block before it.  Spelled out per step so that the register
// part is a compile-time constant and one lane test serves several registers.
template <int LEV>
__device__ __forceinline__ bool joins(int r, int n, int g) {
    if constexpr (LEV == 4) return r < 8 && n >= 16;
    if constexpr (LEV == 3) return ((r >> 2) & 1) == 0 && (n >> 3) == (r >> 2) + 1;
    if constexpr (LEV == 2) return g == 0 && (n >> 2) == 2 * (r >> 2) + 1;
    return ((r & 3) >> 1) == 0 && (n >> 1) == 4 * (r >> 2) + 2 * g + 1;
}

// One doubling step: block size 2^LEV -> 2^(LEV+1).
// LEV = 5 is step 4 forming Z as well as Z^T.
template <typename T, int LEV>
__device__ __forceinline__ void doubling_step(f32x16& z, f32x16& zt, const f32x16& nnt, int n, int g) {
    f32x16 not_;   // acc(-No^T)
#pragma unroll
    for (int r = 0; r < 16; ++r) not_[r] = joins<(LEV < 5 ? LEV : 4)>(r, n, g) ? nnt[r] : 0.f;
    const f32x16 q = mm_acc<T>(not_, z, zero16());   // Q = -No Z
    if constexpr (LEV != 4) {
        const f32x16 zn = mm_acc<T>(zt, q, z);         // Z + Z Q = Z - Z No Z
        zt = mm_acc<T>(q, zt, zt);                     // its transpose, Z^T + Q^T Z^T
        z = zn;
    } else {
        zt = mm_acc<T>(q, zt, zt);                     // the last step needs Z^T only
    }
}

// Inverse of (I + Nd) for one 32x32 diagonal block, Nd = diag(beta) strict_lower(S),
// from acc(S) and acc(S^T) (the same registers when S is symmetric).  Returns
// acc(T0^T): lane n holds row n of T0 = (I + Nd)^{-1} at columns rho.
//
// Recursive block inversion on MFMA: with Z the inverse of the block-diagonal
// part of I + Nd at block size b, and No the entries of Nd that join block pairs
// (rows in block 2m+1, columns in block 2m), the inverse at block size 2b is
// Z - Z No Z (Z No is strictly block-lower inside each pair, so its square is
// zero).  Starting from b = 1 (Z = I) this takes four doubling steps to b = 32.
// Every product forms entries of a true inverse (block forward substitution in
// matrix form), so no intermediate grows beyond the inverse's own entries and
// rounding stays at the operands' precision for any keys (a power series in Nd,
// exact only in exact arithmetic, cancels catastrophically when a chunk's keys
// are strongly correlated).  With bf16 operands the entries come out within
// about twice the rounding of storing them as bf16 (which the block solve does
// with every inverse block); float32 operands give float32 accuracy.
template <typename T, bool REFINE = true>
__device__ __forceinline__ f32x16 diag_inverse_t(const f32x16& S, const f32x16& St, const f32x16& beta_rows,
                                                 float beta_n, int n, int g) {
    // row = (8 (r >> 2) + (r & 3)) | 4 g, so comparing u = n ^ 4g with a constant
    // per register tests row == n (and row == n +- 1 for the pairs below)
    const int u = n ^ (g << 2);
    f32x16 z, zt, nnt;   // acc(Z), acc(Z^T), acc(-Nd^T)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int c = 8 * (r >> 2) + (r & 3), row = rho(g, r);
        const float nn = n < row ? -beta_rows[r] * S[r] : 0.f;   // -Nd[row][n]
        nnt[r] = row < n ? -beta_n * St[r] : 0.f;                // -Nd[n][row]
        // b = 1 -> 2: Z = I - Nd on the pairs (2m + 1, 2m)
        z[r] = u == c ? 1.f : ((r & 1) && u == c - 1) ? nn : 0.f;
        zt[r] = u == c ? 1.f : (!(r & 1) && u == c + 1) ? nnt[r] : 0.f;
    }
    doubling_step<T, 1>(z, zt, nnt, n, g);
    doubling_step<T, 2>(z, zt, nnt, n, g);
    doubling_step<T, 3>(z, zt, nnt, n, g);
    if constexpr (sizeof(T) == 2) {
        // With bf16 operands the doubling's error grows with the largest entry of
        // Nd (about 0.3 % of the inverse's largest entry at 0.5, 1.3 % near 2).
        // With unit keys and beta <= 1 no entry exceeds 1; a block with a larger
        // one (beta up to 2, or longer keys) gets one Newton step, Z <- Z + Z R
        // with R = I - (I + Nd) Z formed in split precision, which brings Z to
        // about float32 accuracy.  The test is wave-uniform.  REFINE = false
        // leaves it out where registers are short (the gate-free transition of
        // pass 1, whose blocks are stored in bf16 in any case).
        float big = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) big = fmaxf(big, fabsf(nnt[r]));
        if (REFINE && __builtin_amdgcn_ballot_w64(big > 1.f) != 0) {
            doubling_step<T, 5>(z, zt, nnt, n, g);   // step 4 forming Z as well
            const f32x16 ndz = mm_acc_split<T>(nnt, z, zero16());   // -Nd Z
            f32x16 res;                                            // acc(R)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int c = 8 * (r >> 2) + (r & 3);
                res[r] = (u == c ? 1.f : 0.f) - z[r] + ndz[r];
            }
            return mm_acc<T>(res, zt, zt);   // Z^T + R^T Z^T
        }
    }
    doubling_step<T, 4>(z, zt, nnt, n, g);
    return zt;
}

// Gate factor Gamma_r / Gamma_s for lane row r and accumulator-row columns s:
// fr is the row value (gamma_r or exp(gamma_r - gC/2)), fc the column values.
template <bool PW>
__device__ __forceinline__ float gate_factor(float fr, float fc) {
    if constexpr (PW) return __expf(fr - fc);
    else return fr * fc;
}

// acc(K_p K_p^T) of diagonal block p.  p is a template parameter so that every
// per-lane address-table index is a compile-time constant.
template <typename T, int p>
__device__ __forceinline__ f32x16 diag_gram(const Lane<T>& L, const T* kt) {
    using F = typename FragOf<T>::type;
    f32x16 S = zero16();
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        F kf = L.f128(kt, p, ks);
        S = mma(kf, kf, S);
    }
    return S;
}

// T0_pp of diagonal block p = pw (prep waves 0 and 1): one copy of the inverse
// for both blocks and both gate forms.  Returns acc(T0_pp^T): lane n holds row
// 32p + n of T0_pp, registers columns 32p + rho.
template <typename T, int MODE>
__device__ __forceinline__ f32x16 diag_t0(const Lane<T>& L, int pw, const T* kt, const float* s_beta) {
    const f32x16 S = pw == 0 ? diag_gram<T, 0>(L, kt) : diag_gram<T, 1>(L, kt);
    return diag_inverse_t<T, MODE != MODE_PASS1>(S, S, rows_of(s_beta, pw, L.g), s_beta[32 * pw + L.n], L.n,
                                                 L.g);
}

// Outputs of diagonal block p from zt = acc(T0_pp^T): the gated Tt_pp (and the
// gate-free T0_pp diag(beta) in pass-1).
template <typename T, int MODE, int p, bool PW>
__device__ __forceinline__ void diag_block(const Lane<T>& L, const f32x16& zt, T (*t32)[kT32],
                                           const float* s_row, const float* s_col,
                                           const float* s_beta) {
    using F = typename FragOf<T>::type;
    const int n = L.n, g = L.g;
    const f32x16 brow = rows_of(s_beta, p, g);
    const float fr = s_row[32 * p + n];
    const f32x16 fc = rows_of(s_col, p, g);
#pragma unroll
    for (int ksl = 0; ksl < 2; ++ksl) {
        F f, f0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int r = 8 * ksl + j;
            const float t0v = zt[r] * brow[r];
            f[j] = (T)(rho(g, r) <= n ? t0v * gate_factor<PW>(fr, fc[r]) : 0.f);
            f0[j] = (T)t0v;
        }
        L.st32(t32[p], ksl, f);
        if (MODE == MODE_PASS1) L.st32(t32[p == 0 ? 3 : 5], ksl, f0);
    }
}

// Matrix part of the chunk prep for prep wave pw, with the gate factor taken as
// the product of the re-centred exponentials (PW = false) or pairwise (PW = true).
template <typename T, int MODE, bool PW>
__device__ __forceinline__ void chunk_prep_mats(const Lane<T>& L, int pw, const T* kt, const T* qt,
                                                T (*t32)[kT32], const float* scr, bool emit,
                                                const f32x16& zt) {
    using F = typename FragOf<T>::type;
    const int n = L.n, g = L.g;
    const float* s_row = scr + (PW ? 0 : 1) * kChunk;   // gamma or exp(gamma - gC/2)
    const float* s_col = scr + (PW ? 0 : 2) * kChunk;   // gamma or exp(gC/2 - gamma)
    const float* s_beta = scr + 3 * kChunk;
    if (pw == 0) {
        diag_block<T, MODE, 0, PW>(L, zt, t32, s_row, s_col, s_beta);
    } else if (pw == 1) {
        diag_block<T, MODE, 1, PW>(L, zt, t32, s_row, s_col, s_beta);
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
                f[j] = (T)(-x[r] * gate_factor<PW>(fr, fc[r]));
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
                    f[j] = (T)(y[r] * gate_factor<PW>(fr, fc[r]));
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
                    f[j] = (T)(rho(g, r) <= n ? y[r] * gate_factor<PW>(fr, fc[r]) : 0.f);
                }
                L.st32(t32[j2 == 0 ? 3 : 5], ksl, f);
            }
        }
    }
}

// Chunk-independent prep of one chunk by prep wave pw.
template <typename T, int MODE>
__device__ __forceinline__ void chunk_prep(Smem<T>& sm, const Lane<T>& L, int pw, const T* kt,
                                           const T* qt, T (*t32)[kT32], float* gam_vec,
                                           float* e_vec, float* gc, float gv, float bv, bool emit,
                                           float& gsum) {
    const int lane = L.lane;
    float* scr = &sm.pscr[pw][0][0];
    // in-chunk scan and the 2C+1 exponentials of the factored gate (paragraph 6),
    // re-centred at gamma_C/2 so both factors stay within exp(|gamma_C|/2); chunks
    // whose decay exceeds that safe range use pairwise exponentials.
    const float gam = wave_inclusive_scan(gv);
    const float gC = lane_value(gam, 63);
    const float half = 0.5f * gC;
    const bool pairwise = gC < -160.f;   // wave-uniform
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
    f32x16 zt;   // prep waves 0 and 1: the diagonal block's T0, before the gate form splits
    if (pw < 2) zt = diag_t0<T, MODE>(L, pw, kt, scr + 3 * kChunk);
    if (pairwise)
        chunk_prep_mats<T, MODE, true>(L, pw, kt, qt, t32, scr, emit, zt);
    else
        chunk_prep_mats<T, MODE, false>(L, pw, kt, qt, t32, scr, emit, zt);
}

// X = K Hm for the two 32-row position tiles (Hm: the four dk tiles of a state).
// The K fragments are in column order, so Hm's fragments are reordered to match.
template <typename T>
__device__ __forceinline__ void k_times(const Lane<T>& L, const T* kt, const f32x16* Hm, f32x16* X) {
    X[0] = zero16();
    X[1] = zero16();
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        const typename FragOf<T>::type hf = nat_frag<T>(acc_frag<T>(Hm[ks >> 1], ks & 1));
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
    // software-pipelined over the 16 (ht, ks) steps: the transposed fragment of
    // the next step is requested before the product of the current one
    using F = typename FragOf<T>::type;
    F cur = L.trK(kt, 0, 0);
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
        f32x16 acc = Hm[ht] * a;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int nx = 4 * ht + ks + 1;
            F nxt;
            if (nx < 16) nxt = L.trK(kt, nx >> 2, nx & 3);
            acc = mma(cur, bf[ks], acc);
            if (nx < 16) cur = nxt;
        }
        Hm[ht] = acc;
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
// Buffer stores: one lane offset register, the row offsets as constants
// (keeps the 64 stores from holding 64 address registers).
__device__ __forceinline__ void store_state(float* dst, int w, int lane, const f32x16* Hs) {
    const int n = lane & 31, g = lane >> 5;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(dst, (short)0, (int)(kDk * kDv * 4), 0x00020000);
    const int voff = ((4 * g) * kDv + 32 * w + n) * 4;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(Hs[ht][r]), rs, voff,
                                                  (32 * ht + 8 * (r >> 2) + (r & 3)) * kDv * 4, 0);
}

// The state as bf16 in the transposed layout [dv][dk]: a lane's four
// consecutive accumulator rows 32ht + 8q + 4g .. +3 of column 32w + n are one
// 8-byte word.  Buffer stores with the row offsets as constants.
__device__ __forceinline__ void store_state_bf16t(__bf16* dst, int w, int lane, const f32x16* Hs) {
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 b4_t __attribute__((ext_vector_type(4)));
    const int n = lane & 31, g = lane >> 5;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(dst, (short)0, (int)(kDk * kDv * 2), 0x00020000);
    const int voff = ((32 * w + n) * kDk + 4 * g) * 2;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            b4_t v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (__bf16)Hs[ht][4 * q + e];
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, v), rs, voff,
                                                  (32 * ht + 8 * q) * 2, 0);
        }
}

// Number of valid tokens in chunk c of a sequence of T tokens.
__device__ __forceinline__ int chunk_len(int T, int c) {
    return T - c * kChunk < kChunk ? T - c * kChunk : kChunk;
}

// g (into gv) and beta (into bv) of chunk c of head (b, h) at position = lane;
// zero past the end of the sequence.
__device__ __forceinline__ void load_gate_beta(const float* g, const float* beta, int T, int H,
                                               int b, int h, int c, int lane, float& gv, float& bv) {
    gv = 0.f;
    bv = 0.f;
    if (lane < chunk_len(T, c)) {
        typedef __attribute__((address_space(1))) const float gfloat;
        const size_t go = ((size_t)b * T + c * kChunk + lane) * H + h;
        gv = ((gfloat*)g)[go];
        bv = ((gfloat*)beta)[go];
    }
}

}  // namespace
}  // namespace gdn
