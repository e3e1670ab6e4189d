// Chunkwise-parallel prompt form on the gfx950 matrix cores (bf16 inputs,
// 64-token chunks, fp32 state and accumulation).
//
// The form (Qwen3.5-9B-npu model page, "How it works" -> "Gated DeltaNet on
// the NPU"), per chunk of C = 64 tokens with incoming state S (dk x dv):
//     G  = cumsum(g)                                    inclusive, in the chunk
//     N  = diag(beta) [exp(G_t - G_j) k_t.k_j]_{j<t}     strictly lower
//     T  = (I + N)^-1                                    unit lower triangular
//     R  = diag(beta) (V - diag(exp G) K S)
//     D  = T R                                           per-token deltas
//     O  = diag(exp G) Q S + A D,  A = [exp(G_t - G_j) q_t.k_j]_{j<=t}
//     S <- exp(G_C) S + K^T diag(exp(G_C - G)) D
// Rows past a sequence's end are the page's token_valid padding (g = 0,
// beta = 0, zero q/k/v): they leave S untouched and are not stored.
//
// One 512-thread workgroup (8 waves) per (sequence, head), two roles:
//   * consumer waves 0..3 walk the chunks in order.  Wave w owns dv columns
//     [32w, 32w+32) of S, R, D and O; its share of S lives in 8 x 2 result
//     tiles of v_mfma_f32_16x16x32_bf16 (16 dk rows x 16 dv columns, 4 fp32 per
//     lane) for the whole walk.  Each state-dependent product keeps one
//     operand in registers: a result tile (lane holds rows 4q..4q+3 of column
//     l%16, q = l/16) is reused as the B operand of the next product over those
//     rows, by reading the partner A operand in the matching permuted k order
//     (lane group q takes k = 4q..4q+3 and 16+4q..16+4q+3 of a 32-wide k step).
//   * producer waves 4..7 prepare chunk c+1 while the consumers work on chunk
//     c: they load its rows (prefetched into registers a period ahead), stage
//     K, Q, V in LDS, run the Gram tiles K K^T and Q K^T (exact bf16 products,
//     fp32 accumulation) with the decay and beta applied on the accumulators,
//     invert the 16x16 diagonal blocks of I+N by forward substitution in fp32
//     and fill in T's off-diagonal blocks with T_ij = -T_ii sum_k N_ik T_kj
//     (one wave per column block).
//   Each chunk period has three barrier-separated phases:
//     A: consumers K S, Q S, R          | producers write K(c+1), scan its decay;
//                                       |   A(c) from Q(c) K(c)^T
//     B: consumers T R, A D -> O        | producers write V(c+1); N(c+1); T_ii
//     C: consumers state update         | producers write Q(c+1); T_ij, i > j
//   K, T, A and the per-token scalars are double-buffered; Q and V are read by
//   the consumers only in phase A, so one buffer each serves.
//   The two roles run as two separate loops under a wave-uniform branch; both
//   execute exactly three barriers per period (and three for the period in
//   which the producers prepare chunk 0), so their live registers never
//   overlap and each fits the 256 registers that two waves per SIMD allow.
// fp32 quantities that feed a bf16 MFMA (S, R, T, A, D and the decayed D) are
// split x = hi + lo into two bf16 parts (both rounded to nearest) and multiplied as hi*hi + hi*lo + lo*hi (or hi + lo against an
// exact bf16 operand), which keeps every product at ~2^-16 relative accuracy.  Where a row's scale factor (exp(G_t) for K S and
// Q S, exp(G_C - G_t) for the state update) stays below 2^-8 over a whole
// 16/32-row block, the lo term's contribution is below 2^-17 of the product
// and is not issued.

#include "gdn_internal.hpp"

namespace gdn {
namespace {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int C = 64;             // chunk length
constexpr int D = kHeadDim;       // 128
constexpr int RS = D + 8;         // bf16 row stride of K, Q, V tiles (272 B)
constexpr int TS = C + 8;         // bf16 row stride of T and A tiles (144 B)
constexpr float kLoSkip = 1.0f / 256.0f;
constexpr float kLog2e = 1.4426950408889634f;

// Rows are padded by 16 bytes so that the 16 rows a lane group touches in one
// instruction start on different LDS banks, and every address a lane forms is
// one per-lane base plus a compile-time offset.
struct __attribute__((aligned(16))) Smem {
    bf16 K[2][C * RS];            // chunk keys, double-buffered
    bf16 Q[C * RS];               // chunk queries
    bf16 V[C * RS];               // chunk values
    bf16 T[2][2][C * TS];         // [buffer][hi, lo] T = (I+N)^-1
    bf16 A[2][2][C * TS];         // [buffer][hi, lo] decayed masked Q K^T
    float NdT[4][16 * 20];        // fp32 diagonal blocks of N, transposed: [j][t]
    bf16 No[6][2][16 * 24];       // off-diagonal blocks (bi > bj) of N as hi/lo, [t][j]
    float G2[2][C];               // cumsum(g) * log2(e)
    float EG[2][C];               // exp(G_t)
    float EC[2][C];               // exp(G_last - G_t)
    float Bt[2][C];               // beta
    int lo_ks[2][4];              // per 16-token tile: max exp(G_t) >= 2^-8
    int lo_kd[2][2];              // per 32-token step: max exp(G_last - G_t) >= 2^-8
};

// index of the off-diagonal block (bi, bj), bi > bj, of N in Smem::No
__device__ __forceinline__ constexpr int oblk(int bi, int bj) { return bi * (bi - 1) / 2 + bj; }
constexpr int NOS = 24;           // bf16 row stride of an off-diagonal block (48 B)

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma3(bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl, f32x4 c) {
    c = mfma(ah, bh, c);
    c = mfma(ah, bl, c);
    return mfma(al, bh, c);
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ bf16 bz() { return static_cast<bf16>(0.f); }

__device__ __forceinline__ bf16x8 cat4(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ bf16x8 half4(bf16x4 a) {
    bf16x4 z;
#pragma unroll
    for (int e = 0; e < 4; ++e) z[e] = bz();
    return cat4(a, z);
}

// A operand in the permuted k order: row `row` of a row-major tile with row
// stride rs, k step starting at column kb; lane group q reads kb+4q..+3 and
// kb+16+4q..+3.
__device__ __forceinline__ bf16x8 rd_pk(const bf16 *m, int rs, int row, int kb, int q) {
    const bf16 *p = m + row * rs + kb + 4 * q;
    return cat4(*reinterpret_cast<const bf16x4 *>(p), *reinterpret_cast<const bf16x4 *>(p + 16));
}
// K^T as an A operand (row = dk index, k = tokens in the permuted order of
// step kb), gathered from the row-major key tile.
__device__ __forceinline__ bf16x8 rd_pkT(const bf16 *m, int row, int kb, int q) {
    const bf16 *p = m + (kb + 4 * q) * RS + row;
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        r[e] = p[e * RS];
        r[e + 4] = p[(16 + e) * RS];
    }
    return r;
}

// x = hi + lo with hi = x rounded to bf16 and lo the rounded remainder:
// |x - hi - lo| <= 2^-17 |x|.  Two values are split at a time: one packed
// conversion gives the hi pair; v_dot2_f32_bf16 against (-1, 0) or (0, -1)
// subtracts one bf16 half from its fp32 source exactly, giving the remainders
// in one instruction each; a second packed conversion rounds them.  The two
// multiplier pairs are held in SGPRs that the compiler cannot see through (as
// folded inline constants the bf16 pair encodings are not preserved).
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
struct Splitter {
    bf16x2 m_lo, m_hi;            // (-1, 0) and (0, -1)
    __device__ static Splitter make() {
        uint32_t a, b;
        asm volatile("s_mov_b32 %0, 0x0000bf80" : "=s"(a));
        asm volatile("s_mov_b32 %0, 0xbf800000" : "=s"(b));
        return Splitter{__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b)};
    }
    __device__ void split2(float a, float b, uint32_t *hi, uint32_t *lo) const {
        bf16x2 h;
        h[0] = static_cast<bf16>(a);
        h[1] = static_cast<bf16>(b);
        bf16x2 r;
        r[0] = static_cast<bf16>(__builtin_amdgcn_fdot2_f32_bf16(h, m_lo, a, false));
        r[1] = static_cast<bf16>(__builtin_amdgcn_fdot2_f32_bf16(h, m_hi, b, false));
        *hi = __builtin_bit_cast(uint32_t, h);
        *lo = __builtin_bit_cast(uint32_t, r);
    }
};

// hi/lo split of two result tiles (rows kb..kb+15 -> elements 0..3, rows
// kb+16..kb+31 -> elements 4..7): a B operand in the permuted k order.
__device__ __forceinline__ void split_pk(const Splitter &sp, f32x4 a, f32x4 b, bf16x8 &hi, bf16x8 &lo) {
    uint32_t h[4], o[4];
    sp.split2(a[0], a[1], &h[0], &o[0]);
    sp.split2(a[2], a[3], &h[1], &o[1]);
    sp.split2(b[0], b[1], &h[2], &o[2]);
    sp.split2(b[2], b[3], &h[3], &o[3]);
    hi = __builtin_bit_cast(bf16x8, u32x4{h[0], h[1], h[2], h[3]});
    lo = __builtin_bit_cast(bf16x8, u32x4{o[0], o[1], o[2], o[3]});
}
// hi/lo split of one tile used as a 16-deep operand (elements 4..7 zero).
__device__ __forceinline__ void split_half(const Splitter &sp, f32x4 a, bf16x8 &hi, bf16x8 &lo) {
    uint32_t h[2], o[2];
    sp.split2(a[0], a[1], &h[0], &o[0]);
    sp.split2(a[2], a[3], &h[1], &o[1]);
    hi = __builtin_bit_cast(bf16x8, u32x4{h[0], h[1], 0u, 0u});
    lo = __builtin_bit_cast(bf16x8, u32x4{o[0], o[1], 0u, 0u});
}
__device__ __forceinline__ void store_hilo(bf16 *hi, bf16 *lo, int idx, float x) {
    const bf16 h = static_cast<bf16>(x);
    hi[idx] = h;
    lo[idx] = static_cast<bf16>(x - static_cast<float>(h));
}

// Rows of one 16-token block held by a producer lane: row 16p+r16, k step s
// covers columns 32s+8q..+7 (the natural MFMA operand layout), as 16-byte
// entries.
__device__ __forceinline__ bf16x8 as_bf(f32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// Loads are always issued, rows past the chunk reading the sequence's first row
// instead, so that every period issues the same load sequence.  Nothing here
// consumes the loaded registers: the tail mask is applied when the rows are
// stored (store_rows), so the loads stay in flight until then.
__device__ __forceinline__ void load_rows(f32x4 *dst, const bf16 *src, int64_t start, int64_t row0,
                                          int r, int nv, int64_t H, int64_t h, int q) {
    const bf16 *p = src + ((r < nv ? row0 + r : start) * H + h) * D + 8 * q;
#pragma unroll
    for (int s = 0; s < 4; ++s) dst[s] = *reinterpret_cast<const f32x4 *>(p + 32 * s);
}
// Zero the rows past the chunk's end (the token_valid padding), in place.
__device__ __forceinline__ void mask_rows(f32x4 *x, bool ok) {
#pragma unroll
    for (int s = 0; s < 4; ++s) x[s] = ok ? x[s] : zero4();
}
__device__ __forceinline__ void store_rows(bf16 *tile, const f32x4 *src, int r, int q) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
        *reinterpret_cast<f32x4 *>(&tile[r * RS + 32 * s + 8 * q]) = src[s];
}

struct Unit {
    const bf16 *q, *k, *v;
    const float *g, *beta;
    int64_t start, len, H, h;
    __device__ int rows_in(int pc) const {
        const int64_t rem = len - int64_t(pc) * C;
        return static_cast<int>(rem < C ? rem : C);
    }
    __device__ int64_t row0(int pc) const { return start + int64_t(pc) * C; }
};

// Producer waves 4..7 (row block p): prepare chunk pc in buffer set nb over the
// three phases of one period.  Rows of the chunk are prefetched into pK, pQ,
// pV (rows 16p+r16) a period ahead.
struct Producer {
    f32x4 pK[4], pQ[4], pV[4];
    float pg, pb;
    Splitter sp;

    // chunk pc may lie past the sequence (nothing valid is read then); the
    // sequence has at least one token whenever these are called.
    __device__ void prefetch_kv(const Unit &u, int pc, int p, int l, int r16, int qd) {
        const int nv = u.rows_in(pc);
        load_rows(pK, u.k, u.start, u.row0(pc), 16 * p + r16, nv, u.H, u.h, qd);
        load_rows(pV, u.v, u.start, u.row0(pc), 16 * p + r16, nv, u.H, u.h, qd);
        const int64_t gi = (l < nv ? u.row0(pc) + l : u.start) * u.H + u.h;
        pg = u.g[gi];
        pb = u.beta[gi];
    }
    __device__ void prefetch_q(const Unit &u, int pc, int p, int r16, int qd) {
        load_rows(pQ, u.q, u.start, u.row0(pc), 16 * p + r16, u.rows_in(pc), u.H, u.h, qd);
    }

    // phase A: stage K (masked in place: the Gram tiles use these registers);
    // scan the log-decay (wave p = 0)
    __device__ void phase_a(Smem &sm, int nb, int nv, int p, int l, int r16, int qd) {
        mask_rows(pK, 16 * p + r16 < nv);
        store_rows(sm.K[nb], pK, 16 * p + r16, qd);
        if (p == 0) {
            const bool ok = l < nv;
            float x = ok ? pg : 0.f;
            pb = ok ? pb : 0.f;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(x, off);
                if (l >= off) x += y;
            }
            const float x2 = x * kLog2e;
            const float last = __shfl(x2, 63);
            const float eg = __builtin_amdgcn_exp2f(x2), ec = __builtin_amdgcn_exp2f(last - x2);
            sm.G2[nb][l] = x2;
            sm.EG[nb][l] = eg;
            sm.EC[nb][l] = ec;
            sm.Bt[nb][l] = pb;
            float m16 = eg, m32 = ec;
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) m16 = fmaxf(m16, __shfl_xor(m16, off));
#pragma unroll
            for (int off = 1; off < 32; off <<= 1) m32 = fmaxf(m32, __shfl_xor(m32, off));
            if ((l & 15) == 0) sm.lo_ks[nb][l >> 4] = m16 >= kLoSkip;
            if ((l & 31) == 0) sm.lo_kd[nb][l >> 5] = m32 >= kLoSkip;
        }
    }

    // Q K^T tiles of chunk pc (its K and Q are in LDS, buffers nb) -> A (hi/lo).
    // The ten lower 16x16 tiles are dealt out to the four waves: wave P takes
    // tiles P, P+4, P+8 of (0,0), (1,0), (1,1), (2,0), (2,1), (2,2), (3,0), ...
    template <int P>
    __device__ void gram_qk(Smem &sm, int nb, int r16, int qd) {
        constexpr int NT = P < 2 ? 3 : 2;
        constexpr int TI[4][3] = {{0, 2, 3}, {1, 2, 3}, {1, 3, 0}, {2, 3, 0}};
        constexpr int TJ[4][3] = {{0, 1, 2}, {0, 2, 3}, {1, 0, 0}, {0, 1, 0}};
        const bf16 *Kn = sm.K[nb];
        const float *G2 = sm.G2[nb];
        f32x4 acc[NT];
#pragma unroll
        for (int i = 0; i < NT; ++i) acc[i] = zero4();
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int i = 0; i < NT; ++i) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(&sm.Q[(16 * TI[P][i] + r16) * RS + 32 * s + 8 * qd]);
                const bf16x8 b = *reinterpret_cast<const bf16x8 *>(&Kn[(16 * TJ[P][i] + r16) * RS + 32 * s + 8 * qd]);
                acc[i] = mfma(a, b, acc[i]);
            }
        }
        // acc[i][e] = q_t . k_j, t = 16 mi + 4q + e, j = 16 mj + r16
        bf16 *An = sm.A[nb][0], *Anl = sm.A[nb][1];
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            const int j = 16 * TJ[P][i] + r16;
            const float g2j = G2[j];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 16 * TI[P][i] + 4 * qd + e;
                const float a = j <= t ? __builtin_amdgcn_exp2f(G2[t] - g2j) * acc[i][e] : 0.f;
                store_hilo(An, Anl, t * TS + j, a);
            }
        }
    }

    // phase B: stage V; K K^T tiles -> N; diagonal block P of T.  Compiled
    // once per row block P so that every tile loop is unrolled.
    template <int P>
    __device__ void phase_b(Smem &sm, int nb, int nv, int r16, int qd) {
        mask_rows(pV, 16 * P + r16 < nv);
        store_rows(sm.V, pV, 16 * P + r16, qd);
        const bf16 *Kn = sm.K[nb];
        const float *G2 = sm.G2[nb];
        const float *Bt = sm.Bt[nb];
        // K K^T tiles of row block P: (P, mj >= P).
        f32x4 kk[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) kk[m] = zero4();
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int mj = P; mj < 4; ++mj) {
                const bf16x8 b = mj == P ? as_bf(pK[s])
                                         : *reinterpret_cast<const bf16x8 *>(&Kn[(16 * mj + r16) * RS + 32 * s + 8 * qd]);
                kk[mj] = mfma(as_bf(pK[s]), b, kk[mj]);
            }
        }
        // kk[mj][e] = k_j . k_t with j = 16P+4q+e (row), t = 16mj+r16 (column):
        // the transpose of N's block (mj, P).
        {
            const int t = 16 * P + r16;
            const float g2t = G2[t], bt = Bt[t];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 4 * qd + e;          // local row of the diagonal block
                const float nv = j < r16 ? bt * (__builtin_amdgcn_exp2f(g2t - G2[16 * P + j]) * kk[P][e]) : 0.f;
                sm.NdT[P][j * 20 + r16] = nv;      // N^T[j][t]
            }
        }
#pragma unroll
        for (int mj = P + 1; mj < 4; ++mj) {
            const int t = 16 * mj + r16;
            const float g2t = G2[t], bt = Bt[t];
            f32x4 nv;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                nv[e] = bt * (__builtin_amdgcn_exp2f(g2t - G2[16 * P + 4 * qd + e]) * kk[mj][e]);
            bf16x8 h, lo;
            split_half(sp, nv, h, lo);
            bf16 *blk = sm.No[oblk(mj, P)][0];
            *reinterpret_cast<bf16x4 *>(&blk[r16 * NOS + 4 * qd]) = h.lo;
            *reinterpret_cast<bf16x4 *>(&sm.No[oblk(mj, P)][1][r16 * NOS + 4 * qd]) = lo.lo;
        }
        // Diagonal block P of T by forward substitution (lane r16 = column j):
        // once x_t is final, x_u -= N_ut x_t for every u > t.
        const int j = r16;
        const float *Nt = sm.NdT[P];
        float x[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) x[t] = t == j ? 1.f : 0.f;
#pragma unroll
        for (int t = 0; t < 15; ++t) {
            f32x4 col[4];
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4)
                if (4 * v4 + 3 > t) col[v4] = *reinterpret_cast<const f32x4 *>(&Nt[t * 20 + 4 * v4]);
#pragma unroll
            for (int u = t + 1; u < 16; ++u) x[u] -= col[u >> 2][u & 3] * x[t];
        }
        if (qd == 0) {
            bf16 *Tn = sm.T[nb][0], *Tnl = sm.T[nb][1];
#pragma unroll
            for (int t = 0; t < 16; ++t) store_hilo(Tn, Tnl, (16 * P + t) * TS + 16 * P + j, x[t]);
        }
    }

    // phase C: stage Q; column block p (< 3) of T: T_ip = -T_ii sum_k N_ik T_kp
    __device__ void phase_c(Smem &sm, int nb, int nv, int p, int r16, int qd) {
        mask_rows(pQ, 16 * p + r16 < nv);
        store_rows(sm.Q, pQ, 16 * p + r16, qd);
        if (p >= 3) return;
        const int j = p;
        bf16 *Tn = sm.T[nb][0], *Tnl = sm.T[nb][1];
        f32x4 Tc[4];
#pragma unroll
        for (int i = 1; i < 4; ++i) {
            if (i <= j) continue;
            f32x4 Z = zero4();
#pragma unroll
            for (int kk = 0; kk < 3; ++kk) {
                if (kk < j || kk >= i) continue;
                bf16x8 bh, bl;
                const bf16x8 ah = half4(*reinterpret_cast<const bf16x4 *>(&sm.No[oblk(i, kk)][0][r16 * NOS + 4 * qd]));
                const bf16x8 al = half4(*reinterpret_cast<const bf16x4 *>(&sm.No[oblk(i, kk)][1][r16 * NOS + 4 * qd]));
                if (kk == j) {
                    // B = T_jj (rows 4q+e, column r16) straight from its hi/lo parts
                    bf16x4 th, tl;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        th[e] = Tn[(16 * j + 4 * qd + e) * TS + 16 * j + r16];
                        tl[e] = Tnl[(16 * j + 4 * qd + e) * TS + 16 * j + r16];
                    }
                    bh = half4(th);
                    bl = half4(tl);
                } else {
                    split_half(sp, Tc[kk], bh, bl);
                }
                Z = mfma3(ah, al, bh, bl, Z);
            }
            // A = T_ii (row r16, columns 4q..4q+3) from its hi/lo parts
            const int ti = (16 * i + r16) * TS + 16 * i + 4 * qd;
            const bf16x8 ah = half4(*reinterpret_cast<const bf16x4 *>(&Tn[ti]));
            const bf16x8 al = half4(*reinterpret_cast<const bf16x4 *>(&Tnl[ti]));
            bf16x8 bh, bl;
            split_half(sp, Z, bh, bl);
            f32x4 Tij = mfma3(ah, al, bh, bl, zero4());
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                Tij[e] = -Tij[e];
                store_hilo(Tn, Tnl, (16 * i + 4 * qd + e) * TS + 16 * j + r16, Tij[e]);
            }
            Tc[i] = Tij;
        }
    }
};

__global__ __launch_bounds__(512) void prefill_mfma_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta,
    const float *__restrict__ S0, const int32_t *__restrict__ cu_seqlens, int64_t T,
    int64_t H, bf16 *__restrict__ O, float *__restrict__ S_T) {
    __shared__ Smem sm;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, l = tid & 63, r16 = l & 15, qd = l >> 4;
    const int w = wave & 3;                 // consumer column group / producer row block
    const int64_t unit = blockIdx.x;
    Unit u;
    u.q = q; u.k = k; u.v = v; u.g = g; u.beta = beta;
    u.H = H;
    u.h = unit % H;
    sequence_span(cu_seqlens, unit / H, T, u.start, u.len);
    const int nch = static_cast<int>((u.len + C - 1) / C);

    // T and A entries above the diagonal blocks are never written: zero both
    // buffers once.
    for (int i = tid * 8; i < 4 * C * TS; i += 512 * 8) {
        *reinterpret_cast<f32x4 *>(&sm.T[0][0][i]) = zero4();
        *reinterpret_cast<f32x4 *>(&sm.A[0][0][i]) = zero4();
    }

    if (wave >= 4) {
        // ======================= producer waves =======================
        // Barrier count matches the consumers': 4 + 3 * nch.  The prologue
        // prepares chunk 0, each loop period prepares chunk c+1 (and A of chunk
        // c), the last period only A of the last chunk.  The loop body is
        // straight-line so that the prefetch loads (K, V after phase B, Q after
        // phase C) are consumed in the order they were issued.
        if (nch == 0) {
            __syncthreads();
            __syncthreads();
            __syncthreads();
            __syncthreads();
            return;
        }
        Producer pr;
        pr.pg = pr.pb = 0.f;
        pr.sp = Splitter::make();
        auto gram_qk = [&](int c) {
            switch (w) {
            case 0: pr.gram_qk<0>(sm, c & 1, r16, qd); break;
            case 1: pr.gram_qk<1>(sm, c & 1, r16, qd); break;
            case 2: pr.gram_qk<2>(sm, c & 1, r16, qd); break;
            default: pr.gram_qk<3>(sm, c & 1, r16, qd); break;
            }
        };
        auto prepare = [&](int pc) {          // phases A..C for chunk pc, three barriers
            const int nb = pc & 1, pnv = u.rows_in(pc);
            pr.phase_a(sm, nb, pnv, w, l, r16, qd);
            __syncthreads();
            switch (w) {
            case 0: pr.phase_b<0>(sm, nb, pnv, r16, qd); break;
            case 1: pr.phase_b<1>(sm, nb, pnv, r16, qd); break;
            case 2: pr.phase_b<2>(sm, nb, pnv, r16, qd); break;
            default: pr.phase_b<3>(sm, nb, pnv, r16, qd); break;
            }
            pr.prefetch_kv(u, pc + 1, w, l, r16, qd);
            __syncthreads();
            pr.phase_c(sm, nb, pnv, w, r16, qd);
            pr.prefetch_q(u, pc + 1, w, r16, qd);
            __syncthreads();
        };
        pr.prefetch_kv(u, 0, w, l, r16, qd);
        pr.prefetch_q(u, 0, w, r16, qd);
        __syncthreads();
        prepare(0);                           // the period before the consumers start
        for (int c = 0; c + 1 < nch; ++c) {
            gram_qk(c);                       // A of chunk c, consumed in its phase B
            prepare(c + 1);
        }
        gram_qk(nch - 1);
        __syncthreads();
        __syncthreads();
        __syncthreads();
        return;
    }

    // ======================= consumer waves =======================
    // S[2i+c] holds state rows 16i+4q+e, column 32w+16c+r16.
    f32x4 S[16];
    if (S0) {
        const float *S0u = S0 + unit * (D * D);
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    S[2 * i + c][e] = S0u[(16 * i + 4 * qd + e) * D + 32 * w + 16 * c + r16];
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) S[i] = zero4();
    }
    __syncthreads();
    // the period in which the producers prepare chunk 0
    __syncthreads();
    __syncthreads();
    __syncthreads();

    const uint32_t HD = static_cast<uint32_t>(H) * D;
    const Splitter sp = Splitter::make();
    for (int c = 0; c < nch; ++c) {
        const int cur = c & 1;
        const int cnv = u.rows_in(c);
        bf16x8 Rhi[2][2], Rlo[2][2];
        f32x4 QS[4][2];

        // ================= phase A: K S, Q S (one split of S); R =================
        {
            const bf16 *Kc = sm.K[cur];
            f32x4 KS[4][2];
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) KS[m][cc] = QS[m][cc] = zero4();
            // the lo part of S is needed for tile 0 in practice; other tiles
            // only when the decay is slow
            const bool full = sm.lo_ks[cur][1] | sm.lo_ks[cur][2] | sm.lo_ks[cur][3];
            const bool lo0 = sm.lo_ks[cur][0];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                bf16x8 sh[2], sl[2];
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) split_pk(sp, S[4 * s + cc], S[4 * s + 2 + cc], sh[cc], sl[cc]);
                bf16x8 ak[4], aq[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    ak[m] = rd_pk(Kc, RS, 16 * m + r16, 32 * s, qd);
                    aq[m] = rd_pk(sm.Q, RS, 16 * m + r16, 32 * s, qd);
                }
#pragma unroll
                for (int m = 0; m < 4; ++m)
#pragma unroll
                    for (int cc = 0; cc < 2; ++cc) {
                        KS[m][cc] = mfma(ak[m], sh[cc], KS[m][cc]);
                        QS[m][cc] = mfma(aq[m], sh[cc], QS[m][cc]);
                    }
                if (lo0 | full) {
#pragma unroll
                    for (int cc = 0; cc < 2; ++cc) {
                        KS[0][cc] = mfma(ak[0], sl[cc], KS[0][cc]);
                        QS[0][cc] = mfma(aq[0], sl[cc], QS[0][cc]);
                    }
                }
                if (full) {
#pragma unroll
                    for (int m = 1; m < 4; ++m)
#pragma unroll
                        for (int cc = 0; cc < 2; ++cc) {
                            KS[m][cc] = mfma(ak[m], sl[cc], KS[m][cc]);
                            QS[m][cc] = mfma(aq[m], sl[cc], QS[m][cc]);
                        }
                }
            }
            // R = beta (V - exp(G) K S), in place of K S; exp(G) Q S
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = 16 * m + 4 * qd + e;
                    const float bt = sm.Bt[cur][t], eg = sm.EG[cur][t];
#pragma unroll
                    for (int cc = 0; cc < 2; ++cc) {
                        const float vt = static_cast<float>(sm.V[t * RS + 32 * w + 16 * cc + r16]);
                        KS[m][cc][e] = bt * (vt - eg * KS[m][cc][e]);
                        QS[m][cc][e] *= eg;
                    }
                }
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int cc = 0; cc < 2; ++cc)
                    split_pk(sp, KS[2 * s][cc], KS[2 * s + 1][cc], Rhi[s][cc], Rlo[s][cc]);
        }
        __syncthreads();

        // ================= phase B: D = T R; O = exp(G) Q S + A D =================
        bf16x8 Phi[2][2], Plo[2][2];
        {
            f32x4 Dt[4][2];
            const bf16 *Th = sm.T[cur][0], *Tl = sm.T[cur][1];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) Dt[m][cc] = zero4();
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    if (s > m / 2) continue;
                    const bf16x8 th = rd_pk(Th, TS, 16 * m + r16, 32 * s, qd);
                    const bf16x8 tl = rd_pk(Tl, TS, 16 * m + r16, 32 * s, qd);
#pragma unroll
                    for (int cc = 0; cc < 2; ++cc)
                        Dt[m][cc] = mfma3(th, tl, Rhi[s][cc], Rlo[s][cc], Dt[m][cc]);
                }
            }
            // D's hi/lo parts, and the decayed deltas for the state update
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) {
                    split_pk(sp, Dt[2 * s][cc], Dt[2 * s + 1][cc], Rhi[s][cc], Rlo[s][cc]);   // now D
                    f32x4 a = Dt[2 * s][cc], b = Dt[2 * s + 1][cc];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        a[e] *= sm.EC[cur][32 * s + 4 * qd + e];
                        b[e] *= sm.EC[cur][32 * s + 16 + 4 * qd + e];
                    }
                    split_pk(sp, a, b, Phi[s][cc], Plo[s][cc]);
                }
            const bf16 *Ah = sm.A[cur][0], *Al = sm.A[cur][1];
            bf16 *obase = O + (u.row0(c) * H + u.h) * D + 32 * w;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    if (s > m / 2) continue;
                    const bf16x8 ah = rd_pk(Ah, TS, 16 * m + r16, 32 * s, qd);
                    const bf16x8 al = rd_pk(Al, TS, 16 * m + r16, 32 * s, qd);
#pragma unroll
                    for (int cc = 0; cc < 2; ++cc) QS[m][cc] = mfma3(ah, al, Rhi[s][cc], Rlo[s][cc], QS[m][cc]);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = 16 * m + 4 * qd + e;
                    if (t < cnv) {
                        const uint32_t off = static_cast<uint32_t>(t) * HD + static_cast<uint32_t>(r16);
                        obase[off] = static_cast<bf16>(QS[m][0][e]);
                        obase[off + 16] = static_cast<bf16>(QS[m][1][e]);
                    }
                }
            }
        }
        __syncthreads();

        // ================= phase C: S <- exp(G_C) S + K^T diag(exp(G_C - G)) D =================
        {
            const bf16 *Kc = sm.K[cur];
            const float eC = sm.EG[cur][C - 1];
            const bool lo0 = sm.lo_kd[cur][0], lo1 = sm.lo_kd[cur][1];
#pragma unroll
            for (int i = 0; i < 16; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) S[i][e] *= eC;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const bf16x8 a0 = rd_pkT(Kc, 16 * i + r16, 0, qd);
                const bf16x8 a1 = rd_pkT(Kc, 16 * i + r16, 32, qd);
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) {
                    S[2 * i + cc] = mfma(a0, Phi[0][cc], S[2 * i + cc]);
                    S[2 * i + cc] = mfma(a1, Phi[1][cc], S[2 * i + cc]);
                }
                if (lo1) {
#pragma unroll
                    for (int cc = 0; cc < 2; ++cc) S[2 * i + cc] = mfma(a1, Plo[1][cc], S[2 * i + cc]);
                }
                if (lo0) {
#pragma unroll
                    for (int cc = 0; cc < 2; ++cc) S[2 * i + cc] = mfma(a0, Plo[0][cc], S[2 * i + cc]);
                }
            }
        }
        __syncthreads();
    }

    float *STu = S_T + unit * (D * D);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                STu[(16 * i + 4 * qd + e) * D + 32 * w + 16 * c + r16] = S[2 * i + c][e];
}

}  // namespace

bool prefill_mfma_supports(const PrefillArgs &a) { return a.bf16 && a.chunk == C; }

hipError_t launch_prefill_mfma(const PrefillArgs &a, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(a.N * a.H)), block(512);
    prefill_mfma_kernel<<<grid, block, 0, stream>>>(
        static_cast<const bf16 *>(a.q), static_cast<const bf16 *>(a.k),
        static_cast<const bf16 *>(a.v), a.g, a.beta, a.S0, a.cu_seqlens, a.T, a.H,
        static_cast<bf16 *>(a.O), a.S_T);
    return hipGetLastError();
}

}  // namespace gdn
