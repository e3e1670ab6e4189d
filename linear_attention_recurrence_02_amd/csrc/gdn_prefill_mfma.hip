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
//     A: consumers K S, R               | producers write K(c+1), decay scan
//     B: consumers T R, Q S, A D -> O   | producers write V(c+1); Gram; T_ii
//     C: consumers state update         | producers write Q(c+1); T_ij, i > j
//   K, T, A and the per-token scalars are double-buffered; V is read by the
//   consumers only in phase A and Q only in phase B, so one buffer each serves.
//   The two roles run as two separate loops under a wave-uniform branch; both
//   execute exactly three barriers per period (and three for the period in
//   which the producers prepare chunk 0), so their live registers never
//   overlap and each fits the 256 registers that two waves per SIMD allow.
// fp32 quantities that feed a bf16 MFMA (S, R, T, A, D and the decayed D) are
// split x = hi + lo into two bf16 parts and multiplied as hi*hi + hi*lo + lo*hi
// (or hi + lo against an exact bf16 operand), which keeps every product at
// ~2^-16 relative accuracy.  Where a row's scale factor (exp(G_t) for K S and
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
constexpr int FS = C + 4;         // fp32 row stride of the N scratch
constexpr int DS = 17;            // fp32 row stride of the 16x16 diagonal inverses
constexpr float kLoSkip = 1.0f / 256.0f;
constexpr float kLog2e = 1.4426950408889634f;

// Row-swizzled LDS tiles: a 128-wide bf16 row is 16 chunks of 16 bytes and
// chunk c of row r is stored at chunk c ^ (r & 15); a 64-wide row is 8 chunks
// stored at c ^ ((r >> 1) & 7).  Both keep the 16 rows a lane group reads in
// one instruction on distinct LDS banks.
__device__ __forceinline__ int sw128(int r, int i) { return r * D + ((((i >> 3) ^ (r & 15))) << 3) + (i & 7); }
__device__ __forceinline__ int sw64(int r, int j) { return r * C + ((((j >> 3) ^ ((r >> 1) & 7))) << 3) + (j & 7); }

struct Smem {
    bf16 K[2][C * D];             // chunk keys, double-buffered (sw128)
    bf16 Q[C * D];                // chunk queries (sw128)
    bf16 V[C * D];                // chunk values (sw128)
    bf16 T[2][2][C * C];          // [buffer][hi, lo] T = (I+N)^-1 (sw64)
    bf16 A[2][2][C * C];          // [buffer][hi, lo] decayed masked Q K^T (sw64)
    float N[C * FS];              // fp32 N of the chunk being prepared
    float Td[4 * 16 * DS];        // fp32 diagonal blocks of T
    float G2[2][C];               // cumsum(g) * log2(e)
    float EG[2][C];               // exp(G_t)
    float EC[2][C];               // exp(G_last - G_t)
    float Bt[2][C];               // beta
    int lo_ks[2][4];              // per 16-token tile: max exp(G_t) >= 2^-8
    int lo_kd[2][2];              // per 32-token step: max exp(G_last - G_t) >= 2^-8
};

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma3(bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl, f32x4 c) {
    c = mfma(ah, bh, c);
    c = mfma(ah, bl, c);
    return mfma(al, bh, c);
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// A zero the compiler cannot see through.  Lane indices are re-derived from it
// at the top of every loop iteration so that the many swizzled LDS addresses
// are recomputed in the loop (a few VALU ops) instead of being hoisted out of
// it and held in registers for the whole walk.
__device__ __forceinline__ int opaque_zero() {
    int z;
    asm volatile("s_mov_b32 %0, 0" : "=s"(z));
    return z;
}
__device__ __forceinline__ bf16 bz() { return static_cast<bf16>(0.f); }

__device__ __forceinline__ bf16x8 cat4(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// A operand in the permuted k order from a sw128 tile: row `row`, k step
// starting at column kb (multiple of 32).
__device__ __forceinline__ bf16x8 pk128(const bf16 *m, int row, int kb, int q) {
    const bf16x4 a = *reinterpret_cast<const bf16x4 *>(&m[sw128(row, kb + 4 * q)]);
    const bf16x4 b = *reinterpret_cast<const bf16x4 *>(&m[sw128(row, kb + 16 + 4 * q)]);
    return cat4(a, b);
}
// Same from a sw64 tile.
__device__ __forceinline__ bf16x8 pk64(const bf16 *m, int row, int kb, int q) {
    const bf16x4 a = *reinterpret_cast<const bf16x4 *>(&m[sw64(row, kb + 4 * q)]);
    const bf16x4 b = *reinterpret_cast<const bf16x4 *>(&m[sw64(row, kb + 16 + 4 * q)]);
    return cat4(a, b);
}
// K^T as an A operand (rows = dk index `row`, k = tokens in the permuted
// order of step kb), gathered from the row-major sw128 key tile.
__device__ __forceinline__ bf16x8 pkT128(const bf16 *m, int row, int kb, int q) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        r[e] = m[sw128(kb + 4 * q + e, row)];
        r[e + 4] = m[sw128(kb + 16 + 4 * q + e, row)];
    }
    return r;
}

// hi/lo split of two result tiles (rows kb..kb+15 -> elements 0..3, rows
// kb+16..kb+31 -> elements 4..7): a B operand in the permuted k order.
__device__ __forceinline__ void split_pk(f32x4 a, f32x4 b, bf16x8 &hi, bf16x8 &lo) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const bf16 ha = static_cast<bf16>(a[e]), hb = static_cast<bf16>(b[e]);
        hi[e] = ha;
        hi[e + 4] = hb;
        lo[e] = static_cast<bf16>(a[e] - static_cast<float>(ha));
        lo[e + 4] = static_cast<bf16>(b[e] - static_cast<float>(hb));
    }
}
// hi/lo split of one result tile used as a 16-deep operand (elements 4..7 zero).
__device__ __forceinline__ void split_half(f32x4 a, bf16x8 &hi, bf16x8 &lo) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const bf16 h = static_cast<bf16>(a[e]);
        hi[e] = h;
        lo[e] = static_cast<bf16>(a[e] - static_cast<float>(h));
        hi[e + 4] = lo[e + 4] = bz();
    }
}
__device__ __forceinline__ void store_hilo(bf16 *hi, bf16 *lo, int idx, float x) {
    const bf16 h = static_cast<bf16>(x);
    hi[idx] = h;
    lo[idx] = static_cast<bf16>(x - static_cast<float>(h));
}

// Rows of one 16-token block of a chunk held by a producer lane (row 16p+r16,
// k step s covers columns 32s+8q..+7, the natural MFMA operand layout), kept as
// four 16-byte entries of the shared register block.
__device__ __forceinline__ bf16x8 as_bf(f32x4 x) { return __builtin_bit_cast(bf16x8, x); }
__device__ __forceinline__ f32x4 as_f(bf16x8 x) { return __builtin_bit_cast(f32x4, x); }

__device__ __forceinline__ void load_rows(f32x4 *dst, const bf16 *src, int64_t row0, int r,
                                          int nv, int64_t H, int64_t h, int q) {
    if (r < nv) {
        const bf16 *p = src + ((row0 + r) * H + h) * D + 8 * q;
#pragma unroll
        for (int s = 0; s < 4; ++s) dst[s] = *reinterpret_cast<const f32x4 *>(p + 32 * s);
    } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) dst[s] = zero4();
    }
}
__device__ __forceinline__ void store_rows(bf16 *tile, const f32x4 *src, int r, int q) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
        *reinterpret_cast<f32x4 *>(&tile[sw128(r, 32 * s + 8 * q)]) = src[s];
}

struct Unit {
    const bf16 *q, *k, *v;
    const float *g, *beta;
    int64_t start, len, H, h;
    int nch;
    __device__ int rows_in(int pc) const {
        const int64_t rem = len - int64_t(pc) * C;
        return static_cast<int>(rem < C ? rem : C);
    }
    __device__ int64_t row0(int pc) const { return start + int64_t(pc) * C; }
};

// Producer waves 4..7 (row block p): prepare chunk pc in buffer set nb over the
// three phases of one period.  Rows of the chunk are prefetched into pK, pQ,
// pV (rows 16p+r16) one period ahead.
struct Producer {
    f32x4 pK[4], pQ[4], pV[4];
    float pg, pb;

    __device__ void prefetch_kv(const Unit &u, int pc, int p, int l, int r16, int qd) {
        const int nv = u.rows_in(pc);
        load_rows(pK, u.k, u.row0(pc), 16 * p + r16, nv, u.H, u.h, qd);
        load_rows(pV, u.v, u.row0(pc), 16 * p + r16, nv, u.H, u.h, qd);
        if (p == 0) {
            pg = l < nv ? u.g[(u.row0(pc) + l) * u.H + u.h] : 0.f;
            pb = l < nv ? u.beta[(u.row0(pc) + l) * u.H + u.h] : 0.f;
        }
    }
    __device__ void prefetch_q(const Unit &u, int pc, int p, int r16, int qd) {
        load_rows(pQ, u.q, u.row0(pc), 16 * p + r16, u.rows_in(pc), u.H, u.h, qd);
    }

    // phase A: stage K; scan the log-decay (wave p = 0)
    __device__ void phase_a(Smem &sm, int nb, int p, int l, int r16, int qd) {
        store_rows(sm.K[nb], pK, 16 * p + r16, qd);
        if (p == 0) {
            float x = pg;
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

    // phase B: stage V; Gram tiles; diagonal block p of T
    __device__ void phase_b(Smem &sm, int nb, int p, int r16, int qd) {
        store_rows(sm.V, pV, 16 * p + r16, qd);
        const bf16 *Kn = sm.K[nb];
        const float *G2 = sm.G2[nb];
        const float *Bt = sm.Bt[nb];
        // K K^T tiles (p, mj >= p): their transposes are the N tiles (mj, p).
        for (int mj = p; mj < 4; ++mj) {
            f32x4 acc = zero4();
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const bf16x8 b = mj == p ? as_bf(pK[s])
                                         : *reinterpret_cast<const bf16x8 *>(&Kn[sw128(16 * mj + r16, 32 * s + 8 * qd)]);
                acc = mfma(as_bf(pK[s]), b, acc);
            }
            // acc[e] = k_j . k_t with j = 16p+4q+e (row), t = 16mj+r16 (column)
            const int t = 16 * mj + r16;
            const float g2t = G2[t], bt = Bt[t];
            f32x4 out;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 16 * p + 4 * qd + e;
                out[e] = j < t ? bt * (__builtin_amdgcn_exp2f(g2t - G2[j]) * acc[e]) : 0.f;
            }
            *reinterpret_cast<f32x4 *>(&sm.N[t * FS + 16 * p + 4 * qd]) = out;
        }
        // Q K^T tiles (p, mj <= p) -> A (hi/lo)
        bf16 *An = sm.A[nb][0], *Anl = sm.A[nb][1];
        for (int mj = 0; mj <= p; ++mj) {
            f32x4 acc = zero4();
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const bf16x8 b = mj == p ? as_bf(pK[s])
                                         : *reinterpret_cast<const bf16x8 *>(&Kn[sw128(16 * mj + r16, 32 * s + 8 * qd)]);
                acc = mfma(as_bf(pQ[s]), b, acc);
            }
            const int j = 16 * mj + r16;
            const float g2j = G2[j];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 16 * p + 4 * qd + e;
                const float a = j <= t ? __builtin_amdgcn_exp2f(G2[t] - g2j) * acc[e] : 0.f;
                store_hilo(An, Anl, sw64(t, j), a);
            }
        }
        // Diagonal block p of T by forward substitution (lane r16 = column j).
        const int j = r16;
        float x[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) x[t] = t == j ? 1.f : 0.f;
#pragma unroll
        for (int t = 0; t < 16; ++t)
#pragma unroll
            for (int u = t + 1; u < 16; ++u) x[u] -= sm.N[(16 * p + u) * FS + 16 * p + t] * x[t];
        if (qd == 0) {
            bf16 *Tn = sm.T[nb][0], *Tnl = sm.T[nb][1];
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                sm.Td[(p * 16 + t) * DS + j] = x[t];
                store_hilo(Tn, Tnl, sw64(16 * p + t, 16 * p + j), x[t]);
            }
        }
    }

    // phase C: stage Q; column block p (< 3) of T: T_ip = -T_ii sum_k N_ik T_kp
    __device__ void phase_c(Smem &sm, int nb, int p, int r16, int qd) {
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
                bf16x8 ah, al, bh, bl;
                split_half(*reinterpret_cast<const f32x4 *>(&sm.N[(16 * i + r16) * FS + 16 * kk + 4 * qd]), ah, al);
                if (kk == j) {
                    f32x4 tj;
#pragma unroll
                    for (int e = 0; e < 4; ++e) tj[e] = sm.Td[(j * 16 + 4 * qd + e) * DS + r16];
                    split_half(tj, bh, bl);
                } else {
                    split_half(Tc[kk], bh, bl);
                }
                Z = mfma3(ah, al, bh, bl, Z);
            }
            bf16x8 ah, al, bh, bl;
            f32x4 ti;
#pragma unroll
            for (int e = 0; e < 4; ++e) ti[e] = sm.Td[(i * 16 + r16) * DS + 4 * qd + e];
            split_half(ti, ah, al);
            split_half(Z, bh, bl);
            f32x4 Tij = mfma3(ah, al, bh, bl, zero4());
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                Tij[e] = -Tij[e];
                store_hilo(Tn, Tnl, sw64(16 * i + 4 * qd + e, 16 * j + r16), Tij[e]);
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
    u.nch = static_cast<int>((u.len + C - 1) / C);
    const int nch = u.nch;

    // T and A tiles above the diagonal blocks are never written: zero them once.
    for (int i = tid * 8; i < 4 * C * C; i += 512 * 8) {
        *reinterpret_cast<f32x4 *>(&sm.T[0][0][i]) = zero4();
        *reinterpret_cast<f32x4 *>(&sm.A[0][0][i]) = zero4();
    }

    if (wave >= 4) {
        // ======================= producer waves =======================
        // Every iteration executes exactly three barriers, as the consumers do.
        Producer pr;
        pr.pg = pr.pb = 0.f;
        if (nch > 0) {
            pr.prefetch_kv(u, 0, w, l, r16, qd);
            pr.prefetch_q(u, 0, w, r16, qd);
        }
        __syncthreads();
        for (int c = -1; c < nch; ++c) {
            const int pc = c + 1, nb = pc & 1;   // chunk being prepared, its buffers
            const bool work = pc < nch;
            const int z = opaque_zero();
            const int r16 = l + z - (l & ~15), qd = (l >> 4) + z;
            if (work) pr.phase_a(sm, nb, w, l, r16, qd);
            __syncthreads();
            if (work) {
                pr.phase_b(sm, nb, w, r16, qd);
                if (pc + 1 < nch) pr.prefetch_kv(u, pc + 1, w, l, r16, qd);
            }
            __syncthreads();
            if (work) {
                pr.phase_c(sm, nb, w, r16, qd);
                if (pc + 1 < nch) pr.prefetch_q(u, pc + 1, w, r16, qd);
            }
            __syncthreads();
        }
        return;
    }

    // ======================= consumer waves =======================
    // S[2i+c] holds state rows 16i+4q+e, column 32w+16c+r16.
    const int l16 = r16, q4 = qd;
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

    for (int c = 0; c < nch; ++c) {
        const int cur = c & 1;
        const int cnv = u.rows_in(c);
        const int z = opaque_zero();
        const int r16 = l16 + z, qd = q4 + z;
        bf16x8 Rhi[2][2], Rlo[2][2], Phi[2][2], Plo[2][2];
        // outputs of this chunk: uniform base plus 32-bit lane offsets
        bf16 *obase = O + (u.row0(c) * H + u.h) * D + 32 * w;
        const uint32_t HD = static_cast<uint32_t>(H) * D;

        // ================= phase A: K S, R =================
        {
            const bf16 *Kc = sm.K[cur];
            f32x4 KS[4][2];
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) KS[m][cc] = zero4();
            bool lo[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) lo[m] = sm.lo_ks[cur][m];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                bf16x8 sh[2], sl[2];
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) split_pk(S[4 * s + cc], S[4 * s + 2 + cc], sh[cc], sl[cc]);
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const bf16x8 ak = pk128(Kc, 16 * m + r16, 32 * s, qd);
#pragma unroll
                    for (int cc = 0; cc < 2; ++cc) {
                        KS[m][cc] = mfma(ak, sh[cc], KS[m][cc]);
                        if (lo[m]) KS[m][cc] = mfma(ak, sl[cc], KS[m][cc]);
                    }
                }
            }
            // R = beta (V - exp(G) K S), in place of K S
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = 16 * m + 4 * qd + e;
                    const float bt = sm.Bt[cur][t], eg = sm.EG[cur][t];
#pragma unroll
                    for (int cc = 0; cc < 2; ++cc) {
                        const float vt = static_cast<float>(sm.V[sw128(t, 32 * w + 16 * cc + r16)]);
                        KS[m][cc][e] = bt * (vt - eg * KS[m][cc][e]);
                    }
                }
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int cc = 0; cc < 2; ++cc)
                    split_pk(KS[2 * s][cc], KS[2 * s + 1][cc], Rhi[s][cc], Rlo[s][cc]);
        }
        __syncthreads();

        // ================= phase B: D = T R; O = exp(G) Q S + A D =================
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
                    const bf16x8 th = pk64(Th, 16 * m + r16, 32 * s, qd);
                    const bf16x8 tl = pk64(Tl, 16 * m + r16, 32 * s, qd);
#pragma unroll
                    for (int cc = 0; cc < 2; ++cc)
                        Dt[m][cc] = mfma3(th, tl, Rhi[s][cc], Rlo[s][cc], Dt[m][cc]);
                }
            }
            // decayed deltas (state update operand), then D's own hi/lo parts
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) {
                    f32x4 a = Dt[2 * s][cc], b = Dt[2 * s + 1][cc];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        a[e] *= sm.EC[cur][32 * s + 4 * qd + e];
                        b[e] *= sm.EC[cur][32 * s + 16 + 4 * qd + e];
                    }
                    split_pk(a, b, Phi[s][cc], Plo[s][cc]);
                    split_pk(Dt[2 * s][cc], Dt[2 * s + 1][cc], Rhi[s][cc], Rlo[s][cc]);   // now D
                }
            f32x4 QS[4][2];
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) QS[m][cc] = zero4();
            bool lo[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) lo[m] = sm.lo_ks[cur][m];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                bf16x8 sh[2], sl[2];
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) split_pk(S[4 * s + cc], S[4 * s + 2 + cc], sh[cc], sl[cc]);
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const bf16x8 aq = pk128(sm.Q, 16 * m + r16, 32 * s, qd);
#pragma unroll
                    for (int cc = 0; cc < 2; ++cc) {
                        QS[m][cc] = mfma(aq, sh[cc], QS[m][cc]);
                        if (lo[m]) QS[m][cc] = mfma(aq, sl[cc], QS[m][cc]);
                    }
                }
            }
            const bf16 *Ah = sm.A[cur][0], *Al = sm.A[cur][1];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
#pragma unroll
                for (int cc = 0; cc < 2; ++cc)
#pragma unroll
                    for (int e = 0; e < 4; ++e) QS[m][cc][e] *= sm.EG[cur][16 * m + 4 * qd + e];
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    if (s > m / 2) continue;
                    const bf16x8 ah = pk64(Ah, 16 * m + r16, 32 * s, qd);
                    const bf16x8 al = pk64(Al, 16 * m + r16, 32 * s, qd);
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
            for (int i = 0; i < 8; ++i) {
#pragma unroll
                for (int cc = 0; cc < 2; ++cc)
#pragma unroll
                    for (int e = 0; e < 4; ++e) S[2 * i + cc][e] *= eC;
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const bf16x8 a = pkT128(Kc, 16 * i + r16, 32 * s, qd);
                    const bool lo = s ? lo1 : lo0;
#pragma unroll
                    for (int cc = 0; cc < 2; ++cc) {
                        S[2 * i + cc] = mfma(a, Phi[s][cc], S[2 * i + cc]);
                        if (lo) S[2 * i + cc] = mfma(a, Plo[s][cc], S[2 * i + cc]);
                    }
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
