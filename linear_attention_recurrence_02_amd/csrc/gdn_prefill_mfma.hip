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
// Mapping (one 256-thread workgroup = 4 waves per (sequence, head); the
// chunks of the sequence are walked in order with S held in registers):
//   * wave w owns dv columns [32w, 32w+32) of S, R, D and O.  Its share of S
//     lives as 8 x 2 accumulator tiles of v_mfma_f32_16x16x32_bf16 (16 dk rows
//     x 16 dv columns each, 4 fp32 per lane) and never leaves the registers
//     between the first and the last chunk.
//   * every state-dependent product keeps one operand in registers: an MFMA
//     result tile (lane holds rows 4q..4q+3 of column l%16, q = l/16) is
//     reused as the B operand of the next product over those rows by reading
//     the partner A operand with the matching permuted k order (lane group q
//     takes k = 4q..4q+3 and 16+4q..16+4q+3 of each 32-wide k step).
//   * the shared operands (K, Q, V, K^T, T, A) are staged in LDS once per
//     chunk; the Gram tiles K K^T and Q K^T are exact bf16 products with fp32
//     accumulation; T is built per chunk from 16x16 diagonal inverses (fp32
//     forward substitution) and the block recurrence
//     T_ij = -T_ii sum_{k=j}^{i-1} N_ik T_kj (one wave per column block).
//   * fp32 quantities that feed a bf16 MFMA (S, R, T, A, D, the decayed D) are
//     split x = hi + lo into two bf16 parts and multiplied as
//     hi*hi + hi*lo + lo*hi (or hi + lo against an exact bf16 operand), which
//     keeps products at ~2^-16 relative accuracy.  Where a row's scale factor
//     (exp(G_t) for K S and Q S, exp(G_C - G_t) for the state update) is below
//     2^-8 over a whole 16/32-row block, the lo term's contribution is below
//     2^-17 of the product and is not issued.

#include "gdn_internal.hpp"

namespace gdn {
namespace {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int C = 64;             // chunk length
constexpr int D = kHeadDim;       // 128
constexpr int RS = D + 8;         // bf16 row stride of K, Q, V staging (272 B)
constexpr int TS = C + 8;         // bf16 row stride of K^T, T, A (144 B)
constexpr int FS = C + 4;         // fp32 row stride of N (272 B)
constexpr int DS = 17;            // fp32 row stride of the 16x16 diagonal inverses
constexpr float kLoSkip = 1.0f / 256.0f;

struct Smem {
    bf16 K[C * RS], Q[C * RS], V[C * RS];
    bf16 KT[D * TS];                         // K transposed: [dk][token]
    bf16 Th[C * TS], Tl[C * TS];             // T = (I+N)^-1, hi and lo parts
    bf16 Ah[C * TS], Al[C * TS];             // decayed, masked Q K^T, hi and lo
    union {
        float N[C * FS];                     // strictly lower N (fp32), chunk setup
        bf16 O[C * RS];                      // output staging, after T is built
    } u;
    float Td[4 * 16 * DS];                   // fp32 diagonal 16x16 blocks of T
    float G[C], EG[C], EC[C], B[C];
    int lo_ks[4];                            // per 16-row token tile: exp(G) max >= 2^-8
    int lo_kd[2];                            // per 32-token step: exp(G_C - G) max >= 2^-8
};

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 cat4(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// A operand with the permuted k order: row `row` of a bf16 LDS matrix, k step
// starting at column kb; lane group q reads kb+4q..+3 and kb+16+4q..+3.
__device__ __forceinline__ bf16x8 read_pk(const bf16 *m, int stride, int row, int kb, int q) {
    const bf16 *p = m + row * stride + kb + 4 * q;
    return cat4(*reinterpret_cast<const bf16x4 *>(p), *reinterpret_cast<const bf16x4 *>(p + 16));
}

// hi/lo split of two result tiles (rows kb..kb+15 -> elements 0..3, rows
// kb+16..kb+31 -> elements 4..7), giving a B operand in the permuted k order.
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

// hi/lo split of one result tile used as a 16-deep B operand (elements 4..7 zero).
__device__ __forceinline__ void split_half(f32x4 a, bf16x8 &hi, bf16x8 &lo) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const bf16 h = static_cast<bf16>(a[e]);
        hi[e] = h;
        lo[e] = static_cast<bf16>(a[e] - static_cast<float>(h));
        hi[e + 4] = static_cast<bf16>(0.f);
        lo[e + 4] = static_cast<bf16>(0.f);
    }
}

// 16-deep A operand from an fp32 LDS matrix (row `row`, columns c0+4q..+3),
// split into hi/lo; elements 4..7 zero.
__device__ __forceinline__ void read_half_f32(const float *m, int stride, int row, int c0, int q,
                                              bf16x8 &hi, bf16x8 &lo) {
    const float *p = m + row * stride + c0 + 4 * q;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float x = p[e];
        const bf16 h = static_cast<bf16>(x);
        hi[e] = h;
        lo[e] = static_cast<bf16>(x - static_cast<float>(h));
        hi[e + 4] = static_cast<bf16>(0.f);
        lo[e + 4] = static_cast<bf16>(0.f);
    }
}

__device__ __forceinline__ f32x4 mfma3(bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl, f32x4 c) {
    c = mfma(ah, bh, c);
    c = mfma(ah, bl, c);
    return mfma(al, bh, c);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

__global__ __launch_bounds__(256) void prefill_mfma_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta,
    const float *__restrict__ S0, const int32_t *__restrict__ cu_seqlens, int64_t T,
    int64_t H, bf16 *__restrict__ O, float *__restrict__ S_T) {
    __shared__ Smem sm;

    const int tid = threadIdx.x;
    const int w = tid >> 6, l = tid & 63, r16 = l & 15, qd = l >> 4;
    const int64_t unit = blockIdx.x;
    const int64_t n = unit / H, h = unit % H;
    int64_t start, len;
    sequence_span(cu_seqlens, n, T, start, len);

    // The upper-triangular tiles of T and A stay zero for the whole walk.
    for (int i = tid; i < C * TS; i += 256) {
        sm.Th[i] = sm.Tl[i] = sm.Ah[i] = sm.Al[i] = static_cast<bf16>(0.f);
    }

    // State tiles: S[i][c] holds rows 16i+4q+e, column 32w+16c+r16.
    f32x4 S[8][2];
    {
        const float *S0u = S0 ? S0 + unit * (D * D) : nullptr;
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    S[i][c][e] = S0u ? S0u[(16 * i + 4 * qd + e) * D + 32 * w + 16 * c + r16] : 0.f;
    }

    for (int64_t c0 = 0; c0 < len; c0 += C) {
        const int nv = static_cast<int>(len - c0 < C ? len - c0 : C);
        const int64_t row0 = start + c0;

        // ---- stage K, Q, V (and K^T) of the chunk; scan the log-decay ----
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int p = tid + 256 * r;
            const int row = p >> 4, cc = p & 15;
            bf16x8 kv, qv, vv;
            if (row < nv) {
                const int64_t off = ((row0 + row) * H + h) * D + cc * 8;
                kv = *reinterpret_cast<const bf16x8 *>(k + off);
                qv = *reinterpret_cast<const bf16x8 *>(q + off);
                vv = *reinterpret_cast<const bf16x8 *>(v + off);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) kv[e] = qv[e] = vv[e] = static_cast<bf16>(0.f);
            }
            *reinterpret_cast<bf16x8 *>(&sm.K[row * RS + cc * 8]) = kv;
            *reinterpret_cast<bf16x8 *>(&sm.Q[row * RS + cc * 8]) = qv;
            *reinterpret_cast<bf16x8 *>(&sm.V[row * RS + cc * 8]) = vv;
#pragma unroll
            for (int e = 0; e < 8; ++e) sm.KT[(cc * 8 + e) * TS + row] = kv[e];
        }
        if (w == 0) {
            const bool ok = l < nv;
            float x = ok ? g[(row0 + l) * H + h] : 0.f;
            const float bt = ok ? beta[(row0 + l) * H + h] : 0.f;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(x, off);
                if (l >= off) x += y;
            }
            const float Gc = __shfl(x, 63);
            const float eg = expf(x), ec = expf(Gc - x);
            sm.G[l] = x;
            sm.EG[l] = eg;
            sm.EC[l] = ec;
            sm.B[l] = bt;
            // block maxima of the two scale factors (16-row and 32-row groups)
            float m16 = eg, m32 = ec;
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) m16 = fmaxf(m16, __shfl_xor(m16, off));
#pragma unroll
            for (int off = 1; off < 32; off <<= 1) m32 = fmaxf(m32, __shfl_xor(m32, off));
            if ((l & 15) == 0) sm.lo_ks[l >> 4] = m16 >= kLoSkip;
            if ((l & 31) == 0) sm.lo_kd[l >> 5] = m32 >= kLoSkip;
        }
        __syncthreads();

        // ---- Gram tiles: N (from K K^T) and A (from Q K^T), lower tiles only ----
        for (int job = w; job < 20; job += 4) {
            const int kind = job / 10, idx = job % 10;
            const int mi = idx < 1 ? 0 : idx < 3 ? 1 : idx < 6 ? 2 : 3;
            const int mj = idx - (mi * (mi + 1)) / 2;
            const bf16 *X = kind ? sm.Q : sm.K;
            f32x4 acc = zero4();
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(&X[(16 * mi + r16) * RS + 32 * s + 8 * qd]);
                const bf16x8 b = *reinterpret_cast<const bf16x8 *>(&sm.K[(16 * mj + r16) * RS + 32 * s + 8 * qd]);
                acc = mfma(a, b, acc);
            }
            const int jj = 16 * mj + r16;
            const float Gj = sm.G[jj];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 16 * mi + 4 * qd + e;
                const float E = jj <= t ? expf(sm.G[t] - Gj) : 0.f;
                if (kind == 0) {
                    sm.u.N[t * FS + jj] = jj < t ? sm.B[t] * (E * acc[e]) : 0.f;
                } else {
                    const float a = E * acc[e];
                    const bf16 hi = static_cast<bf16>(a);
                    sm.Ah[t * TS + jj] = hi;
                    sm.Al[t * TS + jj] = static_cast<bf16>(a - static_cast<float>(hi));
                }
            }
        }
        __syncthreads();

        // ---- state-dependent, T-independent: K S, Q S, R ----
        bf16x8 Shi[4][2], Slo[4][2];
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int c = 0; c < 2; ++c) split_pk(S[2 * s][c], S[2 * s + 1][c], Shi[s][c], Slo[s][c]);

        f32x4 QS[4][2];
        bf16x8 Rhi[2][2], Rlo[2][2];
        {
            f32x4 KS[4][2];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const bool lo = sm.lo_ks[m];
#pragma unroll
                for (int c = 0; c < 2; ++c) KS[m][c] = QS[m][c] = zero4();
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const bf16x8 ak = read_pk(sm.K, RS, 16 * m + r16, 32 * s, qd);
                    const bf16x8 aq = read_pk(sm.Q, RS, 16 * m + r16, 32 * s, qd);
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        KS[m][c] = mfma(ak, Shi[s][c], KS[m][c]);
                        QS[m][c] = mfma(aq, Shi[s][c], QS[m][c]);
                        if (lo) {
                            KS[m][c] = mfma(ak, Slo[s][c], KS[m][c]);
                            QS[m][c] = mfma(aq, Slo[s][c], QS[m][c]);
                        }
                    }
                }
            }
            // R = beta (V - exp(G) K S), in result-tile layout
            f32x4 R[4][2];
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int c = 0; c < 2; ++c)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int t = 16 * m + 4 * qd + e;
                        const float vt = static_cast<float>(sm.V[t * RS + 32 * w + 16 * c + r16]);
                        R[m][c][e] = sm.B[t] * (vt - sm.EG[t] * KS[m][c][e]);
                    }
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int c = 0; c < 2; ++c) split_pk(R[2 * s][c], R[2 * s + 1][c], Rhi[s][c], Rlo[s][c]);
        }

        // ---- T = (I + N)^-1: diagonal 16x16 blocks by forward substitution ----
        if (w == 3) {
            const int b = qd, j = r16;       // block b, column j of its inverse
            float x[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) x[t] = t == j ? 1.f : 0.f;
#pragma unroll
            for (int t = 0; t < 16; ++t)
#pragma unroll
                for (int u = t + 1; u < 16; ++u)
                    x[u] -= sm.u.N[(16 * b + u) * FS + 16 * b + t] * x[t];
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                sm.Td[(b * 16 + t) * DS + j] = x[t];
                const bf16 hi = static_cast<bf16>(x[t]);
                sm.Th[(16 * b + t) * TS + 16 * b + j] = hi;
                sm.Tl[(16 * b + t) * TS + 16 * b + j] = static_cast<bf16>(x[t] - static_cast<float>(hi));
            }
        }
        __syncthreads();

        // ---- T off-diagonal blocks: wave j walks column block j ----
        if (w < 3) {
            const int j = w;
            f32x4 Tc[4];                         // T_ij tiles of this column block, i > j
#pragma unroll
            for (int i = 1; i < 4; ++i) {
                if (i <= j) continue;
                f32x4 Z = zero4();
#pragma unroll
                for (int kk = 0; kk < 3; ++kk) {
                    if (kk < j || kk >= i) continue;
                    bf16x8 ah, al, bh, bl;
                    read_half_f32(sm.u.N, FS, 16 * i + r16, 16 * kk, qd, ah, al);
                    if (kk == j) {
                        // B = T_jj from the fp32 diagonal store: rows 4q+e, column r16
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float x = sm.Td[(j * 16 + 4 * qd + e) * DS + r16];
                            const bf16 hx = static_cast<bf16>(x);
                            bh[e] = hx;
                            bl[e] = static_cast<bf16>(x - static_cast<float>(hx));
                            bh[e + 4] = bl[e + 4] = static_cast<bf16>(0.f);
                        }
                    } else {
                        split_half(Tc[kk], bh, bl);
                    }
                    Z = mfma3(ah, al, bh, bl, Z);
                }
                bf16x8 ah, al, bh, bl;
                read_half_f32(sm.Td, DS, i * 16 + r16, 0, qd, ah, al);   // T_ii rows
                split_half(Z, bh, bl);
                f32x4 Tij = mfma3(ah, al, bh, bl, zero4());
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    Tij[e] = -Tij[e];
                    const int t = 16 * i + 4 * qd + e, col = 16 * j + r16;
                    const bf16 hi = static_cast<bf16>(Tij[e]);
                    sm.Th[t * TS + col] = hi;
                    sm.Tl[t * TS + col] = static_cast<bf16>(Tij[e] - static_cast<float>(hi));
                }
                Tc[i] = Tij;
            }
        }
        __syncthreads();

        // ---- D = T R; O = exp(G) Q S + A D ----
        f32x4 Dt[4][2];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
#pragma unroll
            for (int c = 0; c < 2; ++c) Dt[m][c] = zero4();
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                if (s > m / 2) continue;
                const bf16x8 th = read_pk(sm.Th, TS, 16 * m + r16, 32 * s, qd);
                const bf16x8 tl = read_pk(sm.Tl, TS, 16 * m + r16, 32 * s, qd);
#pragma unroll
                for (int c = 0; c < 2; ++c) Dt[m][c] = mfma3(th, tl, Rhi[s][c], Rlo[s][c], Dt[m][c]);
            }
        }
        bf16x8 Dhi[2][2], Dlo[2][2];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int c = 0; c < 2; ++c) split_pk(Dt[2 * s][c], Dt[2 * s + 1][c], Dhi[s][c], Dlo[s][c]);

#pragma unroll
        for (int m = 0; m < 4; ++m) {
            f32x4 Ot[2];
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int e = 0; e < 4; ++e) Ot[c][e] = sm.EG[16 * m + 4 * qd + e] * QS[m][c][e];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                if (s > m / 2) continue;
                const bf16x8 ah = read_pk(sm.Ah, TS, 16 * m + r16, 32 * s, qd);
                const bf16x8 al = read_pk(sm.Al, TS, 16 * m + r16, 32 * s, qd);
#pragma unroll
                for (int c = 0; c < 2; ++c) Ot[c] = mfma3(ah, al, Dhi[s][c], Dlo[s][c], Ot[c]);
            }
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sm.u.O[(16 * m + 4 * qd + e) * RS + 32 * w + 16 * c + r16] = static_cast<bf16>(Ot[c][e]);
        }

        // ---- S <- exp(G_C) S + K^T diag(exp(G_C - G)) D ----
        {
            bf16x8 Phi[2][2], Plo[2][2];
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    f32x4 a = Dt[2 * s][c], b = Dt[2 * s + 1][c];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        a[e] *= sm.EC[32 * s + 4 * qd + e];
                        b[e] *= sm.EC[32 * s + 16 + 4 * qd + e];
                    }
                    split_pk(a, b, Phi[s][c], Plo[s][c]);
                }
            const float eC = sm.EG[C - 1];
            const bool lo0 = sm.lo_kd[0], lo1 = sm.lo_kd[1];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
#pragma unroll
                for (int c = 0; c < 2; ++c)
#pragma unroll
                    for (int e = 0; e < 4; ++e) S[i][c][e] *= eC;
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const bf16x8 a = read_pk(sm.KT, TS, 16 * i + r16, 32 * s, qd);
                    const bool lo = s ? lo1 : lo0;
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        S[i][c] = mfma(a, Phi[s][c], S[i][c]);
                        if (lo) S[i][c] = mfma(a, Plo[s][c], S[i][c]);
                    }
                }
            }
        }
        __syncthreads();

        // ---- store the chunk's output rows (16 bytes per lane, coalesced) ----
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int p = tid + 256 * r;
            const int row = p >> 4, cc = p & 15;
            if (row < nv)
                *reinterpret_cast<bf16x8 *>(O + ((row0 + row) * H + h) * D + cc * 8) =
                    *reinterpret_cast<const bf16x8 *>(&sm.u.O[row * RS + cc * 8]);
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
                STu[(16 * i + 4 * qd + e) * D + 32 * w + 16 * c + r16] = S[i][c][e];
}

}  // namespace

bool prefill_mfma_supports(const PrefillArgs &a) { return a.bf16 && a.chunk == C; }

hipError_t launch_prefill_mfma(const PrefillArgs &a, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(a.N * a.H)), block(256);
    prefill_mfma_kernel<<<grid, block, 0, stream>>>(
        static_cast<const bf16 *>(a.q), static_cast<const bf16 *>(a.k),
        static_cast<const bf16 *>(a.v), a.g, a.beta, a.S0, a.cu_seqlens, a.T, a.H,
        static_cast<bf16 *>(a.O), a.S_T);
    return hipGetLastError();
}

}  // namespace gdn
