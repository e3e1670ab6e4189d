// Prompt form for batches of short sequences (bf16 inputs, fp32 state): the
// chunks are 16 tokens, and one 256-thread workgroup per (sequence, head)
// needs about 21 KB of LDS and at most 256 registers a lane, so that two
// workgroups share a CU (the 64-token kernel's 512-thread workgroup fills
// one) and the loads and stores of their states overlap.  A verify block (16
// tokens from a stored state) is one chunk: its cost is the state read and
// write.
//
// The form (Qwen3.5-9B-npu model page, "How it works" -> "Gated DeltaNet on
// the NPU"), per chunk with incoming state S (dk x dv):
//     G = cumsum(g) (inclusive),  N = diag(beta) [exp(G_t - G_j) k_t.k_j]_{j<t},
//     T = (I + N)^-1,  W = T diag(beta exp G) K,  U = T diag(beta) V,
//     D = U - W S,
//     O = diag(exp G) Q S + A D,  A = [exp(G_t - G_j) q_t.k_j]_{j<=t},
//     S <- exp(G_C) S + K^T diag(exp(G_C - G)) D.
// Rows past a sequence's end are zero rows with g = 0 and beta = 0 (the
// page's token_valid padding); they change nothing and are not stored.
//
// Wave w owns dv columns [32w, 32w+32) of S, U, D and O, its share of S held
// in 8 x 2 result tiles of v_mfma_f32_16x16x32_f16 for the whole walk (lane
// l: rows 4(l/16)..+3 of column l%16 of each 16 x 16 tile).  Per chunk:
//   1. all waves stage K, Q (fp16) and V (bf16) in LDS; wave 0 scans the
//      log-decay;
//   2. wave 0 forms K K^T -> N and T = (I + N)^-1 by forward substitution in
//      fp32 (one column per lane), scaled to P = T diag(beta exp G) and
//      P' = T diag(beta); wave 1 forms Q K^T -> A;
//   3. each wave forms W = P K for 32 dk columns (to LDS) and U = P' V for its
//      own dv columns (kept in registers);
//   4. each wave: D = U - W S, O = diag(exp G) Q S + A D (as O^T, so that a
//      lane ends with four adjacent columns of one token row), and the state
//      update.
// The state is loaded before the first chunk is staged and first used in
// step 4, so its load overlaps steps 1 to 3.  A null v stands for zero values
// and a null O for no output rows.
//
// Precision.  Sums are fp32; the state, D and U are fp32 between products.
// K and Q enter the products as fp16 copies of the bf16 inputs (exact for
// unit-scale keys and queries), V as the bf16 input itself.  Correlated keys
// make the chunk's deltas D large next to the quantities built from them (the
// terms of A D and of K^T D nearly cancel), so an operand rounded once to fp16
// (2^-11 relative) is not enough where it multiplies D or enters D: P, A, D and
// the decayed D are split into fp16 hi + lo pairs, and P' into a bf16 pair
// (against the bf16 V).  S and W stay single fp16 operands.  Each wave holds
// its value-side quantities (its state columns, U, D, O) at a power-of-two
// scale chosen per chunk so that their largest entry lies in [8, 16): the fp16
// operands then have their full precision relative to it, whatever the
// magnitude of the values and states passed in.  Scaling by a power of two is
// exact; O and S_T are unscaled when stored.

#include "gdn_mfma.hpp"

namespace gdn {
namespace {

constexpr int CS = 16;            // chunk length
constexpr int D = kHeadDim;       // 128
constexpr int RS = D + 8;         // fp16 row stride of the token-major K, Q, V, W tiles
constexpr int TS = CS + 4;        // fp16 row stride of the 16 x 16 tiles A, P, P'
constexpr int NS = CS + 4;        // fp32 row stride of N (16-byte aligned rows)

struct __attribute__((aligned(16))) ShortSmem {
    f16 K[CS * RS];
    f16 Q[CS * RS];
    bf16 V[CS * RS];              // the bf16 inputs as they are
    f16 W[CS * RS];               // -W, token-major
    f16 A[2][CS * TS];            // decayed masked Q K^T, token-major: hi, lo
    f16 P[2][CS * TS];            // T diag(beta exp G): hi, lo
    bf16 Pv[2][CS * TS];          // T diag(beta): hi, lo
    float N[CS * NS];             // strictly lower N
    float G2[CS];                 // cumsum(g) * log2(e)
    float Bt[CS];                 // beta
    float EG[CS];                 // exp(G_t)
    float EC[CS];                 // exp(G_last - G_t)
};

template <typename OutT>
__global__ __launch_bounds__(256, 2) void prefill_short_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, const float *__restrict__ S0,
    const int32_t *__restrict__ cu_seqlens, int64_t T, int64_t H, OutT *__restrict__ O,
    float *__restrict__ S_T) {
    __shared__ ShortSmem sm;
    const int tid = threadIdx.x;
    const int w = tid >> 6, l = tid & 63, r16 = l & 15, qd = l >> 4;
    const int64_t unit = blockIdx.x, seq = unit / H, h = unit % H;
    int64_t start, len;
    sequence_span(cu_seqlens, seq, T, start, len);
    const int nch = static_cast<int>((len + CS - 1) / CS);

    // S[i][c]: state rows 16i + 4qd + e, column 32w + 16c + r16
    f32x4 S[8][2];
    if (S0) {
        const float *S0u = S0 + unit * (D * D);
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    S[i][c][e] = S0u[(16 * i + 4 * qd + e) * D + 32 * w + 16 * c + r16];
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) S[i][0] = S[i][1] = zero4();
    }
    // S holds the state at scale 2^sc_exp (wave-uniform)
    int sc_exp = 0;
    float *STu = S_T + unit * (D * D);
    auto store_state = [&]() {
        const float un = pow2i(-sc_exp);
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    STu[(16 * i + 4 * qd + e) * D + 32 * w + 16 * c + r16] = S[i][c][e] * un;
    };
    if (nch == 0) {
        store_state();
        return;
    }

    // Staging: thread t moves columns 8 (t % 16)..+7 of row t / 16 of K, Q
    // and V; lane r16 of wave 0 reads token r16's g and beta.  Rows past the
    // sequence read its first row (in bounds) and are zeroed when staged.
    const int sr = tid >> 4, sc = 8 * (tid & 15);
    f32x4 xk, xq, xv;
    float xg = 0.f, xb = 0.f;
    auto rows_in = [&](int c) {
        const int64_t rem = len - int64_t(c) * CS;
        return static_cast<int>(rem < CS ? rem : CS);
    };
    auto fetch = [&](int c) {
        const int nv = rows_in(c);
        const int64_t row = sr < nv ? start + int64_t(c) * CS + sr : start;
        const int64_t off = (row * H + h) * D + sc;
        xk = *reinterpret_cast<const f32x4 *>(k + off);
        xq = *reinterpret_cast<const f32x4 *>(q + off);
        xv = v ? *reinterpret_cast<const f32x4 *>(v + off) : zero4();
        if (w == 0) {
            const int64_t gi = (r16 < nv ? start + int64_t(c) * CS + r16 : start) * H + h;
            xg = g[gi];
            xb = beta[gi];
        }
    };
    fetch(0);

    for (int c = 0; c < nch; ++c) {
        const int nv = rows_in(c);
        // ---- 1. stage the chunk ----
        {
            const bool ok = sr < nv;
            const f32x4 hk = ok ? __builtin_bit_cast(f32x4, bf_to_h8(xk)) : zero4();
            const f32x4 hq = ok ? __builtin_bit_cast(f32x4, bf_to_h8(xq)) : zero4();
            const f32x4 hv = ok ? xv : zero4();
            *reinterpret_cast<f32x4 *>(&sm.K[sr * RS + sc]) = hk;
            *reinterpret_cast<f32x4 *>(&sm.Q[sr * RS + sc]) = hq;
            *reinterpret_cast<f32x4 *>(&sm.V[sr * RS + sc]) = hv;
        }
        float bt = 0.f, eg = 0.f;          // wave 0: token r16's beta and exp(G)
        if (w == 0) {
            const bool ok = r16 < nv;
            bt = ok ? xb : 0.f;
            const float g2 = log2e_times(row16_prefix_sum(ok ? bounded_log_decay(xg) : 0.f));
            const float last = __builtin_bit_cast(
                float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, g2), CS - 1));
            eg = __builtin_amdgcn_exp2f(g2);
            if (qd == 0) {
                sm.G2[r16] = g2;
                sm.Bt[r16] = bt;
                sm.EG[r16] = eg;
                sm.EC[r16] = __builtin_amdgcn_exp2f(last - g2);
            }
        }
        if (c + 1 < nch) fetch(c + 1);
        __syncthreads();

        // ---- 2. N, T (wave 0) and A (wave 1) ----
        if (w < 2) {
            const f16 *X = w == 0 ? sm.K : sm.Q;
            f32x4 acc = zero4();
#pragma unroll
            for (int s = 0; s < 4; ++s)
                acc = mfma(rd8(X + r16 * RS + 32 * s + 8 * qd), rd8(sm.K + r16 * RS + 32 * s + 8 * qd), acc);
            // acc[e] = x_t . k_j with t = 4qd + e (row), j = r16 (column)
            constexpr float kNegInf = -__builtin_huge_valf();
            const f32x4 g2t = *reinterpret_cast<const f32x4 *>(&sm.G2[4 * qd]);
            const float g2j = sm.G2[r16];
            if (w == 0) {
                const f32x4 btt = *reinterpret_cast<const f32x4 *>(&sm.Bt[4 * qd]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = 4 * qd + e;
                    sm.N[t * NS + r16] =
                        btt[e] * (__builtin_amdgcn_exp2f(r16 < t ? g2t[e] - g2j : kNegInf) * acc[e]);
                }
                // T = (I + N)^-1, column r16 per lane: T_ic = [i == c] - sum_{j<i} N_ij T_jc.
                // The rows read below were stored by other lanes of this wave: the
                // wave's LDS operations complete in order, and the fence keeps the
                // compiler from moving the reads above the stores.
                __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
                float tc[CS];
#pragma unroll
                for (int i = 0; i < CS; ++i) {
                    float x = i == r16 ? 1.f : 0.f;
#pragma unroll
                    for (int j4 = 0; j4 < i; j4 += 4) {
                        const f32x4 n4 = *reinterpret_cast<const f32x4 *>(&sm.N[i * NS + j4]);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (j4 + e < i) x -= n4[e] * tc[j4 + e];
                    }
                    tc[i] = x;
                }
                if (qd == 0) {
                    const float sp = bt * eg;
#pragma unroll
                    for (int i = 0; i < CS; ++i) {
                        const float p = tc[i] * sp, pv = tc[i] * bt;
                        const f16 ph = static_cast<f16>(p);
                        const bf16 pvh = static_cast<bf16>(pv);
                        sm.P[0][i * TS + r16] = ph;
                        sm.P[1][i * TS + r16] = static_cast<f16>(p - static_cast<float>(ph));
                        sm.Pv[0][i * TS + r16] = pvh;
                        sm.Pv[1][i * TS + r16] = static_cast<bf16>(pv - static_cast<float>(pvh));
                    }
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = 4 * qd + e;
                    const float a = __builtin_amdgcn_exp2f(r16 <= t ? g2t[e] - g2j : kNegInf) * acc[e];
                    const f16 ah = static_cast<f16>(a);
                    sm.A[0][t * TS + r16] = ah;
                    sm.A[1][t * TS + r16] = static_cast<f16>(a - static_cast<float>(ah));
                }
            }
        }
        __syncthreads();

        // ---- 3. W = P K (dk columns 32w..), U = P' V (this wave's dv columns) ----
        // transpose load: lane (r16, qd) receives X[4qd..4qd+3][16b + r16]
        const int trow = (4 * qd + (r16 >> 2)) * RS + 4 * (r16 & 3);
        f32x4 U[2];
        {
            const f16x8 pa = cat(rd4(sm.P[0] + r16 * TS + 4 * qd), rd4(sm.P[1] + r16 * TS + 4 * qd));
            const bf16x8 pva = catb(*reinterpret_cast<const bf16x4 *>(sm.Pv[0] + r16 * TS + 4 * qd),
                                    *reinterpret_cast<const bf16x4 *>(sm.Pv[1] + r16 * TS + 4 * qd));
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) {
                const int b = 2 * w + bb;
                const f16x4 kt = rd_tr(sm.K + trow + 16 * b);
                const f32x4 wt = mfma(pa, cat(kt, kt), zero4());
#pragma unroll
                for (int e = 0; e < 4; ++e) sm.W[(4 * qd + e) * RS + 16 * b + r16] = static_cast<f16>(-wt[e]);
                const bf16x4 vt = __builtin_bit_cast(bf16x4, rd_tr(reinterpret_cast<const f16 *>(sm.V) + trow + 16 * b));
                U[bb] = mfma_bf(pva, catb(vt, vt), zero4());
            }
        }
        __syncthreads();

        // ---- the wave's scale for this chunk: its state columns (held at
        // 2^sc_exp) and U (unscaled) ----
        {
            float ms = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) ms = absmax4(S[i][1], absmax4(S[i][0], ms));
            const float mu = absmax4(U[1], absmax4(U[0], 0.f));
            const float m = wave_max_nonneg(fmax_ieee(ms * pow2i(-sc_exp), mu));
            const int nx = choose_scale(0.f, sc_exp, m);
            if (nx != sc_exp) {
                const float f = pow2i(nx - sc_exp);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    S[i][0] *= f;
                    S[i][1] *= f;
                }
                sc_exp = nx;
            }
        }

        // ---- 4. D = U - W S; O = diag(exp G) Q S + A D; state update ----
        const float up = pow2i(sc_exp);
        f32x4 Dt[2] = {U[0] * up, U[1] * up};
        f32x4 Ot[2] = {zero4(), zero4()};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const f16 *wp = sm.W + r16 * RS + 32 * s + 4 * qd;
            const f16 *qp = sm.Q + r16 * RS + 32 * s + 4 * qd;
            const f16x8 wa = cat(rd4(wp), rd4(wp + 16));
            const f16x8 qb = cat(rd4(qp), rd4(qp + 16));
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                // k = 32s + 4qd..+3 and 32s + 16 + 4qd..+3: the matching order
                const f16x8 sh = cat(h4(S[2 * s][cc]), h4(S[2 * s + 1][cc]));
                Dt[cc] = mfma(wa, sh, Dt[cc]);
                Ot[cc] = mfma(sh, qb, Ot[cc]);
            }
        }
        {
            // A D with both split: (D_hi + D_lo) A_hi + D_hi A_lo
            const float egt = sm.EG[r16];
            const f16x4 ah = rd4(sm.A[0] + r16 * TS + 4 * qd), al = rd4(sm.A[1] + r16 * TS + 4 * qd);
            const float un = pow2i(-sc_exp);
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                const h4x2 d = split_h4(Dt[cc]);
                Ot[cc] = mfma(cat(d.hi, d.lo), cat(ah, ah), Ot[cc] * egt);
                Ot[cc] = mfma16(d.hi, al, Ot[cc]) * un;
            }
            if (O && r16 < nv) {
                OutT *orow = O + ((start + int64_t(c) * CS + r16) * H + h) * D + 32 * w + 4 * qd;
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) {
                    if constexpr (sizeof(OutT) == 4)
                        *reinterpret_cast<f32x4 *>(orow + 16 * cc) = Ot[cc];
                    else
                        *reinterpret_cast<bf16x4 *>(orow + 16 * cc) = __builtin_convertvector(Ot[cc], bf16x4);
                }
            }
        }
        {
            const f32x4 ect = *reinterpret_cast<const f32x4 *>(&sm.EC[4 * qd]);
            const float eC = sm.EG[CS - 1];
            f16x8 Dp[2];
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                const h4x2 d = split_h4(Dt[cc] * ect);
                Dp[cc] = cat(d.hi, d.lo);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const f16x4 ka = rd_tr(sm.K + trow + 16 * i);
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) S[i][cc] = mfma(cat(ka, ka), Dp[cc], S[i][cc] * eC);
            }
        }
        __syncthreads();
    }
    store_state();
}

}  // namespace

// Whether a call is a batch of short sequences: at most 16 rows per sequence
// on average (a uniform batch of at most 16 tokens, or a packed batch with
// T <= 16 N), so that most sequences are one chunk of this kernel.  Not for
// the gated output (no norm epilogue here) or when the caller has named the
// 64-token kernel's inverse method.
bool prefill_short_pays(const PrefillArgs &a) {
    if (!a.bf16 || a.z || !a.short_ok) return false;
    return a.cu_seqlens ? a.T <= int64_t(CS) * a.N : a.T <= CS;
}

hipError_t launch_prefill_short(const PrefillArgs &a, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(a.N * a.H)), block(256);
    const bf16 *q = static_cast<const bf16 *>(a.q), *k = static_cast<const bf16 *>(a.k),
               *v = static_cast<const bf16 *>(a.v);
    if (a.out_f32)
        prefill_short_kernel<float><<<grid, block, 0, stream>>>(q, k, v, a.g, a.beta, a.S0, a.cu_seqlens,
                                                                a.T, a.H, static_cast<float *>(a.O), a.S_T);
    else
        prefill_short_kernel<bf16><<<grid, block, 0, stream>>>(q, k, v, a.g, a.beta, a.S0, a.cu_seqlens,
                                                               a.T, a.H, static_cast<bf16 *>(a.O), a.S_T);
    return hipGetLastError();
}

}  // namespace gdn
