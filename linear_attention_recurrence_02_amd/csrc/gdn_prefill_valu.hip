// Chunkwise-parallel prompt form on the vector ALUs, all arithmetic in fp32
// (the in-chunk cumulative log-decay in fp64).  This kernel serves fp32 inputs
// and the 16/32-token chunk sizes; bf16 inputs at 64-token chunks go to the
// matrix-core kernel.
//
// The form (Qwen3.5-9B-npu model page, "How it works" -> "Gated DeltaNet on
// the NPU"), per chunk of C tokens with incoming state S:
//     G   = cumsum(g)                                   (inclusive)
//     N   = diag(beta) [exp(G_t - G_j) k_t.k_j]_{j<t}    (strictly lower)
//     D   = (I + N)^-1 diag(beta) (V - diag(exp G) K S)
//     O   = diag(exp G) Q S + [exp(G_t - G_j) q_t.k_j]_{j<=t} D
//     S  <- exp(G_last) S + K^T diag(exp(G_last - G)) D
// Rows past the end of a sequence carry g = 0, beta = 0 and zero q/k/v (the
// page's token_valid padding), so a partial last chunk leaves S exactly as after
// the last real token.
//
// Work split: one 512-thread workgroup per (sequence, head).  Column j of the
// state (and of D and O) belongs to the four lanes of one quad; lane p of the
// quad holds the 32 state rows whose 16-byte groups are p, p + 4, ..., p + 28
// (rows 16m + 4p .. 16m + 4p + 3, m = 0..7), so each product of a key or query
// row with the column is four partial sums of 32 terms, added across the quad
// by two DPP exchanges.  The forward substitution for D runs down the column
// token by token inside the quad (every lane computes the same value and
// stores it to LDS, so that no lane depends on another's store), with no
// barrier.  The chunk's K and Q (fp32, 16-byte
// rows of 132 words: the four lanes of a quad read four distinct bank groups),
// D, N and the masked decayed Q K^T live in LDS; the chunk's V is staged into
// D's rows with K and Q, so the per-token loop reads no global memory.  The
// Gram entries are computed the same way, one entry per quad.
//
// A null v stands for zero values and a null O for no output rows.
//
// With the gated RMS norm on the output (the norm a Gated DeltaNet block
// applies after the recurrence), each output row is reduced across the
// workgroup as it is produced (one barrier per row, partial sums
// double-buffered by row parity) and stored as
// w_j o_j / sqrt(mean(o^2) + eps) silu(z_j).

#include "gdn_internal.hpp"

namespace gdn {
namespace {

constexpr int kThreads = 512;                      // 8 waves, 128 quads
constexpr int kQuads = kThreads / 4;
constexpr int kRows = kHeadDim / 4;                // state rows per lane
constexpr int kRow = kHeadDim + 4;                 // LDS row stride of K and Q (16-byte rows)

// Sum over the four lanes of a quad, returned to all four (the same bits in
// each: both steps add two values whose order does not change the sum).
__device__ __forceinline__ float quad_sum(float x) {
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xb1, 0xf, 0xf, false));   // quad_perm [1,0,3,2]
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4e, 0xf, 0xf, false));   // quad_perm [2,3,0,1]
    return x;
}

// Lane p's part of the product of a 128-word LDS row (16-byte aligned) with
// the 32 values x it holds for its state rows: four partial chains.
__device__ __forceinline__ float part_dot(const float *row, const float *x, int p) {
    const float4 *r4 = reinterpret_cast<const float4 *>(row);
    float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < kRows / 4; ++m) {
        const float4 r = r4[4 * m + p];
        a[0] += r.x * x[4 * m];
        a[1] += r.y * x[4 * m + 1];
        a[2] += r.z * x[4 * m + 2];
        a[3] += r.w * x[4 * m + 3];
    }
    return (a[0] + a[1]) + (a[2] + a[3]);
}

template <typename IO, typename OutT, int C, bool kGated>
__global__ __launch_bounds__(kThreads) void prefill_valu_kernel(
    const IO *__restrict__ q, const IO *__restrict__ k, const IO *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta,
    const float *__restrict__ S0, const int32_t *__restrict__ cu_seqlens, int64_t T,
    int64_t H, OutT *__restrict__ O, float *__restrict__ S_T, const IO *__restrict__ z,
    const float *__restrict__ norm_w, float eps) {
    static_assert((C * C) % kQuads == 0, "Gram entries per quad");
    __shared__ __attribute__((aligned(16))) float sK[C * kRow];
    __shared__ __attribute__((aligned(16))) float sQ[C * kRow];
    __shared__ float sD[C * kHeadDim];
    __shared__ float sN[C * C], sA[C * C];
    __shared__ double sG[C];
    __shared__ float sg[C], sB[C], sEG[C], sEC[C];
    __shared__ float sRed[2][kThreads / 64];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int j = 16 * wv + (lane >> 2);           // the quad's state column
    const int p = lane & 3;                        // the lane's row part
    auto row_of = [&](int m) { return 16 * (m >> 2) + 4 * p + (m & 3); };
    const int64_t unit = blockIdx.x;
    const int64_t n = unit / H, h = unit % H;
    int64_t start, len;
    sequence_span(cu_seqlens, n, T, start, len);

    const float nw = kGated ? norm_w[j] : 0.f;
    float S[kRows];
    const float *S0u = S0 ? S0 + unit * (kHeadDim * kHeadDim) : nullptr;
#pragma unroll
    for (int m = 0; m < kRows; ++m) S[m] = S0u ? S0u[row_of(m) * kHeadDim + j] : 0.f;

    // The rows of a chunk (zero past the sequence's end) are loaded into
    // registers a chunk ahead: thread tid holds elements tid + 512 e of the
    // chunk's C x 128 K, Q and V, and (tid < C) token tid's g and beta.
    constexpr int kPer = C * kHeadDim / kThreads;
    float xk[kPer], xq[kPer], xv[kPer], xg = 0.f, xb = 0.f;
    auto fetch = [&](int64_t c0n) {
        const int64_t rem = len - c0n;
        const int nvn = static_cast<int>(rem < 0 ? 0 : (rem < C ? rem : C));
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
            const int idx = tid + kThreads * e, t = idx / kHeadDim, i = idx % kHeadDim;
            xk[e] = xq[e] = xv[e] = 0.f;
            if (t < nvn) {
                const int64_t off = ((start + c0n + t) * H + h) * kHeadDim + i;
                xk[e] = to_f32(k[off]);
                xq[e] = to_f32(q[off]);
                if (v) xv[e] = to_f32(v[off]);
            }
        }
        if (tid < C) {
            const bool ok = tid < nvn;
            xg = ok ? g[(start + c0n + tid) * H + h] : 0.f;
            xb = ok ? beta[(start + c0n + tid) * H + h] : 0.f;
        }
    };
    if (len > 0) fetch(0);

    for (int64_t c0 = 0; c0 < len; c0 += C) {
        const int nv = static_cast<int>(len - c0 < C ? len - c0 : C);
        const int64_t row0 = start + c0;   // first token row of this chunk

        // stage the chunk's rows (V into D's rows, where each column is
        // overwritten by its own quad), then load the next chunk's
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
            const int idx = tid + kThreads * e, t = idx / kHeadDim, i = idx % kHeadDim;
            sK[t * kRow + i] = xk[e];
            sQ[t * kRow + i] = xq[e];
            sD[t * kHeadDim + i] = xv[e];
        }
        if (tid < C) {
            sg[tid] = xg;
            sB[tid] = xb;
        }
        if (c0 + C < len) fetch(c0 + C);
        __syncthreads();
        if (tid == 0) {
            double acc = 0.0;
            for (int t = 0; t < C; ++t) {
                acc += static_cast<double>(sg[t]);
                sG[t] = acc;
            }
        }
        __syncthreads();
        if (tid < C) {
            sEG[tid] = static_cast<float>(exp(sG[tid]));
            sEC[tid] = static_cast<float>(exp(sG[C - 1] - sG[tid]));
        }
        // Gram entries (t, s), one per quad at a time, with the decay applied on
        // the fp32 sums; entries above the diagonal are zero.
        for (int e = tid >> 2; e < C * C; e += kQuads) {
            const int t = e / C, s = e % C;
            float kk = 0.f, qk = 0.f;
            if (s <= t) {
                const float4 *kt = reinterpret_cast<const float4 *>(&sK[t * kRow]);
                const float4 *qt = reinterpret_cast<const float4 *>(&sQ[t * kRow]);
                const float4 *ks = reinterpret_cast<const float4 *>(&sK[s * kRow]);
#pragma unroll
                for (int m = 0; m < kRows / 4; ++m) {
                    const float4 a = kt[4 * m + p], b = qt[4 * m + p], c = ks[4 * m + p];
                    kk += a.x * c.x + a.y * c.y + a.z * c.z + a.w * c.w;
                    qk += b.x * c.x + b.y * c.y + b.z * c.z + b.w * c.w;
                }
            }
            kk = quad_sum(kk);
            qk = quad_sum(qk);
            if (p == 0) {
                float nn = 0.f, aa = 0.f;
                if (s <= t) {
                    const float E = expf(static_cast<float>(sG[t] - sG[s]));
                    aa = E * qk;
                    nn = s < t ? sB[t] * (E * kk) : 0.f;
                }
                sN[e] = nn;
                sA[e] = aa;
            }
        }
        __syncthreads();

        // Column j, token by token: right-hand side, forward substitution, output.
        for (int t = 0; t < C; ++t) {
            const int64_t oi = ((row0 + t) * H + h) * kHeadDim + j;
            float zf = 0.f;
            if constexpr (kGated) {
                if (p == 0 && t < nv) zf = to_f32(z[oi]);
            }
            const float ks = quad_sum(part_dot(&sK[t * kRow], S, p));
            const float qs = quad_sum(part_dot(&sQ[t * kRow], S, p));
            const float vt = sD[t * kHeadDim + j];
            float r = sB[t] * (vt - sEG[t] * ks);
            float o = sEG[t] * qs;
#pragma unroll 4
            for (int s = 0; s < t; ++s) {
                const float ds = sD[s * kHeadDim + j];
                r -= sN[t * C + s] * ds;
                o += sA[t * C + s] * ds;
            }
            o += sA[t * C + t] * r;
            // every lane of the quad stores the value it computed (the same in all
            // four), so each lane later reads only its own stores of D
            sD[t * kHeadDim + j] = r;
            if constexpr (kGated) {
                // the row's sum of o^2 over its 128 columns: one value per quad
                float ss = p == 0 ? o * o : 0.f;
#pragma unroll
                for (int off = 32; off >= 4; off >>= 1) ss += __shfl_xor(ss, off);
                if (lane == 0) sRed[t & 1][wv] = ss;
                __syncthreads();
                float tot = 0.f;
#pragma unroll
                for (int w2 = 0; w2 < kThreads / 64; ++w2) tot += sRed[t & 1][w2];
                const float ms = tot * (1.f / kHeadDim);
                if (p == 0 && t < nv) {
                    const float silu = zf / (1.f + expf(-zf));
                    O[oi] = from_f32<OutT>(nw * (o / sqrtf(ms + eps)) * silu);
                }
            } else {
                if (O && p == 0 && t < nv) O[oi] = from_f32<OutT>(o);
            }
        }

        // Carry the state to the end of the chunk.
        const float eC = sEG[C - 1];
#pragma unroll
        for (int m = 0; m < kRows; ++m) S[m] *= eC;
        for (int t = 0; t < C; ++t) {
            const float wt = sEC[t] * sD[t * kHeadDim + j];
            const float4 *kt = reinterpret_cast<const float4 *>(&sK[t * kRow]);
#pragma unroll
            for (int m = 0; m < kRows / 4; ++m) {
                const float4 a = kt[4 * m + p];
                S[4 * m] += a.x * wt;
                S[4 * m + 1] += a.y * wt;
                S[4 * m + 2] += a.z * wt;
                S[4 * m + 3] += a.w * wt;
            }
        }
        __syncthreads();   // LDS is rewritten by the next chunk
    }

    float *STu = S_T + unit * (kHeadDim * kHeadDim);
#pragma unroll
    for (int m = 0; m < kRows; ++m) STu[row_of(m) * kHeadDim + j] = S[m];
}

template <typename IO, typename OutT, int C>
hipError_t launch_typed(const PrefillArgs &a, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(a.N * a.H)), block(kThreads);
    // (the gated output is only offered with O in the io dtype)
    auto kern = a.z ? prefill_valu_kernel<IO, OutT, C, true> : prefill_valu_kernel<IO, OutT, C, false>;
    kern<<<grid, block, 0, stream>>>(
        static_cast<const IO *>(a.q), static_cast<const IO *>(a.k),
        static_cast<const IO *>(a.v), a.g, a.beta, a.S0, a.cu_seqlens, a.T, a.H,
        static_cast<OutT *>(a.O), a.S_T, static_cast<const IO *>(a.z), a.norm_w, a.eps);
    return hipGetLastError();
}

template <typename IO, typename OutT>
hipError_t launch_chunk(const PrefillArgs &a, hipStream_t stream) {
    switch (a.chunk) {
    case 16: return launch_typed<IO, OutT, 16>(a, stream);
    case 32: return launch_typed<IO, OutT, 32>(a, stream);
    default: return launch_typed<IO, OutT, 64>(a, stream);
    }
}

}  // namespace

hipError_t launch_prefill_valu(const PrefillArgs &a, hipStream_t stream) {
    if (!a.bf16) return launch_chunk<float, float>(a, stream);
    return a.out_f32 ? launch_chunk<__hip_bfloat16, float>(a, stream)
                     : launch_chunk<__hip_bfloat16, __hip_bfloat16>(a, stream);
}

}  // namespace gdn
