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
// Work split: one 128-thread workgroup per (sequence, head); thread j owns
// column j of the state (128 fp32 registers, S[i][j] for all i) and of D, so the
// forward substitution for D runs down one column per thread with no barrier.
// The chunk's K and Q (fp32, rows padded to 132 words: 16-byte rows, so that
// the per-token products, which every thread reads in the same order, take
// them four words at a time), D, N and the masked decayed QK^T live in LDS.
// The chunk's V is staged into D's rows as they are loaded (thread j stages
// and later overwrites only column j), so the per-token loop reads no global
// memory; the per-token products k_t.S and q_t.S each sum four partial chains.
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

constexpr int kThreads = 128;
constexpr int kRow = kHeadDim + 4;   // LDS row stride for K and Q (16-byte rows)

template <typename IO, typename OutT, int C, bool kGated>
__global__ __launch_bounds__(kThreads) void prefill_valu_kernel(
    const IO *__restrict__ q, const IO *__restrict__ k, const IO *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta,
    const float *__restrict__ S0, const int32_t *__restrict__ cu_seqlens, int64_t T,
    int64_t H, OutT *__restrict__ O, float *__restrict__ S_T, const IO *__restrict__ z,
    const float *__restrict__ norm_w, float eps) {
    __shared__ __attribute__((aligned(16))) float sK[C * kRow];   // rows read as float4
    __shared__ __attribute__((aligned(16))) float sQ[C * kRow];
    __shared__ float sD[C * kHeadDim];
    __shared__ float sN[C * C], sA[C * C];
    __shared__ double sG[C];
    __shared__ float sg[C], sB[C], sEG[C], sEC[C];
    __shared__ float sRed[2][kThreads / 64];

    const int64_t unit = blockIdx.x;
    const int64_t n = unit / H, h = unit % H;
    const int j = threadIdx.x;
    int64_t start, len;
    sequence_span(cu_seqlens, n, T, start, len);

    const float nw = kGated ? norm_w[j] : 0.f;
    float S[kHeadDim];
    const float *S0u = S0 ? S0 + unit * (kHeadDim * kHeadDim) : nullptr;
#pragma unroll
    for (int i = 0; i < kHeadDim; ++i) S[i] = S0u ? S0u[i * kHeadDim + j] : 0.f;

    for (int64_t c0 = 0; c0 < len; c0 += C) {
        const int nv = static_cast<int>(len - c0 < C ? len - c0 : C);
        const int64_t row0 = start + c0;   // first token row of this chunk

        for (int idx = j; idx < C * kHeadDim; idx += kThreads) {
            const int t = idx / kHeadDim, i = idx % kHeadDim;
            float kv = 0.f, qv = 0.f, vv = 0.f;
            if (t < nv) {
                const int64_t off = ((row0 + t) * H + h) * kHeadDim + i;
                kv = to_f32(k[off]);
                qv = to_f32(q[off]);
                if (v) vv = to_f32(v[off]);
            }
            sK[t * kRow + i] = kv;
            sQ[t * kRow + i] = qv;
            sD[t * kHeadDim + i] = vv;   // column i is thread i's: it reads v_t there, then writes D
        }
        if (j < C) {
            const bool ok = j < nv;
            sg[j] = ok ? g[(row0 + j) * H + h] : 0.f;
            sB[j] = ok ? beta[(row0 + j) * H + h] : 0.f;
        }
        __syncthreads();
        if (j == 0) {
            double acc = 0.0;
            for (int t = 0; t < C; ++t) {
                acc += static_cast<double>(sg[t]);
                sG[t] = acc;
            }
        }
        __syncthreads();
        if (j < C) {
            sEG[j] = static_cast<float>(exp(sG[j]));
            sEC[j] = static_cast<float>(exp(sG[C - 1] - sG[j]));
        }
        // Gram entries (t, s) for s <= t, with the decay applied on the fp32 sums.
        for (int e = j; e < C * C; e += kThreads) {
            const int t = e / C, s = e % C;
            float nn = 0.f, aa = 0.f;
            if (s <= t) {
                float kk = 0.f, qk = 0.f;
                const float *kt = &sK[t * kRow], *qt = &sQ[t * kRow], *ks = &sK[s * kRow];
#pragma unroll 16
                for (int i = 0; i < kHeadDim; ++i) {
                    kk += kt[i] * ks[i];
                    qk += qt[i] * ks[i];
                }
                const float E = expf(static_cast<float>(sG[t] - sG[s]));
                aa = E * qk;
                nn = s < t ? sB[t] * (E * kk) : 0.f;
            }
            sN[e] = nn;
            sA[e] = aa;
        }
        __syncthreads();

        // Column j: right-hand side, forward substitution, output rows.
        for (int t = 0; t < C; ++t) {
            float ka[4] = {0.f, 0.f, 0.f, 0.f}, qa[4] = {0.f, 0.f, 0.f, 0.f};
            const float4 *kt = reinterpret_cast<const float4 *>(&sK[t * kRow]);
            const float4 *qt = reinterpret_cast<const float4 *>(&sQ[t * kRow]);
#pragma unroll
            for (int i4 = 0; i4 < kHeadDim / 4; ++i4) {
                const float4 a = kt[i4], b = qt[i4];
                ka[0] += a.x * S[4 * i4];     qa[0] += b.x * S[4 * i4];
                ka[1] += a.y * S[4 * i4 + 1]; qa[1] += b.y * S[4 * i4 + 1];
                ka[2] += a.z * S[4 * i4 + 2]; qa[2] += b.z * S[4 * i4 + 2];
                ka[3] += a.w * S[4 * i4 + 3]; qa[3] += b.w * S[4 * i4 + 3];
            }
            const float ks = (ka[0] + ka[1]) + (ka[2] + ka[3]);
            const float qs = (qa[0] + qa[1]) + (qa[2] + qa[3]);
            const float vt = sD[t * kHeadDim + j];
            float r = sB[t] * (vt - sEG[t] * ks);
            for (int s = 0; s < t; ++s) r -= sN[t * C + s] * sD[s * kHeadDim + j];
            sD[t * kHeadDim + j] = r;
            float o = sEG[t] * qs;
            for (int s = 0; s <= t; ++s) o += sA[t * C + s] * sD[s * kHeadDim + j];
            const int64_t oi = ((row0 + t) * H + h) * kHeadDim + j;
            if constexpr (kGated) {
                float ss = o * o;
#pragma unroll
                for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
                if ((j & 63) == 0) sRed[t & 1][j >> 6] = ss;
                __syncthreads();
                const float ms = (sRed[t & 1][0] + sRed[t & 1][1]) * (1.f / kHeadDim);
                if (t < nv) {
                    const float zf = to_f32(z[oi]);
                    const float silu = zf / (1.f + expf(-zf));
                    O[oi] = from_f32<OutT>(nw * (o / sqrtf(ms + eps)) * silu);
                }
            } else {
                if (O && t < nv) O[oi] = from_f32<OutT>(o);
            }
        }

        // Carry the state to the end of the chunk.
        const float eC = sEG[C - 1];
#pragma unroll
        for (int i = 0; i < kHeadDim; ++i) S[i] *= eC;
        for (int t = 0; t < C; ++t) {
            const float wt = sEC[t] * sD[t * kHeadDim + j];
            const float4 *kt = reinterpret_cast<const float4 *>(&sK[t * kRow]);
#pragma unroll
            for (int i4 = 0; i4 < kHeadDim / 4; ++i4) {
                const float4 a = kt[i4];
                S[4 * i4] += a.x * wt;
                S[4 * i4 + 1] += a.y * wt;
                S[4 * i4 + 2] += a.z * wt;
                S[4 * i4 + 3] += a.w * wt;
            }
        }
        __syncthreads();   // LDS is rewritten by the next chunk
    }

    float *STu = S_T + unit * (kHeadDim * kHeadDim);
#pragma unroll
    for (int i = 0; i < kHeadDim; ++i) STu[i * kHeadDim + j] = S[i];
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
