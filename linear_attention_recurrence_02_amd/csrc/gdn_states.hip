// The prompt form with the state after every token kept (the rewindable verify
// form): for each (sequence, head), starting from S0, the per-token gated delta
// rule (Qwen3.5-9B-npu model page, "How it works" -> "Gated DeltaNet on the
// NPU", the 1-token matrix form applied token by token):
//     d = exp(g_t), a = S^T k_t, b = S^T q_t
//     delta = beta_t (v_t - d a)
//     o_t = d b + (q_t.k_t) delta
//     S   = d S + k_t delta^T            -> written to S_tok[t]
// A verify pass over a block of drafted tokens (the same page, section "New in
// v2", prompt lookup decoding: the state is snapshotted because it cannot be
// rewound) can then be rolled back to any accepted prefix by taking S_tok at
// its last accepted token: no snapshot and no second pass.
//
// The work is bound by the state writes (64 KiB per token and head).  As in the
// decode step, each head state is split into two 64-column halves, one
// 256-thread workgroup per half; the half stays in registers across the
// sequence (thread (wave w, lane l): columns 64 half + 4 (l%16)..+3, rows
// rp + 16m with rp = 4w + l/16), and after each token every thread writes its
// 8 x 16 bytes of the new state.  The column sums a and b are reduced across
// lanes and then across the four waves through LDS, which takes the token's
// one barrier; q and k of the next token are written to LDS before that
// barrier, into one of three buffers (the one two tokens back, which every
// thread has finished reading once it reaches this token's barrier), so the
// same barrier publishes them.

#include "gdn_internal.hpp"

namespace gdn {
namespace {

// Four consecutive values of v as one load, widened to fp32 on use.
template <typename IO> struct Vals4;
template <> struct Vals4<__hip_bfloat16> {
    uint2 r;
    __device__ float4 f() const {
        return make_float4(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u),
                           __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u));
    }
};
template <> struct Vals4<float> {
    float4 r;
    __device__ float4 f() const { return r; }
};

// One token's inputs as loaded by a thread: q and k at channel tid % 128 (put
// in LDS by the threads below 128), its 4 values of v, g and beta.
template <typename IO> struct TokenIn {
    IO q, k;
    Vals4<IO> v;
    float g, b;
};

// One workgroup per 64-column half of a head state.  kAhead loads a token's
// inputs two tokens ahead (see load_token); without it a token's inputs are
// loaded in its own iteration, after the previous token's state stores, so
// that every token waits for those stores.  The wait costs a launch with few
// workgroups (a few long sequences) about 15%, but with many workgroups per
// CU it acts as flow control on the write stream: the verify workload (8192
// workgroups) ran 0.885 ms with it and 0.932 ms without.
template <typename IO, bool kAhead>
__global__ __launch_bounds__(256) void states_kernel(const IO *__restrict__ q,
                                                     const IO *__restrict__ k,
                                                     const IO *__restrict__ v,
                                                     const float *__restrict__ g,
                                                     const float *__restrict__ beta,
                                                     const float *__restrict__ S0,
                                                     const int32_t *__restrict__ cu_seqlens,
                                                     int64_t T, int64_t H,
                                                     IO *__restrict__ O,
                                                     float *__restrict__ S_tok) {
    constexpr int D = kHeadDim;
    const int64_t unit = blockIdx.x >> 1;       // (sequence, head)
    const int half = blockIdx.x & 1;            // value columns [64 half, 64 half + 64)
    const int64_t h = unit % H;
    int64_t start, len;
    sequence_span(cu_seqlens, unit / H, T, start, len);

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int cg = lane & 15;
    const int rp = 4 * w + (lane >> 4);
    const int c0 = 64 * half + 4 * cg;          // first of this thread's 4 columns

    __shared__ float sq[3][D], sk[3][D];
    __shared__ float4 red_a[2][4][16], red_b[2][4][16];
    if (len == 0) return;                       // uniform over the workgroup

    float4 s[8];
    if (S0) {
        const float *S0u = S0 + unit * (D * D) + c0;
#pragma unroll
        for (int m = 0; m < 8; ++m) s[m] = *reinterpret_cast<const float4 *>(S0u + (rp + 16 * m) * D);
    } else {
#pragma unroll
        for (int m = 0; m < 8; ++m) s[m] = make_float4(0.f, 0.f, 0.f, 0.f);
    }

    // With kAhead a token's inputs are loaded two tokens ahead: the vector
    // memory counter retires in issue order, so a load issued after a token's
    // state stores cannot be waited for without waiting for the stores too.
    // Every thread loads (the index clamped into the sequence), so that every
    // iteration issues the same memory operations.
    auto load_token = [&](int64_t t) {
        const int64_t row = start + (t < len ? t : len - 1);
        const int64_t tok = (row * H + h) * D;
        TokenIn<IO> x;
        x.q = q[tok + (tid & (D - 1))];
        x.k = k[tok + (tid & (D - 1))];
        x.v.r = *reinterpret_cast<const decltype(x.v.r) *>(v + tok + c0);
        x.g = g[row * H + h];
        x.b = beta[row * H + h];
        return x;
    };
    TokenIn<IO> cur, nxt;
    if constexpr (kAhead) {
        cur = load_token(0);
        nxt = load_token(1);
        if (tid < D) {
            sq[0][tid] = to_f32(cur.q);
            sk[0][tid] = to_f32(cur.k);
        }
        // every load so far complete (no state store is in flight yet), so
        // that the loop's waits count only from its own iterations
        __builtin_amdgcn_s_waitcnt(0x0f70);      // vmcnt(0)
    } else if (tid < D) {
        const int64_t tok = (start * H + h) * D;
        sq[0][tid] = to_f32(q[tok + tid]);
        sk[0][tid] = to_f32(k[tok + tid]);
    }
    __syncthreads();
    for (int64_t t = 0; t < len; ++t) {
        const int buf = static_cast<int>(t % 3), rb = static_cast<int>(t & 1);
        const int64_t row = start + t;
        const int64_t tok = (row * H + h) * D;
        TokenIn<IO> nn;
        float4 vv;
        float d, bt;
        if constexpr (kAhead) {
            nn = load_token(t + 2);
            vv = cur.v.f();
            d = expf(cur.g);
            bt = cur.b;
        } else {
            vv.x = to_f32(v[tok + c0]);
            vv.y = to_f32(v[tok + c0 + 1]);
            vv.z = to_f32(v[tok + c0 + 2]);
            vv.w = to_f32(v[tok + c0 + 3]);
            d = expf(g[row * H + h]);
            bt = beta[row * H + h];
        }

        {
            float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const float kr = sk[buf][rp + 16 * m], qr = sq[buf][rp + 16 * m];
                a.x += s[m].x * kr; a.y += s[m].y * kr; a.z += s[m].z * kr; a.w += s[m].w * kr;
                b.x += s[m].x * qr; b.y += s[m].y * qr; b.z += s[m].z * qr; b.w += s[m].w * qr;
            }
#pragma unroll
            for (int off = 16; off <= 32; off <<= 1) {
                a.x += __shfl_xor(a.x, off); a.y += __shfl_xor(a.y, off);
                a.z += __shfl_xor(a.z, off); a.w += __shfl_xor(a.w, off);
                b.x += __shfl_xor(b.x, off); b.y += __shfl_xor(b.y, off);
                b.z += __shfl_xor(b.z, off); b.w += __shfl_xor(b.w, off);
            }
            if (lane < 16) {
                red_a[rb][w][cg] = a;
                red_b[rb][w][cg] = b;
            }
        }
        float qk = sq[buf][lane] * sk[buf][lane] + sq[buf][lane + 64] * sk[buf][lane + 64];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) qk += __shfl_xor(qk, off);
        // the next token's q and k, published by the same barrier
        if (t + 1 < len && tid < D) {
            const int nb = static_cast<int>((t + 1) % 3);
            if constexpr (kAhead) {
                sq[nb][tid] = to_f32(nxt.q);
                sk[nb][tid] = to_f32(nxt.k);
            } else {
                sq[nb][tid] = to_f32(q[tok + H * D + tid]);
                sk[nb][tid] = to_f32(k[tok + H * D + tid]);
            }
        }
        __syncthreads();

        {
            float4 A = red_a[rb][0][cg], Bq = red_b[rb][0][cg];
#pragma unroll
            for (int ww = 1; ww < 4; ++ww) {
                const float4 x = red_a[rb][ww][cg], y = red_b[rb][ww][cg];
                A.x += x.x; A.y += x.y; A.z += x.z; A.w += x.w;
                Bq.x += y.x; Bq.y += y.y; Bq.z += y.z; Bq.w += y.w;
            }
            float4 dl;
            dl.x = bt * (vv.x - d * A.x);
            dl.y = bt * (vv.y - d * A.y);
            dl.z = bt * (vv.z - d * A.z);
            dl.w = bt * (vv.w - d * A.w);

            float *St = S_tok + (row * H + h) * (D * D) + c0;
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const float kr = sk[buf][rp + 16 * m];
                s[m].x = d * s[m].x + kr * dl.x;
                s[m].y = d * s[m].y + kr * dl.y;
                s[m].z = d * s[m].z + kr * dl.z;
                s[m].w = d * s[m].w + kr * dl.w;
                *reinterpret_cast<float4 *>(St + (rp + 16 * m) * D) = s[m];
            }
            if (rp == 0) {
                IO *ou = O + tok + c0;
                ou[0] = from_f32<IO>(d * Bq.x + qk * dl.x);
                ou[1] = from_f32<IO>(d * Bq.y + qk * dl.y);
                ou[2] = from_f32<IO>(d * Bq.z + qk * dl.z);
                ou[3] = from_f32<IO>(d * Bq.w + qk * dl.w);
            }
        }
        if constexpr (kAhead) {
            cur = nxt;
            nxt = nn;
        }
    }
}

}  // namespace

hipError_t launch_prefill_states(const PrefillArgs &a, float *S_tok, hipStream_t stream) {
    const int64_t wgs = 2 * a.N * a.H;
    const dim3 grid(static_cast<unsigned>(wgs)), block(256);
    // loading ahead pays while the workgroups fit on the CUs at once (four per
    // CU at this kernel's register use)
    const bool ahead = wgs <= 4 * static_cast<int64_t>(compute_units());
    if (a.bf16) {
        using T = __hip_bfloat16;
        auto kern = ahead ? states_kernel<T, true> : states_kernel<T, false>;
        kern<<<grid, block, 0, stream>>>(
            static_cast<const T *>(a.q), static_cast<const T *>(a.k),
            static_cast<const T *>(a.v), a.g, a.beta, a.S0, a.cu_seqlens, a.T, a.H,
            static_cast<T *>(a.O), S_tok);
    } else {
        auto kern = ahead ? states_kernel<float, true> : states_kernel<float, false>;
        kern<<<grid, block, 0, stream>>>(
            static_cast<const float *>(a.q), static_cast<const float *>(a.k),
            static_cast<const float *>(a.v), a.g, a.beta, a.S0, a.cu_seqlens, a.T, a.H,
            static_cast<float *>(a.O), S_tok);
    }
    return hipGetLastError();
}

}  // namespace gdn
