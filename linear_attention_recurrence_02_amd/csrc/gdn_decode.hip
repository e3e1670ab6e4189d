// One-token decode step (Qwen3.5-9B-npu model page, "How it works" -> "Gated
// DeltaNet on the NPU", the 1-token matrix form): per (sequence, head)
//     d = exp(g), a = S^T k, b = S^T q      (one pass over S)
//     delta = beta (v - d a)
//     o  = d b + (q.k) delta
//     S' = d S + k delta^T                  (written back in place)
//
// The step is bound by HBM: 64 KiB of fp32 state is read and 64 KiB written per
// head against ~1 KiB of token I/O.  The value columns of S are independent,
// so each head state is split into two 64-column halves, one 256-thread
// workgroup per half (2 x B x H workgroups fill the 256 CUs several times
// over).  Thread (wave w, lane l) owns the 4 columns 4*(l%16).. of its half and
// the 8 rows r = rp + 16m (rp = 4w + l/16, m = 0..7), so each load instruction
// of a wave covers four 256-byte row segments with 16 bytes per lane.  All 8
// loads are issued before any arithmetic; the column sums a and b are reduced
// over the 16 row phases (lanes l, l^16, l^32 by cross-lane swaps, then the 4
// waves through LDS), after which each thread writes its rows back with
// 16-byte stores.  kStream marks the state loads and stores non-temporal,
// which streams state that is not in cache faster (the plain form keeps a
// small batch stepped over and over in the last-level cache); that form runs
// one workgroup per head state, each thread doing the same rows and columns in
// both halves (16 loads in flight), with each half's arithmetic unchanged, so
// the two forms give bit-identical results.

#include "gdn_internal.hpp"

namespace gdn {
namespace {

typedef float f32x4v __attribute__((ext_vector_type(4)));

template <bool kStream>
__device__ __forceinline__ float4 load_state(const float *p) {
    if constexpr (kStream) {
        const f32x4v t = __builtin_nontemporal_load(reinterpret_cast<const f32x4v *>(p));
        return make_float4(t.x, t.y, t.z, t.w);
    } else {
        return *reinterpret_cast<const float4 *>(p);
    }
}
template <bool kStream>
__device__ __forceinline__ void store_state(float *p, float4 x) {
    if constexpr (kStream) {
        const f32x4v t = {x.x, x.y, x.z, x.w};
        __builtin_nontemporal_store(t, reinterpret_cast<f32x4v *>(p));
    } else {
        *reinterpret_cast<float4 *>(p) = x;
    }
}

// kHalves = 1: one workgroup per half; kHalves = 2: one workgroup per head
// state, each thread doing its rows and columns in both halves, with the
// arithmetic of each half, and its order, exactly as for kHalves = 1.
template <typename IO, bool kStream, int kHalves>
__global__ __launch_bounds__(256) void decode_kernel(const IO *__restrict__ q,
                                                     const IO *__restrict__ k,
                                                     const IO *__restrict__ v,
                                                     const float *__restrict__ g,
                                                     const float *__restrict__ beta,
                                                     float *__restrict__ S,
                                                     IO *__restrict__ o) {
    const int64_t u = blockIdx.x / (2 / kHalves);                    // head state
    const int half0 = kHalves == 2 ? 0 : static_cast<int>(blockIdx.x & 1);
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int cg = lane & 15;
    const int rp = 4 * w + (lane >> 4);
    float *Su = S + u * (kHeadDim * kHeadDim) + 64 * half0;

    __shared__ float sq[kHeadDim], sk[kHeadDim];
    __shared__ float4 red_a[kHalves][4][16], red_b[kHalves][4][16];

    float4 s[kHalves][8];
#pragma unroll
    for (int hh = 0; hh < kHalves; ++hh) {
#pragma unroll
        for (int m = 0; m < 8; ++m)
            s[hh][m] = load_state<kStream>(Su + (rp + 16 * m) * kHeadDim + 64 * hh + 4 * cg);
        // one half's loads go out before the next half's addresses are made
        // (with both halves in one batch the compiler computed all sixteen
        // addresses first; the streaming form measured 24.0-24.5 against
        // 23.2-23.7 us per step on state streamed from HBM, same result)
        __builtin_amdgcn_sched_barrier(0);
    }

    if (tid < kHeadDim) {
        sq[tid] = to_f32(q[u * kHeadDim + tid]);
        sk[tid] = to_f32(k[u * kHeadDim + tid]);
    }
    float4 vv[kHalves];
#pragma unroll
    for (int hh = 0; hh < kHalves; ++hh) {
        const int c0 = 64 * (half0 + hh) + 4 * cg;   // first of this thread's 4 columns
        vv[hh].x = to_f32(v[u * kHeadDim + c0]);
        vv[hh].y = to_f32(v[u * kHeadDim + c0 + 1]);
        vv[hh].z = to_f32(v[u * kHeadDim + c0 + 2]);
        vv[hh].w = to_f32(v[u * kHeadDim + c0 + 3]);
    }
    const float d = expf(g[u]);
    const float bt = beta[u];
    __syncthreads();

#pragma unroll
    for (int hh = 0; hh < kHalves; ++hh) {
        float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const float kr = sk[rp + 16 * m], qr = sq[rp + 16 * m];
            a.x += s[hh][m].x * kr; a.y += s[hh][m].y * kr; a.z += s[hh][m].z * kr; a.w += s[hh][m].w * kr;
            b.x += s[hh][m].x * qr; b.y += s[hh][m].y * qr; b.z += s[hh][m].z * qr; b.w += s[hh][m].w * qr;
        }
#pragma unroll
        for (int off = 16; off <= 32; off <<= 1) {
            a.x += __shfl_xor(a.x, off); a.y += __shfl_xor(a.y, off);
            a.z += __shfl_xor(a.z, off); a.w += __shfl_xor(a.w, off);
            b.x += __shfl_xor(b.x, off); b.y += __shfl_xor(b.y, off);
            b.z += __shfl_xor(b.z, off); b.w += __shfl_xor(b.w, off);
        }
        if (lane < 16) {
            red_a[hh][w][cg] = a;
            red_b[hh][w][cg] = b;
        }
    }
    // q.k, reduced within every wave (each wave needs it; no extra barrier)
    float qk = sq[lane] * sk[lane] + sq[lane + 64] * sk[lane + 64];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) qk += __shfl_xor(qk, off);
    __syncthreads();

#pragma unroll
    for (int hh = 0; hh < kHalves; ++hh) {
        float4 A = red_a[hh][0][cg], Bq = red_b[hh][0][cg];
#pragma unroll
        for (int ww = 1; ww < 4; ++ww) {
            const float4 x = red_a[hh][ww][cg], y = red_b[hh][ww][cg];
            A.x += x.x; A.y += x.y; A.z += x.z; A.w += x.w;
            Bq.x += y.x; Bq.y += y.y; Bq.z += y.z; Bq.w += y.w;
        }
        float4 dl;
        dl.x = bt * (vv[hh].x - d * A.x);
        dl.y = bt * (vv[hh].y - d * A.y);
        dl.z = bt * (vv[hh].z - d * A.z);
        dl.w = bt * (vv[hh].w - d * A.w);

#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const float kr = sk[rp + 16 * m];
            float4 x = s[hh][m];
            x.x = d * x.x + kr * dl.x;
            x.y = d * x.y + kr * dl.y;
            x.z = d * x.z + kr * dl.z;
            x.w = d * x.w + kr * dl.w;
            store_state<kStream>(Su + (rp + 16 * m) * kHeadDim + 64 * hh + 4 * cg, x);
        }
        if (rp == 0) {
            IO *ou = o + u * kHeadDim + 64 * (half0 + hh) + 4 * cg;
            ou[0] = from_f32<IO>(d * Bq.x + qk * dl.x);
            ou[1] = from_f32<IO>(d * Bq.y + qk * dl.y);
            ou[2] = from_f32<IO>(d * Bq.z + qk * dl.z);
            ou[3] = from_f32<IO>(d * Bq.w + qk * dl.w);
        }
    }
}

// The decode step with the block's pre-operations in front, for one token per
// sequence: from the raw projections xq, xk, xv and the gate inputs a, b, with
// each sequence's causal-conv FIFO read and advanced, to o and the new state.
// The pre-operations are those of gdn_preop (conv over the FIFO rows and the
// token, silu, L2 norm of q and k, g = -softplus(a), beta = sigmoid(b)); q, k
// and v stay fp32 on chip.  One 512-thread workgroup per head state: its two
// halves do the two 64-column halves exactly as decode_kernel does, after the
// workgroup has made q, k, v, g and beta in LDS.  The workgroup owns its head's
// FIFO rows, so they can be advanced in place.  The state loads are issued
// first, so that their latency covers the pre-operations.  kGated applies the
// block's gated RMS norm to the output row, y = w o / sqrt(mean(o^2) + eps)
// silu(z), on the fp32 o, the whole row being in this workgroup.
template <typename IO, bool kStream, bool kGated>
__global__ __launch_bounds__(512) void decode_preop_kernel(
    const IO *__restrict__ xq, const IO *__restrict__ xk, const IO *__restrict__ xv,
    const float *__restrict__ ga, const float *__restrict__ gb, const float *__restrict__ conv_w,
    const IO *state_in, IO *state_out, float eps, const IO *__restrict__ z,
    const float *__restrict__ norm_w, float norm_eps, float *__restrict__ S, int64_t H,
    IO *__restrict__ o) {
    const int64_t u = blockIdx.x;               // head state n * H + h
    const int64_t n = u / H, h = u % H;
    const int tid = threadIdx.x;
    const int half = tid >> 8, t = tid & 255;   // value columns [64 half, 64 half + 64)
    const int lane = t & 63, w = t >> 6;
    const int cg = lane & 15;
    const int rp = 4 * w + (lane >> 4);
    float *Su = S + u * (kHeadDim * kHeadDim) + 64 * half;

    __shared__ float sq[kHeadDim], sk[kHeadDim], sv[kHeadDim];
    __shared__ float nrm[2][2];                 // (q, k) x two waves: partial sums of y^2
    __shared__ float sgate[2];                  // g, beta
    __shared__ float4 red_a[2][4][16], red_b[2][4][16];

    float4 s[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) s[m] = load_state<kStream>(Su + (rp + 16 * m) * kHeadDim + 4 * cg);

    // pre-operations: thread tid < 384 makes channel c of stream st (q, k, v)
    float y = 0.f;
    const int st = tid >> 7, c = tid & (kHeadDim - 1);
    if (tid < 3 * kHeadDim) {
        const IO *x = st == 0 ? xq : (st == 1 ? xk : xv);
        const int64_t fi = ((n * 3 + st) * H + h) * 3 * kHeadDim + c;   // FIFO row j at fi + j D
        const IO r0 = state_in[fi], r1 = state_in[fi + kHeadDim], r2 = state_in[fi + 2 * kHeadDim];
        const IO xr = x[u * kHeadDim + c];
        const float4 wc = *reinterpret_cast<const float4 *>(conv_w + ((st * H + h) * kHeadDim + c) * 4);
        const float cv = wc.x * to_f32(r0) + wc.y * to_f32(r1) + wc.z * to_f32(r2) + wc.w * to_f32(xr);
        y = cv * __builtin_amdgcn_rcpf(1.f + __expf(-cv));
        // the FIFO's rows move up by one (all three were read above, by this thread)
        state_out[fi] = r1;
        state_out[fi + kHeadDim] = r2;
        state_out[fi + 2 * kHeadDim] = xr;
        if (st < 2) {
            float ss = y * y;
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
            if (lane == 0) nrm[st][(tid >> 6) & 1] = ss;
        }
    } else if (tid == 3 * kHeadDim) {
        const float av = ga[u], bv = gb[u];
        // softplus(av) = max(av, 0) + log1p(exp(-|av|)), without overflow
        sgate[0] = -(fmaxf(av, 0.f) + log1pf(__expf(-fabsf(av))));
        sgate[1] = 1.f / (1.f + __expf(-bv));
    }
    __syncthreads();
    if (tid < 3 * kHeadDim) {
        if (st < 2) y *= rsqrtf(nrm[st][0] + nrm[st][1] + eps);
        (st == 0 ? sq : (st == 1 ? sk : sv))[c] = y;
    }
    __syncthreads();

    // the step itself, as decode_kernel, per half
    const int c0 = 64 * half + 4 * cg;
    const float4 vv = make_float4(sv[c0], sv[c0 + 1], sv[c0 + 2], sv[c0 + 3]);
    const float d = expf(sgate[0]);
    const float bt = sgate[1];
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const float kr = sk[rp + 16 * m], qr = sq[rp + 16 * m];
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
        red_a[half][w][cg] = a;
        red_b[half][w][cg] = b;
    }
    float qk = sq[lane] * sk[lane] + sq[lane + 64] * sk[lane + 64];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) qk += __shfl_xor(qk, off);
    __syncthreads();

    float4 A = red_a[half][0][cg], Bq = red_b[half][0][cg];
#pragma unroll
    for (int ww = 1; ww < 4; ++ww) {
        const float4 x = red_a[half][ww][cg], yq = red_b[half][ww][cg];
        A.x += x.x; A.y += x.y; A.z += x.z; A.w += x.w;
        Bq.x += yq.x; Bq.y += yq.y; Bq.z += yq.z; Bq.w += yq.w;
    }
    float4 dl;
    dl.x = bt * (vv.x - d * A.x);
    dl.y = bt * (vv.y - d * A.y);
    dl.z = bt * (vv.z - d * A.z);
    dl.w = bt * (vv.w - d * A.w);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const float kr = sk[rp + 16 * m];
        float4 x = s[m];
        x.x = d * x.x + kr * dl.x;
        x.y = d * x.y + kr * dl.y;
        x.z = d * x.z + kr * dl.z;
        x.w = d * x.w + kr * dl.w;
        store_state<kStream>(Su + (rp + 16 * m) * kHeadDim + 4 * cg, x);
    }
    // lanes 0..15 of each half's first wave (rp = 0) own the output columns c0..c0+3
    float ov[4] = {d * Bq.x + qk * dl.x, d * Bq.y + qk * dl.y, d * Bq.z + qk * dl.z,
                   d * Bq.w + qk * dl.w};
    if constexpr (kGated) {
        __shared__ float osq[2];
        if (w == 0) {
            float ss = ov[0] * ov[0] + ov[1] * ov[1] + ov[2] * ov[2] + ov[3] * ov[3];
#pragma unroll
            for (int off = 8; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);   // lanes 0..15
            if (lane == 0) osq[half] = ss;
        }
        __syncthreads();
        if (rp == 0) {
            const float rs = __builtin_amdgcn_rsqf((osq[0] + osq[1]) * (1.f / kHeadDim) + norm_eps);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float zf = to_f32(z[u * kHeadDim + c0 + e]);
                const float sg = __builtin_amdgcn_rcpf(1.f + __expf(-zf));
                ov[e] = norm_w[c0 + e] * (ov[e] * rs) * (zf * sg);
            }
        }
    }
    if (rp == 0) {
        IO *ou = o + u * kHeadDim + c0;
#pragma unroll
        for (int e = 0; e < 4; ++e) ou[e] = from_f32<IO>(ov[e]);
    }
}

}  // namespace

template <typename IO>
void launch_decode_preop_io(const DecodePreopArgs &a, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(a.units)), block(512);
    auto kern = a.z ? (a.stream_state ? decode_preop_kernel<IO, true, true>
                                      : decode_preop_kernel<IO, false, true>)
                    : (a.stream_state ? decode_preop_kernel<IO, true, false>
                                      : decode_preop_kernel<IO, false, false>);
    kern<<<grid, block, 0, stream>>>(
        static_cast<const IO *>(a.xq), static_cast<const IO *>(a.xk), static_cast<const IO *>(a.xv),
        a.a, a.b, a.conv_w, static_cast<const IO *>(a.state_in), static_cast<IO *>(a.state_out),
        a.eps, static_cast<const IO *>(a.z), a.norm_w, a.norm_eps, a.S, a.H,
        static_cast<IO *>(a.o));
}

hipError_t launch_decode_preop(const DecodePreopArgs &a, hipStream_t stream) {
    if (a.bf16)
        launch_decode_preop_io<__hip_bfloat16>(a, stream);
    else
        launch_decode_preop_io<float>(a, stream);
    return hipGetLastError();
}

template <typename IO>
void launch_decode_io(const DecodeArgs &a, hipStream_t stream) {
    // Non-temporal state streams faster with one workgroup per head state (16
    // loads in flight per thread); cached state with one per half.
    const int halves = a.stream_state ? 2 : 1;
    const dim3 grid(static_cast<unsigned>((2 / halves) * a.units)), block(256);
    auto kern = a.stream_state ? decode_kernel<IO, true, 2> : decode_kernel<IO, false, 1>;
    kern<<<grid, block, 0, stream>>>(static_cast<const IO *>(a.q), static_cast<const IO *>(a.k),
                                     static_cast<const IO *>(a.v), a.g, a.beta, a.S,
                                     static_cast<IO *>(a.o));
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) {
    if (a.bf16)
        launch_decode_io<__hip_bfloat16>(a, stream);
    else
        launch_decode_io<float>(a, stream);
    return hipGetLastError();
}

}  // namespace gdn
