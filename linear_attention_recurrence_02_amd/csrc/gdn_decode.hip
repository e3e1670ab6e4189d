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
// small batch stepped over and over in the last-level cache).

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

template <typename IO, bool kStream>
__global__ __launch_bounds__(256) void decode_kernel(const IO *__restrict__ q,
                                                     const IO *__restrict__ k,
                                                     const IO *__restrict__ v,
                                                     const float *__restrict__ g,
                                                     const float *__restrict__ beta,
                                                     float *__restrict__ S,
                                                     IO *__restrict__ o) {
    const int64_t u = blockIdx.x >> 1;          // head state
    const int half = blockIdx.x & 1;            // value columns [64 half, 64 half + 64)
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int cg = lane & 15;
    const int rp = 4 * w + (lane >> 4);
    float *Su = S + u * (kHeadDim * kHeadDim) + 64 * half;

    __shared__ float sq[kHeadDim], sk[kHeadDim];
    __shared__ float4 red_a[4][16], red_b[4][16];

    float4 s[8];
#pragma unroll
    for (int m = 0; m < 8; ++m)
        s[m] = load_state<kStream>(Su + (rp + 16 * m) * kHeadDim + 4 * cg);

    if (tid < kHeadDim) {
        sq[tid] = to_f32(q[u * kHeadDim + tid]);
        sk[tid] = to_f32(k[u * kHeadDim + tid]);
    }
    const int c0 = 64 * half + 4 * cg;          // first of this thread's 4 columns
    float4 vv;
    vv.x = to_f32(v[u * kHeadDim + c0]);
    vv.y = to_f32(v[u * kHeadDim + c0 + 1]);
    vv.z = to_f32(v[u * kHeadDim + c0 + 2]);
    vv.w = to_f32(v[u * kHeadDim + c0 + 3]);
    const float d = expf(g[u]);
    const float bt = beta[u];
    __syncthreads();

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
        red_a[w][cg] = a;
        red_b[w][cg] = b;
    }
    // q.k, reduced within every wave (each wave needs it; no extra barrier)
    float qk = sq[lane] * sk[lane] + sq[lane + 64] * sk[lane + 64];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) qk += __shfl_xor(qk, off);
    __syncthreads();

    float4 A = red_a[0][cg], Bq = red_b[0][cg];
#pragma unroll
    for (int ww = 1; ww < 4; ++ww) {
        const float4 x = red_a[ww][cg], y = red_b[ww][cg];
        A.x += x.x; A.y += x.y; A.z += x.z; A.w += x.w;
        Bq.x += y.x; Bq.y += y.y; Bq.z += y.z; Bq.w += y.w;
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
    if (rp == 0) {
        IO *ou = o + u * kHeadDim + c0;
        ou[0] = from_f32<IO>(d * Bq.x + qk * dl.x);
        ou[1] = from_f32<IO>(d * Bq.y + qk * dl.y);
        ou[2] = from_f32<IO>(d * Bq.z + qk * dl.z);
        ou[3] = from_f32<IO>(d * Bq.w + qk * dl.w);
    }
}

}  // namespace

template <typename IO>
void launch_decode_io(const DecodeArgs &a, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(2 * a.units)), block(256);
    auto kern = a.stream_state ? decode_kernel<IO, true> : decode_kernel<IO, false>;
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
