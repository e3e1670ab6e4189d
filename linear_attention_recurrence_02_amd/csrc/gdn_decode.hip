// One-token decode step (Qwen3.5-9B-npu model page, "How it works" -> "Gated
// DeltaNet on the NPU", the 1-token matrix form): per (sequence, head)
//     d = exp(g), a = S^T k, b = S^T q      (one pass over S)
//     delta = beta (v - d a)
//     o  = d b + (q.k) delta
//     S' = d S + k delta^T                  (written back in place)
//
// The step is bound by HBM: 64 KiB of fp32 state is read and 64 KiB written per
// head against ~1.5 KiB of token I/O.  One 256-thread workgroup owns one head
// state.  Thread (wave w, lane l) owns the 4 columns 4*(l%32).. and the 16 rows
// r = rp + 8m (rp = 2w + l/32, m = 0..15), so every load instruction of a wave
// covers two adjacent 512-byte rows (1 KiB contiguous, 16 bytes per lane).  All
// 16 loads are issued before any arithmetic; the column sums a and b are
// reduced across the 8 row phases (lane pair l, l^32 by a cross-lane swap,
// then the 4 waves through LDS), after which each thread writes its 16 rows
// back with 16-byte stores.

#include "gdn_internal.hpp"

namespace gdn {
namespace {

template <typename IO>
__global__ __launch_bounds__(256) void decode_kernel(const IO *__restrict__ q,
                                                     const IO *__restrict__ k,
                                                     const IO *__restrict__ v,
                                                     const float *__restrict__ g,
                                                     const float *__restrict__ beta,
                                                     float *__restrict__ S,
                                                     IO *__restrict__ o) {
    const int64_t u = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int cg = lane & 31;
    const int rp = 2 * w + (lane >> 5);
    float *Su = S + u * (kHeadDim * kHeadDim);

    __shared__ float sq[kHeadDim], sk[kHeadDim], sv[kHeadDim];
    __shared__ float4 red_a[4][32], red_b[4][32];

    float4 s[16];
#pragma unroll
    for (int m = 0; m < 16; ++m)
        s[m] = *reinterpret_cast<const float4 *>(Su + (rp + 8 * m) * kHeadDim + 4 * cg);

    if (tid < kHeadDim) {
        sq[tid] = to_f32(q[u * kHeadDim + tid]);
        sk[tid] = to_f32(k[u * kHeadDim + tid]);
        sv[tid] = to_f32(v[u * kHeadDim + tid]);
    }
    const float d = expf(g[u]);
    const float bt = beta[u];
    __syncthreads();

    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
#pragma unroll
    for (int m = 0; m < 16; ++m) {
        const float kr = sk[rp + 8 * m], qr = sq[rp + 8 * m];
        a.x += s[m].x * kr; a.y += s[m].y * kr; a.z += s[m].z * kr; a.w += s[m].w * kr;
        b.x += s[m].x * qr; b.y += s[m].y * qr; b.z += s[m].z * qr; b.w += s[m].w * qr;
    }
    a.x += __shfl_xor(a.x, 32); a.y += __shfl_xor(a.y, 32);
    a.z += __shfl_xor(a.z, 32); a.w += __shfl_xor(a.w, 32);
    b.x += __shfl_xor(b.x, 32); b.y += __shfl_xor(b.y, 32);
    b.z += __shfl_xor(b.z, 32); b.w += __shfl_xor(b.w, 32);
    if (lane < 32) {
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
    const float4 vv = *reinterpret_cast<const float4 *>(&sv[4 * cg]);
    float4 dl;
    dl.x = bt * (vv.x - d * A.x);
    dl.y = bt * (vv.y - d * A.y);
    dl.z = bt * (vv.z - d * A.z);
    dl.w = bt * (vv.w - d * A.w);

#pragma unroll
    for (int m = 0; m < 16; ++m) {
        const float kr = sk[rp + 8 * m];
        float4 x = s[m];
        x.x = d * x.x + kr * dl.x;
        x.y = d * x.y + kr * dl.y;
        x.z = d * x.z + kr * dl.z;
        x.w = d * x.w + kr * dl.w;
        *reinterpret_cast<float4 *>(Su + (rp + 8 * m) * kHeadDim + 4 * cg) = x;
    }
    if (rp == 0) {
        IO *ou = o + u * kHeadDim + 4 * cg;
        ou[0] = from_f32<IO>(d * Bq.x + qk * dl.x);
        ou[1] = from_f32<IO>(d * Bq.y + qk * dl.y);
        ou[2] = from_f32<IO>(d * Bq.z + qk * dl.z);
        ou[3] = from_f32<IO>(d * Bq.w + qk * dl.w);
    }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(a.units)), block(256);
    if (a.bf16) {
        using T = __hip_bfloat16;
        decode_kernel<T><<<grid, block, 0, stream>>>(
            static_cast<const T *>(a.q), static_cast<const T *>(a.k),
            static_cast<const T *>(a.v), a.g, a.beta, a.S, static_cast<T *>(a.o));
    } else {
        decode_kernel<float><<<grid, block, 0, stream>>>(
            static_cast<const float *>(a.q), static_cast<const float *>(a.k),
            static_cast<const float *>(a.v), a.g, a.beta, a.S, static_cast<float *>(a.o));
    }
    return hipGetLastError();
}

}  // namespace gdn
