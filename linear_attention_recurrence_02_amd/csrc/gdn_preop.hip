// The block's pre-operations, from the per-token projections to the
// recurrence's inputs (Qwen3.5-4B -- Hexagon NPU (QHexRT) -- v81 page, the
// opening description of the text decoder: a causal convolution over a short
// window carried between calls comes before the recurrent state; the QCS6490
// page's port notes name Softplus among the gate's operations), in one
// pass over the tokens.  For each of the streams q, k, v and every channel c:
//     conv_t[c] = sum_j w[c][j] x_{t-3+j}[c]  (rows before a sequence's first
//                 token come from its FIFO state), y_t = silu(conv_t),
//     q_t, k_t  = y_t / sqrt(sum_c y_t[c]^2 + eps),  v_t = y_t,
//     g_t = -softplus(a_t),  beta_t = sigmoid(b_t);
// then the FIFO holds each sequence's last three raw rows.
//
// Work split (HBM-bound streaming): one 256-thread workgroup per 256 token
// rows of one (head, stream); a thread owns 8 channels (one 16-byte row
// segment) of 16 consecutive tokens; it loads the 19 rows those need (three
// before the first) at once, so that they are in flight together, and the 32
// conv weights once.  Each input row is read about 19/16 times (the overlap
// hits cache).  The 16 threads of a token row reduce the row's sum of squares
// with lane shuffles.  When no sequence starts within a thread's window and
// all its tokens exist, the tokens run as straight-line code; otherwise window
// rows before a sequence's first token come from that sequence's FIFO state.
// The FIFO update runs as a second small kernel on the same stream, after
// every read of the old state.

#include "gdn_internal.hpp"

namespace gdn {
namespace {

constexpr int kK = 4;                 // conv taps
constexpr int kW = kK - 1;            // FIFO rows
constexpr int kTok = 16;              // tokens per thread
constexpr int kRowsPerBlock = 256;    // 16 token groups x 16 tokens

struct Vec8 {
    float v[8];
};

// A 16-byte row segment as loaded (8 bf16 or, for fp32, two of these).
template <typename IO> struct Raw;
template <> struct Raw<__hip_bfloat16> { uint4 u; };
template <> struct Raw<float> { float4 a, b; };
template <typename IO> __device__ __forceinline__ Raw<IO> load_raw(const IO *p);
template <> __device__ __forceinline__ Raw<__hip_bfloat16> load_raw(const __hip_bfloat16 *p) {
    return Raw<__hip_bfloat16>{*reinterpret_cast<const uint4 *>(p)};
}
template <> __device__ __forceinline__ Raw<float> load_raw(const float *p) {
    return Raw<float>{*reinterpret_cast<const float4 *>(p), *reinterpret_cast<const float4 *>(p + 4)};
}
__device__ __forceinline__ Vec8 widen(const Raw<__hip_bfloat16> &r) {
    const uint32_t w[4] = {r.u.x, r.u.y, r.u.z, r.u.w};
    Vec8 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o.v[2 * i] = __uint_as_float(w[i] << 16);
        o.v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
    return o;
}
__device__ __forceinline__ Vec8 widen(const Raw<float> &r) {
    return Vec8{{r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w}};
}

// Sum over the 16 lanes of a DPP row (lanes 16r .. 16r+15), left in every
// lane: swap neighbours, swap pairs (quad permutes), then mirror within each
// half row and within the row.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_f<0xb1>(x);     // quad_perm [1,0,3,2]
    x += dpp_f<0x4e>(x);     // quad_perm [2,3,0,1]
    x += dpp_f<0x141>(x);    // row_half_mirror
    x += dpp_f<0x140>(x);    // row_mirror
    return x;
}

template <typename IO> __device__ __forceinline__ Vec8 load8(const IO *p);
template <> __device__ __forceinline__ Vec8 load8<float>(const float *p) {
    const float4 a = *reinterpret_cast<const float4 *>(p), b = *reinterpret_cast<const float4 *>(p + 4);
    return Vec8{{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w}};
}
template <> __device__ __forceinline__ Vec8 load8<__hip_bfloat16>(const __hip_bfloat16 *p) {
    const uint4 u = *reinterpret_cast<const uint4 *>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    Vec8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r.v[2 * i] = __uint_as_float(w[i] << 16);
        r.v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
    return r;
}
template <typename IO> __device__ __forceinline__ void store8(IO *p, const float *v);
template <> __device__ __forceinline__ void store8<float>(float *p, const float *v) {
    *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4 *>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}
// two values per conversion (round to nearest even, as __float2bfloat16)
template <> __device__ __forceinline__ void store8<__hip_bfloat16>(__hip_bfloat16 *p, const float *v) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        w[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{v[2 * i], v[2 * i + 1]}, bf16x2));
    *reinterpret_cast<uint4 *>(p) = make_uint4(w[0], w[1], w[2], w[3]);
}

// Sequence of packed row t: the last n with cu[n] <= t (so empty sequences are
// skipped).  Offsets are clamped into [0, T] like everywhere else.
__device__ __forceinline__ int64_t seq_of(const int32_t *cu, int64_t N, int64_t T, int64_t t,
                                          int64_t &start, int64_t &end) {
    if (!cu) {
        const int64_t n = t / T;
        start = n * T;
        end = start + T;
        return n;
    }
    int64_t lo = 0, hi = N;                  // invariant: clamp(cu[lo]) <= t < clamp(cu[hi])
    auto at = [&](int64_t i) {
        int64_t c = cu[i];
        return c < 0 ? int64_t(0) : (c > T ? T : c);
    };
    while (hi - lo > 1) {
        const int64_t mid = (lo + hi) >> 1;
        if (at(mid) <= t) lo = mid; else hi = mid;
    }
    start = at(lo);
    end = at(lo + 1);
    return lo;
}

template <typename IO>
__global__ __launch_bounds__(256) void preop_kernel(
    const IO *__restrict__ xq, const IO *__restrict__ xk, const IO *__restrict__ xv,
    const float *__restrict__ a, const float *__restrict__ b, const float *__restrict__ conv_w,
    const IO *__restrict__ state, const int32_t *__restrict__ cu, int64_t N, int64_t T,
    int64_t rows, int64_t H, float eps, IO *__restrict__ q, IO *__restrict__ k,
    IO *__restrict__ v, float *__restrict__ g, float *__restrict__ beta) {
    constexpr int D = kHeadDim;
    const int s = blockIdx.z;                         // stream: 0 q, 1 k, 2 v
    const int64_t h = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int cg = lane & 15;                         // channels 8cg .. 8cg+7
    const int tg = 4 * wave + (lane >> 4);            // token group 0..15
    const int64_t t0 = static_cast<int64_t>(blockIdx.y) * kRowsPerBlock + kTok * tg;
    if (t0 >= rows) return;                           // uniform over the 16 lanes of the group

    const IO *x = s == 0 ? xq : (s == 1 ? xk : xv);
    IO *y = s == 0 ? q : (s == 1 ? k : v);
    const int64_t HD = H * D;
    const int c0 = 8 * cg;

    float w[8][kK];
    {
        const float *wp = conv_w + ((s * H + h) * D + c0) * kK;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float4 t = *reinterpret_cast<const float4 *>(wp + kK * i);
            w[i][0] = t.x; w[i][1] = t.y; w[i][2] = t.z; w[i][3] = t.w;
        }
    }
    // state rows of sequence n: ((n * 3 + s) * H + h) * kW * D
    auto state_row = [&](int64_t n, int j) {
        return load8<IO>(state + (((n * 3 + s) * H + h) * kW + j) * D + c0);
    };

    // All rows the thread needs, t0-3 .. t0+7, are loaded up front so that
    // they are in flight together; rows outside [0, rows) are never used.
    // x and y are addressed from the thread's first row with 32-bit offsets
    // (rows of one call stay below 2^40 elements, but a thread spans 11 rows)
    const IO *xb = x + t0 * HD + h * D + c0;
    IO *yb = y + t0 * HD + h * D + c0;
    const uint32_t hd = static_cast<uint32_t>(HD);
    Raw<IO> xr[kW + kTok];
#pragma unroll
    for (int j = 0; j < kW + kTok; ++j) {
        const int64_t r = t0 - kW + j;
        const IO *p = r < 0 ? x + h * D + c0 : (r >= rows ? xb + (rows - 1 - t0) * HD : xb + (j - kW) * static_cast<int64_t>(hd));
        xr[j] = load_raw<IO>(p);
    }
    // g and beta, one token per lane: lane L < 4 kTok of wave w takes the
    // wave's token 4 kTok w + L of the block (in stream q's workgroups only);
    // a lane whose group returned above has its token at or past the end
    if (s == 0 && lane < 4 * kTok) {
        const int64_t t = static_cast<int64_t>(blockIdx.y) * kRowsPerBlock + 4 * kTok * wave + lane;
        if (t < rows) {
            const int64_t gi = t * H + h;
            const float av = a[gi], bv = b[gi];
            // softplus(av) = max(av, 0) + log1p(exp(-|av|)), without overflow
            g[gi] = -(fmaxf(av, 0.f) + log1pf(__expf(-fabsf(av))));
            beta[gi] = 1.f / (1.f + __expf(-bv));
        }
    }

    // token t0 + i from the conv window r0, r1, r2 (rows t-3 .. t-1) and row xt
    auto emit = [&](int i, const Vec8 &r0, const Vec8 &r1, const Vec8 &r2, const Vec8 &xt) {
        float out[8];
        float ss = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const float u = w[c][0] * r0.v[c] + w[c][1] * r1.v[c] + w[c][2] * r2.v[c] + w[c][3] * xt.v[c];
            const float yv = u * __builtin_amdgcn_rcpf(1.f + __expf(-u));
            out[c] = yv;
            ss += yv * yv;
        }
        if (s < 2) {
            const float inv = rsqrtf(row16_sum(ss) + eps);
#pragma unroll
            for (int c = 0; c < 8; ++c) out[c] *= inv;
        }
        store8<IO>(yb + static_cast<uint32_t>(i) * hd, out);
    };

    int64_t start, end;
    int64_t n = seq_of(cu, N, T, t0, start, end);
    if (start <= t0 - kW && t0 + kTok <= end && t0 + kTok <= rows) {
        // the common case, uniform over the 16 lanes of the group: all 8 tokens
        // and their window in one sequence, straight-line code
        Vec8 wd[kW + kTok];
#pragma unroll
        for (int j = 0; j < kW + kTok; ++j) wd[j] = widen(xr[j]);
#pragma unroll
        for (int i = 0; i < kTok; ++i) emit(i, wd[i], wd[i + 1], wd[i + 2], wd[i + 3]);
        return;
    }
    // a sequence starts within the window, or the rows end: the window rows
    // t0-3 .. t0-1, widened once; those before the sequence's start come from
    // its FIFO state
    Vec8 win[kW];
#pragma unroll
    for (int j = 0; j < kW; ++j) {
        const int64_t r = t0 - kW + j;
        win[j] = r >= start ? widen(xr[j]) : state_row(n, kW + static_cast<int>(r - start));
    }
#pragma unroll
    for (int i = 0; i < kTok; ++i) {
        const int64_t t = t0 + i;
        if (t < rows) {                               // uniform over the group
            if (t >= end) {                           // a new sequence starts at t
                n = seq_of(cu, N, T, t, start, end);
#pragma unroll
                for (int j = 0; j < kW; ++j) win[j] = state_row(n, j);
            }
            const Vec8 xt = widen(xr[i + kW]);
            emit(i, win[0], win[1], win[2], xt);
            win[0] = win[1];
            win[1] = win[2];
            win[2] = xt;
        }
    }
}

// FIFO after the call: the last three raw rows of [state_in; rows of the
// sequence].  One thread per channel of a (sequence, stream, head); it reads
// everything it needs before writing, so state_out may be state_in.
template <typename IO>
__global__ __launch_bounds__(128) void preop_state_kernel(
    const IO *__restrict__ xq, const IO *__restrict__ xk, const IO *__restrict__ xv,
    const IO *state_in, const int32_t *__restrict__ cu, int64_t T, int64_t H, IO *state_out) {
    constexpr int D = kHeadDim;
    const int64_t n = blockIdx.x;
    const int s = blockIdx.y;
    const int64_t h = blockIdx.z;
    const int c = threadIdx.x;
    int64_t start, len;
    sequence_span(cu, n, T, start, len);
    const IO *x = s == 0 ? xq : (s == 1 ? xk : xv);
    const int64_t base = ((n * 3 + s) * H + h) * kW * D + c;
    IO r[kW];
#pragma unroll
    for (int j = 0; j < kW; ++j) {
        const int64_t row = len - kW + j;            // row within the sequence
        r[j] = row >= 0 ? x[((start + row) * H + h) * D + c] : state_in[base + (kW + row) * D];
    }
#pragma unroll
    for (int j = 0; j < kW; ++j) state_out[base + j * D] = r[j];
}

template <typename IO>
hipError_t launch_state(const PreopArgs &p, hipStream_t stream) {
    const dim3 sgrid(static_cast<unsigned>(p.N), 3, static_cast<unsigned>(p.H));
    preop_state_kernel<IO><<<sgrid, kHeadDim, 0, stream>>>(
        static_cast<const IO *>(p.xq), static_cast<const IO *>(p.xk), static_cast<const IO *>(p.xv),
        static_cast<const IO *>(p.state_in), p.cu_seqlens, p.T, p.H, static_cast<IO *>(p.state_out));
    return hipGetLastError();
}

template <typename IO>
hipError_t launch_typed(const PreopArgs &p, hipStream_t stream) {
    const int64_t rows = p.rows;
    if (rows > 0) {
        // heads vary fastest, so that the workgroups in flight together cover
        // whole token rows (all heads) and use every DRAM page they open
        const dim3 grid(static_cast<unsigned>(p.H),
                        static_cast<unsigned>((rows + kRowsPerBlock - 1) / kRowsPerBlock), 3);
        preop_kernel<IO><<<grid, 256, 0, stream>>>(
            static_cast<const IO *>(p.xq), static_cast<const IO *>(p.xk),
            static_cast<const IO *>(p.xv), p.a, p.b, p.conv_w, static_cast<const IO *>(p.state_in),
            p.cu_seqlens, p.N, p.T, rows, p.H, p.eps, static_cast<IO *>(p.q),
            static_cast<IO *>(p.k), static_cast<IO *>(p.v), p.g, p.beta);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return launch_state<IO>(p, stream);
}

}  // namespace

hipError_t launch_preop(const PreopArgs &p, hipStream_t stream) {
    return p.bf16 ? launch_typed<__hip_bfloat16>(p, stream) : launch_typed<float>(p, stream);
}

hipError_t launch_preop_state(const PreopArgs &p, hipStream_t stream) {
    return p.bf16 ? launch_state<__hip_bfloat16>(p, stream) : launch_state<float>(p, stream);
}

}  // namespace gdn
