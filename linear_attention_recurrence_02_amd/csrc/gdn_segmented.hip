// Helpers of the segmented prompt form (context parallelism on one GPU).
//
// Each sequence is cut into segments of L tokens (at least one, so an empty
// sequence has one empty segment).  Over a segment the
// recurrence is affine in the state that enters it: S_out = M S_in + B, with
// M (dk x dk) the segment's state map (the prompt form run with V = 0 from
// S = I) and B (dk x dv) the state the segment reaches from zero.  Both come
// from the ordinary prompt kernel run over all segments at once as one packed
// batch.  A scan over the segments of each sequence,
//     S_in(0) = S0,   S_in(p+1) = M_p S_in(p) + B_p,
// gives every segment its entering state, and a third run of the prompt
// kernel from those states produces O and the segment end states.  Each run
// keeps the whole GPU busy even when a batch holds only a few long sequences.
//
// This file holds the small kernels around those runs: the plan (each
// sequence's first segment and the segments' offsets, for a uniform or a
// packed batch), the identity states the map run starts from (it runs with no
// values: a null v), the scan, and the gather of each sequence's final state.

#include "gdn_internal.hpp"

namespace gdn {
namespace {

constexpr int D = kHeadDim;
constexpr int kCols = 8;        // state columns per scan workgroup
constexpr int64_t kState = int64_t(D) * D;

// One launch prepares the three runs.  Workgroup 0 makes the plan: sequence n
// (rows [start, start + len), from cu_seqlens clamped as the prompt kernels
// clamp it, or n T .. for a uniform batch) gets P_n = max(1, ceil(len / L))
// segments, numbered from seg[n] = P_0 + .. + P_{n-1}; segment seg[n] + j
// starts at row start + j L.  The numbering is capped at Ns, the workspace's
// segment count (reached only by offsets that overlap, which give wrong
// results but stay in bounds); the segments past the last sequence start, and
// end, at the last row.  The other workgroups write one identity state per
// segment unit.
constexpr int kPrepThreads = 256;
__global__ __launch_bounds__(kPrepThreads) void segment_prep_kernel(
    const int32_t *__restrict__ cu_in, int64_t N, int64_t T, int64_t L, int64_t Ns,
    int32_t *__restrict__ seg, int32_t *__restrict__ cu_out, float *__restrict__ sid,
    int64_t units) {
    const int tid = threadIdx.x;
    if (blockIdx.x == 0) {
        __shared__ int64_t sc[kPrepThreads];
        const int64_t rows = cu_in ? T : N * T;
        int64_t running = 0;
        for (int64_t base = 0; base < N; base += kPrepThreads) {
            const int64_t n = base + tid;
            int64_t start = 0, len = 0, p = 0;
            if (n < N) {
                sequence_span(cu_in, n, T, start, len);
                p = len > 0 ? (len + L - 1) / L : 1;
            }
            sc[tid] = p;
            __syncthreads();
            for (int off = 1; off < kPrepThreads; off <<= 1) {   // inclusive scan
                const int64_t x = tid >= off ? sc[tid - off] : 0;
                __syncthreads();
                sc[tid] += x;
                __syncthreads();
            }
            const int64_t incl = running + sc[tid], total = sc[kPrepThreads - 1];
            if (n < N) {
                const int64_t s0 = incl - p < Ns ? incl - p : Ns, s1 = incl < Ns ? incl : Ns;
                seg[n] = static_cast<int32_t>(s0);
                for (int64_t s = s0; s < s1; ++s)
                    cu_out[s] = static_cast<int32_t>(start + (s - s0) * L);
            }
            running += total;
            __syncthreads();                                      // sc is reused
        }
        const int64_t used = running < Ns ? running : Ns;
        if (tid == 0) seg[N] = static_cast<int32_t>(used);
        for (int64_t s = used + tid; s <= Ns; s += kPrepThreads) cu_out[s] = static_cast<int32_t>(rows);
        return;
    }
    const int64_t stride = static_cast<int64_t>(gridDim.x - 1) * kPrepThreads;
    const int64_t i0 = static_cast<int64_t>(blockIdx.x - 1) * kPrepThreads + tid;
    static_assert(kState / 4 == 4096 && D == 128, "index bits below");
    for (int64_t i = i0; i < units * (kState / 4); i += stride) {
        const int e = 4 * static_cast<int>(i & 4095);          // first of 4 elements
        const int row = e >> 7, col = e & 127;                  // col .. col+3 in one row
        const int d = row - col;                                // the diagonal's slot, if any
        const float4 x = make_float4(d == 0 ? 1.f : 0.f, d == 1 ? 1.f : 0.f, d == 2 ? 1.f : 0.f,
                                     d == 3 ? 1.f : 0.f);
        reinterpret_cast<float4 *>(sid)[i] = x;
    }
}

// The scan, S_in(p+1) = M_p S_in(p) + B_p, for one (sequence, head) and
// kCols state columns, by 512 threads.  Lane 16 a + s of wave w owns rows
// 4 g .. 4 g + 3 (row group g = 4 w + a) and the products over
// l in [8 s, 8 s + 8): its slice of M stays in registers, and the 8 rows of
// S it needs come from LDS, each read serving 4 rows x kCols products.  The
// 16 l-splits of a row group are then summed by a reduce-scatter across the
// 16 lanes, which leaves every lane two adjacent columns of one row.  Each
// workgroup reads all of M_p (64 KB) per step: the next segment's slice is
// loaded while the current one is used.
//
// LDS holds S twice (ping-pong): state row l sits at slot 16 (l % 8) + l / 8,
// so that the 16 l-splits read 16 consecutive slots, and its two 16-byte
// halves are swapped when bit 6 of l is set, which puts the 16 lanes of one
// read on distinct banks.
__device__ __forceinline__ int scan_slot(int l, int half) {
    return ((l & 7) * 16 + (l >> 3)) * kCols + 4 * (half ^ ((l >> 6) & 1));
}

template <int CTRL>
__device__ __forceinline__ float scan_dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                                 0xf, 0xf, false));
}

// One level of the reduce-scatter: entries [0, n) and [n, 2 n) of v are the
// two halves; the lane keeps one (the upper if `upper`) and adds the other
// half's partial from the partner lane that the DPP pattern CTRL names (the
// partner keeps the opposite half).
template <int CTRL, int n>
__device__ __forceinline__ void scan_fold(float (&v)[32], bool upper) {
#pragma unroll
    for (int j = 0; j < n; ++j) {
        const float a = v[j], b = v[j + n];
        v[j] = (upper ? b : a) + scan_dpp<CTRL>(upper ? a : b);
    }
}

__global__ __launch_bounds__(512) void segment_scan_kernel(const float *__restrict__ M,
                                                           const float *__restrict__ B,
                                                           const float *__restrict__ S0,
                                                           float *__restrict__ Sin,
                                                           const int32_t *__restrict__ seg,
                                                           int64_t H) {
    static_assert(kCols == 8 && D == 128, "thread layout below");
    const int64_t nh = blockIdx.x;                 // sequence n, head h: n * H + h
    const int64_t n = nh / H, h = nh % H;
    const int64_t first = seg[n], P = seg[n + 1] - first;   // this sequence's segments
    if (P <= 0) return;                            // (capped plan: nothing to scan)
    const int c0 = kCols * blockIdx.y;             // columns c0 .. c0 + 7
    const int t = threadIdx.x, s = t & 15, g = t >> 4;
    const int row0 = 4 * g;                        // rows row0 .. row0 + 3
    // after the reduce-scatter: row row0 + 2 b3 + b2, columns 4 b1 + 2 b0 + {0, 1}
    const bool b3 = (s >> 3) & 1, b2 = (s >> 2) & 1, b1 = (s >> 1) & 1, b0 = s & 1;
    const int orow = row0 + 2 * b3 + b2, ocol = 4 * b1 + 2 * b0;
    __shared__ __attribute__((aligned(16))) float Ss[2][D * kCols];

    // S_in(0): 512 threads x 2 floats
    {
        const int r = t >> 2, c = 2 * (t & 3);
        float2 x = make_float2(0.f, 0.f);
        if (S0) x = *reinterpret_cast<const float2 *>(S0 + nh * kState + r * D + c0 + c);
        *reinterpret_cast<float2 *>(&Ss[0][scan_slot(r, c >> 2) + (c & 3)]) = x;
    }
    auto unit = [&](int64_t p) { return (first + p) * H + h; };   // segment unit index
    auto load = [&](int64_t p, float4 (&dst)[8], float2 &bdst) {
        const float *mp = M + unit(p) * kState + row0 * D + 8 * s;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            dst[2 * rr] = *reinterpret_cast<const float4 *>(mp + rr * D);
            dst[2 * rr + 1] = *reinterpret_cast<const float4 *>(mp + rr * D + 4);
        }
        bdst = *reinterpret_cast<const float2 *>(B + unit(p) * kState + orow * D + c0 + ocol);
    };
    // LDS read addresses of this lane's 8 rows l = 8 s + j (the j-th at +j*16*kCols)
    const int rd0 = scan_slot(8 * s, 0), rd1 = scan_slot(8 * s, 1);
    const int wr = scan_slot(orow, ocol >> 2) + (ocol & 3);

    // One step: S(p+1) = M_p S(p) + B_p from the operands in (mc, bc) while
    // segment p+1's load into (mx, bx); the two register sets alternate.  The
    // load is unconditional (the last step reloads the last segment): with a
    // path that skipped it, the compiler could no longer count which loads
    // are still in flight and would wait for all of them.
    auto step = [&](int64_t p, float4 (&mc)[8], float2 &bc, float4 (&mx)[8], float2 &bx) {
        const int cur = static_cast<int>(p & 1);
        load(p + 1 < P ? p + 1 : P - 1, mx, bx);
        float acc[32];
#pragma unroll
        for (int e = 0; e < 32; ++e) acc[e] = 0.f;
        const float *sb = Ss[cur];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float4 lo = *reinterpret_cast<const float4 *>(sb + rd0 + j * 16 * kCols);
            const float4 hi = *reinterpret_cast<const float4 *>(sb + rd1 + j * 16 * kCols);
            const float x[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const float4 mq = mc[2 * rr + (j >> 2)];
                const float m = (j & 3) == 0 ? mq.x : (j & 3) == 1 ? mq.y : (j & 3) == 2 ? mq.z : mq.w;
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[8 * rr + c] += m * x[c];
            }
        }
        // acc[8 rr + c]: halves by row pair (bit 3), row (bit 2), column
        // quad (bit 1), column pair (bit 0)
        scan_fold<0x140, 16>(acc, b3);   // row_mirror: partner 15 - s
        scan_fold<0x141, 8>(acc, b2);    // row_half_mirror: partner s ^ 7
        scan_fold<0x4e, 4>(acc, b1);     // quad_perm [2,3,0,1]: partner s ^ 2
        scan_fold<0xb1, 2>(acc, b0);     // quad_perm [1,0,3,2]: partner s ^ 1
        const float2 y = make_float2(acc[0] + bc.x, acc[1] + bc.y);
        *reinterpret_cast<float2 *>(&Ss[cur ^ 1][wr]) = y;
        *reinterpret_cast<float2 *>(Sin + unit(p + 1) * kState + orow * D + c0 + ocol) = y;
        __syncthreads();
    };
    // S_in(0) out
    {
        const int r = t >> 2, c = 2 * (t & 3);
        __syncthreads();
        *reinterpret_cast<float2 *>(Sin + unit(0) * kState + r * D + c0 + c) =
            *reinterpret_cast<const float2 *>(&Ss[0][scan_slot(r, c >> 2) + (c & 3)]);
    }
    // P - 1 steps, in pairs that always run both halves: a pair that could
    // stop after its first step would let the compiler sink that step's
    // loads into the second (their only user), which undoes the prefetch
    float4 ma[8], mb[8];
    float2 ba, bb;
    load(0, ma, ba);
    if ((P - 1) & 1) {
        step(0, ma, ba, mb, bb);
        for (int64_t p = 1; p + 1 < P; p += 2) {
            step(p, mb, bb, ma, ba);
            step(p + 1, ma, ba, mb, bb);
        }
    } else {
        for (int64_t p = 0; p + 1 < P; p += 2) {
            step(p, ma, ba, mb, bb);
            step(p + 1, mb, bb, ma, ba);
        }
    }
}

// S_T of sequence n = the end state of its last segment (its S0, or zero, if
// a capped plan left it none).
__global__ __launch_bounds__(256) void segment_gather_kernel(const float *__restrict__ Sout,
                                                             const float *__restrict__ S0,
                                                             const int32_t *__restrict__ seg,
                                                             float *__restrict__ S_T, int64_t H) {
    const int64_t nh = blockIdx.x, n = nh / H, h = nh % H;
    const int64_t last = static_cast<int64_t>(seg[n + 1]) - 1;
    float4 *dst = reinterpret_cast<float4 *>(S_T + nh * kState);
    if (last >= seg[n]) {
        const float4 *src = reinterpret_cast<const float4 *>(Sout + (last * H + h) * kState);
        for (int i = threadIdx.x; i < kState / 4; i += 256) dst[i] = src[i];
    } else {
        const float4 *src = S0 ? reinterpret_cast<const float4 *>(S0 + nh * kState) : nullptr;
        for (int i = threadIdx.x; i < kState / 4; i += 256)
            dst[i] = src ? src[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
}

}  // namespace

hipError_t launch_segment_prep(const int32_t *cu_in, int64_t N, int64_t T, int64_t L, int64_t Ns,
                               int32_t *seg, int32_t *cu_out, float *sid, int64_t units,
                               hipStream_t stream) {
    segment_prep_kernel<<<1025, kPrepThreads, 0, stream>>>(cu_in, N, T, L, Ns, seg, cu_out, sid,
                                                          units);
    return hipGetLastError();
}

hipError_t launch_segment_scan(const float *M, const float *B, const float *S0, float *Sin,
                               const int32_t *seg, int64_t N, int64_t H, hipStream_t stream) {
    segment_scan_kernel<<<dim3(static_cast<unsigned>(N * H), D / kCols), 512, 0, stream>>>(
        M, B, S0, Sin, seg, H);
    return hipGetLastError();
}

hipError_t launch_segment_gather(const float *Sout, const float *S0, const int32_t *seg,
                                 float *S_T, int64_t N, int64_t H, hipStream_t stream) {
    segment_gather_kernel<<<static_cast<unsigned>(N * H), 256, 0, stream>>>(Sout, S0, seg, S_T, H);
    return hipGetLastError();
}

}  // namespace gdn
